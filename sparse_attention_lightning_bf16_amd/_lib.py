"""ctypes loader of liblix.so; fails loudly when the library is not built."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblix.so")

LIX_OK = 0
LIX_ERR_NULL = -1
LIX_ERR_SHAPE = -2
LIX_ERR_UNSUPPORTED = -3
LIX_ERR_DEVICE = -4
LIX_ERR_LAUNCH = -5
LIX_FUSED_TOPK_MAX = 2048
LIX_NOALLOC_SCRATCH_BYTES = 64 << 20

# Symbols exported by liblix.so, with their C signatures (include/lix.h).
_P = ctypes.c_void_p
_I = ctypes.c_int
_LL = ctypes.c_longlong
SIGNATURES = {
    "lix_status_string": (ctypes.c_char_p, [_I]),
    "lix_version": (_I, []),
    "lix_indexer_logits": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "lix_indexer_logits_visible": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "lix_topk": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P]),
    "lix_topk_fused_supported": (_I, [_I, _I, _I, _I]),
    "lix_topk_streaming": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _LL, _P]),
    "lix_topk_streaming_workspace_bytes": (_LL, [_I, _I, _I, _I, _I]),
    "lix_topk_scores": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "lix_indexer_scores_v41": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "lix_indexer_scores_at": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P]),
    "lix_topk_bf16": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "lix_indexer_backward": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _LL,
                                  _P]),
    "lix_indexer_backward_workspace_bytes": (_LL, [_I, _I, _I, _I, _I, _I]),
    "lix_indexer_backward_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P,
                                          _P]),
}

_lib = None


class LixError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load():
    """Load liblix.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_lightning_bf16_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status):
    return load().lix_status_string(int(status)).decode()


def check(status, where):
    if status != LIX_OK:
        raise LixError(status, where)

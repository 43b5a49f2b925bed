"""The C ABI loads, exports what include/lix.h declares, and validates its
arguments on the host (no GPU needed: every case here fails validation before
any HIP call)."""

import os
import re

import pytest

import sparse_attention_lightning_bf16_amd as lx
from sparse_attention_lightning_bf16_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lix.h")

NULL, SHAPE, UNSUP, DEVICE = -1, -2, -3, -4
P = 1 << 20          # a fake, 16-byte aligned address: never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lix_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = lx.load()
    names = declared_functions()
    assert set(names) == {"lix_status_string", "lix_version", "lix_indexer_logits", "lix_indexer_logits_visible",
                          "lix_topk",
                          "lix_topk_scores", "lix_indexer_scores_v41", "lix_indexer_scores_at", "lix_topk_bf16",
                          "lix_indexer_backward", "lix_indexer_backward_workspace_bytes",
                          "lix_topk_fused_supported", "lix_indexer_backward_noalloc", "lix_topk_streaming",
                          "lix_topk_streaming_workspace_bytes"}
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES


def test_status_strings():
    for code in (0, NULL, SHAPE, UNSUP, DEVICE, -5):
        assert lx.status_string(code).startswith("LIX_")
    assert "UNKNOWN" in lx.status_string(-99)
    assert lx.load().lix_version() >= 100


def logits_call(q=P, k=P, w=P, B=1, S=8, Skv=2, H=64, D=128, c=4, ks=None, ke=None, out=P, visible=False):
    lib = lx.load()
    fn = lib.lix_indexer_logits_visible if visible else lib.lix_indexer_logits
    return fn(q, k, w, B, S, Skv, H, D, c, ks, ke, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(w=None), NULL), (dict(out=None), NULL),
    (dict(B=0), SHAPE), (dict(S=-1), SHAPE), (dict(Skv=0), SHAPE), (dict(H=0), SHAPE), (dict(D=0), SHAPE),
    (dict(c=0), SHAPE), (dict(ks=P), SHAPE), (dict(ke=P), SHAPE),
    (dict(H=3), UNSUP), (dict(H=256), UNSUP), (dict(H=96), UNSUP), (dict(D=24), UNSUP), (dict(D=272), UNSUP),
    (dict(q=P + 8), UNSUP), (dict(k=P + 2), UNSUP), (dict(w=P + 2), UNSUP), (dict(out=P + 1), UNSUP),
    (dict(ks=P + 1, ke=P), UNSUP),
    (dict(B=1 << 16, S=1 << 16, Skv=1 << 16), UNSUP),
    (dict(B=131072, S=8, D=128), UNSUP),           # key row stride B * index_dim = 2^24
    (dict(B=131071, S=8, D=128), DEVICE),          # just below: passes validation
])
@pytest.mark.parametrize("visible", [False, True])
def test_indexer_logits_validation(kw, code, visible):
    # lix_indexer_logits_visible validates exactly as lix_indexer_logits
    assert logits_call(**kw, visible=visible) == code


def topk_call(q=P, k=P, w=P, logits=None, B=1, S=8, Skv=4, H=64, D=128, c=4, ks=None, ke=None, topk=2,
              scores=P, idx=P):
    return lx.load().lix_topk(q, k, w, logits, B, S, Skv, H, D, c, ks, ke, topk, scores, idx, None)


@pytest.mark.parametrize("kw,code", [
    (dict(scores=None), NULL), (dict(idx=None), NULL), (dict(q=None), NULL),
    (dict(q=None, k=None, w=None, logits=None), NULL),
    (dict(topk=0), SHAPE), (dict(topk=5), SHAPE), (dict(c=0), SHAPE), (dict(S=0), SHAPE),
    (dict(ks=P), SHAPE),
    (dict(H=5), UNSUP), (dict(D=20), UNSUP),
    (dict(Skv=4096, topk=4096), UNSUP),            # fused: above the on-chip capacity
    (dict(H=4), UNSUP),                            # fused path needs heads >= 8
    (dict(Skv=70000, topk=16), UNSUP),             # fused: index above 16 bits
    (dict(H=8, Skv=4096, topk=1024), UNSUP),       # fused: candidates of 32 queries do not fit in LDS
    (dict(H=8, Skv=4096, topk=576), DEVICE),       # ... up to the documented capacity
    (dict(H=8, Skv=4096, topk=577), UNSUP),
    (dict(H=16, Skv=4096, topk=1217), UNSUP),
    (dict(H=32, D=256, Skv=4096, topk=1857), UNSUP),
    (dict(H=64, Skv=4096, topk=2048), DEVICE),
    (dict(B=131072, S=8, Skv=4, D=128), UNSUP),    # key row stride
    (dict(scores=P + 2), UNSUP), (dict(q=P + 4), UNSUP),
])
def test_topk_validation(kw, code):
    assert topk_call(**kw) == code


def streaming_call(q=P, k=P, w=P, B=1, S=8, Skv=4, H=64, D=128, c=4, ks=None, ke=None, topk=2, scores=P, idx=P,
                   ws=P, ws_bytes=1 << 20):
    return lx.load().lix_topk_streaming(q, k, w, B, S, Skv, H, D, c, ks, ke, topk, scores, idx, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(w=None), NULL), (dict(scores=None), NULL),
    (dict(idx=None), NULL), (dict(ws=None), NULL),
    (dict(topk=0), SHAPE), (dict(topk=5), SHAPE), (dict(c=0), SHAPE), (dict(S=0), SHAPE), (dict(ks=P), SHAPE),
    (dict(H=5), UNSUP), (dict(D=20), UNSUP), (dict(H=256), UNSUP),
    (dict(Skv=8193, topk=16), UNSUP),              # a row must fit the in-register selection
    (dict(Skv=8192, topk=8192, ws_bytes=4 * 8192 * 4), DEVICE),   # one slot of four queries (64 heads)
    (dict(Skv=8192, topk=16, ws_bytes=4 * 8192 * 4 - 1), SHAPE),  # less than one slot
    (dict(H=4, Skv=100, topk=50, ws_bytes=64 * 100 * 4), DEVICE),  # heads 4: 64 queries per block
    (dict(H=4, Skv=100, topk=50, ws_bytes=64 * 100 * 4 - 4), SHAPE),
    (dict(B=131072, S=8, D=128), UNSUP),           # key row stride
    (dict(scores=P + 2), UNSUP), (dict(q=P + 4), UNSUP), (dict(ws=P + 128), UNSUP), (dict(ks=P + 1, ke=P), UNSUP),
])
def test_topk_streaming_validation(kw, code):
    assert streaming_call(**kw) == code


def test_streaming_workspace_bytes_rejects_unsupported_sizes():
    f = lx.load().lix_topk_streaming_workspace_bytes
    for args in ((0, 8, 4, 64, 128), (1, 8, 8193, 64, 128), (1, 8, 4, 48, 128), (1, 8, 4, 64, 24),
                 (131072, 8, 4, 64, 128)):
        assert f(*args) == -1, args


# (heads, index_dim) -> largest topk of the fused path, as listed in include/lix.h
FUSED_CAPACITY = {
    8: {32: 704, 64: 640, 128: 576, 256: 384},
    16: {32: 1472, 64: 1408, 128: 1216, 256: 896},
    32: {32: 2048, 64: 2048, 128: 2048, 256: 1856},
    64: {32: 2048, 64: 2048, 128: 2048, 256: 2048},
    128: {32: 2048, 64: 2048, 128: 2048, 256: 2048},
}


def test_topk_fused_supported_matches_the_documented_limits_and_validation():
    lib = lx.load()
    for H in (1, 2, 4, 8, 16, 32, 64, 128):
        for D in (16, 32, 48, 64, 128, 256):
            dp = 32 if D <= 32 else 64 if D <= 64 else 128 if D <= 128 else 256
            cap = FUSED_CAPACITY.get(H, {}).get(dp, 0)
            for tk in sorted({1, 64, cap, cap + 1, 2048, 2049}):
                if tk < 1:
                    continue
                want = 1 if 1 <= tk <= cap else 0
                assert lib.lix_topk_fused_supported(65536, H, D, tk) == want, (H, D, tk)
                code = topk_call(H=H, D=D, Skv=65536, topk=tk)
                assert code == (DEVICE if want else UNSUP), (H, D, tk, code)
    assert lib.lix_topk_fused_supported(65537, 64, 128, 16) == 0
    assert lib.lix_topk_fused_supported(16, 64, 128, 17) == 0          # topk > Skv
    assert lib.lix_topk_fused_supported(4096, 48, 128, 16) == 0        # heads not a power of two
    assert lib.lix_topk_fused_supported(4096, 64, 24, 16) == 0         # index_dim not a multiple of 16


def test_topk_from_logits_ignores_q_k_w_shapes():
    # with logits given, q/k/w may be NULL and H/D are not checked; the call
    # passes validation and stops at the device check (no GPU here, or a
    # fake pointer on a GPU machine)
    assert topk_call(q=None, k=None, w=None, logits=P, H=0, D=0) == DEVICE


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), NULL), (dict(indices=None), NULL), (dict(scores=None), NULL),
    (dict(B=0), SHAPE), (dict(topk=0), SHAPE), (dict(Skv=-3), SHAPE),
    (dict(scores=P + 2), UNSUP),
])
def test_topk_scores_validation(kw, code):
    a = dict(logits=P, indices=P, B=1, S=4, Skv=8, topk=2, scores=P)
    a.update(kw)
    assert lx.load().lix_topk_scores(a["logits"], a["indices"], a["B"], a["S"], a["Skv"], a["topk"],
                                     a["scores"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(queries=None), NULL), (dict(keys=None), NULL), (dict(weights=None), NULL),
    (dict(allowed=None), NULL), (dict(scores=None), NULL),
    (dict(B=0), SHAPE), (dict(L=0), SHAPE), (dict(G=0), SHAPE), (dict(H=0), SHAPE), (dict(D=-16), SHAPE),
    (dict(H=6), UNSUP), (dict(H=256), UNSUP), (dict(D=40), UNSUP),
    (dict(queries=P + 8), UNSUP), (dict(weights=P + 1), UNSUP), (dict(scores=P + 1), UNSUP),
])
def test_v41_validation(kw, code):
    a = dict(queries=P, keys=P, weights=P, allowed=P, B=1, L=4, G=2, H=64, D=128, scores=P)
    a.update(kw)
    assert lx.load().lix_indexer_scores_v41(a["queries"], a["keys"], a["weights"], a["allowed"], a["B"], a["L"],
                                            a["G"], a["H"], a["D"], a["scores"], None) == code


def scores_at_call(q=P, k=P, w=P, idx=P, B=1, S=8, Skv=4, H=64, D=128, c=4, ks=None, ke=None, topk=2, out=P):
    return lx.load().lix_indexer_scores_at(q, k, w, idx, B, S, Skv, H, D, c, ks, ke, topk, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(w=None), NULL), (dict(idx=None), NULL),
    (dict(out=None), NULL),
    (dict(B=0), SHAPE), (dict(S=0), SHAPE), (dict(Skv=-3), SHAPE), (dict(topk=0), SHAPE), (dict(c=0), SHAPE),
    (dict(ks=P), SHAPE),
    (dict(H=48), UNSUP), (dict(D=40), UNSUP), (dict(q=P + 4), UNSUP), (dict(k=P + 8), UNSUP),
    (dict(idx=P + 2), UNSUP), (dict(out=P + 1), UNSUP),
    (dict(B=1 << 16, S=1 << 16, topk=1 << 16), UNSUP),
    (dict(B=131072, S=2, D=128), UNSUP),           # key row stride B * index_dim = 2^24
])
def test_scores_at_validation(kw, code):
    # topk may exceed Skv here (given indices need not be distinct)
    assert scores_at_call(**kw) == code


def backward_call(q=P, k=P, w=P, idx=P, g=P, B=1, S=8, Skv=4, H=64, D=128, c=4, ks=None, ke=None, topk=2, dq=P,
                  dk=P, dw=P, ws=P, ws_bytes=1 << 40):
    return lx.load().lix_indexer_backward(q, k, w, idx, g, B, S, Skv, H, D, c, ks, ke, topk, dq, dk, dw, ws, ws_bytes,
                                          None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(w=None), NULL), (dict(idx=None), NULL), (dict(g=None), NULL),
    (dict(dq=None), NULL), (dict(dk=None), NULL), (dict(dw=None), NULL),
    (dict(B=0), SHAPE), (dict(S=0), SHAPE), (dict(Skv=-3), SHAPE), (dict(topk=0), SHAPE), (dict(c=0), SHAPE),
    (dict(ke=P), SHAPE),
    (dict(H=128), UNSUP), (dict(H=48), UNSUP), (dict(D=32), UNSUP), (dict(D=144), UNSUP), (dict(D=40), UNSUP),
    (dict(q=P + 4), UNSUP), (dict(g=P + 2), UNSUP), (dict(dk=P + 4), UNSUP), (dict(dq=P + 2), UNSUP),
    (dict(dw=P + 1), UNSUP), (dict(B=1 << 16, S=1 << 16, topk=1 << 16), UNSUP),
    (dict(B=262144, S=2, D=64), UNSUP),            # key row stride B * index_dim = 2^24
    (dict(ws=None), NULL), (dict(ws_bytes=767), SHAPE), (dict(ws=P + 16), UNSUP), (dict(Skv=32769), UNSUP),
])
def test_backward_validation(kw, code):
    assert backward_call(**kw) == code


def test_backward_workspace_bytes():
    lib = lx.load()
    up = lambda x: (x + 255) // 256 * 256

    def parts(B, S, Skv, H, D, tk):
        # ReLU masks per entry and 32 heads, bucket bounds per 64 keys, 16-byte
        # bucketed entries: no [B,S,Skv] term and no copy of q
        nhg = max(1, H // 32)
        return up(B * S * tk * nhg * 4) + up(B * S * ((Skv + 63) // 64 + 1) * 4) + up(B * S * tk * 16)
    for args in ((1, 8, 4, 64, 128, 2), (2, 100, 30, 16, 48, 7), (1, 32768, 8192, 64, 128, 2048),
                 (1, 131072, 32768, 64, 128, 2048)):
        assert lib.lix_indexer_backward_workspace_bytes(*args) == parts(*args), args
    assert lib.lix_indexer_backward_workspace_bytes(1, 8, 4, 64, 128, 2) == 3 * 256
    # 32K: 1.5 GiB, 131K: 6.3 GiB (a dense [B,S,Skv] fp32 gradient alone would be 1 GiB / 16 GiB)
    assert lib.lix_indexer_backward_workspace_bytes(1, 32768, 8192, 64, 128, 2048) < 1.6 * (1 << 30)
    assert lib.lix_indexer_backward_workspace_bytes(1, 131072, 32768, 64, 128, 2048) < 6.5 * (1 << 30)
    assert lib.lix_indexer_backward_workspace_bytes(1, 8, 4, 128, 128, 2) == -1
    assert lib.lix_indexer_backward_workspace_bytes(1, 8, 40000, 64, 128, 2) == -1
    assert lib.lix_indexer_backward_workspace_bytes(1, 8, 4, 64, 128, 0) == -1


def topk_bf16_call(sc=P, B=1, L=8, G=16, topk=4, out=P, idx=P):
    return lx.load().lix_topk_bf16(sc, B, L, G, topk, out, idx, None)


@pytest.mark.parametrize("kw,code", [
    (dict(sc=None), NULL), (dict(out=None), NULL), (dict(idx=None), NULL),
    (dict(B=0), SHAPE), (dict(L=-1), SHAPE), (dict(G=0), SHAPE), (dict(topk=0), SHAPE), (dict(topk=17), SHAPE),
    (dict(G=8193, topk=4), UNSUP), (dict(sc=P + 1), UNSUP), (dict(out=P + 1), UNSUP), (dict(idx=P + 2), UNSUP),
])
def test_topk_bf16_validation(kw, code):
    assert topk_bf16_call(**kw) == code


def test_python_binding_rejects_bad_tensors_before_the_library():
    import torch
    q = torch.zeros(8, 1, 64, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 1, 128, dtype=torch.bfloat16)
    w = torch.zeros(8, 1, 64)
    with pytest.raises(ValueError):          # CPU tensors are refused
        lx.indexer_logits(q, k, w, 4)
    with pytest.raises(TypeError):
        lx.indexer_logits(q.float(), k, w, 4)


def backward_noalloc_call(q=P, k=P, w=P, idx=P, g=P, B=1, S=8, Skv=4, H=64, D=128, c=4, ks=None, ke=None, topk=2,
                          dq=P, dk=P, dw=P):
    return lx.load().lix_indexer_backward_noalloc(q, k, w, idx, g, B, S, Skv, H, D, c, ks, ke, topk, dq, dk, dw,
                                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(idx=None), NULL), (dict(g=None), NULL), (dict(dk=None), NULL),
    (dict(B=0), SHAPE), (dict(topk=0), SHAPE), (dict(ke=P), SHAPE),
    (dict(H=128), UNSUP), (dict(D=32), UNSUP), (dict(dk=P + 4), UNSUP), (dict(Skv=32769), UNSUP),
    # workspace above the static array: the entries alone are 256 MiB here
    (dict(B=1, S=32768, Skv=8192, topk=512), UNSUP),
    (dict(B=1, S=1024, Skv=1024), DEVICE),       # fits, stops at the device check
])
def test_backward_noalloc_validation(kw, code):
    assert backward_noalloc_call(**kw) == code


def test_backward_noalloc_limit_matches_the_workspace_size():
    lib = lx.load()
    cap = _lib.LIX_NOALLOC_SCRATCH_BYTES
    assert lib.lix_indexer_backward_workspace_bytes(1, 4096, 4096, 64, 128, 512) <= cap
    assert backward_noalloc_call(B=1, S=4096, Skv=4096, topk=512) == DEVICE
    assert lib.lix_indexer_backward_workspace_bytes(1, 4096, 4096, 64, 128, 1024) > cap
    assert backward_noalloc_call(B=1, S=4096, Skv=4096, topk=1024) == UNSUP

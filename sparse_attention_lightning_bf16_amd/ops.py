"""Python face of liblix: the C entry points plus the pages' entry point.

Every function only checks and marshals arguments (shapes, dtypes,
contiguity, output allocation, the current HIP stream) and calls the C ABI;
all arithmetic runs in the HIP kernels.  Inputs must be contiguous tensors on
the current GPU.
"""

import torch

from . import _lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ranges(ks, ke, S):
    if (ks is None) != (ke is None):
        raise ValueError("cu_seqlen_ks and cu_seqlen_ke must be given together")
    if ks is not None:
        _need(ks, "cu_seqlen_ks", torch.int32, 1)
        _need(ke, "cu_seqlen_ke", torch.int32, 1)
        if ks.shape[0] != S or ke.shape[0] != S:
            raise ValueError("cu_seqlen_ks/ke must have seqlen entries")
    return ks, ke


def _v4_shapes(q, k, w):
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 3)
    _need(w, "weights", torch.float32, 3)
    S, B, H, D = q.shape
    Skv = k.shape[0]
    if k.shape[1] != B or k.shape[2] != D:
        raise ValueError(f"k must be [seqlen_kv, {B}, {D}], got {tuple(k.shape)}")
    if tuple(w.shape) != (S, B, H):
        raise ValueError(f"weights must be [{S}, {B}, {H}], got {tuple(w.shape)}")
    if k.device != q.device or w.device != q.device:
        raise ValueError("q, k and weights must be on the same device")
    return S, B, H, D, Skv


def indexer_logits(q, k, weights, compress_ratio, cu_seqlen_ks=None, cu_seqlen_ke=None, out=None,
                   visible_only=False):
    """lix_indexer_logits: q [S,B,H,D] bf16, k [Skv,B,D] bf16, weights [S,B,H] fp32 -> [B,S,Skv] fp32.

    Positions outside [ks, ke) (causal [0, (t+1)//compress_ratio) when no
    ranges are given) hold -inf.  visible_only=True calls
    lix_indexer_logits_visible: the positions inside the ranges get the same
    bits, the others hold -inf or keep out's previous contents (for readers of
    the visible positions only, such as topk_from_logits).
    """
    S, B, H, D, Skv = _v4_shapes(q, k, weights)
    ks, ke = _ranges(cu_seqlen_ks, cu_seqlen_ke, S)
    if out is None:
        out = torch.empty(B, S, Skv, dtype=torch.float32, device=q.device)
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (B, S, Skv):
            raise ValueError("out must be [B, S, Skv]")
    lib = _lib.load()
    fn = lib.lix_indexer_logits_visible if visible_only else lib.lix_indexer_logits
    st = fn(q.data_ptr(), k.data_ptr(), weights.data_ptr(), B, S, Skv, H, D, int(compress_ratio), _ptr(ks),
            _ptr(ke), out.data_ptr(), _stream(q.device))
    _lib.check(st, "lix_indexer_logits_visible" if visible_only else "lix_indexer_logits")
    return out


def topk(q, k, weights, compress_ratio, topk, logits=None, cu_seqlen_ks=None, cu_seqlen_ke=None):
    """lix_topk.  With logits=None: fused scoring + top-k from q, k, weights (within the on-chip limits
    of include/lix.h; LixError LIX_ERR_UNSUPPORTED beyond them, see fused_topk_supported).
    With logits [B,S,Skv] fp32: top-k of the given logits (q, k, weights may
    be None).  Ranges are causal for compress_ratio unless cu_seqlen_ks/ke
    are given.

    Returns (scores fp32 [B,S,topk], indices int32 [B,S,topk]); selected keys
    in ascending index order, rows with fewer visible keys padded (-inf, -1).
    """
    if logits is not None:
        _need(logits, "logits", torch.float32, 3)
        B, S, Skv = logits.shape
        H = D = 0
        dev = logits.device
        qp = kp = wp = None
    else:
        S, B, H, D, Skv = _v4_shapes(q, k, weights)
        dev = q.device
        qp, kp, wp = q.data_ptr(), k.data_ptr(), weights.data_ptr()
    ks, ke = _ranges(cu_seqlen_ks, cu_seqlen_ke, S)
    scores = torch.empty(B, S, topk, dtype=torch.float32, device=dev)
    indices = torch.empty(B, S, topk, dtype=torch.int32, device=dev)
    st = _lib.load().lix_topk(qp, kp, wp, None if logits is None else logits.data_ptr(), B, S, Skv, H, D,
                              int(compress_ratio), _ptr(ks), _ptr(ke), int(topk), scores.data_ptr(),
                              indices.data_ptr(), _stream(dev))
    _lib.check(st, "lix_topk")
    return scores, indices


def fused_topk_supported(seqlen_kv, heads, index_dim, topk):
    """lix_topk_fused_supported: whether lix_topk's fused path takes these sizes (the on-chip limits are
    listed in include/lix.h at lix_topk)."""
    return bool(_lib.load().lix_topk_fused_supported(int(seqlen_kv), int(heads), int(index_dim), int(topk)))


STREAMING_MAX_SEQLEN_KV = 8192       # lix_topk_streaming: a row sits in registers while it is selected


def streaming_workspace_bytes(batch, seqlen, seqlen_kv, heads, index_dim):
    """lix_topk_streaming_workspace_bytes: the workspace lix_topk_streaming uses at full occupancy on the
    current device (-1 for sizes it does not take)."""
    return int(_lib.load().lix_topk_streaming_workspace_bytes(int(batch), int(seqlen), int(seqlen_kv), int(heads),
                                                              int(index_dim)))


def topk_streaming(q, k, weights, compress_ratio, topk, cu_seqlen_ks=None, cu_seqlen_ke=None, workspace=None):
    """lix_topk_streaming: scoring with each query block's top-k selected as soon as the block is scored
    (seqlen_kv <= 8192; no [B,S,Skv] tensor).  Same results, bit for bit, as indexer_logits followed by
    topk_from_logits.  workspace: an optional uint8 GPU tensor (allocated at the full-occupancy size when
    None).  Returns (scores fp32 [B,S,topk], indices int32 [B,S,topk])."""
    S, B, H, D, Skv = _v4_shapes(q, k, weights)
    ks, ke = _ranges(cu_seqlen_ks, cu_seqlen_ke, S)
    lib = _lib.load()
    if workspace is None:
        nbytes = int(lib.lix_topk_streaming_workspace_bytes(B, S, Skv, H, D))
        if nbytes < 0:
            raise _lib.LixError(_lib.LIX_ERR_UNSUPPORTED, "lix_topk_streaming_workspace_bytes")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    scores = torch.empty(B, S, topk, dtype=torch.float32, device=q.device)
    indices = torch.empty(B, S, topk, dtype=torch.int32, device=q.device)
    st = lib.lix_topk_streaming(q.data_ptr(), k.data_ptr(), weights.data_ptr(), B, S, Skv, H, D,
                                int(compress_ratio), _ptr(ks), _ptr(ke), int(topk), scores.data_ptr(),
                                indices.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(q.device))
    _lib.check(st, "lix_topk_streaming")
    return scores, indices


def select_topk(q, k, weights, compress_ratio, topk):
    """Top-k of the causal indexer scores by the route the library offers for these sizes without a
    [B,S,Skv] buffer where it can: the streaming kernel (lix_topk_streaming) for seqlen_kv <= 8192,
    else the fused kernel (lix_topk with no logits) where it holds the candidates on chip, else the
    materialized route (lix_indexer_logits_visible into a [B,S,Skv] fp32 buffer, then lix_topk over
    it). Every route selects the same keys and returns the same bits."""
    S, B, H, D, Skv = _v4_shapes(q, k, weights)
    if Skv <= STREAMING_MAX_SEQLEN_KV:
        return topk_streaming(q, k, weights, compress_ratio, topk)
    if fused_topk_supported(Skv, H, D, topk):
        return globals()["topk"](q, k, weights, compress_ratio, topk)
    logits = indexer_logits(q, k, weights, compress_ratio, visible_only=True)
    return topk_from_logits(logits, compress_ratio, topk)


def topk_from_logits(logits, compress_ratio, k, cu_seqlen_ks=None, cu_seqlen_ke=None):
    """lix_topk over materialized logits [B,S,Skv] fp32 (k = number of keys to select)."""
    return topk(None, None, None, compress_ratio, k, logits=logits, cu_seqlen_ks=cu_seqlen_ks,
                cu_seqlen_ke=cu_seqlen_ke)


def topk_scores(logits, topk_indices):
    """lix_topk_scores: logits [B,S,Skv] fp32 gathered at topk_indices [B,S,topk] int32 (-inf outside [0,Skv))."""
    _need(logits, "logits", torch.float32, 3)
    _need(topk_indices, "topk_indices", torch.int32, 3)
    B, S, Skv = logits.shape
    if topk_indices.shape[0] != B or topk_indices.shape[1] != S:
        raise ValueError("topk_indices must be [B, S, topk]")
    tk = topk_indices.shape[2]
    out = torch.empty(B, S, tk, dtype=torch.float32, device=logits.device)
    st = _lib.load().lix_topk_scores(logits.data_ptr(), topk_indices.data_ptr(), B, S, Skv, tk, out.data_ptr(),
                                     _stream(logits.device))
    _lib.check(st, "lix_topk_scores")
    return out


def indexer_scores_at(q, k, weights, compress_ratio, topk_indices, cu_seqlen_ks=None, cu_seqlen_ke=None):
    """lix_indexer_scores_at: the indexer scores at topk_indices [B,S,topk] int32, from q, k, weights
    (layouts as indexer_logits) without forming the logits; -inf where an index is outside the query's
    range (causal for compress_ratio unless cu_seqlen_ks/ke are given) or outside [0, Skv)."""
    S, B, H, D, Skv = _v4_shapes(q, k, weights)
    ks, ke = _ranges(cu_seqlen_ks, cu_seqlen_ke, S)
    _need(topk_indices, "topk_indices", torch.int32, 3)
    if topk_indices.shape[0] != B or topk_indices.shape[1] != S:
        raise ValueError("topk_indices must be [B, S, topk]")
    if topk_indices.device != q.device:
        raise ValueError("topk_indices must be on the device of q")
    tk = topk_indices.shape[2]
    out = torch.empty(B, S, tk, dtype=torch.float32, device=q.device)
    st = _lib.load().lix_indexer_scores_at(q.data_ptr(), k.data_ptr(), weights.data_ptr(), topk_indices.data_ptr(),
                                           B, S, Skv, H, D, int(compress_ratio), _ptr(ks), _ptr(ke), tk,
                                           out.data_ptr(), _stream(q.device))
    _lib.check(st, "lix_indexer_scores_at")
    return out


def indexer_backward(q, k, weights, compress_ratio, topk_indices, grad_scores, cu_seqlen_ks=None,
                     cu_seqlen_ke=None):
    """lix_indexer_backward: gradients of indexer_scores_at's scores.  grad_scores fp32 [B,S,topk]
    (the upstream gradient of the scores at topk_indices).  Returns fp32 (dq [S,B,H,D], dk [Skv,B,D],
    dw [S,B,H]); entries outside the query's range contribute nothing.  The workspace the call needs
    (lix_indexer_backward_workspace_bytes) is allocated here with torch."""
    S, B, H, D, Skv = _v4_shapes(q, k, weights)
    ks, ke = _ranges(cu_seqlen_ks, cu_seqlen_ke, S)
    _need(topk_indices, "topk_indices", torch.int32, 3)
    _need(grad_scores, "grad_scores", torch.float32, 3)
    if topk_indices.shape[0] != B or topk_indices.shape[1] != S:
        raise ValueError("topk_indices must be [B, S, topk]")
    if grad_scores.shape != topk_indices.shape:
        raise ValueError("grad_scores must have the shape of topk_indices")
    if topk_indices.device != q.device or grad_scores.device != q.device:
        raise ValueError("topk_indices and grad_scores must be on the device of q")
    tk = topk_indices.shape[2]
    lib = _lib.load()
    ws_bytes = lib.lix_indexer_backward_workspace_bytes(B, S, Skv, H, D, tk)
    if ws_bytes < 0:
        raise _lib.LixError(-3, "lix_indexer_backward_workspace_bytes")
    dq = torch.empty(S, B, H, D, dtype=torch.float32, device=q.device)
    dk = torch.empty(Skv, B, D, dtype=torch.float32, device=q.device)
    dw = torch.empty(S, B, H, dtype=torch.float32, device=q.device)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.lix_indexer_backward(q.data_ptr(), k.data_ptr(), weights.data_ptr(), topk_indices.data_ptr(),
                                  grad_scores.data_ptr(), B, S, Skv, H, D, int(compress_ratio), _ptr(ks), _ptr(ke), tk,
                                  dq.data_ptr(), dk.data_ptr(), dw.data_ptr(), ws.data_ptr(), ws_bytes,
                                  _stream(q.device))
    _lib.check(st, "lix_indexer_backward")
    return dq, dk, dw


class V4IndexerFunction(torch.autograd.Function):
    """Autograd Function of the indexer (page "...tilelang_indexer", class V4IndexerFunction).

    forward(index_q, index_k, weights, compress_ratio, topk, topk_indices=None) returns
    (scores, indices): the top-k (select_topk: the streaming kernel, the fused kernel or the
    materialized route, by size) when topk_indices is None, else the scores at topk_indices
    (returned unchanged as the indices).  backward(grad_scores, grad_indices) gives the
    gradients of q, k and weights through the selected scores (lix_indexer_backward), in their dtypes;
    the indices and the integer arguments get none.
    """

    @staticmethod
    def forward(ctx, index_q, index_k, weights, compress_ratio, topk, topk_indices=None):
        if topk_indices is None:
            scores, indices = select_topk(index_q, index_k, weights, compress_ratio, topk)
        else:
            indices = topk_indices
            scores = indexer_scores_at(index_q, index_k, weights, compress_ratio, indices)
        ctx.save_for_backward(index_q, index_k, weights, indices)
        ctx.compress_ratio = int(compress_ratio)
        ctx.mark_non_differentiable(indices)
        return scores, indices

    @staticmethod
    def backward(ctx, grad_scores, grad_indices):
        q, k, w, indices = ctx.saved_tensors
        if grad_scores is None:
            return None, None, None, None, None, None
        dq, dk, dw = indexer_backward(q, k, w, ctx.compress_ratio, indices, grad_scores.contiguous().float())
        return dq.to(q.dtype), dk.to(k.dtype), dw.to(w.dtype), None, None, None


def indexer_scores_v41(queries, keys, weights, allowed):
    """lix_indexer_scores_v41: queries [B,L,H,D], keys [B,G,D], weights [B,L,H] (bf16),
    allowed [B,L,G] bool -> bf16 [B,L,G] (-inf where hidden)."""
    _need(queries, "queries", torch.bfloat16, 4)
    _need(keys, "keys", torch.bfloat16, 3)
    _need(weights, "weights", torch.bfloat16, 3)
    _need(allowed, "allowed", torch.bool, 3)
    B, L, H, D = queries.shape
    G = keys.shape[1]
    if tuple(keys.shape) != (B, G, D) or tuple(weights.shape) != (B, L, H) or tuple(allowed.shape) != (B, L, G):
        raise ValueError("shapes must be queries [B,L,H,D], keys [B,G,D], weights [B,L,H], allowed [B,L,G]")
    out = torch.empty(B, L, G, dtype=torch.bfloat16, device=queries.device)
    st = _lib.load().lix_indexer_scores_v41(queries.data_ptr(), keys.data_ptr(), weights.data_ptr(),
                                            allowed.data_ptr(), B, L, G, H, D, out.data_ptr(),
                                            _stream(queries.device))
    _lib.check(st, "lix_indexer_scores_v41")
    return out


def topk_bf16(scores, topk):
    """lix_topk_bf16: per-row top-k of V4.1 bf16 scores [B,L,G] over the visible keys (score != bf16 -inf).
    Returns (scores bf16 [B,L,topk], indices int32 [B,L,topk]); selected keys in ascending index order,
    rows with fewer visible keys padded (-inf, -1)."""
    _need(scores, "scores", torch.bfloat16, 3)
    B, L, G = scores.shape
    out = torch.empty(B, L, topk, dtype=torch.bfloat16, device=scores.device)
    idx = torch.empty(B, L, topk, dtype=torch.int32, device=scores.device)
    st = _lib.load().lix_topk_bf16(scores.data_ptr(), B, L, G, int(topk), out.data_ptr(), idx.data_ptr(),
                                   _stream(scores.device))
    _lib.check(st, "lix_topk_bf16")
    return out, idx


def v4_lighting_indexer(index_q, index_k, weights, compress_ratio, topk, topk_indices=None):
    """The pages' main entry point (the misspelt name is the pages' own).

    Without topk_indices: scoring + top-k, returns (scores, indices): the streaming kernel for
    seqlen_kv <= 8192, else the fused kernel, or for sizes it cannot hold on chip (heads < 8,
    seqlen_kv > 65536, topk above the per-head capacity listed in include/lix.h) the materialized
    logits then the row top-k; all give the same bits.
    With topk_indices [B,S,topk] int32: the scores at those indices, scored
    directly (lix_indexer_scores_at; equal bit for bit to gathering the
    materialized logits), returns scores.  Both go through V4IndexerFunction,
    so the scores carry gradients to index_q, index_k and weights.
    """
    scores, indices = V4IndexerFunction.apply(index_q, index_k, weights, compress_ratio, topk, topk_indices)
    return (scores, indices) if topk_indices is None else scores

"""Plain, slow, float64 oracle of the lightning-indexer forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module, and this module imports nothing from it.

What is computed, and from which passage of the pages:

* Causal range.  Page "deepseek_v4.kernels.tilelang_indexer_fwd", section
  ``_make_causal_cu_seqlens``: a query at position p may see the compressed
  key groups in the half-open range [0, (p+1) // compress_ratio).
* Scores.  Page "deepseek_v4.kernels.tilelang_indexer" (header: the DSA
  indexer adapted to V4's SBHD layout and causal masking) and page
  "deepseek_v4.kernels.tilelang_indexer_fwd", section ``batched_indexer_fwd``
  (shapes q [S,B,H,D], k [Skv,B,D], weights [S,B,H] -> logits [B,S,Skv]):
  logits[b,t,s] = sum_h w[t,b,h] * max(0, q[t,b,h,:] . k[s,b,:]) for s inside
  the query's range and -inf outside it (section ``clean_logits_``).
* Top-k.  Page "deepseek_v4.kernels.tilelang_indexer", section
  ``v4_lighting_indexer`` (topk = the number of indices to select; returns
  [B,S,topk] fp32 scores and int32 indices).
* Gather at given indices.  Same page, section ``pytorch_extract_topk_scores``.
* Top-k of V4.1 scores over the visible keys.  Page "deepseek_v41.indexer",
  module description (candidate selection follows the scoring), with V4's
  selection rule.
* V4.1 scores.  Page "deepseek_v41.indexer", module description and section
  ``indexer_scores``: the GEMM output and each weighted head score are
  rounded to BF16 before the FP32 head reduction; ``allowed`` selects the
  visible (query, key) pairs; the result is BF16.

Readings where the pages are silent (each listed in the design notes):
half-open ranges with ke clamped to [0, Skv]; -inf outside the range; top-k
ties broken towards the lower key index; rows with fewer than topk valid keys
padded with (index -1, score -inf); the selected entries are returned in
ascending key-index order; bf16 rounding is round-to-nearest-even; positions
that ``allowed`` hides hold bf16 -inf.

Inputs are NumPy arrays.  bfloat16 tensors are passed as their raw uint16 bit
patterns, float32 tensors as float32; both are upcast to float64 exactly.
Plain float64 or integer arrays are used as they are.
"""

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper half of the float32 with the same sign,
    exponent and leading 7 fraction bits.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _f64(a):
    """Exact upcast of an input array to float64 (uint16 means bf16 bits)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def rne_bf16(x):
    """Round float64 values to bfloat16, round-to-nearest, ties-to-even.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's
    exponent range: normal numbers down to 2**-126, subnormals with the fixed
    spacing 2**-133, largest finite value (2 - 2**-7) * 2**127.  For a value
    with |x| in [2**(e-1), 2**e) the spacing of representable values is
    2**(e-8) (never below 2**-133); x is divided by that spacing (exact, a
    power of two), rounded to the nearest integer with ties to the even one,
    and scaled back.  A result of magnitude 2**128 or more overflows to inf.
    Infinities pass through unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)                       # |xf| in [2**(e-1), 2**e)
    q = np.maximum(e - 8, -133)               # exponent of the spacing
    r = np.rint(np.ldexp(xf, -q))             # np.rint rounds ties to even
    y = np.ldexp(r, q)
    big = np.abs(y) >= 2.0 ** 128
    y[big] = np.copysign(np.inf, xf[big])
    out[fin] = y
    return out


def f64_to_bf16_bits(x):
    """bfloat16-representable float64 values -> uint16 bit patterns.

    The value must already be representable (for instance the output of
    rne_bf16); it then converts to float32 exactly and its upper half is the
    bfloat16 pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    u = x.astype(np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def ulp_bf16(x):
    """Spacing of bfloat16 values at |x| (2**(e-8) for |x| in [2**(e-1), 2**e), 2**-133 at 0)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)
    e = np.where(x == 0.0, -133 + 8, e)            # zero: the subnormal spacing
    return np.ldexp(1.0, np.maximum(e - 8, -133))


# ---------------------------------------------------------------------------
# V4: causal range, logits, top-k, gather
# ---------------------------------------------------------------------------

def causal_ranges(seq_len_q, seq_len_kv, compress_ratio):
    """Per-query visible key range [ks, ke) over compressed positions.

    Page "deepseek_v4.kernels.tilelang_indexer_fwd", ``_make_causal_cu_seqlens``:
    the query at position p sees the groups [0, (p+1) // compress_ratio).
    The end is clamped to seq_len_kv, which that function also receives.
    Returns (ks, ke) as int64 arrays of length seq_len_q.
    """
    p = np.arange(seq_len_q, dtype=np.int64)
    ke = np.minimum((p + 1) // int(compress_ratio), int(seq_len_kv))
    ks = np.zeros_like(ke)
    return ks, ke


def _clamped_range(ks, ke, t, n):
    lo = min(max(int(ks[t]), 0), n)
    hi = min(max(int(ke[t]), 0), n)
    return lo, hi


def indexer_logits_rows(q, k, w, b, rows, ks, ke, with_magnitude=False):
    """Logits of the query rows ``rows`` of batch element ``b``.

    q [S,B,H,D], k [Skv,B,D], w [S,B,H] (SBHD, as on page
    "deepseek_v4.kernels.tilelang_indexer", ``V4IndexerFunction``).
    For each query t and key s:  sum_h w[t,b,h] * max(0, q[t,b,h,:] . k[s,b,:])
    where ks[t] <= s < ke[t], and -inf elsewhere.

    With ``with_magnitude`` also returns sum_h |w[t,b,h]| * |q[t,b,h,:] . k[s,b,:]|
    (the scale of the float32 rounding error a kernel may make), 0 outside the
    range.  Returns float64 arrays of shape [len(rows), Skv].
    """
    rows = np.asarray(rows, dtype=np.int64)
    kb = _f64(k[:, b, :])                                   # [Skv, D]
    n_kv = kb.shape[0]
    H = q.shape[2]
    out = np.full((len(rows), n_kv), NEG_INF)
    mag = np.zeros((len(rows), n_kv)) if with_magnitude else None
    group = max(1, (1 << 22) // max(1, H * n_kv))           # bounds the [R,H,Skv] temporary
    for g0 in range(0, len(rows), group):
        rr = rows[g0:g0 + group]
        qg = _f64(q[rr, b])                                 # [R, H, D]
        wg = _f64(w[rr, b])                                 # [R, H]
        d = np.matmul(qg, kb.T)                             # [R, H, Skv]: q_h . k_s
        lg = np.einsum("rh,rhs->rs", wg, np.maximum(d, 0.0))
        if with_magnitude:
            mg = np.einsum("rh,rhs->rs", np.abs(wg), np.abs(d))
        for i, t in enumerate(rr):
            lo, hi = _clamped_range(ks, ke, t, n_kv)
            if hi > lo:
                out[g0 + i, lo:hi] = lg[i, lo:hi]
                if with_magnitude:
                    mag[g0 + i, lo:hi] = mg[i, lo:hi]
    return (out, mag) if with_magnitude else out


def indexer_logits(q, k, w, ks, ke, with_magnitude=False):
    """Full logits [B,S,Skv] (page "...tilelang_indexer_fwd", ``batched_indexer_fwd``).

    The batch loop mirrors the page: ks/ke are [S] and shared by every batch
    element.
    """
    S, B = q.shape[0], q.shape[1]
    n_kv = k.shape[0]
    out = np.empty((B, S, n_kv))
    mag = np.empty((B, S, n_kv)) if with_magnitude else None
    rows = np.arange(S)
    for b in range(B):
        r = indexer_logits_rows(q, k, w, b, rows, ks, ke, with_magnitude)
        if with_magnitude:
            out[b], mag[b] = r
        else:
            out[b] = r
    return (out, mag) if with_magnitude else out


def topk_select(scores, ks, ke, topk):
    """Top-k of each row of ``scores`` [R, Skv] over the row's range [ks, ke).

    The m = min(topk, ke - ks) best keys are chosen by score, descending,
    with equal scores ordered by key index, ascending (the lower index wins).
    They are returned in ascending key-index order; slots m..topk-1 hold
    index -1 and score -inf.  ``ks``/``ke`` are indexed by row.
    Returns (scores float64 [R, topk], indices int64 [R, topk]).
    """
    scores = np.asarray(scores, dtype=np.float64)
    R, n_kv = scores.shape
    out_s = np.full((R, topk), NEG_INF)
    out_i = np.full((R, topk), -1, dtype=np.int64)
    for r in range(R):
        lo, hi = _clamped_range(ks, ke, r, n_kv)
        if hi <= lo:
            continue
        idx = np.arange(lo, hi)
        val = scores[r, lo:hi]
        order = np.lexsort((idx, -val))        # last key is primary: -val ascending
        m = min(topk, hi - lo)
        chosen = np.sort(idx[order[:m]])
        out_i[r, :m] = chosen
        out_s[r, :m] = scores[r, chosen]
    return out_s, out_i


def topk_select_visible_bf16(score_bits, topk):
    """Top-k of each row of V4.1 bf16 scores [R, G] over the row's visible keys.

    Page "deepseek_v41.indexer", module description: the scores feed a top-k /
    candidate selection that runs after ``indexer_scores``; positions the
    ``allowed`` mask hides hold bf16 -inf (0xFF80), so a key is visible when
    its score is anything else.  The selection rule is V4's (``topk_select``):
    the m = min(topk, visible keys) best by score, descending, equal scores by
    key index, ascending; returned in ascending key-index order, slots
    m..topk-1 holding index -1 and score 0xFF80.  Scores are compared as the
    exact values of their bit patterns (so -0 and +0 tie).
    Returns (score bits uint16 [R, topk], indices int64 [R, topk]).
    """
    bits = np.asarray(score_bits, dtype=np.uint16)
    vals = bf16_bits_to_f64(bits)
    R = bits.shape[0]
    out_b = np.full((R, topk), 0xFF80, dtype=np.uint16)
    out_i = np.full((R, topk), -1, dtype=np.int64)
    for r in range(R):
        vis = np.nonzero(bits[r] != 0xFF80)[0]
        if len(vis) == 0:
            continue
        order = np.lexsort((vis, -vals[r, vis]))
        m = min(topk, len(vis))
        chosen = np.sort(vis[order[:m]])
        out_i[r, :m] = chosen
        out_b[r, :m] = bits[r, chosen]
    return out_b, out_i


def topk_scores_gather(logits, indices):
    """logits[..., idx] for each index; -inf where idx is outside [0, Skv).

    Page "deepseek_v4.kernels.tilelang_indexer", ``pytorch_extract_topk_scores``
    (gather along the last dimension).  An index of -1 is the padding value
    of ``topk_select`` and maps to -inf.
    """
    logits = np.asarray(logits, dtype=np.float64)
    indices = np.asarray(indices, dtype=np.int64)
    n_kv = logits.shape[-1]
    valid = (indices >= 0) & (indices < n_kv)
    safe = np.where(valid, indices, 0)
    got = np.take_along_axis(logits, safe, axis=-1)
    return np.where(valid, got, NEG_INF)


# ---------------------------------------------------------------------------
# V4.1: BF16-rounded scores with an ``allowed`` mask
# ---------------------------------------------------------------------------

def _v41_group(queries, keys, weights, b, rr):
    qg = _f64(queries[b, rr])                              # [R, H, D]
    kb = _f64(keys[b])                                     # [G, D]
    wg = _f64(weights[b, rr])                              # [R, H]
    d = np.matmul(qg, kb.T)                                # [R, H, G]
    return qg, kb, wg, d


def indexer_scores_v41_rows(queries, keys, weights, allowed, b, rows):
    """V4.1 scores of the query rows ``rows`` of batch element ``b``.

    Page "deepseek_v41.indexer": queries [B,L,H,D], keys [B,G,D], weights
    [B,L,H] (all BF16), allowed [B,L,G] bool.  Steps, in the page's order:
      d   = q_h . k_s                 (the GEMM output, float64 here)
      r   = bf16(d)                   (GEMM output rounded to BF16)
      a   = max(0, r)
      e_h = bf16(w_h * a)             (weighted head score rounded to BF16;
                                       the product of two BF16 values is exact)
      S   = sum_h e_h                 (head reduction, float64 here)
      out = bf16(S) where allowed, else -inf.
    Returns float64 values (each a BF16 value) of shape [len(rows), G].
    """
    rows = np.asarray(rows, dtype=np.int64)
    H = queries.shape[2]
    G = keys.shape[1]
    out = np.empty((len(rows), G))
    group = max(1, (1 << 22) // max(1, H * G))
    for g0 in range(0, len(rows), group):
        rr = rows[g0:g0 + group]
        _, _, wg, d = _v41_group(queries, keys, weights, b, rr)
        r = rne_bf16(d)
        a = np.maximum(r, 0.0)
        e = rne_bf16(wg[:, :, None] * a)
        s = e.sum(axis=1)
        o = rne_bf16(s)
        vis = np.asarray(allowed[b, rr], dtype=bool)
        out[g0:g0 + len(rr)] = np.where(vis, o, NEG_INF)
    return out


def indexer_scores_v41(queries, keys, weights, allowed):
    """Full V4.1 scores [B,L,G] (float64 holding BF16 values)."""
    B, L = queries.shape[0], queries.shape[1]
    out = np.empty((B, L, keys.shape[1]))
    for b in range(B):
        out[b] = indexer_scores_v41_rows(queries, keys, weights, allowed, b, np.arange(L))
    return out


def indexer_scores_v41_bounds_rows(queries, keys, weights, allowed, b, rows,
                                   unit=2.0 ** -24, slack=2.0):
    """Interval [lo, hi] that any float32-accumulating kernel's V4.1 result lies in.

    A kernel forms d in float32 (D exact BF16 products summed in some order)
    and the head sum in float32 (H exact BF16 terms in some order).  With u the
    float32 unit roundoff, |fl(d) - d| <= slack*D*u * sum_i |q_i k_i| and
    |fl(S) - S| <= slack*H*u * sum_h |e_h|.  Rounding is monotone, so pushing
    both ends of each error interval through the page's rounding steps gives
    bounds on every BF16 value the kernel may legitimately return.  Hidden
    positions get lo = hi = -inf.
    """
    rows = np.asarray(rows, dtype=np.int64)
    H, D = queries.shape[2], queries.shape[3]
    G = keys.shape[1]
    lo_out = np.empty((len(rows), G))
    hi_out = np.empty((len(rows), G))
    group = max(1, (1 << 21) // max(1, H * G))
    for g0 in range(0, len(rows), group):
        rr = rows[g0:g0 + group]
        qg, kb, wg, d = _v41_group(queries, keys, weights, b, rr)
        eps = slack * D * unit * np.matmul(np.abs(qg), np.abs(kb).T)
        a_lo = np.maximum(rne_bf16(d - eps), 0.0)
        a_hi = np.maximum(rne_bf16(d + eps), 0.0)
        p1 = rne_bf16(wg[:, :, None] * a_lo)
        p2 = rne_bf16(wg[:, :, None] * a_hi)
        e_lo = np.minimum(p1, p2)
        e_hi = np.maximum(p1, p2)
        delta = slack * H * unit * np.maximum(np.abs(e_lo), np.abs(e_hi)).sum(axis=1)
        lo = rne_bf16(e_lo.sum(axis=1) - delta)
        hi = rne_bf16(e_hi.sum(axis=1) + delta)
        vis = np.asarray(allowed[b, rr], dtype=bool)
        lo_out[g0:g0 + len(rr)] = np.where(vis, lo, NEG_INF)
        hi_out[g0:g0 + len(rr)] = np.where(vis, hi, NEG_INF)
    return lo_out, hi_out

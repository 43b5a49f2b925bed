"""Comparison rules between a kernel's results and the oracle's.

Test infrastructure.  Tolerances:
* V4 logits: |g - o| <= 1e-4 * sum_h |w_h| |q_h . k| + 1e-6 inside the range,
  the exact -inf bit pattern outside it.
* Top-k (per row, tau = the largest logit tolerance in the row, theta = the
  oracle's m-th best score): the indices are distinct, inside [ks, ke), m of
  them, in ascending order, with exact (-1, -inf) padding; every key whose
  oracle score exceeds theta + 2 tau is selected and every selected key's
  oracle score is at least theta - 2 tau (so where the oracle's m-th and
  (m+1)-th scores are more than 2 tau apart the set is the oracle's exactly);
  the sorted selected scores match the oracle's sorted top-m within tau; each
  returned score is within its own tolerance of the oracle's value.
* V4.1 scores: within 2 bf16 ulp of the oracle, or inside the interval the
  oracle derives for float32 accumulation in any order; -inf exactly where
  hidden.
* Backward (dq, dk, dw): |g - o| <= (2**-8 + 2**-11) * mag + amb + 1e-6,
  with mag and amb from the oracle.  Each term of a gradient product carries
  one bfloat16 rounding, as in a bfloat16 autograd graph of the forward (the
  upstream factor: g for dq, g * w_h for dk; q and k are the exact bf16
  inputs): round-to-nearest to 8 significant bits is off by at most 2**-8 of
  the value.  A few float32 roundings per term (the product g * w_h, the
  final scaling by w in dq) add at most ~2**-22.  The terms of one output
  element are summed in float32 in some order; for n terms, the probabilistic
  bound of Higham and Mary ("A new approach to probabilistic rounding error
  analysis", SIAM J. Sci. Comput. 41(5), 2019, Theorem 3.1) gives
  |error| <= lambda * sqrt(n) * 2**-24 * sum |terms| with probability at least
  1 - 2n exp(-lambda**2 / 2); with lambda = 9 and n <= 2**18 (4096 queries x 64
  heads into one dk element, the largest count checked element by element)
  that is 2.8e-4 < 2**-11, failing with probability below 2e-12 per element.
  amb covers (head, key) pairs whose dot product a float32 sum may put on the
  other side of 0, and, for dw, the float32 error of each dot product itself.
"""

import numpy as np

NEG_INF_F32_BITS = np.uint32(0xFF800000)
NEG_INF_BF16_BITS = np.uint16(0xFF80)


def logits_tolerance(mag):
    return 1e-4 * mag + 1e-6


def check_logits(gpu, ora, mag, where=""):
    """gpu: float32 array; ora/mag: float64 arrays of the same shape."""
    gpu = np.asarray(gpu, dtype=np.float32)
    valid = np.isfinite(ora)
    gbits = gpu.view(np.uint32)
    bad_mask = ~valid & (gbits != NEG_INF_F32_BITS)
    assert not bad_mask.any(), f"{where}: {int(bad_mask.sum())} masked positions are not -inf"
    g = gpu.astype(np.float64)
    assert np.isfinite(g[valid]).all(), f"{where}: non-finite value inside the range"
    err = np.abs(g[valid] - ora[valid])
    tol = logits_tolerance(mag[valid])
    if err.size:
        worst = int(np.argmax(err - tol))
        assert (err <= tol).all(), (f"{where}: {int((err > tol).sum())} logits out of tolerance; "
                                    f"worst err {err[worst]:.3e} tol {tol[worst]:.3e}")


def check_topk_rows(g_scores, g_idx, ora_row_scores, ora_row_mag, ks, ke, topk, where=""):
    """Check one kernel top-k result per row against the oracle's full rows.

    g_scores/g_idx: [R, topk]; ora_row_scores/mag: [R, Skv] float64 oracle
    logits and magnitudes of those rows; ks/ke: [R].
    Returns the number of rows where the oracle's boundary gap forced an
    exact set (for reporting).
    """
    g_scores = np.asarray(g_scores, dtype=np.float32)
    g_idx = np.asarray(g_idx, dtype=np.int64)
    R, n_kv = ora_row_scores.shape
    exact_rows = 0
    for r in range(R):
        lo = min(max(int(ks[r]), 0), n_kv)
        hi = min(max(int(ke[r]), 0), n_kv)
        n = max(0, hi - lo)
        m = min(topk, n)
        idx = g_idx[r]
        sc = g_scores[r]
        tag = f"{where} row {r}"
        # padding
        assert (idx[m:] == -1).all(), f"{tag}: padding indices wrong"
        assert (sc[m:].view(np.uint32) == NEG_INF_F32_BITS).all(), f"{tag}: padding scores not -inf"
        if m == 0:
            continue
        sel = idx[:m]
        assert ((sel >= lo) & (sel < hi)).all(), f"{tag}: index outside [ks, ke)"
        assert (np.diff(sel) > 0).all(), f"{tag}: indices not distinct and ascending"
        o = ora_row_scores[r, lo:hi]
        tol_row = logits_tolerance(ora_row_mag[r, lo:hi])
        tau = float(tol_row.max())
        # each returned score close to the oracle's value at that key
        o_sel = ora_row_scores[r, sel]
        tol_sel = logits_tolerance(ora_row_mag[r, sel])
        err = np.abs(sc[:m].astype(np.float64) - o_sel)
        assert (err <= tol_sel).all(), f"{tag}: selected score off by {err.max():.3e}"
        if m == n:
            continue
        order = np.sort(o)[::-1]
        theta = order[m - 1]
        must = np.nonzero(o > theta + 2 * tau)[0] + lo
        assert np.isin(must, sel).all(), f"{tag}: a key well above the threshold was not selected"
        assert (o_sel >= theta - 2 * tau).all(), f"{tag}: a key well below the threshold was selected"
        gs = np.sort(sc[:m].astype(np.float64))[::-1]
        assert np.all(np.abs(gs - order[:m]) <= tau), f"{tag}: sorted top-m scores differ"
        if order[m - 1] - order[m] > 2 * tau:
            exact_rows += 1
    return exact_rows


def check_v41(gpu_bits, ora, lo, hi, where=""):
    """gpu_bits: uint16 [.., G]; ora, lo, hi: float64 (bf16 values or -inf)."""
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    g = (gpu_bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    hidden = ~np.isfinite(ora)
    assert (gpu_bits[hidden] == NEG_INF_BF16_BITS).all(), f"{where}: hidden positions not bf16 -inf"
    vis = ~hidden
    gv, ov = g[vis], ora[vis]
    assert np.isfinite(gv).all(), f"{where}: non-finite visible score"
    _, e = np.frexp(np.abs(ov))
    e = np.where(ov == 0.0, -125, e)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    near = np.abs(gv - ov) <= 2 * ulp
    inside = (gv >= lo[vis]) & (gv <= hi[vis])
    ok = near | inside
    assert ok.all(), (f"{where}: {int((~ok).sum())} V4.1 scores beyond 2 ulp and outside the "
                      f"accumulation interval")
    return int((~near & inside).sum())


BACKWARD_REL = 2.0 ** -8 + 2.0 ** -11


def check_backward_one(got, name, ora, bound, where=""):
    """One gradient: got[name] float32 against the oracle's array and its (mag, amb)."""
    g = np.asarray(got[name], dtype=np.float64)
    assert g.shape == ora.shape, (name, g.shape, ora.shape)
    mag, amb = bound
    tol = BACKWARD_REL * mag + amb + 1e-6
    err = np.abs(g - ora)
    bad = ~(err <= tol)
    if bad.any():
        i = tuple(int(x) for x in np.argwhere(bad)[0])
        raise AssertionError(f"{where} {name}: {int(bad.sum())} of {bad.size} outside tolerance; first at {i}: "
                             f"got {g[i]!r} oracle {ora[i]!r} tol {tol[i]!r}")


def check_backward(got, grads, bounds, where=""):
    """got: dict name -> float32 array for "dq", "dk", "dw"; grads: the
    oracle's (dq, dk, dw); bounds: its with_bounds dict."""
    for name, ora in zip(("dq", "dk", "dw"), grads):
        check_backward_one(got, name, ora, bounds[name], where)

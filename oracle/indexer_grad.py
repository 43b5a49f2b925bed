"""Plain, slow, float64 oracle of the indexer's backward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module, and this module imports nothing from it.

What is computed, and from which passage of the pages:

* Page "deepseek_v4.kernels.tilelang_indexer", class ``V4IndexerFunction``:
  an autograd Function whose ``forward`` takes index_q [S,B,H,D], index_k
  [Skv,B,D], weights [S,B,H] (and topk_indices) and whose ``backward``
  receives ``grad_scores`` and ``grad_indices``.  The pages print no formula
  for the backward, so the oracle takes the plain reading: the gradient of
  the selected scores with respect to q, k and weights, by the chain rule on
  the forward definition (spec formula, as in ``indexer.py``)

      score[b,t,j] = sum_h w[t,b,h] * max(0, d[t,b,h,j]),
      d[t,b,h,j]   = q[t,b,h,:] . k[s,b,:],   s = idx[b,t,j] in [ks[t], ke[t]).

  With g = grad_scores[b,t,j] and m = 1[d > 0] (the ReLU's derivative, 0 at
  d = 0):

      dw[t,b,h] += g * max(0, d)
      dq[t,b,h,:] += g * w[t,b,h] * m * k[s,b,:]
      dk[s,b,:]   += g * w[t,b,h] * m * q[t,b,h,:]

  summed over every valid entry j (a key listed twice in a row contributes
  twice).  Entries whose index lies outside [ks, ke) carry the constant
  score -inf and contribute nothing, whatever their grad_scores value.  The
  indices are integers and get no gradient (grad_indices is not used).

Inputs follow ``indexer.py``: bfloat16 tensors as uint16 bit patterns,
float32 as float32, float64 used as it is.
"""

import numpy as np

from .indexer import _f64, _clamped_range


def _valid_entries(indices_row, lo, hi):
    idx = np.asarray(indices_row, dtype=np.int64)
    return (idx >= lo) & (idx < hi)


def indexer_backward(q, k, w, indices, grad_scores, ks, ke, with_bounds=False, rows=None):
    """dq [S,B,H,D], dk [Skv,B,D], dw [S,B,H] in float64.

    q [S,B,H,D], k [Skv,B,D], w [S,B,H]; indices and grad_scores [B,S,topk];
    ks, ke [S] shared by every batch element (``causal_ranges`` gives the
    causal ones).  With ``rows`` (query positions) only those queries are
    processed: their dq and dw are complete, other queries' stay 0, and dk
    holds only their contributions.

    With ``with_bounds`` also returns, for each output, a pair (mag, amb):

    * mag: the sum of the magnitudes of the terms that make up the output
      (the scale of the rounding error of a kernel that forms them in low
      precision and adds them in float32);
    * amb: the part of the output that comes from (head, key) pairs whose d
      lies within ``eps = 2 * D * 2**-24 * sum_i |q_i k_i|`` of 0, where a
      float32 dot product may take the ReLU's other branch; for such a pair
      the term of dq and dk may be present or absent, and the term of dw is at
      most that size.  For dw it also holds sum |g| * eps over every pair: eps
      bounds the error of a float32 dot product of D exact products summed in
      any order (at most D - 1 additions, each off by at most 2**-24 of the
      partial sum), and dw takes d itself, not only its sign.
    """
    S, B, H, D = q.shape
    n_kv = k.shape[0]
    indices = np.asarray(indices, dtype=np.int64)
    g_all = np.asarray(grad_scores, dtype=np.float64)
    dq = np.zeros((S, B, H, D))
    dk = np.zeros((n_kv, B, D))
    dw = np.zeros((S, B, H))
    if with_bounds:
        mag = {n: np.zeros_like(a) for n, a in (("dq", dq), ("dk", dk), ("dw", dw))}
        amb = {n: np.zeros_like(a) for n, a in (("dq", dq), ("dk", dk), ("dw", dw))}
    query_rows = range(S) if rows is None else [int(t) for t in rows]
    for b in range(B):
        kb = _f64(k[:, b, :])                               # [Skv, D]
        for t in query_rows:
            lo, hi = _clamped_range(ks, ke, t, n_kv)
            ok = _valid_entries(indices[b, t], lo, hi)
            if not ok.any():
                continue
            sel = indices[b, t][ok]                         # [m] key rows
            g = g_all[b, t][ok]                             # [m]
            ksel = kb[sel]                                  # [m, D]
            qt = _f64(q[t, b])                              # [H, D]
            wt = _f64(w[t, b])                              # [H]
            d = qt @ ksel.T                                 # [H, m]
            m = (d > 0).astype(np.float64)
            dw[t, b] = np.maximum(d, 0.0) @ g
            dq[t, b] = wt[:, None] * ((m * g[None, :]) @ ksel)
            contrib = g[:, None] * ((m * wt[:, None]).T @ qt)    # [m, D]
            np.add.at(dk[:, b, :], sel, contrib)
            if with_bounds:
                ag, aw = np.abs(g), np.abs(wt)
                eps = 2.0 * D * 2.0 ** -24 * (np.abs(qt) @ np.abs(ksel).T)      # [H, m]
                amb_pair = (np.abs(d) <= eps).astype(np.float64)
                mag["dw"][t, b] = np.abs(d) @ ag
                amb["dw"][t, b] = (amb_pair * np.abs(d)) @ ag + eps @ ag
                mag["dq"][t, b] = aw[:, None] * ((m * ag[None, :]) @ np.abs(ksel))
                amb["dq"][t, b] = aw[:, None] * ((amb_pair * ag[None, :]) @ np.abs(ksel))
                np.add.at(mag["dk"][:, b, :], sel, ag[:, None] * ((m * aw[:, None]).T @ np.abs(qt)))
                np.add.at(amb["dk"][:, b, :], sel, ag[:, None] * ((amb_pair * aw[:, None]).T @ np.abs(qt)))
    if with_bounds:
        return (dq, dk, dw), {n: (mag[n], amb[n]) for n in ("dq", "dk", "dw")}
    return dq, dk, dw

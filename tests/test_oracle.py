"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests needs a GPU.  Each pin is chosen so that a plausible
mistake in the oracle (a dropped ReLU, a wrong sign, a transposed operand, a
batch or head index mix-up, double rounding, a wrong tie rule) fails it.
"""

import heapq
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import checkers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    return -math.inf if x == "-inf" else float(x)


def _arr(nested):
    return np.vectorize(_num, otypes=[np.float64])(np.array(nested, dtype=object))


# ---------------------------------------------------------------- bf16 rounding

def test_rne_bf16_matches_torch_cast_on_float32_values():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    u[::4] = (u[::4] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)       # exact ties
    specials = np.array([0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000,
                         0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x7F800000,
                         0xFF800000, 0x3F808000, 0x3F818000, 0x00800000], dtype=np.uint32)
    u = np.concatenate([u, specials])
    finite_or_inf = (u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)
    finite_or_inf |= (u & np.uint32(0x007FFFFF)) == 0
    u = u[finite_or_inf]
    x32 = u.view(np.float32)
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(oracle.rne_bf16(x32.astype(np.float64)))
    assert np.array_equal(got, ref)


def test_rne_bf16_rounds_float64_directly_without_double_rounding():
    # 1 + 2**-8 is the midpoint between 1 and 1 + 2**-7.  A hair above it must
    # round up; rounding through float32 first would land on the midpoint and
    # then tie to even (down to 1).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.rne_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert oracle.rne_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert oracle.rne_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # subnormal spacing 2**-133; half of it ties to zero, 1.5 of it to 2
    assert oracle.rne_bf16(np.array([2.0 ** -134]))[0] == 0.0
    assert oracle.rne_bf16(np.array([3 * 2.0 ** -134]))[0] == 2.0 ** -132
    # overflow
    assert oracle.rne_bf16(np.array([2.0 ** 128 * (1 - 2.0 ** -9)]))[0] == math.inf
    assert oracle.rne_bf16(np.array([-(2.0 ** 128)]))[0] == -math.inf


def test_rne_bf16_golden_integer_ties():
    cases = {257.0: 256.0, 259.0: 260.0, 261.0: 260.0, 263.0: 264.0, -259.0: -260.0, 37.0: 37.0}
    for x, want in cases.items():
        assert oracle.rne_bf16(np.array([x]))[0] == want, x


def test_ulp_bf16():
    assert oracle.ulp_bf16(np.array([1.0]))[0] == 2.0 ** -7
    assert oracle.ulp_bf16(np.array([256.0]))[0] == 2.0
    assert oracle.ulp_bf16(np.array([300.0]))[0] == 2.0
    assert oracle.ulp_bf16(np.array([0.0]))[0] == 2.0 ** -133


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, size=10000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    assert np.array_equal(oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(bits)), bits)


# ---------------------------------------------------------------- causal range

def test_causal_ranges_golden():
    g = _load("causal_ranges.json")
    ks, ke = oracle.causal_ranges(10, 100, 4)
    assert list(ke) == g["ke_c4_first10"] and not ks.any()
    _, ke = oracle.causal_ranges(10, 1, 4)
    assert list(ke) == g["clamped_S10_Skv1_c4"]
    for n, want in g["valid_pairs_c4"].items():
        n = int(n)
        _, ke = oracle.causal_ranges(4 * n, n, 4)
        assert int(ke.sum()) == want


def test_causal_ranges_brute_force_small():
    for S in (1, 7, 33):
        for Skv in (1, 5, 16):
            for c in (1, 2, 3, 4):
                ks, ke = oracle.causal_ranges(S, Skv, c)
                for p in range(S):
                    visible = [s for s in range(Skv) if (s + 1) * c <= p + 1]
                    assert list(range(ks[p], ke[p])) == visible


# ---------------------------------------------------------------- V4 logits

def test_logits_handworked_example():
    g = _load("v4_handworked.json")
    q = np.array(g["q_SBHD"], dtype=np.float64)
    k = np.array(g["k_SBD"], dtype=np.float64)
    w = np.array(g["w_SBH"], dtype=np.float64)
    ks, ke = oracle.causal_ranges(q.shape[0], k.shape[0], g["compress_ratio"])
    assert list(ke) == g["ke"]
    got = oracle.indexer_logits(q, k, w, ks, ke)
    assert np.array_equal(got, _arr(g["logits_BSS"]))
    for tk in (1, 2):
        s, i = oracle.topk_select(got[0], ks, ke, tk)
        assert np.array_equal(i, np.array(g[f"topk{tk}_indices"][0]))
        assert np.array_equal(s, _arr(g[f"topk{tk}_scores"][0]))
    gi = np.array(g["gather_indices"])
    assert np.array_equal(oracle.topk_scores_gather(got, gi), _arr(g["gather_scores"]))


def _rand_case(seed, S=37, B=3, H=4, D=6, Skv=11, c=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, B, H, D))
    k = rng.standard_normal((Skv, B, D))
    w = rng.standard_normal((S, B, H))
    return q, k, w, oracle.causal_ranges(S, Skv, c)


def test_logits_relu_difference_is_a_gemv():
    # max(0,x) - max(0,-x) = x, so logits(q,k) - logits(q,-k) must equal
    # sum_h w_h (q_h . k) = k . (sum_h w_h q_h): a plain matrix-vector product
    # that involves neither a ReLU nor a per-head dot product.
    q, k, w, (ks, ke) = _rand_case(2)
    a = oracle.indexer_logits(q, k, w, ks, ke)
    b = oracle.indexer_logits(q, -k, w, ks, ke)
    S, B = q.shape[:2]
    for bb in range(B):
        u = np.einsum("th,thd->td", w[:, bb], q[:, bb])            # [S, D]
        gemv = u @ k[:, bb].T                                        # [S, Skv]
        for t in range(S):
            lo, hi = ks[t], ke[t]
            assert np.allclose(a[bb, t, lo:hi] - b[bb, t, lo:hi], gemv[t, lo:hi], rtol=1e-12, atol=1e-12)
            # sum gives sum_h w_h |q_h . k|, checked against a per-head loop with abs()
            absd = np.abs(q[t, bb] @ k[lo:hi, bb].T)                # [H, n]
            assert np.allclose(a[bb, t, lo:hi] + b[bb, t, lo:hi], w[t, bb] @ absd, rtol=1e-12, atol=1e-12)


def test_logits_nonnegative_operands_reduce_to_gemv():
    q, k, w, (ks, ke) = _rand_case(3)
    q, k = np.abs(q), np.abs(k)
    a = oracle.indexer_logits(q, k, w, ks, ke)
    for bb in range(q.shape[1]):
        gemv = np.einsum("th,thd->td", w[:, bb], q[:, bb]) @ k[:, bb].T
        fin = np.isfinite(a[bb])
        assert np.allclose(a[bb][fin], gemv[fin], rtol=1e-12, atol=1e-12)


def test_logits_all_nonpositive_dots_give_zero():
    q, k, w, (ks, ke) = _rand_case(4)
    a = oracle.indexer_logits(np.abs(q), -np.abs(k), w, ks, ke)
    fin = np.isfinite(a)
    assert fin.sum() > 0 and np.all(a[fin] == 0.0)


def test_logits_single_head_unit_weight_is_relu_of_qk():
    q, k, w, (ks, ke) = _rand_case(5, H=1)
    a = oracle.indexer_logits(q, k, np.ones_like(w), ks, ke)
    for bb in range(q.shape[1]):
        ref = np.maximum(q[:, bb, 0] @ k[:, bb].T, 0.0)
        fin = np.isfinite(a[bb])
        assert np.allclose(a[bb][fin], ref[fin], rtol=1e-12, atol=0)


def test_logits_batch_and_head_structure():
    q, k, w, (ks, ke) = _rand_case(6)
    a = oracle.indexer_logits(q, k, w, ks, ke)
    # swapping two batch elements swaps the outputs
    perm = np.array([2, 0, 1])
    b = oracle.indexer_logits(q[:, perm], k[:, perm], w[:, perm], ks, ke)
    assert np.array_equal(b, a[perm])
    # permuting heads of q and w together changes nothing (up to reassociation)
    hp = np.array([3, 1, 0, 2])
    c = oracle.indexer_logits(q[:, :, hp], k, w[:, :, hp], ks, ke)
    fin = np.isfinite(a)
    assert np.array_equal(np.isfinite(c), fin)
    assert np.allclose(c[fin], a[fin], rtol=1e-12, atol=1e-12)
    # scaling q by a power of two scales logits exactly
    d = oracle.indexer_logits(q * 8.0, k, w, ks, ke)
    assert np.array_equal(d[fin], 8.0 * a[fin])
    # a row of one query depends on that query only
    q2 = q.copy()
    q2[5] += 1.0
    e = oracle.indexer_logits(q2, k, w, ks, ke)
    rows = np.arange(q.shape[0]) != 5
    assert np.array_equal(e[:, rows], a[:, rows])


def test_logits_exact_inputs_match_rational_brute_force():
    inp = synth.v4_exact_inputs(batch=2, seqlen=24, seqlen_kv=6, heads=4, index_dim=8, seed=7)
    q, k, w = (synth.bits(inp[x]) for x in "qkw")
    ks, ke = oracle.causal_ranges(24, 6, 4)
    a = oracle.indexer_logits(q, k, w, ks, ke)
    qf, kf = oracle.bf16_bits_to_f64(q), oracle.bf16_bits_to_f64(k)
    for b in range(2):
        for t in range(24):
            for s in range(6):
                if s >= ke[t]:
                    assert a[b, t, s] == -math.inf
                    continue
                tot = Fraction(0)
                for h in range(4):
                    dot = sum(Fraction(qf[t, b, h, i]) * Fraction(kf[s, b, i]) for i in range(8))
                    tot += Fraction(float(w[t, b, h])) * max(Fraction(0), dot)
                assert Fraction(a[b, t, s]) == tot


def test_logits_given_ranges_and_clamping():
    q, k, w, _ = _rand_case(8, S=9, Skv=7)
    ks = np.array([0, 2, 3, 5, 0, 6, 1, 4, 0])
    ke = np.array([0, 5, 3, 7, 9, 7, 2, 4, 100])       # empty, normal, empty, tail, clamp ...
    a = oracle.indexer_logits(q, k, w, ks, ke)
    full = oracle.indexer_logits(q, k, w, np.zeros(9, int), np.full(9, 7))
    for t in range(9):
        lo, hi = min(ks[t], 7), min(ke[t], 7)
        for s in range(7):
            if lo <= s < hi:
                assert a[0, t, s] == full[0, t, s]
            else:
                assert a[0, t, s] == -math.inf


def test_logits_rows_and_magnitude():
    q, k, w, (ks, ke) = _rand_case(9)
    a, m = oracle.indexer_logits(q, k, w, ks, ke, with_magnitude=True)
    r, rm = oracle.indexer_logits_rows(q, k, w, 1, [30, 4, 17], ks, ke, with_magnitude=True)
    assert np.array_equal(r, a[1, [30, 4, 17]])
    assert np.array_equal(rm, m[1, [30, 4, 17]])
    assert (m >= np.abs(np.where(np.isfinite(a), a, 0))).all()


# ---------------------------------------------------------------- top-k

def test_topk_distinct_values_match_heapq():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((20, 50))
    ks = rng.integers(0, 20, size=20)
    ke = ks + rng.integers(0, 31, size=20)
    for tk in (1, 5, 17, 50):
        s, i = oracle.topk_select(x, ks, ke, tk)
        for r in range(20):
            items = [(x[r, j], -j) for j in range(ks[r], min(ke[r], 50))]
            best = sorted(-nj for _, nj in heapq.nlargest(tk, items))
            m = len(best)
            assert list(i[r, :m]) == best
            assert np.array_equal(s[r, :m], x[r, best])
            assert (i[r, m:] == -1).all() and (s[r, m:] == -math.inf).all()


def test_topk_ties_prefer_lower_index():
    x = np.zeros((3, 10))
    x[1, [2, 7]] = 1.0
    x[2] = [5, 1, 1, 1, 5, 1, 1, 1, 1, 1]
    ks, ke = np.zeros(3, int), np.full(3, 10)
    s, i = oracle.topk_select(x, ks, ke, 4)
    assert list(i[0]) == [0, 1, 2, 3]
    assert list(i[1]) == [0, 1, 2, 7]             # both 1.0s, then the lowest zeros
    assert list(i[2]) == [0, 1, 2, 4]


def test_topk_padding_and_empty_rows():
    x = np.arange(12, dtype=np.float64).reshape(2, 6)
    s, i = oracle.topk_select(x, np.array([0, 3]), np.array([0, 5]), 4)
    assert list(i[0]) == [-1] * 4 and (s[0] == -math.inf).all()
    assert list(i[1]) == [3, 4, -1, -1] and list(s[1][:2]) == [9.0, 10.0]


def test_topk_visible_bf16_brute_force():
    # Rows drawn from a handful of bf16 values (heavy ties, both zeros) with
    # hidden keys; the expected selection is a plain Python sort.
    rng = np.random.default_rng(12)
    pool = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4000, 0x3F00, 0xC040], dtype=np.uint16)
    value = {0x3F80: 1.0, 0xBF80: -1.0, 0x0000: 0.0, 0x8000: 0.0, 0x4000: 2.0, 0x3F00: 0.5, 0xC040: -3.0}
    bits = pool[rng.integers(0, len(pool), size=(30, 40))]
    bits[rng.random((30, 40)) < 0.35] = 0xFF80          # hidden
    bits[5] = 0xFF80                                    # a row with nothing visible
    for tk in (1, 3, 11, 40):
        got_b, got_i = oracle.topk_select_visible_bf16(bits, tk)
        for r in range(30):
            vis = [j for j in range(40) if bits[r, j] != 0xFF80]
            best = sorted(sorted(vis, key=lambda j: (-value[int(bits[r, j])], j))[:tk])
            m = len(best)
            assert list(got_i[r, :m]) == best, (tk, r)
            assert list(got_b[r, :m]) == [bits[r, j] for j in best]
            assert (got_i[r, m:] == -1).all() and (got_b[r, m:] == 0xFF80).all()


def test_gather_brute_force():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((2, 5, 9))
    idx = rng.integers(-3, 12, size=(2, 5, 4))
    got = oracle.topk_scores_gather(lg, idx)
    for b in range(2):
        for t in range(5):
            for j in range(4):
                v = idx[b, t, j]
                want = lg[b, t, v] if 0 <= v < 9 else -math.inf
                assert got[b, t, j] == want


# ---------------------------------------------------------------- V4.1

def test_v41_golden_rounding_cases():
    g = _load("v41_rounding.json")
    D = g["index_dim"]
    for case in g["cases"]:
        H = len(case["heads"])
        qv = np.zeros((1, 1, H, D))
        wv = np.zeros((1, 1, H))
        for h, hd in enumerate(case["heads"]):
            qv[0, 0, h, :len(hd["q"])] = hd["q"]
            wv[0, 0, h] = hd["w"]
        kv = np.zeros((1, 1, D))
        kv[0, 0, :len(case["k"])] = case["k"]
        allowed = np.array([[[case["allowed"]]]])
        out = oracle.indexer_scores_v41(qv, kv, wv, allowed)[0, 0, 0]
        assert out == _num(case["out"]), case["name"]
        assert int(oracle.f64_to_bf16_bits(np.array([out]))[0]) == int(case["out_bits"], 16), case["name"]


def test_v41_reduces_to_v4_when_every_step_is_representable():
    # q,k in {-1,0,1} with D=16 give integer dots |d| <= 16; w = +-2**-j with
    # j <= 2 gives products that are multiples of 1/4 of magnitude <= 16, and
    # two heads sum to at most 32 in steps of 1/4: every intermediate needs at
    # most 8 significant bits, so every BF16 rounding is exact and V4.1 must
    # equal the V4 formula on the visible positions.
    rng = np.random.default_rng(12)
    B, L, G, H, D = 2, 12, 5, 2, 16
    q = rng.integers(-1, 2, size=(B, L, H, D)).astype(np.float64)
    k = rng.integers(-1, 2, size=(B, G, D)).astype(np.float64)
    w = rng.choice([-1.0, -0.5, -0.25, 0.25, 0.5, 1.0], size=(B, L, H))
    allowed = rng.random((B, L, G)) < 0.6
    got = oracle.indexer_scores_v41(q, k, w, allowed)
    v4 = oracle.indexer_logits(np.transpose(q, (1, 0, 2, 3)), np.transpose(k, (1, 0, 2)),
                               np.transpose(w, (1, 0, 2)), np.zeros(L, int), np.full(L, G))
    assert np.array_equal(got[allowed], v4[allowed])
    assert (got[~allowed] == -math.inf).all()


def test_v41_rounding_changes_results_against_unrounded_form():
    # On random inputs the rounded path must differ from the plain V4 value
    # by more than float noise somewhere (a missing rounding step would not).
    inp = synth.v41_exact_inputs(batch=1, local_sequence=8, global_compressed=16, heads=8,
                                 index_dim=32, seed=13, density=1.0)
    q, k, w, al = (synth.bits(inp[x]) for x in ("queries", "keys", "weights", "allowed"))
    got = oracle.indexer_scores_v41(q, k, w, al)
    qf, kf, wf = (oracle.bf16_bits_to_f64(x) for x in (q, k, w))
    v4 = oracle.indexer_logits(np.transpose(qf, (1, 0, 2, 3)), np.transpose(kf, (1, 0, 2)),
                               np.transpose(wf, (1, 0, 2)), np.zeros(8, int), np.full(8, 16))
    assert np.array_equal(got, oracle.rne_bf16(got))              # outputs are bf16 values
    assert not np.array_equal(got, v4)


def test_v41_bounds_contain_oracle_and_are_tight():
    inp = synth.v41_inputs(batch=1, local_sequence=64, global_compressed=16, heads=16,
                           index_dim=32, seed=14, doc_min=8, doc_max=40)
    q, k, w, al = (synth.bits(inp[x]) for x in ("queries", "keys", "weights", "allowed"))
    o = oracle.indexer_scores_v41(q, k, w, al)[0]
    lo, hi = oracle.indexer_scores_v41_bounds_rows(q, k, w, al, 0, np.arange(64))
    vis = np.isfinite(o)
    assert vis.sum() > 50
    assert (lo[vis] <= o[vis]).all() and (o[vis] <= hi[vis]).all()
    _, e = np.frexp(np.abs(o[vis]))
    width_ulps = (hi[vis] - lo[vis]) / np.ldexp(1.0, np.maximum(e - 8, -133))
    assert np.median(width_ulps) <= 1.0
    assert (lo[~vis] == -math.inf).all() and (hi[~vis] == -math.inf).all()


def test_v41_inputs_mask_structure():
    inp = synth.v41_inputs(batch=1, local_sequence=300, global_compressed=75, heads=2,
                           index_dim=16, seed=15, doc_min=20, doc_max=90)
    al = inp["allowed"][0].numpy()
    for t in range(300):
        vis = np.nonzero(al[t])[0]
        if len(vis):
            assert vis.max() < (t + 1) // 4
            assert (np.diff(vis) == 1).all()      # one contiguous run of groups per query


# ---------------------------------------------------------------- checkers

def test_topk_checker_accepts_oracle_and_rejects_planted_errors():
    inp = synth.v4_inputs(batch=1, seqlen=64, seqlen_kv=16, heads=8, index_dim=32, seed=16)
    q, k, w = (synth.bits(inp[x]) for x in "qkw")
    ks, ke = oracle.causal_ranges(64, 16, 4)
    lg, mag = oracle.indexer_logits(q, k, w, ks, ke, with_magnitude=True)
    s, i = oracle.topk_select(lg[0], ks, ke, 4)
    checkers.check_topk_rows(s.astype(np.float32), i, lg[0], mag[0], ks, ke, 4)
    bad_i = i.copy()
    r = 40
    worst = int(np.argmin(np.where(np.isfinite(lg[0, r]), lg[0, r], np.inf)))
    bad_i[r, 0] = worst
    bad_i[r] = np.sort(bad_i[r])
    with pytest.raises(AssertionError):
        checkers.check_topk_rows(s.astype(np.float32), bad_i, lg[0], mag[0], ks, ke, 4)
    bad_s = s.copy()
    bad_s[r, 1] += 0.01
    with pytest.raises(AssertionError):
        checkers.check_topk_rows(bad_s.astype(np.float32), i, lg[0], mag[0], ks, ke, 4)
    bad_pad = i.copy()
    bad_pad[0, 0] = 0
    with pytest.raises(AssertionError):
        checkers.check_topk_rows(s.astype(np.float32), bad_pad, lg[0], mag[0], ks, ke, 4)


# ---------------------------------------------------------------------------
# Backward: gradients of the selected scores with respect to q, k and w
# ---------------------------------------------------------------------------

def _bw_case(seed, S=6, B=2, Skv=9, H=4, D=8, topk=5, ratio=1, nonneg=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, B, H, D))
    k = rng.standard_normal((Skv, B, D))
    w = rng.standard_normal((S, B, H))
    if nonneg:
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    ks, ke = oracle.causal_ranges(S, Skv, ratio)
    idx = rng.integers(-2, Skv + 2, size=(B, S, topk))     # -2, -1, Skv, Skv+1 are invalid
    g = rng.standard_normal((B, S, topk))
    return q, k, w, ks, ke, idx, g


def _selected_loss(q, k, w, idx, g, ks, ke):
    """sum of g * score over the valid entries, with the scores taken from the
    forward oracle (full logits, then the gather at the indices)."""
    sc = oracle.topk_scores_gather(oracle.indexer_logits(q, k, w, ks, ke), idx)
    return float(np.sum(np.where(np.isfinite(sc), sc * g, 0.0)))


def _valid_mask(k, idx, ks, ke):
    S = len(ks)
    t = np.arange(S)[None, :, None]
    lo = np.clip(np.asarray(ks)[t], 0, k.shape[0])
    hi = np.clip(np.asarray(ke)[t], 0, k.shape[0])
    return (idx >= lo) & (idx < hi)


@pytest.mark.parametrize("ratio", [1, 2])
def test_backward_matches_central_differences_of_the_forward(ratio):
    # The loss is piecewise linear along any direction in q, k or w (d is
    # linear in each, the ReLU piecewise linear), so a central difference
    # with a small step equals the directional derivative up to rounding.
    q, k, w, ks, ke, idx, g = _bw_case(10 + ratio, ratio=ratio)
    grads = dict(zip("qkw", oracle.indexer_backward(q, k, w, idx, g, ks, ke)))
    rng = np.random.default_rng(7)
    eps = 1e-6
    for name in "qkw":
        for _ in range(3):
            v = rng.standard_normal(grads[name].shape)

            def loss(step):
                args = {"q": q, "k": k, "w": w}
                args[name] = args[name] + step * v
                return _selected_loss(args["q"], args["k"], args["w"], idx, g, ks, ke)

            fd = (loss(eps) - loss(-eps)) / (2 * eps)
            assert fd == pytest.approx(float(np.sum(grads[name] * v)), rel=1e-6, abs=1e-8), name


def test_backward_coordinate_differences():
    q, k, w, ks, ke, idx, g = _bw_case(20, S=4, Skv=5, H=2, D=4, topk=4)
    dq, dk, dw = oracle.indexer_backward(q, k, w, idx, g, ks, ke)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("w", w, dw)):
        for pos in np.ndindex(x.shape):
            e = np.zeros_like(x)
            e[pos] = eps
            args_p = {"q": q, "k": k, "w": w}
            args_m = dict(args_p)
            args_p[name], args_m[name] = x + e, x - e
            fd = (_selected_loss(args_p["q"], args_p["k"], args_p["w"], idx, g, ks, ke)
                  - _selected_loss(args_m["q"], args_m["k"], args_m["w"], idx, g, ks, ke)) / (2 * eps)
            assert fd == pytest.approx(grad[pos], rel=1e-6, abs=1e-8), (name, pos)


def test_backward_nonnegative_operands_closed_form():
    # q, k > 0 puts every d above 0: the score is k_s . u with u = sum_h w_h q_h,
    # so dq_h = w_h sum_j g_j k_j, dk_s = sum_(t,j) g_j u_t, dw_h = sum_j g_j q_h . k_j.
    q, k, w, ks, ke, idx, g = _bw_case(30, nonneg=True)
    dq, dk, dw = oracle.indexer_backward(q, k, w, idx, g, ks, ke)
    S, B, H, D = q.shape
    e_dq, e_dk, e_dw = np.zeros_like(q), np.zeros_like(k), np.zeros_like(w)
    for b in range(B):
        for t in range(S):
            u = w[t, b] @ q[t, b]
            for j in range(idx.shape[2]):
                s = idx[b, t, j]
                if not (ks[t] <= s < min(ke[t], k.shape[0])):
                    continue
                e_dq[t, b] += g[b, t, j] * np.outer(w[t, b], k[s, b])
                e_dk[s, b] += g[b, t, j] * u
                e_dw[t, b] += g[b, t, j] * (q[t, b] @ k[s, b])
    np.testing.assert_allclose(dq, e_dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, e_dk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, e_dw, rtol=1e-12, atol=1e-12)


def test_backward_all_nonpositive_dots_give_no_q_k_gradient():
    # k = -q_0-like signs: with q >= 0 and k <= 0 every d <= 0, so the ReLU
    # is flat: every gradient is zero.
    q, k, w, ks, ke, idx, g = _bw_case(31, nonneg=True)
    dq, dk, dw = oracle.indexer_backward(q, -k, w, idx, g, ks, ke)
    assert not dq.any() and not dk.any() and not dw.any()


def test_backward_ignores_invalid_entries_and_is_linear_in_the_gradient():
    q, k, w, ks, ke, idx, g = _bw_case(40)
    valid = _valid_mask(k, idx, ks, ke)
    assert valid.any() and (~valid).any()
    base = oracle.indexer_backward(q, k, w, idx, g, ks, ke)
    noisy = np.where(valid, g, 1e6)
    for a, b in zip(base, oracle.indexer_backward(q, k, w, idx, noisy, ks, ke)):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(base, oracle.indexer_backward(q, k, w, idx, 2.0 * g, ks, ke)):
        np.testing.assert_allclose(b, 2.0 * a, rtol=1e-13, atol=1e-13)
    for a in oracle.indexer_backward(q, k, w, idx, np.zeros_like(g), ks, ke):
        assert not a.any()


def test_backward_duplicate_index_counts_twice():
    q, k, w, ks, ke, _, _ = _bw_case(50, S=5, Skv=5, topk=3)
    B = q.shape[1]
    idx = np.full((B, 5, 3), -1)
    g = np.zeros((B, 5, 3))
    idx[1, 4, :2] = 3
    g[1, 4, :2] = (0.75, -2.0)
    one = np.full_like(idx, -1)
    g1 = np.zeros_like(g)
    one[1, 4, 2] = 3
    g1[1, 4, 2] = -1.25
    for a, b in zip(oracle.indexer_backward(q, k, w, idx, g, ks, ke),
                    oracle.indexer_backward(q, k, w, one, g1, ks, ke)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_backward_bounds_contain_values():
    q, k, w, ks, ke, idx, g = _bw_case(60)
    grads, bounds = oracle.indexer_backward(q, k, w, idx, g, ks, ke, with_bounds=True)
    for name, x in zip(("dq", "dk", "dw"), grads):
        mag, amb = bounds[name]
        assert np.all(np.abs(x) <= mag * (1 + 1e-12) + 1e-300)
        assert np.all(amb >= 0)
        if name != "dw":
            assert np.all(amb <= mag + 1e-300)
    # Only near-zero dot products count as ambiguous: none here, so dq and dk
    # have no ambiguous part and dw's is the dot-product error bound alone,
    # far below its magnitude.
    assert not bounds["dq"][1].any() and not bounds["dk"][1].any()
    assert np.all(bounds["dw"][1] <= 1e-3 * bounds["dw"][0] + 1e-300)
    for a, b in zip(grads, oracle.indexer_backward(q, k, w, idx, g, ks, ke)):
        np.testing.assert_array_equal(a, b)


def test_backward_bounds_flag_zero_dot_products():
    # A key orthogonal to one head's query: d = 0 exactly, which a float32
    # dot product may place on either side of 0.
    q, k, w, ks, ke, idx, g = _bw_case(61, S=3, B=1, Skv=3, H=2, D=4, topk=2, nonneg=True)
    q[2, 0, 1] = (1.0, -1.0, 0.0, 0.0)
    k[1, 0] = (2.0, 2.0, 5.0, 1.0)
    idx[0, 2] = (1, -1)
    _, bounds = oracle.indexer_backward(q, k, w, idx, g, ks, ke, with_bounds=True)
    amb_dq = bounds["dq"][1]
    assert amb_dq[2, 0, 1].any() and not amb_dq[2, 0, 0].any()


def test_backward_checker_accepts_bf16_rounding_and_rejects_planted_errors():
    q, k, w, ks, ke, idx, g = _bw_case(70, S=8, Skv=10, H=8, D=16, topk=6)
    grads, bounds = oracle.indexer_backward(q, k, w, idx, g, ks, ke, with_bounds=True)
    names = ("dq", "dk", "dw")
    checkers.check_backward(dict(zip(names, grads)), grads, bounds)
    # One bf16 rounding per term passes: g rounded for dq; g * w_h rounded
    # for dk (q exact), as a bf16 autograd graph of the forward rounds them.
    g16 = oracle.rne_bf16(g)
    dq16 = oracle.indexer_backward(q, k, w, idx, g16, ks, ke)[0]
    checkers.check_backward({"dq": dq16, "dk": grads[1], "dw": grads[2]}, grads, bounds)
    S, B, H, D = q.shape

    def dk_rounded(two_roundings):
        out = np.zeros_like(k)
        for b in range(B):
            for t in range(S):
                for j in range(idx.shape[2]):
                    s_ = idx[b, t, j]
                    if not (ks[t] <= s_ < min(ke[t], k.shape[0])):
                        continue
                    m = (q[t, b] @ k[s_, b] > 0).astype(np.float64)
                    if two_roundings:     # bf16(g) * bf16(w q): two roundings per term
                        wq = oracle.rne_bf16(w[t, b][:, None] * q[t, b])
                        out[s_, b] += oracle.rne_bf16(g[b, t, j]) * (m @ wq)
                    else:                 # bf16(g w_h) * q: one rounding per term
                        out[s_, b] += (m * oracle.rne_bf16(g[b, t, j] * w[t, b])) @ q[t, b]
        return out
    checkers.check_backward({"dq": grads[0], "dk": dk_rounded(False), "dw": grads[2]}, grads, bounds)
    # The rule tells one rounding per term from two: a single term whose
    # factors g and w q each lie just above a bf16 rounding midpoint (1 + a,
    # a = 2**-8 + 2**-12, rounds up to 1 + 2**-7, off by 0.36%).  Rounding the
    # product g * w once stays within 2**-8; rounding g and w q separately is
    # off by 0.73% and fails.
    a = 2.0 ** -8 + 2.0 ** -12
    one = np.ones((1, 1, 1, 1))
    q1, k1, w1 = one.copy(), np.ones((1, 1, 1)), np.full((1, 1, 1), 1.0 + a)
    g1 = np.full((1, 1, 1), 1.0 + a)
    idx1 = np.zeros((1, 1, 1), dtype=np.int64)
    ks1, ke1 = np.array([0]), np.array([1])
    gr1, bd1 = oracle.indexer_backward(q1, k1, w1, idx1, g1, ks1, ke1, with_bounds=True)
    single = oracle.rne_bf16((1.0 + a) * (1.0 + a)) * np.ones((1, 1, 1))
    double = oracle.rne_bf16(1.0 + a) * oracle.rne_bf16((1.0 + a) * 1.0) * np.ones((1, 1, 1))
    assert abs(double[0, 0, 0] / gr1[1][0, 0, 0] - 1.0) > 0.007
    checkers.check_backward({"dq": gr1[0], "dk": single, "dw": gr1[2]}, gr1, bd1)
    with pytest.raises(AssertionError):
        checkers.check_backward({"dq": gr1[0], "dk": double, "dw": gr1[2]}, gr1, bd1)
    # Planted mistakes in the oracle's arithmetic are caught.
    planted = {
        "dq without w": oracle.indexer_backward(q, k, np.ones_like(w), idx, g, ks, ke)[0],
        "dq with the ReLU mask dropped": oracle.indexer_backward(np.abs(q), np.abs(k), w, idx, g, ks, ke)[0],
        "dq with the sign of g flipped": -grads[0],
    }
    for what, bad in planted.items():
        with pytest.raises(AssertionError):
            checkers.check_backward({"dq": bad, "dk": grads[1], "dw": grads[2]}, grads, bounds)
    with pytest.raises(AssertionError):
        checkers.check_backward({"dq": grads[0], "dk": grads[1][::-1].copy(), "dw": grads[2]}, grads, bounds)
    with pytest.raises(AssertionError):
        checkers.check_backward({"dq": grads[0], "dk": grads[1], "dw": grads[2] * 1.01}, grads, bounds)


def test_backward_rows_subset_matches_full():
    q, k, w, ks, ke, idx, g = _bw_case(80, S=7)
    full = oracle.indexer_backward(q, k, w, idx, g, ks, ke)
    rows = [1, 4, 6]
    part = oracle.indexer_backward(q, k, w, idx, g, ks, ke, rows=rows)
    np.testing.assert_array_equal(part[0][rows], full[0][rows])
    np.testing.assert_array_equal(part[2][rows], full[2][rows])
    others = [t for t in range(7) if t not in rows]
    assert not part[0][others].any() and not part[2][others].any()
    g_rows = np.zeros_like(g)
    g_rows[:, rows] = g[:, rows]
    np.testing.assert_allclose(part[1], oracle.indexer_backward(q, k, w, idx, g_rows, ks, ke)[1], rtol=1e-13,
                               atol=1e-13)

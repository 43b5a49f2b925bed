"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input comes from the seeded generators in synth/; the oracle sees the
same bits.  Small cases are compared in full, the 32K/131K/V4.1 workloads on
stratified row samples.  Tolerances are those of tests/checkers.py.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_lightning_bf16_amd as lx
from tests import checkers

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.to(DEV)


def v4_case(B, S, Skv, H, D, seed, exact=False, heavy_fraction=0.0):
    gen = synth.v4_exact_inputs if exact else synth.v4_inputs
    kw = dict(batch=B, seqlen=S, seqlen_kv=Skv, heads=H, index_dim=D, seed=seed)
    if heavy_fraction:
        kw["heavy_fraction"] = heavy_fraction
    inp = gen(**kw)
    return inp, {x: synth.bits(inp[x]) for x in "qkw"}


def ranges(S, Skv, c, ks=None, ke=None):
    if ks is None:
        return oracle.causal_ranges(S, Skv, c)
    return ks.cpu().numpy().astype(np.int64), ke.cpu().numpy().astype(np.int64)


# ------------------------------------------------------------------ V4 logits

@pytest.mark.parametrize("H,D,B,S,Skv,c", [
    (64, 128, 1, 256, 64, 4),       # tiny workload shape
    (64, 128, 3, 333, 100, 3),      # ragged tail in queries and keys
    (128, 256, 2, 70, 40, 2),
    (64, 48, 1, 129, 33, 4),        # index_dim padded inside the kernel
    (32, 64, 2, 90, 70, 1),
    (16, 128, 1, 77, 150, 1),
    (8, 32, 2, 40, 50, 1),
    (4, 16, 1, 61, 70, 1),
    (2, 64, 1, 50, 45, 1),
    (1, 128, 2, 70, 66, 1),
])
def test_logits_match_oracle(H, D, B, S, Skv, c):
    log(f"logits H={H} D={D} B={B} S={S} Skv={Skv} c={c}")
    inp, nb = v4_case(B, S, Skv, H, D, seed=100 + H + D)
    got = lx.indexer_logits(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), c).cpu().numpy()
    ks, ke = ranges(S, Skv, c)
    ora, mag = oracle.indexer_logits(nb["q"], nb["k"], nb["w"], ks, ke, with_magnitude=True)
    checkers.check_logits(got, ora, mag, f"H={H} D={D}")


def test_logits_exact_inputs_are_bitwise_equal():
    B, S, Skv, H, D, c = 2, 300, 75, 64, 128, 4
    inp, nb = v4_case(B, S, Skv, H, D, seed=5, exact=True)
    got = lx.indexer_logits(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), c).cpu().numpy()
    ks, ke = ranges(S, Skv, c)
    ora = oracle.indexer_logits(nb["q"], nb["k"], nb["w"], ks, ke)
    assert np.array_equal(got.astype(np.float64), ora)


def test_logits_given_ranges():
    B, S, Skv, H, D = 2, 200, 150, 64, 128
    inp, nb = v4_case(B, S, Skv, H, D, seed=6)
    g = torch.Generator().manual_seed(7)
    ks = torch.randint(-5, 160, (S,), generator=g, dtype=torch.int32)
    ke = ks + torch.randint(-10, 120, (S,), generator=g, dtype=torch.int32)
    ke[::17] = 10_000                                   # clamped to Skv
    got = lx.indexer_logits(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), 1, dev(ks), dev(ke)).cpu().numpy()
    ksn, ken = ranges(S, Skv, 1, ks, ke)
    ora, mag = oracle.indexer_logits(nb["q"], nb["k"], nb["w"], ksn, ken, with_magnitude=True)
    checkers.check_logits(got, ora, mag, "given ranges")


def test_logits_4k_workload():
    cfg = synth.WORKLOADS["4k"]
    log("4k logits")
    inp, nb = v4_case(cfg["batch"], cfg["seqlen"], cfg["seqlen_kv"], cfg["heads"], cfg["index_dim"], cfg["seed"])
    got = lx.indexer_logits(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), cfg["compress_ratio"]).cpu().numpy()
    ks, ke = oracle.causal_ranges(cfg["seqlen"], cfg["seqlen_kv"], cfg["compress_ratio"])
    ora, mag = oracle.indexer_logits(nb["q"], nb["k"], nb["w"], ks, ke, with_magnitude=True)
    checkers.check_logits(got, ora, mag, "4k")


def test_logits_leave_memory_around_the_output_untouched():
    B, S, Skv, H, D, c = 1, 64, 30, 64, 128, 4
    inp, _ = v4_case(B, S, Skv, H, D, seed=8)
    n = B * S * Skv
    buf = torch.full((n + 2048,), 12345.0, dtype=torch.float32, device=DEV)
    out = buf[1024:1024 + n].view(B, S, Skv)
    lx.indexer_logits(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), c, out=out)
    torch.cuda.synchronize()
    assert bool((buf[:1024] == 12345.0).all()) and bool((buf[1024 + n:] == 12345.0).all())


@pytest.mark.parametrize("H,D,B,S,Skv,c,given", [
    (64, 128, 1, 256, 64, 4, False),
    (64, 128, 3, 333, 100, 3, False),
    (8, 32, 2, 40, 50, 1, False),
    (4, 16, 1, 61, 70, 1, False),       # heads < 8: per-slot stores of the lane halves
    (1, 128, 2, 70, 66, 1, True),
    (64, 128, 2, 200, 150, 1, True),
    (128, 256, 1, 90, 300, 1, True),
])
def test_visible_logits_equal_full_logits_inside_the_ranges(H, D, B, S, Skv, c, given):
    inp, _ = v4_case(B, S, Skv, H, D, seed=31)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    ks = ke = None
    if given:
        g = torch.Generator().manual_seed(32)
        ks = torch.randint(-5, Skv + 10, (S,), generator=g, dtype=torch.int32)
        ke = ks + torch.randint(-10, Skv, (S,), generator=g, dtype=torch.int32)
        ke[::13] = 10_000
        ks, ke = dev(ks), dev(ke)
    full_d = lx.indexer_logits(q, k, w, c, ks, ke)
    # NaN where nothing is written: a reader of a hidden position would see it
    out = torch.full((B, S, Skv), float("nan"), dtype=torch.float32, device=DEV)
    vis_d = lx.indexer_logits(q, k, w, c, ks, ke, out=out, visible_only=True)
    full, vis = full_d.cpu().numpy(), vis_d.cpu().numpy()
    lo, hi = ranges(S, Skv, c, ks, ke)
    key = np.arange(Skv)
    inside = (key[None, :] >= np.maximum(lo, 0)[:, None]) & (key[None, :] < np.minimum(hi, Skv)[:, None])
    inside = np.broadcast_to(inside, vis.shape)
    assert np.array_equal(vis.view(np.uint32)[inside], full.view(np.uint32)[inside])
    rest = vis[~inside]
    assert bool(np.all(np.isnan(rest) | (rest == -np.inf)))
    # the row top-k over either buffer, with the same ranges
    tk = min(16, Skv)
    sc_f, ix_f = lx.topk_from_logits(full_d, c, tk, ks, ke)
    sc_v, ix_v = lx.topk_from_logits(vis_d, c, tk, ks, ke)
    assert torch.equal(ix_v, ix_f) and torch.equal(sc_v.view(torch.int32), sc_f.view(torch.int32))


def test_topk_over_visible_logits_equals_the_full_route():
    cfg = synth.WORKLOADS["4k"]
    log("4k top-k over visible logits")
    B, S, Skv, tk = cfg["batch"], cfg["seqlen"], cfg["seqlen_kv"], cfg["topk"]
    inp, _ = v4_case(B, S, Skv, 64, 128, cfg["seed"])
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    sc_f, ix_f = lx.topk_from_logits(lx.indexer_logits(q, k, w, 4), 4, tk)
    out = torch.full((B, S, Skv), float("nan"), dtype=torch.float32, device=DEV)
    sc_v, ix_v = lx.topk_from_logits(lx.indexer_logits(q, k, w, 4, out=out, visible_only=True), 4, tk)
    assert torch.equal(ix_v, ix_f) and torch.equal(sc_v.view(torch.int32), sc_f.view(torch.int32))


# ------------------------------------------------------------------ top-k

def _check_topk_vs_oracle(sc, ix, nb, b, rows, ks, ke, topk, tag):
    ora, mag = oracle.indexer_logits_rows(nb["q"], nb["k"], nb["w"], b, rows, ks, ke, with_magnitude=True)
    return checkers.check_topk_rows(sc, ix, ora, mag, ks[rows], ke[rows], topk, tag)


def _selection_of(logits_np, ks, ke, topk):
    """The oracle's selection applied to the kernel's own fp32 logits."""
    s, i = oracle.topk_select(logits_np.astype(np.float64), ks, ke, topk)
    return s, i


@pytest.mark.parametrize("topk", [1, 5, 16, 40, 64])
def test_topk_tiny_workload_bitwise_on_kernel_logits(topk):
    cfg = synth.WORKLOADS["tiny"]
    inp, nb = v4_case(1, cfg["seqlen"], cfg["seqlen_kv"], 64, 128, cfg["seed"])
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    logits = lx.indexer_logits(q, k, w, 4)
    sc_m, ix_m = lx.topk_from_logits(logits, 4, topk)
    sc_f, ix_f = lx.topk(q, k, w, 4, topk)
    lg = logits.cpu().numpy()
    ks, ke = oracle.causal_ranges(cfg["seqlen"], cfg["seqlen_kv"], 4)
    want_s, want_i = _selection_of(lg[0], ks, ke, topk)
    for name, sc, ix in (("materialized", sc_m, ix_m), ("fused", sc_f, ix_f)):
        sc, ix = sc.cpu().numpy(), ix.cpu().numpy()
        assert np.array_equal(ix[0], want_i), name
        assert np.array_equal(sc[0].astype(np.float64), want_s), name
    _check_topk_vs_oracle(sc_f.cpu().numpy()[0], ix_f.cpu().numpy()[0], nb, 0, np.arange(cfg["seqlen"]),
                          ks, ke, topk, "tiny fused")


def test_topk_4k_workload_fused_and_materialized():
    cfg = synth.WORKLOADS["4k"]
    log("4k top-k")
    B, S, Skv, tk = cfg["batch"], cfg["seqlen"], cfg["seqlen_kv"], cfg["topk"]
    inp, nb = v4_case(B, S, Skv, 64, 128, cfg["seed"])
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    logits = lx.indexer_logits(q, k, w, 4)
    sc_m, ix_m = lx.topk_from_logits(logits, 4, tk)
    sc_f, ix_f = lx.topk(q, k, w, 4, tk)
    assert torch.equal(ix_m, ix_f) and torch.equal(sc_m, sc_f)
    ks, ke = oracle.causal_ranges(S, Skv, 4)
    lg = logits.cpu().numpy()
    sc, ix = sc_m.cpu().numpy(), ix_m.cpu().numpy()
    rows = np.arange(0, S, 7)
    for b in range(B):
        want_s, want_i = _selection_of(lg[b][rows], ks[rows], ke[rows], tk)
        assert np.array_equal(ix[b][rows], want_i)
        exact = _check_topk_vs_oracle(sc[b][rows], ix[b][rows], nb, b, rows, ks, ke, tk, f"4k b={b}")
        log(f"  batch {b}: rows with a forced exact set: {exact}/{len(rows)}")


def test_topk_ties_and_padding_bitwise():
    # scores drawn from a handful of values: heavy ties at every threshold
    g = torch.Generator().manual_seed(9)
    B, S, Skv = 2, 97, 300
    lg = (torch.randint(0, 6, (B, S, Skv), generator=g).float() - 2.0) * 0.5
    lg[:, :, 7] = -0.0                                   # signed zeros tie with +0
    ks = torch.randint(0, 40, (S,), generator=g, dtype=torch.int32)
    ke = ks + torch.randint(-3, 280, (S,), generator=g, dtype=torch.int32)
    for tk in (1, 3, 50, 128, 300):
        sc, ix = lx.topk_from_logits(dev(lg), 1, tk, dev(ks), dev(ke))
        sc, ix = sc.cpu().numpy(), ix.cpu().numpy()
        for b in range(B):
            want_s, want_i = oracle.topk_select(lg[b].numpy().astype(np.float64), ks.numpy(), ke.numpy(), tk)
            assert np.array_equal(ix[b], want_i), tk
            assert np.array_equal(sc[b].astype(np.float64), want_s), tk


@pytest.mark.parametrize("Skv", [20000, 40000])
def test_topk_long_rows_from_logits(Skv):
    # rows of the sixteen-wave register kernel (up to 32768 keys) and of the
    # radix kernel that re-reads the row (longer)
    g = torch.Generator().manual_seed(10)
    B, S, tk = 1, 12, 700
    step = Skv // 11
    lg = torch.randn(B, S, Skv, generator=g)
    sc, ix = lx.topk_from_logits(dev(lg), 1, tk, dev(torch.zeros(S, dtype=torch.int32)),
                                 dev(torch.arange(S, dtype=torch.int32) * step))
    want_s, want_i = oracle.topk_select(lg[0].numpy().astype(np.float64), np.zeros(S, int), np.arange(S) * step, tk)
    assert np.array_equal(ix.cpu().numpy()[0], want_i)
    assert np.array_equal(sc.cpu().numpy()[0].astype(np.float64), want_s)


def test_topk_causal_long_rows_across_the_kernel_split():
    # Causal rows of 8193..32768 keys: those of at most 16384 keys go to the
    # eight-wave kernel, longer ones to the sixteen-wave kernel.  Both against
    # the fused selection, bit for bit, and sampled rows against the oracle.
    B, S, Skv, H, D, c, tk = 1, 16600, 20000, 64, 128, 1, 1000
    inp, nb = v4_case(B, S, Skv, H, D, seed=620)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    logits = lx.indexer_logits(q, k, w, c)
    sc_m, ix_m = lx.topk_from_logits(logits, c, tk)
    sc_f, ix_f = lx.topk(q, k, w, c, tk)
    assert torch.equal(ix_m, ix_f) and torch.equal(sc_m, sc_f)
    # the same selection over logits that leave the hidden positions unwritten
    vis = lx.indexer_logits(q, k, w, c, out=torch.full_like(logits, float("nan")), visible_only=True)
    sc_v, ix_v = lx.topk_from_logits(vis, c, tk)
    del vis
    assert torch.equal(ix_v, ix_m) and torch.equal(sc_v.view(torch.int32), sc_m.view(torch.int32))
    ks, ke = oracle.causal_ranges(S, Skv, c)
    rows = np.array([0, 999, 1000, 8191, 8192, 16382, 16383, 16384, 16385, S - 1])
    lg = logits[0][torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    for i, t in enumerate(rows):
        want_s, want_i = oracle.topk_select(lg[i:i + 1], ks[t:t + 1], ke[t:t + 1], tk)
        assert np.array_equal(ix_m[0, t].cpu().numpy(), want_i[0]), t
        assert np.array_equal(sc_m[0, t].cpu().numpy().astype(np.float64), want_s[0]), t


@pytest.mark.parametrize("H,D,topk", [(64, 128, 2048), (128, 128, 256), (32, 64, 100), (16, 32, 33),
                                      (8, 128, 64)])
def test_fused_equals_materialized(H, D, topk):
    B, S, Skv, c = 2, 3000, 2800, 1
    log(f"fused vs materialized H={H} D={D} topk={topk}")
    inp, _ = v4_case(B, S, Skv, H, D, seed=11 + H)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    logits = lx.indexer_logits(q, k, w, c)
    sc_m, ix_m = lx.topk_from_logits(logits, c, topk)
    sc_f, ix_f = lx.topk(q, k, w, c, topk)
    assert torch.equal(ix_m, ix_f)
    assert torch.equal(sc_m, sc_f)


def test_fused_exact_inputs_bitwise_vs_oracle():
    B, S, Skv, H, D, c, tk = 1, 2000, 500, 64, 128, 4, 37
    inp, nb = v4_case(B, S, Skv, H, D, seed=12, exact=True)
    sc, ix = lx.topk(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), c, tk)
    ks, ke = oracle.causal_ranges(S, Skv, c)
    ora = oracle.indexer_logits(nb["q"], nb["k"], nb["w"], ks, ke)
    want_s, want_i = oracle.topk_select(ora[0], ks, ke, tk)
    assert np.array_equal(ix.cpu().numpy()[0], want_i)
    assert np.array_equal(sc.cpu().numpy()[0].astype(np.float64), want_s)


def test_topk_edges_select_all_and_single_key():
    inp, nb = v4_case(1, 40, 9, 64, 128, seed=13)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    for tk in (9, 1):
        sc_f, ix_f = lx.topk(q, k, w, 1, tk)
        logits = lx.indexer_logits(q, k, w, 1)
        sc_m, ix_m = lx.topk_from_logits(logits, 1, tk)
        assert torch.equal(ix_f, ix_m) and torch.equal(sc_f, sc_m)
        want_s, want_i = oracle.topk_select(logits.cpu().numpy()[0].astype(np.float64),
                                            *oracle.causal_ranges(40, 9, 1), tk)
        assert np.array_equal(ix_f.cpu().numpy()[0], want_i)
    with pytest.raises(lx.LixError):
        lx.topk(q, k, w, 1, 10)                          # topk > Skv


# ------------------------------------------------------------------ gather

def test_gather_matches_oracle():
    inp, _ = v4_case(2, 100, 50, 64, 128, seed=14)
    logits = lx.indexer_logits(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), 2)
    g = torch.Generator().manual_seed(15)
    idx = torch.randint(-3, 60, (2, 100, 17), generator=g, dtype=torch.int32)
    got = lx.topk_scores(logits, dev(idx)).cpu().numpy()
    want = oracle.topk_scores_gather(logits.cpu().numpy().astype(np.float64), idx.numpy())
    assert np.array_equal(got.astype(np.float64), want)


def test_lighting_indexer_with_given_indices_round_trip():
    inp, _ = v4_case(1, 300, 75, 64, 128, seed=16)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    sc, ix = lx.v4_lighting_indexer(q, k, w, 4, 20)
    again = lx.v4_lighting_indexer(q, k, w, 4, 20, topk_indices=ix)
    assert torch.equal(sc, again)


# ------------------------------------------------------------------ scores at given indices

@pytest.mark.parametrize("H,D,B,S,Skv,c,tk", [
    (64, 128, 2, 300, 75, 4, 40),     # the workloads' heads and index_dim
    (64, 128, 1, 130, 200, 1, 1),
    (128, 256, 1, 70, 40, 2, 33),
    (32, 64, 2, 90, 70, 1, 70),       # topk == Skv, every key
    (16, 48, 1, 61, 50, 1, 100),      # topk > Skv (duplicated indices), index_dim padded
    (8, 32, 2, 40, 50, 1, 65),
    (4, 16, 1, 61, 70, 1, 31),
    (1, 128, 2, 70, 66, 1, 17),
])
def test_scores_at_equals_gathered_logits_bitwise(H, D, B, S, Skv, c, tk):
    # Given indices: a mix of in-range keys, keys outside the causal range,
    # negative and past-the-end indices and duplicates.
    log(f"scores_at H={H} D={D} B={B} S={S} Skv={Skv} c={c} topk={tk}")
    inp, nb = v4_case(B, S, Skv, H, D, seed=200 + H + D)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    g = torch.Generator().manual_seed(201 + H)
    idx = torch.randint(-3, Skv + 3, (B, S, tk), generator=g, dtype=torch.int32)
    idx[:, :, : min(tk, 5)] = idx[:, :, :1]                       # duplicates
    logits = lx.indexer_logits(q, k, w, c)
    want = lx.topk_scores(logits, dev(idx))
    got = lx.indexer_scores_at(q, k, w, c, dev(idx))
    assert torch.equal(got, want)
    ks, ke = ranges(S, Skv, c)
    ora, mag = oracle.indexer_logits(nb["q"], nb["k"], nb["w"], ks, ke, with_magnitude=True)
    o = oracle.topk_scores_gather(ora, idx.numpy())
    m = oracle.topk_scores_gather(mag, np.clip(idx.numpy(), 0, Skv - 1))
    checkers.check_logits(got.cpu().numpy(), o, np.where(np.isfinite(o), m, 0.0), f"scores_at H={H}")


def test_scores_at_given_ranges_and_exact_inputs():
    B, S, Skv, H, D, tk = 2, 150, 90, 64, 128, 50
    inp, nb = v4_case(B, S, Skv, H, D, seed=210, exact=True)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    g = torch.Generator().manual_seed(211)
    ks = torch.randint(0, 30, (S,), generator=g, dtype=torch.int32)
    ke = ks + torch.randint(-5, 80, (S,), generator=g, dtype=torch.int32)
    idx = torch.randint(-2, Skv + 2, (B, S, tk), generator=g, dtype=torch.int32)
    got = lx.indexer_scores_at(q, k, w, 1, dev(idx), dev(ks), dev(ke)).cpu().numpy()
    ora = oracle.indexer_logits(nb["q"], nb["k"], nb["w"], ks.numpy().astype(np.int64), ke.numpy().astype(np.int64))
    want = oracle.topk_scores_gather(ora, idx.numpy())
    assert np.array_equal(got.astype(np.float64), want)


def test_scores_at_32k_fused_selection_bitwise():
    # At full size, in the launch configuration the bench times: the scores at
    # the fused top-k's own indices are the fused top-k's scores, bit for bit.
    cfg = synth.WORKLOADS["32k"]
    S, Skv, tk = cfg["seqlen"], cfg["seqlen_kv"], cfg["topk"]
    inp, _ = v4_case(1, S, Skv, 64, 128, cfg["seed"])
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    log("32k: fused top-k, then scores at its indices")
    sc, ix = lx.topk(q, k, w, 4, tk)
    again = lx.indexer_scores_at(q, k, w, 4, ix)
    assert torch.equal(sc, again)


# ------------------------------------------------------------------ backward

def backward_case(B, S, Skv, H, D, tk, seed, idx_mode="random"):
    inp, nb = v4_case(B, S, Skv, H, D, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    if idx_mode == "random":
        # in-range keys, keys outside the causal range, negative and
        # past-the-end indices, and duplicates
        idx = torch.randint(-3, Skv + 3, (B, S, tk), generator=g, dtype=torch.int32)
        idx[:, :, : min(tk, 4)] = idx[:, :, :1]
    else:
        idx = None
    grad = synth.upstream_gradient(B, S, tk, seed + 2)
    return inp, nb, idx, grad


def check_backward_against_oracle(got, nb, idx, grad, ks, ke, where, rows=None):
    grads, bounds = oracle.indexer_backward(nb["q"], nb["k"], nb["w"], idx, grad, ks, ke, with_bounds=True,
                                            rows=rows)
    if rows is not None:
        got = {"dq": got["dq"][rows], "dw": got["dw"][rows]}
        grads = (grads[0][rows], None, grads[2][rows])
        bounds = {n: (bounds[n][0][rows], bounds[n][1][rows]) for n in ("dq", "dw")}
        for name, i in (("dq", 0), ("dw", 2)):
            sub = {name: got[name]}
            checkers.check_backward_one(sub, name, grads[i], bounds[name], where)
        return
    checkers.check_backward(got, grads, bounds, where)


@pytest.mark.parametrize("H,D,B,S,Skv,c,tk", [
    (64, 128, 1, 256, 64, 4, 16),       # tiny workload shape
    (64, 128, 2, 130, 100, 2, 70),      # ragged block of entries, B = 2
    (64, 96, 1, 70, 90, 1, 45),         # index_dim padded inside the kernel
    (64, 64, 1, 60, 50, 1, 33),
    (32, 128, 2, 50, 80, 1, 64),
    (16, 48, 1, 40, 30, 1, 20),
    (8, 128, 1, 33, 70, 1, 96),
    (1, 64, 2, 30, 40, 1, 9),
    (64, 128, 1, 40, 35, 1, 1),          # one entry per query
])
def test_backward_matches_oracle(H, D, B, S, Skv, c, tk):
    log(f"backward H={H} D={D} B={B} S={S} Skv={Skv} c={c} topk={tk}")
    inp, nb, idx, grad = backward_case(B, S, Skv, H, D, tk, seed=300 + H + D + tk)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    dq, dk, dw = lx.indexer_backward(q, k, w, c, dev(idx), dev(grad))
    torch.cuda.synchronize()
    ks, ke = ranges(S, Skv, c)
    got = {"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dw": dw.cpu().numpy()}
    check_backward_against_oracle(got, nb, idx.numpy(), grad.numpy(), ks, ke, f"backward H={H} D={D}")


def test_backward_given_ranges_and_repeat_runs():
    B, S, Skv, H, D, tk = 2, 90, 70, 64, 128, 40
    inp, nb, idx, grad = backward_case(B, S, Skv, H, D, tk, seed=330)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    g = torch.Generator().manual_seed(331)
    ks = torch.randint(0, 20, (S,), generator=g, dtype=torch.int32)
    ke = ks + torch.randint(-5, 60, (S,), generator=g, dtype=torch.int32)
    first = lx.indexer_backward(q, k, w, 1, dev(idx), dev(grad), dev(ks), dev(ke))
    # A second call with other outputs in flight: dq and dw are the same bits;
    # dk (float32 atomics) agrees within the tolerance.
    second = lx.indexer_backward(q, k, w, 1, dev(idx), dev(grad), dev(ks), dev(ke))
    assert torch.equal(first[0], second[0]) and torch.equal(first[2], second[2])
    got = {"dq": first[0].cpu().numpy(), "dk": first[1].cpu().numpy(), "dw": first[2].cpu().numpy()}
    check_backward_against_oracle(got, nb, idx.numpy(), grad.numpy(), ks.numpy().astype(np.int64),
                                  ke.numpy().astype(np.int64), "backward given ranges")
    got2 = {"dq": second[0].cpu().numpy(), "dk": second[1].cpu().numpy(), "dw": second[2].cpu().numpy()}
    check_backward_against_oracle(got2, nb, idx.numpy(), grad.numpy(), ks.numpy().astype(np.int64),
                                  ke.numpy().astype(np.int64), "backward given ranges, second call")


def test_backward_invalid_entries_and_zero_gradient():
    B, S, Skv, H, D, tk = 1, 40, 30, 64, 128, 32
    inp, _, idx, grad = backward_case(B, S, Skv, H, D, tk, seed=340)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    # every entry invalid: all gradients are exactly zero
    bad = torch.full((B, S, tk), -1, dtype=torch.int32)
    bad[:, :, ::2] = Skv + 5
    for t in (bad, torch.full((B, S, tk), Skv - 1, dtype=torch.int32)):
        dq, dk, dw = lx.indexer_backward(q, k, w, 4 if t is not bad else 1, dev(t), dev(grad))
        if t is bad:
            assert not dq.any() and not dk.any() and not dw.any()
    # zero upstream gradient: all zero
    dq, dk, dw = lx.indexer_backward(q, k, w, 1, dev(idx), torch.zeros(B, S, tk, device=DEV))
    assert not dq.any() and not dk.any() and not dw.any()
    # NaN gradients on invalid entries are ignored
    g_nan = grad.clone()
    valid = (idx >= 0) & (idx < torch.arange(S).view(1, S, 1) + 1) & (idx < Skv)
    g_nan[~valid] = float("nan")
    a = lx.indexer_backward(q, k, w, 1, dev(idx), dev(g_nan))
    b = lx.indexer_backward(q, k, w, 1, dev(idx), dev(torch.where(valid, grad, torch.zeros_like(grad))))
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
    assert torch.isfinite(a[1]).all()


def test_backward_keys_repeated_past_one_bucket():
    # Rows naming a few keys many times: more than 64 entries in one 64-key
    # bucket (the dk kernel's second pass over a bucket), repeated keys summed.
    B, S, Skv, H, D, tk = 2, 60, 300, 64, 128, 200
    inp, nb, _, grad = backward_case(B, S, Skv, H, D, tk, seed=345)
    g = torch.Generator().manual_seed(346)
    idx = torch.randint(0, 10, (B, S, tk), generator=g, dtype=torch.int32)
    idx[:, :, ::7] = torch.randint(0, Skv, (B, S, (tk + 6) // 7), generator=g, dtype=torch.int32)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    dq, dk, dw = lx.indexer_backward(q, k, w, 1, dev(idx), dev(grad))
    ks, ke = oracle.causal_ranges(S, Skv, 1)
    check_backward_against_oracle({"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dw": dw.cpu().numpy()}, nb,
                                  idx.numpy(), grad.numpy(), ks, ke, "repeated keys")


def test_backward_4k_topk_selection():
    # The 4K workload end to end: fused top-k, then the backward of its scores.
    cfg = synth.WORKLOADS["4k"]
    B, S, Skv, tk = cfg["batch"], cfg["seqlen"], cfg["seqlen_kv"], cfg["topk"]
    inp, nb = v4_case(B, S, Skv, 64, 128, cfg["seed"])
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    log("4k: fused top-k, then the backward")
    sc, ix = lx.topk(q, k, w, 4, tk)
    grad = synth.upstream_gradient(B, S, tk, 345)
    dq, dk, dw = lx.indexer_backward(q, k, w, 4, ix, dev(grad))
    torch.cuda.synchronize()
    ks, ke = ranges(S, Skv, 4)
    got = {"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dw": dw.cpu().numpy()}
    log("4k: oracle backward")
    check_backward_against_oracle(got, nb, ix.cpu().numpy(), grad.numpy(), ks, ke, "backward 4k")


@pytest.mark.parametrize("workload", ["32k", "131k"])
def test_backward_workload_sampled_rows_and_homogeneity(workload):
    # Full size, in the launch configuration the bench times (32K) and the
    # longest workload (131K: the workspace grows with topk and Skv/64, not
    # with S * Skv).  dq and dw of a query depend on that query alone: sampled
    # queries against the oracle.  dk sums over every query: checked through
    # Euler's identity for the positively homogeneous score (degree 1 in q, in
    # k and in w): <dq, q> = <dk, k> = <dw, w> = sum over valid entries of
    # g * score.
    cfg = synth.WORKLOADS[workload]
    S, Skv, tk = cfg["seqlen"], cfg["seqlen_kv"], cfg["topk"]
    extra = {"heavy_fraction": cfg["heavy_fraction"]} if "heavy_fraction" in cfg else {}
    inp, nb = v4_case(1, S, Skv, 64, 128, cfg["seed"], **extra)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    log(f"{workload}: fused top-k, then the backward")
    sc, ix = lx.topk(q, k, w, 4, tk)
    grad = dev(synth.upstream_gradient(1, S, tk, 346))
    dq, dk, dw = lx.indexer_backward(q, k, w, 4, ix, grad)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, S, S // 32), [3, 4, 7, 8191, 8192, 8195, S - 1]]))
    ks, ke = ranges(S, Skv, 4)
    log(f"{workload}: oracle backward on {len(rows)} sampled queries")
    check_backward_against_oracle({"dq": dq.cpu().numpy(), "dw": dw.cpu().numpy()}, nb, ix.cpu().numpy(),
                                  grad.cpu().numpy(), ks, ke, f"backward {workload}", rows=rows)
    valid = torch.isfinite(sc)
    gs = torch.where(valid, grad, torch.zeros_like(grad))
    total = (gs.double() * torch.where(valid, sc, torch.zeros_like(sc)).double()).sum().item()
    # error scale: sum |g| * sum_h |w_h| relu(d_h), the scores taken with |w|
    sc_abs = lx.indexer_scores_at(q, k, w.abs(), 4, ix)
    scale = (gs.abs().double() * torch.where(valid, sc_abs, torch.zeros_like(sc_abs)).double()).sum().item()
    for name, grad_t, x in (("dq", dq, q), ("dk", dk, k), ("dw", dw, w)):
        inner = (grad_t.double() * x.double()).sum().item()
        assert abs(inner - total) <= 2.0 ** -8 * scale + 1e-3, (name, inner, total, scale)


def test_autograd_function_matches_the_backward_entry_point():
    B, S, Skv, H, D, c, tk = 1, 64, 40, 64, 128, 2, 12
    inp, _, idx, grad = backward_case(B, S, Skv, H, D, tk, seed=350)
    q = dev(inp["q"]).requires_grad_()
    k = dev(inp["k"]).requires_grad_()
    w = dev(inp["w"]).requires_grad_()
    scores = lx.v4_lighting_indexer(q, k, w, c, tk, dev(idx))
    assert torch.equal(scores.detach(), lx.indexer_scores_at(q.detach(), k.detach(), w.detach(), c, dev(idx)))
    scores.backward(dev(grad))
    dq, dk, dw = lx.indexer_backward(q.detach(), k.detach(), w.detach(), c, dev(idx), dev(grad))
    assert q.grad.dtype == torch.bfloat16 and k.grad.dtype == torch.bfloat16 and w.grad.dtype == torch.float32
    assert torch.equal(q.grad, dq.to(torch.bfloat16)) and torch.equal(w.grad, dw)
    assert torch.allclose(k.grad.float(), dk.to(torch.bfloat16).float(), rtol=2 ** -7, atol=1e-5)
    # Without indices: the fused top-k's scores carry gradients the same way.
    q.grad = k.grad = w.grad = None
    sc2, ix2 = lx.v4_lighting_indexer(q, k, w, c, tk)
    assert not ix2.requires_grad
    sc2.backward(dev(grad))
    dq2, _, dw2 = lx.indexer_backward(q.detach(), k.detach(), w.detach(), c, ix2, dev(grad))
    assert torch.equal(q.grad, dq2.to(torch.bfloat16)) and torch.equal(w.grad, dw2)


# ------------------------------------------------------------------ V4.1

@pytest.mark.parametrize("H,D,B,L,G", [(64, 128, 1, 200, 60), (16, 32, 2, 70, 100), (128, 64, 1, 33, 20),
                                       (1, 16, 1, 64, 70), (4, 48, 2, 50, 30)])
def test_v41_matches_oracle(H, D, B, L, G):
    log(f"v41 H={H} D={D} B={B} L={L} G={G}")
    inp = synth.v41_inputs(batch=B, local_sequence=L, global_compressed=G, heads=H, index_dim=D, seed=20 + H,
                           doc_min=10, doc_max=80)
    nb = {x: synth.bits(inp[x]) for x in ("queries", "keys", "weights", "allowed")}
    got = lx.indexer_scores_v41(*(dev(inp[x]) for x in ("queries", "keys", "weights", "allowed")))
    got = got.cpu().view(torch.int16).numpy().view(np.uint16)
    widened = 0
    for b in range(B):
        rows = np.arange(L)
        o = oracle.indexer_scores_v41_rows(nb["queries"], nb["keys"], nb["weights"], nb["allowed"], b, rows)
        lo, hi = oracle.indexer_scores_v41_bounds_rows(nb["queries"], nb["keys"], nb["weights"], nb["allowed"],
                                                       b, rows)
        widened += checkers.check_v41(got[b], o, lo, hi, f"v41 b={b}")
    log(f"  outputs needing the accumulation interval: {widened}")


def test_v41_exact_inputs_bitwise():
    inp = synth.v41_exact_inputs(batch=2, local_sequence=90, global_compressed=70, heads=64, index_dim=128,
                                 seed=21, density=0.4)
    nb = {x: synth.bits(inp[x]) for x in ("queries", "keys", "weights", "allowed")}
    got = lx.indexer_scores_v41(*(dev(inp[x]) for x in ("queries", "keys", "weights", "allowed")))
    got = got.cpu().view(torch.int16).numpy().view(np.uint16)
    want = oracle.f64_to_bf16_bits(oracle.indexer_scores_v41(nb["queries"], nb["keys"], nb["weights"],
                                                             nb["allowed"]))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("min_heads", [1, 8])
def test_v41_golden_rounding_cases_on_gpu(min_heads):
    # min_heads = 8 pads each case with zero heads (q = 0, w = 0: each adds an
    # exact 0), so the cases also run through the paired-head epilogue
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "v41_rounding.json")))
    D = g["index_dim"]
    for case in g["cases"]:
        H = max(len(case["heads"]), min_heads)
        q = torch.zeros(1, 1, H, D)
        w = torch.zeros(1, 1, H)
        for h, hd in enumerate(case["heads"]):
            q[0, 0, h, :len(hd["q"])] = torch.tensor(hd["q"], dtype=torch.float32)
            w[0, 0, h] = hd["w"]
        k = torch.zeros(1, 1, D)
        k[0, 0, :len(case["k"])] = torch.tensor(case["k"], dtype=torch.float32)
        al = torch.tensor([[[case["allowed"]]]])
        out = lx.indexer_scores_v41(dev(q.bfloat16()), dev(k.bfloat16()), dev(w.bfloat16()), dev(al))
        bits = int(out.cpu().view(torch.int16).item()) & 0xFFFF
        assert bits == int(case["out_bits"], 16), case["name"]


# ------------------------------------------------------------------ full-size workloads (sampled)

def test_32k_workload_sampled_rows():
    cfg = synth.WORKLOADS["32k"]
    S, Skv, tk = cfg["seqlen"], cfg["seqlen_kv"], cfg["topk"]
    log("32k: generating inputs")
    inp, nb = v4_case(1, S, Skv, 64, 128, cfg["seed"])
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    log("32k: fused top-k")
    sc_f, ix_f = lx.topk(q, k, w, 4, tk)
    log("32k: materialized logits + top-k")
    logits = lx.indexer_logits(q, k, w, 4)
    sc_m, ix_m = lx.topk_from_logits(logits, 4, tk)
    assert torch.equal(ix_f, ix_m) and torch.equal(sc_f, sc_m)
    log("32k: streaming top-k")
    sc_s, ix_s = lx.topk_streaming(q, k, w, 4, tk)
    assert torch.equal(ix_s, ix_m) and torch.equal(sc_s, sc_m)
    rows = np.arange(31, S, 64)
    ks, ke = oracle.causal_ranges(S, Skv, 4)
    ora, mag = oracle.indexer_logits_rows(nb["q"], nb["k"], nb["w"], 0, rows, ks, ke, with_magnitude=True)
    checkers.check_logits(logits[0][torch.from_numpy(rows).to(DEV)].cpu().numpy(), ora, mag, "32k rows")
    exact = checkers.check_topk_rows(sc_f[0].cpu().numpy()[rows], ix_f[0].cpu().numpy()[rows], ora, mag,
                                     ks[rows], ke[rows], tk, "32k")
    log(f"  32k: rows with a forced exact set: {exact}/{len(rows)}")


def test_131k_workload_fused_and_materialized_sampled_rows():
    cfg = synth.WORKLOADS["131k"]
    S, Skv, tk = cfg["seqlen"], cfg["seqlen_kv"], cfg["topk"]
    log("131k: generating inputs")
    inp, nb = v4_case(1, S, Skv, 64, 128, cfg["seed"], heavy_fraction=cfg["heavy_fraction"])
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    log("131k: fused top-k")
    sc, ix = lx.topk(q, k, w, 4, tk)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(255, S, 256)[:400], np.arange(S - 64, S)])
    ks, ke = oracle.causal_ranges(S, Skv, 4)
    log("131k: oracle rows")
    ora, mag = oracle.indexer_logits_rows(nb["q"], nb["k"], nb["w"], 0, rows, ks, ke, with_magnitude=True)
    exact = checkers.check_topk_rows(sc[0].cpu().numpy()[rows], ix[0].cpu().numpy()[rows], ora, mag,
                                     ks[rows], ke[rows], tk, "131k")
    log(f"  131k: rows with a forced exact set: {exact}/{len(rows)}")
    log("131k: materialized logits (16 GiB) + row top-k")
    logits = lx.indexer_logits(q, k, w, 4)
    sc_m, ix_m = lx.topk_from_logits(logits, 4, tk)
    assert torch.equal(ix_m, ix) and torch.equal(sc_m, sc)


def test_v41_workload_sampled_rows():
    cfg = synth.WORKLOADS["v41"]
    log("v41 workload: generating inputs")
    inp = synth.v41_inputs(**cfg)
    nb = {x: synth.bits(inp[x]) for x in ("queries", "keys", "weights", "allowed")}
    got = lx.indexer_scores_v41(*(dev(inp[x]) for x in ("queries", "keys", "weights", "allowed")))
    got = got.cpu().view(torch.int16).numpy().view(np.uint16)[0]
    rows = np.arange(15, cfg["local_sequence"], 32)
    o = oracle.indexer_scores_v41_rows(nb["queries"], nb["keys"], nb["weights"], nb["allowed"], 0, rows)
    lo, hi = oracle.indexer_scores_v41_bounds_rows(nb["queries"], nb["keys"], nb["weights"], nb["allowed"], 0,
                                                   rows)
    widened = checkers.check_v41(got[rows], o, lo, hi, "v41 workload")
    allowed_frac = float(inp["allowed"].float().mean())
    log(f"  v41 workload: allowed fraction {allowed_frac:.4f}; outputs needing the interval: {widened}")


# ------------------------------------------------------------------ V4.1 top-k over bf16 scores

def _bf16_rows(g, B, L, G, hidden_frac):
    pool = torch.tensor([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4000, 0x3F00, 0xC040, 0x3E80, 0x4040],
                        dtype=torch.int32)
    bits = pool[torch.randint(0, len(pool), (B, L, G), generator=g)]
    noise = torch.randint(0, 0x7F80, (B, L, G), generator=g, dtype=torch.int32)     # finite magnitudes
    noise = noise | (torch.randint(0, 2, (B, L, G), generator=g, dtype=torch.int32) << 15)   # either sign
    dense = torch.rand(B, L, G, generator=g) < 0.5
    bits = torch.where(dense, noise, bits)                 # half from a small pool (ties), half arbitrary finite
    bits[torch.rand(B, L, G, generator=g) < hidden_frac] = 0xFF80
    return bits.to(torch.int16)


@pytest.mark.parametrize("G", [100, 2048, 4096, 6000, 8192])
def test_topk_bf16_matches_oracle_bitwise(G):
    g = torch.Generator().manual_seed(300 + G)
    B, L = 2, 12
    bits = _bf16_rows(g, B, L, G, 0.4)
    bits[0, 0] = 0xFF80 - 0x10000                          # nothing visible
    bits[0, 1, 5:] = 0xFF80 - 0x10000                      # 5 visible keys
    bits[1, 2] = 0x3F80                                    # all equal
    scores = bits.view(torch.bfloat16)
    for tk in (1, 17, max(1, G // 3), G):
        log(f"topk_bf16 G={G} topk={tk}")
        sc, ix = lx.topk_bf16(dev(scores), tk)
        sc = sc.cpu().view(torch.int16).numpy().view(np.uint16)
        ix = ix.cpu().numpy()
        for b in range(B):
            want_b, want_i = oracle.topk_select_visible_bf16(bits[b].numpy().view(np.uint16), tk)
            assert np.array_equal(ix[b], want_i), (G, tk, b)
            assert np.array_equal(sc[b], want_b), (G, tk, b)


def test_topk_bf16_after_v41_workload_sampled_rows():
    cfg = synth.WORKLOADS["v41"]
    inp = synth.v41_inputs(**cfg)
    got = lx.indexer_scores_v41(*(dev(inp[x]) for x in ("queries", "keys", "weights", "allowed")))
    sc, ix = lx.topk_bf16(got, 512)
    rows = np.arange(7, cfg["local_sequence"], 97)
    bits = got[0].cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    want_b, want_i = oracle.topk_select_visible_bf16(bits, 512)
    assert np.array_equal(ix[0].cpu().numpy()[rows], want_i)
    assert np.array_equal(sc[0].cpu().view(torch.int16).numpy().view(np.uint16)[rows], want_b)


def test_device_properties_logged():
    p = torch.cuda.get_device_properties(0)
    log(f"device: {p.name} gcn={getattr(p, 'gcnArchName', '?')} CUs={p.multi_processor_count} "
        f"shared/block={getattr(p, 'shared_memory_per_block', '?')} "
        f"shared/block optin={getattr(p, 'shared_memory_per_block_optin', '?')} "
        f"L2={getattr(p, 'L2_cache_size', '?')} mem={p.total_memory >> 30} GiB")
    assert "gfx950" in getattr(p, "gcnArchName", "gfx950")


@pytest.mark.parametrize("Skv", [300, 2048, 3000, 4096, 6000, 8192, 9000, 20000, 32768])
def test_topk_from_logits_edge_rows_bitwise(Skv):
    # Every size class of the row kernel, with rows that stress each branch:
    # all-equal scores (degenerate range), a few distinct values (large
    # boundary bins), -inf inside the range (non-finite range), signed zeros,
    # misaligned row starts (ks odd), a crowded boundary bin, scores far from
    # zero relative to their spread, and ragged ends.
    g = torch.Generator().manual_seed(Skv)
    B, S = 2, 24
    lg = torch.randn(B, S, Skv, generator=g)
    lg[:, 0] = 0.5                                       # all equal
    lg[:, 1] = torch.randint(0, 3, (B, Skv), generator=g).float()
    lg[:, 2, ::7] = float("-inf")
    lg[:, 3, ::5] = -0.0
    lg[:, 3, 1::5] = 0.0
    lg[:, 4] = torch.randn(B, Skv, generator=g) * 1e-30     # tiny range
    lg[:, 5] = torch.randn(B, Skv, generator=g) * 1e30      # huge range
    lg[:, 6] = torch.randn(B, Skv, generator=g) * 100.0      # a tight cluster inside a wide range:
    lg[:, 6, : Skv // 2] = 1.0 + torch.randn(B, Skv // 2, generator=g) * 1e-5   # one crowded bin
    lg[:, 7] = 1000.0 + torch.randn(B, Skv, generator=g) * 0.01   # range far from zero relative to its width
    lg[:, 8] = -1000.0 + torch.randn(B, Skv, generator=g) * 0.01  # (the row kernel's subtract-first binning)
    lg[:, 9] = 0.0                                       # zeros plus two tiny values (set below, inside
    lg[:, 10] = -3e-38                                   # the range): spans near 1e-37, whose bin scale
                                                         # would overflow
    ks = torch.randint(0, max(1, Skv // 5), (S,), generator=g, dtype=torch.int32)
    ks[::3] |= 1
    ke = torch.clamp(ks + torch.randint(Skv // 3, Skv + 10, (S,), generator=g, dtype=torch.int32), max=Skv)
    lg[:, 9, int(ks[9]) + 1] = 1e-37
    lg[:, 9, int(ke[9]) - 2] = 2e-37
    lg[:, 10, int(ks[10]) + 3] = 0.0
    for tk in (1, 17, min(1000, Skv // 3), min(2048, Skv // 2), 3 * Skv // 4):
        log(f"Skv={Skv} topk={tk}")
        sc, ix = lx.topk_from_logits(dev(lg), 1, tk, dev(ks), dev(ke))
        sc, ix = sc.cpu().numpy(), ix.cpu().numpy()
        for b in range(B):
            want_s, want_i = oracle.topk_select(lg[b].numpy().astype(np.float64), ks.numpy(), ke.numpy(), tk)
            assert np.array_equal(ix[b], want_i), (Skv, tk, b)
            assert np.array_equal(sc[b].astype(np.float64), want_s), (Skv, tk, b)


# ------------------------------------------------------------------ fused top-k: forced branches

def _fused_case(name):
    """Inputs that drive the fused kernel's candidate buffer through each of its branches.

    Returns (inp, H, D, B, S, Skv, topk, ks, ke) with ks/ke None for causal c=1 ranges.
    """
    g = torch.Generator().manual_seed(sum(map(ord, name)))
    if name == "zero_weights":              # every score +0: the pruning pass sees a zero span
        inp, _ = v4_case(1, 3000, 2800, 64, 128, seed=400)
        inp["w"] = torch.zeros_like(inp["w"])
        return inp, 64, 128, 1, 3000, 2800, 2048, None, None
    if name == "zero_query_rows":           # every 3rd query all-zero: all-zero rows next to normal ones
        inp, _ = v4_case(2, 2500, 2400, 64, 128, seed=401)
        inp["q"][::3] = 0
        return inp, 64, 128, 2, 2500, 2400, 1500, None, None
    if name == "duplicate_keys":            # three distinct key rows: a crowded boundary bin everywhere
        inp, _ = v4_case(1, 3000, 2900, 64, 128, seed=402)
        pool = inp["k"][:3].clone()
        inp["k"] = pool[torch.randint(0, 3, (2900,), generator=g)].contiguous()
        return inp, 64, 128, 1, 3000, 2900, 2048, None, None
    if name == "small_integers":            # exact small-integer scores: many ties, crowded bins
        inp, _ = v4_case(1, 3000, 2900, 64, 128, seed=403, exact=True)
        return inp, 64, 128, 1, 3000, 2900, 2048, None, None
    if name == "long_rows":                 # 16384 keys per row, topk 2048: the buffer is pruned again and again
        inp, _ = v4_case(1, 40, 16384, 64, 128, seed=404)
        ks = torch.zeros(40, dtype=torch.int32)
        ke = torch.full((40,), 16384, dtype=torch.int32)
        ke[::5] = torch.randint(8000, 16384, (8,), generator=g, dtype=torch.int32)
        return inp, 64, 128, 1, 40, 16384, 2048, ks, ke
    if name == "heads128_topk256":          # capacity 512: frequent pruning
        inp, _ = v4_case(1, 2000, 3000, 128, 128, seed=405)
        return inp, 128, 128, 1, 2000, 3000, 256, None, None
    if name == "heads8_capacity":           # heads 8 at the largest topk its LDS holds
        inp, _ = v4_case(2, 1500, 3000, 8, 128, seed=406)
        return inp, 8, 128, 2, 1500, 3000, 576, None, None
    if name == "given_ranges":              # ks > 0, odd starts, ke < ks, empty rows
        S, Skv = 900, 2600
        inp, _ = v4_case(2, S, Skv, 64, 128, seed=407)
        ks = torch.randint(0, 2000, (S,), generator=g, dtype=torch.int32)
        ks[::2] |= 1
        ke = ks + torch.randint(-50, 1500, (S,), generator=g, dtype=torch.int32)
        ke[::11] = ks[::11]                  # empty
        ke[5::13] = ks[5::13] - 7            # ke < ks: empty
        ke[7::17] = 100_000                  # clamped to Skv
        return inp, 64, 128, 2, S, Skv, 300, ks, ke
    raise KeyError(name)


@pytest.mark.parametrize("name", ["zero_weights", "zero_query_rows", "duplicate_keys", "small_integers", "long_rows",
                                  "heads128_topk256", "heads8_capacity", "given_ranges"])
def test_fused_branches_bitwise_vs_materialized_and_oracle(name):
    inp, H, D, B, S, Skv, tk, ks, ke = _fused_case(name)
    log(f"fused branch case {name}: H={H} D={D} B={B} S={S} Skv={Skv} topk={tk}")
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    kd = None if ks is None else dev(ks)
    ked = None if ke is None else dev(ke)
    sc_f, ix_f = lx.topk(q, k, w, 1, tk, cu_seqlen_ks=kd, cu_seqlen_ke=ked)
    logits = lx.indexer_logits(q, k, w, 1, kd, ked)
    sc_m, ix_m = lx.topk_from_logits(logits, 1, tk, kd, ked)
    assert torch.equal(ix_f, ix_m) and torch.equal(sc_f, sc_m), name
    ksn, ken = ranges(S, Skv, 1, ks, ke)
    lg = logits.cpu().numpy()
    for b in range(B):
        want_s, want_i = oracle.topk_select(lg[b].astype(np.float64), ksn, ken, tk)
        assert np.array_equal(ix_f[b].cpu().numpy(), want_i), (name, b)
        assert np.array_equal(sc_f[b].cpu().numpy().astype(np.float64), want_s), (name, b)


@pytest.mark.parametrize("H,S,Skv,tk,route", [
    (4, 400, 1000, 40, "streaming"),      # heads 4: no fused kernel
    (8, 400, 1000, 700, "streaming"),     # heads 8 above the fused capacity
    (4, 60, 9000, 100, "materialized"),   # past the streaming row limit, no fused kernel
    (64, 60, 9000, 100, "fused"),
])
def test_select_topk_routes_every_size_to_a_route(H, S, Skv, tk, route):
    # The pages' entry point answers for every size; each route gives the oracle's selection.
    inp, nb = v4_case(1, S, Skv, H, 64, seed=410 + H + Skv)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    assert (Skv <= 8192) == (route == "streaming")
    assert lx.fused_topk_supported(Skv, H, 64, tk) == (route == "fused")
    log(f"select_topk route {route}: H={H} S={S} Skv={Skv} topk={tk}")
    sc, ix = lx.v4_lighting_indexer(q, k, w, 1, tk)
    ks, ke = oracle.causal_ranges(S, Skv, 1)
    rows = np.arange(S)
    _check_topk_vs_oracle(sc[0].detach().cpu().numpy(), ix[0].cpu().numpy(), nb, 0, rows, ks, ke, tk,
                          f"select_topk {route} H={H}")


# ------------------------------------------------------------------ streaming top-k

def _streaming_vs_materialized(q, k, w, c, tk, kd=None, ked=None, workspace=None):
    sc_s, ix_s = lx.topk_streaming(q, k, w, c, tk, kd, ked, workspace=workspace)
    logits = lx.indexer_logits(q, k, w, c, kd, ked)
    sc_m, ix_m = lx.topk_from_logits(logits, c, tk, kd, ked)
    assert torch.equal(ix_s, ix_m) and torch.equal(sc_s, sc_m)
    return sc_s, ix_s, logits


@pytest.mark.parametrize("H,D,B,S,Skv,c,tk", [
    (64, 128, 1, 256, 64, 4, 16),       # tiny workload shape
    (64, 128, 3, 333, 100, 3, 40),      # ragged tail in queries and keys; topk above early rows' length
    (64, 128, 1, 3000, 2900, 1, 2048),
    (128, 128, 2, 700, 3000, 1, 256),
    (32, 64, 2, 900, 5000, 1, 1000),
    (16, 32, 1, 500, 8192, 1, 4000),     # longest rows the route takes, topk half of them
    (8, 256, 2, 300, 1200, 1, 700),
    (4, 64, 1, 400, 1000, 1, 40),        # heads below 8: the other store layout
    (1, 16, 2, 130, 300, 1, 299),
])
def test_streaming_topk_bitwise_vs_materialized_and_oracle(H, D, B, S, Skv, c, tk):
    log(f"streaming H={H} D={D} B={B} S={S} Skv={Skv} c={c} topk={tk}")
    inp, _ = v4_case(B, S, Skv, H, D, seed=500 + H + D + S)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    sc, ix, logits = _streaming_vs_materialized(q, k, w, c, tk)
    ksn, ken = oracle.causal_ranges(S, Skv, c)
    lg = logits.cpu().numpy()
    for b in range(B):
        want_s, want_i = oracle.topk_select(lg[b].astype(np.float64), ksn, ken, tk)
        assert np.array_equal(ix[b].cpu().numpy(), want_i), b
        assert np.array_equal(sc[b].cpu().numpy().astype(np.float64), want_s), b


@pytest.mark.parametrize("name", ["zero_weights", "zero_query_rows", "duplicate_keys", "small_integers",
                                  "heads128_topk256", "heads8_capacity", "given_ranges"])
def test_streaming_branch_cases_bitwise_vs_materialized(name):
    inp, H, D, B, S, Skv, tk, ks, ke = _fused_case(name)
    log(f"streaming branch case {name}: H={H} D={D} B={B} S={S} Skv={Skv} topk={tk}")
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    kd = None if ks is None else dev(ks)
    ked = None if ke is None else dev(ke)
    _streaming_vs_materialized(q, k, w, 1, tk, kd, ked)


def test_streaming_small_workspaces():
    # One slot (a grid of one workgroup walking every block), a few slots, and
    # a workspace one byte short of a slot (rejected).
    B, S, Skv, H, D, tk = 2, 600, 2000, 64, 128, 300
    inp, _ = v4_case(B, S, Skv, H, D, seed=510)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    slot = 4 * Skv * 4                       # four queries per block at 64 heads
    for nslot in (1, 3, 7):
        log(f"streaming workspace of {nslot} slots")
        ws = torch.empty(nslot * slot, dtype=torch.uint8, device=DEV)
        _streaming_vs_materialized(q, k, w, 1, tk, workspace=ws)
    ws = torch.empty(slot - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(lx.LixError):
        lx.topk_streaming(q, k, w, 1, tk, workspace=ws)
    full = lx.streaming_workspace_bytes(B, S, Skv, H, D)
    n_blocks = 2 * ((S + 3) // 4)
    assert full % slot == 0 and slot <= full <= n_blocks * slot
    assert lx.streaming_workspace_bytes(B, S, 8193, H, D) == -1


# ------------------------------------------------------------------ canaries around every output

def _guarded(n, dtype, fill):
    buf = torch.full((n + 2048,), fill, dtype=dtype, device=DEV)
    return buf, buf[1024:1024 + n]


def _intact(buf, n, fill):
    torch.cuda.synchronize()
    return bool((buf[:1024] == fill).all()) and bool((buf[1024 + n:] == fill).all())


def test_every_output_leaves_memory_around_it_untouched():
    # Each entry point writes into the middle of a larger buffer filled with a
    # sentinel; the sentinel before and after the output must survive.
    lib = lx.load()
    st = torch.cuda.current_stream().cuda_stream
    B, S, Skv, H, D, c, tk = 2, 77, 50, 64, 128, 1, 20
    inp, _ = v4_case(B, S, Skv, H, D, seed=420)
    q, k, w = dev(inp["q"]), dev(inp["k"]), dev(inp["w"])
    n = B * S * tk
    logits = lx.indexer_logits(q, k, w, c)
    idx_given = dev(torch.randint(-2, Skv + 2, (B, S, tk), generator=torch.Generator().manual_seed(421),
                                  dtype=torch.int32))
    grad = dev(synth.upstream_gradient(B, S, tk, 422))
    F, I = 12345.0, 0x5A5A5A5A
    for route in ("fused", "materialized"):
        sbuf, so = _guarded(n, torch.float32, F)
        ibuf, io = _guarded(n, torch.int32, I)
        lp = None if route == "fused" else logits.data_ptr()
        rc = lib.lix_topk(q.data_ptr(), k.data_ptr(), w.data_ptr(), lp, B, S, Skv, H, D, c, None, None, tk,
                          so.data_ptr(), io.data_ptr(), st)
        assert rc == 0 and _intact(sbuf, n, F) and _intact(ibuf, n, I), route
    ws_s = lib.lix_topk_streaming_workspace_bytes(B, S, Skv, H, D)
    wbuf = torch.full((ws_s + 4096,), 0x5A, dtype=torch.uint8, device=DEV)
    sbuf, so = _guarded(n, torch.float32, F)
    ibuf, io = _guarded(n, torch.int32, I)
    assert lib.lix_topk_streaming(q.data_ptr(), k.data_ptr(), w.data_ptr(), B, S, Skv, H, D, c, None, None, tk,
                                  so.data_ptr(), io.data_ptr(), wbuf.data_ptr(), ws_s, st) == 0
    assert _intact(sbuf, n, F) and _intact(ibuf, n, I), "streaming"
    assert bool((wbuf[ws_s:] == 0x5A).all()), "streaming workspace"
    sbuf, so = _guarded(n, torch.float32, F)
    assert lib.lix_topk_scores(logits.data_ptr(), idx_given.data_ptr(), B, S, Skv, tk, so.data_ptr(), st) == 0
    assert _intact(sbuf, n, F), "gather"
    sbuf, so = _guarded(n, torch.float32, F)
    assert lib.lix_indexer_scores_at(q.data_ptr(), k.data_ptr(), w.data_ptr(), idx_given.data_ptr(), B, S, Skv, H,
                                     D, c, None, None, tk, so.data_ptr(), st) == 0
    assert _intact(sbuf, n, F), "scores_at"
    ws_bytes = lib.lix_indexer_backward_workspace_bytes(B, S, Skv, H, D, tk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    bufs = {name: _guarded(m, torch.float32, F) for name, m in
            (("dq", S * B * H * D), ("dk", Skv * B * D), ("dw", S * B * H))}
    # dk needs 16-byte alignment: the guard of 1024 floats keeps it
    assert lib.lix_indexer_backward(q.data_ptr(), k.data_ptr(), w.data_ptr(), idx_given.data_ptr(), grad.data_ptr(),
                                    B, S, Skv, H, D, c, None, None, tk, bufs["dq"][1].data_ptr(),
                                    bufs["dk"][1].data_ptr(), bufs["dw"][1].data_ptr(), ws.data_ptr(), ws_bytes,
                                    st) == 0
    for name, (buf, view) in bufs.items():
        assert _intact(buf, view.numel(), F), f"backward {name}"
    vin = synth.v41_inputs(batch=2, local_sequence=70, global_compressed=45, heads=64, index_dim=128, seed=423,
                           doc_min=10, doc_max=40)
    vq, vk, vw, va = (dev(vin[x]) for x in ("queries", "keys", "weights", "allowed"))
    nv = 2 * 70 * 45
    hb = torch.tensor([0x1234], dtype=torch.int16).view(torch.bfloat16).item()
    vbuf, vo = _guarded(nv, torch.bfloat16, hb)
    assert lib.lix_indexer_scores_v41(vq.data_ptr(), vk.data_ptr(), vw.data_ptr(), va.data_ptr(), 2, 70, 45, 64, 128,
                                      vo.data_ptr(), st) == 0
    assert _intact(vbuf, nv, hb), "v41"
    v41 = vo.view(2, 70, 45).clone()
    nt = 2 * 70 * 9
    tbuf, to = _guarded(nt, torch.bfloat16, hb)
    ibuf, io = _guarded(nt, torch.int32, I)
    assert lib.lix_topk_bf16(v41.data_ptr(), 2, 70, 45, 9, to.data_ptr(), io.data_ptr(), st) == 0
    assert _intact(tbuf, nt, hb) and _intact(ibuf, nt, I), "topk_bf16"

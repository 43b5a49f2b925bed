"""lix_indexer_backward_noalloc (the backward with its workspace in a static
device array, for callers that cannot allocate) against lix_indexer_backward,
through the C ABI: two calls in a row, the second smaller, so the second runs
on the array the first left behind."""

import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_lightning_bf16_amd as lx
from tests import checkers

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(B, S, Skv, H, D, tk, seed):
    inp = synth.v4_inputs(batch=B, seqlen=S, seqlen_kv=Skv, heads=H, index_dim=D, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    idx = torch.randint(-3, Skv + 3, (B, S, tk), generator=g, dtype=torch.int32)
    idx[:, :, :3] = idx[:, :, :1]                        # duplicates
    grad = synth.upstream_gradient(B, S, tk, seed + 2)
    return inp, idx, grad


def _noalloc(q, k, w, idx, grad, c):
    S, B, H, D = q.shape
    Skv, tk = k.shape[0], idx.shape[2]
    dq = torch.full((S, B, H, D), float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.full((Skv, B, D), float("nan"), dtype=torch.float32, device=DEV)
    dw = torch.full((S, B, H), float("nan"), dtype=torch.float32, device=DEV)
    st = lx.load().lix_indexer_backward_noalloc(q.data_ptr(), k.data_ptr(), w.data_ptr(), idx.data_ptr(),
                                                grad.data_ptr(), B, S, Skv, H, D, c, None, None, tk, dq.data_ptr(),
                                                dk.data_ptr(), dw.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, lx.status_string(st)
    return dq, dk, dw


@pytest.mark.parametrize("order", ["larger_then_smaller"])
def test_backward_noalloc_matches_the_workspace_entry_point(order):
    for (B, S, Skv, H, D, c, tk, seed) in ((2, 300, 200, 64, 128, 2, 64, 500), (1, 100, 60, 32, 64, 1, 20, 510)):
        print(f"noalloc backward B={B} S={S} Skv={Skv} H={H} D={D} c={c} topk={tk}", flush=True)
        inp, idx, grad = _case(B, S, Skv, H, D, tk, seed)
        q, k, w = (inp[x].to(DEV) for x in "qkw")
        idx_d, grad_d = idx.to(DEV), grad.to(DEV)
        dq, dk, dw = _noalloc(q, k, w, idx_d, grad_d, c)
        rq, rk, rw = lx.indexer_backward(q, k, w, c, idx_d, grad_d)
        torch.cuda.synchronize()
        # dq and dw are deterministic: the same bits as the workspace entry point
        assert torch.equal(dq, rq) and torch.equal(dw, rw)
        # dk sums workgroup partials with float32 atomics: both within the rule against the oracle
        nb = {x: synth.bits(inp[x]) for x in "qkw"}
        ks, ke = oracle.causal_ranges(S, Skv, c)
        grads, bounds = oracle.indexer_backward(nb["q"], nb["k"], nb["w"], idx.numpy(), grad.numpy(), ks, ke,
                                                with_bounds=True)
        for name, got in (("noalloc", dk), ("workspace", rk)):
            checkers.check_backward_one({"dk": got.cpu().numpy()}, "dk", grads[1], bounds["dk"], name)
        checkers.check_backward({"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dw": dw.cpu().numpy()}, grads,
                                bounds, "noalloc")

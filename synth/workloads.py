"""Seeded input generators (CPU, torch.Generator) for every workload.

Draw order is fixed (q, then k, then w, then extras) so a seed names one
input exactly.  All tensors are generated on the CPU; callers copy them to
the device, so the oracle and the GPU see identical bits.

Workloads (shapes and distributions of the lightning-indexer configurations):
  tiny   B=1  S=256     Skv=64     H=64 D=128 c=4 topk=16    seed 0
  4k     B=2  S=4096    Skv=1024   H=64 D=128 c=4 topk=512   seed 1
  32k    B=1  S=32768   Skv=8192   H=64 D=128 c=4 topk=2048  seed 2
  v41    B=1  L=16384   G=4096     H=64 D=128 (c=4 for the mask)  seed 3
  131k   B=1  S=131072  Skv=32768  H=64 D=128 c=4 topk=2048  seed 4,
         with round(0.01*Skv) key rows scaled by 4 (heavy-tailed scores)
q and k are N(0,1) rounded to bf16; w is N(0,1)/sqrt(H*D) in fp32 (bf16 for
V4.1).  V4.1 documents have integer lengths drawn uniformly from [512, 4096]
until they cover L (the last one truncated); ``allowed`` marks key group s as
visible to query t when the group is complete before t (s < (t+1)//4) and
starts inside t's document (4*s >= start of t's document).
"""

import math

import numpy as np
import torch

WORKLOADS = {
    "tiny": dict(batch=1, seqlen=256, seqlen_kv=64, heads=64, index_dim=128,
                 compress_ratio=4, topk=16, seed=0),
    "4k": dict(batch=2, seqlen=4096, seqlen_kv=1024, heads=64, index_dim=128,
               compress_ratio=4, topk=512, seed=1),
    "32k": dict(batch=1, seqlen=32768, seqlen_kv=8192, heads=64, index_dim=128,
                compress_ratio=4, topk=2048, seed=2),
    "v41": dict(batch=1, local_sequence=16384, global_compressed=4096, heads=64,
                index_dim=128, compress_ratio=4, doc_min=512, doc_max=4096, seed=3),
    "131k": dict(batch=1, seqlen=131072, seqlen_kv=32768, heads=64, index_dim=128,
                 compress_ratio=4, topk=2048, seed=4, heavy_fraction=0.01, heavy_scale=4.0),
}


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def v4_inputs(batch, seqlen, seqlen_kv, heads, index_dim, seed,
              heavy_fraction=0.0, heavy_scale=4.0, **_):
    """q bf16 [S,B,H,D], k bf16 [Skv,B,D], w fp32 [S,B,H] (SBHD), CPU tensors."""
    g = _gen(seed)
    q = torch.randn(seqlen, batch, heads, index_dim, generator=g).to(torch.bfloat16)
    k = torch.randn(seqlen_kv, batch, index_dim, generator=g).to(torch.bfloat16)
    w = torch.randn(seqlen, batch, heads, generator=g) / math.sqrt(heads * index_dim)
    if heavy_fraction > 0.0:
        n_heavy = int(round(heavy_fraction * seqlen_kv))
        rows = torch.randperm(seqlen_kv, generator=g)[:n_heavy]
        k[rows] = (k[rows].float() * heavy_scale).to(torch.bfloat16)   # x4 is exact in bf16
    return dict(q=q.contiguous(), k=k.contiguous(), w=w.contiguous())


def v4_exact_inputs(batch, seqlen, seqlen_kv, heads, index_dim, seed, **_):
    """Inputs whose every product and partial sum is exact in fp32.

    q, k are integers in [-2, 2]; w = +-2**-j with j in [0, 6].  A dot product
    is an integer of magnitude <= 4*D, and each weighted term is that integer
    times a power of two, so any summation order gives the same fp32 value.
    """
    g = _gen(seed)
    q = torch.randint(-2, 3, (seqlen, batch, heads, index_dim), generator=g).to(torch.bfloat16)
    k = torch.randint(-2, 3, (seqlen_kv, batch, index_dim), generator=g).to(torch.bfloat16)
    j = torch.randint(0, 7, (seqlen, batch, heads), generator=g).float()
    sgn = torch.randint(0, 2, (seqlen, batch, heads), generator=g).float() * 2 - 1
    w = sgn * torch.pow(2.0, -j)
    return dict(q=q.contiguous(), k=k.contiguous(), w=w.contiguous())


def document_starts(length, doc_min, doc_max, g):
    """Start position of each token's document; lengths ~ U[doc_min, doc_max]."""
    starts = np.empty(length, dtype=np.int64)
    pos = 0
    while pos < length:
        n = int(torch.randint(doc_min, doc_max + 1, (1,), generator=g))
        end = min(length, pos + n)
        starts[pos:end] = pos
        pos = end
    return starts


def v41_inputs(batch, local_sequence, global_compressed, heads, index_dim, seed,
               compress_ratio=4, doc_min=512, doc_max=4096, **_):
    """queries bf16 [B,L,H,D], keys bf16 [B,G,D], weights bf16 [B,L,H], allowed bool [B,L,G]."""
    g = _gen(seed)
    L, G = local_sequence, global_compressed
    queries = torch.randn(batch, L, heads, index_dim, generator=g).to(torch.bfloat16)
    keys = torch.randn(batch, G, index_dim, generator=g).to(torch.bfloat16)
    weights = (torch.randn(batch, L, heads, generator=g) / math.sqrt(heads * index_dim)).to(torch.bfloat16)
    allowed = torch.zeros(batch, L, G, dtype=torch.bool)
    s = torch.arange(G)
    for b in range(batch):
        starts = torch.from_numpy(document_starts(L, doc_min, doc_max, g))
        t = torch.arange(L)
        causal = s[None, :] < ((t + 1) // compress_ratio)[:, None]
        in_doc = (compress_ratio * s)[None, :] >= starts[:, None]
        allowed[b] = causal & in_doc
    return dict(queries=queries.contiguous(), keys=keys.contiguous(),
                weights=weights.contiguous(), allowed=allowed.contiguous())


def v41_exact_inputs(batch, local_sequence, global_compressed, heads, index_dim, seed,
                     density=0.5, **_):
    """Small-integer V4.1 inputs: every dot product is exact in fp32.

    queries and keys are integers in [-3, 3] (so |d| <= 9*D is exact in fp32),
    weights are +-2**-j; ``allowed`` is a Bernoulli(density) mask.
    """
    g = _gen(seed)
    queries = torch.randint(-3, 4, (batch, local_sequence, heads, index_dim), generator=g).to(torch.bfloat16)
    keys = torch.randint(-3, 4, (batch, global_compressed, index_dim), generator=g).to(torch.bfloat16)
    j = torch.randint(0, 7, (batch, local_sequence, heads), generator=g).float()
    sgn = torch.randint(0, 2, (batch, local_sequence, heads), generator=g).float() * 2 - 1
    weights = (sgn * torch.pow(2.0, -j)).to(torch.bfloat16)
    allowed = torch.rand(batch, local_sequence, global_compressed, generator=g) < density
    return dict(queries=queries.contiguous(), keys=keys.contiguous(),
                weights=weights.contiguous(), allowed=allowed.contiguous())


def upstream_gradient(batch, seqlen, topk, seed):
    """grad_scores fp32 [B,S,topk] ~ N(0,1): the gradient a loss sends to the selected scores."""
    g = _gen(seed)
    return torch.randn(batch, seqlen, topk, generator=g, dtype=torch.float32)


def bits(t):
    """CPU tensor -> NumPy array of its raw bits (bf16 -> uint16, fp32 -> float32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.bool:
        return t.numpy()
    return t.numpy()

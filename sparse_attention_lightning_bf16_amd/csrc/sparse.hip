// Indexer scores at given key indices, computed from q, k and w.
//
// Page "...deepseek_v4.kernels.tilelang_indexer", v4_lighting_indexer with
// topk_indices given, and section pytorch_extract_topk_scores: the result is
// the cleaned logit at each given index,
//     out[b,t,j] = sum_h w[t,b,h] * max(0, q[t,b,h,:] . k[i,b,:])   i = indices[b,t,j] in [ks, ke)
//     out[b,t,j] = -inf                                             otherwise,
// but only the given keys are scored: no logits row is formed.
//
// One wave (one workgroup) per (b, t).  Its MFMA rows are the query's heads,
// padded with zero rows of zero weight up to whole 32-row tiles; its columns
// walk the indices in blocks of 32.  A block's key rows are gathered by
// direct global->LDS loads into the wave's own LDS buffer, double buffered,
// so no barrier is needed.  Each load moves whole row segments of up to 128
// bytes (one cache line) per group of lanes, not one 16-byte chunk of 32
// different rows, and places the chunks with an XOR swizzle so that the
// B-fragment reads stay free of bank conflicts (BlockMap).  The MFMA chain
// and the epilogue visit a score's terms in the same order as the scoring
// stage of the logits kernel (padded rows add exact zeros), so each score
// equals the materialized logit bit for bit.
#include "score_core.h"
#include "gathered_block.h"
#include "launch.h"

namespace lix {

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (no wait): vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int kWaitVmcnt0 = 0x0F70;

template <int H_, int DP_>
struct SparseTiling {
    static constexpr int H = H_;
    static constexpr int DP = DP_;
    static constexpr int NRT = H >= 32 ? H / 32 : 1;    // 32-row tiles (heads) per wave
    static constexpr int NSTEP = DP / 16;               // MFMA k-steps over index_dim
    static constexpr int PER = 16 / NSTEP;              // epilogue elements per tile per k-step
    static constexpr int BLOCK_BYTES = NSTEP * 1024;    // one 32-key block in LDS
};

template <int H, int DP>
__global__ __launch_bounds__(64, H >= 128 ? 1 : 2) void sparse_scores_kernel(InLayout L, const float* __restrict__ w,
                                                              const int32_t* __restrict__ indices, int B, int S,
                                                              int skv, int ratio, const int32_t* __restrict__ ks,
                                                              const int32_t* __restrict__ ke, int topk,
                                                              float* __restrict__ out) {
    using T = SparseTiling<H, DP>;
    using M = BlockMap<DP>;
    __shared__ __attribute__((aligned(16))) uint8_t buf0[T::BLOCK_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[T::BLOCK_BYTES];

    const int lane = threadIdx.x, hf = lane >> 5;
    const int b = blockIdx.x % B, t = blockIdx.x / B;
    int lo, hi;
    key_range(ks, ke, t, S, skv, ratio, lo, hi);

    // A fragments: row = head; rows >= H and index_dim entries >= D read as zero.
    bf16x8 a[T::NRT][T::NSTEP];
    const uint16_t* qrow = L.q + (long)t * L.q_t + (long)b * L.q_b;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) {
        const int h = 32 * r + (lane & 31);
        const uint16_t* base = qrow + (long)min(h, H - 1) * L.D;
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const int d0 = 16 * st + 8 * hf;
            u32x4 v = *reinterpret_cast<const u32x4*>(base + min(d0, L.D - 8));
            if (!(h < H && d0 < L.D)) v = u32x4{0u, 0u, 0u, 0u};
            a[r][st] = as_bf16x8(v);
        }
    }
    float wr[T::NRT][16];
    const float* wrow = w + ((long)t * B + b) * H;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 32 * r + c_row(i, hf);
            const float v = wrow[min(h, H - 1)];
            wr[r][i] = (h < H) ? v : 0.0f;
        }

    const int32_t* ib = indices + ((long)b * S + t) * topk;
    float* ob = out + ((long)b * S + t) * topk;
    const uint16_t* kb = L.k + (long)b * L.k_b;
    const int dlim = (L.D >> 3) - 1;
    const int nb = (topk + 31) >> 5;

    // Key index of this lane's entry in block blk (clamped load; the entry
    // number is checked where the index is used, so the load is not waited
    // for until the next block).
    auto load_idx = [&](int blk) { return ib[min(32 * blk + (lane & 31), topk - 1)]; };
    auto visible = [&](int idx, int blk) { return 32 * blk + (lane & 31) < topk && idx >= lo && idx < hi; };
    // Gather the 32 key rows of a block (invalid entries fetch key row 0).
    auto gather = [&](uint8_t* buf, int idx, int blk) {
        gather_block<DP>(buf, kb, L.k_s, dlim, visible(idx, blk) ? idx : 0, lane);
    };
    int fofs[M::KR];
#pragma unroll
    for (int k = 0; k < M::KR; ++k) fofs[k] = M::frag_off(k, lane);
    auto bfrag = [&](const uint8_t* buf, int st) {
        return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + fofs[st % M::KR] + 4096 * (st / M::KR)));
    };
    // Score block blk from buf: the MFMA chain, then the epilogue in the
    // scoring stage's element order, then the half-wave sum.
    auto score = [&](const uint8_t* buf, int blk, int idx, bool active) {
        float res = neg_inf();
        if (active) {
            f32x16 acc[T::NRT];
            bf16x8 bn = bfrag(buf, 0);
#pragma unroll
            for (int st = 0; st < T::NSTEP; ++st) {
                const bf16x8 bc = bn;
                if (st + 1 < T::NSTEP) bn = bfrag(buf, st + 1);
#pragma unroll
                for (int r = 0; r < T::NRT; ++r)
                    acc[r] = mfma_32x32x16(a[r][st], bc, st == 0 ? f32x16{} : acc[r]);
            }
            float pend = 0.0f;
#pragma unroll
            for (int st = 0; st < T::NSTEP; ++st)
#pragma unroll
                for (int r = 0; r < T::NRT; ++r)
#pragma unroll
                    for (int i = st * T::PER; i < (st + 1) * T::PER; ++i)
                        pend = fmaf(wr[r][i], relu(acc[r][i]), pend);
            pend = xor32_add(pend);
            if (visible(idx, blk)) res = pend;
        }
        return res;
    };

    // Block order per step: wait for every outstanding vector-memory
    // operation (the gather of this block, issued one block earlier, the
    // previous block's store and the index loads; all had a block of compute
    // to land), store the previous block, load indices two blocks ahead,
    // gather the next block into the other buffer, score this block.  The
    // explicit wait is what orders the LDS reads after the gather: there is
    // no barrier in a one-wave workgroup.
    float res_p = 0.0f;
    int e_p = -1;                                     // entry of res_p in this lane, or -1
    auto store_prev = [&]() {
        if (hf == 0 && e_p >= 0 && e_p < topk) ob[e_p] = res_p;
    };
    int idx_c = load_idx(0), idx_n = load_idx(1);
    bool act_c = __ballot(visible(idx_c, 0)) != 0ull;
    if (act_c) gather(buf0, idx_c, 0);
    auto step = [&](const uint8_t* cur, uint8_t* other, int blk) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);      // no memory access moves across the wait
        store_prev();
        const int idx_nn = load_idx(blk + 2);
        const bool act_n = (blk + 1 < nb) && __ballot(visible(idx_n, blk + 1)) != 0ull;
        if (act_n) gather(other, idx_n, blk + 1);
        res_p = score(cur, blk, idx_c, act_c);
        e_p = 32 * blk + (lane & 31);
        idx_c = idx_n; act_c = act_n; idx_n = idx_nn;
    };
    for (int blk = 0; blk < nb; blk += 2) {
        step(buf0, buf1, blk);
        if (blk + 1 >= nb) break;
        step(buf1, buf0, blk + 1);
    }
    store_prev();
}

template <int H, int DP>
static hipError_t launch_sparse_t(const SparseArgs& p) {
    InLayout L{static_cast<const uint16_t*>(p.q), (long)p.B * H * p.D, (long)H * p.D,
               static_cast<const uint16_t*>(p.k), (long)p.B * p.D, (long)p.D, p.D};
    dim3 grid((unsigned)((long)p.B * p.S));
    hipLaunchKernelGGL((sparse_scores_kernel<H, DP>), grid, dim3(kWave), 0, p.stream, L, p.w, p.indices, p.B, p.S,
                       p.Skv, p.ratio, p.ks, p.ke, p.topk, p.scores);
    return hipGetLastError();
}

template <int H>
static hipError_t dispatch_dp_sparse(const SparseArgs& p) {
    switch (padded_dim(p.D)) {
        case 32: return launch_sparse_t<H, 32>(p);
        case 64: return launch_sparse_t<H, 64>(p);
        case 128: return launch_sparse_t<H, 128>(p);
        case 256: return launch_sparse_t<H, 256>(p);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sparse_scores(const SparseArgs& p) {
    switch (p.H) {
        case 1: return dispatch_dp_sparse<1>(p);
        case 2: return dispatch_dp_sparse<2>(p);
        case 4: return dispatch_dp_sparse<4>(p);
        case 8: return dispatch_dp_sparse<8>(p);
        case 16: return dispatch_dp_sparse<16>(p);
        case 32: return dispatch_dp_sparse<32>(p);
        case 64: return dispatch_dp_sparse<64>(p);
        case 128: return dispatch_dp_sparse<128>(p);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lix

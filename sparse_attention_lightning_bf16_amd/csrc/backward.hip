// Backward of the indexer scores at given indices: gradients with respect to
// q, k and w.
//
// Page "...deepseek_v4.kernels.tilelang_indexer", V4IndexerFunction.backward
// (grad_scores, grad_indices), by the chain rule on the forward: for each
// valid entry j of query (b, t), key s = idx[b,t,j] in [ks, ke), upstream
// gradient g = grad_scores[b,t,j],
//     d_h = q[t,b,h,:] . k[s,b,:],   m_h = 1[d_h > 0]
//     dw[t,b,h]   += g * max(0, d_h)
//     dq[t,b,h,:] += g * w[t,b,h] * m_h * k[s,b,:]
//     dk[s,b,:]   += g * sum_h w[t,b,h] * m_h * q[t,b,h,:]
// Entries outside [ks, ke) (their score is the constant -inf) and the
// indices themselves get no gradient.
//
// One wave per (b, t), walking the entries in blocks of 32 with the gathered
// key blocks of the scores-at kernel.  Per block:
//   * d is recomputed twice from the same register fragments: D = Q K^T
//     (lanes are keys, accumulator rows heads) and D^T = K Q^T (lanes are
//     heads, rows keys).
//   * dw: g * relu(D^T) summed per lane (head) in registers.
//   * dq += (m * g) K: the A operand is built from D^T's accumulators (the
//     contraction index, the key, runs along each lane's rows), the B operand
//     is the gathered block read key-major with 2-byte reads; dq stays in
//     registers for the whole row and is scaled by w at the end.
//   * the block's rows of dk = (m * w) Q, with the A operand built from D's
//     accumulators and the B operand Q^T, staged in LDS once per query; each
//     row is scaled by its g and added to dk with float32 atomics, issued
//     before the dq product so that they complete while it runs.
// The gradient products take bfloat16 operands (g rounded to bf16 for dq, w
// for dk) and accumulate in float32; dw and the final scalings are float32.
#include "score_core.h"
#include "gathered_block.h"
#include "launch.h"

namespace lix {

namespace {

constexpr int kBwWaitVmcnt0 = 0x0F70;     // s_waitcnt vmcnt(0), expcnt/lgkmcnt untouched

template <int H_, int DP_>
struct BwTiling {
    static constexpr int H = H_;
    static constexpr int DP = DP_;
    static constexpr int NRT = H > 32 ? 2 : 1;       // 32-row head tiles (padded rows are zero)
    static constexpr int NSTEP = DP / 16;            // k-steps of the recompute over index_dim
    static constexpr int NDT = DP / 32;              // 32-column index_dim tiles of dq and dk
    static constexpr int NHS = 2 * NRT;              // 16-head k-steps of the dk product
    static constexpr int QT_BYTES = NHS * NDT * 1024;
    static_assert(H <= 64 && (DP == 64 || DP == 128), "backward tiles cover H <= 64, index_dim 33..128");
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
}

// Keep the low and/or high bf16 of v where the matching accumulator is > 0.
__device__ __forceinline__ uint32_t mask_pair(uint32_t v, float a_lo, float a_hi) {
    const uint32_t m = (a_lo > 0.0f ? 0x0000FFFFu : 0u) | (a_hi > 0.0f ? 0xFFFF0000u : 0u);
    return v & m;
}

}  // namespace

template <int H, int DP>
__global__ __launch_bounds__(64, 1) void indexer_backward_kernel(InLayout L, const float* __restrict__ w,
                                                                const int32_t* __restrict__ indices,
                                                                const float* __restrict__ grad, int B, int S,
                                                                int skv, int ratio, const int32_t* __restrict__ ks,
                                                                const int32_t* __restrict__ ke, int topk,
                                                                float* __restrict__ dq, float* __restrict__ dk,
                                                                float* __restrict__ dw) {
    using T = BwTiling<H, DP>;
    using M = BlockMap<DP>;
    __shared__ __attribute__((aligned(16))) uint8_t buf0[M::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[M::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t qt[T::QT_BYTES];
    __shared__ float wsh[64];
    __shared__ __attribute__((aligned(16))) float stage_g[32];
    __shared__ __attribute__((aligned(16))) int32_t stage_i[32];

    const int lane = threadIdx.x, hf = lane >> 5, l32 = lane & 31;
    const int b = blockIdx.x % B, t = blockIdx.x / B;
    const int D = L.D;
    int lo, hi;
    key_range(ks, ke, t, S, skv, ratio, lo, hi);

    // Q fragments: a[r][st] = q[head 32r + lane%32][16 st + 8 hf .. +7]; heads >= H
    // and index_dim entries >= D are zero.
    bf16x8 a[T::NRT][T::NSTEP];
    const uint16_t* qrow = L.q + (long)t * L.q_t + (long)b * L.q_b;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) {
        const int h = 32 * r + l32;
        const uint16_t* base = qrow + (long)min(h, H - 1) * D;
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const int d0 = 16 * st + 8 * hf;
            u32x4 v = *reinterpret_cast<const u32x4*>(base + min(d0, D - 8));
            if (!(h < H && d0 < D)) v = u32x4{0u, 0u, 0u, 0u};
            a[r][st] = as_bf16x8(v);
        }
    }
    // Q^T for the dk product: fragment (hs, dt), lane l holds q[head][32 dt + l%32]
    // for the 8 heads 32(hs/2) + 16(hs%2) + 8(jj/4) + 4(l/32) + jj%4, jj = 0..7 (the
    // order in which the dk A operand walks a D accumulator's rows).
    {
        const int sq = l32 >> 4, ho = l32 & 15;
        const int jj = 4 * (ho >> 3) + (ho & 3), hw = (ho >> 2) & 1;
#pragma unroll
        for (int r = 0; r < T::NRT; ++r)
#pragma unroll
            for (int st = 0; st < T::NSTEP; ++st) {
                const u32x4 v = __builtin_bit_cast(u32x4, a[r][st]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = 16 * st + 8 * hf + e;
                    const int off = ((2 * r + sq) * T::NDT + (d >> 5)) * 1024 + 16 * ((d & 31) + 32 * hw) + 2 * jj;
                    *reinterpret_cast<uint16_t*>(qt + off) = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                }
            }
    }
    // w of the query's heads in LDS (0 for padded heads); wpk[r][p] holds, as
    // bf16, rows i = 2p, 2p+1 of tile r (heads 32r + c_row(i, hf)).
    const float* wrow = w + ((long)t * B + b) * H;
    {
        const float v = wrow[min(lane, H - 1)];
        wsh[lane] = lane < H ? v : 0.0f;
    }
    uint32_t wpk[T::NRT][8];
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int p = 0; p < 8; ++p)
            wpk[r][p] = pack_bf16(wsh[32 * r + c_row(2 * p, hf)], wsh[32 * r + c_row(2 * p + 1, hf)]);
    // Key-major reads of a gathered block: element (key 16s + 8(jj/4) + 4hf + jj%4,
    // index_dim 32dt + lane%32) lies at kbase[dt%2][(jj%4) ^ (jj/4)]
    // + 1024(4(dt/2) + 2s + jj/4) + 128(jj%4) (the BlockMap placement, 8-chunk segments).
    int kbase[2][4];
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
        for (int x = 0; x < 4; ++x)
            kbase[p2][x] = 512 * hf + 64 * (p2 ^ hf) + 16 * ((l32 >> 3) ^ x) + 2 * (lane & 7);
    int fofs[M::KR];
#pragma unroll
    for (int kq = 0; kq < M::KR; ++kq) fofs[kq] = M::frag_off(kq, lane);

    const int32_t* irow = indices + ((long)b * S + t) * topk;
    const float* grow = grad + ((long)b * S + t) * topk;
    const uint16_t* kb = L.k + (long)b * L.k_b;
    const int dlim = (D >> 3) - 1;
    const int nb = (topk + 31) >> 5;

    // This lane's entry of block blk is 32 blk + lane%32 (clamped loads; the
    // entry number is checked where it is used).
    auto load_idx = [&](int blk) { return irow[min(32 * blk + l32, topk - 1)]; };
    auto load_g = [&](int blk) { return grow[min(32 * blk + l32, topk - 1)]; };
    auto visible = [&](int idx, int blk) { return 32 * blk + l32 < topk && idx >= lo && idx < hi; };
    // g and key row of the entries on this lane's accumulator rows (row i is
    // entry 32 blk + c_row(i, hf)), through LDS: invalid entries get g = 0 and
    // row -1.  One wave: its LDS operations run in order, no barrier needed.
    auto rows_from_lanes = [&](float g_own, int idx_own, bool vis, float (&gv)[16], int (&iv)[16]) {
        if (hf == 0) {
            stage_g[l32] = vis ? g_own : 0.0f;
            stage_i[l32] = vis ? idx_own : -1;
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 gg = *reinterpret_cast<const float4*>(stage_g + 8 * q4 + 4 * hf);
            const int4 ii = *reinterpret_cast<const int4*>(stage_i + 8 * q4 + 4 * hf);
            gv[4 * q4 + 0] = gg.x; gv[4 * q4 + 1] = gg.y; gv[4 * q4 + 2] = gg.z; gv[4 * q4 + 3] = gg.w;
            iv[4 * q4 + 0] = ii.x; iv[4 * q4 + 1] = ii.y; iv[4 * q4 + 2] = ii.z; iv[4 * q4 + 3] = ii.w;
        }
    };

    f32x16 dqacc[T::NRT][T::NDT];
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt) dqacc[r][dt] = f32x16{};
    float dwacc[T::NRT];
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) dwacc[r] = 0.0f;
    typedef __attribute__((address_space(1))) float gfloat;
    gfloat* const dkb = (gfloat*)dk + (long)b * D + l32;

    auto compute = [&](const uint8_t* buf, float g_own, int idx_own, bool vis) {
        f32x16 accd[T::NRT], acct[T::NRT];
#pragma unroll
        for (int r = 0; r < T::NRT; ++r) { accd[r] = f32x16{}; acct[r] = f32x16{}; }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + fofs[st % M::KR] + 4096 * (st / M::KR)));
#pragma unroll
            for (int r = 0; r < T::NRT; ++r) {
                accd[r] = mfma_32x32x16(a[r][st], kf, accd[r]);
                acct[r] = mfma_32x32x16(kf, a[r][st], acct[r]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        float gv[16];
        int iv[16];
        rows_from_lanes(g_own, idx_own, vis, gv, iv);
        // The block's rows of dk = (m * w) Q, scaled by each row's g, added to dk
        // (first, so that the adds overlap the rest of the block).
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt) {
            f32x16 dkt = f32x16{};
#pragma unroll
            for (int r = 0; r < T::NRT; ++r)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    u32x4 av;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        av[p] = mask_pair(wpk[r][4 * s + p], accd[r][8 * s + 2 * p], accd[r][8 * s + 2 * p + 1]);
                    const bf16x8 qf = as_bf16x8(
                        *reinterpret_cast<const u32x4*>(qt + ((2 * r + s) * T::NDT + dt) * 1024 + 16 * lane));
                    dkt = mfma_32x32x16(as_bf16x8(av), qf, dkt);
                }
            // An invalid row adds +0.0 to key row 0: dk starts at +0.0 and never
            // holds -0.0, so that add changes nothing (and needs no branch).
            if (32 * dt + l32 < D) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    __hip_atomic_fetch_add(dkb + (long)max(iv[i], 0) * B * D + 32 * dt,
                                           iv[i] >= 0 ? dkt[i] * gv[i] : 0.0f, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // dw: lane = head 32r + lane%32, rows = keys c_row(i, hf).
#pragma unroll
        for (int r = 0; r < T::NRT; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) dwacc[r] = fmaf(gv[i], relu(acct[r][i]), dwacc[r]);
        // dq += (m * g) K over the block's 32 keys (two k-steps of 16).
        uint32_t gpk[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) gpk[p] = pack_bf16(gv[2 * p], gv[2 * p + 1]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 kt[T::NDT];
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) {
                uint32_t pk[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t half[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int jj = 2 * p + u;
                        const int off = kbase[dt & 1][(jj & 3) ^ (jj >> 2)] + 1024 * (4 * (dt >> 1) + 2 * s + (jj >> 2)) +
                                        128 * (jj & 3);
                        half[u] = *reinterpret_cast<const uint16_t*>(buf + off);
                    }
                    pk[p] = half[0] | (half[1] << 16);
                }
                kt[dt] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
            }
#pragma unroll
            for (int r = 0; r < T::NRT; ++r) {
                u32x4 av;
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    av[p] = mask_pair(gpk[4 * s + p], acct[r][8 * s + 2 * p], acct[r][8 * s + 2 * p + 1]);
                const bf16x8 af = as_bf16x8(av);
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt) dqacc[r][dt] = mfma_32x32x16(af, kt[dt], dqacc[r][dt]);
            }
        }
    };

    // Block order per step: wait for every outstanding vector-memory operation
    // (this block's gather and g, issued one step earlier, and the previous
    // step's dk adds), load the next block's g and the indices two blocks
    // ahead, gather the next block into the other buffer, compute this block.  The explicit wait orders the LDS
    // reads after the gather (one wave, no barrier).
    int idx_c = load_idx(0), idx_n = load_idx(1);
    float g_c = load_g(0);
    bool act_c = __ballot(visible(idx_c, 0)) != 0ull;
    if (act_c) gather_block<DP>(buf0, kb, L.k_s, dlim, visible(idx_c, 0) ? idx_c : 0, lane);
    for (int blk = 0; blk < nb; ++blk) {
        const uint8_t* cur = (blk & 1) ? buf1 : buf0;
        uint8_t* other = (blk & 1) ? buf0 : buf1;
        __builtin_amdgcn_s_waitcnt(kBwWaitVmcnt0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const float g_n = load_g(blk + 1);
        const int idx_nn = load_idx(blk + 2);
        const bool act_n = (blk + 1 < nb) && __ballot(visible(idx_n, blk + 1)) != 0ull;
        if (act_n) gather_block<DP>(other, kb, L.k_s, dlim, visible(idx_n, blk + 1) ? idx_n : 0, lane);
        if (act_c) compute(cur, g_c, idx_c, visible(idx_c, blk));
        idx_c = idx_n; act_c = act_n; idx_n = idx_nn; g_c = g_n;
    }

    // dq = w * accumulated (m g) K: rows are heads 32r + c_row(i, hf), columns
    // index_dim 32 dt + lane%32.
    float* dqrow = dq + ((long)t * B + b) * H * D;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 32 * r + c_row(i, hf);
            if (H < 32 && h >= H) continue;
            const float wh = wsh[h];
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) {
                const int d = 32 * dt + l32;
                if (d < D) dqrow[(long)h * D + d] = wh * dqacc[r][dt][i];
            }
        }
    // dw: the two half-waves hold the same heads over different keys.
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) {
        const float v = xor32_add(dwacc[r]);
        const int h = 32 * r + l32;
        if (hf == 0 && h < H) dw[((long)t * B + b) * H + h] = v;
    }
}

__global__ void zero_f32_kernel(float* __restrict__ p, long n4) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x)
        reinterpret_cast<float4*>(p)[i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
}

template <int H, int DP>
static hipError_t launch_backward_t(const BackwardArgs& p) {
    InLayout L{static_cast<const uint16_t*>(p.q), (long)p.B * H * p.D, (long)H * p.D,
               static_cast<const uint16_t*>(p.k), (long)p.B * p.D, (long)p.D, p.D};
    hipLaunchKernelGGL((indexer_backward_kernel<H, DP>), dim3((unsigned)((long)p.B * p.S)), dim3(kWave), 0, p.stream,
                       L, p.w, p.indices, p.grad, p.B, p.S, p.Skv, p.ratio, p.ks, p.ke, p.topk, p.dq, p.dk, p.dw);
    return hipGetLastError();
}

template <int H>
static hipError_t dispatch_dp_backward(const BackwardArgs& p) {
    switch (padded_dim(p.D)) {
        case 64: return launch_backward_t<H, 64>(p);
        case 128: return launch_backward_t<H, 128>(p);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_indexer_backward(const BackwardArgs& p) {
    // dk accumulates: clear it first (a fill kernel, so the sequence can be captured).
    const long n4 = (long)p.Skv * p.B * p.D / 4;
    const long blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, p.stream,
                       p.dk, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (p.H) {
        case 1: return dispatch_dp_backward<1>(p);
        case 2: return dispatch_dp_backward<2>(p);
        case 4: return dispatch_dp_backward<4>(p);
        case 8: return dispatch_dp_backward<8>(p);
        case 16: return dispatch_dp_backward<16>(p);
        case 32: return dispatch_dp_backward<32>(p);
        case 64: return dispatch_dp_backward<64>(p);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lix

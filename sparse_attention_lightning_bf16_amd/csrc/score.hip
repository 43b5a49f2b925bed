// Scoring kernels: V4 masked fp32 logits (materialized) and V4.1 BF16 scores.
//
// V4 (page "...deepseek_v4.kernels.tilelang_indexer_fwd", batched_indexer_fwd
// and clean_logits_):
//     logits[b,t,s] = sum_h w[t,b,h] * max(0, q[t,b,h,:] . k[s,b,:])  for s in [ks,ke)
//     logits[b,t,s] = -inf                                            otherwise
// V4.1 (page "...deepseek_v41.indexer", module description, indexer_scores):
//     out[b,t,s] = bf16( sum_h bf16( w[b,t,h] * max(0, bf16(q[b,t,h,:] . k[b,s,:])) ) )
// where allowed[b,t,s], bf16 -inf elsewhere; the head sum is fp32.
//
// One workgroup = 4 waves = QB consecutive queries of one batch element.
// Key stages [s0, s0+64) that lie outside every range of the workgroup are
// never computed (causal tile skip); their logits are filled with -inf.
#include "score_core.h"
#include "launch.h"

namespace lix {

template <class T>
__device__ __forceinline__ void load_weights_f32(float (&wr)[T::NRT][16], const float* __restrict__ w, long w_t,
                                                 long w_b, int b, int tq0, int S, int lane) {
    const int hf = lane >> 5;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * r + c_row(i, hf);
            const int t = tq0 + row / T::H, h = row % T::H;
            const float v = w[(long)min(t, S - 1) * w_t + (long)b * w_b + h];
            wr[r][i] = (t < S) ? v : 0.0f;
        }
}

// ---------------------------------------------------------------- V4 logits

template <int H, int DP>
__global__ __launch_bounds__(256, stage_min_waves(H, DP)) void v4_logits_kernel(InLayout L, const float* __restrict__ w, int B, int S,
                                                        int skv, int ratio, const int32_t* __restrict__ ks,
                                                        const int32_t* __restrict__ ke, float* __restrict__ out) {
    using T = Tiling<H, DP>;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[T::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[T::STAGE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5;
    const int nqb = (S + T::QB - 1) / T::QB;
    const int nblk = nqb * B;
    const int G = gridDim.x;
    // block j: batch j % B, query block nqb-1-j/B (longest causal rows first)
    auto block_b = [&](int j) { return j % B; };
    auto block_t0 = [&](int j) { return (nqb - 1 - j / B) * T::QB; };

    for (int i = 0;; ++i) {
        const int j = sched_block(blockIdx.x, G, i);
        if (j >= nblk) break;
        const int b = block_b(j), t0 = block_t0(j);
        const int tq0 = t0 + wave * T::QW;
        bf16x8 a[T::NRT][T::NSTEP];
        load_q_frags<T>(a, L, b, tq0, S, lane);
        float wr[T::NRT][16];
        load_weights_f32<T>(wr, w, (long)B * H, H, b, tq0, S, lane);

        // Key span of the workgroup, in whole stages.
        int wg_lo = skv, wg_hi = 0;
        for (int q = 0; q < T::QB; ++q) {
            int lo, hi;
            key_range(ks, ke, t0 + q, S, skv, ratio, lo, hi);
            if (hi > lo) { wg_lo = min(wg_lo, lo); wg_hi = max(wg_hi, hi); }
        }
        const int tile_lo = (wg_hi > wg_lo) ? wg_lo / T::KT : 0;
        const int tile_hi = (wg_hi > wg_lo) ? (wg_hi + T::KT - 1) / T::KT : 0;
        const int span_lo = tile_lo * T::KT, span_hi = min(skv, tile_hi * T::KT);
        const int ntile = tile_hi - tile_lo;

        int lo_s[T::QW], hi_s[T::QW];
        int wave_lo = skv, wave_hi = 0;
#pragma unroll
        for (int q = 0; q < T::QW; ++q)
            key_range(ks, ke, slot_query<T>(tq0, q, hf), S, skv, ratio, lo_s[q], hi_s[q]);
        for (int q = 0; q < T::QW; ++q) {
            int lo, hi;
            key_range(ks, ke, tq0 + q, S, skv, ratio, lo, hi);
            if (hi > lo) { wave_lo = min(wave_lo, lo); wave_hi = max(wave_hi, hi); }
        }

        float* out_b = out + (long)b * S * skv;
        // Results of a stage are stored at the start of the next one (see
        // stream_key_stages): pend[cb][q], first key of that stage pend_s0.
        float pend[T::NCB][T::QW];
        int pend_s0 = -1;
        auto flush = [&]() {
            if (pend_s0 < 0) return;
            if constexpr (H >= 8) {
                // Both halves hold full sums; per pair of column blocks the lower
                // half writes the first and the upper half the second: 64
                // consecutive keys per query and store.
#pragma unroll
                for (int cp = 0; cp < T::NCB / 2; ++cp) {
                    const int s = pend_s0 + 64 * cp + lane;
#pragma unroll
                    for (int q = 0; q < T::QW; ++q) {
                        const int t = tq0 + q;
                        if (t < S && s < skv) {
                            const float v = pick(hf != 0, pend[2 * cp + 1][q], pend[2 * cp][q]);
                            __builtin_nontemporal_store((s >= lo_s[q] && s < hi_s[q]) ? v : neg_inf(),
                                                        out_b + (long)t * skv + s);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int cb = 0; cb < T::NCB; ++cb) {
                    const int s = pend_s0 + 32 * cb + (lane & 31);
#pragma unroll
                    for (int q = 0; q < T::QW; ++q) {
                        if ((q % (2 * T::half_step())) >= T::half_step()) continue;   // slot owned via hf
                        const int t = slot_query<T>(tq0, q, hf);
                        if (t < S && s < skv)
                            __builtin_nontemporal_store((s >= lo_s[q] && s < hi_s[q]) ? pend[cb][q] : neg_inf(),
                                                        out_b + (long)t * skv + s);
                    }
                }
            }
        };
        if (ntile > 0) {
            stream_key_stages<T>(L, b, skv, tile_lo, ntile, lds0, lds1, tid, [&](int it, const uint8_t* stage) {
                flush();
                const int s0 = (tile_lo + it) * T::KT;
                const bool active = (s0 < wave_hi) && (s0 + T::KT > wave_lo);
#pragma unroll
                for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
                    for (int q = 0; q < T::QW; ++q) pend[cb][q] = 0.0f;
                if (active) {
                    rolling_stage<T>(a, stage, lane, [&](int cb, const f32x16 (&acc)[T::NRT], int r, int i) {
                        pend[cb][T::slot(r, i)] = fmaf(wr[r][i], relu(acc[r][i]), pend[cb][T::slot(r, i)]);
                    });
                    if constexpr (H >= 8) {
#pragma unroll
                        for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
                            for (int q = 0; q < T::QW; ++q) pend[cb][q] = xor32_add(pend[cb][q]);
                    }
                }
                pend_s0 = s0;
            });
            flush();
        }
        // -inf outside the staged span: no query of the block sees those keys.
        for (int q = 0; q < T::QB; ++q) {
            const int t = t0 + q;
            if (t >= S) break;
            float* row = out_b + (long)t * skv;
            fill_neg_inf(row, span_lo, tid, T::THREADS);
            fill_neg_inf(row + span_hi, skv - span_hi, tid, T::THREADS);
        }
    }
}

// ---------------------------------------------------------------- V4.1 scores

template <int H, int DP>
__global__ __launch_bounds__(256, stage_min_waves(H, DP)) void v41_scores_kernel(InLayout L, const uint16_t* __restrict__ wts,
                                                         const uint8_t* __restrict__ allowed, int B, int Lq,
                                                         int G, uint16_t* __restrict__ out) {
    using T = Tiling<H, DP>;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[T::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[T::STAGE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5;
    const int nqb = (Lq + T::QB - 1) / T::QB;
    const int b = blockIdx.x % B;
    const int qb = nqb - 1 - (int)(blockIdx.x / B);
    const int t0 = qb * T::QB;
    const int tq0 = t0 + wave * T::QW;
    const int ntile = (G + T::KT - 1) / T::KT;

    bf16x8 a[T::NRT][T::NSTEP];
    load_q_frags<T>(a, L, b, tq0, Lq, lane);
    float wr[T::NRT][16];
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * r + c_row(i, hf);
            const int t = tq0 + row / H, h = row % H;
            wr[r][i] = (t < Lq) ? bf16_to_f32(wts[((long)b * Lq + t) * H + h]) : 0.0f;
        }

    const uint16_t kNegInfBf16 = 0xff80u;
    stream_key_stages<T>(L, b, G, 0, ntile, lds0, lds1, tid, [&](int it, const uint8_t* stage) {
        const int s0 = it * T::KT;
        // Visibility of this lane's keys for each of its queries.
        bool vis[T::NCB][T::QW];
        bool any = false;
#pragma unroll
        for (int cb = 0; cb < T::NCB; ++cb) {
            const int s = s0 + 32 * cb + (lane & 31);
#pragma unroll
            for (int j = 0; j < T::QW; ++j) {
                const int t = slot_query<T>(tq0, j, hf);
                vis[cb][j] = (t < Lq && s < G) ? (allowed[((long)b * Lq + t) * G + s] != 0) : false;
                any |= vis[cb][j];
            }
        }
        const bool active = __ballot(any) != 0ull;

        float part[T::NCB][T::QW];
#pragma unroll
        for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
            for (int j = 0; j < T::QW; ++j) part[cb][j] = 0.0f;
        if (active) {
            auto term = [&](float acc_v, float w_v) {
                const float rr = round_bf16(relu(acc_v));    // bf16(d); ReLU commutes with rounding
                return round_bf16(w_v * rr);                  // exact product, then bf16
            };
            rolling_stage<T>(a, stage, lane, [&](int cb, const f32x16 (&acc)[T::NRT], int r, int i) {
                part[cb][T::slot(r, i)] += term(acc[r][i], wr[r][i]);
            });
            if constexpr (H >= 8) {
#pragma unroll
                for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
                    for (int j = 0; j < T::QW; ++j) part[cb][j] = xor32_add(part[cb][j]);
            }
        }

#pragma unroll
        for (int cb = 0; cb < T::NCB; ++cb) {
            const int s = s0 + 32 * cb + (lane & 31);
#pragma unroll
            for (int j = 0; j < T::QW; ++j) {
                if constexpr (H >= 8) {
                    if (hf != (cb & 1)) continue;      // lower half stores even blocks, upper half odd
                } else {
                    if ((j % (2 * T::half_step())) >= T::half_step()) continue;
                }
                const int t = slot_query<T>(tq0, j, hf);
                if (t < Lq && s < G)
                    out[((long)b * Lq + t) * G + s] = vis[cb][j] ? bf16_bits(part[cb][j]) : kNegInfBf16;
            }
        }
    });
}

// ---------------------------------------------------------------- launchers

template <int H, int DP>
static hipError_t launch_v4_logits_t(const LogitsArgs& p) {
    using T = Tiling<H, DP>;
    InLayout L{static_cast<const uint16_t*>(p.q), (long)p.B * H * p.D, (long)H * p.D,
               static_cast<const uint16_t*>(p.k), (long)p.B * p.D, (long)p.D, p.D};
    const long nblk = (long)((p.S + T::QB - 1) / T::QB) * p.B;
    dim3 grid((unsigned)nblk);                 // one block per workgroup (see sched_block)
    hipLaunchKernelGGL((v4_logits_kernel<H, DP>), grid, dim3(T::THREADS), 0, p.stream, L, p.w, p.B, p.S, p.Skv,
                       p.ratio, p.ks, p.ke, p.logits);
    return hipGetLastError();
}

template <int H, int DP>
static hipError_t launch_v41_t(const V41Args& p) {
    using T = Tiling<H, DP>;
    InLayout L{static_cast<const uint16_t*>(p.queries), (long)H * p.D, (long)p.L * H * p.D,
               static_cast<const uint16_t*>(p.keys), (long)p.D, (long)p.G * p.D, p.D};
    const int nqb = (p.L + T::QB - 1) / T::QB;
    dim3 grid((unsigned)((long)nqb * p.B));
    hipLaunchKernelGGL((v41_scores_kernel<H, DP>), grid, dim3(T::THREADS), 0, p.stream, L,
                       static_cast<const uint16_t*>(p.weights), p.allowed, p.B, p.L, p.G,
                       static_cast<uint16_t*>(p.scores));
    return hipGetLastError();
}

template <int H>
static hipError_t dispatch_dp_logits(const LogitsArgs& p) {
    switch (padded_dim(p.D)) {
        case 32: return launch_v4_logits_t<H, 32>(p);
        case 64: return launch_v4_logits_t<H, 64>(p);
        case 128: return launch_v4_logits_t<H, 128>(p);
        case 256: return launch_v4_logits_t<H, 256>(p);
        default: return hipErrorInvalidValue;
    }
}

template <int H>
static hipError_t dispatch_dp_v41(const V41Args& p) {
    switch (padded_dim(p.D)) {
        case 32: return launch_v41_t<H, 32>(p);
        case 64: return launch_v41_t<H, 64>(p);
        case 128: return launch_v41_t<H, 128>(p);
        case 256: return launch_v41_t<H, 256>(p);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_v4_logits(const LogitsArgs& p) {
    switch (p.H) {
        case 1: return dispatch_dp_logits<1>(p);
        case 2: return dispatch_dp_logits<2>(p);
        case 4: return dispatch_dp_logits<4>(p);
        case 8: return dispatch_dp_logits<8>(p);
        case 16: return dispatch_dp_logits<16>(p);
        case 32: return dispatch_dp_logits<32>(p);
        case 64: return dispatch_dp_logits<64>(p);
        case 128: return dispatch_dp_logits<128>(p);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_v41_scores(const V41Args& p) {
    switch (p.H) {
        case 1: return dispatch_dp_v41<1>(p);
        case 2: return dispatch_dp_v41<2>(p);
        case 4: return dispatch_dp_v41<4>(p);
        case 8: return dispatch_dp_v41<8>(p);
        case 16: return dispatch_dp_v41<16>(p);
        case 32: return dispatch_dp_v41<32>(p);
        case 64: return dispatch_dp_v41<64>(p);
        case 128: return dispatch_dp_v41<128>(p);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lix

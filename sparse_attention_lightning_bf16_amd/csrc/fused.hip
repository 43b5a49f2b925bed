// Fused scoring + streaming top-k: v4_lighting_indexer's forward with no
// [B,S,Skv] logits in memory (page "...deepseek_v4.kernels.tilelang_indexer",
// v4_lighting_indexer / V4IndexerFunction.forward with topk_indices = None).
//
// The scoring loop is the one of the materialized kernel.  Instead of storing
// a stage's 64 scores per query, each wave appends the ones that can still
// reach its query's top-k to a candidate buffer in LDS:
//   * a candidate is accepted when its order-preserving key exceeds the
//     query's threshold thr (initially below every real score);
//   * when an append would overflow the buffer (capacity cap > topk), the
//     wave compacts it in place to its topk best entries (radix select,
//     8-bit digits, lower index wins ties) and raises thr to the key of the
//     topk-th best.  A later key can only enter the final top-k if it beats
//     that entry (ties go to the lower, earlier index), so dropping every
//     key <= thr is exact.
// The buffer stays in index order (appends are in key order and compaction
// is stable), so the final selection writes the top-k in ascending key order,
// exactly as the row top-k over materialized logits does.
#include "score_core.h"
#include "launch.h"

namespace lix {

__device__ __forceinline__ int lanes_below_f(unsigned long long mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

// Select the `want` best of keys/idx[0..cnt) (key descending, index
// ascending).  OUT = false: compact them in place to [0..want) keeping index
// order.  OUT = true: write them, in index order, as scores/indices.
// Returns the key of the want-th best entry.  Wave-local: `hist` (256 words)
// belongs to this wave; all 64 lanes must call it together.
template <bool OUT>
__device__ uint32_t wave_select(uint32_t* keys, uint16_t* idx, int cnt, int want, uint32_t* hist, int lane,
                                float* __restrict__ so, int32_t* __restrict__ io) {
    uint32_t prefix = 0, pmask = 0;
    int need = want;
    const int nch = (cnt + 63) >> 6;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0u;
        for (int c = 0; c < nch; ++c) {
            const int e = 64 * c + lane;
            if (e < cnt) {
                const uint32_t key = keys[e];
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
        }
        // lane l owns bins 4l..4l+3; suffix sums over higher bins
        int h[4];
        int local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) { h[i] = (int)hist[4 * lane + i]; local += h[i]; }
        int v = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_down(v, off, 64);
            if (lane + off < 64) v += u;
        }
        int above = v - local;
        int bin = -1, rank = 0;
        if (above < need && need <= above + local) {
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                if (bin < 0) {
                    if (need <= above + h[i]) { bin = 4 * lane + i; rank = need - above; }
                    else above += h[i];
                }
            }
        }
        const unsigned long long found = __ballot(bin >= 0);
        const int src = __ffsll((long long)found) - 1;
        bin = __shfl(bin, src, 64);
        rank = __shfl(rank, src, 64);
        prefix |= (uint32_t)bin << shift;
        pmask |= 255u << shift;
        need = rank;
    }
    const uint32_t T = prefix;
    const int need_eq = need;

    int run_out = 0, run_eq = 0;
    for (int c = 0; c < nch; ++c) {
        const int e = 64 * c + lane;
        const bool valid = e < cnt;
        const uint32_t key = valid ? keys[e] : 0u;
        const int id = valid ? (int)idx[e] : 0;
        const bool is_gt = valid && key > T;
        const bool is_eq = valid && key == T;
        const unsigned long long eqm = __ballot(is_eq);
        const bool sel = is_gt || (is_eq && run_eq + lanes_below_f(eqm, lane) < need_eq);
        const unsigned long long selm = __ballot(sel);
        const int pos = run_out + lanes_below_f(selm, lane);
        if (sel && pos < want) {
            if constexpr (OUT) {
                so[pos] = key_to_f32(key);
                io[pos] = id;
            } else {
                keys[pos] = key;
                idx[pos] = (uint16_t)id;
            }
        }
        run_out += __popcll(selm);
        run_eq += __popcll(eqm);
    }
    return T;
}

// Make room in a full candidate buffer: keys[0..cnt) binned linearly in the
// score between the smallest and largest (256 bins, monotone); every key in the
// bins from the one holding the want-th best upward is kept, in index order,
// and the rest is dropped.  At least want kept keys are strictly above every
// dropped key, so a later key that is not above the largest dropped one
// cannot enter the final top-want (ties go to the earlier, lower index): that
// key becomes the new threshold, returned in *thr.  Returns the kept count,
// or -1 (buffer untouched) when the boundary bin is so crowded that fewer than
// `room` slots would be freed; the caller then selects exactly.  Wave-local:
// `hist` (256 words) belongs to this wave; all 64 lanes call it together.
__device__ int wave_prune(uint32_t* keys, uint16_t* idx, int cnt, int want, int room, uint32_t* hist, int lane,
                          uint32_t* thr) {
    const int nch = (cnt + 63) >> 6;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int c = 0; c < nch; ++c) {
        const int e = 64 * c + lane;
        if (e < cnt) { const uint32_t k = keys[e]; kmin = min(kmin, k); kmax = max(kmax, k); }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off, 64));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off, 64));
    }
    // bins linear in the score (the keys' order is the scores' order)
    const float vmin = key_to_f32(kmin), span = key_to_f32(kmax) - vmin;
    if (!(span > 1.0e-30f && span < 3.0e38f)) return -1;      // one value, or a range the scale cannot hold
    const float sc = 255.0f / span;
    auto bin_of = [&](uint32_t k) { return min(255, (int)((key_to_f32(k) - vmin) * sc)); };
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0u;
    for (int c = 0; c < nch; ++c) {
        const int e = 64 * c + lane;
        if (e < cnt) atomicAdd(&hist[bin_of(keys[e])], 1u);
    }
    // bin holding the want-th best: lane l owns bins 4l..4l+3
    int h[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[i] = (int)hist[4 * lane + i]; local += h[i]; }
    int v = local;                                            // suffix sum over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_down(v, off, 64);
        if (lane + off < 64) v += u;
    }
    int above = v - local, bin = -1, kept = 0;
    if (above < want && want <= above + local) {
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            if (bin < 0) {
                if (want <= above + h[i]) { bin = 4 * lane + i; kept = above + h[i]; }
                else above += h[i];
            }
        }
    }
    const unsigned long long found = __ballot(bin >= 0);
    const int src = found ? __ffsll((long long)found) - 1 : 0;
    bin = __shfl(bin, src, 64);
    kept = __shfl(kept, src, 64);
    if (bin < 0 || cnt - kept < room) return -1;
    // keep bins >= bin in order; the largest dropped key is the new threshold
    int run = 0;
    uint32_t dmax = 0u;
    for (int c = 0; c < nch; ++c) {
        const int e = 64 * c + lane;
        const bool valid = e < cnt;
        const uint32_t k = valid ? keys[e] : 0u;
        const int id = valid ? (int)idx[e] : 0;
        const bool keep = valid && bin_of(k) >= bin;
        if (valid && !keep) dmax = max(dmax, k);
        const unsigned long long km = __ballot(keep);
        if (keep) {
            const int pos = run + lanes_below_f(km, lane);   // <= e: nothing unread is overwritten
            keys[pos] = k;
            idx[pos] = (uint16_t)id;
        }
        run += __popcll(km);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dmax = max(dmax, (uint32_t)__shfl_xor((int)dmax, off, 64));
    *thr = max(*thr, dmax);
    return run;
}

template <int H, int DP>
__global__ __launch_bounds__(256) void v4_fused_topk_kernel(InLayout L, const float* __restrict__ w, int B, int S,
                                                            int skv, int ratio, const int32_t* __restrict__ ks,
                                                            const int32_t* __restrict__ ke, int topk, int cap,
                                                            float* __restrict__ scores,
                                                            int32_t* __restrict__ indices) {
    using T = FusedTiling<H, DP>;
    static_assert(H >= 8, "the fused path keeps each query inside one lane pair");
    __shared__ __attribute__((aligned(16))) uint8_t lds0[T::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[T::STAGE_BYTES];
    __shared__ uint32_t hist_all[T::NWAVE][256];
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];

    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int nqb = (S + T::QB - 1) / T::QB;
    const int b = blockIdx.x % B;
    const int qb = nqb - 1 - (int)(blockIdx.x / B);
    const int t0 = qb * T::QB;
    const int tq0 = t0 + wave * T::QW;
    uint32_t* hist = hist_all[wave];

    // Candidate buffers of this wave's queries.
    uint32_t* bkey[T::QW];
    uint16_t* bidx[T::QW];
#pragma unroll
    for (int j = 0; j < T::QW; ++j) {
        const int qs = wave * T::QW + j;
        bkey[j] = reinterpret_cast<uint32_t*>(dyn) + (long)qs * cap;
        bidx[j] = reinterpret_cast<uint16_t*>(dyn + (long)T::QB * cap * 4) + (long)qs * cap;
    }

    int wg_lo = skv, wg_hi = 0;
    for (int j = 0; j < T::QB; ++j) {
        int lo, hi;
        key_range(ks, ke, t0 + j, S, skv, ratio, lo, hi);
        if (hi > lo) { wg_lo = min(wg_lo, lo); wg_hi = max(wg_hi, hi); }
    }
    const int tile_lo = (wg_hi > wg_lo) ? wg_lo / T::KT : 0;
    const int tile_hi = (wg_hi > wg_lo) ? (wg_hi + T::KT - 1) / T::KT : 0;
    const int ntile = tile_hi - tile_lo;

    int lo_s[T::QW], hi_s[T::QW], cnt[T::QW];
    uint32_t thr[T::QW];
    int wave_lo = skv, wave_hi = 0;
#pragma unroll
    for (int j = 0; j < T::QW; ++j) {
        key_range(ks, ke, tq0 + j, S, skv, ratio, lo_s[j], hi_s[j]);
        if (hi_s[j] > lo_s[j]) { wave_lo = min(wave_lo, lo_s[j]); wave_hi = max(wave_hi, hi_s[j]); }
        cnt[j] = 0;
        thr[j] = 0u;
    }

    if (ntile > 0) {
        bf16x8 a[T::NRT][T::NSTEP];
        load_q_frags<T>(a, L, b, tq0, S, lane);
        float wr[T::NRT][16];
#pragma unroll
        for (int r = 0; r < T::NRT; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * r + c_row(i, hf);
                const int t = tq0 + row / H, h = row % H;
                wr[r][i] = (t < S) ? w[((long)t * B + b) * H + h] : 0.0f;
            }

        stream_key_stages<T>(L, b, skv, tile_lo, ntile, lds0, lds1, tid, [&](int it, const uint8_t* stage) {
            const int s0 = (tile_lo + it) * T::KT;
            const bool active = (s0 < wave_hi) && (s0 + T::KT > wave_lo);
            if (!active) return;
            float part[T::NCB][T::QW];
#pragma unroll
            for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
                for (int j = 0; j < T::QW; ++j) part[cb][j] = 0.0f;
            // same accumulation order as the materialized logits kernel; column
            // blocks past the wave's last visible key are left out
            const int ncb = __builtin_amdgcn_readfirstlane(min(T::NCB, (wave_hi - s0 + 31) >> 5));
            rolling_stage_first<T>(a, stage, lane, ncb, [&](int cb, const f32x16 (&acc)[T::NRT], int r, int i) {
                part[cb][T::slot(r, i)] = fmaf(wr[r][i], relu(acc[r][i]), part[cb][T::slot(r, i)]);
            });
#pragma unroll
            for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
                for (int j = 0; j < T::QW; ++j) part[cb][j] = xor32_add(part[cb][j]);

            // Per pair of column blocks, lane l holds key s0 + 64 cp + l of each of
            // its queries (the lower half's sums are block 2cp's, the upper half's
            // block 2cp+1's); keys are appended in ascending order.
#pragma unroll
            for (int cp = 0; cp < T::NCB / 2; ++cp)
#pragma unroll
            for (int j = 0; j < T::QW; ++j) {
                const int s = s0 + 64 * cp + lane;
                const float v = pick(hf != 0, part[2 * cp + 1][j], part[2 * cp][j]);
                const uint32_t key = f32_to_key(v);
                const bool in_range = (s >= lo_s[j]) && (s < hi_s[j]);
                bool acc_ok = in_range && key > thr[j];
                unsigned long long m = __ballot(acc_ok);
                if (m != 0ull && cnt[j] + __popcll(m) > cap) {
                    const int kept = wave_prune(bkey[j], bidx[j], cnt[j], topk, kWave, hist, lane, &thr[j]);
                    if (kept >= 0) {
                        cnt[j] = kept;
                    } else {
                        thr[j] = wave_select<false>(bkey[j], bidx[j], cnt[j], topk, hist, lane, nullptr, nullptr);
                        cnt[j] = topk;
                    }
                    acc_ok = in_range && key > thr[j];
                    m = __ballot(acc_ok);
                }
                if (acc_ok) {
                    const int pos = cnt[j] + lanes_below_f(m, lane);
                    bkey[j][pos] = key;
                    bidx[j][pos] = (uint16_t)s;
                }
                cnt[j] += __popcll(m);
            }
        });
    }

    // Final selection per query, then padding.
#pragma unroll
    for (int j = 0; j < T::QW; ++j) {
        const int t = tq0 + j;
        if (t >= S) continue;
        float* so = scores + ((long)b * S + t) * topk;
        int32_t* io = indices + ((long)b * S + t) * topk;
        const int n = hi_s[j] - lo_s[j];
        const int m = min(topk, n);
        if (cnt[j] <= topk) {
            for (int e = lane; e < cnt[j]; e += 64) {
                so[e] = key_to_f32(bkey[j][e]);
                io[e] = bidx[j][e];
            }
        } else {
            wave_select<true>(bkey[j], bidx[j], cnt[j], m, hist, lane, so, io);
        }
        for (int e = m + lane; e < topk; e += 64) {
            so[e] = neg_inf();
            io[e] = -1;
        }
    }
}

template <int H, int DP>
static hipError_t launch_fused_t(const FusedArgs& p) {
    using T = FusedTiling<H, DP>;
    const long cap = fused_cap<H, DP>(p.topk);
    if (cap < 0) return hipErrorInvalidValue;
    const size_t dyn = (size_t)T::QB * cap * 6;
    auto kern = v4_fused_topk_kernel<H, DP>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    InLayout L{static_cast<const uint16_t*>(p.q), (long)p.B * H * p.D, (long)H * p.D,
               static_cast<const uint16_t*>(p.k), (long)p.B * p.D, (long)p.D, p.D};
    const int nqb = (p.S + T::QB - 1) / T::QB;
    dim3 grid((unsigned)((long)nqb * p.B));
    hipLaunchKernelGGL(kern, grid, dim3(T::THREADS), dyn, p.stream, L, p.w, p.B, p.S, p.Skv, p.ratio, p.ks, p.ke,
                       p.topk, (int)cap, p.scores, p.indices);
    return hipGetLastError();
}

template <int H>
static hipError_t dispatch_fused_dp(const FusedArgs& p) {
    switch (padded_dim(p.D)) {
        case 32: return launch_fused_t<H, 32>(p);
        case 64: return launch_fused_t<H, 64>(p);
        case 128: return launch_fused_t<H, 128>(p);
        case 256: return launch_fused_t<H, 256>(p);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused_topk(const FusedArgs& p) {
    switch (p.H) {
        case 8: return dispatch_fused_dp<8>(p);
        case 16: return dispatch_fused_dp<16>(p);
        case 32: return dispatch_fused_dp<32>(p);
        case 64: return dispatch_fused_dp<64>(p);
        case 128: return dispatch_fused_dp<128>(p);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lix

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
// One workgroup = 4 or 8 waves (logits_wg_waves, v41_waves) = QB consecutive
// queries of one batch element.  Key stages [s0, s0+KT) that lie outside
// every range of the workgroup are never computed (causal tile skip); their
// logits are filled with -inf, except by lix_indexer_logits_visible.  In the
// stage holding a wave's last visible key, the 32-key column blocks past it
// are left out as well.
#include "score_core.h"
#include "row_select.h"
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

// SELECT = false (lix_indexer_logits): out is the [B,S,Skv] logits; each
// workgroup handles one query block; positions outside the staged span are
// filled with -inf when FILL (lix_indexer_logits_visible leaves them as
// they are).
// SELECT = true (lix_topk_streaming): out is the workspace, one slot of
// QB rows of skv floats per workgroup; the grid is persistent (workgroup w
// handles blocks sched_block(w, gridDim.x, i)), a block's scores go to the
// workgroup's slot (only the staged span is written), and right after the
// block's stage loop the workgroup selects each of its rows' top-k from the
// slot (select_row_binned, the selection of the row top-k kernel; the rows
// are still in L2) into scores / indices [B,S,topk].  Requires skv <= 8192.
constexpr int logits_wg_waves(int H, int DP, bool select) { return select ? 4 : logits_waves(H, DP); }

template <int H, int DP, bool SELECT>
using LogitsTiling = Tiling<H, DP, default_kt(H, DP), logits_wg_waves(H, DP, SELECT)>;

template <int H, int DP, bool SELECT, bool FILL = !SELECT>
__global__ __launch_bounds__(kWave * logits_wg_waves(H, DP, SELECT), stage_min_waves(H, DP)) void v4_logits_kernel(InLayout L, const float* __restrict__ w, int B, int S,
                                                        int skv, int ratio, const int32_t* __restrict__ ks,
                                                        const int32_t* __restrict__ ke, float* __restrict__ out,
                                                        int topk, float* __restrict__ scores,
                                                        int32_t* __restrict__ indices) {
    using T = LogitsTiling<H, DP, SELECT>;
    // The two stage buffers; in SELECT mode the selection state reuses them
    // (the array grows where it is larger than both).
    constexpr int kStages = 2 * T::STAGE_BYTES;
    constexpr int kBytes = (SELECT && (int)sizeof(BinShared) > kStages) ? (int)sizeof(BinShared) : kStages;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kBytes];
    uint8_t* const lds0 = lds;
    uint8_t* const lds1 = lds + T::STAGE_BYTES;

    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
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

        // Row of query t: its logits row, or its row in the workgroup's slot.
        auto row_off = [&](int t) -> long {
            if constexpr (SELECT) return ((long)blockIdx.x * T::QB + (t - t0)) * skv;
            else return ((long)b * S + t) * skv;
        };
        // Logits go past the caches (nothing reads them back soon); slot
        // rows are read back by this workgroup right after the block.
        auto put = [](float v, float* p) {
            if constexpr (SELECT) *p = v;
            else __builtin_nontemporal_store(v, p);
        };
        // Results of a stage are stored at the start of the next one (see
        // stream_key_stages): pend[cb][q], first key of that stage pend_s0.
        float pend[T::NCB][T::QW];
        int pend_s0 = -1;
        auto flush = [&]() {
            if (pend_s0 < 0) return;
            if constexpr (H >= 8) {
                // Both halves hold full sums; per pair of column blocks the lower
                // half writes the first and the upper half the second: 64
                // consecutive keys per query and store.  (For H >= 8 a slot's
                // query and range are wave-uniform: a stage inside every range
                // of the wave stores without per-key checks.)
                bool inside = pend_s0 + T::KT <= skv;
#pragma unroll
                for (int q = 0; q < T::QW; ++q)
                    inside = inside && tq0 + q < S && lo_s[q] <= pend_s0 && pend_s0 + T::KT <= hi_s[q];
                if (inside) {
#pragma unroll
                    for (int cp = 0; cp < T::NCB / 2; ++cp) {
                        const int s = pend_s0 + 64 * cp + lane;
#pragma unroll
                        for (int q = 0; q < T::QW; ++q)
                            put(pick(hf != 0, pend[2 * cp + 1][q], pend[2 * cp][q]),
                                                        out + row_off(tq0 + q) + s);
                    }
                    return;
                }
#pragma unroll
                for (int cp = 0; cp < T::NCB / 2; ++cp) {
                    const int s = pend_s0 + 64 * cp + lane;
#pragma unroll
                    for (int q = 0; q < T::QW; ++q) {
                        const int t = tq0 + q;
                        if (t < S && s < skv) {
                            const float v = pick(hf != 0, pend[2 * cp + 1][q], pend[2 * cp][q]);
                            put((s >= lo_s[q] && s < hi_s[q]) ? v : neg_inf(),
                                                        out + row_off(t) + s);
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
                            put((s >= lo_s[q] && s < hi_s[q]) ? pend[cb][q] : neg_inf(),
                                                        out + row_off(t) + s);
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
                    // column blocks up to the wave's last visible key
                    const int ncb = __builtin_amdgcn_readfirstlane(min(T::NCB, (wave_hi - s0 + 31) >> 5));
                    rolling_stage_first<T>(a, stage, lane, ncb, [&](int cb, const f32x16 (&acc)[T::NRT], int r, int i) {
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
        if constexpr (!SELECT) {
            // -inf outside the staged span: no query of the block sees those keys
            // (left out when only the visible logits are asked for).
            for (int q = 0; q < T::QB && FILL; ++q) {
                const int t = t0 + q;
                if (t >= S) break;
                float* row = out + row_off(t);
                fill_neg_inf(row, span_lo, tid, T::THREADS);
                fill_neg_inf(row + span_hi, skv - span_hi, tid, T::THREADS);
            }
        } else {
            // The block's rows are in the slot (every store of the workgroup
            // has completed at the barrier); select each row's top-k.  The
            // selection state reuses the stage buffers.
            static_assert(!SELECT || T::THREADS == kBinThreads, "the selection runs on the whole workgroup");
            BinShared& sh = *reinterpret_cast<BinShared*>(lds);
            for (int q = 0; q < T::QB; ++q) {
                const int t = t0 + q;
                if (t >= S) break;
                __syncthreads();
                int lo, hi;
                key_range(ks, ke, t, S, skv, ratio, lo, hi);
                // The range is the same in every lane; loaded after this
                // workgroup's stores it arrives in vector registers.
                lo = __builtin_amdgcn_readfirstlane(lo);
                hi = __builtin_amdgcn_readfirstlane(hi);
                const long o = ((long)b * S + t) * topk;
                select_row_binned<8, false>(out + row_off(t) + lo, hi - lo, lo, topk, scores + o, indices + o, sh,
                                            tid);
            }
            __syncthreads();      // before the next block writes the stage buffers and the slot
        }
    }
}

// ---------------------------------------------------------------- V4.1 scores

// Span [lo, hi) of keys visible to any of the workgroup's rows t0..t0+nrows-1
// (hi <= lo when none is): a scan of those rows of `allowed` by the whole
// workgroup, 16 bytes per load where rows are 16-byte aligned.  Ends with a
// barrier.
template <int NT>
__device__ __forceinline__ void allowed_span(const uint8_t* __restrict__ rows0, int nrows, int G, int tid,
                                             int* sh_lo, int* sh_hi, int& lo, int& hi) {
    if (tid == 0) { *sh_lo = G; *sh_hi = 0; }
    __syncthreads();
    int my_lo = G, my_hi = 0;
    const bool vec = ((reinterpret_cast<uintptr_t>(rows0) | (uintptr_t)G) & 15) == 0;
    if (vec) {
        // Rows are contiguous, so chunk c covers bytes 16c .. 16c+15 of the
        // rows' block; four clamped loads per thread are in flight at once.
        const int nch = nrows * (G >> 4);
        for (int c0 = 0; c0 < nch; c0 += 4 * NT) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = *reinterpret_cast<const u32x4*>(rows0 + 16L * min(c0 + u * NT + tid, nch - 1));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * NT + tid;
                if (c >= nch) continue;
                const int s0 = (int)((16L * c) % G);
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (w[i] != 0u) {
                        my_lo = min(my_lo, s0 + 4 * i + (__builtin_ctz(w[i]) >> 3));
                        my_hi = max(my_hi, s0 + 4 * i + ((31 - __builtin_clz(w[i])) >> 3) + 1);
                    }
                }
            }
        }
    } else {
        for (long e = tid; e < (long)nrows * G; e += NT) {
            if (rows0[e] != 0) {
                const int sidx = (int)(e % G);
                my_lo = min(my_lo, sidx);
                my_hi = max(my_hi, sidx + 1);
            }
        }
    }
    if (my_lo < my_hi) { atomicMin(sh_lo, my_lo); atomicMax(sh_hi, my_hi); }
    __syncthreads();
    lo = *sh_lo;
    hi = *sh_hi;
}

// Fill p[0..n) of bf16 with -inf (0xFF80), 16 bytes per store where aligned.
__device__ __forceinline__ void fill_bf16_neg_inf(uint16_t* __restrict__ p, long n, int tid, int nthreads) {
    if (n <= 0) return;
    long head = (long)(((16 - ((uintptr_t)p & 15)) & 15) >> 1);
    if (head > n) head = n;
    for (long i = tid; i < head; i += nthreads) p[i] = 0xff80u;
    uint16_t* body = p + head;
    const long nb = (n - head) >> 3;
    const u32x4 v = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
    for (long i = tid; i < nb; i += nthreads) reinterpret_cast<u32x4*>(body)[i] = v;
    for (long i = head + 8 * nb + tid; i < n; i += nthreads) p[i] = 0xff80u;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// acc + bf16(w0 * max(0, bf16(d0))) + bf16(w1 * max(0, bf16(d1))) for two
// heads of one query: both dots rounded to bf16 by one packed convert (round
// to nearest even), the ReLU as a packed int16 max with 0 (a bf16 with the
// sign bit set is a negative int16; -0 becomes +0), the products with the
// bf16 weights exact in fp32 and rounded by one packed convert, and the two
// terms added to the fp32 sum by one bf16 dot product with (1, 1).
__device__ __forceinline__ float v41_pair_terms(float d0, float d1, float w0, float w1, float acc) {
    const bf16x2 r = __builtin_convertvector(f32x2{d0, d1}, bf16x2);
    const i16x2 rm = __builtin_elementwise_max(__builtin_bit_cast(i16x2, r), i16x2{0, 0});
    const uint32_t u = __builtin_bit_cast(uint32_t, rm);
    const float r0 = __uint_as_float(u << 16), r1 = __uint_as_float(u & 0xffff0000u);
    const bf16x2 e = __builtin_convertvector(f32x2{w0 * r0, w1 * r1}, bf16x2);
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(e, ones, acc, false);
}

// Key stages of the V4.1 kernel: 64 keys.  On the packed-document mask most
// of a workgroup's time is its own memory traffic (queries, mask rows, the
// -inf fill) around a few stages, so it runs three waves per SIMD where the
// registers allow (index_dim <= 128, heads >= 8: plain_stage, no rolling
// epilogue) to overlap one workgroup's loads with another's MFMAs.
// Waves per workgroup: four (three workgroups per CU); eight waves sharing each
// stage measured 14% slower on the packed-document workload.
constexpr int v41_waves(int /*H*/, int /*DP*/) { return 4; }
template <int H, int DP>
using V41Tiling = Tiling<H, DP, 64, v41_waves(H, DP)>;
constexpr int v41_min_waves(int H, int DP) {
    return H < 8 ? 1                                     // rolling_stage: its own register budget
         : H == 128 ? (DP <= 64 ? 2 : 1)                 // 128 heads: the query fragments alone are large
         : DP > 128 ? 1
         : (H == 8 && DP > 64) ? 2                       // 8 heads, index_dim 128: spills at three
         : 3;
}

template <int H, int DP>
__global__ __launch_bounds__(kWave * v41_waves(H, DP), v41_min_waves(H, DP)) void v41_scores_kernel(InLayout L, const uint16_t* __restrict__ wts,
                                                         const uint8_t* __restrict__ allowed, int B, int Lq,
                                                         int G, uint16_t* __restrict__ out) {
    using T = V41Tiling<H, DP>;
    constexpr bool PAIRS = H >= 8;           // a query's heads fill lane pairs: the paired epilogue
    __shared__ __attribute__((aligned(16))) uint8_t lds0[T::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[T::STAGE_BYTES];
    __shared__ int span_lo, span_hi;

    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int nqb = (Lq + T::QB - 1) / T::QB;
    const int b = blockIdx.x % B;
    const int qb = nqb - 1 - (int)(blockIdx.x / B);
    const int t0 = qb * T::QB;
    const int tq0 = t0 + wave * T::QW;
    const int nrows = min(T::QB, Lq - t0);
    const uint8_t* al_b = allowed + (long)b * Lq * G;

    // Query fragments and weights are requested first so their latency
    // overlaps the span scan.
    bf16x8 a[T::NRT][T::NSTEP];
    load_q_frags<T>(a, L, b, tq0, Lq, lane);
    float wr[T::NRT][16];
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * r + c_row(i, hf);
            const int t = tq0 + row / H, h = row % H;
            const float v = bf16_to_f32(wts[((long)b * Lq + min(t, Lq - 1)) * H + h]);
            wr[r][i] = (t < Lq) ? v : 0.0f;
        }

    // Keys visible to some row of the workgroup, in whole stages; the rest of
    // the rows is hidden and filled with -inf below without being computed.
    int vlo, vhi;
    allowed_span<T::THREADS>(al_b + (long)t0 * G, nrows, G, tid, &span_lo, &span_hi, vlo, vhi);
    const int tile_lo = (vhi > vlo) ? vlo / T::KT : 0;
    const int tile_hi = (vhi > vlo) ? (vhi + T::KT - 1) / T::KT : 0;
    const int ntile = tile_hi - tile_lo;
    const int fill_lo = tile_lo * T::KT, fill_hi = min(G, tile_hi * T::KT);

    const uint16_t kNegInfBf16 = 0xff80u;
    if (ntile > 0) {

        // Visibility bytes of this lane's keys, loaded one stage ahead (the
        // barrier that opens a stage waits for them with the key tile).
        uint8_t nxt[T::NCB][T::QW];
        auto load_vis = [&](int s0) {
#pragma unroll
            for (int cb = 0; cb < T::NCB; ++cb) {
                const int s = min(s0 + 32 * cb + (lane & 31), G - 1);
#pragma unroll
                for (int j = 0; j < T::QW; ++j) {
                    const int t = min(slot_query<T>(tq0, j, hf), Lq - 1);
                    nxt[cb][j] = al_b[(long)t * G + s];
                }
            }
        };
        load_vis(fill_lo);
        stream_key_stages<T>(L, b, G, tile_lo, ntile, lds0, lds1, tid, [&](int it, const uint8_t* stage) {
            const int s0 = (tile_lo + it) * T::KT;
            bool vis[T::NCB][T::QW];
            bool any = false;
#pragma unroll
            for (int cb = 0; cb < T::NCB; ++cb) {
                const int s = s0 + 32 * cb + (lane & 31);
#pragma unroll
                for (int j = 0; j < T::QW; ++j) {
                    const int t = slot_query<T>(tq0, j, hf);
                    vis[cb][j] = (t < Lq && s < G) && nxt[cb][j] != 0;
                    any |= vis[cb][j];
                }
            }
            if (it + 1 < ntile) load_vis(s0 + T::KT);
            const bool active = __ballot(any) != 0ull;
            // Column blocks with no key visible to any of the wave's queries
            // skip their epilogue (their MFMAs run in the pipeline regardless;
            // every output of such a block is -inf).
            bool blk_live[T::NCB];
#pragma unroll
            for (int cb = 0; cb < T::NCB; ++cb) {
                bool v = false;
#pragma unroll
                for (int j = 0; j < T::QW; ++j) v |= vis[cb][j];
                blk_live[cb] = __ballot(v) != 0ull;
            }

            float part[T::NCB][T::QW];
#pragma unroll
            for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
                for (int j = 0; j < T::QW; ++j) part[cb][j] = 0.0f;
            if (active) {
                if constexpr (PAIRS) {
                    // heads in pairs (elements i, i + 1 share a query)
                    plain_stage<T>(a, stage, lane, [&](int cb, const f32x16 (&acc)[T::NRT]) {
                        if (!blk_live[cb]) return;
#pragma unroll
                        for (int r = 0; r < T::NRT; ++r)
#pragma unroll
                            for (int i = 0; i < 16; i += 2)
                                part[cb][T::slot(r, i)] = v41_pair_terms(acc[r][i], acc[r][i + 1], wr[r][i],
                                                                         wr[r][i + 1], part[cb][T::slot(r, i)]);
                    });
#pragma unroll
                    for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
                        for (int j = 0; j < T::QW; ++j) part[cb][j] = xor32_add(part[cb][j]);
                } else {
                    rolling_stage<T>(a, stage, lane, [&](int cb, const f32x16 (&acc)[T::NRT], int r, int i) {
                        if (blk_live[cb]) {
                            const float rr = round_bf16(relu(acc[r][i]));    // bf16(d); ReLU commutes with rounding
                            part[cb][T::slot(r, i)] += round_bf16(wr[r][i] * rr);   // exact product, then bf16
                        }
                    });
                }
            }

            if constexpr (PAIRS) {
                // Per pair of column blocks lane l holds key s0 + 64 cp + l (the
                // lower half's sums are block 2cp's, the upper half's block
                // 2cp+1's): one store of 64 consecutive keys per query.
#pragma unroll
                for (int cp = 0; cp < T::NCB / 2; ++cp) {
                    const int s = s0 + 64 * cp + lane;
#pragma unroll
                    for (int j = 0; j < T::QW; ++j) {
                        const int t = tq0 + j;
                        const float v = pick(hf != 0, part[2 * cp + 1][j], part[2 * cp][j]);
                        const bool vv = hf ? vis[2 * cp + 1][j] : vis[2 * cp][j];
                        if (t < Lq && s < G) out[((long)b * Lq + t) * G + s] = vv ? bf16_bits(v) : kNegInfBf16;
                    }
                }
            } else {
#pragma unroll
                for (int cb = 0; cb < T::NCB; ++cb) {
                    const int s = s0 + 32 * cb + (lane & 31);
#pragma unroll
                    for (int j = 0; j < T::QW; ++j) {
                        if ((j % (2 * T::half_step())) >= T::half_step()) continue;
                        const int t = slot_query<T>(tq0, j, hf);
                        if (t < Lq && s < G)
                            out[((long)b * Lq + t) * G + s] = vis[cb][j] ? bf16_bits(part[cb][j]) : kNegInfBf16;
                    }
                }
            }
        });
    }
    // Hidden outside the streamed span.
    for (int q = 0; q < nrows; ++q) {
        uint16_t* orow = out + ((long)b * Lq + t0 + q) * G;
        fill_bf16_neg_inf(orow, fill_lo, tid, T::THREADS);
        fill_bf16_neg_inf(orow + fill_hi, G - fill_hi, tid, T::THREADS);
    }
}

// ---------------------------------------------------------------- launchers

template <int H, int DP>
static hipError_t launch_v4_logits_t(const LogitsArgs& p) {
    using T = LogitsTiling<H, DP, false>;
    InLayout L{static_cast<const uint16_t*>(p.q), (long)p.B * H * p.D, (long)H * p.D,
               static_cast<const uint16_t*>(p.k), (long)p.B * p.D, (long)p.D, p.D};
    const long nblk = (long)((p.S + T::QB - 1) / T::QB) * p.B;
    dim3 grid((unsigned)nblk);                 // one block per workgroup (see sched_block)
    if (p.fill)
        hipLaunchKernelGGL((v4_logits_kernel<H, DP, false, true>), grid, dim3(T::THREADS), 0, p.stream, L, p.w, p.B,
                           p.S, p.Skv, p.ratio, p.ks, p.ke, p.logits, 0, nullptr, nullptr);
    else
        hipLaunchKernelGGL((v4_logits_kernel<H, DP, false, false>), grid, dim3(T::THREADS), 0, p.stream, L, p.w, p.B,
                           p.S, p.Skv, p.ratio, p.ks, p.ke, p.logits, 0, nullptr, nullptr);
    return hipGetLastError();
}

// Persistent grid of the streaming top-k: as many workgroups as are resident
// at once on the device (occupancy x compute units), at most one per block.
template <int H, int DP>
static hipError_t streaming_grid_t(int B, int S, long* grid) {
    using T = LogitsTiling<H, DP, true>;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, v4_logits_kernel<H, DP, true>, T::THREADS, 0);
    if (e != hipSuccess) return e;
    const long nblk = (long)((S + T::QB - 1) / T::QB) * B;
    const long resident = (long)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    *grid = nblk < resident ? nblk : resident;
    return hipSuccess;
}

template <int H, int DP>
static hipError_t launch_streaming_t(const StreamArgs& p) {
    using T = LogitsTiling<H, DP, true>;
    InLayout L{static_cast<const uint16_t*>(p.q), (long)p.B * H * p.D, (long)H * p.D,
               static_cast<const uint16_t*>(p.k), (long)p.B * p.D, (long)p.D, p.D};
    long grid = 0;
    const hipError_t e = streaming_grid_t<H, DP>(p.B, p.S, &grid);
    if (e != hipSuccess) return e;
    const long slot = (long)T::QB * p.Skv * 4;
    const long fit = p.workspace_bytes / slot;
    if (fit < grid) grid = fit;
    if (grid < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((v4_logits_kernel<H, DP, true>), dim3((unsigned)grid), dim3(T::THREADS), 0, p.stream, L,
                       p.w, p.B, p.S, p.Skv, p.ratio, p.ks, p.ke, p.workspace, p.topk, p.scores, p.indices);
    return hipGetLastError();
}

template <int H, int DP>
static hipError_t launch_v41_t(const V41Args& p) {
    using T = V41Tiling<H, DP>;
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

template <int H>
static hipError_t dispatch_dp_streaming(const StreamArgs& p, long* grid) {
    switch (padded_dim(p.D)) {
        case 32: return grid ? streaming_grid_t<H, 32>(p.B, p.S, grid) : launch_streaming_t<H, 32>(p);
        case 64: return grid ? streaming_grid_t<H, 64>(p.B, p.S, grid) : launch_streaming_t<H, 64>(p);
        case 128: return grid ? streaming_grid_t<H, 128>(p.B, p.S, grid) : launch_streaming_t<H, 128>(p);
        case 256: return grid ? streaming_grid_t<H, 256>(p.B, p.S, grid) : launch_streaming_t<H, 256>(p);
        default: return hipErrorInvalidValue;
    }
}

// grid == nullptr: launch; else: store the persistent grid size only.
static hipError_t dispatch_streaming(const StreamArgs& p, long* grid) {
    switch (p.H) {
        case 1: return dispatch_dp_streaming<1>(p, grid);
        case 2: return dispatch_dp_streaming<2>(p, grid);
        case 4: return dispatch_dp_streaming<4>(p, grid);
        case 8: return dispatch_dp_streaming<8>(p, grid);
        case 16: return dispatch_dp_streaming<16>(p, grid);
        case 32: return dispatch_dp_streaming<32>(p, grid);
        case 64: return dispatch_dp_streaming<64>(p, grid);
        case 128: return dispatch_dp_streaming<128>(p, grid);
        default: return hipErrorInvalidValue;
    }
}

hipError_t streaming_grid(int B, int S, int H, int D, long* grid) {
    StreamArgs p{};
    p.B = B; p.S = S; p.H = H; p.D = D;
    return dispatch_streaming(p, grid);
}

hipError_t launch_topk_streaming(const StreamArgs& p) { return dispatch_streaming(p, nullptr); }

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

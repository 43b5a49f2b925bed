// Exact top-k of one score row by a workgroup of 256 threads, with the row in
// registers (rows of at most 8192 keys): shared by the row top-k kernels over
// materialized scores (topk.hip) and the streaming mode of the scoring kernel
// (score.hip), so both select the same keys and write the same bits.
//
// Selection rule (page "...deepseek_v4.kernels.tilelang_indexer",
// v4_lighting_indexer: select topk indices per query): the m = min(topk, n)
// largest scores, equal scores ordered by key index (the lower first),
// written in ascending key-index order; slots [m, topk) hold index -1 and
// score -inf.  Scores are copied bit for bit.
#pragma once

#include <type_traits>

#include "common.h"

namespace lix {

constexpr int kBins = 2048;
// Word 3 of a raw buffer resource on gfx9 (32-bit data format; the range
// check against num_records is on).
constexpr int kBufWord3 = 0x00020000;

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS): shifts by
// 1, 2, 4, 8 inside each row of 16 lanes, then the totals of rows 0 and 2
// broadcast into rows 1 and 3 (row_bcast:15), then the total of rows 0-1 into
// rows 2 and 3 (row_bcast:31).  Lanes without a source add the `old` value 0.
__device__ __forceinline__ int wave_incl_scan(int x, int /*lane*/) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return x;
}

// ---------------------------------------------------------------- binned workgroup row top-k
//
// Rows of at most 1024*NCH visible keys, one workgroup (four waves) per row.
// The row is cut into chunks of 256 keys dealt round-robin to the waves:
// chunk c = 4j + w sits in wave w's registers as x[j][m] = key 256c + 64m +
// lane (one coalesced 4- or 2-byte load per slot), so every wave holds about
// a quarter of any row; the row's last, partial chunk holds NaN past the row.
// Walking chunk c's slots in m order visits its keys in ascending order, 64
// at a time, so the output position of a selected slot is the selection count
// of the chunks before c, plus a wave-uniform running count, plus the
// selected lanes below it (mbcnt over the compare mask): no per-lane scans.
//
// The bin of a score is a monotone function of it: u = v*sc + c0 lies in
// [1, 2) for every v in [vmin, vmax] (sc = (1 - 2^-11)/span, c0 = 1 + 2^-12 -
// vmin*sc; one fma, and the margins of 2^-12 absorb the rounding of c0 while
// |vmin*sc| <= 256; otherwise u = (v - vmin)*sc + 1 + 2^-12), so the 11
// leading mantissa bits of u are a linear bin in 0..2047.  A 2048-bin LDS
// histogram locates the bin holding the topk-th best element; that bin's
// elements (a handful for smooth score distributions) are gathered and ranked
// exactly by (score descending, key index ascending), which gives the cut
// element (vT, iT).  Equal scores share a bin, so the ranking also tells
// whether any other key ties with vT; when none does, the selection is the
// single compare v >= vT.  A boundary bin of more than kBinCand elements, or a
// row whose score range is zero or not finite, falls back to a radix select
// on order-preserving keys.
constexpr int kBinCand = 256;
constexpr int kBinThreads = 256;                  // four waves: rows of up to 8192 keys
constexpr int kBinMaxWaves = 16;                  // sixteen waves: rows of up to 32768 keys
constexpr int kBinChunks = 128;                   // 256-key chunks per row (32768 keys)

struct BinShared {
    alignas(16) uint32_t hist[kBins];
    alignas(16) float cand_v[kBinCand];
    alignas(16) int cand_i[kBinCand];
    int ccnt[kBinChunks];                         // per-chunk counts, row order
    float wmin[kBinMaxWaves], wmax[kBinMaxWaves];
    int wtot[kBinMaxWaves];
    int ncand;
    int bstar, rstar;
    float cut_v;
    int cut_i;
    int cut_ties;                                 // another key has score vT
};

// Block-wide (NW waves): the bin holding the need-th largest element of
// hist[0..NB) and the element's 1-based rank inside it, counted from the top,
// into sh.bstar / sh.rstar.  Thread tid owns bins [BPT*tid, BPT*tid + BPT)
// (none past the last bin), read rotated by tid so a wave's reads spread over
// the LDS banks; the suffix sums over lanes come from a DPP prefix scan.
// Every thread calls it; it ends with a barrier.  Requires 1 <= need <= sum
// of hist.
template <int NB, int NW>
__device__ void block_find_bin(BinShared& sh, int need, int tid) {
    constexpr int BPT = NB >= 64 * NW ? NB / (64 * NW) : 1;
    const int lane = tid & 63, wv = tid >> 6;
    const int base = BPT * tid;
    int local = 0;
    if (base < NB) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) local += (int)sh.hist[base + ((i + tid) & (BPT - 1))];
    }
    const int incl = wave_incl_scan(local, lane);
    const int wsum = __builtin_amdgcn_readlane(incl, 63);
    const int v = wsum - incl + local;               // inclusive suffix sum over lanes >= this one
    if (lane == 0) sh.wtot[wv] = wsum;
    __syncthreads();
    int above = v - local;
    for (int w2 = wv + 1; w2 < NW; ++w2) above += sh.wtot[w2];
    if (base < NB && above < need && need <= above + local) {
        for (int i = BPT - 1; i >= 0; --i) {
            const int h = (int)sh.hist[base + i];
            if (need <= above + h) {
                sh.bstar = base + i;
                sh.rstar = need - above;
                break;
            }
            above += h;
        }
    }
    __syncthreads();
}

// One wave: the bin holding the need-th largest element of hist[0..NB) and
// the element's 1-based rank inside it, counted from the top, into sh.bstar /
// sh.rstar, in two levels: lane l sums bins [32l, 32l + 32) (16-byte reads,
// rotated by lane across the LDS banks) and a DPP scan finds the lane whose
// bins hold it; then lane i < 32 takes that lane's bin i and a second scan
// finds the bin.  Requires 1 <= need <= sum of hist.
template <int NB>
__device__ __forceinline__ void wave_find_bin_lds(BinShared& sh, int need, int lane) {
    constexpr int BPL = NB / 64;
    static_assert(BPL == 32, "two levels of 32 bins");
    int local = 0;
#pragma unroll
    for (int i = 0; i < BPL / 4; ++i) {
        const int k = (i + lane) & (BPL / 4 - 1);
        const uint4 q = *reinterpret_cast<const uint4*>(&sh.hist[BPL * lane + 4 * k]);
        local += (int)(q.x + q.y + q.z + q.w);
    }
    const int incl = wave_incl_scan(local, lane);
    const int above = __builtin_amdgcn_readlane(incl, 63) - incl;   // bins of the lanes above this one
    const unsigned long long m = __ballot(above < need && need <= above + local);
    const int L = m ? __ffsll((long long)m) - 1 : 0;                  // wave-uniform
    const int above_l = __builtin_amdgcn_readlane(above, L);
    const int hb = lane < BPL ? (int)sh.hist[BPL * L + lane] : 0;
    const int incl2 = wave_incl_scan(hb, lane);
    const int above_i = above_l + __builtin_amdgcn_readlane(incl2, 63) - incl2;   // bins above bin i of lane L
    const unsigned long long m2 = __ballot(lane < BPL && above_i < need && need <= above_i + hb);
    if (m2 && lane == __ffsll((long long)m2) - 1) {
        sh.bstar = BPL * L + lane;
        sh.rstar = need - above_i;
    }
}

// Number of set bits of mask in lanes below this one, plus acc.
__device__ __forceinline__ int mbcnt(unsigned long long mask, int acc) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, (uint32_t)acc));
}

// f(j, partial) for the wave's chunks j < jmax that hold keys; partial is a
// compile-time flag, true for chunk jpart (the row's last chunk, which may
// hold NaN slots) or for every chunk when ALL_PARTIAL.  The bounds pass
// through an empty asm statement so each pass recomputes its scalar chunk
// conditions instead of keeping them live across the kernel.
template <int NCH, bool ALL_PARTIAL, class F>
__device__ __forceinline__ void visit_chunks(int jmax, int jpart, F&& f) {
    asm volatile("" : "+s"(jmax), "+s"(jpart));
    static_for<0, NCH>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (j < jmax) {
            if (ALL_PARTIAL || j == jpart) f(j, std::true_type{});
            else f(j, std::false_type{});
        }
    });
}

// Exclusive prefixes of sh.ccnt over the row's chunks, as lane values: lane l
// holds those of chunks CPL*l .. CPL*l + CPL - 1 in off[0 .. CPL); *total =
// count of all chunks.
template <int CPL>
__device__ __forceinline__ void chunk_offsets(const BinShared& sh, int nch, int lane, int (&off)[CPL], int* total) {
    int c[CPL], local = 0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        c[k] = CPL * lane + k < nch ? sh.ccnt[CPL * lane + k] : 0;
        local += c[k];
    }
    const int incl = wave_incl_scan(local, lane);
    *total = __builtin_amdgcn_readlane(incl, 63);
    int run = incl - local;
#pragma unroll
    for (int k = 0; k < CPL; ++k) { off[k] = run; run += c[k]; }
}

// Exclusive prefix of chunk cidx (wave-uniform) from chunk_offsets' lane values.
template <int CPL>
__device__ __forceinline__ int chunk_offset(const int (&off)[CPL], int cidx) {
    int v = off[0];
#pragma unroll
    for (int k = 1; k < CPL; ++k) v = (cidx % CPL == k) ? off[k] : v;
    return __builtin_amdgcn_readlane(v, cidx / CPL);
}

template <bool BF16>
using RowIn = typename std::conditional<BF16, uint16_t, float>::type;

// Top-k of one row by the whole workgroup (NW waves, all calling together; it
// synchronises with barriers).  row: the n visible scores (key lo + e at
// row[e]); so / io: the topk output slots.  n <= 256 * NW * NCH.
// BF16 = false: fp32 logits of the causal or given ranges (lix_topk).
// BF16 = true: V4.1 bf16 scores over whole rows, where bf16 -inf (0xFF80)
// marks a hidden key: hidden keys are loaded as NaN slots, so they are
// never binned, ranked or selected; a row with at most topk visible keys
// selects all of them and pads the rest with (-1, bf16 -inf).  Selected
// values are written back in the input's type, bit for bit.
template <int NCH, bool BF16, int NW = 4>
__device__ __forceinline__ void select_row_binned(const RowIn<BF16>* __restrict__ row, int n, int lo, int topk,
                                                  RowIn<BF16>* __restrict__ so, int32_t* __restrict__ io,
                                                  BinShared& sh, int tid) {
    static_assert(NW * NCH <= kBinChunks && NW <= kBinMaxWaves, "chunk table too small");
    static_assert(NW * 64 >= kBinCand, "one thread per boundary candidate");
    constexpr int NT = 64 * NW;                               // threads of the workgroup
    constexpr int CPL = (NW * NCH + 63) / 64;                 // chunks per lane in the chunk prefix
    using In = RowIn<BF16>;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    auto out_val = [](float v) -> In {
        if constexpr (BF16) return bf16_bits(v);              // v holds a bf16 value: exact
        else return v;
    };
    const In pad_val = out_val(neg_inf());

    if constexpr (!BF16) {
        if (n <= topk) {                                      // everything is selected
            for (int i0 = 0; i0 < n; i0 += 8 * NT) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = row[min(i0 + u * NT + tid, n - 1)];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u * NT + tid;
                    if (i < n) { so[i] = v[u]; io[i] = lo + i; }
                }
            }
            for (int i = n + tid; i < topk; i += NT) { so[i] = pad_val; io[i] = -1; }
            return;
        }
    }

    // ---- chunks: nch of the row, jmax of this wave, jpart the wave's partial one
    const int nch = (n + 255) >> 8;
    const int jmax = (nch - wv + NW - 1) / NW;
    const int jpart = (((nch - 1) % NW) == wv && (n & 255) != 0) ? (nch - 1) / NW : -1;
    auto key_of = [&](int j, int m) { return (NW * j + wv) * 256 + 64 * m + lane; };  // key - lo
    constexpr bool AP = BF16;                                 // bf16: hidden keys anywhere

    // ---- this wave's chunks (every load issues before the first use)
    const float qnan = __uint_as_float(0x7fc00000u);
    auto cvt = [&](In raw) -> float {
        if constexpr (BF16) return raw == (uint16_t)0xff80u ? qnan : bf16_to_f32(raw);
        else return raw;
    };
    float x[NCH][4];
    if constexpr (BF16) {
        // The wave's chunks only (bf16 rows are whole rows of the V4.1
        // scores): the raw 16 bits of every slot are loaded before any is
        // used (the partial chunk's addresses clamped into the row), then
        // converted, hidden keys and slots past the row becoming NaN (a select
        // on bit patterns, which cannot turn into a select of addresses).
        static_for<0, NCH>([&](auto jc) {
#pragma unroll
            for (int m = 0; m < 4; ++m) x[decltype(jc)::value][m] = qnan;   // chunks past the row
        });
        // (Raw buffer loads over the row's n scores: a slot past the row reads
        // 0 and is made NaN below.)
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(row)), (short)0, n * 2, kBufWord3);
        visit_chunks<NCH, false>(jmax, jpart, [&](int j, auto) {
            const int vo = 2 * key_of(j, 0);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                x[j][m] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, vo + 128 * m, 0, 0));
        });
        visit_chunks<NCH, true>(jmax, jpart, [&](int j, auto) {
            const bool partial = j == jpart;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float v = cvt((uint16_t)__float_as_uint(x[j][m]));
                x[j][m] = partial ? pick(key_of(j, m) < n, v, qnan) : v;
            }
        });
    } else {
        // Every slot is loaded with no branch between the loads, so all of
        // them are in flight before the first is used (loads under per-chunk
        // branches are waited for chunk by chunk): raw buffer loads over the
        // row's n scores (n > topk >= 1 here), whose range check returns 0
        // for a slot past the row, at one per-lane offset per chunk and the
        // slot's 64-key step as the instruction's offset.  Then the slots past
        // the row become NaN, in the chunks that reach past it (a uniform test
        // per chunk).
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<In*>(row), (short)0, n * (int)sizeof(float), kBufWord3);
        static_for<0, NCH>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int vo = 4 * key_of(j, 0);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                x[j][m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo + 256 * m, 0, 0));
        });
        static_for<0, NCH>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if ((NW * j + wv + 1) * 256 > n) {
#pragma unroll
                for (int m = 0; m < 4; ++m) x[j][m] = pick(key_of(j, m) < n, x[j][m], qnan);
            }
        });
    }

    // ---- bf16 rows: count the visible keys; at most topk of them means all
    int visible = n;
    if constexpr (BF16) {
        int c = 0;
        visit_chunks<NCH, AP>(jmax, jpart, [&](int j, auto) {
#pragma unroll
            for (int m = 0; m < 4; ++m) c += __popcll(__ballot(x[j][m] == x[j][m]));
        });
        if (lane == 0) sh.wtot[wv] = c;
        __syncthreads();
        visible = 0;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) visible += sh.wtot[w2];
        __syncthreads();                                      // wtot is reused below
    }
    const bool take_all = visible <= topk;                    // same in every thread

    // ---- row min / max over every slot (NaN slots are ignored)
    float vmin = __uint_as_float(0x7f800000u), vmax = neg_inf();
    static_for<0, NCH>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int m = 0; m < 4; ++m) { vmin = fminf(vmin, x[j][m]); vmax = fmaxf(vmax, x[j][m]); }
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, off, 64));
        vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    }
    if (lane == 0) { sh.wmin[wv] = vmin; sh.wmax[wv] = vmax; }
#pragma unroll
    for (int i = 4 * tid; i < kBins; i += 4 * NT) *reinterpret_cast<uint4*>(&sh.hist[i]) = uint4{0u, 0u, 0u, 0u};
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
    vmin = sh.wmin[0];
    vmax = sh.wmax[0];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) { vmin = fminf(vmin, sh.wmin[w2]); vmax = fmaxf(vmax, sh.wmax[w2]); }
    const float span = vmax - vmin;
    // (A span below 1e-30 would overflow the scale; such rows take the radix path.)
    const bool binned = span > 1.0e-30f && span < 3.0e38f;   // same in every thread
    const float sc = binned ? 0.99951171875f / span : 0.0f;  // (1 - 2^-11) / span
    const bool one_fma = binned && fabsf(vmin) * sc <= 256.0f;
    const float c0 = one_fma ? 1.000244140625f - vmin * sc : 1.000244140625f;   // 1 + 2^-12
    // bin_of(one, v): `one` selects the one-fma form at compile time; each
    // pass branches once (uniformly) between the two forms.
    auto u_bits = [&](auto one, float v) -> uint32_t {
        return __float_as_uint(decltype(one)::value ? fmaf(v, sc, c0) : fmaf(v - vmin, sc, c0));
    };
    auto bin_of = [&](auto one, float v) -> int { return (int)((u_bits(one, v) >> 12) & (uint32_t)(kBins - 1)); };
    auto with_form = [&](auto&& f) {
        if (one_fma) f(std::true_type{});
        else f(std::false_type{});
    };

    int bstar = 0, rstar = topk, cb = 1 << 30;
    bool counted = false;                                     // sh.ccnt holds the chunk counts
    if (binned && !take_all) {
        with_form([&](auto one) {
            visit_chunks<NCH, AP>(jmax, jpart, [&](int j, auto partial) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float v = x[j][m];
                    if (!decltype(partial)::value || v == v) atomicAdd(&sh.hist[bin_of(one, v)], 1u);
                }
            });
        });
        __syncthreads();
        if (wv == 0) wave_find_bin_lds<kBins>(sh, topk, lane);
        __syncthreads();
        bstar = sh.bstar;
        rstar = sh.rstar;
        cb = (int)sh.hist[bstar];
    }

    if (take_all) {
        // ---- at most topk visible keys: every visible key is selected
        if (tid == 0) { sh.cut_v = neg_inf(); sh.cut_i = 0x7fffffff; sh.cut_ties = 1; }
        __syncthreads();
    } else if (cb <= kBinCand) {
        // ---- gather the boundary bin (exactly the cb keys the histogram
        // counted there) and rank it exactly.  The same pass counts, per
        // chunk, the keys in bins above it (all selected); each selected
        // candidate then adds itself to its chunk's count.
        int ccv = 0;                                          // lane j: count of chunk j
        const uint32_t ub_lo = 0x3f800000u + ((uint32_t)bstar << 12), ub_hi = ub_lo + 4096u;
        with_form([&](auto one) {
            visit_chunks<NCH, AP>(jmax, jpart, [&](int j, auto partial) {
                int above = 0;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float v = x[j][m];
                    // bins compared on the bits of u (in [1, 2)): bin > bstar
                    // iff bits >= ub_hi, bin == bstar iff ub_lo <= bits < ub_hi
                    const uint32_t ub = u_bits(one, v);
                    const bool ok = !decltype(partial)::value || v == v;
                    const bool hi = ub >= ub_hi;
                    above += __popcll(__ballot(hi && ok));
                    const bool c = ub >= ub_lo && !hi && ok;
                    const unsigned long long mask = __ballot(c);
                    if (mask != 0ull) {
                        int base = 0;
                        if (lane == 0) base = atomicAdd(&sh.ncand, __popcll(mask));
                        base = __shfl(base, 0, 64);
                        if (c) {
                            const int p = mbcnt(mask, base);
                            sh.cand_v[p] = v;
                            sh.cand_i[p] = key_of(j, m);
                        }
                    }
                }
                ccv = (lane == j) ? above : ccv;
            });
        });
        if (lane < jmax) sh.ccnt[NW * lane + wv] = ccv;
        __syncthreads();
        if (tid < cb) {
            // rank = candidates before this one in (score desc, key asc);
            // the other candidates are read 8 at a time (broadcast reads)
            const float vi = sh.cand_v[tid];
            const int ii = sh.cand_i[tid];
            int rank = 0, eq = 0;
            auto visit = [&](float vj, int ij) {
                rank += (vj > vi) || (vj == vi && ij < ii);
                eq += (vj == vi);
            };
            int jj = 0;
            for (; jj + 8 <= cb; jj += 8) {
                const float4 va = *reinterpret_cast<const float4*>(&sh.cand_v[jj]);
                const float4 vb = *reinterpret_cast<const float4*>(&sh.cand_v[jj + 4]);
                const int4 ia = *reinterpret_cast<const int4*>(&sh.cand_i[jj]);
                const int4 ib = *reinterpret_cast<const int4*>(&sh.cand_i[jj + 4]);
                visit(va.x, ia.x); visit(va.y, ia.y); visit(va.z, ia.z); visit(va.w, ia.w);
                visit(vb.x, ib.x); visit(vb.y, ib.y); visit(vb.z, ib.z); visit(vb.w, ib.w);
            }
            for (; jj < cb; ++jj) visit(sh.cand_v[jj], sh.cand_i[jj]);
            if (rank == rstar - 1) { sh.cut_v = vi; sh.cut_i = ii; sh.cut_ties = eq > 1; }
            if (rank < rstar) atomicAdd(&sh.ccnt[ii >> 8], 1);
        }
        __syncthreads();
        counted = true;
    } else {
        // ---- radix select on the keys of the boundary bin (or of the whole
        // row when it is not binned), 8-bit digits ...
        uint32_t prefix = 0, pmask = 0;
        int need = rstar;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += NT) sh.hist[i] = 0u;
            __syncthreads();
            with_form([&](auto one) {
                visit_chunks<NCH, true>(jmax, jpart, [&](int j, auto) {
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float v = x[j][m];
                        const bool in = (v == v) && (!binned || bin_of(one, v) == bstar);
                        const uint32_t k = f32_to_key(v);
                        if (in && (k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
                    }
                });
            });
            __syncthreads();
            block_find_bin<256, NW>(sh, need, tid);
            prefix |= (uint32_t)sh.bstar << shift;
            pmask |= 255u << shift;
            need = sh.rstar;
            __syncthreads();                                  // bstar / rstar read before reuse
        }
        // ... then the need-th smallest key index among the scores equal to
        // it: count them per chunk, then walk the chunks in row order
        const float vt = key_to_f32(prefix);
        visit_chunks<NCH, true>(jmax, jpart, [&](int j, auto) {
            int c = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m) c += __popcll(__ballot(x[j][m] == vt));
            if (lane == 0) sh.ccnt[NW * j + wv] = c;
        });
        __syncthreads();
        int total_eq, off[CPL];
        chunk_offsets<CPL>(sh, nch, lane, off, &total_eq);
        visit_chunks<NCH, true>(jmax, jpart, [&](int j, auto) {
            int run = chunk_offset<CPL>(off, NW * j + wv);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const unsigned long long mask = __ballot(x[j][m] == vt);
                const int c = __popcll(mask);
                if (run < need && need <= run + c && ((mask >> lane) & 1ull) && mbcnt(mask, run) == need - 1) {
                    sh.cut_v = vt;
                    sh.cut_i = key_of(j, m);
                    sh.cut_ties = total_eq > 1;
                }
                run += c;
            }
        });
        __syncthreads();
    }

    // ---- ordered write of the selection: an element is selected iff its
    // score is above vT, or equal to it with key index <= iT (with no tie,
    // iff its score is >= vT).  Bins are monotone in the score, so that is
    // every key in a bin above the boundary bin plus the selected candidates:
    // the counts the boundary pass made.  The other routes count each chunk's
    // selection in a pass of their own.  The write pass puts each selected
    // slot at its position (32-bit byte offsets from the row's output base).
    // Each pass reads the cut from LDS, so no compare mask stays live across
    // a barrier.
    auto selected = [&](auto tie, int j, int m, float vT, int iT) -> bool {
        const float v = x[j][m];
        if constexpr (!decltype(tie)::value) return v >= vT;
        else return (v > vT) | ((v == vT) & (key_of(j, m) <= iT));
    };
    auto with_ties = [&](bool ties, auto&& f) {
        if (ties) f(std::true_type{});
        else f(std::false_type{});
    };
    if (!counted) {
        const float vT = sh.cut_v;
        const int iT = sh.cut_i;
        int ccv = 0;                                          // lane j: count of chunk j
        with_ties(sh.cut_ties != 0, [&](auto tie) {
            visit_chunks<NCH, AP>(jmax, jpart, [&](int j, auto) {
                int c = 0;
#pragma unroll
                for (int m = 0; m < 4; ++m) c += __popcll(__ballot(selected(tie, j, m, vT, iT)));
                ccv = (lane == j) ? c : ccv;
            });
        });
        if (lane < jmax) sh.ccnt[NW * lane + wv] = ccv;
        __syncthreads();
    }
    int total, off[CPL];
    chunk_offsets<CPL>(sh, nch, lane, off, &total);
    const int key0 = lo + lane + 256 * wv;                    // key of slot (j, m): key0 + 256 NW j + 64 m
    char* so_b = reinterpret_cast<char*>(so);
    char* io_b = reinterpret_cast<char*>(io);
    {
        const float vT = sh.cut_v;
        const int iT = sh.cut_i;
        with_ties(sh.cut_ties != 0, [&](auto tie) {
            visit_chunks<NCH, AP>(jmax, jpart, [&](int j, auto) {
                int run = chunk_offset<CPL>(off, NW * j + wv);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bool f = selected(tie, j, m, vT, iT);
                    const unsigned long long mask = __ballot(f);
                    const uint32_t pos = (uint32_t)mbcnt(mask, run);
                    if (f && pos < (uint32_t)topk) {
                        *reinterpret_cast<In*>(so_b + pos * (uint32_t)sizeof(In)) = out_val(x[j][m]);
                        *reinterpret_cast<int32_t*>(io_b + pos * 4u) = key0 + 256 * NW * j + 64 * m;
                    }
                    run += __popcll(mask);
                }
            });
        });
    }
    for (int i = total + tid; i < topk; i += NT) { so[i] = pad_val; io[i] = -1; }
}

}  // namespace lix

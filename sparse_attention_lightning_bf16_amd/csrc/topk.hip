// Per-row top-k over materialized fp32 logits, and the gather at given indices.
//
// Top-k (page "...deepseek_v4.kernels.tilelang_indexer", v4_lighting_indexer:
// select topk indices per query; [B,S,topk] fp32 scores and int32 indices).
// One workgroup selects one row.  Scores become order-preserving 32-bit keys;
// a three-pass MSB-first radix select (11 + 11 + 10 bits, LDS histograms)
// finds the key T of the m-th largest element and how many elements equal
// to T are taken.  A last pass writes the elements with key > T plus the
// first `need` elements with key == T in index order, so ties go to the lower
// index and the output is in ascending key order.  Each wave owns a
// contiguous quarter of the row, which makes the output positions a prefix
// count over (wave totals, 64-element chunks, lanes).
//
// Gather (section pytorch_extract_topk_scores): out = logits[b,t,idx], or -inf
// for an index outside [0, Skv).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace lix {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;

struct RadixShared {
    uint32_t hist[2048];
    int wave_tot[kTopkWaves];
    int gt[kTopkWaves];
    int eq[kTopkWaves];
    int sel_bin;
    int sel_need;
};

__device__ __forceinline__ int lanes_below(unsigned long long mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

// Locate the bin holding the need-th largest element of hist[0..nbins):
// sets sh.sel_bin and sh.sel_need (rank of the element inside that bin).
__device__ void find_bin(RadixShared& sh, int nbins, int need, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    const int bpt = nbins / kTopkThreads;
    const int base = tid * bpt;
    int local = 0;
    for (int i = 0; i < bpt; ++i) local += (int)sh.hist[base + i];
    int v = local;                       // inclusive suffix sum within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_down(v, off, 64);
        if (lane + off < 64) v += u;
    }
    if (lane == 0) sh.wave_tot[wave] = v;
    __syncthreads();
    int above = v - local;
    for (int w2 = wave + 1; w2 < kTopkWaves; ++w2) above += sh.wave_tot[w2];
    if (above < need && need <= above + local) {
        for (int i = bpt - 1; i >= 0; --i) {
            const int h = (int)sh.hist[base + i];
            if (need <= above + h) {
                sh.sel_bin = base + i;
                sh.sel_need = need - above;
                break;
            }
            above += h;
        }
    }
    __syncthreads();
}

// Visit chunk slots j = 0..jmax-1; with a register cache the loop is fully
// unrolled so the cache is indexed by constants.
template <int CACHE, class F>
__device__ __forceinline__ void for_chunks(int jmax, F&& f) {
    if constexpr (CACHE > 0) {
#pragma unroll
        for (int j = 0; j < CACHE; ++j)
            if (j < jmax) f(j);
    } else {
        for (int j = 0; j < jmax; ++j) f(j);
    }
}

template <int CACHE>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float* __restrict__ logits, int B, int S,
                                                                 int skv, int ratio, const int32_t* __restrict__ ks,
                                                                 const int32_t* __restrict__ ke, int topk,
                                                                 float* __restrict__ scores,
                                                                 int32_t* __restrict__ indices) {
    __shared__ RadixShared sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x % B;
    const int t = S - 1 - (int)(blockIdx.x / B);           // longest causal rows first
    int lo, hi;
    key_range(ks, ke, t, S, skv, ratio, lo, hi);
    const int n = hi - lo;
    const float* row = logits + ((long)b * S + t) * skv + lo;
    float* so = scores + ((long)b * S + t) * topk;
    int32_t* io = indices + ((long)b * S + t) * topk;

    if (n <= topk) {
        for (int i = tid; i < n; i += kTopkThreads) { so[i] = row[i]; io[i] = lo + i; }
        for (int i = n + tid; i < topk; i += kTopkThreads) { so[i] = neg_inf(); io[i] = -1; }
        return;
    }

    const int nch = (n + 63) >> 6;
    const int cw = (nch + kTopkWaves - 1) / kTopkWaves;     // chunks per wave
    const int c_begin = wave * cw;
    const int c_end = min(nch, c_begin + cw);

    uint32_t cache[CACHE > 0 ? CACHE : 1];
    if constexpr (CACHE > 0) {
        // Clamped addresses and a select instead of a guarded load: every load
        // issues before the first wait (a guarded load would be waited for at
        // its branch merge, serialising the row's loads).
        // (The invalid slots are cleared with a mask, not a select, so the
        // compiler cannot move a load under a branch.)
        const int e_end = min(c_end * 64, n);
#pragma unroll
        for (int j = 0; j < CACHE; ++j) {
            const int e = (c_begin + j) * 64 + lane;
            const float v = row[min(e, n - 1)];
            cache[j] = f32_to_key(v) & (0u - (uint32_t)(e < e_end));
        }
    }
    auto key_at = [&](int j, int e) -> uint32_t {
        if constexpr (CACHE > 0) return cache[j];
        else return f32_to_key(row[e]);
    };
    const int jmax = (CACHE > 0) ? min(cw, CACHE) : cw;

    // Radix select of the m-th largest key.
    uint32_t prefix = 0, pmask = 0;
    int need = topk;
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass < 2 ? 2048 : 1024;
        for (int i = tid; i < nbins; i += kTopkThreads) sh.hist[i] = 0u;
        __syncthreads();
        for_chunks<CACHE>(jmax, [&](int j) {
            const int c = c_begin + j;
            const int e = c * 64 + lane;
            if (c < c_end && e < n) {
                const uint32_t key = key_at(j, e);
                if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
            }
        });
        __syncthreads();
        find_bin(sh, nbins, need, tid);
        prefix |= (uint32_t)sh.sel_bin << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
        need = sh.sel_need;
    }
    const uint32_t T = prefix;
    const int need_eq = need;

    // Per-wave counts of keys above / equal to T.
    int gt = 0, eq = 0;
    for_chunks<CACHE>(jmax, [&](int j) {
        const int c = c_begin + j;
        const int e = c * 64 + lane;
        const bool valid = (c < c_end) && (e < n);
        const uint32_t key = valid ? key_at(j, e) : 0u;
        gt += __popcll(__ballot(valid && key > T));
        eq += __popcll(__ballot(valid && key == T));
    });
    if (lane == 0) { sh.gt[wave] = gt; sh.eq[wave] = eq; }
    __syncthreads();
    int eq_before = 0, out_before = 0;
    for (int w2 = 0; w2 < wave; ++w2) {
        const int take_eq = min(sh.eq[w2], max(0, need_eq - eq_before));
        out_before += sh.gt[w2] + take_eq;
        eq_before += sh.eq[w2];
    }

    // Ordered write of the selection.
    int run_out = out_before, run_eq = eq_before;
    for_chunks<CACHE>(jmax, [&](int j) {
        const int c = c_begin + j;
        const int e = c * 64 + lane;
        const bool valid = (c < c_end) && (e < n);
        const uint32_t key = valid ? key_at(j, e) : 0u;
        const bool is_gt = valid && key > T;
        const bool is_eq = valid && key == T;
        const unsigned long long eqm = __ballot(is_eq);
        const bool sel = is_gt || (is_eq && run_eq + lanes_below(eqm, lane) < need_eq);
        const unsigned long long selm = __ballot(sel);
        const int pos = run_out + lanes_below(selm, lane);
        if (sel && pos < topk) {
            so[pos] = key_to_f32(key);
            io[pos] = lo + e;
        }
        run_out += __popcll(selm);
        run_eq += __popcll(eqm);
    });
}


// ---------------------------------------------------------------- register-resident row top-k
//
// Rows of at most 8192 visible keys.  WPR waves (1 or 2) select one row; the
// row sits in their registers (wave w of the row holds elements
// w*VEC*256 + 256*j + 4*lane + m in slot [j][m]; slots past the row hold NaN)
// and the row has a private LDS histogram.  The m-th best element in the
// order (score descending, key index ascending) is located in two steps: a
// 2048-bin histogram linear in the score between the row's min and max gives
// the bin holding it (NaN slots land in per-lane trash bins past the end);
// inside that bin it is ranked exactly (pairwise when the bin has at most 64
// elements, else radix on order-preserving keys plus an ordered count for
// ties).  With that element (vT, iT), an element is selected iff its score is
// above vT, or equal to it with index <= iT; one ordered pass writes the
// selection in ascending index order.  Scores are copied bit for bit.

constexpr int kBins = 2048;
constexpr int kRowThreads = 256;                     // threads per workgroup

template <int WPR>
struct RowShared {
    uint32_t hist[kBins + 64 * WPR];                 // + one trash bin per lane
    float cand_val[64];
    int cand_idx[64];
    float wmin[WPR], wmax[WPR];
    int wcnt[WPR];
    float cut_v;
    int cut_i;
};

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

// Bin (0..nbins-1) holding the need-th largest of hist[0..nbins) and the rank
// of that element inside it (1-based, counted from the top).  One wave; lane l
// owns bins [l*nbins/64, (l+1)*nbins/64).
__device__ __forceinline__ void wave_find_bin(const uint32_t* hist, int nbins, int need, int lane, int& bin,
                                              int& rank) {
    const int bpl = nbins >> 6;
    const int base = lane * bpl;
    int local = 0;
    for (int i = 0; i < bpl; ++i) local += (int)hist[base + i];
    int v = local;                                   // inclusive suffix sum over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_down(v, off, 64);
        if (lane + off < 64) v += u;
    }
    int above = v - local;
    int b = -1, r = 0;
    if (above < need && need <= above + local) {
        for (int i = bpl - 1; i >= 0; --i) {
            const int h = (int)hist[base + i];
            if (need <= above + h) { b = base + i; r = need - above; break; }
            above += h;
        }
    }
    const unsigned long long found = __ballot(b >= 0);
    const int src = found ? __ffsll((long long)found) - 1 : 0;
    bin = __shfl(b, src, 64);
    rank = __shfl(r, src, 64);
    if (bin < 0) { bin = 0; rank = 1; }
}

template <int WPR>
__device__ __forceinline__ void row_sync() {
    if constexpr (WPR > 1) __syncthreads();
}

template <int VEC, int WPR, int MINB>
__global__ __launch_bounds__(kRowThreads, MINB) void topk_rows_reg_kernel(
    const float* __restrict__ logits, int B, int S, int skv, int ratio, const int32_t* __restrict__ ks,
    const int32_t* __restrict__ ke, int topk, float* __restrict__ scores, int32_t* __restrict__ indices) {
    constexpr int RPB = kRowThreads / (64 * WPR);            // rows per workgroup
    constexpr int SPAN = VEC * 256;                           // elements per wave
    __shared__ RowShared<WPR> shr[RPB];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int rw = wv / WPR, wr = wv % WPR;                   // row slot in the block, wave within the row
    RowShared<WPR>& sh = shr[rw];
    const long rid = (long)blockIdx.x * RPB + rw;
    const bool live = rid < (long)B * S;
    const int b = live ? (int)(rid % B) : 0;
    const int t = live ? S - 1 - (int)(rid / B) : 0;         // longest causal rows first
    int lo = 0, hi = 0;
    if (live) key_range(ks, ke, t, S, skv, ratio, lo, hi);
    const int n = hi - lo;
    const float* row = logits + ((long)b * S + t) * skv + lo;
    float* so = scores + ((long)b * S + t) * topk;
    int32_t* io = indices + ((long)b * S + t) * topk;
    // every wave of the block reaches every barrier: rows that need no
    // selection (or do not exist) only skip the work between them
    const bool work = live && n > topk;
    if (live && !work && wr == 0) {
        for (int i = lane; i < n; i += 64) { so[i] = row[i]; io[i] = lo + i; }
        for (int i = n + lane; i < topk; i += 64) { so[i] = neg_inf(); io[i] = -1; }
    }
    if constexpr (WPR == 1) {
        if (!work) return;
    }

    // ---- load this wave's part of the row
    const float qnan = __uint_as_float(0x7fc00000u);
    const int ebase = wr * SPAN;                              // first element of this wave
    const int nloc = work ? max(0, min(n - ebase, SPAN)) : 0;
    // All loads issue before the first wait: addresses are clamped into the
    // wave's part of the row and slots past it are set by a select.  16-byte
    // loads need an aligned logits base, skv % 4 == 0 and lo % 4 == 0: then
    // every row starts and the buffer ends on a 16-byte boundary, so the
    // aligned group holding the row's last element lies inside the buffer.
    const bool vec_ok = (reinterpret_cast<uintptr_t>(logits) & 15) == 0 && ((skv | lo) & 3) == 0;
    float x[VEC][4];
#pragma unroll
    for (int j = 0; j < VEC; ++j) x[j][0] = x[j][1] = x[j][2] = x[j][3] = qnan;
    if (nloc > 0) {
        const float* wrow = row + ebase;
        if (vec_ok) {
            const int last = (nloc - 1) & ~3;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int e0 = j * 256 + 4 * lane;
                const float4 y = *reinterpret_cast<const float4*>(wrow + min(e0, last));
                x[j][0] = (e0 + 0 < nloc) ? y.x : qnan;
                x[j][1] = (e0 + 1 < nloc) ? y.y : qnan;
                x[j][2] = (e0 + 2 < nloc) ? y.z : qnan;
                x[j][3] = (e0 + 3 < nloc) ? y.w : qnan;
            }
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = j * 256 + 4 * lane + m;
                    const float v = wrow[min(e, nloc - 1)];
                    x[j][m] = (e < nloc) ? v : qnan;
                }
        }
    }

    // ---- row min / max (NaN slots are ignored)
    float vmin = __uint_as_float(0x7f800000u), vmax = neg_inf();
#pragma unroll
    for (int j = 0; j < VEC; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) { vmin = fminf(vmin, x[j][m]); vmax = fmaxf(vmax, x[j][m]); }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, off, 64));
        vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    }
    if constexpr (WPR > 1) {
        if (lane == 0) { sh.wmin[wr] = vmin; sh.wmax[wr] = vmax; }
        for (int i = wr * 64 + lane; i < kBins + 64 * WPR; i += 64 * WPR) sh.hist[i] = 0u;
        row_sync<WPR>();                                      // (1)
        vmin = sh.wmin[0]; vmax = sh.wmax[0];
#pragma unroll
        for (int w2 = 1; w2 < WPR; ++w2) { vmin = fminf(vmin, sh.wmin[w2]); vmax = fmaxf(vmax, sh.wmax[w2]); }
    } else {
        for (int i = lane; i < kBins + 64; i += 64) sh.hist[i] = 0u;
    }
    const float span = vmax - vmin;
    // Finite, non-degenerate range whose bin scale kBins / span stays finite
    // (a span below ~6e-36 would overflow it to inf, and the elements equal to
    // vmin would then bin as (0 * inf) = NaN); other rows take the radix path.
    const bool binned = span > 1.0e-30f && span < 3.0e38f;
    const float scale = binned ? (float)kBins / span : 0.0f;
    const int trash = kBins + 64 * wr + lane;
    auto bin_with = [&](float v, float org, float sc) -> int {
        const float f = (v - org) * sc;                       // NaN for NaN slots
        return f >= 0.0f ? min((int)f, kBins - 1) : trash;
    };

    int bstar = 0, rstar = topk;
    int cb = 1 << 30;                                         // boundary bin size; huge -> radix path
    if (binned) {
#pragma unroll
        for (int j = 0; j < VEC; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) atomicAdd(&sh.hist[bin_with(x[j][m], vmin, scale)], 1u);
        row_sync<WPR>();                                      // (2)
        if (work) {
            wave_find_bin(sh.hist, kBins, topk, lane, bstar, rstar);
            cb = (int)sh.hist[bstar];
        }
    }
    // Later passes recompute bins from copies of (vmin, scale) that the compiler
    // cannot tie to the first pass, so no per-element bin stays in a register.
    const float vmin2 = __shfl(vmin, 0, 64), scale2 = __shfl(scale, 0, 64);
    auto bin_of = [&](float v) -> int { return bin_with(v, vmin2, scale2); };
    const int ecut_lo = ebase;                                // this wave's first element index

    if (__builtin_amdgcn_readfirstlane(cb) <= 64) {
        // ---- small boundary bin: gather it in index order and rank pairwise
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < VEC; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) cnt += bin_of(x[j][m]) == bstar ? 1 : 0;
        int run = 0;
        if constexpr (WPR > 1) {
            int tot = cnt;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
            if (lane == 0) sh.wcnt[wr] = tot;
            row_sync<WPR>();                                  // (3)
            for (int w2 = 0; w2 < wr; ++w2) run += sh.wcnt[w2];
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            int c = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m) c += bin_of(x[j][m]) == bstar ? 1 : 0;
            const int incl = wave_incl_scan(c, lane);
            int pos = run + incl - c;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (bin_of(x[j][m]) == bstar) {
                    sh.cand_val[pos] = x[j][m];
                    sh.cand_idx[pos] = ecut_lo + j * 256 + 4 * lane + m;
                    ++pos;
                }
            run += __shfl(incl, 63, 64);
        }
        row_sync<WPR>();                                      // (4)
        if (wr == 0 && work) {
            float vi = 0.0f;
            int ii = 0x7fffffff, rank = 1 << 30;
            if (lane < cb) {
                vi = sh.cand_val[lane];
                ii = sh.cand_idx[lane];
                rank = 0;
                for (int jj = 0; jj < cb; ++jj) {
                    const float vj = sh.cand_val[jj];
                    const int ij = sh.cand_idx[jj];
                    rank += (vj > vi) || (vj == vi && ij < ii);
                }
            }
            if (rank == rstar - 1) { sh.cut_v = vi; sh.cut_i = ii; }
        }
    } else {
        // ---- large boundary bin (or unbinned row): radix select on the keys
        // of its elements, 8-bit digits ...
        uint32_t prefix = 0, pmask = 0;
        int need = rstar;
        for (int shift = 24; shift >= 0; shift -= 8) {
            row_sync<WPR>();
            for (int i = wr * 64 + lane; i < 256; i += 64 * WPR) sh.hist[i] = 0u;
            row_sync<WPR>();
#pragma unroll
            for (int j = 0; j < VEC; ++j)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float v = x[j][m];
                    const bool in = (v == v) && (!binned || bin_of(v) == bstar);
                    const uint32_t k = f32_to_key(v);
                    if (in && (k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
                }
            row_sync<WPR>();
            int bb = 0, rr = 1;
            if (work) wave_find_bin(sh.hist, 256, need, lane, bb, rr);
            prefix |= (uint32_t)bb << shift;
            pmask |= 255u << shift;
            need = rr;
        }
        const float vt = key_to_f32(prefix);
        // ... then the need-th smallest index among scores equal to it
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < VEC; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) cnt += (x[j][m] == vt) ? 1 : 0;
        int run = 0;
        if constexpr (WPR > 1) {
            int tot = cnt;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
            if (lane == 0) sh.wcnt[wr] = tot;
            row_sync<WPR>();
            for (int w2 = 0; w2 < wr; ++w2) run += sh.wcnt[w2];
        }
        int found = -1;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            int c = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m) c += (x[j][m] == vt) ? 1 : 0;
            const int incl = wave_incl_scan(c, lane);
            int r = run + incl - c;
            if (r < need && need <= r + c) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (x[j][m] == vt) {
                        ++r;
                        if (r == need) found = ecut_lo + j * 256 + 4 * lane + m;
                    }
            }
            run += __shfl(incl, 63, 64);
        }
        if (found >= 0 && work) { sh.cut_v = vt; sh.cut_i = found; }
    }
    row_sync<WPR>();                                          // (5) cut visible
    const float vT = sh.cut_v;
    const int iT = sh.cut_i;

    // ---- ordered write of the selection
    auto sel = [&](int j, int m) {
        const float v = x[j][m];
        return v > vT || (v == vT && ecut_lo + j * 256 + 4 * lane + m <= iT);
    };
    int run = 0;
    if constexpr (WPR > 1) {
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < VEC; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) cnt += sel(j, m) ? 1 : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
        row_sync<WPR>();
        if (lane == 0) sh.wcnt[wr] = cnt;
        row_sync<WPR>();                                      // (6)
        for (int w2 = 0; w2 < wr; ++w2) run += sh.wcnt[w2];
    }
    if (!work) return;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        bool f[4];
        int c = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) { f[m] = sel(j, m); c += f[m] ? 1 : 0; }
        const int incl = wave_incl_scan(c, lane);
        int pos = run + incl - c;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (f[m] && pos < topk) {
                so[pos] = x[j][m];
                io[pos] = lo + ecut_lo + j * 256 + 4 * lane + m;
                ++pos;
            }
        run += __shfl(incl, 63, 64);
    }
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
constexpr int kBinThreads = 256;
constexpr int kBinChunks = 32;                    // 256-key chunks per row (8192 keys)

struct BinShared {
    alignas(16) uint32_t hist[kBins];
    alignas(16) float cand_v[kBinCand];
    alignas(16) int cand_i[kBinCand];
    int ccnt[kBinChunks];                         // per-chunk counts, row order
    float wmin[4], wmax[4];
    int wtot[4];
    int ncand;
    int bstar, rstar;
    float cut_v;
    int cut_i;
    int cut_ties;                                 // another key has score vT
};

// Block-wide: the bin holding the need-th largest element of hist[0..NB) and
// the element's 1-based rank inside it, counted from the top, into sh.bstar /
// sh.rstar.  Thread tid owns bins [BPT*tid, BPT*tid + BPT), read rotated by
// tid so a wave's reads spread over the LDS banks; the suffix sums over lanes
// come from a DPP prefix scan.  Every thread calls it; it ends with a
// barrier.  Requires 1 <= need <= sum of hist.
template <int NB>
__device__ void block_find_bin(BinShared& sh, int need, int tid) {
    constexpr int BPT = NB / kBinThreads;
    const int lane = tid & 63, wv = tid >> 6;
    const int base = BPT * tid;
    int local = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) local += (int)sh.hist[base + ((i + tid) & (BPT - 1))];
    const int incl = wave_incl_scan(local, lane);
    const int wsum = __builtin_amdgcn_readlane(incl, 63);
    const int v = wsum - incl + local;               // inclusive suffix sum over lanes >= this one
    if (lane == 0) sh.wtot[wv] = wsum;
    __syncthreads();
    int above = v - local;
    for (int w2 = wv + 1; w2 < 4; ++w2) above += sh.wtot[w2];
    if (above < need && need <= above + local) {
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
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if (j >= jmax) break;
        if (ALL_PARTIAL || j == jpart) f(j, std::true_type{});
        else f(j, std::false_type{});
    }
}

// Exclusive prefix of sh.ccnt over the row's chunks, as a lane value: lane c
// (< nch) holds the count of chunks 0..c-1; *total = count of all chunks.
__device__ __forceinline__ int chunk_offsets(const BinShared& sh, int nch, int lane, int* total) {
    const int c = lane < nch ? sh.ccnt[lane] : 0;
    const int incl = wave_incl_scan(c, lane);
    *total = __builtin_amdgcn_readlane(incl, 63);
    return incl - c;
}

// BF16 = false: fp32 logits of the causal or given ranges (lix_topk).
// BF16 = true: V4.1 bf16 scores over whole rows, where bf16 -inf (0xFF80)
// marks a hidden key: hidden keys are loaded as NaN slots, so they are
// never binned, ranked or selected; a row with at most topk visible keys
// selects all of them and pads the rest with (-1, bf16 -inf).  Selected
// values are written back in the input's type, bit for bit.
template <int NCH, bool BF16>
__global__ __launch_bounds__(kBinThreads) void topk_rows_bin_kernel(const void* __restrict__ logits_v, int B, int S,
                                                                    int skv, int ratio,
                                                                    const int32_t* __restrict__ ks,
                                                                    const int32_t* __restrict__ ke, int topk,
                                                                    void* __restrict__ scores_v,
                                                                    int32_t* __restrict__ indices) {
    static_assert(4 * NCH <= kBinChunks, "chunk table too small");
    using In = typename std::conditional<BF16, uint16_t, float>::type;
    __shared__ BinShared sh;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int b = blockIdx.x % B;
    const int t = S - 1 - (int)(blockIdx.x / B);              // longest causal rows first
    int lo = 0, hi = skv;
    if constexpr (!BF16) key_range(ks, ke, t, S, skv, ratio, lo, hi);
    const int n = hi - lo;
    const In* logits = static_cast<const In*>(logits_v);
    const In* row = logits + ((long)b * S + t) * skv + lo;
    In* so = static_cast<In*>(scores_v) + ((long)b * S + t) * topk;
    int32_t* io = indices + ((long)b * S + t) * topk;
    auto out_val = [](float v) -> In {
        if constexpr (BF16) return bf16_bits(v);              // v holds a bf16 value: exact
        else return v;
    };
    const In pad_val = out_val(neg_inf());

    if constexpr (!BF16) {
        if (n <= topk) {                                      // everything is selected
            for (int i0 = 0; i0 < n; i0 += 8 * kBinThreads) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = row[min(i0 + u * kBinThreads + tid, n - 1)];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u * kBinThreads + tid;
                    if (i < n) { so[i] = v[u]; io[i] = lo + i; }
                }
            }
            for (int i = n + tid; i < topk; i += kBinThreads) { so[i] = pad_val; io[i] = -1; }
            return;
        }
    }

    // ---- chunks: nch of the row, jmax of this wave, jpart the wave's partial one
    const int nch = (n + 255) >> 8;
    const int jmax = (nch - wv + 3) >> 2;
    const int jpart = (((nch - 1) & 3) == wv && (n & 255) != 0) ? (nch - 1) >> 2 : -1;
    auto key_of = [&](int j, int m) { return (4 * j + wv) * 256 + 64 * m + lane; };   // key - lo
    constexpr bool AP = BF16;                                 // bf16: hidden keys anywhere

    // ---- this wave's chunks (every load issues before the first use)
    const float qnan = __uint_as_float(0x7fc00000u);
    auto cvt = [&](In raw) -> float {
        if constexpr (BF16) return raw == (uint16_t)0xff80u ? qnan : bf16_to_f32(raw);
        else return raw;
    };
    float x[NCH][4];
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) x[j][m] = qnan;           // chunks past the row
    // Loads first (the partial chunk's addresses clamped into the row), then
    // the partial chunk's slots past the row set to NaN in a pass of their
    // own: consuming a loaded value before every chunk's loads are issued
    // would make each chunk wait for the one before it.  (The masking is a
    // select on bit patterns: a select of the two values lets the optimiser
    // turn the load into a select of addresses, through a generic pointer and
    // a private NaN.)
    // (bf16 inputs: the raw 16 bits are loaded and converted in the second
    // pass, for the same reason.)
    visit_chunks<NCH, false>(jmax, jpart, [&](int j, auto partial) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = key_of(j, m);
            const In raw = row[decltype(partial)::value ? min(e, n - 1) : e];
            if constexpr (BF16) x[j][m] = __uint_as_float((uint32_t)raw);
            else x[j][m] = raw;
        }
    });
    if constexpr (BF16) {
        visit_chunks<NCH, true>(jmax, jpart, [&](int j, auto) {
            const bool partial = j == jpart;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float v = cvt((uint16_t)__float_as_uint(x[j][m]));
                x[j][m] = partial ? pick(key_of(j, m) < n, v, qnan) : v;
            }
        });
    } else {
        visit_chunks<NCH, false>(jmax, jpart, [&](int j, auto partial) {
            if constexpr (decltype(partial)::value) {
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
        visible = sh.wtot[0] + sh.wtot[1] + sh.wtot[2] + sh.wtot[3];
        __syncthreads();                                      // wtot is reused below
    }
    const bool take_all = visible <= topk;                    // same in every thread

    // ---- row min / max over every slot (NaN slots are ignored)
    float vmin = __uint_as_float(0x7f800000u), vmax = neg_inf();
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) { vmin = fminf(vmin, x[j][m]); vmax = fmaxf(vmax, x[j][m]); }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, off, 64));
        vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    }
    if (lane == 0) { sh.wmin[wv] = vmin; sh.wmax[wv] = vmax; }
#pragma unroll
    for (int i = 4 * tid; i < kBins; i += 4 * kBinThreads) *reinterpret_cast<uint4*>(&sh.hist[i]) = uint4{0u, 0u, 0u, 0u};
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
    vmin = fminf(fminf(sh.wmin[0], sh.wmin[1]), fminf(sh.wmin[2], sh.wmin[3]));
    vmax = fmaxf(fmaxf(sh.wmax[0], sh.wmax[1]), fmaxf(sh.wmax[2], sh.wmax[3]));
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
        if (lane < jmax) sh.ccnt[4 * lane + wv] = ccv;
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
            for (int i = tid; i < 256; i += kBinThreads) sh.hist[i] = 0u;
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
            block_find_bin<256>(sh, need, tid);
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
            if (lane == 0) sh.ccnt[4 * j + wv] = c;
        });
        __syncthreads();
        int total_eq;
        const int off = chunk_offsets(sh, nch, lane, &total_eq);
        visit_chunks<NCH, true>(jmax, jpart, [&](int j, auto) {
            int run = __builtin_amdgcn_readlane(off, 4 * j + wv);
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
        if (lane < jmax) sh.ccnt[4 * lane + wv] = ccv;
        __syncthreads();
    }
    int total;
    const int off = chunk_offsets(sh, nch, lane, &total);
    const int key0 = lo + lane + 256 * wv;
    char* so_b = reinterpret_cast<char*>(so);
    char* io_b = reinterpret_cast<char*>(io);
    {
        const float vT = sh.cut_v;
        const int iT = sh.cut_i;
        with_ties(sh.cut_ties != 0, [&](auto tie) {
            visit_chunks<NCH, AP>(jmax, jpart, [&](int j, auto) {
                int run = __builtin_amdgcn_readlane(off, 4 * j + wv);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bool f = selected(tie, j, m, vT, iT);
                    const unsigned long long mask = __ballot(f);
                    const uint32_t pos = (uint32_t)mbcnt(mask, run);
                    if (f && pos < (uint32_t)topk) {
                        *reinterpret_cast<In*>(so_b + pos * (uint32_t)sizeof(In)) = out_val(x[j][m]);
                        *reinterpret_cast<int32_t*>(io_b + pos * 4u) = key0 + 1024 * j + 64 * m;
                    }
                    run += __popcll(mask);
                }
            });
        });
    }
    for (int i = total + tid; i < topk; i += kBinThreads) { so[i] = pad_val; io[i] = -1; }
}

__global__ __launch_bounds__(256) void gather_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ idx, long total, int skv,
                                                     int topk, float* __restrict__ out) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const long row = i / topk;
    const int v = idx[i];
    out[i] = (v >= 0 && v < skv) ? logits[row * skv + v] : neg_inf();
}

template <int VEC, int WPR, int MINB>
static void launch_reg(const TopkArgs& p) {
    constexpr int rpb = kRowThreads / (64 * WPR);
    const long rows = (long)p.B * p.S;
    dim3 grid((unsigned)((rows + rpb - 1) / rpb));
    hipLaunchKernelGGL((topk_rows_reg_kernel<VEC, WPR, MINB>), grid, dim3(kRowThreads), 0, p.stream, p.logits, p.B,
                       p.S, p.Skv, p.ratio, p.ks, p.ke, p.topk, p.scores, p.indices);
}

hipError_t launch_topk_rows(const TopkArgs& p) {
    // Measured on MI355X: one register-resident wave per row wins for rows of
    // up to 2048 keys; longer rows go to the workgroup-per-row radix kernel
    // (register cache up to 8192 keys, re-reads beyond).  The two-wave
    // register variant (WPR = 2) measured slower at 8192 keys and is not used.
    if (p.Skv <= 2048) {
        launch_reg<8, 1, 4>(p);
    } else {
        dim3 grid((unsigned)((long)p.B * p.S));
        if (p.Skv <= 8192)
            hipLaunchKernelGGL((topk_rows_bin_kernel<8, false>), grid, dim3(kBinThreads), 0, p.stream,
                               static_cast<const void*>(p.logits), p.B, p.S, p.Skv, p.ratio, p.ks, p.ke, p.topk,
                               static_cast<void*>(p.scores), p.indices);
        else
            hipLaunchKernelGGL(topk_rows_kernel<0>, grid, dim3(kTopkThreads), 0, p.stream, p.logits, p.B, p.S,
                               p.Skv, p.ratio, p.ks, p.ke, p.topk, p.scores, p.indices);
    }
    return hipGetLastError();
}

hipError_t launch_topk_bf16(const TopkBf16Args& p) {
    dim3 grid((unsigned)((long)p.B * p.L));
    hipLaunchKernelGGL((topk_rows_bin_kernel<8, true>), grid, dim3(kBinThreads), 0, p.stream, p.scores, p.B, p.L,
                       p.G, 1, nullptr, nullptr, p.topk, p.out_scores, p.indices);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& p) {
    const long total = (long)p.B * p.S * p.topk;
    dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, p.stream, p.logits, p.indices, total, p.Skv, p.topk,
                       p.scores);
    return hipGetLastError();
}

}  // namespace lix

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

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "row_select.h"

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

// One workgroup of NW waves per row of materialized scores (select_row_binned):
// rows t_end - 1, t_end - 2, ... (longest causal rows first), gridDim.x / B of
// them.
template <int NCH, bool BF16, int NW>
__global__ __launch_bounds__(64 * NW) void topk_rows_bin_kernel(const void* __restrict__ logits_v, int B, int S,
                                                                    int t_end, int skv, int ratio,
                                                                    const int32_t* __restrict__ ks,
                                                                    const int32_t* __restrict__ ke, int topk,
                                                                    void* __restrict__ scores_v,
                                                                    int32_t* __restrict__ indices) {
    using In = RowIn<BF16>;
    __shared__ BinShared sh;
    const int b = blockIdx.x % B;
    const int t = t_end - 1 - (int)(blockIdx.x / B);
    int lo = 0, hi = skv;
    if constexpr (!BF16) key_range(ks, ke, t, S, skv, ratio, lo, hi);
    const In* row = static_cast<const In*>(logits_v) + ((long)b * S + t) * skv + lo;
    In* so = static_cast<In*>(scores_v) + ((long)b * S + t) * topk;
    int32_t* io = indices + ((long)b * S + t) * topk;
    select_row_binned<NCH, BF16, NW>(row, hi - lo, lo, topk, so, io, sh, threadIdx.x);
}

// Scores at given indices: one workgroup per row (rows blockIdx.x,
// blockIdx.x + gridDim.x, ...); each thread takes eight of the row's entries
// 256 apart, their index loads and then their gathers all in flight at once.
constexpr int kGatherUnroll = 8;
__global__ __launch_bounds__(256) void gather_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ idx, long rows, int skv,
                                                     int topk, float* __restrict__ out) {
    const int tid = threadIdx.x;
    for (long row = blockIdx.x; row < rows; row += gridDim.x) {
        const float* lrow = logits + row * skv;
        const int32_t* irow = idx + row * topk;
        float* orow = out + row * topk;
        for (int j0 = 0; j0 < topk; j0 += 256 * kGatherUnroll) {
            int v[kGatherUnroll];
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) {
                const int j = j0 + 256 * u + tid;
                v[u] = irow[min(j, topk - 1)];
            }
            float r[kGatherUnroll];
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) r[u] = lrow[min(max(v[u], 0), skv - 1)];
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) {
                const int j = j0 + 256 * u + tid;
                if (j < topk) orow[j] = (v[u] >= 0 && v[u] < skv) ? r[u] : neg_inf();
            }
        }
    }
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
    // up to 2048 keys; rows up to 8192 keys go to the binned workgroup kernel
    // (the row in the registers of four waves), up to 32768 keys to the same
    // kernel with eight or sixteen waves, longer ones to the radix kernel that
    // re-reads the row.  The two-wave register variant
    // (WPR = 2) measured slower at 8192 keys and is not used.
    if (p.Skv <= 2048) {
        launch_reg<8, 1, 4>(p);
    } else {
        dim3 grid((unsigned)((long)p.B * p.S));
        auto rows = [&](int t_lo, int t_hi) { return dim3((unsigned)((long)p.B * (t_hi - t_lo))); };
        if (p.Skv <= 8192) {
            hipLaunchKernelGGL((topk_rows_bin_kernel<8, false, 4>), grid, dim3(256), 0, p.stream,
                               static_cast<const void*>(p.logits), p.B, p.S, p.S, p.Skv, p.ratio, p.ks, p.ke, p.topk,
                               static_cast<void*>(p.scores), p.indices);
        } else if (p.Skv <= 32768) {
            // Causal rows of at most 16384 keys (t < 16384 ratio) fit the
            // registers of eight waves, which leaves room for two workgroups
            // per CU; longer rows take sixteen.
            const int t_split = p.ks == nullptr ? (int)std::min<long>(p.S, 16384L * p.ratio) : 0;
            if (t_split < p.S)
                hipLaunchKernelGGL((topk_rows_bin_kernel<8, false, 16>), rows(t_split, p.S), dim3(1024), 0, p.stream,
                                   static_cast<const void*>(p.logits), p.B, p.S, p.S, p.Skv, p.ratio, p.ks, p.ke,
                                   p.topk, static_cast<void*>(p.scores), p.indices);
            if (t_split > 0)
                hipLaunchKernelGGL((topk_rows_bin_kernel<8, false, 8>), rows(0, t_split), dim3(512), 0, p.stream,
                                   static_cast<const void*>(p.logits), p.B, p.S, t_split, p.Skv, p.ratio, p.ks, p.ke,
                                   p.topk, static_cast<void*>(p.scores), p.indices);
        } else {
            hipLaunchKernelGGL(topk_rows_kernel<0>, grid, dim3(kTopkThreads), 0, p.stream, p.logits, p.B, p.S,
                               p.Skv, p.ratio, p.ks, p.ke, p.topk, p.scores, p.indices);
        }
    }
    return hipGetLastError();
}

hipError_t launch_topk_bf16(const TopkBf16Args& p) {
    dim3 grid((unsigned)((long)p.B * p.L));
    hipLaunchKernelGGL((topk_rows_bin_kernel<8, true, 4>), grid, dim3(256), 0, p.stream, p.scores, p.B, p.L, p.L,
                       p.G, 1, nullptr, nullptr, p.topk, p.out_scores, p.indices);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& p) {
    const long rows = (long)p.B * p.S;
    dim3 grid((unsigned)(rows < (1L << 20) ? rows : (1L << 20)));
    hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, p.stream, p.logits, p.indices, rows, p.Skv, p.topk,
                       p.scores);
    return hipGetLastError();
}

}  // namespace lix

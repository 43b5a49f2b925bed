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
#pragma unroll
        for (int j = 0; j < CACHE; ++j) {
            const int e = (c_begin + j) * 64 + lane;
            cache[j] = (j < cw && c_begin + j < c_end && e < n) ? f32_to_key(row[e]) : 0u;
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

__global__ __launch_bounds__(256) void gather_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ idx, long total, int skv,
                                                     int topk, float* __restrict__ out) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const long row = i / topk;
    const int v = idx[i];
    out[i] = (v >= 0 && v < skv) ? logits[row * skv + v] : neg_inf();
}

hipError_t launch_topk_rows(const TopkArgs& p) {
    dim3 grid((unsigned)((long)p.B * p.S));
    const int cw = ((p.Skv + 63) / 64 + kTopkWaves - 1) / kTopkWaves;
    if (cw <= 32)
        hipLaunchKernelGGL(topk_rows_kernel<32>, grid, dim3(kTopkThreads), 0, p.stream, p.logits, p.B, p.S, p.Skv,
                           p.ratio, p.ks, p.ke, p.topk, p.scores, p.indices);
    else
        hipLaunchKernelGGL(topk_rows_kernel<0>, grid, dim3(kTopkThreads), 0, p.stream, p.logits, p.B, p.S, p.Skv,
                           p.ratio, p.ks, p.ke, p.topk, p.scores, p.indices);
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

// Shared pieces of the scoring kernels: tiling constants, query-fragment
// loads, key-tile staging through LDS and the per-column-block MFMA loop.
//
// GEMM view (one batch element): rows are (query t, head h) pairs, columns
// are keys s, the contraction runs over index_dim:
//     d[(t,h), s] = sum_i q[t,h,i] * k[s,i].
// A wave keeps the bf16 fragments of its rows (QW queries x H heads) in
// registers for the whole key loop; keys stream through LDS in stages of
// KT keys shared by the workgroup's waves.  Each 32-key column block of a
// stage is contracted with one MFMA chain per 32-row tile, and the per-head
// results are reduced into per-query scores in registers by the caller's
// epilogue, so per-head values never leave the chip.
#pragma once

#include "common.h"

namespace lix {

template <int H_, int DP_>
struct Tiling {
    static constexpr int H = H_;                    // heads (power of two, <= 128)
    static constexpr int DP = DP_;                  // index_dim padded up to 32/64/128/256
    static constexpr int NRT = (H >= 128) ? 4 : 2;  // 32-row MFMA tiles per wave
    static constexpr int ROWS = 32 * NRT;           // (query, head) rows per wave
    static constexpr int QW = ROWS / H;             // queries per wave
    static constexpr int NSTEP = DP / 16;           // MFMA k-steps over index_dim
    static constexpr int NWAVE = 4;
    static constexpr int THREADS = NWAVE * kWave;
    static constexpr int QB = QW * NWAVE;           // queries per workgroup
    static constexpr int KT = 64;                   // keys per LDS stage
    static constexpr int NCB = KT / 32;             // 32-key column blocks per stage
    static constexpr int STAGE_BYTES = KT * DP * 2;
    static constexpr int CHUNKS = KT * DP / 8;      // 16-byte chunks per stage
    static constexpr int CPT = CHUNKS / THREADS;    // chunks staged per thread
    static constexpr int CPK = DP / 8;              // chunks per key row
    static_assert(CPT >= 1 && CHUNKS % THREADS == 0, "stage must split evenly over the workgroup");
    static_assert(ROWS % H == 0, "a wave holds whole queries");

    // Query slot (0..QW-1) of accumulator i of row tile r, for a lane in the
    // lower half.  For H >= 8 both halves map to the same query; for H < 8
    // the upper half's query is this slot + 4 / H.
    static constexpr int slot(int r, int i) { return (32 * r + c_row(i, 0)) / H; }
    static constexpr int half_step() { return H >= 8 ? 0 : 4 / H; }
};

// Strides (in elements) of the three input tensors; the head stride of q is D.
struct InLayout {
    const uint16_t* q;
    long q_t, q_b;
    const uint16_t* k;
    long k_s, k_b;
    int D;
};

// Fragments of the wave's rows: a[r][st] holds rows 32r + (lane % 32),
// index_dim entries 16 st + 8 (lane / 32) + 0..7.  Queries past S and
// index_dim entries past D read as zero.  The addresses are clamped into q
// and the zeroing is a select, so the loads issue without branches.
template <class T>
__device__ __forceinline__ void load_q_frags(bf16x8 (&a)[T::NRT][T::NSTEP], const InLayout& L, int b,
                                             int tq0, int S, int lane) {
    const int hf = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) {
        const int row = 32 * r + r32;
        const int t = tq0 + row / T::H;
        const int h = row % T::H;
        const bool tv = t < S;
        const uint16_t* base = L.q + (long)min(t, S - 1) * L.q_t + (long)b * L.q_b + (long)h * L.D;
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const int d0 = 16 * st + 8 * hf;
            const bool ok = tv && (d0 < L.D);
            u32x4 v = *reinterpret_cast<const u32x4*>(base + min(d0, L.D - 8));
            if (!ok) v = u32x4{0u, 0u, 0u, 0u};
            a[r][st] = as_bf16x8(v);
        }
    }
}

// Static schedule of a persistent grid of G workgroups over nblk blocks
// ordered longest first: workgroup w takes blocks w, 2G-1-w, 2G+w, 4G-1-w, ...
// so each workgroup's pair of consecutive blocks has about the same total work.
__device__ __forceinline__ int sched_block(int w, int G, int i) {
    return (i & 1) ? (i + 1) * G - 1 - w : i * G + w;
}

// LDS position of the 16-byte chunk (column block cb, k-step st, fragment
// lane lp).  Within each 1 KiB fragment block the lane slot is XOR-swizzled
// so that the staging stores of 16 consecutive threads hit distinct banks;
// the fragment reads of a wave stay a permutation of one 1 KiB block.
template <class T>
__device__ __forceinline__ int stage_offset(int cb, int st, int lp) {
    const int sw = (2 * st + (lp >> 5)) & 15;
    return ((cb * T::NSTEP + st) * kWave + (lp ^ sw)) * 16;
}

// Global -> registers: this thread's chunks of the key stage starting at s0.
// Branch-free: rows past skv are clamped to the last key and index_dim chunks
// past D to the last real chunk, so every access stays inside k.  Clamped rows
// only feed scores of keys >= skv, which are never stored or selected, and
// clamped chunks meet zero query entries (load_q_frags), adding exact zeros.
template <class T>
__device__ __forceinline__ void load_k_stage(u32x4 (&pf)[T::CPT], const InLayout& L, const uint16_t* kb, int s0,
                                             int skv, int tid) {
    const int rowlim = skv - 1 - s0;                       // uniform
    const int dlim = (L.D >> 3) - 1;
    const uint16_t* base = kb + (long)s0 * L.k_s;          // uniform
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
        const int e = tid + i * T::THREADS;
        const int sl = min(e / T::CPK, rowlim);
        const int d8 = min(e % T::CPK, dlim);
        const uint32_t off = __umul24((uint32_t)sl, (uint32_t)L.k_s) + 8u * (uint32_t)d8;
        pf[i] = *reinterpret_cast<const u32x4*>(base + off);
    }
}

// Registers -> LDS in fragment order.
template <class T>
__device__ __forceinline__ void store_k_stage(uint8_t* stage, const u32x4 (&pf)[T::CPT], int tid) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
        const int e = tid + i * T::THREADS;
        const int sl = e / T::CPK, d8 = e % T::CPK;
        const int cb = sl >> 5, st = d8 >> 1, lp = (sl & 31) + 32 * (d8 & 1);
        *reinterpret_cast<u32x4*>(stage + stage_offset<T>(cb, st, lp)) = pf[i];
    }
}

// Key stages tile_lo .. tile_lo+ntile-1 stream through two LDS buffers.
// The global loads of stage it+1 are issued right after the barrier that
// opens stage it and are written to the other buffer once stage it has been
// computed, so they have a whole stage of MFMA work to land.  (The compiler
// waits for every outstanding vector-memory operation before those LDS
// writes, so results a body wants to store should be issued early in the
// next stage, not at the end of this one.)  body(it, stage) computes stage
// tile_lo+it from its LDS copy.  Every thread of the workgroup must call
// this with the same arguments.
template <class T, class Body>
__device__ __forceinline__ void stream_key_stages(const InLayout& L, int b, int skv, int tile_lo, int ntile,
                                                  uint8_t (*lds)[T::STAGE_BYTES], int tid, Body&& body) {
    const uint16_t* kb = L.k + (long)b * L.k_b;
    const int s_first = tile_lo * T::KT;
    u32x4 pf[T::CPT];
    load_k_stage<T>(pf, L, kb, s_first, skv, tid);
    store_k_stage<T>(lds[0], pf, tid);
    __syncthreads();
    for (int it = 0; it < ntile; ++it) {
        const bool more = it + 1 < ntile;
        if (more) load_k_stage<T>(pf, L, kb, s_first + (it + 1) * T::KT, skv, tid);
        body(it, lds[it & 1]);
        if (more) store_k_stage<T>(lds[(it + 1) & 1], pf, tid);
        __syncthreads();
    }
}

// d for the wave's rows against the 32 keys of column block cb of a staged tile.
template <class T>
__device__ __forceinline__ void mfma_block(f32x16 (&acc)[T::NRT], const bf16x8 (&a)[T::NRT][T::NSTEP],
                                           const uint8_t* stage, int cb, int lane) {
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) acc[r] = f32x16{};
#pragma unroll
    for (int st = 0; st < T::NSTEP; ++st) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(stage + stage_offset<T>(cb, st, lane));
        const bf16x8 bfrag = as_bf16x8(bv);
#pragma unroll
        for (int r = 0; r < T::NRT; ++r) acc[r] = mfma_32x32x16(a[r][st], bfrag, acc[r]);
    }
}

// Query handled by slot j of this lane.
template <class T>
__device__ __forceinline__ int slot_query(int tq0, int j, int hf) {
    return tq0 + j + hf * T::half_step();
}

}  // namespace lix

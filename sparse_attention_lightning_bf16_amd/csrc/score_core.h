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
// index_dim entries past D read as zero.
template <class T>
__device__ __forceinline__ void load_q_frags(bf16x8 (&a)[T::NRT][T::NSTEP], const InLayout& L, int b,
                                             int tq0, int S, int lane) {
    const int hf = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) {
        const int row = 32 * r + r32;
        const int t = tq0 + row / T::H;
        const int h = row % T::H;
        const uint16_t* base = L.q + (long)t * L.q_t + (long)b * L.q_b + (long)h * L.D;
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const int d0 = 16 * st + 8 * hf;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t < S && d0 < L.D) v = *reinterpret_cast<const u32x4*>(base + d0);
            a[r][st] = as_bf16x8(v);
        }
    }
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
template <class T>
__device__ __forceinline__ void load_k_stage(u32x4 (&pf)[T::CPT], const InLayout& L, int b, int s0,
                                             int skv, int tid) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
        const int e = tid + i * T::THREADS;
        const int sl = e / T::CPK, d8 = e % T::CPK;
        const int s = s0 + sl;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (s < skv && 8 * d8 < L.D)
            v = *reinterpret_cast<const u32x4*>(L.k + (long)s * L.k_s + (long)b * L.k_b + 8 * d8);
        pf[i] = v;
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

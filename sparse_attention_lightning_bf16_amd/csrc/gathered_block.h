// Gathered 32-key blocks: key rows named by an index list, moved into LDS by
// direct global->LDS loads, in a layout the MFMA B-fragment reads use
// without bank conflicts.
#pragma once

#include "score_core.h"

namespace lix {

// LDS placement of one gathered 32-key block (NLOAD loads of 64 lanes x 16
// bytes).  Load ld, lane L carries row segment p = RPI*ld + L/SEG, i.e. key
// row p % 32, chunks SEG*(p/32) .. +SEG-1, and within the segment the chunk
// (L % SEG) ^ swz(ld, L/SEG): consecutive lanes read one contiguous piece of
// a key row.  The swizzle makes the 16 (and each 8) consecutive lanes of a
// B-fragment read hit distinct 16-byte bank groups, and (8-chunk segments)
// each 32 (and 16) lanes of the backward's transposing reads of 8 keys x 32
// index_dim values distinct banks (an XOR of the row's three bits and the
// load's parity, found by a search over such masks).
template <int DP>
struct BlockMap {
    static constexpr int CPK = DP / 8;                  // 16-byte chunks per key row
    static constexpr int SEG = CPK < 8 ? CPK : 8;       // chunks per row segment
    static constexpr int RPI = 64 / SEG;                // row segments per load
    static constexpr int NLOAD = 32 * CPK / 64;         // loads per block
    static constexpr int NSTEP = DP / 16;
    static constexpr int BYTES = NLOAD * kWave * 16;   // one block in LDS
    static constexpr int KR = SEG == 8 ? 4 : NSTEP;     // distinct per-lane read offsets
    static_assert(SEG == 4 || SEG == 8, "row segments of 4 or 8 chunks");
    __device__ static constexpr int seg_swz(int m) {
        return ((m & 1) ? 2 : 0) ^ ((m & 2) ? 4 : 0) ^ ((m & 4) ? 1 : 0);
    }
    __device__ static constexpr int swz(int ld, int m) {
        return SEG == 8 ? (seg_swz(m) ^ ((ld & 1) ? 2 : 0)) : (((m >> 1) ^ (m >> 3)) & (SEG - 1));
    }
    // Byte offset of this lane's B fragment for k-step st: key row lane % 32,
    // chunk 2 st + lane / 32.  Equals frag_off(st % KR) + 4096 (st / KR).
    __device__ static constexpr int frag_off(int st, int lane) {
        const int r = lane & 31, c = 2 * st + (lane >> 5);
        const int p = 32 * (c / SEG) + r, ld = p / RPI, m = p % RPI;
        return 1024 * ld + 16 * (SEG * m + ((c % SEG) ^ swz(ld, m)));
    }
};

// Gather one block into buf: lane r < 32 holds the key row s of entry r (a
// valid row of kb, so s >= 0); lanes >= 32 hold a copy of lane r - 32's.
// Index_dim chunks past the last real one (dlim) are clamped to it.  Row
// offsets are unsigned 32 x 32 -> 64-bit products (the row stride k_s is
// below 2^24).
template <int DP>
__device__ __forceinline__ void gather_block(uint8_t* buf, const uint16_t* kb, long k_s, int dlim, int s, int lane) {
    using M = BlockMap<DP>;
    constexpr int NR = (32 / M::RPI) < M::NLOAD ? (32 / M::RPI) : M::NLOAD;
    const int m = lane / M::SEG, cp = lane % M::SEG;
    // The row of each load's lane comes from the lane that holds that entry.
    int rows[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) rows[j] = __shfl(s, (M::RPI * j + m) & 31);
#pragma unroll
    for (int ld = 0; ld < M::NLOAD; ++ld) {
        const int p = M::RPI * ld + m;
        const int d8 = min(M::SEG * (p >> 5) + (cp ^ M::swz(ld, m)), dlim);
        const uint16_t* src = kb + (uint64_t)(uint32_t)rows[ld % NR] * (uint32_t)k_s + 8 * d8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_ptr_t)(buf + ld * kWave * 16), 16,
                                         0, 0);
    }
}

}  // namespace lix

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
// lane lp): 1 KiB blocks in fragment order, lane-linear inside a block, so a
// wave's fragment read and a direct global->LDS load of one block both touch
// one contiguous 1 KiB (no bank conflicts).
template <class T>
__device__ __forceinline__ int stage_offset(int cb, int st, int lp) {
    return ((cb * T::NSTEP + st) * kWave + lp) * 16;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct global->LDS loads of the key stage starting at s0: each of the stage's
// NCB*NSTEP fragment blocks is one 64-lane load of 16 bytes per lane, written
// by the hardware to block base + 16*lane; wave w (wave-uniform) issues blocks
// w, w+NWAVE, ...
// Lane lp of block (cb, st) fetches key row s0 + 32cb + lp%32, index_dim chunk
// 2st + lp/32.  Rows past skv are clamped to the last key and chunks past D to
// the last real chunk, so every access stays inside k; clamped rows only feed
// scores of keys >= skv, which are never stored or selected, and clamped chunks
// meet zero query entries (load_q_frags), adding exact zeros.
template <class T>
__device__ __forceinline__ void dma_k_stage(uint8_t* stage, const InLayout& L, const uint16_t* kb, int s0, int skv,
                                            int wave, int lane) {
    static_assert((T::NCB * T::NSTEP) % T::NWAVE == 0, "fragment blocks split evenly over the waves");
    constexpr int PER_WAVE = T::NCB * T::NSTEP / T::NWAVE;
    const int rowlim = skv - 1 - s0;                      // uniform (wave is wave-uniform too)
    const int dlim = (L.D >> 3) - 1;
    const uint16_t* base = kb + (long)s0 * L.k_s;         // uniform
    if (rowlim >= T::KT - 1 && dlim >= 2 * T::NSTEP - 1) {
        // Whole stage inside k: nothing to clamp, and the lane's part of the
        // address is the same for every block (a per-block scalar base plus
        // one lane offset).
        const uint32_t lane_bytes =
            2u * (__umul24((uint32_t)(lane & 31), (uint32_t)L.k_s) + 8u * (uint32_t)(lane >> 5));
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int blk = wave + T::NWAVE * i;
            const int cb = blk / T::NSTEP, st = blk % T::NSTEP;
            const char* p = reinterpret_cast<const char*>(base + (long)(32 * cb) * L.k_s + 16 * st);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p + lane_bytes),
                                             (lds_ptr_t)(stage + blk * kWave * 16), 16, 0, 0);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int blk = wave + T::NWAVE * i;
        const int cb = blk / T::NSTEP, st = blk % T::NSTEP;
        const int row = min(32 * cb + (lane & 31), rowlim);
        const int d8 = min(2 * st + (lane >> 5), dlim);
        const uint32_t off = __umul24((uint32_t)row, (uint32_t)L.k_s) + 8u * (uint32_t)d8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + off),
                                         (lds_ptr_t)(stage + blk * kWave * 16), 16, 0, 0);
    }
}

// Key stages tile_lo .. tile_lo+ntile-1 stream through two LDS buffers (two
// separate arrays, so the compiler can tell that loads into one never alias
// reads of the other).  The loads of stage it+1 are issued right after the
// barrier that opens stage it and land while stage it is computed; the
// barrier's memory wait then covers them.  (That wait also covers every other
// outstanding vector-memory operation, so results a body stores should be
// issued early in the next stage.)  body(it, stage) computes stage
// tile_lo+it.  Every thread of the workgroup calls this with the same arguments.
template <class T, class Body>
__device__ __forceinline__ void stream_key_stages(const InLayout& L, int b, int skv, int tile_lo, int ntile,
                                                  uint8_t* lds0, uint8_t* lds1, int tid, Body&& body) {
    const uint16_t* kb = L.k + (long)b * L.k_b;
    const int s_first = tile_lo * T::KT;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    dma_k_stage<T>(lds0, L, kb, s_first, skv, wave, lane);
    __syncthreads();
    for (int it = 0; it < ntile; it += 2) {
        if (it + 1 < ntile) dma_k_stage<T>(lds1, L, kb, s_first + (it + 1) * T::KT, skv, wave, lane);
        body(it, lds0);
        __syncthreads();
        if (it + 1 >= ntile) break;
        if (it + 2 < ntile) dma_k_stage<T>(lds0, L, kb, s_first + (it + 2) * T::KT, skv, wave, lane);
        body(it + 1, lds1);
        __syncthreads();
    }
}

// B fragment of column block cb, k-step st of a staged tile.
template <class T>
__device__ __forceinline__ bf16x8 b_frag(const uint8_t* stage, int cb, int st, int lane) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(stage + stage_offset<T>(cb, st, lane)));
}

// One stage as a rolling pipeline over its NCB column blocks: each k-step of
// block c issues its MFMAs, each followed by a slice of the epilogue of block
// c-1 (that row tile's elements), so the VALU works on finished accumulators
// while the matrix pipe runs and the wave has VALU work between its MFMAs;
// only the last block's epilogue runs alone.  B fragments are read AHEAD k-steps
// ahead, across block boundaries.  Scheduling fences keep this order (the
// compiler would otherwise hoist the epilogue above the MFMAs and stall on
// results still in flight, or wait for each read right after issuing it).
// epi(cb, acc, r, i) handles element i of row tile r of block cb's finished
// accumulators; within a block the elements are visited in a fixed order, so
// every kernel that uses this stage sums a query's heads in the same order.
template <class T, class Epi>
__device__ __forceinline__ void rolling_stage(const bf16x8 (&a)[T::NRT][T::NSTEP], const uint8_t* stage, int lane,
                                              Epi&& epi) {
    static_assert(16 % T::NSTEP == 0, "the epilogue splits evenly over k-steps");
    constexpr int PER = 16 / T::NSTEP;                    // elements per row tile per step
    constexpr int NF = T::NCB * T::NSTEP;                 // fragments per stage, read in order
    // fragments in flight (one where the wave's A fragments alone fill the
    // register file: 128 heads x index_dim 256)
    constexpr int AHEAD = T::NRT * T::NSTEP >= 64 ? 1 : 3;
    f32x16 accp[T::NRT], accc[T::NRT];
    bf16x8 bq[AHEAD];
#pragma unroll
    for (int n = 0; n < AHEAD && n < NF; ++n) bq[n] = b_frag<T>(stage, n / T::NSTEP, n % T::NSTEP, lane);
#pragma unroll
    for (int cb = 0; cb < T::NCB; ++cb) {
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const int n = cb * T::NSTEP + st;
            const bf16x8 bc = bq[n % AHEAD];
            if (n + AHEAD < NF)
                bq[n % AHEAD] = b_frag<T>(stage, (n + AHEAD) / T::NSTEP, (n + AHEAD) % T::NSTEP, lane);
            // each row tile's MFMA is followed by that tile's epilogue slice,
            // so the wave has VALU work to issue while the matrix pipe runs
#pragma unroll
            for (int r = 0; r < T::NRT; ++r) {
                __builtin_amdgcn_sched_barrier(0);
                accc[r] = mfma_32x32x16(a[r][st], bc, st == 0 ? f32x16{} : accc[r]);
                __builtin_amdgcn_sched_barrier(0);
                if (cb > 0) {
#pragma unroll
                    for (int i = st * PER; i < (st + 1) * PER; ++i) epi(cb - 1, accp, r, i);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < T::NRT; ++r) accp[r] = accc[r];
    }
    __builtin_amdgcn_sched_barrier(0);
    // Same element order as above: (k-step slice, row tile, element).
#pragma unroll
    for (int st = 0; st < T::NSTEP; ++st)
#pragma unroll
        for (int r = 0; r < T::NRT; ++r)
#pragma unroll
            for (int i = st * PER; i < (st + 1) * PER; ++i) epi(T::NCB - 1, accp, r, i);
}

// The first NC column blocks of a T stage (same fragment layout).
template <class T, int NC>
struct FirstBlocks {
    static constexpr int NRT = T::NRT;
    static constexpr int NSTEP = T::NSTEP;
    static constexpr int NCB = NC;
};

// rolling_stage over the stage's first ncb column blocks only (ncb wave-uniform,
// 1 <= ncb): the blocks past it hold keys no query of the wave sees, so their
// MFMAs and epilogue are left out.  Same element order within each block.
template <class T, class Epi>
__device__ __forceinline__ void rolling_stage_first(const bf16x8 (&a)[T::NRT][T::NSTEP], const uint8_t* stage,
                                                    int lane, int ncb, Epi&& epi) {
    static_assert(T::NCB <= 4, "partial stages are instantiated for up to three blocks");
    if (ncb >= T::NCB) {
        rolling_stage<T>(a, stage, lane, epi);
    } else if constexpr (T::NCB > 1) {
        if (ncb == 1) {
            rolling_stage<FirstBlocks<T, 1>>(a, stage, lane, epi);
        } else if constexpr (T::NCB > 2) {
            if (ncb == 2) rolling_stage<FirstBlocks<T, 2>>(a, stage, lane, epi);
            else if constexpr (T::NCB > 3) rolling_stage<FirstBlocks<T, 3>>(a, stage, lane, epi);
        }
    }
}

// One stage block by block: each 32-key column block's MFMA chains (B
// fragments read one k-step ahead), then that block's epilogue, with no
// second set of accumulators.  For kernels run at three or more waves per
// SIMD, where other waves' MFMAs overlap a wave's epilogue.  epi(cb, acc)
// handles block cb's finished accumulators.
template <class T, class Epi>
__device__ __forceinline__ void plain_stage(const bf16x8 (&a)[T::NRT][T::NSTEP], const uint8_t* stage, int lane,
                                            Epi&& epi) {
#pragma unroll
    for (int cb = 0; cb < T::NCB; ++cb) {
        f32x16 acc[T::NRT];
        bf16x8 bn = b_frag<T>(stage, cb, 0, lane);
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const bf16x8 bc = bn;
            if (st + 1 < T::NSTEP) bn = b_frag<T>(stage, cb, st + 1, lane);
#pragma unroll
            for (int r = 0; r < T::NRT; ++r) acc[r] = mfma_32x32x16(a[r][st], bc, st == 0 ? f32x16{} : acc[r]);
        }
        epi(cb, acc);
    }
}

// Query handled by slot j of this lane.
template <class T>
__device__ __forceinline__ int slot_query(int tq0, int j, int hf) {
    return tq0 + j + hf * T::half_step();
}

}  // namespace lix

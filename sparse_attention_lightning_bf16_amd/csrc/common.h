// Device-side building blocks shared by the gfx950 kernels of liblix.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tiling.h"

namespace lix {

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time
// whatever the loop body's size (the register arrays it indexes must never be
// indexed at run time, and I can be a template or asm immediate argument).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 32x32x16 bf16 MFMA (CDNA4).  Operand layout, lane l = 0..63:
//   A (32 x 16): a[j] = A[l % 32][8 * (l / 32) + j], j = 0..7
//   B (16 x 32): b[j] = B[8 * (l / 32) + j][l % 32]
//   C (32 x 32): c[i] = C[8 * (i / 4) + 4 * (l / 32) + (i % 4)][l % 32]
__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// float <-> order-preserving unsigned key: a < b (as floats) iff key(a) < key(b).
// -0.0 is folded onto +0.0 so that equal floats have equal keys.
__device__ __forceinline__ uint32_t f32_to_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_f32(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// bf16 round-to-nearest-even of an fp32 value, returned as fp32
// (v_cvt_pk_bf16_f32 rounds to nearest even on gfx950).
__device__ __forceinline__ float round_bf16(float x) {
    uint16_t h = __builtin_bit_cast(uint16_t, (__bf16)x);
    return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ float neg_inf() { return __uint_as_float(0xff800000u); }

// max(0, x) as one integer max: a float with the sign bit set is a negative
// int32, every other float is a non-negative one whose order matches.
// (-0.0 becomes +0.0.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// c ? a : b on the bit patterns, so no select of addresses reaches the optimiser.
__device__ __forceinline__ float pick(bool c, float a, float b) {
    const int m = -(int)c;
    return __int_as_float((__float_as_int(a) & m) | (__float_as_int(b) & ~m));
}

// Visible key range of query t: [ks, ke) clamped to [0, skv]; causal when ks_arr is null.
__device__ __forceinline__ void key_range(const int32_t* __restrict__ ks_arr, const int32_t* __restrict__ ke_arr,
                                          int t, int S, int skv, int ratio, int& lo, int& hi) {
    if (t >= S) { lo = 0; hi = 0; return; }
    if (ks_arr == nullptr) {
        lo = 0;
        hi = min(skv, (t + 1) / ratio);
    } else {
        lo = min(max(ks_arr[t], 0), skv);
        hi = min(max(ke_arr[t], 0), skv);
    }
    if (hi < lo) hi = lo;
}

// v(lane) + v(lane ^ 32) in every lane.  v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; with v
// in both, the two results hold v's lower and upper halves in every lane, so
// no LDS round trip is needed.  The sum is the same in both halves (fp add
// commutes).
__device__ __forceinline__ float xor32_add(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Fill p[0..n) with -inf using 16-byte stores where alignment allows.
__device__ __forceinline__ void fill_neg_inf(float* __restrict__ p, long n, int tid, int nthreads) {
    if (n <= 0) return;
    const float ninf = neg_inf();
    long head = (long)(((16 - ((uintptr_t)p & 15)) & 15) >> 2);
    if (head > n) head = n;
    for (long i = tid; i < head; i += nthreads) p[i] = ninf;
    float* body = p + head;
    long nb = (n - head) >> 2;
    float4 v = make_float4(ninf, ninf, ninf, ninf);
    for (long i = tid; i < nb; i += nthreads) reinterpret_cast<float4*>(body)[i] = v;
    for (long i = head + 4 * nb + tid; i < n; i += nthreads) p[i] = ninf;
}

}  // namespace lix

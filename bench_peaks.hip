// Achievable-peak microbenchmarks for bench.py on gfx950: a pure bf16 MFMA
// loop (the dense matrix rate the scoring kernel is measured against) and
// streaming copy / read kernels (the HBM rate the top-k and V4.1 kernels are
// measured against).  Measurement infrastructure only: liblix does not use
// these.  Built by __graft_entry__.build() into bench_peaks.so beside this
// file.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// CHAINS independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave,
// iters rounds: 32*32*16*2 FLOP per MFMA.  Operands come from the thread index
// so nothing folds; one float per thread is written so nothing is removed.
template <int CHAINS>
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(int iters, float* __restrict__ out) {
    const int tid = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(float)((tid + j) & 7);
        b[j] = (__bf16)(float)((tid * 3 + j) & 5);
    }
    f32x16 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[c][j];
    out[(long)blockIdx.x * blockDim.x + tid] = s;
}

// dst = src, 16 bytes per thread per step, grid-stride.  NT: non-temporal
// loads and stores (streamed past the caches).
template <bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, long n4) {
    const long stride = (long)gridDim.x * blockDim.x;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        if constexpr (NT) {
            const f32x4 v = __builtin_nontemporal_load(src + i);
            __builtin_nontemporal_store(v, dst + i);
        } else {
            dst[i] = src[i];
        }
    }
}

// Sum of src, 16 bytes per thread per step, four loads in flight per thread;
// one float per thread written.
__global__ __launch_bounds__(256) void read_kernel(const float4* __restrict__ src, long n4, float* __restrict__ out) {
    const long stride = (long)gridDim.x * blockDim.x;
    float s = 0.0f;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        const float4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        s += (v0.x + v0.y + v0.z + v0.w) + (v1.x + v1.y + v1.z + v1.w) + (v2.x + v2.y + v2.z + v2.w) +
             (v3.x + v3.y + v3.z + v3.w);
    }
    for (; i < n4; i += stride) { const float4 v = src[i]; s += v.x + v.y + v.z + v.w; }
    out[(long)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

extern "C" {

// FLOP of one peak_mfma_bf16 launch.
double peak_mfma_flop(int blocks, int iters, int chains) {
    return (double)blocks * 4 /* waves */ * iters * chains * (32.0 * 32 * 16 * 2);
}

// blocks workgroups of 256 threads; out: blocks * 256 floats.  chains 4 or 8.
int peak_mfma_bf16(int blocks, int iters, int chains, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
    if (chains == 4)
        hipLaunchKernelGGL(mfma_loop_kernel<4>, dim3(blocks), dim3(256), 0, stream, iters, out);
    else if (chains == 8)
        hipLaunchKernelGGL(mfma_loop_kernel<8>, dim3(blocks), dim3(256), 0, stream, iters, out);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// n4 16-byte elements; blocks workgroups of 256 threads; nt: non-temporal.
int peak_copy(const void* src, void* dst, long n4, int blocks, int nt, hipStream_t stream) {
    if (src == nullptr || dst == nullptr || n4 <= 0 || blocks <= 0) return -1;
    if (nt)
        hipLaunchKernelGGL(copy_kernel<true>, dim3(blocks), dim3(256), 0, stream, (const f32x4*)src, (f32x4*)dst, n4);
    else
        hipLaunchKernelGGL(copy_kernel<false>, dim3(blocks), dim3(256), 0, stream, (const f32x4*)src, (f32x4*)dst,
                           n4);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// out: blocks * 256 floats.
int peak_read(const void* src, long n4, int blocks, float* out, hipStream_t stream) {
    if (src == nullptr || out == nullptr || n4 <= 0 || blocks <= 0) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, stream, (const float4*)src, n4, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"

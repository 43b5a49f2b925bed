// Backward of the indexer scores at given indices: gradients with respect to
// q, k and w.
//
// Page "...deepseek_v4.kernels.tilelang_indexer", V4IndexerFunction.backward
// (grad_scores, grad_indices), by the chain rule on the forward: for each
// valid entry j of query (b, t), key s = idx[b,t,j] in [ks, ke), upstream
// gradient g = grad_scores[b,t,j],
//     d_h = q[t,b,h,:] . k[s,b,:],   m_h = 1[d_h > 0]
//     dw[t,b,h]   += g * max(0, d_h)
//     dq[t,b,h,:] += g * w[t,b,h] * m_h * k[s,b,:]
//     dk[s,b,:]   += g * sum_h w[t,b,h] * m_h * q[t,b,h,:]
// Entries outside [ks, ke) (their score is the constant -inf) and the
// indices themselves get no gradient.
//
// dq and dw are sums over a query's own entries; dk is a sum over the queries
// that selected a key.  Each is computed where its sum is local, so no output
// element is accumulated with per-entry atomics, and every workspace array is
// sized by the entries (B*S*topk) or by groups of 64 keys, never by B*S*Skv:
//
//   1. backward_rows_kernel (query-major, one workgroup per query with one
//      wave per group of 32 heads, over the gathered 32-key blocks of the
//      scores-at kernel, which the waves share): d^T = K Q^T
//      recomputed per block (lanes are heads, accumulator rows keys); dw += g
//      relu(d^T) per lane; dq += (m g) K, whose A operand comes straight from
//      d^T's accumulators and whose B operand is the gathered block read
//      key-major; dq stays in registers for the whole row and is scaled by w at
//      the end.  Each entry's ReLU mask (one bit per head) goes to the
//      workspace.
//   2. bucket_entries_kernel: each row's valid entries {key, g, masks} sorted
//      into buckets of 64 keys (workspace).
//   3. dk_entries_kernel (key-major): a workgroup owns 256 keys (64 per wave)
//      and streams the queries that can see them; per query, each wave turns
//      its bucket into the A operand bf16(G w_h m_h) of its 64 keys (G the
//      summed g of a key) and dk += A Q accumulates in registers, with no
//      second recompute of q . k; q is read in its own layout.  The
//      workgroup's partial is added to dk once at the end.
//
// Every term of a gradient product carries one bfloat16 rounding, the one a
// bfloat16 autograd graph of the forward makes: the upstream factor is
// rounded (g for dq, with w applied in float32 at the end; the key's summed g
// times w_h for dk), the other operand (k for dq, q for dk) is the exact bf16
// input, and the products accumulate in float32; dw is float32 throughout.
#include <mutex>

#include "score_core.h"
#include "gathered_block.h"
#include "launch.h"
#include "lix.h"

namespace lix {

namespace {

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kKeysPerGroup = 256;        // keys per dk workgroup (64 per wave)
constexpr int kQueryChunk = 128;          // queries per dk workgroup

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (to nearest even) in one packed conversion.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Lane LANE of v takes the wave-uniform value s (v_writelane_b32).
template <int LANE>
__device__ __forceinline__ void write_lane(uint32_t& v, uint32_t s) {
    asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "i"(LANE));
}

// v_writelane_b32 can read an SGPR that a VALU instruction (a compare for a
// ballot) wrote just before it with its old value: wait states between the
// ballots and the lane writes that read them.  Every value passes through
// the statement, so each ballot is complete before it and each lane write
// after it.
__device__ __forceinline__ void settle_sgprs(unsigned long long (&v)[8]) {
    asm volatile("s_nop 4" : "+s"(v[0]), "+s"(v[1]), "+s"(v[2]), "+s"(v[3]), "+s"(v[4]), "+s"(v[5]), "+s"(v[6]),
                 "+s"(v[7]));
}

typedef __attribute__((address_space(1))) float gfloat;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Work items of the dk kernel, (query chunk z, batch b, key group kg), in the
// order the workgroups take them.  Workgroups go to the eight XCDs in turn
// (flat id i to XCD i % 8); XCD x takes the query chunks z = x, x + 8, ...,
// each with every key group that chunk can see, so the workgroups running on
// one XCD at a time are mostly the key groups of one query chunk and share
// that chunk's q through the XCD's L2.  Causal ranges: a chunk sees the key
// groups below its last query's range end; given ranges: all of them.
constexpr int kXcds = 8;

__host__ __device__ inline int dk_groups_seen(int z, int S, int skv, int ratio, bool causal, int nkg) {
    if (!causal) return nkg;
    const int t1 = min(S, (z + 1) * kQueryChunk);
    const int hi = min(skv, t1 / ratio);
    return (hi + kKeysPerGroup - 1) / kKeysPerGroup;
}

__host__ __device__ inline bool dk_item(long i, int B, int S, int skv, int ratio, bool causal, int& z, int& b,
                                        int& kg) {
    const int nkg = (skv + kKeysPerGroup - 1) / kKeysPerGroup;
    const int nz = (S + kQueryChunk - 1) / kQueryChunk;
    long m = i / kXcds;
    for (int zz = (int)(i % kXcds); zz < nz; zz += kXcds) {
        const int nv = dk_groups_seen(zz, S, skv, ratio, causal, nkg);
        const long cnt = (long)nv * B;
        if (m < cnt) {
            z = zz;
            b = (int)(m / nv);
            kg = (int)(m % nv);
            return true;
        }
        m -= cnt;
    }
    return false;
}

// Flat grid of the dk kernel: eight times the longest XCD list.
inline long dk_grid(int B, int S, int skv, int ratio, bool causal) {
    const int nkg = (skv + kKeysPerGroup - 1) / kKeysPerGroup;
    const int nz = (S + kQueryChunk - 1) / kQueryChunk;
    long longest = 0;
    for (int x = 0; x < kXcds; ++x) {
        long n = 0;
        for (int z = x; z < nz; z += kXcds) n += (long)dk_groups_seen(z, S, skv, ratio, causal, nkg) * B;
        longest = n > longest ? n : longest;
    }
    return longest * kXcds;
}

}  // namespace

// ---------------------------------------------------------------- entries by key group

// A head group's ReLU mask (bit l = head l) in pair order: bit i holds head
// 2i and bit 16 + i head 2i + 1 (the even heads in the low half, the odd in
// the high), so one 16-bit-lane shift pair turns a head pair into the mask of
// a packed bf16 pair.
__device__ __forceinline__ uint32_t pair_order(uint32_t x) {
    uint32_t t;
    t = (x ^ (x >> 1)) & 0x22222222u; x ^= t ^ (t << 1);
    t = (x ^ (x >> 2)) & 0x0C0C0C0Cu; x ^= t ^ (t << 2);
    t = (x ^ (x >> 4)) & 0x00F000F0u; x ^= t ^ (t << 4);
    t = (x ^ (x >> 8)) & 0x0000FF00u; x ^= t ^ (t << 8);
    return x;
}

// One workgroup per (b, t) (blockIdx.x = b * S + t): the row's valid entries
// (key in [ks, ke)) sorted into buckets of 64 keys (bucket g holds keys 64g ..
// 64g + 63), each entry {key, g bits, ReLU mask of heads 0-31, of heads
// 32-63} (16 bytes, masks in pair order), at ent[row][off[row][g] .. off[row][g
// + 1]); off has ngroups + 1 entries per row.  The order inside a bucket is
// not specified.
__global__ __launch_bounds__(256) void bucket_entries_kernel(const int32_t* __restrict__ indices,
                                                             const float* __restrict__ grad,
                                                             const uint32_t* __restrict__ masks, int nhg, int S,
                                                             int skv, int ratio, const int32_t* __restrict__ ks,
                                                             const int32_t* __restrict__ ke, int topk, int ngroups,
                                                             int32_t* __restrict__ off, u32x4* __restrict__ ent) {
    extern __shared__ int cnt[];                          // ngroups + 1 counters
    __shared__ int wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const long row = blockIdx.x;
    const int t = (int)(row % S);
    int lo, hi;
    key_range(ks, ke, t, S, skv, ratio, lo, hi);
    const int32_t* irow = indices + row * topk;
    const float* grow = grad + row * topk;
    const uint32_t* mrow = masks + row * topk * nhg;         // [head group][topk]
    for (int g = tid; g <= ngroups; g += 256) cnt[g] = 0;
    __syncthreads();
    for (int j = tid; j < topk; j += 256) {
        const int s = irow[j];
        if (s >= lo && s < hi) atomicAdd(&cnt[s >> 6], 1);
    }
    __syncthreads();
    // Exclusive prefix over the buckets: thread tid owns buckets
    // [PER * tid, PER * tid + PER) (ngroups <= 512 for seqlen_kv <= 32768).
    constexpr int PER = 2;
    int c[PER], local = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int g = PER * tid + k;
        c[k] = g < ngroups ? cnt[g] : 0;
        local += c[k];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d, 64);
        if (lane >= d) incl += u;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w2 = 0; w2 < wv; ++w2) run += wsum[w2];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    int32_t* orow = off + row * (ngroups + 1);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int g = PER * tid + k;
        if (g < ngroups) {
            orow[g] = run;
            cnt[g] = run;                                 // insertion point of bucket g
        }
        run += c[k];
    }
    if (tid == 0) orow[ngroups] = total;
    __syncthreads();
    u32x4* erow = ent + row * topk;
    for (int j = tid; j < topk; j += 256) {
        const int s = irow[j];
        if (s >= lo && s < hi) {
            const int pos = atomicAdd(&cnt[s >> 6], 1);
            const uint32_t m0 = pair_order(mrow[j]);
            const uint32_t m1 = nhg > 1 ? pair_order(mrow[topk + j]) : 0u;
            erow[pos] = u32x4{(uint32_t)s, __float_as_uint(grow[j]), m0, m1};
        }
    }
}

// ---------------------------------------------------------------- dq, dw (query-major)

// One workgroup per query, one wave per group of up to 32 heads: a wave's dq
// accumulators (32 x DP fp32) and q fragments leave room for two waves per
// SIMD, and the waves of a query share each gathered key block (each moves a
// part of it).
constexpr int rows_heads(int H) { return H > 32 ? 32 : H; }
constexpr int rows_waves(int H) { return H > 32 ? H / 32 : 1; }

// The loads ld = part * LPW .. part * LPW + LPW - 1 of gather_block (LPW =
// NLOAD / NPART): one wave's share of a block that NPART waves gather
// together.  The row of each load's lane comes from the lane that holds that
// entry (s >= 0 on every lane).
template <int DP, int NPART>
__device__ __forceinline__ void gather_share(uint8_t* buf, const uint16_t* kb, long k_s, int dlim, int s, int lane,
                                             int part) {
    using M = BlockMap<DP>;
    static_assert(M::NLOAD % NPART == 0, "block loads split evenly over the waves");
    constexpr int LPW = M::NLOAD / NPART;
    const int m = lane / M::SEG, cp = lane % M::SEG;
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int ld = part * LPW + u;
        const int p = M::RPI * ld + m;
        const int row = __shfl(s, p & 31);
        const int d8 = min(M::SEG * (p >> 5) + (cp ^ M::swz(ld, m)), dlim);
        const uint16_t* src = kb + (uint64_t)(uint32_t)row * (uint32_t)k_s + 8 * d8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_ptr_t)(buf + ld * kWave * 16), 16,
                                         0, 0);
    }
}

// LDS reads issued from inline assembly, each statement waiting for its own
// reads: the compiler's wait-count pass treats every ordinary LDS access as
// possibly touching a buffer that direct loads are still filling and waits
// for all of them; these reads (of buffers whose loads are known complete)
// are not held up that way.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
__device__ __forceinline__ void lds_read4_b128(u32x4& v0, u32x4& v1, u32x4& v2, u32x4& v3, uint32_t a0,
                                               uint32_t a1, uint32_t a2, uint32_t a3) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}
__device__ __forceinline__ void lds_read3_b32(uint32_t& v0, uint32_t& v1, uint32_t& v2, uint32_t a0, uint32_t a1,
                                              uint32_t a2) {
    asm volatile(
        "ds_read_b32 %0, %3\n\t"
        "ds_read_b32 %1, %4\n\t"
        "ds_read_b32 %2, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2)
        : "v"(a0), "v"(a1), "v"(a2)
        : "memory");
}
// Transposing reads (ds_read_b64_tr_b16) of N 8-byte pieces, N = 4 or 8.
template <int N>
__device__ __forceinline__ void lds_read_tr(i16x4 (&v)[N], const uint32_t (&a)[N]) {
    static_assert(N == 4 || N == 8, "four or eight transposing reads");
    if constexpr (N == 4) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4\n\t"
            "ds_read_b64_tr_b16 %1, %5\n\t"
            "ds_read_b64_tr_b16 %2, %6\n\t"
            "ds_read_b64_tr_b16 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
            : "memory");
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %9\n\t"
            "ds_read_b64_tr_b16 %2, %10\n\t"
            "ds_read_b64_tr_b16 %3, %11\n\t"
            "ds_read_b64_tr_b16 %4, %12\n\t"
            "ds_read_b64_tr_b16 %5, %13\n\t"
            "ds_read_b64_tr_b16 %6, %14\n\t"
            "ds_read_b64_tr_b16 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
              "=&v"(v[7])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
            : "memory");
    }
}
__device__ __forceinline__ void lds_write_b32(uint32_t a, float v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}

template <int H, int DP>
__global__ __launch_bounds__(kWave * rows_waves(H), 2) void backward_rows_kernel(InLayout L, const float* __restrict__ w,
                                                             const int32_t* __restrict__ indices,
                                                             const float* __restrict__ grad, int B, int S, int skv,
                                                             int ratio, const int32_t* __restrict__ ks,
                                                             const int32_t* __restrict__ ke, int topk,
                                                             float* __restrict__ dq, float* __restrict__ dw,
                                                             uint32_t* __restrict__ masks) {
    constexpr int HW = rows_heads(H);                // heads of this wave: h0 .. h0 + HW - 1
    constexpr int NHG = H / HW;                      // head groups per query: the workgroup's waves
    static_assert(NHG == rows_waves(H), "one wave per head group");
    using T = BwTiling<HW, DP>;
    using M = BlockMap<DP>;
    constexpr int LPW = M::NLOAD / NHG;              // gather loads per wave and block
    // Per block x (slot x % 3): the gathered keys, shared by the head groups,
    // and per wave the block's indices (lanes 0-31) and gradients (32-63).
    __shared__ __attribute__((aligned(16))) uint8_t buf0[M::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[M::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t buf2[M::BYTES];
    __shared__ __attribute__((aligned(16))) uint32_t ig0[NHG][64];
    __shared__ __attribute__((aligned(16))) uint32_t ig1[NHG][64];
    __shared__ __attribute__((aligned(16))) uint32_t ig2[NHG][64];
    __shared__ __attribute__((aligned(16))) float stage_g[NHG][32];

    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
    const int hq = __builtin_amdgcn_readfirstlane(tid >> 6);     // head group of this wave
    const int h0 = HW * hq;
    const int row = blockIdx.x;                                  // t * B + b
    const int b = row % B, t = row / B;
    const int D = L.D;
    int lo, hi;
    key_range(ks, ke, t, S, skv, ratio, lo, hi);

    // Q fragments: a[r][st] = q[head h0 + 32r + lane%32][16 st + 8 hf .. +7];
    // heads past the wave's group and index_dim entries >= D are zero.
    bf16x8 a[T::NRT][T::NSTEP];
    const uint16_t* qrow = L.q + (long)t * L.q_t + (long)b * L.q_b;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) {
        const int h = h0 + 32 * r + l32;
        const uint16_t* base = qrow + (long)min(h, H - 1) * D;
#pragma unroll
        for (int st = 0; st < T::NSTEP; ++st) {
            const int d0 = 16 * st + 8 * hf;
            u32x4 v = *reinterpret_cast<const u32x4*>(base + min(d0, D - 8));
            if (!(32 * r + l32 < HW && d0 < D)) v = u32x4{0u, 0u, 0u, 0u};
            a[r][st] = as_bf16x8(v);
        }
    }
    // Key-major B fragments of the dq product by transposing LDS reads
    // (ds_read_b64_tr_b16): within each group of 16 lanes, output lane 4b + e
    // receives, as its element a, element e of the 4 values source lane 4a + b
    // reads.  Fragment slot jj of lane l must hold (key 16s + 8(jj/4) + 4hf +
    // jj%4, index_dim 32dt + l%32): read rd = jj/4 gives slots 4rd .. 4rd + 3 if
    // source lane (group g, a, b) reads index_dim 32dt + 16(g%2) + 4b .. +3 of key
    // 16s + 8rd + 4(g/2) + a.  In the BlockMap placement (8-chunk segments) that
    // is byte tbase[dt%2][rd] + 1024(4(dt/2) + 2s + rd): load 4(dt/2) + 2s + rd
    // (parity rd), row m = 4(g/2) + a, chunk 4(dt%2) + 2(g%2) + b/2 of the segment.
    static_assert(M::SEG == 8, "transposing reads assume 8-chunk row segments");
    int tbase[2][2];
    {
        const int tg = lane >> 4, ta = (lane & 15) >> 2, tb = lane & 3;
        const int tm = 4 * (tg >> 1) + ta;                      // row within the 8-row load
        const int x0 = 2 * (tg & 1) + (tb >> 1);                 // chunk within the 32 index_dim values
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
            for (int rd = 0; rd < 2; ++rd)
                tbase[p2][rd] = 16 * (8 * tm + ((4 * p2 + x0) ^ M::swz(rd, tm))) + 8 * (tb & 1);
    }
    int fofs[M::KR];
#pragma unroll
    for (int kq = 0; kq < M::KR; ++kq) fofs[kq] = M::frag_off(kq, lane);

    const int32_t* irow = indices + ((long)b * S + t) * topk;
    const float* grow = grad + ((long)b * S + t) * topk;
    const uint16_t* kb = L.k + (long)b * L.k_b;
    const int dlim = (D >> 3) - 1;
    const int nb = (topk + 31) >> 5;

    // This lane's entry of block blk is 32 blk + lane%32 (clamped loads; the
    // entry number is checked where it is used).
    auto visible = [&](int idx, int blk) { return 32 * blk + l32 < topk && idx >= lo && idx < hi; };

    f32x16 dqacc[T::NRT][T::NDT];
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt) dqacc[r][dt] = f32x16{};
    float dwacc[T::NRT];
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) dwacc[r] = 0.0f;

    uint32_t* mrow = masks + (((long)b * S + t) * NHG + hq) * topk;     // [B,S,head group,topk]
    auto compute = [&](int blk, const uint8_t* buf, float g_own, bool vis) {
        f32x16 acct[T::NRT];
#pragma unroll
        for (int r = 0; r < T::NRT; ++r) acct[r] = f32x16{};
        __builtin_amdgcn_sched_barrier(0);
        static_assert(T::NSTEP % 4 == 0, "key fragments read four at a time");
#pragma unroll
        for (int s4 = 0; s4 < T::NSTEP; s4 += 4) {
            u32x4 kv[4];
            uint32_t ka[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int st = s4 + u;
                ka[u] = lds_addr(buf + fofs[st % M::KR] + 4096 * (st / M::KR));
            }
            lds_read4_b128(kv[0], kv[1], kv[2], kv[3], ka[0], ka[1], ka[2], ka[3]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int r = 0; r < T::NRT; ++r) acct[r] = mfma_32x32x16(as_bf16x8(kv[u]), a[r][s4 + u], acct[r]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // g of the entries on this lane's accumulator rows (row i is entry
        // 32 blk + c_row(i, hf)), through LDS; invalid entries get 0.  One
        // wave: its LDS operations run in order, no barrier needed.
        if (hf == 0) lds_write_b32(lds_addr(&stage_g[hq][l32]), vis ? g_own : 0.0f);
        float gv[16];
        {
            u32x4 gg[4];
            lds_read4_b128(gg[0], gg[1], gg[2], gg[3], lds_addr(&stage_g[hq][4 * hf]), lds_addr(&stage_g[hq][8 + 4 * hf]),
                           lds_addr(&stage_g[hq][16 + 4 * hf]), lds_addr(&stage_g[hq][24 + 4 * hf]));
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int e = 0; e < 4; ++e) gv[4 * q4 + e] = __uint_as_float(gg[q4][e]);
        }
        // ReLU masks of the block's entries for this wave's heads, for the dk
        // kernel: bit l of entry (32 blk + k) = d of head h0 + l > 0, where
        // accumulator slot i holds key c_row(i, hf) and lane l%32 head h0 + l%32.
        // Slot i's ballot holds the masks of keys c_row(i, 0) (low half) and
        // c_row(i, 1) (high half); lane k < 32 takes entry k's.
        {
            uint32_t mk = 0u;
            static_for<0, 2>([&](auto hc) {
                constexpr int i0 = 8 * decltype(hc)::value;
                unsigned long long bal[8];
                static_for<0, 8>([&](auto ic) { bal[ic] = __ballot(acct[0][i0 + ic] > 0.0f); });
                settle_sgprs(bal);
                static_for<0, 8>([&](auto ic) {
                    constexpr int i = i0 + decltype(ic)::value;
                    write_lane<c_row(i, 0)>(mk, (uint32_t)bal[ic]);
                    write_lane<c_row(i, 1)>(mk, (uint32_t)(bal[ic] >> 32));
                });
            });
            const int j = 32 * blk + l32;
            if (hf == 0 && j < topk) mrow[j] = mk;
        }
        // dw: lane = head 32r + lane%32, rows = keys c_row(i, hf).
#pragma unroll
        for (int r = 0; r < T::NRT; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) dwacc[r] = fmaf(gv[i], relu(acct[r][i]), dwacc[r]);
        // dq += (m * g) K over the block's 32 keys (two k-steps of 16).
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 kt[T::NDT];
            {
                i16x4 part[2 * T::NDT];
                uint32_t pa[2 * T::NDT];
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
                    for (int rd = 0; rd < 2; ++rd)
                        pa[2 * dt + rd] = lds_addr(buf + tbase[dt & 1][rd] + 1024 * (4 * (dt >> 1) + 2 * s + rd));
                lds_read_tr<2 * T::NDT>(part, pa);
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt)
                    kt[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[2 * dt], part[2 * dt + 1], 0, 1, 2,
                                                                                3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int r = 0; r < T::NRT; ++r) {
                u32x4 av;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int i0 = 8 * s + 2 * p;
                    av[p] = pack_bf16(acct[r][i0] > 0.0f ? gv[i0] : 0.0f, acct[r][i0 + 1] > 0.0f ? gv[i0 + 1] : 0.0f);
                }
                const bf16x8 af = as_bf16x8(av);
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt) dqacc[r][dt] = mfma_32x32x16(af, kt[dt], dqacc[r][dt]);
            }
        }
    };

    // Blocks go through three slots (block x in slot x % 3): each wave moves
    // the block's indices and gradients into its own part of the slot three
    // blocks ahead, and its share of the gathered keys two blocks ahead.
    // Every step issues the same loads (invisible entries and the blocks past
    // the row gather key row 0; the index loads are clamped into the row), in
    // this order: the indices and gradients of block blk + 3, then the share of
    // block blk + 2.  At step blk's start, then, waiting until at most LPW of
    // this wave's vector-memory operations are outstanding completes its
    // indices of block blk + 2 and its share of block blk (the share of block
    // blk + 1 may stay in flight); a barrier covers the other waves' shares
    // and puts every wave past its products on the buffer refilled next.
    // Steps come in threes with fixed buffers, so the compiler sees which
    // buffer each read and each direct load touches; no value read from
    // global memory crosses a step in a register.
    auto load_ig = [&](int blk, uint32_t (*ig)[64]) {
        const int j = min(32 * blk + l32, topk - 1);
        const void* src = hf ? reinterpret_cast<const void*>(grow + j) : reinterpret_cast<const void*>(irow + j);
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(&ig[hq][0]), 4, 0, 0);
    };
    auto gather = [&](int blk, int idx, uint8_t* buf) {
        gather_share<DP, NHG>(buf, kb, L.k_s, dlim, visible(idx, blk) ? idx : 0, lane, hq);
    };
    // (The wait and barrier that open a step end the one before it, and the
    // prologue, so every path into a step has waited the same way.)
    auto wait_and_barrier = [&]() {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(LPW));
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    auto step = [&](int blk, uint32_t (*ig_c)[64], uint32_t (*ig_2)[64], const uint8_t* cur, uint8_t* ahead2) {
        uint32_t i2u, icu, gcu;
        lds_read3_b32(i2u, icu, gcu, lds_addr(&ig_2[hq][l32]), lds_addr(&ig_c[hq][l32]), lds_addr(&ig_c[hq][32 + l32]));
        const int idx2 = (int)i2u, idx_c = (int)icu;
        const float g_c = __uint_as_float(gcu);
        // (The slot of block blk takes block blk + 3's indices after those reads.)
        load_ig(blk + 3, ig_c);
        gather(blk + 2, idx2, ahead2);
        const bool vis = visible(idx_c, blk);
        if (__ballot(vis) != 0ull) compute(blk, cur, g_c, vis);
        wait_and_barrier();
    };
    load_ig(0, ig0);
    load_ig(1, ig1);
    load_ig(2, ig2);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    {
        uint32_t i0, i1, g0;
        lds_read3_b32(i0, i1, g0, lds_addr(&ig0[hq][l32]), lds_addr(&ig1[hq][l32]), lds_addr(&ig0[hq][32 + l32]));
        gather(0, (int)i0, buf0);
        gather(1, (int)i1, buf1);
        // (g0 is read again by step 0; reading it here keeps every output of
        // the statement used.)
        asm volatile("" : : "v"(g0));
    }
    wait_and_barrier();
    for (int blk = 0; blk < nb; blk += 3) {
        step(blk, ig0, ig2, buf0, buf2);
        if (blk + 1 >= nb) break;
        step(blk + 1, ig1, ig0, buf1, buf0);
        if (blk + 2 >= nb) break;
        step(blk + 2, ig2, ig1, buf2, buf1);
    }

    // dq = w * accumulated (m g) K: rows are heads 32r + c_row(i, hf), columns
    // index_dim 32 dt + lane%32.
    const float* wrow = w + ((long)t * B + b) * H;
    float* dqrow = dq + ((long)t * B + b) * H * D;
#pragma unroll
    for (int r = 0; r < T::NRT; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hl = 32 * r + c_row(i, hf), h = h0 + hl;
            if (HW < 32 && hl >= HW) continue;
            const float wh = wrow[min(h, H - 1)];
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) {
                const int d = 32 * dt + l32;
                if (d < D) dqrow[(long)h * D + d] = wh * dqacc[r][dt][i];
            }
        }
    // dw: the two half-waves hold the same heads over different keys.
#pragma unroll
    for (int r = 0; r < T::NRT; ++r) {
        const float v = xor32_add(dwacc[r]);
        const int hl = 32 * r + l32;
        if (hf == 0 && hl < HW) dw[((long)t * B + b) * H + h0 + hl] = v;
    }
}

// ---------------------------------------------------------------- dk (key-major)

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Mask of a packed bf16 pair from a pair-order mask word shifted so that the
// pair's two bits sit at bits 15 and 31: each 16-bit half becomes all ones
// where its bit is set (an arithmetic shift of each half by 15).
__device__ __forceinline__ uint32_t half_masks(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, x) >> (short)15);
}

// Chunk swizzle of the dk kernel's staged q rows: chunk c (16 bytes) of head
// h sits at position c ^ q_swizzle(h) of the head's row.  The transposing
// reads of one fragment take 8 heads x 32 index_dim values; with rows of 256
// (or 128) bytes the unswizzled chunks of heads 4a .. 4a + 3 share their LDS
// banks, and this XOR (a search over XOR masks of the head's low bits) puts
// every 32 lanes of a read on 64 distinct banks and every 16 on 32.
template <int CPK>
__device__ __forceinline__ int q_swizzle(int h) {
    if constexpr (CPK == 16) return ((h & 1) ? 4 : 0) ^ ((h & 2) ? 10 : 0);
    else return ((h & 1) ? 2 : 0) ^ ((h & 2) ? 4 : 0);
}

// A workgroup owns 256 keys (64 per wave: wave w owns bucket 4 kg + w) and
// streams the queries of one chunk that can see them.  Per query, through a
// three-stage rotation of LDS buffers (one barrier per query), it moves in by
// direct loads the query's q rows (16-byte chunks in q_swizzle order) and
// each wave's bucket of entries (up to 64; more only with repeated keys), and
// writes the query's head weights in a replicated layout.  A wave builds a
// 64-slot table of its keys (summed g and ReLU masks, from the rows kernel's
// recompute) and forms the dk A operand bf16(G w_h) where m_h, else 0, for the
// heads of the B fragments, which transposing LDS reads take from the q rows
// (as they take the weights): the product needs no recompute of q . k.  dk
// stays in registers; the workgroup's partial is added to dk once at the end.
template <int H, int DP>
__global__ __launch_bounds__(256, 2) void dk_entries_kernel(const uint16_t* __restrict__ q,
                                                            const float* __restrict__ w,
                                                            const int32_t* __restrict__ off,
                                                            const u32x4* __restrict__ ent, int B, int S, int skv,
                                                            int ratio, const int32_t* __restrict__ ks,
                                                            const int32_t* __restrict__ ke, int topk, int ngroups,
                                                            int D, float* __restrict__ dk) {
    using T = BwTiling<H, DP>;
    // Stage: q rows of heads 0 .. 32 NRT - 1 (rows past H repeat head H - 1,
    // chunks past index_dim repeat its last chunk: they meet zero A entries or
    // feed dk columns that are not stored), the head weights in the layout the
    // transposing reads below take them from (weight h at 16 h: its low 16
    // bits four times, then its high 16 bits four times; heads past H repeat
    // w[H-1]) and each wave's bucket (64 entries of 16 bytes).
    constexpr int CPK = DP / 8;                              // 16-byte chunks per head row
    constexpr int QBYTES = 32 * T::NRT * DP * 2;
    constexpr int QBLK = QBYTES / 1024;                      // 1 KiB direct loads (one per wave instruction)
    constexpr int QT = 0, WS = QBYTES, ES = WS + 4 * 4 * 64;
    constexpr int STAGE = ES + 4 * 64 * 16;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[STAGE];
    __shared__ int offs[kQueryChunk][5];                    // bucket bounds of the chunk's queries
    __shared__ float tab_g[4][64];                          // per wave: summed g of its keys
    __shared__ uint2 tab_m[4][64];                          // per wave: ReLU masks of its keys (pair order)
    static_assert(QBLK % 4 == 0, "q blocks split over 4 waves");

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
    int zc, b, kg;
    if (!dk_item(blockIdx.x, B, S, skv, ratio, ks == nullptr, zc, b, kg)) return;   // uniform: before any barrier
    const int s_group = kg * kKeysPerGroup;
    const int s_wave = s_group + 64 * wave;                          // this wave's first key
    // Queries of this workgroup; with causal ranges no query before
    // ratio * (first key) - 1 sees any of its keys.
    int t0 = zc * kQueryChunk;
    const int t1 = min(S, t0 + kQueryChunk);
    if (ks == nullptr) t0 = (int)max((long)t0, (long)ratio * s_group - 1);
    if (t0 >= t1) return;                                  // uniform: before any barrier

    // Bucket bounds of buckets 4 kg .. 4 kg + 4 for every query of the chunk.
    for (int i = tid; i < (t1 - t0) * 5; i += 256) {
        const int qq = i / 5, k = i % 5;
        const long row = (long)b * S + t0 + qq;
        offs[qq][k] = off[row * (ngroups + 1) + min(4 * kg + k, ngroups)];
    }
    __syncthreads();

    // The q chunks this lane moves: LDS position P = 64 blk + lane holds
    // head P / CPK, chunk (P % CPK) ^ q_swizzle(head) (element offsets in a
    // query's [H, D] rows, clamped as above).
    static_assert(CPK == 8 || CPK == 16, "q rows of 128 or 256 bytes");
    int qofs[QBLK / 4];
#pragma unroll
    for (int u = 0; u < QBLK / 4; ++u) {
        const int pos = 64 * (wave + 4 * u) + lane, head = pos / CPK;
        const int c = (pos % CPK) ^ q_swizzle<CPK>(head);
        qofs[u] = min(head, H - 1) * D + 8 * min(c, D / 8 - 1);
    }
    auto stage = [&](int t, uint8_t* st_base) {
        const uint16_t* qrow = q + ((long)t * B + b) * H * D;
#pragma unroll
        for (int u = 0; u < QBLK / 4; ++u)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(qrow + qofs[u]),
                                             (lds_ptr_t)(st_base + QT + (wave + 4 * u) * 1024), 16, 0, 0);
        // The wave's bucket: lane i carries entry beg + i (clamped into the
        // row's topk entries; lanes past the bucket are ignored where the
        // entries are read).
        const int beg = offs[t - t0][wave], n = offs[t - t0][wave + 1] - beg;
        const long e = ((long)b * S + t) * topk + min(beg + min(lane, max(n - 1, 0)), topk - 1);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ent + e),
                                         (lds_ptr_t)(st_base + ES + 1024 * wave), 16, 0, 0);
    };

    // B fragments by transposing LDS reads (ds_read_b64_tr_b16): within each
    // group of 16 lanes, output lane 4b + e receives, as its element a,
    // element e of the 4 values source lane 4a + b reads.  Fragment (hs, dt)
    // slot jj of lane l must hold q[head 16 hs + 8(jj/4) + 4(l/32) + jj%4]
    // [index_dim 32 dt + l%32]: read rd = jj/4 gives slots 4rd .. 4rd + 3 if
    // source lane (group g, a, b) reads index_dim 32 dt + 16(g%2) + 4b .. +3
    // of head 16 hs + 8 rd + 4(g/2) + a, which the swizzled placement puts at
    // byte tq[dt] + 16 CPK (16 hs + 8 rd) (the swizzle depends on a alone).
    int tq[T::NDT];
    {
        const int sg = lane >> 4, sa = (lane & 15) >> 2, sb = lane & 3;
        const int hm = 4 * (sg >> 1) + sa;                        // head within the 8-head read
        const int x0 = 2 * (sg & 1) + (sb >> 1);                  // chunk within the 32 index_dim values
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt)
            tq[dt] = 16 * (hm * CPK + ((4 * dt + x0) ^ q_swizzle<CPK>(sa))) + 8 * (sb & 1);
    }

    f32x16 dkacc[2][T::NDT];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt) dkacc[kc][dt] = f32x16{};

    // The wave's table for one query: its 64 keys' summed g and ReLU masks,
    // built in LDS from its bucket and read back into registers (G, mw); n is
    // the bucket's size.  It is built one query ahead of the products.
    struct Tab {
        float G[2];
        uint32_t mw[2][T::NRT];
        int n;
    };
    auto prep = [&](int t, const uint8_t* st_base, Tab& tb) {
        const int beg = offs[t - t0][wave], n = offs[t - t0][wave + 1] - beg;
        tb.n = n;
        if (n == 0) return;                                          // no entry of this wave's keys
        // Every LDS operation of one wave runs in program order: clear, then
        // add / store, then read back.
        tab_g[wave][lane] = 0.0f;
        tab_m[wave][lane] = uint2{0u, 0u};
        auto put = [&](const u32x4& e) {
            const int sl = (int)e.x - s_wave;                        // 0..63: the bucket's keys
            atomicAdd(&tab_g[wave][sl], __uint_as_float(e.y));       // repeated keys: their g summed
            tab_m[wave][sl] = uint2{e.z, e.w};                       // repeated keys: the same mask
        };
        if (lane < n) put(*reinterpret_cast<const u32x4*>(st_base + ES + 1024 * wave + 16 * lane));
        for (int i0 = 64; i0 < n; i0 += 64) {                        // more than 64 entries: repeats
            const int i = i0 + lane;
            if (i < n) put(ent[((long)b * S + t) * topk + beg + i]);
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            tb.G[kc] = tab_g[wave][32 * kc + l32];
            const uint2 m = tab_m[wave][32 * kc + l32];
            // Pair i of heads 32r + 2i, + 2i + 1 at bits i and 16 + i; this
            // lane's pairs start at 2 hf.
            tb.mw[kc][0] = m.x >> (2 * hf);
            if constexpr (T::NRT > 1) tb.mw[kc][1] = m.y >> (2 * hf);
        }
    };

    // dk += A Q for one query: A row = key 32 kc + lane%32, k = the 8 heads
    // 32r + 16s + 8(jj/4) + 4hf + jj%4 of fragment hs = 2r + s; A = bf16(G w_h)
    // where the head's mask bit is set, else 0; B the query's exact q.
    // The weights of a stage: thread i loads weight i / 4 (one stage ahead)
    // and writes LDS dword i of the replicated layout, its half (i / 2) % 2
    // twice.
    auto load_w = [&](int t) { return __float_as_uint(w[((long)t * B + b) * H + min(tid >> 2, H - 1)]); };
    auto put_w = [&](uint32_t bits, uint8_t* st_base) {
        const uint32_t h = ((tid >> 1) & 1) ? (bits >> 16) : (bits & 0xFFFFu);
        *reinterpret_cast<uint32_t*>(st_base + WS + 4 * tid) = h | (h << 16);
    };
    // Weights by transposing reads: source lane 4a + b of a 16-lane group
    // reads the 8 bytes at WS + 16 h + 8 a, which hold one half of weight h
    // (a even: low, odd: high; h + 1 for a >= 2) four times, so every output
    // lane receives weights h and h + 1 whole.  (Neither these reads nor the q
    // reads are ordinary LDS loads for the compiler's wait-count pass, so the
    // direct loads of the next stage in flight do not hold them up.)
    const int wofs = WS + 8 * ((lane & 15) >> 2);
    auto products = [&](const uint8_t* st_base, const Tab& tb) {
        if (tb.n == 0) return;
#pragma unroll
        for (int r = 0; r < T::NRT; ++r)
#pragma unroll
            for (int sst = 0; sst < 2; ++sst) {
                const int hs = 2 * r + sst;
                bf16x8 qf[T::NDT];
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt) {
                    i16x4 part[2];
#pragma unroll
                    for (int rd = 0; rd < 2; ++rd)
                        part[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(
                            const_cast<uint8_t*>(st_base) + QT + 16 * CPK * (16 * hs + 8 * rd) + tq[dt]));
                    qf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
                float wv[8];
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) {
                    // weights 32r + 8(2 sst + k2/2) + 4hf + 2(k2%2), + 1
                    const int h = 32 * r + 8 * (2 * sst + (k2 >> 1)) + 4 * hf + 2 * (k2 & 1);
                    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(const_cast<uint8_t*>(st_base) + wofs + 16 * h));
                    const f32x2 f = __builtin_bit_cast(f32x2, v);
                    wv[2 * k2] = f[0];
                    wv[2 * k2 + 1] = f[1];
                }
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    u32x4 av;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        // heads 32r + 16 sst + 8(p/2) + 4hf + 2(p%2) and + 1: pair
                        // 8 sst + 4(p/2) + 2hf + p%2, at bits ip and 16 + ip of mw.
                        const int ip = 8 * sst + 4 * (p >> 1) + (p & 1);
                        av[p] = pack_bf16(tb.G[kc] * wv[2 * p], tb.G[kc] * wv[2 * p + 1]) &
                                half_masks(tb.mw[kc][r] << (15 - ip));
                    }
                    const bf16x8 af = as_bf16x8(av);
#pragma unroll
                    for (int dt = 0; dt < T::NDT; ++dt) dkacc[kc][dt] = mfma_32x32x16(af, qf[dt], dkacc[kc][dt]);
                }
            }
    };

    auto drain_and_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0070);                    // vmcnt(0) lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // Per query t: the weights and the table of t + 1 (the bucket from stage
    // t + 1, complete), then the weight and direct loads of stage t + 2, then
    // the products of t (transposing reads and registers only), then a wait
    // for every load in flight and a barrier: no ordinary LDS access runs
    // while direct loads are outstanding, and the loads of stage t + 2 land
    // during the products.
    Tab tb;
    uint32_t wn = 0;                                           // weight bits of the next stage
    auto iter = [&](int t, const uint8_t* cur, uint8_t* next, uint8_t* ahead2) {
        Tab tn;
        tn.n = 0;
        if (t + 1 < t1) {
            put_w(wn, next);
            prep(t + 1, next, tn);
        }
        if (t + 2 < t1) {
            wn = load_w(t + 2);
            stage(t + 2, ahead2);
        }
        products(cur, tb);
        tb = tn;
        drain_and_barrier();
    };
    stage(t0, lds0);
    if (t0 + 1 < t1) stage(t0 + 1, lds1);
    const uint32_t w0 = load_w(t0);
    if (t0 + 1 < t1) wn = load_w(t0 + 1);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    put_w(w0, lds0);
    prep(t0, lds0, tb);
    drain_and_barrier();
    for (int t = t0; t < t1; t += 3) {
        iter(t, lds0, lds1, lds2);
        if (t + 1 >= t1) break;
        iter(t + 1, lds1, lds2, lds0);
        if (t + 2 >= t1) break;
        iter(t + 2, lds2, lds0, lds1);
    }

    // dk rows of the wave's keys: key s_wave + 32kc + c_row(i, hf), index_dim
    // 32 dt + lane%32; added to dk (other query chunks add theirs).
    gfloat* dkb = (gfloat*)dk + (long)b * D + l32;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int s = s_wave + 32 * kc + c_row(i, hf);
            if (s >= skv) continue;
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt)
                if (32 * dt + l32 < D)
                    __hip_atomic_fetch_add(dkb + (long)s * B * D + 32 * dt, dkacc[kc][dt][i], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
}

// ---------------------------------------------------------------- launch

__global__ void zero_f32_kernel(float* __restrict__ p, long n4) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x)
        reinterpret_cast<float4*>(p)[i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
}

template <int H, int DP>
static hipError_t launch_backward_t(const BackwardArgs& p) {
    InLayout L{static_cast<const uint16_t*>(p.q), (long)p.B * H * p.D, (long)H * p.D,
               static_cast<const uint16_t*>(p.k), (long)p.B * p.D, (long)p.D, p.D};
    const BackwardLayout ly = backward_layout(p.B, p.S, p.Skv, H, p.D, p.topk);
    uint8_t* ws = static_cast<uint8_t*>(p.workspace);
    uint32_t* masks = reinterpret_cast<uint32_t*>(ws + ly.masks);
    int32_t* off = reinterpret_cast<int32_t*>(ws + ly.off);
    u32x4* ent = reinterpret_cast<u32x4*>(ws + ly.ent);
    const unsigned rows = (unsigned)((long)p.B * p.S);
    const int nhg = H / rows_heads(H);
    const int ngroups = (p.Skv + 63) / 64;
    if (ngroups > 512) return hipErrorInvalidValue;          // the bucket kernel's prefix covers 512 buckets
    hipLaunchKernelGGL((backward_rows_kernel<H, DP>), dim3(rows), dim3(kWave * rows_waves(H)), 0, p.stream, L, p.w,
                       p.indices, p.grad, p.B, p.S, p.Skv, p.ratio, p.ks, p.ke, p.topk, p.dq, p.dw, masks);
    hipLaunchKernelGGL(bucket_entries_kernel, dim3(rows), dim3(256), (size_t)(ngroups + 1) * 4, p.stream, p.indices,
                       p.grad, masks, nhg, p.S, p.Skv, p.ratio, p.ks, p.ke, p.topk, ngroups, off, ent);
    const long grid = dk_grid(p.B, p.S, p.Skv, p.ratio, p.ks == nullptr);
    hipLaunchKernelGGL((dk_entries_kernel<H, DP>), dim3((unsigned)grid), dim3(256), 0, p.stream,
                       static_cast<const uint16_t*>(p.q), p.w, off, ent, p.B, p.S, p.Skv, p.ratio, p.ks, p.ke,
                       p.topk, ngroups, p.D, p.dk);
    return hipGetLastError();
}

template <int H>
static hipError_t dispatch_dp_backward(const BackwardArgs& p) {
    switch (padded_dim(p.D)) {
        case 64: return launch_backward_t<H, 64>(p);
        case 128: return launch_backward_t<H, 128>(p);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- allocation-free workspace

// The workspace of lix_indexer_backward_noalloc: one static device array,
// which every GPU the library runs on holds (its own copy) until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory: the launchers only ever receive the device address that
// hipGetSymbolAddress returns for the current device, taken once per device.
static __device__ __align__(256) uint8_t scratch[LIX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t noalloc_workspace(void** ptr, long* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = LIX_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

hipError_t launch_indexer_backward(const BackwardArgs& p) {
    // dk is a sum of workgroup partials: clear it first (a fill kernel, so the
    // sequence can be captured).
    const long n4 = (long)p.Skv * p.B * p.D / 4;
    const long blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, p.stream,
                       p.dk, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (p.H) {
        case 1: return dispatch_dp_backward<1>(p);
        case 2: return dispatch_dp_backward<2>(p);
        case 4: return dispatch_dp_backward<4>(p);
        case 8: return dispatch_dp_backward<8>(p);
        case 16: return dispatch_dp_backward<16>(p);
        case 32: return dispatch_dp_backward<32>(p);
        case 64: return dispatch_dp_backward<64>(p);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lix

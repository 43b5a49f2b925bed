// Tiling constants of the gfx950 kernels, in plain C++ (no HIP types), so the
// host-side size checks (limits.cpp, api.cpp) and the kernels read the same
// numbers.
//
// Scoring GEMM view (one batch element): rows are (query t, head h) pairs,
// columns are keys s, the contraction runs over index_dim.  A wave holds the
// bf16 fragments of its rows (QW queries x H heads) for the whole key loop;
// keys stream through LDS in stages of KT keys shared by the workgroup's
// waves.
#pragma once

namespace lix {

constexpr int kWave = 64;

// Row of the 32x32 MFMA C tile held in accumulator slot i by a lane in half
// `hf` (lane / 32):  c[i] = C[8 * (i / 4) + 4 * hf + (i % 4)][lane % 32].
constexpr int c_row(int i, int hf) { return 8 * (i / 4) + 4 * hf + (i % 4); }

// index_dim rounded up to the compiled fragment depth (zero-padded in the kernels).
constexpr int padded_dim(int D) { return D <= 32 ? 32 : D <= 64 ? 64 : D <= 128 ? 128 : 256; }

// Keys per LDS stage: 128 where the rolling epilogue pipeline fits two
// waves per SIMD (H <= 64, index_dim <= 128), else 64.
constexpr int default_kt(int H, int DP) { return (H <= 64 && DP <= 128) ? 128 : 64; }
// Waves per SIMD the register allocator is held to for those shapes.
constexpr int stage_min_waves(int H, int DP) { return (H >= 16 && default_kt(H, DP) == 128) ? 2 : 1; }

template <int H_, int DP_, int KT_ = default_kt(H_, DP_), int NW_ = 4>
struct Tiling {
    static constexpr int H = H_;                    // heads (power of two, <= 128)
    static constexpr int DP = DP_;                  // index_dim padded up to 32/64/128/256
    static constexpr int NRT = (H >= 128) ? 4 : 2;  // 32-row MFMA tiles per wave
    static constexpr int ROWS = 32 * NRT;           // (query, head) rows per wave
    static constexpr int QW = ROWS / H;             // queries per wave
    static constexpr int NSTEP = DP / 16;           // MFMA k-steps over index_dim
    static constexpr int NWAVE = NW_;               // waves per workgroup, one after another in query order
    static constexpr int THREADS = NWAVE * kWave;
    static constexpr int QB = QW * NWAVE;           // queries per workgroup
    static constexpr int KT = KT_;                  // keys per LDS stage
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

// Waves per workgroup of the logits kernel (lix_indexer_logits): where two
// waves per SIMD fit, eight waves (one workgroup per CU) share each key stage,
// which halves the key traffic from L2 into LDS against two workgroups of
// four.  The streaming top-k keeps four (its selection runs on 256 threads).
constexpr int logits_waves(int H, int DP) { return stage_min_waves(H, DP) == 2 ? 8 : 4; }

// ---------------------------------------------------------------- fused top-k

// Key stages of 128 keys for 64 heads (index_dim <= 128; four queries per
// workgroup), else 64, so that the candidate buffers of the workgroup's
// queries keep room for topk up to 2048 next to the two stage buffers.
template <int H, int DP>
using FusedTiling = Tiling<H, DP, (H == 64 && DP <= 128) ? 128 : 64>;

constexpr long kFusedLdsBudget = 160 * 1024;     // LDS of one CU
constexpr int kFusedEntryBytes = 6;              // u32 order-preserving key + u16 key index
constexpr int kFusedMaxSkv = 65536;              // key indices are stored in 16 bits

// Candidate capacity per query of the fused kernel for this topk: 2 topk (a
// multiple of 64), at least topk + 64 (room for one ballot of appends after a
// compaction), at most what fits next to the staging tiles; -1 when even
// topk + 64 does not fit.
template <int H, int DP>
constexpr long fused_cap(int topk) {
    using T = FusedTiling<H, DP>;
    const long fixed = 2L * T::STAGE_BYTES + T::NWAVE * 256 * 4;
    const long per_entry = (long)T::QB * kFusedEntryBytes;
    const long max_cap = ((kFusedLdsBudget - fixed) / per_entry) & ~63L;
    long want = ((2L * topk + 63) / 64) * 64;
    if (want < topk + 64) want = topk + 64;
    const long cap = want < max_cap ? want : max_cap;
    return cap >= topk + 64 ? cap : -1;
}

// ---------------------------------------------------------------- backward

template <int H_, int DP_>
struct BwTiling {
    static constexpr int H = H_;
    static constexpr int DP = DP_;
    static constexpr int NRT = H > 32 ? 2 : 1;       // 32-row head tiles (padded rows are zero)
    static constexpr int NSTEP = DP / 16;            // k-steps of the recompute over index_dim
    static constexpr int NDT = DP / 32;              // 32-column index_dim tiles of dq and dk
    static constexpr int NHS = 2 * NRT;              // 16-head k-steps of the dk product
    static constexpr int QS_BYTES = NRT * NSTEP * 1024;   // q of one query, A-fragment order
    static constexpr int QT_BYTES = NHS * NDT * 1024;     // q of one query, dk B-fragment order
    static_assert(H <= 64 && (DP == 64 || DP == 128), "backward tiles cover H <= 64, index_dim 33..128");
};

}  // namespace lix

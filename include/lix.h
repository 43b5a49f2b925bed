/*
 * lix.h - C ABI of the MI355X (gfx950) lightning-indexer library, liblix.so.
 *
 * The DeepSeek-V4 lightning indexer scores every (query t, compressed key s)
 * pair as
 *     logits[b,t,s] = sum_h w[t,b,h] * max(0, q[t,b,h,:] . k[s,b,:])
 * (the DSA indexer form adapted to V4's SBHD layout and causal masking, page
 * "nemo_automodel.components.models.deepseek_v4.kernels.tilelang_indexer",
 * module header), keeps only keys inside the query's range and selects the
 * per-query top-k.  The V4.1 variant rounds to BF16 at two points and takes
 * a visibility mask (page "nemo_automodel.components.models.deepseek_v41.indexer").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor argument is a device pointer to dense, row-major
 *           memory on the current HIP device, allocated and owned by the
 *           caller.  The library allocates nothing, keeps no pointer after
 *           the call returns and has no mutable global state.
 * bf16.     bfloat16 tensors travel as raw 16-bit words (const void*).
 * Alignment. q/k/queries/keys: 16 bytes; float and int32 tensors: 4 bytes;
 *           bf16 weights and scores: 2 bytes.
 * Streams.  Work is enqueued on `stream` (a hipStream_t; NULL is the null
 *           stream) and is asynchronous: results are valid once the caller
 *           synchronises with that stream.
 * Ranges.   A query's visible keys are the half-open range [ks[t], ke[t]),
 *           clamped to [0, Skv].  When ks and ke are both NULL the causal
 *           range over compressed positions is used: ks = 0 and
 *           ke = min(Skv, (t+1) / compress_ratio) (page
 *           "...deepseek_v4.kernels.tilelang_indexer_fwd", section
 *           _make_causal_cu_seqlens).  Given arrays are int32 [S], shared
 *           by every batch element (section batched_indexer_fwd).
 * Errors.   Arguments are validated synchronously before anything is
 *           enqueued.  On failure the call returns a negative lix_status,
 *           enqueues nothing and leaves every output untouched:
 *             LIX_ERR_NULL        a required pointer is NULL;
 *             LIX_ERR_SHAPE       a size <= 0, topk < 1 or topk > Skv,
 *                                 compress_ratio < 1, or only one of ks/ke;
 *             LIX_ERR_UNSUPPORTED heads not a power of two <= 128,
 *                                 index_dim not a multiple of 16 or above
 *                                 256, a misaligned pointer, a size whose
 *                                 element count overflows int64 indexing
 *                                 limits, batch * index_dim >= 2^24 (the
 *                                 key row stride of the V4 kernels), or a
 *                                 shape the fused top-k cannot hold on chip
 *                                 (see lix_topk);
 *             LIX_ERR_DEVICE      a pointer that is not device memory of
 *                                 the current device (page
 *                                 "...deepseek_v41.indexer", indexer_scores:
 *                                 all inputs on the same device);
 *             LIX_ERR_LAUNCH      the kernel launch itself failed.
 *           Faults during execution surface at the caller's synchronise.
 */
#ifndef LIX_H
#define LIX_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LIX_OK = 0,
    LIX_ERR_NULL = -1,
    LIX_ERR_SHAPE = -2,
    LIX_ERR_UNSUPPORTED = -3,
    LIX_ERR_DEVICE = -4,
    LIX_ERR_LAUNCH = -5
} lix_status;

/* Largest topk the fused scoring + top-k path (lix_topk with logits == NULL)
 * keeps on chip. */
#define LIX_FUSED_TOPK_MAX 2048

/* Human-readable name of a status code; never NULL, static storage. */
const char* lix_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int lix_version(void);

/*
 * lix_indexer_logits - masked indexer logits for every (query, key) pair.
 *
 * Pages: "...deepseek_v4.kernels.tilelang_indexer_fwd", sections
 * batched_indexer_fwd (q [S,B,H,D] bf16, k [Skv,B,D] bf16, weights [S,B,H]
 * fp32 -> [B,S,Skv] fp32; ranges [S] shared by the batch) and clean_logits_
 * (positions outside a query's range are cleaned; here they hold -inf).
 *
 *   q       bf16 [S, B, H, D]      (SBHD)
 *   k       bf16 [Skv, B, D]
 *   w       fp32 [S, B, H]
 *   ks, ke  int32 [S] each, or both NULL for the causal range of compress_ratio
 *   logits  fp32 [B, S, Skv]  out: the score inside [ks,ke), -inf elsewhere
 */
int lix_indexer_logits(const void* q, const void* k, const float* w,
                       int B, int S, int Skv, int H, int D, int compress_ratio,
                       const int32_t* ks, const int32_t* ke,
                       float* logits, hipStream_t stream);

/*
 * lix_indexer_logits_visible - the same logits at the visible positions only.
 *
 * As lix_indexer_logits (same pages, arguments, validation and errors), for
 * callers that read only the positions inside each query's range, such as
 * lix_topk over the buffer: every position inside [ks, ke) receives the same
 * bits lix_indexer_logits writes there; a position outside holds -inf or
 * keeps its previous contents (the key blocks no query of a block of queries
 * sees are not written).  The buffer is otherwise the caller's, as above.
 */
int lix_indexer_logits_visible(const void* q, const void* k, const float* w,
                               int B, int S, int Skv, int H, int D, int compress_ratio,
                               const int32_t* ks, const int32_t* ke,
                               float* logits, hipStream_t stream);

/*
 * lix_topk - per-query top-k of the indexer scores.
 *
 * Page "...deepseek_v4.kernels.tilelang_indexer", sections v4_lighting_indexer
 * and V4IndexerFunction.forward with topk_indices = None (topk = number of
 * indices to select; [B,S,topk] fp32 scores; int32 indices).
 *
 * logits == NULL: fused path.  Scores are computed from q, k, w (layouts as
 *   in lix_indexer_logits) and selected on chip; no [B,S,Skv] tensor is
 *   written.  The candidates of every query of a workgroup live in LDS, which
 *   bounds the shapes (LIX_ERR_UNSUPPORTED otherwise; lix_topk_fused_supported
 *   answers for given sizes):
 *     heads >= 8 (a query's heads must fill a lane pair of the MFMA tile),
 *     Skv <= 65536 (key indices are held in 16 bits),
 *     topk <= LIX_FUSED_TOPK_MAX and topk <= the capacity for (heads,
 *     index_dim padded to 32/64/128/256):
 *         heads 8:   704 / 640 / 576 / 384
 *         heads 16: 1472 / 1408 / 1216 / 896
 *         heads 32: 2048 / 2048 / 2048 / 1856
 *         heads 64, 128: 2048.
 *   Selecting from materialized logits (lix_indexer_logits, then this call
 *   with logits != NULL) has none of these limits.
 * logits != NULL: selection from a caller-provided fp32 [B,S,Skv] tensor
 *   (for instance the output of lix_indexer_logits); q, k, w, H and D are
 *   ignored and may be NULL / 0.
 *
 * For each (b, t) with n = ke - ks visible keys, the m = min(topk, n) keys
 * with the largest scores are selected; equal scores are ordered by key
 * index, the lower index first.  They are written to slots [0, m) in
 * ascending key-index order; slots [m, topk) hold index -1 and score -inf.
 *
 *   scores   fp32  [B, S, topk]  out
 *   indices  int32 [B, S, topk]  out
 */
int lix_topk(const void* q, const void* k, const float* w, const float* logits,
             int B, int S, int Skv, int H, int D, int compress_ratio,
             const int32_t* ks, const int32_t* ke, int topk,
             float* scores, int32_t* indices, hipStream_t stream);

/*
 * lix_topk_fused_supported - whether lix_topk's fused path (logits == NULL)
 * accepts these sizes: 1 if so, 0 if it would return LIX_ERR_UNSUPPORTED or
 * LIX_ERR_SHAPE for them (limits listed at lix_topk).  Pure host function: no
 * HIP call, no pointer.
 */
int lix_topk_fused_supported(int Skv, int H, int D, int topk);

/*
 * lix_topk_streaming - per-query top-k of the indexer scores, selected block
 * by block as the scores are produced.
 *
 * Same selection, outputs and bits as lix_topk (page
 * "...deepseek_v4.kernels.tilelang_indexer", v4_lighting_indexer), from q,
 * k, w as in lix_indexer_logits, without the fused path's on-chip limits and
 * without writing the [B,S,Skv] logits: a persistent grid scores one query
 * block at a time into its own slot of `workspace` (the block's rows of Skv
 * fp32, written over each row's visible span only) and selects each of that
 * block's rows from the slot at once, while the rows are still in the L2
 * cache.  Every output equals lix_indexer_logits followed by lix_topk on the
 * logits, bit for bit.
 *
 *   q, k, w, ks, ke, compress_ratio  as in lix_indexer_logits
 *   topk       1 <= topk <= Skv
 *   scores     fp32  [B, S, topk]  out
 *   indices    int32 [B, S, topk]  out
 *   workspace  device memory owned by the caller, 256-byte aligned; its
 *              contents on entry do not matter and on return are
 *              unspecified.  lix_topk_streaming_workspace_bytes gives the
 *              size that keeps every resident workgroup busy; a smaller one
 *              (at least one block's rows) runs fewer workgroups, a smaller
 *              still is LIX_ERR_SHAPE.
 * Requires Skv <= 8192 (a row sits in registers while it is selected):
 * LIX_ERR_UNSUPPORTED otherwise.
 */
int lix_topk_streaming(const void* q, const void* k, const float* w,
                       int B, int S, int Skv, int H, int D, int compress_ratio,
                       const int32_t* ks, const int32_t* ke, int topk,
                       float* scores, int32_t* indices,
                       void* workspace, long long workspace_bytes, hipStream_t stream);

/*
 * lix_topk_streaming_workspace_bytes - workspace lix_topk_streaming uses at
 * full occupancy on the current device for these sizes: (workgroups resident
 * at once, at most one per query block) x (queries per block) x Skv x 4
 * bytes.  -1 when the sizes are outside what lix_topk_streaming accepts or
 * the device query fails.
 */
long long lix_topk_streaming_workspace_bytes(int B, int S, int Skv, int H, int D);

/*
 * lix_topk_scores - scores at given key indices.
 *
 * Page "...deepseek_v4.kernels.tilelang_indexer", section
 * pytorch_extract_topk_scores (gather along the last dimension) as used by
 * v4_lighting_indexer with precomputed topk_indices [B,S,topk] int32.
 *
 *   logits   fp32  [B, S, Skv]
 *   indices  int32 [B, S, topk]; an index outside [0, Skv) (such as the -1
 *            padding of lix_topk) yields -inf
 *   scores   fp32  [B, S, topk]  out
 */
int lix_topk_scores(const float* logits, const int32_t* indices,
                    int B, int S, int Skv, int topk, float* scores,
                    hipStream_t stream);

/*
 * lix_indexer_scores_at - indexer scores at given key indices, from q, k, w.
 *
 * Page "...deepseek_v4.kernels.tilelang_indexer", sections
 * v4_lighting_indexer with topk_indices given and
 * pytorch_extract_topk_scores: the scores of the given indices, i.e. the
 * cleaned logits gathered at them.  Only the given keys are scored; no
 * [B,S,Skv] tensor exists.  For i = indices[b,t,j]:
 *   scores[b,t,j] = sum_h w[t,b,h] * max(0, q[t,b,h,:] . k[i,b,:])  if ks[t] <= i < ke[t]
 *   scores[b,t,j] = -inf                                            otherwise
 * (ranges as for lix_indexer_logits; an index outside [0, Skv) is -inf).
 * Each score equals lix_indexer_logits' value at that position bit for bit.
 *
 *   q, k, w  as in lix_indexer_logits
 *   indices  int32 [B, S, topk]  (any values; duplicates allowed)
 *   scores   fp32  [B, S, topk]  out
 */
int lix_indexer_scores_at(const void* q, const void* k, const float* w, const int32_t* indices,
                          int B, int S, int Skv, int H, int D, int compress_ratio,
                          const int32_t* ks, const int32_t* ke, int topk,
                          float* scores, hipStream_t stream);

/*
 * lix_indexer_backward - gradients of the scores at given indices.
 *
 * Page "...deepseek_v4.kernels.tilelang_indexer", class V4IndexerFunction:
 * backward(grad_scores, grad_indices) of the forward above (the pages print
 * no formula; this is the chain rule on the forward definition).  For each
 * entry j of query (b, t) whose key i = indices[b,t,j] lies in [ks[t], ke[t])
 * (ranges as for lix_indexer_logits), with g = grad_scores[b,t,j],
 * d_h = q[t,b,h,:] . k[i,b,:] and m_h = 1 if d_h > 0 else 0:
 *     dw[t,b,h]   += g * max(0, d_h)
 *     dq[t,b,h,:] += g * w[t,b,h] * m_h * k[i,b,:]
 *     dk[i,b,:]   += g * sum_h w[t,b,h] * m_h * q[t,b,h,:]
 * Other entries contribute nothing (their score is the constant -inf,
 * whatever their grad_scores value); a key listed twice contributes twice;
 * the indices get no gradient.  Each term of a gradient product carries one
 * bf16 rounding, as a bf16 autograd graph of the forward would: the upstream
 * factor is rounded (g for dq, w applied in fp32 afterwards; the summed g of a
 * (query, key) pair times w_h for dk) and multiplies the exact bf16 k or q;
 * the products accumulate in fp32.  The ReLU masks m_h come from one
 * recompute of d per entry and serve dq, dw and dk alike.  dk is a sum over
 * queries computed key-major (one partial per 256 keys and 128 queries, added
 * with fp32 atomics; a key listed more than once in a row has its g summed
 * with LDS atomics first), so its low bits may vary from run to run; dq and
 * dw are deterministic.
 *
 *   q, k, w      as in lix_indexer_logits; heads H <= 64, 32 < D <= 128, Skv <= 32768
 *   indices      int32 [B, S, topk]  (any values)
 *   grad_scores  fp32  [B, S, topk]
 *   dq           fp32  [S, B, H, D]    out (every element written)
 *   dk           fp32  [Skv, B, D]     out (cleared by the call, 16-byte aligned)
 *   dw           fp32  [S, B, H]       out (every element written)
 *   workspace    device memory of at least lix_indexer_backward_workspace_bytes
 *                (for the same topk) bytes, 256-byte aligned, owned by the
 *                caller; its contents on
 *                entry do not matter and on return are unspecified.  A smaller
 *                workspace_bytes: LIX_ERR_SHAPE.
 * Other H, D or Skv: LIX_ERR_UNSUPPORTED.
 */
int lix_indexer_backward(const void* q, const void* k, const float* w, const int32_t* indices,
                         const float* grad_scores, int B, int S, int Skv, int H, int D,
                         int compress_ratio, const int32_t* ks, const int32_t* ke, int topk,
                         float* dq, float* dk, float* dw, void* workspace, long long workspace_bytes,
                         hipStream_t stream);

/*
 * lix_indexer_backward_workspace_bytes - device workspace lix_indexer_backward
 * needs for these sizes: the ReLU masks of every entry (B*S*topk*4 bytes per
 * 32 heads), the bucket bounds (B*S*(Skv/64 + 1)*4 bytes) and the entries
 * bucketed by groups of 64 keys (B*S*topk*16 bytes), each part rounded up to
 * 256 bytes: linear in topk and in Skv/64, with no [B, S, Skv] term and no
 * copy of q, k or w.  -1 when the sizes are outside what lix_indexer_backward
 * accepts.
 */
long long lix_indexer_backward_workspace_bytes(int B, int S, int Skv, int H, int D, int topk);

/*
 * lix_indexer_backward_noalloc - lix_indexer_backward without a workspace
 * argument and without any allocation.
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving or training loops, harnesses that
 * forbid hipMalloc.  Same arguments, semantics, outputs and errors as
 * lix_indexer_backward, minus workspace / workspace_bytes: the workspace is a
 * static device array of LIX_NOALLOC_SCRATCH_BYTES bytes that each GPU the
 * library runs on holds until the process ends (its device address is looked
 * up once per device).  Sizes whose workspace
 * (lix_indexer_backward_workspace_bytes) exceeds LIX_NOALLOC_SCRATCH_BYTES:
 * LIX_ERR_UNSUPPORTED.  The call allocates nothing and frees nothing.  Every
 * call on one GPU uses the same array and leaves its contents behind (nothing
 * in it needs to start at zero): calls that overlap on one GPU (concurrent
 * streams or threads) race and are not allowed; calls ordered on one stream
 * are fine.
 */
#define LIX_NOALLOC_SCRATCH_BYTES (64L << 20)
int lix_indexer_backward_noalloc(const void* q, const void* k, const float* w, const int32_t* indices,
                                 const float* grad_scores, int B, int S, int Skv, int H, int D,
                                 int compress_ratio, const int32_t* ks, const int32_t* ke, int topk,
                                 float* dq, float* dk, float* dw, hipStream_t stream);

/*
 * lix_indexer_scores_v41 - V4.1 BF16-rounded scores with a visibility mask.
 *
 * Page "...deepseek_v41.indexer", module description (the GEMM output and
 * each weighted head score are rounded to BF16 before the FP32 head
 * reduction) and section indexer_scores (BSHD inputs, boolean `allowed`,
 * BF16 scores; heads a power of two <= 128; index_dim a multiple of 16).
 * Rounding is round-to-nearest-even.  For every visible (t, s):
 *     out = bf16( sum_h bf16( w_h * max(0, bf16(q_h . k_s)) ) )
 * with the sum in fp32; hidden positions hold bf16 -inf (0xFF80).
 *
 *   queries  bf16 [B, L, H, D]
 *   keys     bf16 [B, G, D]
 *   weights  bf16 [B, L, H]
 *   allowed  uint8 [B, L, G], 0 = hidden, nonzero = visible
 *   scores   bf16 [B, L, G]  out
 */
int lix_indexer_scores_v41(const void* queries, const void* keys, const void* weights,
                           const uint8_t* allowed, int B, int L, int G, int H, int D,
                           void* scores, hipStream_t stream);

/*
 * lix_topk_bf16 - per-query top-k of V4.1 bf16 scores over the visible keys.
 *
 * Page "...deepseek_v41.indexer", module description: the scores of
 * indexer_scores feed a top-k / candidate selection that runs after it; the
 * selection rule is V4's (page "...deepseek_v4.kernels.tilelang_indexer",
 * v4_lighting_indexer: select topk indices per query).  A key is visible when
 * its score is not bf16 -inf (0xFF80, the value indexer_scores writes where
 * `allowed` is false).  For each (b, t) the m = min(topk, visible keys) best
 * visible keys are selected by score, descending, equal scores by key index,
 * the lower first; they are written to slots [0, m) in ascending key-index
 * order with their scores copied bit for bit; slots [m, topk) hold index -1
 * and score bf16 -inf.
 *
 *   scores      bf16  [B, L, G]     (e.g. the output of lix_indexer_scores_v41)
 *   out_scores  bf16  [B, L, topk]  out
 *   indices     int32 [B, L, topk]  out
 * Requires 1 <= topk <= G and G <= 8192 (LIX_ERR_SHAPE / LIX_ERR_UNSUPPORTED).
 */
int lix_topk_bf16(const void* scores, int B, int L, int G, int topk,
                  void* out_scores, int32_t* indices, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIX_H */

// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments have been validated by the caller; launchers only enqueue.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "tiling.h"

namespace lix {

struct LogitsArgs {
    const void* q;
    const void* k;
    const float* w;
    int B, S, Skv, H, D, ratio;
    const int32_t* ks;
    const int32_t* ke;
    float* logits;
    hipStream_t stream;
    int fill;                 // 1: -inf at every position outside the ranges; 0: those not all written
};

struct TopkArgs {
    const float* logits;   // [B,S,Skv]
    int B, S, Skv, ratio, topk;
    const int32_t* ks;
    const int32_t* ke;
    float* scores;
    int32_t* indices;
    hipStream_t stream;
};

struct FusedArgs {
    const void* q;
    const void* k;
    const float* w;
    int B, S, Skv, H, D, ratio, topk;
    const int32_t* ks;
    const int32_t* ke;
    float* scores;
    int32_t* indices;
    hipStream_t stream;
};

struct TopkBf16Args {
    const void* scores;       // bf16 [B,L,G]; bf16 -inf marks a hidden key
    int B, L, G, topk;
    void* out_scores;         // bf16 [B,L,topk]
    int32_t* indices;         // int32 [B,L,topk]
    hipStream_t stream;
};

struct GatherArgs {
    const float* logits;
    const int32_t* indices;
    int B, S, Skv, topk;
    float* scores;
    hipStream_t stream;
};

struct V41Args {
    const void* queries;
    const void* keys;
    const void* weights;
    const uint8_t* allowed;
    int B, L, G, H, D;
    void* scores;
    hipStream_t stream;
};

struct SparseArgs {
    const void* q;
    const void* k;
    const float* w;
    const int32_t* indices;   // [B,S,topk]
    int B, S, Skv, H, D, ratio, topk;
    const int32_t* ks;
    const int32_t* ke;
    float* scores;            // [B,S,topk]
    hipStream_t stream;
};

hipError_t launch_v4_logits(const LogitsArgs& p);

// Scoring with the top-k selected right after each query block is scored
// (lix_topk_streaming): a persistent grid, each workgroup owning one slot of
// the workspace (streaming_slot_bytes) for the rows of its current block.
struct StreamArgs {
    const void* q;
    const void* k;
    const float* w;
    int B, S, Skv, H, D, ratio, topk;
    const int32_t* ks;
    const int32_t* ke;
    float* workspace;         // workspace_bytes / streaming_slot_bytes slots (at least one)
    long workspace_bytes;
    float* scores;            // [B,S,topk]
    int32_t* indices;         // [B,S,topk]
    hipStream_t stream;
};
constexpr int kStreamMaxSkv = 8192;   // a row of the block in registers during its selection
// Bytes of one slot: the scores of one query block (QB rows of Skv fp32).
long streaming_slot_bytes(int H, int D, int Skv);
// Workgroups of the persistent grid on the current device: min(query blocks,
// resident workgroups).
hipError_t streaming_grid(int B, int S, int H, int D, long* grid);
hipError_t launch_topk_streaming(const StreamArgs& p);
hipError_t launch_sparse_scores(const SparseArgs& p);

// Gradients of the scores at given indices (dk is cleared, then accumulated).
struct BackwardArgs {
    const void* q;
    const void* k;
    const float* w;
    const int32_t* indices;   // [B,S,topk]
    const float* grad;        // [B,S,topk]
    int B, S, Skv, H, D, ratio, topk;
    const int32_t* ks;
    const int32_t* ke;
    float* dq;                // [S,B,H,D]
    float* dk;                // [Skv,B,D]
    float* dw;                // [S,B,H]
    void* workspace;          // backward_workspace_bytes(B, S, Skv, H, D, topk) bytes
    hipStream_t stream;
};
// Workspace of the backward, byte offsets of its parts (each 256-byte
// aligned): the rows kernel's ReLU masks ([B,S] x ceil(H/32) x topk uint32);
// bucket bounds ([B,S] x (ceil(Skv/64) + 1) int32); the entries bucketed by
// 64-key group ([B,S,topk] x 16 bytes).  O(B S (topk + Skv/64)).
struct BackwardLayout {
    long masks, off, ent, total;
};
BackwardLayout backward_layout(int B, int S, int Skv, int H, int D, int topk);
long backward_workspace_bytes(int B, int S, int Skv, int H, int D, int topk);
hipError_t launch_indexer_backward(const BackwardArgs& p);
// Device address and size of the current device's static backward workspace
// (lix_indexer_backward_noalloc); taken with hipGetSymbolAddress once per device.
hipError_t noalloc_workspace(void** ptr, long* bytes);
hipError_t launch_topk_rows(const TopkArgs& p);
hipError_t launch_topk_bf16(const TopkBf16Args& p);
hipError_t launch_fused_topk(const FusedArgs& p);
hipError_t launch_gather(const GatherArgs& p);
hipError_t launch_v41_scores(const V41Args& p);

// Nonzero when the fused kernel can hold topk candidates per query on chip
// for this head count and index_dim (limits.cpp).
int fused_supported(int H, int D, int topk);
// Candidate capacity per query the fused kernel uses (tiling.h, fused_cap).
long fused_capacity(int H, int D, int topk);

}  // namespace lix

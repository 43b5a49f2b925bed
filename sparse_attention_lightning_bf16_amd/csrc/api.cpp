// C ABI of liblix: argument validation and kernel dispatch.
//
// Validation happens on the host before any HIP call: a failing call returns
// a negative status, enqueues nothing and writes no output.  The only HIP
// calls made before a launch are the pointer-attribute queries of the
// device check.
#include <stdint.h>

#include <initializer_list>

#include <hip/hip_runtime_api.h>

#include "lix.h"
#include "launch.h"

namespace {

constexpr int kVersion = 100;   // 0.1.0

bool is_pow2_le128(int h) { return h >= 1 && h <= 128 && (h & (h - 1)) == 0; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Element counts must stay far inside int64 and the kernels' 32-bit grid limits.
bool fits(long long a, long long b, long long c = 1, long long d = 1) {
    const long long lim = 1LL << 40;
    long long x = a;
    for (long long f : {b, c, d}) {
        if (f <= 0 || x > lim / f) return false;
        x *= f;
    }
    return true;
}

// One workgroup per row or per query block: the row count must fit a 1-D grid.
bool rows_fit(int B, int S) { return (long long)B * S <= (1LL << 30); }

// The key-stage loads form key-row offsets as 24-bit products of a row
// (< 128) and the key row stride B * index_dim: that stride must stay below 2^24.
bool key_stride_fits(int B, int D) { return (long long)B * D < (1LL << 24); }

int check_dims_v4(int B, int S, int Skv, int H, int D, int ratio, const int32_t* ks, const int32_t* ke) {
    if (B <= 0 || S <= 0 || Skv <= 0 || H <= 0 || D <= 0 || ratio < 1) return LIX_ERR_SHAPE;
    if ((ks == nullptr) != (ke == nullptr)) return LIX_ERR_SHAPE;
    if (!is_pow2_le128(H) || D % 16 != 0 || D > 256) return LIX_ERR_UNSUPPORTED;
    if (!fits(S, B, H, D) || !fits(B, S, Skv) || !fits(Skv, B, D) || !rows_fit(B, S)) return LIX_ERR_UNSUPPORTED;
    if (!key_stride_fits(B, D)) return LIX_ERR_UNSUPPORTED;
    return LIX_OK;
}

// Sizes the fused top-k kernel accepts (beyond check_dims_v4).
bool fused_fits(int Skv, int H, int D, int topk) {
    return topk >= 1 && topk <= LIX_FUSED_TOPK_MAX && Skv <= lix::kFusedMaxSkv && lix::fused_supported(H, D, topk);
}

// Every pointer must be device (or managed) memory of the current device.
int check_device(std::initializer_list<const void*> ptrs) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LIX_ERR_DEVICE;
    for (const void* p : ptrs) {
        if (p == nullptr) continue;
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
            (void)hipGetLastError();
            return LIX_ERR_DEVICE;
        }
        if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return LIX_ERR_DEVICE;
        if (attr.device != dev) return LIX_ERR_DEVICE;
    }
    return LIX_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? LIX_OK : LIX_ERR_LAUNCH; }

// The backward's limits: heads <= 64, 32 < index_dim <= 128, a key row of G in LDS.
int check_dims_backward(int B, int S, int Skv, int H, int D, int ratio, const int32_t* ks, const int32_t* ke,
                        int topk) {
    int st = check_dims_v4(B, S, Skv, H, D, ratio, ks, ke);
    if (st != LIX_OK) return st;
    if (topk < 1) return LIX_ERR_SHAPE;
    if (H > 64 || D <= 32 || D > 128 || Skv > 32768) return LIX_ERR_UNSUPPORTED;
    if (!fits(B, S, topk) || (long long)B * S * topk > (1LL << 38)) return LIX_ERR_UNSUPPORTED;
    if ((long long)B * S > (1LL << 30) - 1) return LIX_ERR_UNSUPPORTED;
    return LIX_OK;
}

}  // namespace

extern "C" {

const char* lix_status_string(int status) {
    switch (status) {
        case LIX_OK: return "LIX_OK";
        case LIX_ERR_NULL: return "LIX_ERR_NULL: a required pointer is NULL";
        case LIX_ERR_SHAPE: return "LIX_ERR_SHAPE: invalid size, topk, compress_ratio or ks/ke pairing";
        case LIX_ERR_UNSUPPORTED:
            return "LIX_ERR_UNSUPPORTED: heads/index_dim/alignment/size/topk outside what the kernels support";
        case LIX_ERR_DEVICE: return "LIX_ERR_DEVICE: a pointer is not device memory of the current device";
        case LIX_ERR_LAUNCH: return "LIX_ERR_LAUNCH: kernel launch failed";
        default: return "LIX_ERR_UNKNOWN";
    }
}

int lix_version(void) { return kVersion; }

namespace {

int indexer_logits(const void* q, const void* k, const float* w, int B, int S, int Skv, int H, int D,
                   int compress_ratio, const int32_t* ks, const int32_t* ke, float* logits, hipStream_t stream,
                   int fill) {
    if (!q || !k || !w || !logits) return LIX_ERR_NULL;
    int st = check_dims_v4(B, S, Skv, H, D, compress_ratio, ks, ke);
    if (st != LIX_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(logits, 4) || !aligned(ks, 4) ||
        !aligned(ke, 4))
        return LIX_ERR_UNSUPPORTED;
    st = check_device({q, k, w, logits, ks, ke});
    if (st != LIX_OK) return st;
    lix::LogitsArgs a{q, k, w, B, S, Skv, H, D, compress_ratio, ks, ke, logits, stream, fill};
    return launch_status(lix::launch_v4_logits(a));
}

}  // namespace

int lix_indexer_logits(const void* q, const void* k, const float* w, int B, int S, int Skv, int H, int D,
                       int compress_ratio, const int32_t* ks, const int32_t* ke, float* logits,
                       hipStream_t stream) {
    return indexer_logits(q, k, w, B, S, Skv, H, D, compress_ratio, ks, ke, logits, stream, 1);
}

int lix_indexer_logits_visible(const void* q, const void* k, const float* w, int B, int S, int Skv, int H, int D,
                               int compress_ratio, const int32_t* ks, const int32_t* ke, float* logits,
                               hipStream_t stream) {
    return indexer_logits(q, k, w, B, S, Skv, H, D, compress_ratio, ks, ke, logits, stream, 0);
}

int lix_topk(const void* q, const void* k, const float* w, const float* logits, int B, int S, int Skv, int H,
             int D, int compress_ratio, const int32_t* ks, const int32_t* ke, int topk, float* scores,
             int32_t* indices, hipStream_t stream) {
    if (!scores || !indices) return LIX_ERR_NULL;
    if (logits == nullptr && (!q || !k || !w)) return LIX_ERR_NULL;
    if (B <= 0 || S <= 0 || Skv <= 0 || compress_ratio < 1) return LIX_ERR_SHAPE;
    if ((ks == nullptr) != (ke == nullptr)) return LIX_ERR_SHAPE;
    if (topk < 1 || topk > Skv) return LIX_ERR_SHAPE;
    if (!fits(B, S, Skv) || !fits(B, S, topk) || !rows_fit(B, S)) return LIX_ERR_UNSUPPORTED;
    if (!aligned(scores, 4) || !aligned(indices, 4) || !aligned(ks, 4) || !aligned(ke, 4) || !aligned(logits, 4))
        return LIX_ERR_UNSUPPORTED;
    if (logits != nullptr) {
        int st = check_device({logits, ks, ke, scores, indices});
        if (st != LIX_OK) return st;
        lix::TopkArgs a{logits, B, S, Skv, compress_ratio, topk, ks, ke, scores, indices, stream};
        return launch_status(lix::launch_topk_rows(a));
    }
    int st = check_dims_v4(B, S, Skv, H, D, compress_ratio, ks, ke);
    if (st != LIX_OK) return st;
    if (!fused_fits(Skv, H, D, topk)) return LIX_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4)) return LIX_ERR_UNSUPPORTED;
    st = check_device({q, k, w, ks, ke, scores, indices});
    if (st != LIX_OK) return st;
    lix::FusedArgs a{q, k, w, B, S, Skv, H, D, compress_ratio, topk, ks, ke, scores, indices, stream};
    return launch_status(lix::launch_fused_topk(a));
}

int lix_topk_fused_supported(int Skv, int H, int D, int topk) {
    if (Skv <= 0 || H <= 0 || D <= 0 || topk < 1 || topk > Skv) return 0;
    if (!is_pow2_le128(H) || D % 16 != 0 || D > 256) return 0;
    return fused_fits(Skv, H, D, topk) ? 1 : 0;
}

long long lix_topk_streaming_workspace_bytes(int B, int S, int Skv, int H, int D) {
    if (check_dims_v4(B, S, Skv, H, D, 1, nullptr, nullptr) != LIX_OK) return -1;
    if (Skv > lix::kStreamMaxSkv) return -1;
    long grid = 0;
    if (lix::streaming_grid(B, S, H, D, &grid) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (long long)grid * lix::streaming_slot_bytes(H, D, Skv);
}

int lix_topk_streaming(const void* q, const void* k, const float* w, int B, int S, int Skv, int H, int D,
                       int compress_ratio, const int32_t* ks, const int32_t* ke, int topk, float* scores,
                       int32_t* indices, void* workspace, long long workspace_bytes, hipStream_t stream) {
    if (!q || !k || !w || !scores || !indices || !workspace) return LIX_ERR_NULL;
    int st = check_dims_v4(B, S, Skv, H, D, compress_ratio, ks, ke);
    if (st != LIX_OK) return st;
    if (topk < 1 || topk > Skv) return LIX_ERR_SHAPE;
    if (Skv > lix::kStreamMaxSkv || !fits(B, S, topk)) return LIX_ERR_UNSUPPORTED;
    if (workspace_bytes < lix::streaming_slot_bytes(H, D, Skv)) return LIX_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(scores, 4) || !aligned(indices, 4) ||
        !aligned(ks, 4) || !aligned(ke, 4) || !aligned(workspace, 256))
        return LIX_ERR_UNSUPPORTED;
    st = check_device({q, k, w, ks, ke, scores, indices, workspace});
    if (st != LIX_OK) return st;
    lix::StreamArgs a{q, k, w, B, S, Skv, H, D, compress_ratio, topk, ks, ke, static_cast<float*>(workspace),
                      (long)workspace_bytes, scores, indices, stream};
    return launch_status(lix::launch_topk_streaming(a));
}

int lix_topk_scores(const float* logits, const int32_t* indices, int B, int S, int Skv, int topk, float* scores,
                    hipStream_t stream) {
    if (!logits || !indices || !scores) return LIX_ERR_NULL;
    if (B <= 0 || S <= 0 || Skv <= 0 || topk < 1) return LIX_ERR_SHAPE;
    if (!fits(B, S, Skv) || !fits(B, S, topk) || (long long)B * S * topk > (1LL << 38)) return LIX_ERR_UNSUPPORTED;
    if (!aligned(logits, 4) || !aligned(indices, 4) || !aligned(scores, 4)) return LIX_ERR_UNSUPPORTED;
    int st = check_device({logits, indices, scores});
    if (st != LIX_OK) return st;
    lix::GatherArgs a{logits, indices, B, S, Skv, topk, scores, stream};
    return launch_status(lix::launch_gather(a));
}

int lix_indexer_scores_at(const void* q, const void* k, const float* w, const int32_t* indices, int B, int S,
                          int Skv, int H, int D, int compress_ratio, const int32_t* ks, const int32_t* ke, int topk,
                          float* scores, hipStream_t stream) {
    if (!q || !k || !w || !indices || !scores) return LIX_ERR_NULL;
    int st = check_dims_v4(B, S, Skv, H, D, compress_ratio, ks, ke);
    if (st != LIX_OK) return st;
    if (topk < 1) return LIX_ERR_SHAPE;
    if (!fits(B, S, topk) || (long long)B * S * topk > (1LL << 38)) return LIX_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(indices, 4) || !aligned(scores, 4) ||
        !aligned(ks, 4) || !aligned(ke, 4))
        return LIX_ERR_UNSUPPORTED;
    st = check_device({q, k, w, indices, scores, ks, ke});
    if (st != LIX_OK) return st;
    lix::SparseArgs a{q, k, w, indices, B, S, Skv, H, D, compress_ratio, topk, ks, ke, scores, stream};
    return launch_status(lix::launch_sparse_scores(a));
}

long long lix_indexer_backward_workspace_bytes(int B, int S, int Skv, int H, int D, int topk) {
    if (check_dims_backward(B, S, Skv, H, D, 1, nullptr, nullptr, topk) != LIX_OK) return -1;
    return lix::backward_workspace_bytes(B, S, Skv, H, D, topk);
}

int lix_indexer_backward(const void* q, const void* k, const float* w, const int32_t* indices,
                         const float* grad_scores, int B, int S, int Skv, int H, int D, int compress_ratio,
                         const int32_t* ks, const int32_t* ke, int topk, float* dq, float* dk, float* dw,
                         void* workspace, long long workspace_bytes, hipStream_t stream) {
    if (!q || !k || !w || !indices || !grad_scores || !dq || !dk || !dw || !workspace) return LIX_ERR_NULL;
    int st = check_dims_backward(B, S, Skv, H, D, compress_ratio, ks, ke, topk);
    if (st != LIX_OK) return st;
    if (workspace_bytes < lix::backward_workspace_bytes(B, S, Skv, H, D, topk)) return LIX_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(indices, 4) || !aligned(grad_scores, 4) ||
        !aligned(dq, 4) || !aligned(dk, 16) || !aligned(dw, 4) || !aligned(ks, 4) || !aligned(ke, 4) ||
        !aligned(workspace, 256))
        return LIX_ERR_UNSUPPORTED;
    st = check_device({q, k, w, indices, grad_scores, dq, dk, dw, ks, ke, workspace});
    if (st != LIX_OK) return st;
    lix::BackwardArgs a{q, k, w, indices, grad_scores, B, S, Skv, H, D, compress_ratio, topk, ks, ke, dq, dk, dw,
                        workspace, stream};
    return launch_status(lix::launch_indexer_backward(a));
}

int lix_indexer_backward_noalloc(const void* q, const void* k, const float* w, const int32_t* indices,
                                 const float* grad_scores, int B, int S, int Skv, int H, int D, int compress_ratio,
                                 const int32_t* ks, const int32_t* ke, int topk, float* dq, float* dk, float* dw,
                                 hipStream_t stream) {
    if (!q || !k || !w || !indices || !grad_scores || !dq || !dk || !dw) return LIX_ERR_NULL;
    int st = check_dims_backward(B, S, Skv, H, D, compress_ratio, ks, ke, topk);
    if (st != LIX_OK) return st;
    if (lix::backward_workspace_bytes(B, S, Skv, H, D, topk) > (long)LIX_NOALLOC_SCRATCH_BYTES)
        return LIX_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(indices, 4) || !aligned(grad_scores, 4) ||
        !aligned(dq, 4) || !aligned(dk, 16) || !aligned(dw, 4) || !aligned(ks, 4) || !aligned(ke, 4))
        return LIX_ERR_UNSUPPORTED;
    st = check_device({q, k, w, indices, grad_scores, dq, dk, dw, ks, ke});
    if (st != LIX_OK) return st;
    void* ws = nullptr;
    long ws_bytes = 0;
    if (lix::noalloc_workspace(&ws, &ws_bytes) != hipSuccess) return LIX_ERR_DEVICE;
    lix::BackwardArgs a{q, k, w, indices, grad_scores, B, S, Skv, H, D, compress_ratio, topk, ks, ke, dq, dk, dw,
                        ws, stream};
    return launch_status(lix::launch_indexer_backward(a));
}

int lix_topk_bf16(const void* scores, int B, int L, int G, int topk, void* out_scores, int32_t* indices,
                  hipStream_t stream) {
    if (!scores || !out_scores || !indices) return LIX_ERR_NULL;
    if (B <= 0 || L <= 0 || G <= 0 || topk < 1 || topk > G) return LIX_ERR_SHAPE;
    if (G > 8192 || !fits(B, L, G) || !fits(B, L, topk) || !rows_fit(B, L)) return LIX_ERR_UNSUPPORTED;
    if (!aligned(scores, 2) || !aligned(out_scores, 2) || !aligned(indices, 4)) return LIX_ERR_UNSUPPORTED;
    int st = check_device({scores, out_scores, indices});
    if (st != LIX_OK) return st;
    lix::TopkBf16Args a{scores, B, L, G, topk, out_scores, indices, stream};
    return launch_status(lix::launch_topk_bf16(a));
}

int lix_indexer_scores_v41(const void* queries, const void* keys, const void* weights, const uint8_t* allowed,
                           int B, int L, int G, int H, int D, void* scores, hipStream_t stream) {
    if (!queries || !keys || !weights || !allowed || !scores) return LIX_ERR_NULL;
    if (B <= 0 || L <= 0 || G <= 0 || H <= 0 || D <= 0) return LIX_ERR_SHAPE;
    if (!is_pow2_le128(H) || D % 16 != 0 || D > 256) return LIX_ERR_UNSUPPORTED;
    if (!fits(B, L, H, D) || !fits(B, L, G) || !fits(B, G, D) || !rows_fit(B, L)) return LIX_ERR_UNSUPPORTED;
    if (!aligned(queries, 16) || !aligned(keys, 16) || !aligned(weights, 2) || !aligned(scores, 2))
        return LIX_ERR_UNSUPPORTED;
    int st = check_device({queries, keys, weights, allowed, scores});
    if (st != LIX_OK) return st;
    lix::V41Args a{queries, keys, weights, allowed, B, L, G, H, D, scores, stream};
    return launch_status(lix::launch_v41_scores(a));
}

}  // extern "C"

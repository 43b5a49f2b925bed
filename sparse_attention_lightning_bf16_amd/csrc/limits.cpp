// Host-side size limits of the kernels: which shapes the fused top-k keeps
// on chip, and how much workspace the backward needs.  Plain C++ over the
// constants of tiling.h (no HIP types), shared by the C ABI's validation and
// the launchers.
#include "launch.h"

namespace lix {

namespace {

template <int H>
long fused_cap_dp(int D, int topk) {
    switch (padded_dim(D)) {
        case 32: return fused_cap<H, 32>(topk);
        case 64: return fused_cap<H, 64>(topk);
        case 128: return fused_cap<H, 128>(topk);
        case 256: return fused_cap<H, 256>(topk);
        default: return -1;
    }
}

}  // namespace

long fused_capacity(int H, int D, int topk) {
    if (topk < 1 || D < 1 || D > 256) return -1;
    switch (H) {
        case 8: return fused_cap_dp<8>(D, topk);
        case 16: return fused_cap_dp<16>(D, topk);
        case 32: return fused_cap_dp<32>(D, topk);
        case 64: return fused_cap_dp<64>(D, topk);
        case 128: return fused_cap_dp<128>(D, topk);
        default: return -1;   // the fused kernel keeps each query inside one lane pair: H >= 8
    }
}

int fused_supported(int H, int D, int topk) { return fused_capacity(H, D, topk) > 0; }

long streaming_slot_bytes(int H, int D, int Skv) {
    int qb = 0;
    switch (H) {
        case 1: qb = Tiling<1, 64>::QB; break;
        case 2: qb = Tiling<2, 64>::QB; break;
        case 4: qb = Tiling<4, 64>::QB; break;
        case 8: qb = Tiling<8, 64>::QB; break;
        case 16: qb = Tiling<16, 64>::QB; break;
        case 32: qb = Tiling<32, 64>::QB; break;
        case 64: qb = Tiling<64, 64>::QB; break;
        case 128: qb = Tiling<128, 64>::QB; break;
        default: return -1;
    }
    (void)D;   // queries per workgroup do not depend on index_dim
    return (long)qb * Skv * 4;
}

BackwardLayout backward_layout(int B, int S, int Skv, int H, int D, int topk) {
    auto up = [](long x) { return (x + 255) & ~255L; };
    (void)D;   // q is read in place
    const int nhg = H > 32 ? H / 32 : 1;
    const long rows = (long)B * S;
    BackwardLayout ly{};
    ly.masks = 0;
    ly.off = ly.masks + up(rows * topk * nhg * 4);
    ly.ent = ly.off + up(rows * ((Skv + 63) / 64 + 1) * 4);
    ly.total = ly.ent + up(rows * topk * 16);
    return ly;
}

long backward_workspace_bytes(int B, int S, int Skv, int H, int D, int topk) {
    return backward_layout(B, S, Skv, H, D, topk).total;
}

}  // namespace lix

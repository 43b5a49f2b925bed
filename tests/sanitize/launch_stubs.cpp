// Stand-ins for the kernel launchers of liblix, for the host-only sanitizer
// build of the C ABI (api.cpp + limits.cpp built by g++ with AddressSanitizer
// and UndefinedBehaviorSanitizer).  The driver only makes calls that fail
// validation or the device check, so none of these may ever run: each one
// aborts, which the driver reports as a failure.
#include <cstdio>
#include <cstdlib>

#include "launch.h"

namespace lix {

static hipError_t reached(const char* name) {
    std::fprintf(stderr, "launcher %s reached from the sanitizer driver\n", name);
    std::abort();
}

hipError_t launch_v4_logits(const LogitsArgs&) { return reached("launch_v4_logits"); }
hipError_t launch_sparse_scores(const SparseArgs&) { return reached("launch_sparse_scores"); }
hipError_t launch_indexer_backward(const BackwardArgs&) { return reached("launch_indexer_backward"); }
hipError_t launch_topk_rows(const TopkArgs&) { return reached("launch_topk_rows"); }
hipError_t launch_topk_bf16(const TopkBf16Args&) { return reached("launch_topk_bf16"); }
hipError_t launch_fused_topk(const FusedArgs&) { return reached("launch_fused_topk"); }
hipError_t launch_gather(const GatherArgs&) { return reached("launch_gather"); }
hipError_t launch_v41_scores(const V41Args&) { return reached("launch_v41_scores"); }
hipError_t noalloc_workspace(void**, long*) { return reached("noalloc_workspace"); }
hipError_t launch_topk_streaming(const StreamArgs&) { return reached("launch_topk_streaming"); }
hipError_t streaming_grid(int, int, int, int, long*) { return reached("streaming_grid"); }

}  // namespace lix

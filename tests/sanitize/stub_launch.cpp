// Launchers for the host-only sanitizer build of the C-ABI layer: a validation
// check must return before any launch, so reaching one of these is a failure.
#include <cstdio>
#include <cstdlib>

#include "kvc_launch.h"

namespace kvc {

static hipError_t reached(const char* what) {
  std::fprintf(stderr, "sanitizer driver: %s reached a launch\n", what);
  std::abort();
}

hipError_t launch_window_scores(const WsArgs&, const WsPlan&, hipStream_t) { return reached("window scores"); }
hipError_t noalloc_scratch(void**) { return reached("no-alloc scratch"); }
hipError_t launch_channel_scores(const CsArgs&, const CsPlan&, hipStream_t) { return reached("channel scores"); }
hipError_t launch_topk(const float*, int, int, int, int, int32_t*, void*, hipStream_t) { return reached("top-k"); }
hipError_t launch_gather(const GatherArgs&, hipStream_t) { return reached("gather"); }
hipError_t launch_chan_rows(const ChanRowsArgs&, hipStream_t) { return reached("channel rows"); }
hipError_t launch_scissor(const ScissorArgs&, hipStream_t) { return reached("scissor update"); }
hipError_t launch_scissor_refill(const ScissorRefillArgs&, hipStream_t) { return reached("scissor refill"); }
hipError_t launch_scissor_insert(const ScissorInsertArgs&, hipStream_t) { return reached("scissor insert"); }

}  // namespace kvc

// Host-only stand-ins for the gfx950 kernel launchers of libfluxattn, so that the
// C ABI's argument validation, workspace sizing and dispatch (csrc/api.cpp) can be
// built and run on a CPU with the host sanitizers.  Each stub records that it was
// reached and launches nothing.  Test infrastructure.
#include <hip/hip_runtime_api.h>

#include "fa_launch.h"

int g_launches = 0;

extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }

namespace fa {
hipError_t launch_router(const RouterArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_block_plan(const PlanArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_noalloc(DecodeArgs, size_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_kv_compact(const CompactArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_xa_scores(const XaScoreArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_xa_select(const XaSelectArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace fa

// Stand-ins for the library's device side, for the host-only build of the
// C-ABI code under the address and undefined-behaviour sanitizers: every
// launcher records that it was reached and returns an error, so a call that
// passes validation ends with KDN_ERR_HIP and nothing runs.  Only the
// validation, aliasing and workspace-planning code is exercised.
#include <hip/hip_runtime.h>

#include "kdn_internal.h"
#include "kdn_ops.h"

int g_launches = 0;

static hipError_t reached()
{
    ++g_launches;
    return hipErrorNotSupported;
}

extern "C" const char* hipGetErrorString(hipError_t) { return "launch stand-in"; }

namespace kdn {
hipError_t launch_walk_fwd(const FwdArgs&, bool, hipStream_t) { return reached(); }
hipError_t launch_chunk_fwd_f32(const FwdArgs&, bool, hipStream_t) { return reached(); }
hipError_t launch_step(const StepArgs&, bool, int, hipStream_t) { return reached(); }
hipError_t launch_dense_fwd(const DenseArgs&, int, hipStream_t) { return reached(); }
hipError_t launch_gain_scan(const GainArgs&, bool, int, hipStream_t) { return reached(); }
hipError_t launch_bwd(const BwdArgs&, bool, int, hipStream_t) { return reached(); }
hipError_t launch_gate_prologue(const PrologueArgs&, int, hipStream_t) { return reached(); }
hipError_t launch_gate_epilogue(const PrologueArgs&, float*, float*, float*, int, hipStream_t)
{
    return reached();
}
hipError_t launch_seqpar_fwd(const FwdArgs&, bool, int, float*, hipStream_t) { return reached(); }
hipError_t gain_static_scratch(float** ptr)
{
    static float dummy[4];
    *ptr = dummy;
    return hipSuccess;
}
}  // namespace kdn

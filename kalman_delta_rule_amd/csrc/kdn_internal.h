// kdn_internal.h -- argument blocks and launchers shared by the host API and
// the kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kdn {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* omega;
    const float* r;
    const float* S0;    // nullable
    const float* var0;  // nullable
    void* o;
    float* S_T;
    float* var_T;
    int B, T, H, dk, dv;
    float mu;
    const float* mu_h;  // nullable [H]: per-head information scale (overrides mu)
    const float* c0;    // nullable [H]: initial variance of every channel of a head when var0 is null
    float* beta;        // nullable [B,T,H]: effective write strength z / (r + z)
    bool split = false; // bf16 Diagonal walk: split-bf16 products (three per contraction)
    bool o_f32 = false; // with split: o is fp32 although q, k, v are bf16
};

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* omega;
    const float* r;
    float* S;
    float* var;
    void* o;
    int B, H, dk, dv;
    float mu;
    const float* mu_h;  // nullable [H]: per-head information scale (overrides mu)
    float* beta;        // nullable [B,H]: effective write strength z / (r + z)
};

// chunked forward: bf16 io runs the walk kernel (kdn_walk.hip), fp32 io the
// fp32 chunk kernel (kdn_chunk.hip)
hipError_t launch_walk_fwd(const FwdArgs& a, bool iso, hipStream_t stream);
hipError_t launch_chunk_fwd_f32(const FwdArgs& a, bool iso, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, bool iso, int io_dtype, hipStream_t stream);

}  // namespace kdn

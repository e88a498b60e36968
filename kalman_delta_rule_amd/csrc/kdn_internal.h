// kdn_internal.h -- argument blocks and launchers shared by the host API and
// the kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>
#include <stdint.h>

namespace kdn {

// Raise a kernel's dynamic-LDS limit to `bytes`, once per device and kernel
// (the attribute holds for the process); later launches skip the call.
template <typename Kernel>
hipError_t set_lds_limit_once(Kernel kern, size_t bytes)
{
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

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
    // bf16 walk only: 0 = full forward; 1 = state only (S_T and var_T; q and o
    // are not touched); 2 = state only with v taken as zero (v not touched)
    int state_only = 0;
    // bf16 walk, full forward only: the gates' bf16 pre-activations, read by
    // the walk itself (alpha = sigmoid(a_pre), Diagonal omega =
    // softplus(w_pre), layouts as alpha and omega); alpha, and Diagonal
    // omega, are then not read.  r, and Isotropic omega, stay fp32 gates.
    const void* a_pre = nullptr;
    const void* w_pre = nullptr;
    // split-product Diagonal walk with state_only = 1 only, nullable: the
    // state at the start of every 16-token chunk, per (b, h, 64-column tile)
    // and chunk a [dk / 4][64][4] fp32 block (rows in fours)
    float* ckpt = nullptr;
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

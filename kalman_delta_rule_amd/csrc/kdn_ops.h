// kdn_ops.h -- argument blocks and launchers of the dense filter, the gain
// scan, the backward pass and the gate prologue (the calls beside the forward
// and decode).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kdn {

// sizes the kernels and the host-side workspace plans (kdn_plan.cpp) share
constexpr int GAIN_CHUNK = 64;  // tokens per gain-scan chunk
constexpr int BWD_L = 16;       // backward: tokens per recompute chunk (checkpoint spacing)
constexpr int BWD_COLS = 16;    // backward: value columns per memory workgroup
constexpr int GR_C = 32;        // backward: tokens per chunk of the gain backward's affine scan
constexpr int SP_MAX = 8;       // split over the sequence: segments at most
constexpr size_t GAIN_STATIC_FLOATS = (size_t)8 << 20;  // the static gain-scan scratch (32 MiB)

struct DenseArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* omega;  // [B,T,H,dk]: diagonal process noise
    const float* r;
    const float* S0;     // nullable
    const float* P0;     // nullable [B,H,dk,dk]: identity when null
    void* o;
    float* S_T;
    float* P_T;          // [B,H,dk,dk]
    float* beta;         // nullable [B,T,H]
    int B, T, H, dk, dv;
};

struct GainArgs {
    const void* k;
    const float* alpha;
    const float* omega;
    const float* r;
    const float* var0;  // nullable
    float* kappa;       // nullable
    float* var_T;
    float* summ;        // workspace: chunk summaries [BH][nchunks][width][4]
    float* carry;       // workspace: chunk-entry variances [BH][nchunks][width]
    int B, T, H, dk;
    float mu;
    // for the backward's recompute (null in the standalone gain scan)
    const float* mu_h = nullptr;  // [H] per-head information scale
    const float* c0 = nullptr;    // [H] initial variance when var0 is null
    float* pprev = nullptr;       // Diagonal [B,T,H,dk]: variance before every token
    float* dd = nullptr;          // Diagonal [B,T,H]: r + z
    float* gsc = nullptr;         // Isotropic [B,T,H,4]: beta, b_{t-1}, mean alpha^2, |k|^2
};

struct BwdArgs {
    // forward inputs (as in FwdArgs)
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* omega;
    const float* r;
    const float* S0;    // nullable
    const float* var0;  // nullable
    const float* c0;    // nullable [H]
    const float* mu_h;  // nullable [H]
    float mu;
    // incoming gradients
    const void* go;       // dL/do, io dtype
    const float* gS_T;    // nullable
    const float* gvar_T;  // nullable
    // outgoing gradients
    void* gq;
    void* gk;
    void* gv;
    float* galpha;
    float* gomega;
    float* gr;
    float* gS0;   // nullable
    float* gvar0; // nullable
    float* gmu;   // nullable [B,H]
    int B, T, H, dk, dv;
    // workspace pieces (set by bwd_carve_workspace)
    float* kap;    // Diagonal [B,T,H,dk]: gain of every token
    float* pprev;  // Diagonal [B,T,H,dk]: variance before every token
    float* dd;     // Diagonal [B,T,H]: r + z
    float* gsc;    // Isotropic [B,T,H,4]: beta, b_{t-1}, mean alpha^2, |k|^2
    float* gscan;  // the gain scan's chunk summaries and carries
    float* gr_sum;   // gain backward: affine map (A, B) per 64-token chunk and channel
    float* gr_carry; // gain backward: carried gradient after each chunk
    float* gr_tok;   // gain backward: dbar / betabar per token
    float* gr_mu;    // gain backward: information-scale gradient per (b,h) and chunk
    float* ckpt;   // S at every 16th token: token-serial path [B*H][dv/16][ceil(T/16)][dk][16];
                   // chunked path [B*H][dv/64][ceil(T/16)][dk/4][64][4] (rows in fours)
    bool ckpt_given = false;  // chunked path: ckpt already holds every chunk-start state
    float* walk_S = nullptr;  // Diagonal chunked path: the checkpoint walk's final state
    float* walk_p = nullptr;  // and final variance (not outputs)
    float* dlt;    // [B*H][dv/16][T][16]: innovations delta of every token
    float* part;   // [4][dv/16][B*T*H][dk]: per-column-block partial row sums
    // the split over the sequence (kdn_seqpar.hip): segments (0: none) and
    // their workspace
    int nseg = 0;
    float* segws = nullptr;
};

struct PrologueArgs {
    const void* a_pre;  // io dtype, n_alpha elements
    const void* w_pre;  // io dtype, n_omega elements
    const void* r_pre;  // io dtype, n_r elements
    float* alpha;
    float* omega;
    float* r;
    size_t n_alpha, n_omega, n_r;
    float r_min;
};

hipError_t launch_dense_fwd(const DenseArgs& a, int io_dtype, hipStream_t stream);
size_t gain_workspace_floats(bool iso, int B, int T, int H, int dk);
// the allocation-free gain scan's static scratch: its size in floats, and its
// device address on the current device
size_t gain_static_scratch_floats();
hipError_t gain_static_scratch(float** ptr);
hipError_t launch_gain_scan(const GainArgs& a, bool iso, int io_dtype, hipStream_t stream);
// the backward's memory part runs in 16-token chunks on the matrix cores
// (kdn_bwd_chunk.hip) for these shapes, token by token otherwise
bool bwd_chunked(int dk, int dv);
constexpr int BWD_CHUNK_COLS = 64;  // value columns per chunked memory workgroup
// adj: the adjoint only (no forward pass, no per-token outputs; bf16 io)
hipError_t launch_bwd_chunk_mem(const BwdArgs& a, bool iso, int io_dtype, bool adj,
                                hipStream_t stream);
size_t bwd_workspace_floats(bool iso, int B, int T, int H, int dk, int dv);
void bwd_carve_workspace(BwdArgs& a, bool iso, float* ws);
// the backward's split over the sequence (kdn_seqpar.hip): the segment count
// for a shape (0: not eligible; the split itself runs with bf16 io only), the
// workspace it adds behind bwd_workspace_floats, and its memory part (after
// the gain scan, in place of launch_bwd_chunk_mem)
int bwd_segments(bool iso, int B, int T, int H, int dk, int dv);
size_t bwd_seg_workspace_floats(bool iso, int B, int T, int H, int dk, int S);
hipError_t launch_seqpar_bwd_mem(const BwdArgs& a, bool iso, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, bool iso, int io_dtype, hipStream_t stream);
hipError_t launch_gate_prologue(const PrologueArgs& a, int io_dtype, hipStream_t stream);
hipError_t launch_gate_epilogue(const PrologueArgs& p, float* da, float* dw, float* dr,
                                int io_dtype, hipStream_t stream);

// sequence-parallel bf16 forward for grids that leave most compute units idle
// (kdn_seqpar.hip): the segment count (0: not eligible), its workspace, and the
// launch over a workspace of that size
int seqpar_segments(bool iso, int B, int T, int H, int dk, int dv, int io_dtype);
size_t seqpar_workspace_floats(bool iso, int B, int T, int H, int dk, int dv, int S);
struct FwdArgs;
hipError_t launch_seqpar_fwd(const FwdArgs& a, bool iso, int S, float* ws, hipStream_t stream);

}  // namespace kdn

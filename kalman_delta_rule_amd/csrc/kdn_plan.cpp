// kdn_plan.cpp -- host-side plans of the library's workspaces: sizes and
// carving of the gain scan's, the split over the sequence's and the
// backward's scratch, and the choice of the split.  Plain C++ (no device code),
// so the host validation code builds and runs on its own, for instance under
// the address and undefined-behaviour sanitizers.
#include <stddef.h>

#include "kdn_internal.h"
#include "kdn_ops.h"

namespace kdn {

static size_t round64(size_t n) { return (n + 63) & ~(size_t)63; }
static size_t r64(size_t n) { return round64(n); }

// ------------------------------------------------------------- gain scan
size_t gain_static_scratch_floats() { return GAIN_STATIC_FLOATS; }

size_t gain_workspace_floats(bool iso, int B, int T, int H, int dk)
{
    const size_t nchunks = (T + GAIN_CHUNK - 1) / GAIN_CHUNK;
    const size_t width = iso ? 1 : (size_t)dk;
    return (size_t)B * H * nchunks * width * 5;  // a 2x2 map and a carry per chunk and channel
}

// --------------------------------------------- forward split over the sequence
int seqpar_segments(bool iso, int B, int T, int H, int dk, int dv, int io_dtype)
{
    (void)iso;
    if (io_dtype != 1 || dk != dv || T <= 0)
        return 0;
    const long ncu = 256;  // MI355X compute units; a fixed figure keeps the size a pure function
    if (B < 1 || H < 1 || dv < 64 || (long)B * H > ncu)
        return 0;          // (also keeps the products below far from overflow)
    const long tiles = (long)B * H * (dv / 64);
    // worth it when the segments multiply the workgroups by 4 or more
    // (three walks of T/S tokens against one of T) and stay long
    for (int s = SP_MAX; s >= 4; s >>= 1)
        if (tiles * s <= ncu && T % (64 * s) == 0 && T / s >= 1024)
            return s;
    return 0;
}

size_t seqpar_workspace_floats(bool iso, int B, int T, int H, int dk, int dv, int S)
{
    const size_t bs = (size_t)B * S, width = iso ? 1 : (size_t)dk;
    const size_t st = bs * H * (size_t)dk * dv;
    size_t n = r64(gain_workspace_floats(iso, B, T, H, dk));
    n += 2 * r64(bs * H * width);                    // segment-entry variances, scratch
    n += 4 * r64(st);                                // N, M, S_in, identity
    return n;
}

// ------------------------------------------------- backward split over the sequence
int bwd_segments(bool iso, int B, int T, int H, int dk, int dv)
{
    // Diagonal only: the segment-entry states come from the forward walk,
    // whose Isotropic form runs single bf16 products (the Diagonal one splits
    // its operands, ~1e-5 relative), below the backward's fp32 accuracy
    if (iso || dk != dv || !bwd_chunked(dk, dv) || T <= 0)
        return 0;
    const long ncu = 256;  // MI355X compute units, as for the forward
    if (B < 1 || H < 1 || (long)B * H > ncu)
        return 0;
    const long tiles = (long)B * H * (dv / BWD_CHUNK_COLS);
    // the chunked backward's step is several times the forward walk's, so
    // doubling the workgroups already pays for the state walks and the
    // adjoint pass the split adds
    for (int s = SP_MAX; s >= 2; s >>= 1)
        if (tiles * s <= ncu && T % (64 * s) == 0 && T / s >= 1024)
            return s;
    return 0;
}

size_t bwd_seg_workspace_floats(bool iso, int B, int T, int H, int dk, int S)
{
    (void)T;
    const size_t bs = (size_t)B * S, width = iso ? 1 : (size_t)dk;
    const size_t st = bs * H * (size_t)dk * dk;
    // segment-entry variances and a scratch plane; N, M, the segment-entry
    // states, the identity, each segment's own adjoint and the adjoint
    // entering it from the right
    return 2 * r64(bs * H * width) + 6 * r64(st);
}

// ------------------------------------------------------------- backward
bool bwd_chunked(int dk, int dv)
{
    return (dk == 64 || dk == 128) && dv >= BWD_CHUNK_COLS && dv % BWD_CHUNK_COLS == 0;
}

size_t bwd_workspace_floats(bool iso, int B, int T, int H, int dk, int dv)
{
    const size_t ntok = (size_t)B * T * H, bh = (size_t)B * H;
    const bool chunked = bwd_chunked(dk, dv);
    const size_t nch = ((size_t)T + BWD_L - 1) / BWD_L,
                 nblk = (size_t)dv / (chunked ? BWD_CHUNK_COLS : BWD_COLS);
    size_t n = 0;
    if (iso)
        n += round64(ntok * 4);
    else
        n += 2 * round64(ntok * dk) + round64(ntok);
    n += round64(gain_workspace_floats(iso, B, T, H, dk));  // gain scan summaries and carries
    const size_t ngc = ((size_t)T + GR_C - 1) / GR_C, width = iso ? 1 : (size_t)dk;
    n += round64(bh * ngc * width * 2) + round64(bh * ngc * width) + round64(ntok) +
         round64(bh * ngc);                  // gain backward: summaries, carries, dbar, mu parts
    n += round64(bh * nch * dk * dv);        // checkpoints
    if (!chunked)
        n += round64(ntok * dv);             // innovations
    if (chunked && !iso && T > 0)            // the checkpoint walk's final state and variance
        n += round64(bh * dk * dv) + round64(bh * dk);
    n += round64(4 * nblk * ntok * dk);      // partials
    return n;
}

void bwd_carve_workspace(BwdArgs& a, bool iso, float* ws)
{
    const size_t ntok = (size_t)a.B * a.T * a.H, bh = (size_t)a.B * a.H;
    const bool chunked = bwd_chunked(a.dk, a.dv);
    const size_t nch = ((size_t)a.T + BWD_L - 1) / BWD_L;
    float* p = ws;
    a.kap = a.pprev = a.dd = a.gsc = nullptr;
    if (iso) {
        a.gsc = p;
        p += round64(ntok * 4);
    } else {
        a.kap = p;
        p += round64(ntok * a.dk);
        a.pprev = p;
        p += round64(ntok * a.dk);
        a.dd = p;
        p += round64(ntok);
    }
    a.gscan = p;
    p += round64(gain_workspace_floats(iso, a.B, a.T, a.H, a.dk));
    const size_t ngc = ((size_t)a.T + GR_C - 1) / GR_C, width = iso ? 1 : (size_t)a.dk;
    a.gr_sum = p;
    p += round64(bh * ngc * width * 2);
    a.gr_carry = p;
    p += round64(bh * ngc * width);
    a.gr_tok = p;
    p += round64(ntok);
    a.gr_mu = p;
    p += round64(bh * ngc);
    a.ckpt = p;
    p += round64(bh * nch * a.dk * a.dv);
    a.dlt = nullptr;
    if (!chunked) {
        a.dlt = p;
        p += round64(ntok * a.dv);
    }
    a.walk_S = a.walk_p = nullptr;
    if (chunked && !iso && a.T > 0) {
        a.walk_S = p;
        p += round64(bh * a.dk * a.dv);
        a.walk_p = p;
        p += round64(bh * a.dk);
    }
    a.part = p;
}

}  // namespace kdn

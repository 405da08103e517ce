// launch.h -- kernel argument blocks and launchers shared by the ABI layer and
// the kernel translation units of libhypic (host and device visible).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "hypic.h"

namespace hy {

constexpr int kMaxSeg = HYPIC_MAX_SEG_PER_LAUNCH;

// Input element kinds of a launch.
enum InKind : int {
    IN_F32 = 0,
    IN_BF16 = 1,
    IN_F16K = 2,   // keys fp16, values fp16 times a power of two per (row, head)
                   // (conv workspace of the fp16-operand build)
};

// Chunkwise gated-delta build, one workgroup per (segment, value head).
struct DeltaArgs {
    const void *k, *v;          // [rows, h_k, D] / [rows, h_v, D], element kind kv_kind
    const void *beta, *alpha;   // [N, h_v], element kind g_kind
    float *T_out, *S0_out;      // at the launch's first segment
    int h_k, h_v;
    int64_t ldk, ldv;           // row strides of k and v in elements
    const float *vscale;        // IN_F16K: [rows, h_v] power-of-two factor of each value row
    int n_seg;
    int64_t tok0[kMaxSeg];      // first row of each range in k / v
    int64_t gtok0[kMaxSeg];     // first row of each range in beta / alpha
    int32_t len[kMaxSeg];
};

// Decay-family build (scalar or diagonal gates), one workgroup per
// (segment, value head, column group).
struct DecayArgs {
    const void *k, *v, *gate;   // gate: [N, h_v] scalar, [N, h_v, D] diag, [h_v] fp32 const
    float *T_out, *S0_out;
    int h_k, h_v;
    int gate_kind;              // HYPIC_GATE_*
    int n_seg;
    int64_t tok0[kMaxSeg];
    int32_t len[kMaxSeg];
};

// Causal conv (+ key L2 normalisation) of the rows a build reads, into a
// packed fp32 workspace.
struct ConvArgs {
    const void *x;              // [N, H, D] raw rows
    const float *w;             // [H*D, W]
    void *out;                  // packed [sum len, H, D], fp32 or fp16 (out_kind)
    float *scale;               // null, or [sum len, H]: fp16 rows are stored divided by this
                                // power of two (their max |y| then lies in [0.5, 1))
    int H, W, l2norm;
    int n_seg;
    int64_t tok0[kMaxSeg];      // first row of each range
    int64_t from[kMaxSeg];      // first row the conv may read
    int64_t out0[kMaxSeg];      // first packed output row of each range
    int32_t len[kMaxSeg];
};

// Seam windows (gated delta).  Per window i the rows are
//   xk[i] [w, h_k, D], tail_k[i] [W-1, h_k, D], beta/alpha[i] [w, h_v].
struct SeamArgs {
    const void *xk, *xv, *tail_k, *tail_v;
    const float *conv_wk, *conv_wv;
    const void *beta, *alpha, *q;
    float *o, *T_w, *S_w0;
    int w, conv_w, k_l2norm, h_k, h_v;
    int gate_diag;              // alpha per key channel [n_win, w, h_v, D] (KDA windows)
};

// Dense / diagonal / scalar composition over a prompt's segments.
struct ComposeArgs {
    const float *T_pool, *S0_pool;
    const float *S_in;          // [h_v, D, D] or null (zero state)
    float *S_out;
    int h_v, n;
    int first_pos;              // prompt position of order[0] (seam i uses window first_pos+i-1)
    int has_seams;
    SeamArgs seam;
    float *S_steps;             // or null: the no-seam fold writes the state entering each step [n, h_v, D, D]
    int32_t order[kMaxSeg];
};

// Rotary re-rotation of cached keys [N, h, d], per segment shift delta.
struct RopeArgs {
    const void *x_in;
    void *x_out;
    int h, d, rot, pairing, copy_rest;   // pairing 0: (i, i + rot/2); 1: (2i, 2i + 1)
    double log2_base;
    int64_t start[kMaxSeg], len[kMaxSeg], delta[kMaxSeg];
};

// Rotary re-rotation of states [h, d_k, d_v] fp32 along d_k.
struct RopeStateArgs {
    const float *S_in;
    float *S_out;
    int h, d_k, d_v, rot, pairing, copy_rest;
    double log2_base;
    int64_t delta;
};

hipError_t launch_rope_keys(const RopeArgs &a, int dtype_bf16, int n_seg, hipStream_t st);
hipError_t launch_rope_state(const RopeStateArgs &a, hipStream_t st);

hipError_t launch_build_delta(const DeltaArgs &a, int D, int kv_kind, int g_kind, bool f16,
                              int n_units, hipStream_t st);
hipError_t launch_build_delta_f16(const DeltaArgs &a, int D, int kv_kind, int g_kind, int n_units,
                                  hipStream_t st);
// d = 128 with bf16 inputs (or their conv workspace): build_gdn.hip
hipError_t launch_build_gdn(const DeltaArgs &a, int kv_kind, int g_kind, int n_units, hipStream_t st);
// delta rule with a diagonal gate (KDA): alpha is the gate [N, h_v, D]
// f16: bf16 inputs at d >= 64 take the fp16-operand state products
hipError_t launch_build_kda(const DeltaArgs &a, int D, int kv_kind, int g_kind, bool f16, int n_units,
                            hipStream_t st);
hipError_t launch_build_decay(const DecayArgs &a, int D, int in_kind, int n_units,
                              hipStream_t st);
hipError_t launch_conv(const ConvArgs &a, int D, int in_kind, bool out_f16, int64_t total_rows,
                       hipStream_t st);
hipError_t launch_compose(const ComposeArgs &a, int D, int tform, int prec, int in_kind,
                          hipStream_t st);
hipError_t launch_seam(const ComposeArgs &a, int D, int in_kind, float *S, int n_win,
                       hipStream_t st);
// split-bf16 dense compose for d in {64, 128}, seam windows from precomputed operators
int64_t seam_ops_floats(int D, int w, int n_win, int h_v, bool ro);
hipError_t launch_seam_ops(const ComposeArgs &a, int D, int in_kind, int n_win, float *ops,
                           hipStream_t st);
hipError_t launch_compose_split(const ComposeArgs &a, int D, const float *ops, hipStream_t st);
// level 1 of the two-level split compose (d in {64, 128}): the a.n positions in
// ng groups of G consecutive ones, each (group, head) folded into one pair,
// written to gT / gS [ng, h_v, D, D].  With window read-outs (a.seam.q set) also
// Y [n_win, h_v, 8, 2D]: the read-out rows A of every window times the
// group-local prefix pair at that window.
hipError_t launch_compose_group(const ComposeArgs &a, int D, const float *ops, int G, int ng, float *gT,
                                float *gS, float *Y, hipStream_t st);
// o of the windows of a launch from Y, the group-start states a.S_steps and
// the windows' read-out records (w <= 8)
hipError_t launch_seam_readout(const ComposeArgs &a, int D, const float *ops, const float *Y, int G,
                               hipStream_t st);

// Allow `bytes` of dynamic LDS for kernel `kern` on the current device, once
// per device (bit d of `done`); concurrent first calls may both set the same
// value, which is harmless, and the flag itself is atomic.
template <typename K>
inline hipError_t allow_dyn_lds(K kern, size_t bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

}  // namespace hy

// abi.hip -- the extern "C" boundary of libhypic: argument validation,
// workspace sizing and kernel dispatch.  See include/hypic.h for the contract.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "hypic.h"
#include "launch.h"

using namespace hy;

namespace {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t esize(int dtype) { return dtype == HYPIC_BF16 ? 2 : 4; }

// gfx950 check, cached per device ordinal
hypic_status device_check()
{
    static std::mutex mu;
    static int state[64];   // 0 unknown, 1 ok, 2 wrong architecture
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return HYPIC_E_HIP;
    if (dev < 0 || dev >= 64) return HYPIC_E_DEVICE;
    std::lock_guard<std::mutex> lk(mu);
    if (state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return HYPIC_E_HIP;
        state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    return state[dev] == 1 ? HYPIC_OK : HYPIC_E_DEVICE;
}

hypic_status from_hip(hipError_t e) { return e == hipSuccess ? HYPIC_OK : HYPIC_E_HIP; }

}  // namespace

// Workspace of hypic_compose_noalloc: a file-scope device array, one copy per
// GPU, allocated when the code object is loaded and held until the process
// ends.  Host code never uses its name as an address: each device's copy is
// looked up once with hipGetSymbolAddress and the looked-up pointer is what the
// kernels receive.
__device__ __align__(256) unsigned char scratch[HYPIC_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of this device's copy of `scratch` (looked up on the first call
// on each device, with that device current).
hypic_status scratch_address(void **out)
{
    static std::mutex mu;
    static void *addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return HYPIC_E_HIP;
    if (dev < 0 || dev >= 64) return HYPIC_E_DEVICE;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HYPIC_E_HIP;
        addr[dev] = p;
    }
    *out = addr[dev];
    return HYPIC_OK;
}

bool build_needs_prep(const hypic_build_desc *d) { return d->conv_w > 0 || d->k_l2norm; }

// Longest gated-delta segment (tokens) built on fp16 matrix-core operands.  Their
// rounding enters once per 64-token chunk, so the error of the transition
// product grows with the chunk count: about 1.4e-3 relative at 4096 tokens and
// 3.3e-3 at 16384 on slowly decaying gates, against the 2e-3 bound for bf16
// inputs.  Longer segments are built with fp32 products (about 1e-6).
constexpr int64_t kF16MaxLen = 4096;

int64_t build_rows(const hypic_build_desc *d)
{
    int64_t n = 0;
    for (int s = 0; s < d->n_seg; ++s) n += d->seg_len[s];
    return n;
}

size_t build_ws_bytes(const hypic_build_desc *d)
{
    if (!build_needs_prep(d)) return 0;
    const int64_t rows = build_rows(d);
    const size_t kb = (size_t)rows * d->h_k * d->d_k * sizeof(float);
    const size_t vb = (size_t)rows * d->h_v * d->d_v * sizeof(float);
    return ((kb + 255) & ~(size_t)255) + vb;
}

hypic_status validate_build(const hypic_build_desc *d)
{
    if (!d) return HYPIC_E_INVALID;
    if (d->n_seg < 0) return HYPIC_E_INVALID;
    if (d->n_seg > 0 && (!d->seg_start || !d->seg_len)) return HYPIC_E_INVALID;
    if (d->h_k <= 0 || d->h_v <= 0 || d->h_v % d->h_k != 0) return HYPIC_E_INVALID;
    if (d->in_dtype != HYPIC_F32 && d->in_dtype != HYPIC_BF16) return HYPIC_E_INVALID;
    if (d->rule != HYPIC_RULE_DECAY && d->rule != HYPIC_RULE_DELTA) return HYPIC_E_INVALID;
    if (d->gate_kind < HYPIC_GATE_HEAD_CONST || d->gate_kind > HYPIC_GATE_DIAG) return HYPIC_E_INVALID;
    if (d->conv_w < 0 || d->conv_w > 4) return HYPIC_E_INVALID;
    if (d->d_k != d->d_v || !dim_ok(d->d_k)) return HYPIC_E_UNSUPPORTED;
    // row pitches h * d enter 24-bit multiplies in the build kernels
    if ((int64_t)d->h_v * d->d_k >= (1 << 24)) return HYPIC_E_UNSUPPORTED;
    if (d->rule == HYPIC_RULE_DELTA && d->gate_kind == HYPIC_GATE_HEAD_CONST) return HYPIC_E_UNSUPPORTED;
    if (d->rule == HYPIC_RULE_DECAY && build_needs_prep(d)) return HYPIC_E_UNSUPPORTED;
    if (!d->k || !d->v || !d->gate || !d->T_out || !d->S0_out) return HYPIC_E_INVALID;
    if (d->rule == HYPIC_RULE_DELTA && !d->beta) return HYPIC_E_INVALID;
    if (!aligned16(d->k) || !aligned16(d->v) || !aligned16(d->T_out) || !aligned16(d->S0_out))
        return HYPIC_E_INVALID;
    if (d->conv_w > 0 && (!d->conv_from || !d->conv_wk || !d->conv_wv)) return HYPIC_E_INVALID;
    if (d->conv_w > 0 && (!aligned16(d->conv_wk) || !aligned16(d->conv_wv))) return HYPIC_E_INVALID;
    for (int s = 0; s < d->n_seg; ++s) {
        if (d->seg_start[s] < 0 || d->seg_len[s] < 0 || d->seg_len[s] > INT32_MAX) return HYPIC_E_INVALID;
        if (d->conv_w > 0 && (d->conv_from[s] < 0 || d->conv_from[s] > d->seg_start[s])) return HYPIC_E_INVALID;
    }
    return HYPIC_OK;
}

hypic_status validate_seams(const hypic_seam_desc *s, int h_v, int D, int max_w)
{
    if (!s) return HYPIC_E_INVALID;
    if (s->rule != HYPIC_RULE_DELTA) return HYPIC_E_UNSUPPORTED;
    if (s->in_dtype != HYPIC_F32 && s->in_dtype != HYPIC_BF16) return HYPIC_E_INVALID;
    if (s->h_v != h_v || s->d_k != D || s->d_v != D) return HYPIC_E_INVALID;
    if (s->h_k <= 0 || s->h_v % s->h_k != 0) return HYPIC_E_INVALID;
    if (s->w < 1) return HYPIC_E_INVALID;
    if (s->w > max_w) return HYPIC_E_UNSUPPORTED;
    if (s->conv_w < 0 || s->conv_w > 4) return HYPIC_E_INVALID;
    if (!s->xk || !s->xv || !s->beta || !s->alpha) return HYPIC_E_INVALID;
    if (s->conv_w > 0 && (!s->conv_wk || !s->conv_wv)) return HYPIC_E_INVALID;
    if (s->conv_w > 1 && (!s->tail_k || !s->tail_v)) return HYPIC_E_INVALID;
    if ((s->q == nullptr) != (s->o == nullptr)) return HYPIC_E_INVALID;
    if (s->gate_diag != 0 && s->gate_diag != 1) return HYPIC_E_INVALID;
    return HYPIC_OK;
}

// dense split compose for d in {64, 128} takes the pipelined kernel
// (windows with per-channel gates run token by token in the serial dense kernel)
bool compose_uses_split(const hypic_compose_desc *d)
{
    return d->tform == HYPIC_T_DENSE && d->prec == HYPIC_PREC_SPLIT &&
           (d->d_k == 64 || d->d_k == 128) && !(d->seams && d->seams->gate_diag);
}

// Group length of the two-level compose for a launch of nb positions (1: the
// serial fold).  Automatic (group_len 0): enough (group, head) workgroups to
// fill the chip once, when the serial fold is long enough to gain from it.
// window read-outs requested (seam q / o)
bool compose_readouts(const hypic_compose_desc *d) { return d->seams && d->seams->q && d->seams->o; }

int compose_group_len(const hypic_compose_desc *d, int nb)
{
    if (compose_readouts(d) && compose_uses_split(d)) {
        // read-outs ride on the group kernel: every launch takes the two-level
        // path, with enough (group, head) workgroups to fill the chip once (groups
        // of one position for a short launch with few heads)
        if (d->group_len >= 1) return std::min(d->group_len, std::max(nb, 1));
        const int per_cu = d->d_k == 128 ? 1 : 2;
        const int ng = std::max(1, 256 * per_cu / d->h_v);
        return std::max(1, (nb + ng - 1) / ng);
    }
    if (!compose_uses_split(d) || nb < 2 || d->group_len == 1) return 1;
    if (d->seams && d->seams->w > 8) return 1;   // the group kernel holds windows of up to 8 rows
    if (d->group_len > 1) return std::min(d->group_len, nb);
    if (nb < 16) return 1;
    const int per_cu = d->d_k == 128 ? 1 : 2;
    const int ng = std::max(1, 256 * per_cu / d->h_v);
    const int G = (nb + ng - 1) / ng;
    return G >= 2 ? G : 1;
}

// group pairs of the largest launch: ceil(nb / G) over the launch sizes of a call
int compose_max_groups(const hypic_compose_desc *d)
{
    int best = 0;
    const int sizes[2] = {std::min(d->n, (int)kMaxSeg), d->n % kMaxSeg};
    for (int nb : sizes) {
        if (nb <= 0) continue;
        const int G = compose_group_len(d, nb);
        if (G > 1 || (compose_readouts(d) && compose_uses_split(d))) best = std::max(best, (nb + G - 1) / G);
    }
    return best;
}

size_t ws_align(size_t b) { return (b + 255) & ~(size_t)255; }

// seam operators (if any), then the group pairs T [ng, h_v, d, d] and S0 likewise
size_t compose_ops_bytes(const hypic_compose_desc *d)
{
    if (!d->seams || !compose_uses_split(d) || d->n <= 1) return 0;
    return ws_align((size_t)seam_ops_floats(d->d_k, d->seams->w, d->n - 1, d->h_v, compose_readouts(d)) *
                    sizeof(float));
}

size_t compose_group_bytes(const hypic_compose_desc *d)
{
    return (size_t)compose_max_groups(d) * d->h_v * d->d_k * d->d_v * sizeof(float);
}

// read-outs of the two-level path: the rows Y [n - 1, h_v, 8, 2 d] and the
// states entering the groups [groups, h_v, d, d]
size_t compose_readout_bytes(const hypic_compose_desc *d)
{
    if (!compose_readouts(d) || !compose_uses_split(d) || d->n <= 1) return 0;
    return ws_align((size_t)(d->n - 1) * d->h_v * 8 * 2 * d->d_k * sizeof(float)) + compose_group_bytes(d);
}

size_t compose_ws_bytes(const hypic_compose_desc *d)
{
    return compose_ops_bytes(d) + 2 * compose_group_bytes(d) + compose_readout_bytes(d);
}

SeamArgs seam_args(const hypic_seam_desc *s)
{
    SeamArgs a;
    a.xk = s->xk; a.xv = s->xv; a.tail_k = s->tail_k; a.tail_v = s->tail_v;
    a.conv_wk = s->conv_wk; a.conv_wv = s->conv_wv;
    a.beta = s->beta; a.alpha = s->alpha; a.q = s->q;
    a.o = s->o; a.T_w = s->T_w; a.S_w0 = s->S_w0;
    a.w = s->w; a.conv_w = s->conv_w; a.k_l2norm = s->k_l2norm; a.h_k = s->h_k; a.h_v = s->h_v;
    a.gate_diag = s->gate_diag;
    return a;
}

}  // namespace

extern "C" {

int32_t hypic_version(void) { return 100; }

const char *hypic_status_string(hypic_status s)
{
    switch (s) {
    case HYPIC_OK: return "ok";
    case HYPIC_E_INVALID: return "invalid argument";
    case HYPIC_E_UNSUPPORTED: return "unsupported configuration";
    case HYPIC_E_WORKSPACE: return "workspace missing or too small";
    case HYPIC_E_HIP: return "HIP runtime error";
    case HYPIC_E_DEVICE: return "device is not gfx950";
    case HYPIC_E_TOO_LARGE: return "request needs more scratch than the allocation-free call holds";
    default: return "unknown status";
    }
}

size_t hypic_workspace_size(const void *desc, int which)
{
    if (!desc) return 0;
    if (which == HYPIC_WS_BUILD) {
        const hypic_build_desc *d = static_cast<const hypic_build_desc *>(desc);
        if (validate_build(d) != HYPIC_OK) return 0;
        return build_ws_bytes(d);
    }
    if (which == HYPIC_WS_COMPOSE) {
        const hypic_compose_desc *d = static_cast<const hypic_compose_desc *>(desc);
        if (d->d_k != d->d_v || !dim_ok(d->d_k) || d->n < 0 || d->h_v <= 0) return 0;
        if (d->seams && (d->seams->w < 1 || d->seams->w > 16)) return 0;
        return compose_ws_bytes(d);
    }
    return 0;
}

hypic_status hypic_segment_build(const hypic_build_desc *d, void *ws, size_t ws_bytes, void *stream)
{
    hypic_status st = validate_build(d);
    if (st != HYPIC_OK) return st;
    const size_t need = build_ws_bytes(d);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return HYPIC_E_WORKSPACE;
    if (d->n_seg == 0) return HYPIC_OK;
    st = device_check();
    if (st != HYPIC_OK) return st;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const int D = d->d_k;
    const int in_kind = d->in_dtype == HYPIC_BF16 ? IN_BF16 : IN_F32;
    const bool prep = build_needs_prep(d);
    const bool kda = d->rule == HYPIC_RULE_DELTA && d->gate_kind == HYPIC_GATE_DIAG;
    // gated-delta segments with bf16 inputs and d >= 64 take the fp16-operand
    // build, up to kF16MaxLen tokens; longer ones the fp32-operand build
    const bool f16_family = d->rule == HYPIC_RULE_DELTA && !kda && d->in_dtype == HYPIC_BF16 && D >= 64;
    // KDA segments with bf16 inputs (no conv) and d >= 64 take the fp16-operand
    // state products under the same length limit
    const bool kda_f16 = kda && d->in_dtype == HYPIC_BF16 && D >= 64 && !prep;
    auto long_seg = [&](int s) { return (f16_family || kda_f16) && d->seg_len[s] > kF16MaxLen; };
    float *wk = nullptr, *wvv = nullptr, *wvs = nullptr;
    if (prep) {
        const int64_t rows = build_rows(d);
        wk = static_cast<float *>(ws);
        const size_t kb = (size_t)rows * d->h_k * D * sizeof(float);
        wvv = reinterpret_cast<float *>(static_cast<char *>(ws) + ((kb + 255) & ~(size_t)255));
        // fp16 value rows take the first half of the value region, their factors the
        // second half
        wvs = wvv + ((size_t)rows * d->h_v * D / 2);
    }
    int64_t packed = 0;
    // launches over runs of consecutive segments of one operand class, at most
    // kMaxSeg each (outputs of a launch stay contiguous)
    for (int s0 = 0, nb = 0; s0 < d->n_seg; s0 += nb) {
        const bool lng = long_seg(s0);
        nb = 1;
        while (nb < kMaxSeg && s0 + nb < d->n_seg && long_seg(s0 + nb) == lng) ++nb;
        // the fp16-operand build takes fp16 keys and scaled fp16 values from the conv
        const bool khalf = prep && f16_family && !lng;
        const size_t tsz = d->rule == HYPIC_RULE_DELTA ? (size_t)D * D
                         : (d->gate_kind == HYPIC_GATE_DIAG ? (size_t)D : 1);
        float *T_out = d->T_out + (size_t)s0 * d->h_v * tsz;
        float *S0_out = d->S0_out + (size_t)s0 * d->h_v * D * D;
        if (d->rule == HYPIC_RULE_DELTA) {
            DeltaArgs a;
            memset(&a, 0, sizeof(a));
            a.beta = d->beta; a.alpha = d->gate;
            a.T_out = T_out; a.S0_out = S0_out;
            a.h_k = d->h_k; a.h_v = d->h_v;
            a.n_seg = nb;
            int64_t rows_b = 0;
            for (int i = 0; i < nb; ++i) {
                a.gtok0[i] = d->seg_start[s0 + i];
                a.len[i] = (int32_t)d->seg_len[s0 + i];
                a.tok0[i] = prep ? packed + rows_b : d->seg_start[s0 + i];
                rows_b += d->seg_len[s0 + i];
            }
            if (prep) {
                ConvArgs c;
                memset(&c, 0, sizeof(c));
                c.W = d->conv_w;
                c.n_seg = nb;
                for (int i = 0; i < nb; ++i) {
                    c.tok0[i] = d->seg_start[s0 + i];
                    c.from[i] = d->conv_w > 0 ? d->conv_from[s0 + i] : d->seg_start[s0 + i];
                    c.out0[i] = a.tok0[i] - packed;
                    c.len[i] = a.len[i];
                }
                // for the fp16-operand build the rows go out in fp16 (normalised keys;
                // value rows divided by a power of two each, kept beside them), which
                // that build rounds its operands to anyway; fp32 otherwise
                c.x = d->k; c.w = d->conv_wk; c.H = d->h_k; c.scale = nullptr;
                c.out = khalf ? static_cast<void *>(reinterpret_cast<_Float16 *>(wk) + packed * d->h_k * D)
                              : static_cast<void *>(wk + packed * d->h_k * D);
                c.l2norm = d->k_l2norm;
                if ((st = from_hip(launch_conv(c, D, in_kind, khalf, rows_b, hs))) != HYPIC_OK) return st;
                c.x = d->v; c.w = d->conv_wv; c.H = d->h_v;
                c.out = khalf ? static_cast<void *>(reinterpret_cast<_Float16 *>(wvv) + packed * d->h_v * D)
                              : static_cast<void *>(wvv + packed * d->h_v * D);
                c.scale = khalf ? wvs + packed * d->h_v : nullptr;
                c.l2norm = 0;
                if ((st = from_hip(launch_conv(c, D, in_kind, khalf, rows_b, hs))) != HYPIC_OK) return st;
                a.k = khalf ? static_cast<const void *>(reinterpret_cast<_Float16 *>(wk)) : wk;
                a.v = khalf ? static_cast<const void *>(reinterpret_cast<_Float16 *>(wvv)) : wvv;
                a.vscale = khalf ? wvs : nullptr;
                a.ldk = (int64_t)d->h_k * D; a.ldv = (int64_t)d->h_v * D;
                packed += rows_b;
            } else {
                a.k = d->k; a.v = d->v;
                a.ldk = (int64_t)d->h_k * D; a.ldv = (int64_t)d->h_v * D;
            }
            const int kv_kind = khalf ? IN_F16K : (prep ? IN_F32 : in_kind);
            st = kda ? from_hip(launch_build_kda(a, D, kv_kind, in_kind, kda_f16 && !lng, nb * d->h_v, hs))
                     : from_hip(launch_build_delta(a, D, kv_kind, in_kind, d->in_dtype == HYPIC_BF16 && !lng,
                                                   nb * d->h_v, hs));
        } else {
            DecayArgs a;
            memset(&a, 0, sizeof(a));
            a.k = d->k; a.v = d->v; a.gate = d->gate;
            a.T_out = T_out; a.S0_out = S0_out;
            a.h_k = d->h_k; a.h_v = d->h_v; a.gate_kind = d->gate_kind;
            a.n_seg = nb;
            for (int i = 0; i < nb; ++i) {
                a.tok0[i] = d->seg_start[s0 + i];
                a.len[i] = (int32_t)d->seg_len[s0 + i];
            }
            st = from_hip(launch_build_decay(a, D, in_kind, nb * d->h_v, hs));
        }
        if (st != HYPIC_OK) return st;
    }
    return HYPIC_OK;
}

}  // extern "C"

namespace {

// Argument checks of a compose (nothing launched); in_kind receives the
// element kind of the seam windows' inputs.
hypic_status validate_compose(const hypic_compose_desc *d, int *in_kind_out)
{
    if (!d) return HYPIC_E_INVALID;
    if (d->tform < HYPIC_T_SCALAR || d->tform > HYPIC_T_DENSE) return HYPIC_E_INVALID;
    if (d->prec != HYPIC_PREC_FP32 && d->prec != HYPIC_PREC_SPLIT) return HYPIC_E_INVALID;
    if (d->h_v <= 0 || d->n < 0 || d->group_len < 0) return HYPIC_E_INVALID;
    if (d->d_k != d->d_v || !dim_ok(d->d_k)) return HYPIC_E_UNSUPPORTED;
    if (!d->S_out || !aligned16(d->S_out) || (d->S_init && !aligned16(d->S_init))) return HYPIC_E_INVALID;
    if (d->n > 0) {
        if (!d->order || !d->T_pool || !d->S0_pool || d->n_slots <= 0) return HYPIC_E_INVALID;
        if (!aligned16(d->T_pool) || !aligned16(d->S0_pool)) return HYPIC_E_INVALID;
        for (int i = 0; i < d->n; ++i)
            if (d->order[i] < 0 || d->order[i] >= d->n_slots) return HYPIC_E_INVALID;
    }
    const int D = d->d_k;
    int in_kind = IN_F32;
    if (d->seams) {
        if (d->tform != HYPIC_T_DENSE) return HYPIC_E_UNSUPPORTED;
        hypic_status st = validate_seams(d->seams, d->h_v, D, 16);
        if (st != HYPIC_OK) return st;
        if (d->seams->n_win != std::max(0, d->n - 1)) return HYPIC_E_INVALID;
        if (d->seams->T_w || d->seams->S_w0) return HYPIC_E_INVALID;
        // read-outs on the split path ride on the group kernel (windows of up to 8 rows)
        if (compose_readouts(d) && compose_uses_split(d) && d->seams->w > 8) return HYPIC_E_UNSUPPORTED;
        in_kind = d->seams->in_dtype == HYPIC_BF16 ? IN_BF16 : IN_F32;
    }
    *in_kind_out = in_kind;
    return HYPIC_OK;
}

// The launches of a validated compose on a workspace of at least
// compose_ws_bytes(d) bytes.
hypic_status run_compose(const hypic_compose_desc *d, int in_kind, void *ws, hipStream_t hs)
{
    const int D = d->d_k;
    hypic_status st = HYPIC_OK;
    ComposeArgs a;
    memset(&a, 0, sizeof(a));
    a.T_pool = d->T_pool; a.S0_pool = d->S0_pool;
    a.h_v = d->h_v;
    a.has_seams = d->seams != nullptr;
    if (d->seams) a.seam = seam_args(d->seams);
    const bool split = compose_uses_split(d);
    float *ops = nullptr;
    if (split && a.has_seams && d->n > 1) {
        ops = static_cast<float *>(ws);
        if ((st = from_hip(launch_seam_ops(a, D, in_kind, d->n - 1, ops, hs))) != HYPIC_OK) return st;
    }
    if (d->n == 0) {
        a.S_in = d->S_init; a.S_out = d->S_out; a.n = 0;
        return from_hip(launch_compose(a, D, HYPIC_T_SCALAR, d->prec, in_kind, hs));
    }
    float *gT = nullptr, *gS = nullptr, *Y = nullptr, *S_steps = nullptr;
    if (compose_group_bytes(d) > 0) {
        gT = reinterpret_cast<float *>(static_cast<char *>(ws) + compose_ops_bytes(d));
        gS = gT + compose_group_bytes(d) / sizeof(float);
    }
    const bool ro = split && compose_readouts(d) && d->n > 1;
    if (ro) {
        Y = reinterpret_cast<float *>(static_cast<char *>(ws) + compose_ops_bytes(d) + 2 * compose_group_bytes(d));
        S_steps = Y + ws_align((size_t)(d->n - 1) * d->h_v * 8 * 2 * D * sizeof(float)) / sizeof(float);
    }
    for (int b = 0; b < d->n; b += kMaxSeg) {
        a.n = std::min(kMaxSeg, d->n - b);
        a.first_pos = b;
        a.S_in = b == 0 ? d->S_init : d->S_out;
        a.S_out = d->S_out;
        for (int i = 0; i < a.n; ++i) a.order[i] = d->order[b + i];
        const int G = compose_group_len(d, a.n);
        if (G > 1 || ro) {
            // level 1: every group of G positions folded into one pair; level 2:
            // the serial fold over the group pairs (with read-outs also the state
            // entering each group, then the windows' read-outs)
            const int ng = (a.n + G - 1) / G;
            if ((st = from_hip(launch_compose_group(a, D, ops, G, ng, gT, gS, Y, hs))) != HYPIC_OK) return st;
            ComposeArgs a2 = a;
            a2.T_pool = gT; a2.S0_pool = gS;
            a2.n = ng; a2.first_pos = 0; a2.has_seams = 0;
            a2.S_steps = S_steps;
            for (int i = 0; i < ng; ++i) a2.order[i] = i;
            st = from_hip(launch_compose_split(a2, D, nullptr, hs));
            if (st == HYPIC_OK && ro) {
                ComposeArgs a3 = a;
                a3.S_steps = S_steps;
                st = from_hip(launch_seam_readout(a3, D, ops, Y, G, hs));
            }
        } else {
            st = split ? from_hip(launch_compose_split(a, D, ops, hs))
                       : from_hip(launch_compose(a, D, d->tform, d->prec, in_kind, hs));
        }
        if (st != HYPIC_OK) return st;
    }
    return HYPIC_OK;
}

}  // namespace

extern "C" {

hypic_status hypic_compose(const hypic_compose_desc *d, void *ws, size_t ws_bytes, void *stream)
{
    int in_kind = IN_F32;
    hypic_status st = validate_compose(d, &in_kind);
    if (st != HYPIC_OK) return st;
    const size_t need = compose_ws_bytes(d);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return HYPIC_E_WORKSPACE;
    if ((st = device_check()) != HYPIC_OK) return st;
    return run_compose(d, in_kind, ws, reinterpret_cast<hipStream_t>(stream));
}

hypic_status hypic_compose_noalloc(const hypic_compose_desc *d, void *stream)
{
    int in_kind = IN_F32;
    hypic_status st = validate_compose(d, &in_kind);
    if (st != HYPIC_OK) return st;
    if (compose_ws_bytes(d) > (size_t)HYPIC_NOALLOC_SCRATCH_BYTES) return HYPIC_E_TOO_LARGE;
    if ((st = device_check()) != HYPIC_OK) return st;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != HYPIC_OK) return st;
    return run_compose(d, in_kind, ws, reinterpret_cast<hipStream_t>(stream));
}

hypic_status hypic_rope_rerotate(const hypic_rope_desc *d, void *stream)
{
    if (!d || d->n_seg < 0 || d->h <= 0) return HYPIC_E_INVALID;
    if (d->dtype != HYPIC_F32 && d->dtype != HYPIC_BF16) return HYPIC_E_INVALID;
    if (d->pairing != HYPIC_ROPE_HALF && d->pairing != HYPIC_ROPE_INTERLEAVED) return HYPIC_E_INVALID;
    if (!(d->base > 0.0) || !std::isfinite(d->base)) return HYPIC_E_INVALID;
    if (d->d < 8 || d->d > 512 || d->d % 8 != 0) return HYPIC_E_UNSUPPORTED;
    if (d->rot_dim < 8 || d->rot_dim > d->d || d->rot_dim % 8 != 0) return HYPIC_E_UNSUPPORTED;
    if (d->n_seg == 0) return HYPIC_OK;
    if (!d->seg_start || !d->seg_len || !d->delta) return HYPIC_E_INVALID;
    if (!d->x_in || !d->x_out || !aligned16(d->x_in) || !aligned16(d->x_out)) return HYPIC_E_INVALID;
    for (int i = 0; i < d->n_seg; ++i)
        if (d->seg_start[i] < 0 || d->seg_len[i] < 0 || d->seg_len[i] > INT32_MAX) return HYPIC_E_INVALID;
    hypic_status st = device_check();
    if (st != HYPIC_OK) return st;
    RopeArgs a;
    memset(&a, 0, sizeof(a));
    a.x_in = d->x_in; a.x_out = d->x_out;
    a.h = d->h; a.d = d->d; a.rot = d->rot_dim; a.pairing = d->pairing;
    a.copy_rest = d->x_out != d->x_in && d->rot_dim < d->d;
    a.log2_base = std::log2(d->base);
    for (int b = 0; b < d->n_seg; b += kMaxSeg) {
        const int nb = std::min(kMaxSeg, d->n_seg - b);
        for (int i = 0; i < nb; ++i) {
            a.start[i] = d->seg_start[b + i];
            a.len[i] = d->seg_len[b + i];
            a.delta[i] = d->delta[b + i];
        }
        if ((st = from_hip(launch_rope_keys(a, d->dtype == HYPIC_BF16, nb, reinterpret_cast<hipStream_t>(stream)))) != HYPIC_OK)
            return st;
    }
    return HYPIC_OK;
}

hypic_status hypic_rope_rerotate_state(int32_t h, int32_t d_k, int32_t d_v, int32_t rot_dim, int32_t pairing,
                                       double base, int64_t delta, const float *S_in, float *S_out, void *stream)
{
    if (h <= 0 || d_v <= 0 || !S_in || !S_out || !aligned16(S_in) || !aligned16(S_out)) return HYPIC_E_INVALID;
    if (pairing != HYPIC_ROPE_HALF && pairing != HYPIC_ROPE_INTERLEAVED) return HYPIC_E_INVALID;
    if (!(base > 0.0) || !std::isfinite(base)) return HYPIC_E_INVALID;
    if (d_k < 8 || d_k > 512 || d_v % 4 != 0) return HYPIC_E_UNSUPPORTED;
    if (rot_dim < 8 || rot_dim > d_k || rot_dim % 8 != 0) return HYPIC_E_UNSUPPORTED;
    hypic_status st = device_check();
    if (st != HYPIC_OK) return st;
    RopeStateArgs a;
    memset(&a, 0, sizeof(a));
    a.S_in = S_in; a.S_out = S_out;
    a.h = h; a.d_k = d_k; a.d_v = d_v; a.rot = rot_dim; a.pairing = pairing;
    a.copy_rest = S_out != S_in && rot_dim < d_k;
    a.log2_base = std::log2(base);
    a.delta = delta;
    return from_hip(launch_rope_state(a, reinterpret_cast<hipStream_t>(stream)));
}

hypic_status hypic_seam_advance(const hypic_seam_desc *d, float *S_inout, void *stream)
{
    if (!d || !S_inout || !aligned16(S_inout)) return HYPIC_E_INVALID;
    if (d->d_k != d->d_v || !dim_ok(d->d_k)) return HYPIC_E_UNSUPPORTED;
    if (d->h_v <= 0) return HYPIC_E_INVALID;
    hypic_status st = validate_seams(d, d->h_v, d->d_k, 64);
    if (st != HYPIC_OK) return st;
    if (d->gate_diag && (d->T_w || d->S_w0)) return HYPIC_E_UNSUPPORTED;
    if (d->n_win < 0) return HYPIC_E_INVALID;
    if (d->n_win == 0) return HYPIC_OK;
    st = device_check();
    if (st != HYPIC_OK) return st;
    ComposeArgs a;
    memset(&a, 0, sizeof(a));
    a.h_v = d->h_v;
    a.seam = seam_args(d);
    const int in_kind = d->in_dtype == HYPIC_BF16 ? IN_BF16 : IN_F32;
    return from_hip(launch_seam(a, d->d_k, in_kind, S_inout, d->n_win,
                                reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

// conv.hip -- depthwise causal conv of the key / value rows a segment build
// reads, with optional key L2 normalisation, into a packed workspace: fp32,
// or fp16 for the fp16-operand build (value rows then carry a power-of-two
// factor each) (HYPIC reading notes ch.2 sec.6: the
// QKV path's width-k causal conv; a segment prefilled on its own sees zeros
// before its first row).
//   y[t][c] = sum_{j<W} w[c][j] * x[t - W + 1 + j][c],  rows before `from` read 0
// One thread per (16 consecutive rows, head, 8 columns): a row of a head is D/8
// consecutive lanes with 16-byte loads, its L2 norm a reduction over them; the
// weights load once per thread and the taps slide along the rows in registers.
#include "common.h"
#include "launch.h"

namespace hy {

__device__ __forceinline__ void st8(float *p, const float (&y)[8]) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(y[0], y[1], y[2], y[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(y[4], y[5], y[6], y[7]);
}
__device__ __forceinline__ void st8(_Float16 *p, const float (&y)[8]) {
    h8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (_Float16)y[e];
    *reinterpret_cast<h8 *>(p) = v;
}

template <int D, typename TIN, typename TOUT>
__global__ void __launch_bounds__(256) conv_kernel(const ConvArgs a, int64_t total_rows)
{
    constexpr int CH = D / 8;   // threads per (row, head)
    constexpr int R = 16;       // consecutive packed rows per thread
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int cc = (int)(gid % CH);
    const int64_t rh = gid / CH;
    const int hh = (int)(rh % a.H);
    const int64_t p0 = (rh / a.H) * R;          // first packed row of this thread
    const TIN *x = reinterpret_cast<const TIN *>(a.x);
    const int64_t ld = (int64_t)a.H * D;
    const int64_t col = (int64_t)hh * D + 8 * cc;
    // weights of the 8 columns, once, by offset from the output row: wo[e][o] is the
    // weight of x[row - o] (tap W-1-o), zero for o >= W
    float wo[8][4];
    if (a.W == 4) {
        const float4 *wp = reinterpret_cast<const float4 *>(a.w + col * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float4 q = wp[e];
            wo[e][0] = q.w; wo[e][1] = q.z; wo[e][2] = q.y; wo[e][3] = q.x;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int o = 0; o < 4; ++o) wo[e][o] = o < a.W ? a.w[(col + e) * a.W + (a.W - 1 - o)] : 0.f;
    }
    // segment of the first row: binary search for the wave's first (smallest) row on
    // the scalar side, then each lane steps forward past segment starts
    const int64_t pc = min(p0, total_rows - 1);
    const int64_t p_w = (int64_t)__builtin_amdgcn_readfirstlane((int)(pc & 0xffffffff)) |
                        ((int64_t)__builtin_amdgcn_readfirstlane((int)(pc >> 32)) << 32);
    int lo = 0, hi = a.n_seg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.out0[mid] <= p_w) lo = mid; else hi = mid - 1;
    }
    int s = lo;
    // taps: h[k] = x[row - 1 - k] (k < 3), zero before the segment's conv start
    float h[3][8];
    for (int i = 0; i < R; ++i) {
        const int64_t p = min(p0 + i, total_rows - 1);   // tail rows computed, not stored
        while (s + 1 < a.n_seg && a.out0[s + 1] <= p) ++s;
        const int64_t row = a.tok0[s] + (p - a.out0[s]);
        if (i == 0 || p == a.out0[s]) {   // group or segment start: load the taps
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int64_t r = row - 1 - k;
                const bool in = r >= a.from[s] && k < a.W - 1;
                float xv[8];
                ld8(x + (in ? r : row) * ld + col, xv);   // address clamped, value masked
#pragma unroll
                for (int e = 0; e < 8; ++e) h[k][e] = in ? xv[e] : 0.f;
            }
        }
        float cur[8], y[8];
        ld8(x + row * ld + col, cur);
        if (a.W > 0) {
            // y = sum_o wo[o] x[row - o]: x[row] = cur, x[row - 1 - k] = h[k]
#pragma unroll
            for (int e = 0; e < 8; ++e)
                y[e] = wo[e][0] * cur[e] + wo[e][1] * h[0][e] + wo[e][2] * h[1][e] + wo[e][3] * h[2][e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = cur[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { h[2][e] = h[1][e]; h[1][e] = h[0][e]; h[0][e] = cur[e]; }
        if (a.l2norm) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
#pragma unroll
            for (int m = 1; m < CH; m <<= 1) ss += __shfl_xor(ss, m);   // the CH lanes of the row
            const float sc = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= sc;
        }
        const bool live = p0 + i < total_rows;
        if (a.scale) {
            // per-row power of two so the fp16 row keeps its range: max |y| / f in [0.5, 1)
            float m = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[e]));
#pragma unroll
            for (int k = 1; k < CH; k <<= 1) m = fmaxf(m, __shfl_xor(m, k));
            const int ex = pow2_exponent(m);
            const float inv = ldexpf(1.f, -ex);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= inv;
            if (live && cc == 0) a.scale[p * a.H + hh] = ldexpf(1.f, ex);
        }
        if (live) st8(reinterpret_cast<TOUT *>(a.out) + p * ld + col, y);
    }
}

template <int D, typename TIN>
static hipError_t launch_d(const ConvArgs &a, bool out_f16, int64_t total_rows, hipStream_t st)
{
    const int64_t threads = (total_rows + 15) / 16 * a.H * (D / 8);
    const int64_t blocks = (threads + 255) / 256;
    if (out_f16)
        hipLaunchKernelGGL((conv_kernel<D, TIN, _Float16>), dim3((unsigned)blocks), dim3(256), 0, st, a, total_rows);
    else
        hipLaunchKernelGGL((conv_kernel<D, TIN, float>), dim3((unsigned)blocks), dim3(256), 0, st, a, total_rows);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dd(const ConvArgs &a, int in_kind, bool out_f16, int64_t total_rows, hipStream_t st)
{
    return in_kind == IN_BF16 ? launch_d<D, bf16_t>(a, out_f16, total_rows, st)
                              : launch_d<D, float>(a, out_f16, total_rows, st);
}

hipError_t launch_conv(const ConvArgs &a, int D, int in_kind, bool out_f16, int64_t total_rows, hipStream_t st)
{
    if (total_rows <= 0) return hipSuccess;
    switch (D) {
    case 16: return launch_dd<16>(a, in_kind, out_f16, total_rows, st);
    case 32: return launch_dd<32>(a, in_kind, out_f16, total_rows, st);
    case 64: return launch_dd<64>(a, in_kind, out_f16, total_rows, st);
    case 128: return launch_dd<128>(a, in_kind, out_f16, total_rows, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hy

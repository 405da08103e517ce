// conv.hip -- depthwise causal conv of the key / value rows a segment build
// reads, with optional key L2 normalisation, into a packed fp32 workspace
// (HYPIC reading notes ch.2 sec.6: the QKV path's width-k causal conv; a
// segment prefilled on its own sees zeros before its first row).
//   y[t][c] = sum_{j<W} w[c][j] * x[t - W + 1 + j][c],  rows before `from` read 0
// One wave per (row, head).
#include "common.h"
#include "launch.h"

namespace hy {

template <int D, typename TIN>
__global__ void __launch_bounds__(256) conv_kernel(const ConvArgs a, int64_t total_pairs)
{
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= total_pairs) return;
    const int64_t prow = pair / a.H;
    const int hh = (int)(pair % a.H);
    // segment of this packed row (binary search in the launch table)
    int lo = 0, hi = a.n_seg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.out0[mid] <= prow) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const int64_t t = prow - a.out0[s];
    const int64_t row = a.tok0[s] + t;
    const TIN *x = reinterpret_cast<const TIN *>(a.x);
    const int64_t ld = (int64_t)a.H * D;
    constexpr int PER = D >= 64 ? D / 64 : 1;
    float y[PER];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int d = lane + 64 * q;
        float acc = 0.f;
        if (d < D) {
            const int64_t col = (int64_t)hh * D + d;
            if (a.W > 0) {
                for (int j = 0; j < a.W; ++j) {
                    const int64_t r = row - (a.W - 1) + j;
                    if (r >= a.from[s]) acc += a.w[col * a.W + j] * ld1(x + r * ld + col);
                }
            } else {
                acc = ld1(x + row * ld + col);
            }
        }
        y[q] = acc;
        ss += acc * acc;
    }
    float sc = 1.f;
    if (a.l2norm) {
        ss = wave_sum(ss);
        sc = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
    }
    float *out = a.out + prow * ld + (int64_t)hh * D;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int d = lane + 64 * q;
        if (d < D) out[d] = y[q] * sc;
    }
}

template <int D>
static hipError_t launch_d(const ConvArgs &a, int in_kind, int64_t total_rows, hipStream_t st)
{
    const int64_t pairs = total_rows * a.H;
    const int64_t blocks = (pairs + 3) / 4;
    if (in_kind == IN_BF16)
        hipLaunchKernelGGL((conv_kernel<D, bf16_t>), dim3((unsigned)blocks), dim3(256), 0, st, a, pairs);
    else
        hipLaunchKernelGGL((conv_kernel<D, float>), dim3((unsigned)blocks), dim3(256), 0, st, a, pairs);
    return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs &a, int D, int in_kind, int64_t total_rows, hipStream_t st)
{
    if (total_rows <= 0) return hipSuccess;
    switch (D) {
    case 16: return launch_d<16>(a, in_kind, total_rows, st);
    case 32: return launch_d<32>(a, in_kind, total_rows, st);
    case 64: return launch_d<64>(a, in_kind, total_rows, st);
    case 128: return launch_d<128>(a, in_kind, total_rows, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hy

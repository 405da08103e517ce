// rope.hip -- rotary re-rotation on the reuse path (HYPIC reading notes,
// ch.2 sec.6): cached full-attention keys stored from a zero start are moved
// to their positions in the request, K_b = R(b - a) K_a (Eq. (8)), and the
// state of a scalar-transition linear layer moves the same way,
// S_{C|b} = R(b - a) S_{C|a} along its key dimension (Eq. (7)).
//
// R(delta) turns pair i of the leading rot_dim entries by delta * theta_i,
// theta_i = base^(-2i / rot_dim); pairs are (i, i + rot_dim/2) or (2i, 2i + 1).
// The angles are formed and reduced modulo 2 pi in fp64 once per thread, so a
// shift of 1e5 positions keeps the fp32 rounding of cos and sin.  Both kernels
// are HBM-bound: every element is read once and written once.
#include "common.h"
#include "launch.h"

namespace hy {

// cos and sin of delta * base^(-2i / rot), the angle reduced to [-pi, pi] in fp64
__device__ __forceinline__ void rope_cs(double delta, double log2_base, int i, int rot, float &c, float &s)
{
    const double th = delta * exp2(-2.0 * (double)i / (double)rot * log2_base);
    const double two_pi = 6.283185307179586476925286766559;
    const double r = th - two_pi * rint(th / two_pi);
    double sd, cd;
    sincos(r, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
}

__device__ __forceinline__ void rot2(float &x1, float &x2, float c, float s)
{
    const float a = x1 * c - x2 * s, b = x1 * s + x2 * c;
    x1 = a;
    x2 = b;
}

// 4 consecutive elements <-> fp32
__device__ __forceinline__ void ld4(const float *p, float (&x)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void st4(float *p, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void ld4(const bf16_t *p, float (&x)[4]) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
    const uint16_t a = __builtin_bit_cast(uint16_t, (__bf16)lo), b = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return (uint32_t)a | ((uint32_t)b << 16);
}
__device__ __forceinline__ void st4(bf16_t *p, const float (&x)[4]) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(bf16x2(x[0], x[1]), bf16x2(x[2], x[3]));
}

// Keys: rows (token, head) of length d; thread (slot, q) turns pairs 4q .. 4q+3
// of one row per step and copies pass-through chunks q, q + G, ... of it.
template <typename T, bool HALF>
__global__ void __launch_bounds__(256) rope_keys_kernel(const RopeArgs a)
{
    const int seg = blockIdx.y;
    const int G = a.rot / 8, rpi = 256 / G;
    const int tid = threadIdx.x, slot = tid / G, q = tid % G;
    if (slot >= rpi) return;   // threads past the last whole row slot
    const int64_t rows = a.len[seg] * (int64_t)a.h;
    const int half = a.rot / 2;
    float c[4], s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rope_cs((double)a.delta[seg], a.log2_base, 4 * q + e, a.rot, c[e], s[e]);
    const T *xi = reinterpret_cast<const T *>(a.x_in);
    T *xo = reinterpret_cast<T *>(a.x_out);
    const int npass = a.copy_rest ? (a.d - a.rot) / 4 : 0;
    for (int64_t r = (int64_t)blockIdx.x * rpi + slot; r < rows; r += (int64_t)gridDim.x * rpi) {
        const int64_t o = (a.start[seg] * a.h + r) * a.d;
        float x1[4], x2[4];
        if constexpr (HALF) {
            ld4(xi + o + 4 * q, x1);
            ld4(xi + o + half + 4 * q, x2);
#pragma unroll
            for (int e = 0; e < 4; ++e) rot2(x1[e], x2[e], c[e], s[e]);
            st4(xo + o + 4 * q, x1);
            st4(xo + o + half + 4 * q, x2);
        } else {
            ld4(xi + o + 8 * q, x1);          // pairs (8q, 8q+1), (8q+2, 8q+3)
            ld4(xi + o + 8 * q + 4, x2);      // pairs (8q+4, 8q+5), (8q+6, 8q+7)
            rot2(x1[0], x1[1], c[0], s[0]);
            rot2(x1[2], x1[3], c[1], s[1]);
            rot2(x2[0], x2[1], c[2], s[2]);
            rot2(x2[2], x2[3], c[3], s[3]);
            st4(xo + o + 8 * q, x1);
            st4(xo + o + 8 * q + 4, x2);
        }
        for (int k = q; k < npass; k += G) {
            float y[4];
            ld4(xi + o + a.rot + 4 * k, y);
            st4(xo + o + a.rot + 4 * k, y);
        }
    }
}

// State [h, d_k, d_v] fp32, turned along d_k: thread (head, pair i, column
// chunk j) turns rows (i, i + rot/2) or (2i, 2i + 1) at columns 4j .. 4j+3;
// rows past rot are copied when the output is another array.
template <bool HALF>
__global__ void __launch_bounds__(256) rope_state_kernel(const RopeStateArgs a)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nj = a.d_v / 4, half = a.rot / 2;
    const int64_t npair = (int64_t)a.h * half * nj;
    const float *Si = a.S_in;
    float *So = a.S_out;
    if (idx < npair) {
        const int j = (int)(idx % nj);
        const int i = (int)((idx / nj) % half);
        const int hh = (int)(idx / ((int64_t)nj * half));
        float c, s;
        rope_cs((double)a.delta, a.log2_base, i, a.rot, c, s);
        const int ra = HALF ? i : 2 * i, rb = HALF ? i + half : 2 * i + 1;
        const int64_t base = (int64_t)hh * a.d_k * a.d_v + 4 * j;
        float x1[4], x2[4];
        ld4(Si + base + (int64_t)ra * a.d_v, x1);
        ld4(Si + base + (int64_t)rb * a.d_v, x2);
#pragma unroll
        for (int e = 0; e < 4; ++e) rot2(x1[e], x2[e], c, s);
        st4(So + base + (int64_t)ra * a.d_v, x1);
        st4(So + base + (int64_t)rb * a.d_v, x2);
    } else if (a.copy_rest) {
        const int64_t k = idx - npair;
        const int rest = a.d_k - a.rot;
        if (k < (int64_t)a.h * rest * nj) {
            const int j = (int)(k % nj);
            const int row = a.rot + (int)((k / nj) % rest);
            const int hh = (int)(k / ((int64_t)nj * rest));
            const int64_t off = ((int64_t)hh * a.d_k + row) * a.d_v + 4 * j;
            float y[4];
            ld4(Si + off, y);
            st4(So + off, y);
        }
    }
}

hipError_t launch_rope_keys(const RopeArgs &a, int dtype_bf16, int n_seg, hipStream_t st)
{
    const int G = a.rot / 8, rpi = 256 / G;
    int64_t maxrows = 0;
    for (int i = 0; i < n_seg; ++i) {
        const int64_t r = a.len[i] * (int64_t)a.h;
        maxrows = r > maxrows ? r : maxrows;
    }
    if (maxrows == 0) return hipSuccess;
    // up to ~2048 workgroups over the launch (8 per CU), each looping over rows
    const int64_t want = (maxrows + rpi - 1) / rpi, cap = n_seg < 2048 ? 2048 / n_seg : 1;
    const dim3 grid((unsigned)(want < cap ? want : cap), (unsigned)n_seg);
    if (dtype_bf16) {
        if (a.pairing == 0) hipLaunchKernelGGL((rope_keys_kernel<bf16_t, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((rope_keys_kernel<bf16_t, false>), grid, dim3(256), 0, st, a);
    } else {
        if (a.pairing == 0) hipLaunchKernelGGL((rope_keys_kernel<float, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((rope_keys_kernel<float, false>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_rope_state(const RopeStateArgs &a, hipStream_t st)
{
    const int64_t total = (int64_t)a.h * (a.rot / 2) * (a.d_v / 4) +
                          (a.copy_rest ? (int64_t)a.h * (a.d_k - a.rot) * (a.d_v / 4) : 0);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (a.pairing == 0) hipLaunchKernelGGL((rope_state_kernel<true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((rope_state_kernel<false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace hy

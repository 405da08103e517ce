// common.h -- device helpers shared by the gfx950 kernels of libhypic.
//
// Matrix-core fragments (wave64, 16x16 output tiles), as used throughout:
//   16x16x32 f16/bf16 : lane l holds A[l&15][k(l>>4, e)], B[k(l>>4, e)][l&15], e = 0..7
//   16x16x4  f32      : lane l holds A[l&15][k(l>>4)],    B[k(l>>4)][l&15]
//   accumulator       : lane l, register i holds D[4*(l>>4) + i][l&15]
// The reduction index k only has to agree between A and B, so every product
// picks the k-order that makes its operands cheap to fetch:
//   natural     k = 8g + e (16x16x32) or k = g*(K/4) + s (16x16x4, step s),
//   from-acc    a B operand taken straight from two accumulator tiles of the
//               previous product: k = 4g + (e & 3) + 16*(e >> 2); for 16x16x4,
//               step (tile t, register i) has k = 16t + 4g + i.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

struct bf16_t { uint16_t bits; };   // storage type of bf16 inputs

__device__ __forceinline__ f4 mma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma(b8 a, b8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// ---- input element access (bf16 inputs are widened exactly) ----------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }
__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const bf16_t *p) { return to_f32(*p); }

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for f32)
__device__ __forceinline__ void ld8(const bf16_t *p, float (&x)[8]) {
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void ld8(const float *p, float (&x)[8]) {
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Raw 8-element vectors as loaded from global memory; widened when staged,
// so a register prefetch does not wait for its data at the load.
struct raw8_bf16 { uint4 u; };
struct raw8_f16 { uint4 u; };
struct raw8_f32 { float4 a, b; };
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> { typedef raw8_bf16 type; };
template <> struct Raw8<_Float16> { typedef raw8_f16 type; };
template <> struct Raw8<float> { typedef raw8_f32 type; };
__device__ __forceinline__ void ld_raw8(const _Float16 *p, raw8_f16 &r) { r.u = *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void mask_raw8(raw8_f16 &r, bool keep) {
    r.u = make_uint4(keep ? r.u.x : 0u, keep ? r.u.y : 0u, keep ? r.u.z : 0u, keep ? r.u.w : 0u);
}
__device__ __forceinline__ void widen8(const raw8_f16 &r, float (&x)[8]) {
    const h8 v = __builtin_bit_cast(h8, r.u);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}

__device__ __forceinline__ void ld_raw8(const bf16_t *p, raw8_bf16 &r) { r.u = *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void ld_raw8(const float *p, raw8_f32 &r) {
    r.a = reinterpret_cast<const float4 *>(p)[0];
    r.b = reinterpret_cast<const float4 *>(p)[1];
}
__device__ __forceinline__ void zero_raw8(raw8_bf16 &r) { r.u = make_uint4(0u, 0u, 0u, 0u); }
__device__ __forceinline__ void zero_raw8(raw8_f32 &r) { r.a = make_float4(0.f, 0.f, 0.f, 0.f); r.b = r.a; }
// zero a raw row piece (rows past a segment end are loaded clamped, then zeroed)
__device__ __forceinline__ void mask_raw8(raw8_bf16 &r, bool keep) {
    r.u = make_uint4(keep ? r.u.x : 0u, keep ? r.u.y : 0u, keep ? r.u.z : 0u, keep ? r.u.w : 0u);
}
__device__ __forceinline__ void mask_raw8(raw8_f32 &r, bool keep) {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    r.a = keep ? r.a : z;
    r.b = keep ? r.b : z;
}
__device__ __forceinline__ void widen8(const raw8_bf16 &r, float (&x)[8]) {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen8(const raw8_f32 &r, float (&x)[8]) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip, each with
// its own L2.  Remap the hardware block id so that consecutive logical ids run
// on one XCD (they then share operands through that L2).  Identity when the
// grid is not a multiple of 8.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
    if (nblocks % 8 != 0) return b;
    return (b % 8) * (nblocks / 8) + b / 8;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// and meets the other waves, but leaves global loads in flight, so register
// prefetches issued before it keep streaming.  (The full __syncthreads also
// drains every outstanding global load.)  The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- bf16 hi/lo split of an fp32 value (x ~= hi + lo, |x - hi - lo| <~ 2^-17|x|)
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// ---- wave64 reductions and scans -------------------------------------------
// Within each 16-lane row by DPP lane moves (plain VALU operations), across the
// four rows through lane reads into scalar registers.
//   DPP controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror
//   0x141, row_mirror 0x140, row_shl:n 0x100+n and row_shr:n 0x110+n (zero fill).
#define HY_DPP(x, ctrl) __builtin_amdgcn_update_dpp(0.f, (x), (ctrl), 0xf, 0xf, true)
__device__ __forceinline__ float lane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, HY_DPP(x, 0xB1));
    x = fmaxf(x, HY_DPP(x, 0x4E));
    x = fmaxf(x, HY_DPP(x, 0x141));
    x = fmaxf(x, HY_DPP(x, 0x140));
    return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += HY_DPP(x, 0xB1);
    x += HY_DPP(x, 0x4E);
    x += HY_DPP(x, 0x141);
    x += HY_DPP(x, 0x140);
    return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
// exclusive suffix sum over the 64 lanes: returns sum_{j > lane} x_j
__device__ __forceinline__ float wave_suffix_excl(float x) {
    float s = x;   // inclusive suffix within the row: lane i <- sum of lanes i..15
    s += HY_DPP(s, 0x101);
    s += HY_DPP(s, 0x102);
    s += HY_DPP(s, 0x104);
    s += HY_DPP(s, 0x108);
    const float t1 = lane_f(s, 16), t2 = lane_f(s, 32), t3 = lane_f(s, 48);   // row totals
    const int row = (threadIdx.x & 63) >> 4;
    const float later = (row < 1 ? t1 : 0.f) + (row < 2 ? t2 : 0.f) + (row < 3 ? t3 : 0.f);
    return (s + later) - x;
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ float wave_prefix_incl(float x) {
    float s = x;   // inclusive prefix within the row: lane i <- sum of lanes 0..i
    s += HY_DPP(s, 0x111);
    s += HY_DPP(s, 0x112);
    s += HY_DPP(s, 0x114);
    s += HY_DPP(s, 0x118);
    const float t0 = lane_f(s, 15), t1 = lane_f(s, 31), t2 = lane_f(s, 47);   // row totals
    const int row = (threadIdx.x & 63) >> 4;
    const float earlier = (row > 0 ? t0 : 0.f) + (row > 1 ? t1 : 0.f) + (row > 2 ? t2 : 0.f);
    return s + earlier;
}

// ---- 16 x 16 unit lower triangular solve, one column per lane -------------
// x_r += (value of nv in lane Q of this lane's 16-lane row) * x_q: the row
// broadcast rides on the multiply-add.  The caller keeps two wait states
// between the last write of nv and the first use here (a lane move reads its
// source register that late).
template <int Q>
__device__ __forceinline__ void fmac_rowbcast(float &acc, float nv, float xq)
{
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc) : "v"(nv), "v"(xq), "n"(Q));
}
// forward substitution steps Q..14: x_r += N_r[lane Q] x_Q for r > Q
template <int Q>
__device__ __forceinline__ void subst_steps(float (&x)[16], const float (&n)[16])
{
#pragma unroll
    for (int r = Q + 1; r < 16; ++r) fmac_rowbcast<Q>(x[r], n[r], x[Q]);
    if constexpr (Q < 14) subst_steps<Q + 1>(x, n);
}

// Power-of-two exponent that brings m (>= 0) into [0.5, 1); 0 for m == 0 or non-finite.
__device__ __forceinline__ int pow2_exponent(float m) {
    if (!(m > 0.f) || !(m < INFINITY)) return 0;
    int e;
    (void)frexpf(m, &e);
    return e;
}

// 2^e * x for a double exponent e, exact split into integer and fraction;
// underflows to (signed) zero below the float range.
__device__ __forceinline__ float scale_pow2(float x, double e) {
    if (e < -400.0) return 0.f * x;
    double fl = floor(e);
    float fr = (float)(e - fl);
    return ldexpf(x * exp2f(fr), (int)fl);
}

}  // namespace hy

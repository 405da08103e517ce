// build_decay.hip -- cached pair of the decay family T_i = gate_i (scalar
// gamma I, per-token a_i I, or diag(g_i)), u_i = k_i v_i^T (HYPIC reading
// notes, ch.2 sec.3 Tables 1 and 3: the cached T_C is then a scalar or a d_k
// vector).  From the pair definition (ch.2 sec.2), with dec_t the product of
// the gates after token t,
//   S_{C|0} = sum_t diag(dec_t) k_t v_t^T = (K * dec)^T V,   T_C = prod_t gate_t,
// a decay-weighted contraction over the tokens.  The kernel streams the
// segment in chunks of 64 tokens, S <- diag(chunk product) S + Khat^T V with
// Khat = K * (gate product over the rest of the chunk), so every factor is a
// suffix product (<= 1).  One workgroup per (segment, head, 64-column group);
// operands bf16 with the computed Khat split into hi + lo (V exact), or fp32.
#include "common.h"
#include "launch.h"

namespace hy {

template <int D, bool SPLIT>
struct DecayCfg {
    static constexpr int NC = D < 64 ? D : 64;    // value columns per workgroup
    static constexpr int NW = NC / 16;            // waves, one 16-column tile each
    static constexpr int NT = 64 * NW;
    static constexpr int MT = D / 16;
    static constexpr int P = NT / D;              // token parts per key dim in the scan
    static constexpr int TP = 64 / P;             // tokens per part
    static constexpr int LDT = 64 + 8;
};

template <int D, bool SPLIT>
struct DecaySmem {
    using C = DecayCfg<D, SPLIT>;
    typedef typename std::conditional<SPLIT, __bf16, float>::type AT;
    AT KhT[D][C::LDT];                 // Khat, dim-major (hi part when split)
    AT KlT[SPLIT ? D : 1][C::LDT];     // lo part of Khat
    AT VT[C::NC][C::LDT];              // values of this column group, column-major
    float part_tot[C::P][D];           // log2 gate totals per token part
    float gam[D];                      // chunk gate product per key dim
};

template <int D, bool SPLIT, typename TIN>
__global__ void __launch_bounds__((DecayCfg<D, SPLIT>::NT))
build_decay_kernel(const DecayArgs a)
{
    using C = DecayCfg<D, SPLIT>;
    using AT = typename DecaySmem<D, SPLIT>::AT;
    constexpr int NC = C::NC, MT = C::MT, P = C::P, TP = C::TP;
    __shared__ __align__(16) DecaySmem<D, SPLIT> sm;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int ngrp = D / NC;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);   // column groups of a unit share an XCD
    const int unit = lb / ngrp, grp = lb % ngrp;
    const int s = unit / a.h_v, h = unit % a.h_v;
    const int kh = h / (a.h_v / a.h_k);
    const int len = a.len[s];
    const int c0 = grp * NC;
    const TIN *kp = reinterpret_cast<const TIN *>(a.k) + (a.tok0[s] * a.h_k + kh) * D;
    const TIN *vp = reinterpret_cast<const TIN *>(a.v) + (a.tok0[s] * a.h_v + h) * D + c0;
    const int64_t ldk = (int64_t)a.h_k * D, ldv = (int64_t)a.h_v * D;

    // gate source: scan thread (d, part)
    const int d = tid % D, part = tid / D;
    float l2c = 0.f;   // log2 gamma for a per-head constant gate
    if (a.gate_kind == HYPIC_GATE_HEAD_CONST) l2c = log2f(reinterpret_cast<const float *>(a.gate)[h]);
    const TIN *gp = nullptr;
    int64_t ldg = 0;
    if (a.gate_kind == HYPIC_GATE_DIAG) {
        gp = reinterpret_cast<const TIN *>(a.gate) + (a.tok0[s] * a.h_v + h) * D + d;
        ldg = (int64_t)a.h_v * D;
    } else if (a.gate_kind == HYPIC_GATE_SCALAR) {
        gp = reinterpret_cast<const TIN *>(a.gate) + a.tok0[s] * a.h_v + h;
        ldg = a.h_v;
    }

    // prefetch registers (raw input words): keys and gates of (d, part), values
    // 8 columns x VPASS rows.  Rows are loaded clamped into the segment and masked
    // when used, so the loads carry no branches and the compiler waits for them
    // only where the values are consumed, a chunk later.
    TIN kr[TP], gr[TP];
    constexpr int CPR = NC / 8;
    const int vrow = tid / CPR, vcol = 8 * (tid % CPR);
    constexpr int VROWS = C::NT / CPR;          // rows per pass
    constexpr int VPASS = 64 / VROWS;
    typename Raw8<TIN>::type vraw[VPASS];
    const unsigned ldk32 = (unsigned)ldk, ldv32 = (unsigned)ldv, ldg32 = (unsigned)ldg;
    auto fetch = [&](int c) {
        const int last = len - 1 - 64 * c;      // >= 0 for every chunk of the segment
        const TIN *kc = kp + (int64_t)(64 * c) * ldk + d;
#pragma unroll
        for (int j = 0; j < TP; ++j) kr[j] = kc[__umul24(min(part * TP + j, last), ldk32)];
        if (gp) {
            const TIN *gc = gp + (int64_t)(64 * c) * ldg;
#pragma unroll
            for (int j = 0; j < TP; ++j) gr[j] = gc[__umul24(min(part * TP + j, last), ldg32)];
        }
        const TIN *vc = vp + (int64_t)(64 * c) * ldv + vcol;
#pragma unroll
        for (int p = 0; p < VPASS; ++p) ld_raw8(vc + __umul24(min(vrow + VROWS * p, last), ldv32), vraw[p]);
    };

    f4 S[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) S[mt] = zero4();
    double cl = 0.0;   // log2 of the gate product over the segment, per key dim d
    const int nch = (len + 63) / 64;
    if (nch > 0) fetch(0);

    for (int c = 0; c < nch; ++c) {
        lds_barrier();
        // log2-gates of this part (rows past the segment end: gate 1, key 0), and
        // their local suffix sums
        float run = 0.f;
        float sfx[TP];
#pragma unroll
        for (int j = TP - 1; j >= 0; --j) {
            const bool in = 64 * c + part * TP + j < len;
            const float lq = in ? (gp ? log2f(to_f32(gr[j])) : l2c) : 0.f;
            sfx[j] = run;
            run += lq;
        }
        sm.part_tot[part][d] = run;
#pragma unroll
        for (int p = 0; p < VPASS; ++p) {
            mask_raw8(vraw[p], 64 * c + vrow + VROWS * p < len);
            float vr[8];
            widen8(vraw[p], vr);
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.VT[vcol + e][vrow + VROWS * p] = (AT)vr[e];
        }
        lds_barrier();
        float off = 0.f, tot = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float x = sm.part_tot[p][d];
            if (p > part) off += x;
            tot += x;
        }
        if (part == 0) {
            double dt = 0.0;
#pragma unroll
            for (int p = 0; p < P; ++p) dt += (double)sm.part_tot[p][d];
            cl += dt;
            sm.gam[d] = scale_pow2(1.f, dt);
        }
#pragma unroll
        for (int j = 0; j < TP; ++j) {
            const bool in = 64 * c + part * TP + j < len;
            const float kh_ = (in ? to_f32(kr[j]) : 0.f) * exp2f(sfx[j] + off);
            const int t = part * TP + j;
            if constexpr (SPLIT) {
                __bf16 hi, lo;
                split_bf16(kh_, hi, lo);
                sm.KhT[d][t] = hi;
                sm.KlT[d][t] = lo;
            } else {
                sm.KhT[d][t] = kh_;
            }
        }
        (void)tot;
        if (c + 1 < nch) fetch(c + 1);
        lds_barrier();

        // S <- diag(gam) S + Khat^T V for this wave's 16 columns
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S[mt][i] *= sm.gam[16 * mt + 4 * g + i];
            if constexpr (SPLIT) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int k0 = 32 * kb + 8 * g;
                    const b8 Ah = *reinterpret_cast<const b8 *>(&sm.KhT[16 * mt + r16][k0]);
                    const b8 Al = *reinterpret_cast<const b8 *>(&sm.KlT[16 * mt + r16][k0]);
                    const b8 B = *reinterpret_cast<const b8 *>(&sm.VT[16 * w + r16][k0]);
                    S[mt] = mma(Ah, B, S[mt]);
                    S[mt] = mma(Al, B, S[mt]);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < 16; ++ks) {
                    const int k = 16 * g + ks;
                    S[mt] = mma((float)sm.KhT[16 * mt + r16][k], (float)sm.VT[16 * w + r16][k], S[mt]);
                }
            }
        }
    }

    float *Su = a.S0_out + (int64_t)unit * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Su[(16 * mt + 4 * g + i) * D + c0 + 16 * w + r16] = S[mt][i];
    if (grp == 0) {
        if (a.gate_kind == HYPIC_GATE_DIAG) {
            if (part == 0) a.T_out[(int64_t)unit * D + d] = scale_pow2(1.f, cl);
        } else if (tid == 0) {
            a.T_out[unit] = scale_pow2(1.f, cl);
        }
    }
}

template <int D, bool SPLIT, typename TIN>
static hipError_t launch_one(const DecayArgs &a, int n_units, hipStream_t st)
{
    using C = DecayCfg<D, SPLIT>;
    hipLaunchKernelGGL((build_decay_kernel<D, SPLIT, TIN>), dim3(n_units * (D / C::NC)),
                       dim3(C::NT), 0, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const DecayArgs &a, int in_kind, int n_units, hipStream_t st)
{
    if (in_kind == IN_BF16) return launch_one<D, true, bf16_t>(a, n_units, st);
    return launch_one<D, false, float>(a, n_units, st);
}

hipError_t launch_build_decay(const DecayArgs &a, int D, int in_kind, int n_units, hipStream_t st)
{
    switch (D) {
    case 16: return launch_d<16>(a, in_kind, n_units, st);
    case 32: return launch_d<32>(a, in_kind, n_units, st);
    case 64: return launch_d<64>(a, in_kind, n_units, st);
    case 128: return launch_d<128>(a, in_kind, n_units, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hy

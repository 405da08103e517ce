// build_delta.hip -- chunkwise build of the cached pair (T_C, S_{C|0}) for the
// gated-delta family T_i = a_i (I - b_i k_i k_i^T), u_i = b_i k_i v_i^T
// (HYPIC reading notes, ch.2 sec.3 Table 1; pair definition ch.2 sec.2; the
// pages build it by running the recurrence twice, from S_0 = 0 with the writes
// and from S_0 = I without them, ch.2 sec.4).
//
// Here both runs are one pass over the segment in chunks of b = 64 tokens,
// carrying X = [Tbar | S] (d_k x 2d) in matrix-core accumulators.  The scalar
// gate factors out of the transition, T_C = (prod a_i) Tbar with Tbar the
// gate-free product of (I - b_i k_i k_i^T).  Within a chunk, with
//   G = K K^T, M = (I + diag(b) strictlower(G))^-1   (unit lower triangular),
//   W = M diag(b) K,  U = M diag(b * dec) V,  dec_t = prod_{s>t} a_s, g_b = prod a,
// the exact chunk update (compact WY / UT representation of the product of
// the rank-one factors) is
//   Tbar <- Tbar - K^T (W Tbar)
//   S    <- g_b S;   S <- S + K^T (U - W S)
// Every exponent applied is a decay over a suffix (<= 1), so no gate ratio
// can overflow.  Per chunk: Gram and triangular inverse in LDS, then four
// matrix-core products.  Operands are fp16 (bf16 inputs, with power-of-two
// block scaling of every computed operand) or fp32 (fp32 inputs).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace hy {

template <int D, bool F16>
struct DeltaCfg {
    static constexpr int MT = D / 16;         // 16-row tiles of the state
    static constexpr int NW = D / 16;         // waves; wave w owns column tiles 2w, 2w+1 of X
    static constexpr int NT = 64 * NW;
    static constexpr int KB = D >= 32 ? D / 32 : 1;  // 32-wide k blocks over the state rows
    using OT = typename std::conditional<F16, _Float16, float>::type;
    static constexpr int LDK = D + 8;         // Ks row stride (halves)
    static constexpr int LDT = 64 + (F16 ? 8 : 4);
    static constexpr int LDW = D + (F16 ? 8 : 4);
    static constexpr int LDG = 68;
};

template <int D, bool F16>
struct DeltaSmem {
    using C = DeltaCfg<D, F16>;
    using OT = typename C::OT;
    OT Ks[F16 ? 64 : 1][C::LDK];   // keys, token-major (fp16 path)
    OT KT[D][C::LDT];              // keys, dim-major
    OT VT[D][C::LDT];              // values * 2^-sv, dim-major
    OT Wb[64][C::LDW];             // W = M diag(b) K
    float Gm[64][C::LDG];          // b_r k_r.k_s for s < r, else 0
    float Mm[64][C::LDG];          // M = (I + Gm)^-1
    float beta[64];
    float bd[64];                  // b_t * dec_t
    float wmax[16];
    double chunk_l2;               // log2 of the chunk's gate product
};

// Gram tiles on or below the diagonal of the 4x4 token-tile grid
__constant__ int kGramTi[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kGramTj[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <typename T>
__device__ __forceinline__ const T *typed(const void *p) { return reinterpret_cast<const T *>(p); }

template <int D, bool F16, typename TKV, typename TG>
__global__ void __launch_bounds__((DeltaCfg<D, F16>::NT))
build_delta_kernel(const DeltaArgs a)
{
    using C = DeltaCfg<D, F16>;
    using OT = typename C::OT;
    constexpr int MT = C::MT, NW = C::NW, KB = C::KB;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    DeltaSmem<D, F16> &sm = *reinterpret_cast<DeltaSmem<D, F16> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int unit = xcd_logical_block(blockIdx.x, gridDim.x);   // value heads of one key head share an XCD
    const int s = unit / a.h_v, h = unit % a.h_v;
    const int kh = h / (a.h_v / a.h_k);
    const int len = a.len[s];
    const TKV *kp = typed<TKV>(a.k) + a.tok0[s] * a.ldk + (int64_t)kh * D;
    const TKV *vp = typed<TKV>(a.v) + a.tok0[s] * a.ldv + (int64_t)h * D;
    const TG *bp = typed<TG>(a.beta) + a.gtok0[s] * a.h_v + h;
    const TG *ap = typed<TG>(a.alpha) + a.gtok0[s] * a.h_v + h;

    // upper tile blocks of M are never written: zero them once
    for (int idx = tid; idx < 64 * 64; idx += C::NT) {
        int r = idx >> 6, c = idx & 63;
        if ((c >> 4) > (r >> 4)) sm.Mm[r][c] = 0.f;
    }

    // state X = [Tbar | S] in accumulator layout: X[mt][jn] is rows 16mt.., column tile 2w+jn
    f4 X[MT][2];
    int sig[2] = {0, 0};     // X = 2^sig * Xhat per column tile (fp16 path)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int n = 2 * w + jn;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                X[mt][jn][i] = (n < MT && 16 * mt + 4 * g + i == 16 * n + r16) ? 1.f : 0.f;
    }

    // register prefetch of one chunk (kept raw until staged): rows prow and
    // prow + 32, columns pcol..pcol+7
    constexpr int CPR = D / 8;
    const int prow = tid / CPR, pcol = 8 * (tid % CPR);
    typename Raw8<TKV>::type kraw[2], vraw[2];
    float br = 0.f, ar = 1.f;
    auto fetch = [&](int c) {
        const int t0 = 64 * c;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int t = t0 + prow + 32 * p;
            if (t < len) {
                ld_raw8(kp + (int64_t)t * a.ldk + pcol, kraw[p]);
                ld_raw8(vp + (int64_t)t * a.ldv + pcol, vraw[p]);
            } else {
                zero_raw8(kraw[p]);
                zero_raw8(vraw[p]);
            }
        }
        if (w == 0) {
            const int t = t0 + lane;
            if (t < len) {
                br = ld1(bp + (int64_t)t * a.h_v);
                ar = ld1(ap + (int64_t)t * a.h_v);
            } else {
                br = 0.f;
                ar = 1.f;
            }
        }
    };
    float kr[2][8], vr[2][8];

    const int nch = (len + 63) / 64;
    double cl_lane = 0.0;  // wave 0: log2 of the gate product of this lane's tokens, all chunks
    if (nch > 0) fetch(0);

    for (int c = 0; c < nch; ++c) {
        lds_barrier();   // readers of the previous chunk are done

        // ---- stage the chunk: keys, gates ---------------------------------
        {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                widen8(kraw[p], kr[p]);
                widen8(vraw[p], vr[p]);
            }
            float vm = 0.f;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int t = prow + 32 * p;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    vm = fmaxf(vm, fabsf(vr[p][e]));
                    sm.KT[pcol + e][t] = (OT)kr[p][e];
                }
                if constexpr (F16) {
                    h8 kk;
#pragma unroll
                    for (int e = 0; e < 8; ++e) kk[e] = (_Float16)kr[p][e];
                    *reinterpret_cast<h8 *>(&sm.Ks[t][pcol]) = kk;
                }
            }
            vm = wave_max(vm);
            if (lane == 0) sm.wmax[w] = vm;
            if (w == 0) {
                const float l2 = log2f(ar);
                const float sfx = wave_suffix_excl(l2);    // log2 prod_{s>t} a_s
                cl_lane += (double)l2;
                sm.beta[lane] = br;
                sm.bd[lane] = br * exp2f(sfx);
                if (lane == 0) sm.chunk_l2 = (double)(sfx + l2);   // whole-chunk total
            }
        }
        lds_barrier();

        // ---- values (scaled), Gram ------------------------------------------
        int sv = 0;
        {
            float vm = 0.f;
            for (int i = 0; i < NW; ++i) vm = fmaxf(vm, sm.wmax[i]);
            if constexpr (F16) sv = pow2_exponent(vm);
            const float vsc = ldexpf(1.f, -sv);
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.VT[pcol + e][prow + 32 * p] = (OT)(vr[p][e] * vsc);
        }
        const float gb = scale_pow2(1.f, sm.chunk_l2);
        if (c + 1 < nch) fetch(c + 1);

        for (int q = w; q < 10; q += NW) {
            const int ti = kGramTi[q], tj = kGramTj[q];
            f4 acc = zero4();
            if constexpr (F16) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    h8 A, B;
                    if (D >= 32 || g < 2) {
                        A = *reinterpret_cast<const h8 *>(&sm.Ks[16 * ti + r16][32 * kb + 8 * g]);
                        B = *reinterpret_cast<const h8 *>(&sm.Ks[16 * tj + r16][32 * kb + 8 * g]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) { A[e] = 0; B[e] = 0; }
                    }
                    acc = mma(A, B, acc);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < D / 4; ++ks) {
                    const int k = g * (D / 4) + ks;
                    acc = mma((float)sm.KT[k][16 * ti + r16], (float)sm.KT[k][16 * tj + r16], acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * ti + 4 * g + i, cc = 16 * tj + r16;
                sm.Gm[rr][cc] = (cc < rr) ? sm.beta[rr] * acc[i] : 0.f;
            }
        }
        lds_barrier();

        // ---- M = (I + Gm)^-1: diagonal 16x16 blocks by forward substitution ----
        if (w == 0) {
            const int o = 16 * (lane >> 4), cc = lane & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == cc) ? 1.f : 0.f;
#pragma unroll
                for (int q = 0; q < r; ++q) acc -= sm.Gm[o + r][o + q] * x[q];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.Mm[o + r][o + cc] = x[r];
        }
        lds_barrier();
        // 32x32 blocks: M10 = -M11 (L10 M00)
        for (int p = w; p < 2; p += NW) {
            const int o0 = 32 * p, o1 = 32 * p + 16;
            f4 y = zero4();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int k = 4 * g + ks;
                y = mma(sm.Gm[o1 + r16][o0 + k], sm.Mm[o0 + k][o0 + r16], y);
            }
            f4 m = zero4();
#pragma unroll
            for (int i = 0; i < 4; ++i) m = mma(sm.Mm[o1 + r16][o1 + 4 * g + i], y[i], m);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.Mm[o1 + 4 * g + i][o0 + r16] = -m[i];
        }
        lds_barrier();
        // 64x64: rows 32..63, columns of tile tj: M[hi][lo] = -M[hi][hi] (L[hi][lo] M[lo][lo])
        for (int tj = w; tj < 2; tj += NW) {
            f4 y2 = zero4(), y3 = zero4();
            for (int tk = tj; tk < 2; ++tk) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int k = 4 * g + ks;
                    const float bm = sm.Mm[16 * tk + k][16 * tj + r16];
                    y2 = mma(sm.Gm[32 + r16][16 * tk + k], bm, y2);
                    y3 = mma(sm.Gm[48 + r16][16 * tk + k], bm, y3);
                }
            }
            f4 m2 = zero4(), m3 = zero4();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                m2 = mma(sm.Mm[32 + r16][32 + 4 * g + i], y2[i], m2);
                m3 = mma(sm.Mm[48 + r16][32 + 4 * g + i], y2[i], m3);
                m3 = mma(sm.Mm[48 + r16][48 + 4 * g + i], y3[i], m3);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sm.Mm[32 + 4 * g + i][16 * tj + r16] = -m2[i];
                sm.Mm[48 + 4 * g + i][16 * tj + r16] = -m3[i];
            }
        }
        lds_barrier();

        // ---- W = M diag(b) K: wave w produces key-column tile w ---------------
        {
            const int td = w;
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f4 acc = zero4();
                if constexpr (F16) {
                    const int kbmax = (16 * ti + 15) / 32;
                    for (int kb = 0; kb <= kbmax; ++kb) {
                        h8 A;
                        const int k0 = 32 * kb + 8 * g;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            A[e] = (_Float16)(sm.Mm[16 * ti + r16][k0 + e] * sm.beta[k0 + e]);
                        const h8 B = *reinterpret_cast<const h8 *>(&sm.KT[16 * td + r16][k0]);
                        acc = mma(A, B, acc);
                    }
                } else {
#pragma unroll
                    for (int ks = 0; ks < 16; ++ks) {
                        const int k = 16 * g + ks;
                        acc = mma(sm.Mm[16 * ti + r16][k] * sm.beta[k],
                                  (float)sm.KT[16 * td + r16][k], acc);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.Wb[16 * ti + 4 * g + i][16 * td + r16] = (OT)acc[i];
            }
        }
        lds_barrier();

        // ---- state update of this wave's two column tiles ----------------------
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int n = 2 * w + jn;
            const bool isS = n >= MT;
            if (isS) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) X[mt][jn] *= gb;
            }
            f4 E[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) E[ti] = zero4();
            if (isS) {   // E = U (value columns of this tile), in units of 2^sig
                const int cc = 16 * (n - MT);
                const float usc = F16 ? ldexpf(1.f, sv - sig[jn]) : 1.f;
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    f4 acc = zero4();
                    if constexpr (F16) {
                        const int kbmax = (16 * ti + 15) / 32;
                        for (int kb = 0; kb <= kbmax; ++kb) {
                            h8 A;
                            const int k0 = 32 * kb + 8 * g;
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                A[e] = (_Float16)(sm.Mm[16 * ti + r16][k0 + e] * sm.bd[k0 + e]);
                            const h8 B = *reinterpret_cast<const h8 *>(&sm.VT[cc + r16][k0]);
                            acc = mma(A, B, acc);
                        }
                    } else {
#pragma unroll
                        for (int ks = 0; ks < 16; ++ks) {
                            const int k = 16 * g + ks;
                            acc = mma(sm.Mm[16 * ti + r16][k] * sm.bd[k],
                                      (float)sm.VT[cc + r16][k], acc);
                        }
                    }
                    E[ti] = acc * usc;
                }
            }
            // E -= W Xhat
            if constexpr (F16) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    h8 B;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        B[i] = (_Float16)(-X[2 * kb][jn][i]);
                        B[4 + i] = (D >= 32) ? (_Float16)(-X[(2 * kb + 1) % MT][jn][i]) : (_Float16)0;
                    }
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) {
                        h8 A;
                        const h4 lo = *reinterpret_cast<const h4 *>(&sm.Wb[16 * ti + r16][32 * kb + 4 * g]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) A[e] = lo[e];
                        if (D >= 32) {
                            const h4 hi = *reinterpret_cast<const h4 *>(&sm.Wb[16 * ti + r16][32 * kb + 16 + 4 * g]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) A[4 + e] = hi[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) A[4 + e] = 0;
                        }
                        E[ti] = mma(A, B, E[ti]);
                    }
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti)
                            E[ti] = mma((float)sm.Wb[16 * ti + r16][16 * mt + 4 * g + i], -X[mt][jn][i], E[ti]);
            }
            // X += K^T E
            if constexpr (F16) {
                float em = 0.f;
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int i = 0; i < 4; ++i) em = fmaxf(em, fabsf(E[ti][i]));
                const int tau = pow2_exponent(wave_max(em));
                const float esc = ldexpf(1.f, -tau);
                h8 Eb[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        Eb[kb][i] = (_Float16)(E[2 * kb][i] * esc);
                        Eb[kb][4 + i] = (_Float16)(E[2 * kb + 1][i] * esc);
                    }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    X[mt][jn] *= esc;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        h8 A;
                        const h4 lo = *reinterpret_cast<const h4 *>(&sm.KT[16 * mt + r16][32 * kb + 4 * g]);
                        const h4 hi = *reinterpret_cast<const h4 *>(&sm.KT[16 * mt + r16][32 * kb + 16 + 4 * g]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) { A[e] = lo[e]; A[4 + e] = hi[e]; }
                        X[mt][jn] = mma(A, Eb[kb], X[mt][jn]);
                    }
                }
                float xm = 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xm = fmaxf(xm, fabsf(X[mt][jn][i]));
                const int rho = pow2_exponent(wave_max(xm));
                const float xsc = ldexpf(1.f, -rho);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) X[mt][jn] *= xsc;
                sig[jn] += tau + rho;
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            X[mt][jn] = mma((float)sm.KT[16 * mt + r16][16 * ti + 4 * g + i], E[ti][i], X[mt][jn]);
            }
        }
    }

    // ---- outputs: T_C = 2^(sig + log2 prod a) Tbar, S_{C|0} = 2^sig Shat ------
    // the segment's gate product, summed in fp64 over every token
    if (w == 0) {
        const double tot = wave_sum_f64(cl_lane);
        if (lane == 0) sm.chunk_l2 = tot;
    }
    lds_barrier();
    const double cl_tot = sm.chunk_l2;
    float *Tu = a.T_out + (int64_t)unit * D * D;
    float *Su = a.S0_out + (int64_t)unit * D * D;
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int n = 2 * w + jn;
        const bool isS = n >= MT;
        const double e = (double)sig[jn] + (isS ? 0.0 : cl_tot);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * g + i;
                const float val = scale_pow2(X[mt][jn][i], e);
                if (isS) Su[row * D + 16 * (n - MT) + r16] = val;
                else     Tu[row * D + 16 * n + r16] = val;
            }
    }
}

template <int D, bool F16, typename TKV, typename TG>
static hipError_t launch_one(const DeltaArgs &a, int n_units, hipStream_t st)
{
    using C = DeltaCfg<D, F16>;
    const size_t smem = sizeof(DeltaSmem<D, F16>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&build_delta_kernel<D, F16, TKV, TG>, smem, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL((build_delta_kernel<D, F16, TKV, TG>), dim3(n_units), dim3(C::NT), smem, st, a);
    return hipGetLastError();
}

// bf16 inputs use the fp16-operand pipelined kernels: build_gdn.hip at d = 128,
// build_delta_f16.hip at d = 64.  Below that a 64-token chunk erases most of the key space, so
// Tbar - K^T (W Tbar) cancels heavily and fp16 rounding of W, Tbar and E is
// amplified: small heads, like fp32 inputs, use fp32 products here.
template <int D>
static hipError_t launch_d(const DeltaArgs &a, int kv_kind, int g_kind, bool f16, int n_units,
                           hipStream_t st)
{
    if (f16 && D == 128) return launch_build_gdn(a, kv_kind, g_kind, n_units, st);
    if (f16 && D >= 64) return launch_build_delta_f16(a, D, kv_kind, g_kind, n_units, st);
    if (kv_kind == IN_BF16 && g_kind == IN_BF16) return launch_one<D, false, bf16_t, bf16_t>(a, n_units, st);
    if (kv_kind == IN_F32 && g_kind == IN_BF16) return launch_one<D, false, float, bf16_t>(a, n_units, st);
    if (kv_kind == IN_F32 && g_kind == IN_F32) return launch_one<D, false, float, float>(a, n_units, st);
    return hipErrorInvalidValue;
}

hipError_t launch_build_delta(const DeltaArgs &a, int D, int kv_kind, int g_kind, bool f16,
                              int n_units, hipStream_t st)
{
    switch (D) {
    case 16: return launch_d<16>(a, kv_kind, g_kind, f16, n_units, st);
    case 32: return launch_d<32>(a, kv_kind, g_kind, f16, n_units, st);
    case 64: return launch_d<64>(a, kv_kind, g_kind, f16, n_units, st);
    case 128: return launch_d<128>(a, kv_kind, g_kind, f16, n_units, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hy

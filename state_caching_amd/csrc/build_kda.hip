// build_kda.hip -- chunkwise build of the cached pair (T_C, S_{C|0}) for the
// delta rule with a diagonal gate, T_i = (I - b_i k_i k_i^T) diag(g_i),
// u_i = b_i k_i v_i^T (HYPIC reading notes, ch.2 sec.3 Table 1, the KDA row;
// pair definition ch.2 sec.2, built there by two runs of the recurrence,
// ch.2 sec.4).
//
// One pass over the segment in chunks of b = 64 tokens carries X = [T | S]
// (d_k x 2d, fp32 in matrix-core accumulators).  The per-channel gate does
// not commute with the rank-one erase, so it cannot be factored out of the
// product as a scalar gate can; it is carried inside the chunk algebra.
// Within a chunk, with cl_r[d] = sum_{s <= r} log2 g_s[d] (cumulative from
// the chunk start) and Gam_r = diag(2^cl_r):
//   A_r = diag(g_r) S_{r-1},   S_r = A_r + k_r e_r^T,
//   e_r = b_r (v_r - (Gam_r k_r)^T S_0 - sum_{s<r} L_rs e_s),
//   L_rs = sum_d k_r[d] k_s[d] 2^(cl_r[d] - cl_s[d])          (s < r)
// so with M = (I + diag(b) L)^-1 (unit lower triangular),
//   W = M diag(b) Kt,  Kt_r = Gam_r k_r,   U = M diag(b) V,
//   E = [0 | U] - W X,   X <- Gam_b X + Kh^T E,  Kh_s = (Gam_b Gam_s^-1) k_s.
// Every decay factor applied is 2^(non-positive); the Gram tiles take a
// reference token per tile pair so that both operand factors stay bounded
// (off the diagonal both are <= 1; on a diagonal 16-token tile the reference
// is its middle token).  Products are fp32 16x16x4 on the matrix cores.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace hy {

template <int D>
struct KdaCfg {
    static constexpr int MT = D / 16;         // 16-row tiles of the state
    static constexpr int NW = D / 16;         // waves; wave w owns column tiles 2w, 2w+1 of X
    static constexpr int NT = 64 * NW;
    static constexpr int LDT = 68;            // token-contiguous row stride (floats)
    static constexpr int LDG = 68;
};

template <int D>
struct KdaSmem {
    using C = KdaCfg<D>;
    float KT[D][C::LDT];     // keys (dim-major); then Gam k; then W^T
    float CL[D][C::LDT];     // cumulative log2 gates (dim-major); then Kh^T
    float VT[D][C::LDT];     // values (dim-major)
    float Gm[64][C::LDG];    // b_r L_rs for s < r, else 0
    float Mm[64][C::LDG];    // M = (I + Gm)^-1
    float beta[64];
    float clb[D];            // cl of the chunk's last token per channel
    float gamb[D];           // 2^clb
};

// Gram tiles on or below the diagonal of the 4x4 token-tile grid
__constant__ int kKdaTi[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kKdaTj[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
// the eight Gram tiles that the reduced-precision build forms whole (the tiles (3,1)
// and (3,2) go in two reduction halves each)
__constant__ int kKdaWi[8] = {0, 1, 1, 2, 2, 2, 3, 3};
__constant__ int kKdaWj[8] = {0, 0, 1, 0, 1, 2, 0, 3};

template <int D, typename TKV, typename TG>
__global__ void __launch_bounds__((KdaCfg<D>::NT)) build_kda_kernel(const DeltaArgs a)
{
    using C = KdaCfg<D>;
    constexpr int MT = C::MT, NW = C::NW;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    KdaSmem<D> &sm = *reinterpret_cast<KdaSmem<D> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int unit = xcd_logical_block(blockIdx.x, gridDim.x);
    const int s = unit / a.h_v, h = unit % a.h_v;
    const int kh = h / (a.h_v / a.h_k);
    const int len = a.len[s];
    const TKV *kp = reinterpret_cast<const TKV *>(a.k) + a.tok0[s] * a.ldk + (int64_t)kh * D;
    const TKV *vp = reinterpret_cast<const TKV *>(a.v) + a.tok0[s] * a.ldv + (int64_t)h * D;
    const TG *bp = reinterpret_cast<const TG *>(a.beta) + a.gtok0[s] * a.h_v + h;
    const TG *gp = reinterpret_cast<const TG *>(a.alpha) + (a.gtok0[s] * a.h_v + h) * (int64_t)D;
    const int64_t ldg = (int64_t)a.h_v * D;

    // upper tile blocks of M are never written: zero them once
    for (int idx = tid; idx < 64 * 64; idx += C::NT) {
        const int r = idx >> 6, c = idx & 63;
        if ((c >> 4) > (r >> 4)) sm.Mm[r][c] = 0.f;
    }

    // X = [T | S] in accumulator layout: X[mt][jn] holds rows 16 mt .., column tile 2w + jn
    f4 X[MT][2];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int n = 2 * w + jn;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                X[mt][jn][i] = (n < MT && 16 * mt + 4 * g + i == 16 * n + r16) ? 1.f : 0.f;
    }

    // register prefetch of one chunk: rows prow and prow + 32, columns pcol .. pcol + 7
    constexpr int CPR = D / 8;
    const int prow = tid / CPR, pcol = 8 * (tid % CPR);
    typename Raw8<TKV>::type kraw[2], vraw[2];
    typename Raw8<TG>::type graw[2];
    float br = 0.f;
    auto fetch = [&](int c) {
        const int t0 = 64 * c;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int t = t0 + prow + 32 * p;
            if (t < len) {
                ld_raw8(kp + (int64_t)t * a.ldk + pcol, kraw[p]);
                ld_raw8(vp + (int64_t)t * a.ldv + pcol, vraw[p]);
                ld_raw8(gp + (int64_t)t * ldg + pcol, graw[p]);
            } else {
                zero_raw8(kraw[p]);
                zero_raw8(vraw[p]);
                zero_raw8(graw[p]);
            }
        }
        if (w == 0) {
            const int t = t0 + lane;
            br = t < len ? ld1(bp + (int64_t)t * a.h_v) : 0.f;
        }
    };

    const int nch = (len + 63) / 64;
    if (nch > 0) fetch(0);

    for (int c = 0; c < nch; ++c) {
        lds_barrier();   // readers of the previous chunk are done

        // ---- stage keys, values, log2 gates (dim-major), betas -------------------
        {
            float kr[2][8], vr[2][8], gr[2][8];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                widen8(kraw[p], kr[p]);
                widen8(vraw[p], vr[p]);
                widen8(graw[p], gr[p]);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int t = prow + 32 * p;
                const bool in = 64 * c + t < len;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sm.KT[pcol + e][t] = kr[p][e];
                    sm.VT[pcol + e][t] = vr[p][e];
                    // past the segment end the transition is the identity (g = 1); a
                    // gate below 2^-126 is taken as 2^-126 (the state is wiped either way)
                    sm.CL[pcol + e][t] = in ? fmaxf(log2f(gr[p][e]), -126.f) : 0.f;
                }
            }
            if (w == 0) sm.beta[lane] = br;
        }
        if (c + 1 < nch) fetch(c + 1);
        lds_barrier();

        // ---- cumulative log2 gates over the chunk, per channel (one wave scan each)
        for (int d = w; d < D; d += NW) {
            const float cl = wave_prefix_incl(sm.CL[d][lane]);
            sm.CL[d][lane] = cl;
            if (lane == 63) {
                sm.clb[d] = cl;
                sm.gamb[d] = exp2f(cl);
            }
        }
        lds_barrier();

        // ---- decay-aware Gram: b_r sum_d k_r k_s 2^(cl_r - cl_s), s < r ------------
        for (int q = w; q < 10; q += NW) {
            const int ti = kKdaTi[q], tj = kKdaTj[q];
            const int ref = ti == tj ? 16 * ti + 8 : 16 * tj + 15;
            f4 acc = zero4();
#pragma unroll 4
            for (int ks = 0; ks < D / 4; ++ks) {
                const int k = g * (D / 4) + ks;
                const float cr = sm.CL[k][ref];
                const float A = sm.KT[k][16 * ti + r16] * exp2f(sm.CL[k][16 * ti + r16] - cr);
                const float B = sm.KT[k][16 * tj + r16] * exp2f(cr - sm.CL[k][16 * tj + r16]);
                acc = mma(A, B, acc);
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

        // ---- decayed keys: KT <- Gam k, CL <- (Gam_b / Gam) k ----------------------
        for (int idx = tid; idx < D * 64; idx += C::NT) {
            const int d = idx >> 6, t = idx & 63;
            const float kv = sm.KT[d][t], cl = sm.CL[d][t];
            sm.KT[d][t] = kv * exp2f(cl);
            sm.CL[d][t] = kv * exp2f(sm.clb[d] - cl);
        }
        lds_barrier();

        // ---- W^T = (M diag(b) Kt)^T in place of Kt^T: wave w owns key rows 16w .. --
        {
            const int td = w;
            f4 acc[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                acc[ti] = zero4();
#pragma unroll
                for (int ks = 0; ks < 16; ++ks) {
                    const int k = 16 * g + ks;
                    acc[ti] = mma(sm.Mm[16 * ti + r16][k] * sm.beta[k], sm.KT[16 * td + r16][k], acc[ti]);
                }
            }
            // every read of this wave's rows is issued above (LDS operations of a
            // wave complete in order)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.KT[16 * td + r16][16 * ti + 4 * g + i] = acc[ti][i];
        }
        lds_barrier();

        // ---- state update of this wave's two column tiles ----------------------
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int n = 2 * w + jn;
            const bool isS = n >= MT;
            f4 E[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) E[ti] = zero4();
            if (isS) {   // U = M diag(b) V for the value columns of this tile
                const int cc = 16 * (n - MT);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
                    for (int ks = 0; ks < 16; ++ks) {
                        const int k = 16 * g + ks;
                        E[ti] = mma(sm.Mm[16 * ti + r16][k] * sm.beta[k], sm.VT[cc + r16][k], E[ti]);
                    }
                }
            }
            // E -= W X (X before the chunk)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
                        E[ti] = mma(sm.KT[16 * mt + 4 * g + i][16 * ti + r16], -X[mt][jn][i], E[ti]);
            // X <- Gam_b X + Kh^T E
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float4 gq = *reinterpret_cast<const float4 *>(&sm.gamb[16 * mt + 4 * g]);
                X[mt][jn] *= f4{gq.x, gq.y, gq.z, gq.w};
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        X[mt][jn] = mma(sm.CL[16 * mt + r16][16 * ti + 4 * g + i], E[ti][i], X[mt][jn]);
            }
        }
    }

    float *Tu = a.T_out + (int64_t)unit * D * D;
    float *Su = a.S0_out + (int64_t)unit * D * D;
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int n = 2 * w + jn;
        const bool isS = n >= MT;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * g + i;
                if (isS) Su[row * D + 16 * (n - MT) + r16] = X[mt][jn][i];
                else     Tu[row * D + 16 * n + r16] = X[mt][jn][i];
            }
    }
}

// ---------------------------------------------------------------------------
// bf16 inputs, d >= 64: the same chunk algebra with the two state products on
// fp16 matrix-core operands (16x16x32, fp32 accumulation):
//   E = [0 | U] - W X     (A = W, token rows with keys permuted inside each
//                          32-key block; B = -X from the state's accumulators)
//   X <- Gam_b X + Kh^T E (A = Kh^T, key rows with tokens permuted the same way;
//                          B = E from its accumulators)
// The state's column tiles are carried in power-of-two units (renormalised every
// 4 chunks, the S tiles also when a chunk's values run more than 2^4 ahead), so
// every fp16 operand stays in range.  W = M diag(b) (Gam K) and U = M diag(b) V
// take fp16 operands too (A = M diag(b) rounded once per chunk; the value
// columns scaled by a power of two per tile and chunk); the Gram and the
// inverse stay fp32.
template <int D>
struct KdaHSmem {
    using C = KdaCfg<D>;
    static constexpr int LDW = D + 8;         // W row stride (halves)
    static constexpr int LDK = 64 + 8;        // Kh^T row stride (halves)
    float KT[D][C::LDT];     // keys (dim-major); then Gam k
    float CL[D][C::LDT];     // cumulative log2 gates (dim-major)
    uint16_t VT[D][LDK];     // raw bf16 values (dim-major)
    union {
        float bp[8][D];              // log2-gate totals of the chunk's 8-token blocks (staging)
        float Gm[64][C::LDG];        // then b_r L_rs for s < r, else 0
        _Float16 Wh[64][LDW];        // then W (token rows, keys permuted)
    };
    float Mm[64][C::LDG];    // M = (I + Gm)^-1
    float Gx[2][16][16];     // second k-halves of the Gram tiles (3,1) and (3,2)
    _Float16 Mb[64][LDK];    // M diag(b) in fp16 (token rows, columns permuted)
    _Float16 Kh[D][LDK];     // Kh^T (key rows, tokens permuted)
    float beta[64];
    float clb[D];
    float gamb[D];
};

// position of index k inside its block of 32 in the permuted operand order: lane
// group g's 8 elements are k = 4g + (e & 3) + 16 (e >> 2), e = 0..7
__device__ __forceinline__ int kda_perm(int k)
{
    return (k & ~31) + 8 * ((k & 15) >> 2) + 4 * ((k >> 4) & 1) + (k & 3);
}

template <int D, typename TG>
__global__ void __launch_bounds__((KdaCfg<D>::NT)) build_kda_f16_kernel(const DeltaArgs a)
{
    using C = KdaCfg<D>;
    using SM = KdaHSmem<D>;
    constexpr int MT = C::MT, NW = C::NW, KB = D / 32, LDW = SM::LDW, LDK = SM::LDK;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM &sm = *reinterpret_cast<SM *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int unit = xcd_logical_block(blockIdx.x, gridDim.x);
    const int s = unit / a.h_v, h = unit % a.h_v;
    const int kh = h / (a.h_v / a.h_k);
    const int len = a.len[s];
    const bf16_t *kp = reinterpret_cast<const bf16_t *>(a.k) + a.tok0[s] * a.ldk + (int64_t)kh * D;
    const bf16_t *vp = reinterpret_cast<const bf16_t *>(a.v) + a.tok0[s] * a.ldv + (int64_t)h * D;
    const TG *bp = reinterpret_cast<const TG *>(a.beta) + a.gtok0[s] * a.h_v + h;
    const TG *gp = reinterpret_cast<const TG *>(a.alpha) + (a.gtok0[s] * a.h_v + h) * (int64_t)D;
    const int64_t ldg = (int64_t)a.h_v * D;

    for (int idx = tid; idx < 64 * 64; idx += C::NT) {
        const int r = idx >> 6, c = idx & 63;
        if ((c >> 4) > (r >> 4)) sm.Mm[r][c] = 0.f;
    }

    // X = [T | S] in power-of-two units: X[mt][jn] holds rows 16 mt .. of column tile
    // n = w (jn = 0, a T tile) or MT + w (jn = 1, an S tile): every wave carries one
    // of each, so the value products of the S tiles spread over all waves
    f4 X[MT][2];
    float sig[2] = {0.f, 0.f};
    int svq = 0;   // value exponent of the last chunk (S tile waves)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int n = jn ? MT + w : w;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                X[mt][jn][i] = (n < MT && 16 * mt + 4 * g + i == 16 * n + r16) ? 1.f : 0.f;
    }
    // Xhat <- Xhat 2^(sig - target): the unit follows the tile's largest entry,
    // never below 2^(ev - 4) for S (keeps the value term of E within fp16 range)
    auto renorm = [&](int jn, bool isS, int ev) {
        float xm = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) xm = fmaxf(xm, fabsf(X[mt][jn][i]));
        xm = wave_max(xm);
        float target = (float)pow2_exponent(xm) + sig[jn];
        if (xm == 0.f) target = isS ? (float)ev : sig[jn];
        if (isS && target < (float)ev - 4.f) target = (float)ev - 4.f;
        // an integer shift, exact, and finite however far the tile has decayed
        const int sh = (int)(sig[jn] - target);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) X[mt][jn][i] = ldexpf(X[mt][jn][i], sh);
        sig[jn] = target;
    };

    // staging role: thread (dp, blk) owns key dims 2 dp, 2 dp + 1 of the 8 tokens
    // 8 blk .. 8 blk + 7 of a chunk; a wave's loads are whole rows.
    // log2 and exp2 below are the hardware instructions: log-gates are clamped at
    // -126 anyway, and a decay factor below 2^-126 flushes to zero (its term is
    // below the fp32 range of the chunk's own contributions)
    static_assert(std::is_same<TG, bf16_t>::value, "bf16 gates");
    constexpr int LPR = D / 2;                 // lanes per row
    constexpr int NB = C::NT / LPR;            // token blocks per chunk
    static_assert(NB == 8, "8 blocks of 8 tokens");
    const int dp = tid % LPR, blk = tid / LPR;
    uint32_t kraw[8], vraw[8], graw[8];
    float br = 0.f;
    // rows through buffer loads: per chunk a resource based at its first row and
    // sized to its rows inside the segment (rows past the end read as zero; the
    // staging masks them anyway), offsets = this thread's row and dims plus i rows
    const uint32_t ldk_b = (uint32_t)a.ldk * 2u, ldv_b = (uint32_t)a.ldv * 2u, ldg_b = (uint32_t)ldg * 2u;
    auto fetch = [&](int c) {
        const int rows = min(len - 64 * c, 64);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kp + (int64_t)(64 * c) * a.ldk), (short)0, (int)((uint32_t)rows * ldk_b), 0x00020000);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vp + (int64_t)(64 * c) * a.ldv), (short)0, (int)((uint32_t)rows * ldv_b), 0x00020000);
        const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(gp + (int64_t)(64 * c) * ldg), (short)0, (int)((uint32_t)rows * ldg_b), 0x00020000);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t t = (uint32_t)(8 * blk + i);
            kraw[i] = __builtin_amdgcn_raw_buffer_load_b32(kr, (int)(t * ldk_b + 4u * dp), 0, 0);
            vraw[i] = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)(t * ldv_b + 4u * dp), 0, 0);
            graw[i] = __builtin_amdgcn_raw_buffer_load_b32(gr, (int)(t * ldg_b + 4u * dp), 0, 0);
        }
        if (w == 0) {
            const int t = 64 * c + lane;
            br = t < len ? ld1(bp + (int64_t)t * a.h_v) : 0.f;
        }
    };
    auto lo16 = [](uint32_t x) { return __uint_as_float(x << 16); };
    auto hi16 = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };

    const int nch = (len + 63) / 64;
    if (nch > 0) fetch(0);

    for (int c = 0; c < nch; ++c) {
        lds_barrier();   // readers of the previous chunk are done

        // ---- stage keys, values (dim-major) and the in-block cumulative log2 gates;
        //      the block totals go to LDS for the cross-block offsets
        float cp[8][2];
        // MK: the chunk runs past the segment end (rows beyond it stage as zero keys
        // and values and gate 1); a full chunk takes no masks
        auto stage = [&](auto mk) {
            constexpr bool MK = decltype(mk)::value;
            float kf[8][2];
            uint32_t vw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool in = !MK || 64 * c + 8 * blk + i < len;
                kf[i][0] = in ? lo16(kraw[i]) : 0.f;
                kf[i][1] = in ? hi16(kraw[i]) : 0.f;
                vw[i] = in ? vraw[i] : 0u;
                const float l0 = in ? fmaxf(__builtin_amdgcn_logf(lo16(graw[i])), -126.f) : 0.f;
                const float l1 = in ? fmaxf(__builtin_amdgcn_logf(hi16(graw[i])), -126.f) : 0.f;
                cp[i][0] = i ? cp[i - 1][0] + l0 : l0;
                cp[i][1] = i ? cp[i - 1][1] + l1 : l1;
            }
            *reinterpret_cast<float2 *>(&sm.bp[blk][2 * dp]) = make_float2(cp[7][0], cp[7][1]);
            // tokens 8 blk + i sit at kda_perm positions pb + i (i < 4) and pb + 8 + i - 4
            const int pb = 32 * (blk >> 2) + 16 * (blk & 1) + 4 * ((blk >> 1) & 1);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float *kt = &sm.KT[2 * dp + e][8 * blk];
                *reinterpret_cast<float4 *>(kt) = make_float4(kf[0][e], kf[1][e], kf[2][e], kf[3][e]);
                *reinterpret_cast<float4 *>(kt + 4) = make_float4(kf[4][e], kf[5][e], kf[6][e], kf[7][e]);
                uint32_t vv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    vv[q] = e ? ((vw[2 * q] >> 16) | (vw[2 * q + 1] & 0xffff0000u))
                              : ((vw[2 * q] & 0xffffu) | (vw[2 * q + 1] << 16));
                *reinterpret_cast<uint2 *>(&sm.VT[2 * dp + e][pb]) = make_uint2(vv[0], vv[1]);
                *reinterpret_cast<uint2 *>(&sm.VT[2 * dp + e][pb + 8]) = make_uint2(vv[2], vv[3]);
            }
            if (w == 0) sm.beta[lane] = br;
        };
        if (64 * (c + 1) <= len) stage(std::false_type{});
        else stage(std::true_type{});
        if (c + 1 < nch) fetch(c + 1);
        lds_barrier();

        // ---- cumulative log2 gates over the chunk: the block's own prefix plus the
        //      totals of the earlier blocks; the chunk total per channel
        {
            float off0 = 0.f, off1 = 0.f;
#pragma unroll
            for (int b = 0; b < NB - 1; ++b) {
                const float2 q = *reinterpret_cast<const float2 *>(&sm.bp[b][2 * dp]);
                if (b < blk) { off0 += q.x; off1 += q.y; }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float off = e ? off1 : off0;
                float *cl = &sm.CL[2 * dp + e][8 * blk];
                *reinterpret_cast<float4 *>(cl) = make_float4(off + cp[0][e], off + cp[1][e], off + cp[2][e], off + cp[3][e]);
                *reinterpret_cast<float4 *>(cl + 4) = make_float4(off + cp[4][e], off + cp[5][e], off + cp[6][e], off + cp[7][e]);
            }
            if (blk == NB - 1) {
                // the last block's last token carries the chunk total
                sm.clb[2 * dp] = off0 + cp[7][0];
                sm.clb[2 * dp + 1] = off1 + cp[7][1];
                sm.gamb[2 * dp] = __builtin_amdgcn_exp2f(off0 + cp[7][0]);
                sm.gamb[2 * dp + 1] = __builtin_amdgcn_exp2f(off1 + cp[7][1]);
            }
        }
        lds_barrier();

        // ---- decay-aware Gram: b_r sum_d k_r k_s 2^(cl_r - cl_s), s < r ------------
        // The per-element exp2 of the operands bounds this phase, so the work is spread
        // evenly over the SIMDs: eight whole tiles, one per wave (two per wave at
        // NW = 4), and the tiles (3,1) and (3,2) as two reduction halves each on waves
        // 0-3 (the second halves' partial sums are added in below, while wave 0 inverts)
        auto gram = [&](int ti, int tj, int ks0, int ks1) {
            const int ref = ti == tj ? 16 * ti + 8 : 16 * tj + 15;
            f4 acc = zero4();
#pragma unroll 4
            for (int ks = ks0; ks < ks1; ++ks) {
                const int k = g * (D / 4) + ks;
                const float cr = sm.CL[k][ref];
                const float A = sm.KT[k][16 * ti + r16] * __builtin_amdgcn_exp2f(sm.CL[k][16 * ti + r16] - cr);
                const float B = sm.KT[k][16 * tj + r16] * __builtin_amdgcn_exp2f(cr - sm.CL[k][16 * tj + r16]);
                acc = mma(A, B, acc);
            }
            return acc;
        };
        for (int q = w; q < 8; q += NW) {
            const int ti = kKdaWi[q], tj = kKdaWj[q];
            const f4 acc = gram(ti, tj, 0, D / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * ti + 4 * g + i, cc = 16 * tj + r16;
                sm.Gm[rr][cc] = (cc < rr) ? sm.beta[rr] * acc[i] : 0.f;
            }
        }
        if (w < 4) {
            const int tj = 1 + (w >> 1), hf = w & 1;
            const f4 acc = gram(3, tj, hf * (D / 8), (hf + 1) * (D / 8));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = sm.beta[48 + 4 * g + i] * acc[i];
                if (hf == 0) sm.Gm[48 + 4 * g + i][16 * tj + r16] = v;
                else         sm.Gx[tj - 1][4 * g + i][r16] = v;
            }
        }
        lds_barrier();

        // ---- M = (I + Gm)^-1: diagonal 16x16 blocks by forward substitution ----
        //      lane (o, c) carries column c of block o and the multipliers -Gm[o + r][o + c],
        //      which the step for column q broadcasts from lane q along the 16-lane row
        if (w == 0) {
            const int o = 16 * (lane >> 4), cc = lane & 15;
            float n[16], x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                n[r] = -sm.Gm[o + r][o + cc];
                x[r] = (r == cc) ? 1.f : 0.f;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(n[r]));   // n complete here
            asm volatile("s_nop 1");   // the two wait states before the lane moves read n
            subst_steps<0>(x, n);
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.Mm[o + r][o + cc] = x[r];
        } else {
            // the second halves of the split Gram tiles (3,1) and (3,2)
            for (int e = tid - 64; e < 2 * 256; e += C::NT - 64) {
                const int t = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
                sm.Gm[48 + rr][16 * (t + 1) + cc] += sm.Gx[t][rr][cc];
            }
        }
        lds_barrier();
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

        // ---- decayed keys: KT <- Gam k (fp32), Kh^T = (Gam_b / Gam) k (fp16, tokens
        //      permuted), 4 tokens per step (kda_perm keeps runs of 4), by waves 2 ..
        //      while waves 0 and 1 finish the inverse above
        if (w >= 2) {
            for (int u = tid - 128; u < D * 16; u += C::NT - 128) {
                const int d = u >> 4, t4 = 4 * (u & 15);
                const float4 kv = *reinterpret_cast<const float4 *>(&sm.KT[d][t4]);
                const float4 cl = *reinterpret_cast<const float4 *>(&sm.CL[d][t4]);
                const float cb = sm.clb[d];
                *reinterpret_cast<float4 *>(&sm.KT[d][t4]) =
                    make_float4(kv.x * __builtin_amdgcn_exp2f(cl.x), kv.y * __builtin_amdgcn_exp2f(cl.y),
                                kv.z * __builtin_amdgcn_exp2f(cl.z), kv.w * __builtin_amdgcn_exp2f(cl.w));
                const h4 kh = h4{(_Float16)(kv.x * __builtin_amdgcn_exp2f(cb - cl.x)),
                                 (_Float16)(kv.y * __builtin_amdgcn_exp2f(cb - cl.y)),
                                 (_Float16)(kv.z * __builtin_amdgcn_exp2f(cb - cl.z)),
                                 (_Float16)(kv.w * __builtin_amdgcn_exp2f(cb - cl.w))};
                *reinterpret_cast<h4 *>(&sm.Kh[d][kda_perm(t4)]) = kh;
            }
        }
        lds_barrier();   // M complete; the last reads of Gm are above
        // ---- Mb = M diag(b) in fp16, columns permuted (the A operand of W and U)
        for (int idx = tid; idx < 64 * 64; idx += C::NT) {
            const int r = idx >> 6, t = idx & 63;
            sm.Mb[r][kda_perm(t)] = (_Float16)(sm.Mm[r][t] * sm.beta[t]);
        }
        lds_barrier();

        // ---- W = M diag(b) Kt, stored fp16 by token rows, keys permuted: wave w forms
        //      key columns 16w .. 16w + 15; A = M diag(b) (fp16, the chunk's Mb),
        //      B = Kt (rows 32 sb + 4g + (e & 3) + 16 (e >> 2) of key 16w + r16)
        {
            const int td = w;
            f4 acc[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) acc[ti] = zero4();
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const float4 b0 = *reinterpret_cast<const float4 *>(&sm.KT[16 * td + r16][32 * sb + 4 * g]);
                const float4 b1 = *reinterpret_cast<const float4 *>(&sm.KT[16 * td + r16][32 * sb + 16 + 4 * g]);
                const h8 B = h8{(_Float16)b0.x, (_Float16)b0.y, (_Float16)b0.z, (_Float16)b0.w,
                                (_Float16)b1.x, (_Float16)b1.y, (_Float16)b1.z, (_Float16)b1.w};
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const h8 A = *reinterpret_cast<const h8 *>(&sm.Mb[16 * ti + r16][32 * sb + 8 * g]);
                    acc[ti] = mma(A, B, acc[ti]);
                }
            }
            const int kpos = kda_perm(16 * td + r16);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.Wh[16 * ti + 4 * g + i][kpos] = (_Float16)acc[ti][i];
        }
        lds_barrier();

        // ---- state update of this wave's two column tiles ----------------------
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int n = jn ? MT + w : w;
            const bool isS = n >= MT;
            f4 E[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) E[ti] = zero4();
            if (isS) {
                // U = M diag(b) V for the value columns of this tile: B = the raw values of
                // column 16 (n - MT) + r16 (tokens permuted as stored) divided by 2^ev, ev the
                // exponent of the tile's largest value in the chunk
                const int cc = 16 * (n - MT);
                float vb[2][8];
                float am = 0.f;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const uint4 raw = *reinterpret_cast<const uint4 *>(&sm.VT[cc + r16][32 * sb + 8 * g]);
                    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        vb[sb][2 * q] = __uint_as_float(wv[q] << 16);
                        vb[sb][2 * q + 1] = __uint_as_float(wv[q] & 0xffff0000u);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(vb[sb][e]));
                }
                const int ev = pow2_exponent(wave_max(am));
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    h8 B;
#pragma unroll
                    for (int e = 0; e < 8; ++e) B[e] = (_Float16)ldexpf(vb[sb][e], -ev);
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) {
                        const h8 A = *reinterpret_cast<const h8 *>(&sm.Mb[16 * ti + r16][32 * sb + 8 * g]);
                        E[ti] = mma(A, B, E[ti]);
                    }
                }
                // the S unit: the chunk's value scale on the first chunk (S is zero),
                // renormalised when the values run more than 2^4 ahead of it
                float vmax = 0.f;
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int i = 0; i < 4; ++i) vmax = fmaxf(vmax, fabsf(E[ti][i]));
                svq = pow2_exponent(wave_max(vmax)) + ev;
                if (c == 0) sig[jn] = (float)svq;
                else if ((float)svq > sig[jn] + 4.f) renorm(jn, true, svq);
                const int isg = (int)sig[jn] - ev;
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int i = 0; i < 4; ++i) E[ti][i] = ldexpf(E[ti][i], -isg);
            }
            // E -= W Xhat (Xhat before the chunk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                h8 B;   // -Xhat, keys 32 kb + 4g + (e & 3) + 16 (e >> 2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    B[i] = (_Float16)(-X[2 * kb][jn][i]);
                    B[4 + i] = (_Float16)(-X[2 * kb + 1][jn][i]);
                }
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const h8 A = *reinterpret_cast<const h8 *>(&sm.Wh[16 * ti + r16][32 * kb + 8 * g]);
                    E[ti] = mma(A, B, E[ti]);
                }
            }
            h4 Eh[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) Eh[ti] = h4{(_Float16)E[ti][0], (_Float16)E[ti][1], (_Float16)E[ti][2], (_Float16)E[ti][3]};
            // Xhat <- Gam_b Xhat + Kh^T E
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float4 gq = *reinterpret_cast<const float4 *>(&sm.gamb[16 * mt + 4 * g]);
                X[mt][jn] *= f4{gq.x, gq.y, gq.z, gq.w};
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const h8 A = *reinterpret_cast<const h8 *>(&sm.Kh[16 * mt + r16][32 * jb + 8 * g]);
                    const h8 Bv = h8{Eh[2 * jb][0], Eh[2 * jb][1], Eh[2 * jb][2], Eh[2 * jb][3],
                                     Eh[2 * jb + 1][0], Eh[2 * jb + 1][1], Eh[2 * jb + 1][2], Eh[2 * jb + 1][3]};
                    X[mt][jn] = mma(A, Bv, X[mt][jn]);
                }
            }
        }
        // periodic renormalisation of each tile every 4 chunks, the two tiles two chunks apart
        if ((c & 3) == 1) renorm(0, false, svq);
        else if ((c & 3) == 3) renorm(1, true, svq);
    }

    float *Tu = a.T_out + (int64_t)unit * D * D;
    float *Su = a.S0_out + (int64_t)unit * D * D;
    // opaque lane offsets: keeps the output addresses from being formed before the
    // chunk loop (they would be held, or spilled, across it)
    int g4 = 4 * g, cl16 = r16;
    asm volatile("" : "+v"(g4), "+v"(cl16));
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int n = jn ? MT + w : w;
        const bool isS = n >= MT;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + g4 + i;
                const float val = ldexpf(X[mt][jn][i], (int)sig[jn]);
                if (isS) Su[row * D + 16 * (n - MT) + cl16] = val;
                else     Tu[row * D + 16 * n + cl16] = val;
            }
    }
}

template <int D, typename TG>
static hipError_t launch_kda_f16_one(const DeltaArgs &a, int n_units, hipStream_t st)
{
    const size_t smem = sizeof(KdaHSmem<D>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&build_kda_f16_kernel<D, TG>, smem, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL((build_kda_f16_kernel<D, TG>), dim3(n_units), dim3(KdaCfg<D>::NT), smem, st, a);
    return hipGetLastError();
}

template <int D, typename TKV, typename TG>
static hipError_t launch_kda_one(const DeltaArgs &a, int n_units, hipStream_t st)
{
    const size_t smem = sizeof(KdaSmem<D>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&build_kda_kernel<D, TKV, TG>, smem, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL((build_kda_kernel<D, TKV, TG>), dim3(n_units), dim3(KdaCfg<D>::NT), smem, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_kda_d(const DeltaArgs &a, int kv_kind, int g_kind, bool f16, int n_units, hipStream_t st)
{
    if constexpr (D >= 64) {
        if (f16 && kv_kind == IN_BF16 && g_kind == IN_BF16) return launch_kda_f16_one<D, bf16_t>(a, n_units, st);
    }
    if (kv_kind == IN_BF16 && g_kind == IN_BF16) return launch_kda_one<D, bf16_t, bf16_t>(a, n_units, st);
    if (kv_kind == IN_F32 && g_kind == IN_BF16) return launch_kda_one<D, float, bf16_t>(a, n_units, st);
    if (kv_kind == IN_F32 && g_kind == IN_F32) return launch_kda_one<D, float, float>(a, n_units, st);
    return hipErrorInvalidValue;
}

hipError_t launch_build_kda(const DeltaArgs &a, int D, int kv_kind, int g_kind, bool f16, int n_units,
                            hipStream_t st)
{
    switch (D) {
    case 16: return launch_kda_d<16>(a, kv_kind, g_kind, false, n_units, st);
    case 32: return launch_kda_d<32>(a, kv_kind, g_kind, false, n_units, st);
    case 64: return launch_kda_d<64>(a, kv_kind, g_kind, f16, n_units, st);
    case 128: return launch_kda_d<128>(a, kv_kind, g_kind, f16, n_units, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hy

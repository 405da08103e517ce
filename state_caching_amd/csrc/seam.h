// seam.h -- seam-window advance for the gated-delta family, device side.
//
// HYPIC reading notes ch.2 sec.5: the first w tokens of every inner segment
// are recomputed from the running prefix state, after which the cached body
// pair jumps to the segment end; ch.2 sec.6: the causal conv at the segment
// head reads the previous segment's last W-1 raw rows (its cached tail).
//
// A workgroup owns one value head h and 16 state columns [c0, c0+16); the
// state block lives in LDS as ST[col][row].  The window is applied in its
// compact form (the same algebra as the chunkwise build): with
//   G = K K^T, M = (I + diag(b) strictlower(G))^-1, W = M diag(b) K,
//   U = M diag(b dec) V, dec_t = prod_{s>t} a_s, gw = prod a,
// the state after the window is S' = gw S + K^T (U - W (gw S)).
// The window's own pair is T_w = gw (I - K^T W), S_w0 = K^T U, and the
// per-token read-outs are o_t = gam_t (q_t^T S - sum_{s<=t} (q_t.k_s) (W S)_s)
//                            + sum_{r<=t} H_tr b_r (gam_t / gam_r) v_r,
// H = strictlower-inclusive(QK) M, gam_t = prod_{s<=t} a_s (all in fp32).
#pragma once
#include "common.h"
#include "launch.h"

namespace hy {

template <int D, int WMAX, int NC = 16>
struct WinSmem {
    static constexpr int LD = D + 4;
    static constexpr int LC = NC + 4;
    float K[WMAX][LD];     // keys after conv / normalisation
    float W[WMAX][LD];     // M diag(b) K
    float V[WMAX][LC];     // values of this column block
    float U[WMAX][LC];     // M diag(b dec) V
    float P[WMAX][LC];     // W S
    float E[WMAX][LC];     // U - gw P
    float G[WMAX][WMAX + 1];   // b_r k_r.k_s (s < r); later q_t.k_s when read-outs are asked for
    float M[WMAX][WMAX + 1];
    float beta[WMAX], dec[WMAX], cl[WMAX];
    float gw;
};

// xext(t') of window rows: t' >= 0 from the window, t' < 0 from the tail
template <typename TIN>
__device__ __forceinline__ float win_row(const TIN *x, const TIN *tail, int t, int Wc,
                                         int64_t row_stride, int64_t col)
{
    if (t >= 0) return ld1(x + (int64_t)t * row_stride + col);
    return ld1(tail + (int64_t)(Wc - 1 + t) * row_stride + col);
}

// The window's keys (after conv and, if asked, L2 normalisation) into ws.K and
// its value columns [c0, c0 + NC) of head h (after conv) into ws.V.  Ends with
// a barrier.
template <int D, int WMAX, typename TIN, int NC = 16>
__device__ void seam_stage_kv(WinSmem<D, WMAX, NC> &ws, const SeamArgs &a, int win, int h, int c0)
{
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6, nwv = nt >> 6;
    const int w = a.w, Wc = a.conv_w;
    const int kh = h / (a.h_v / a.h_k);
    const int64_t ldk = (int64_t)a.h_k * D, ldv = (int64_t)a.h_v * D;
    const TIN *xk = reinterpret_cast<const TIN *>(a.xk) + (int64_t)win * w * ldk;
    const TIN *xv = reinterpret_cast<const TIN *>(a.xv) + (int64_t)win * w * ldv;
    const TIN *tk = Wc > 1 ? reinterpret_cast<const TIN *>(a.tail_k) + (int64_t)win * (Wc - 1) * ldk : nullptr;
    const TIN *tv = Wc > 1 ? reinterpret_cast<const TIN *>(a.tail_v) + (int64_t)win * (Wc - 1) * ldv : nullptr;

    for (int idx = tid; idx < w * D; idx += nt) {
        const int t = idx / D, d = idx % D;
        const int64_t col = (int64_t)kh * D + d;
        float y;
        if (Wc > 0) {
            y = 0.f;
            const float *wk = a.conv_wk + col * Wc;
            for (int j = 0; j < Wc; ++j) y += wk[j] * win_row(xk, tk, t - (Wc - 1) + j, Wc, ldk, col);
        } else {
            y = ld1(xk + (int64_t)t * ldk + col);
        }
        ws.K[t][d] = y;
    }
    for (int idx = tid; idx < w * NC; idx += nt) {
        const int t = idx / NC, cc = idx % NC;
        const int64_t col = (int64_t)h * D + c0 + cc;
        float y;
        if (Wc > 0) {
            y = 0.f;
            const float *wvp = a.conv_wv + col * Wc;
            for (int j = 0; j < Wc; ++j) y += wvp[j] * win_row(xv, tv, t - (Wc - 1) + j, Wc, ldv, col);
        } else {
            y = ld1(xv + (int64_t)t * ldv + col);
        }
        ws.V[t][cc] = y;
    }
    lds_barrier();
    if (a.k_l2norm) {
        for (int t = wv; t < w; t += nwv) {
            float ss = 0.f;
            for (int d = lane; d < D; d += 64) ss += ws.K[t][d] * ws.K[t][d];
            ss = wave_sum(ss);
            const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
            for (int d = lane; d < D; d += 64) ws.K[t][d] *= inv;
        }
        lds_barrier();
    }
}

// Window prep (scalar gates): everything that does not depend on the state
// (value columns [c0, c0 + NC) of head h).
template <int D, int WMAX, typename TIN, int NC = 16>
__device__ void seam_prep(WinSmem<D, WMAX, NC> &ws, const SeamArgs &a, int win, int h, int c0)
{
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
    const int w = a.w;
    seam_stage_kv<D, WMAX, TIN, NC>(ws, a, win, h, c0);
    if (wv == 0) {   // gates: inclusive prefix and exclusive suffix of log2 a over the window
        const TIN *bp = reinterpret_cast<const TIN *>(a.beta) + (int64_t)win * w * a.h_v + h;
        const TIN *ap = reinterpret_cast<const TIN *>(a.alpha) + (int64_t)win * w * a.h_v + h;
        float l2 = 0.f, b = 0.f;
        if (lane < w) {
            b = ld1(bp + (int64_t)lane * a.h_v);
            l2 = log2f(ld1(ap + (int64_t)lane * a.h_v));
        }
        const float pre = wave_prefix_incl(l2);
        const float sfx = wave_suffix_excl(l2);
        const double tot = wave_sum_f64((double)l2);
        if (lane < w) {
            ws.beta[lane] = b;
            ws.dec[lane] = exp2f(sfx);
            ws.cl[lane] = pre;
        }
        if (lane == 0) ws.gw = scale_pow2(1.f, tot);
    }
    lds_barrier();
    // G (strictly lower, scaled by b_r)
    for (int idx = tid; idx < w * w; idx += nt) {
        const int r = idx / w, c = idx % w;
        float acc = 0.f;
        if (c < r)
            for (int d = 0; d < D; ++d) acc += ws.K[r][d] * ws.K[c][d];
        ws.G[r][c] = ws.beta[r] * acc;
    }
    lds_barrier();
    // M = (I + G)^-1 by forward substitution, one column per lane
    if (tid < w) {
        const int c = tid;
        for (int r = 0; r < w; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
            for (int q = c; q < r; ++q) acc -= ws.G[r][q] * ws.M[q][c];
            ws.M[r][c] = acc;
        }
    }
    lds_barrier();
    for (int idx = tid; idx < w * D; idx += nt) {
        const int t = idx / D, d = idx % D;
        float acc = 0.f;
        for (int q = 0; q <= t; ++q) acc += ws.M[t][q] * ws.beta[q] * ws.K[q][d];
        ws.W[t][d] = acc;
    }
    for (int idx = tid; idx < w * NC; idx += nt) {
        const int t = idx / NC, cc = idx % NC;
        float acc = 0.f;
        for (int q = 0; q <= t; ++q) acc += ws.M[t][q] * ws.beta[q] * ws.dec[q] * ws.V[q][cc];
        ws.U[t][cc] = acc;
    }
    lds_barrier();
}

// Apply the prepared window to the state block ST[16][ldst] (in place).
// With read-outs (q != null) also writes o for this window and column block.
template <int D, int WMAX, typename TIN>
__device__ void seam_apply(WinSmem<D, WMAX, 16> &ws, float *ST, int ldst, const SeamArgs &a, int win,
                           int h, int c0)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    const int w = a.w;
    const float gw = ws.gw;
    // P = W S, E = U - gw P
    for (int idx = tid; idx < w * 16; idx += nt) {
        const int t = idx / 16, cc = idx % 16;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += ws.W[t][d] * ST[cc * ldst + d];
        ws.P[t][cc] = acc;
        ws.E[t][cc] = ws.U[t][cc] - gw * acc;
    }
    if (a.q != nullptr) {   // q_t.k_s for s <= t
        const int kh = h / (a.h_v / a.h_k);
        const int64_t ldk = (int64_t)a.h_k * D;
        const TIN *qp = reinterpret_cast<const TIN *>(a.q) + (int64_t)win * w * ldk + (int64_t)kh * D;
        lds_barrier();
        for (int idx = tid; idx < w * w; idx += nt) {
            const int t = idx / w, s = idx % w;
            float acc = 0.f;
            if (s <= t)
                for (int d = 0; d < D; ++d) acc += ld1(qp + (int64_t)t * ldk + d) * ws.K[s][d];
            ws.G[t][s] = acc;
        }
        lds_barrier();
        float *op = a.o + (int64_t)win * w * a.h_v * D + (int64_t)h * D + c0;
        for (int idx = tid; idx < w * 16; idx += nt) {
            const int t = idx / 16, cc = idx % 16;
            float qs = 0.f;
            for (int d = 0; d < D; ++d) qs += ld1(qp + (int64_t)t * ldk + d) * ST[cc * ldst + d];
            float corr = 0.f, wr = 0.f;
            for (int s2 = 0; s2 <= t; ++s2) corr += ws.G[t][s2] * ws.P[s2][cc];
            for (int r = 0; r <= t; ++r) {
                float hh = 0.f;   // H_tr = sum_{r<=s<=t} QK_ts M_sr
                for (int s2 = r; s2 <= t; ++s2) hh += ws.G[t][s2] * ws.M[s2][r];
                wr += hh * ws.beta[r] * exp2f(ws.cl[t] - ws.cl[r]) * ws.V[r][cc];
            }
            const float gt = exp2f(ws.cl[t]);
            op[(int64_t)t * a.h_v * D + cc] = gt * (qs - corr) + wr;
        }
    }
    lds_barrier();
    // S' = gw S + K^T E
    for (int idx = tid; idx < D * 16; idx += nt) {
        const int cc = idx / D, d = idx % D;
        float acc = gw * ST[cc * ldst + d];
        for (int t = 0; t < w; ++t) acc += ws.K[t][d] * ws.E[t][cc];
        ST[cc * ldst + d] = acc;
    }
    lds_barrier();
}

// Window with a gate per key channel (the delta rule with a diagonal gate,
// KDA: T_t = (I - b_t k_t k_t^T) diag(g_t), u_t = b_t k_t v_t^T; ch.2 sec.3
// Table 1), applied token by token to the state block ST[16][ldst] (in
// place): S <- diag(g_t) S, then S <- S + b_t k_t (v_t^T - k_t^T S); with
// read-outs also o_t = q_t^T S after the token.  Each wave owns whole columns
// of the block, so the token loop needs no barrier.  fp32 throughout.
template <int D, int WMAX, typename TIN>
__device__ void seam_apply_diag(WinSmem<D, WMAX, 16> &ws, float *ST, int ldst, const SeamArgs &a,
                                int win, int h, int c0)
{
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6, nwv = nt >> 6;
    const int w = a.w;
    seam_stage_kv<D, WMAX, TIN, 16>(ws, a, win, h, c0);
    // gates g_t[d] (into the W rows, unused on this path) and write strengths
    const TIN *ap = reinterpret_cast<const TIN *>(a.alpha) + ((int64_t)win * w * a.h_v + h) * D;
    for (int idx = tid; idx < w * D; idx += nt) {
        const int t = idx / D, d = idx % D;
        ws.W[t][d] = ld1(ap + (int64_t)t * a.h_v * D + d);
    }
    if (tid < w) ws.beta[tid] = ld1(reinterpret_cast<const TIN *>(a.beta) + ((int64_t)win * w + tid) * a.h_v + h);
    lds_barrier();
    const int kh = h / (a.h_v / a.h_k);
    const int64_t ldk = (int64_t)a.h_k * D;
    const TIN *qp = a.q ? reinterpret_cast<const TIN *>(a.q) + (int64_t)win * w * ldk + (int64_t)kh * D : nullptr;
    float *op = a.o ? a.o + (int64_t)win * w * a.h_v * D + (int64_t)h * D + c0 : nullptr;
    for (int t = 0; t < w; ++t) {
        const float bt = ws.beta[t];
        for (int cc = wv; cc < 16; cc += nwv) {
            float *col = ST + cc * ldst;
            float x = 0.f;
            for (int d = lane; d < D; d += 64) {
                const float sv = col[d] * ws.W[t][d];
                col[d] = sv;
                x += ws.K[t][d] * sv;
            }
            x = wave_sum(x);
            const float coef = bt * (ws.V[t][cc] - x);
            float o = 0.f;
            for (int d = lane; d < D; d += 64) {
                const float sv = col[d] + coef * ws.K[t][d];
                col[d] = sv;
                if (qp) o += ld1(qp + (int64_t)t * ldk + d) * sv;
            }
            if (qp) {
                o = wave_sum(o);
                if (lane == 0) op[(int64_t)t * a.h_v * D + cc] = o;
            }
        }
    }
    lds_barrier();
}

// Workspace record of one (window, head): the window's operators, fp32, with
// the token count padded to wp = w rounded up to 4 (padding rows are zero):
//   W  [wp][D]  M diag(b) K                       (token-major)
//   K  [wp][D]  keys after conv and normalisation (token-major)
//   UT [D][wp]  (M diag(b dec) V)^T               (value column-major)
// with read-outs (ro) also, o_t = A_t^T S + C_t for the state S entering the
// window (the read-out formula above, split into its state-linear part and
// the rest):
//   A  [wp][D]  gam_t (q_t - sum_{s<=t} (q_t.k_s) W_s)
//   C  [wp][D]  sum_{r<=t} H_tr b_r (gam_t / gam_r) v_r
// and last
//   gw          gate product over the window
__host__ __device__ __forceinline__ int winop_wp(int w) { return (w + 3) & ~3; }
template <int D>
__host__ __device__ __forceinline__ int64_t winop_gw(int w, bool ro) { return (int64_t)(ro ? 5 : 3) * winop_wp(w) * D; }
template <int D>
__host__ __device__ __forceinline__ int64_t winop_floats(int w, bool ro) { return winop_gw<D>(w, ro) + 4; }

// Read-out operators of one (window, head) (one wave; K, V rows of this lane's
// columns d = lane + 64 c in registers, M and the gates in LDS):
//   A_t = gam_t (q_t - sum_{s<=t} (q_t.k_s) W_s),  W_s = sum_{r<=s} M_sr b_r k_r,
//   C_t = sum_{r<=t} H_tr b_r (gam_t / gam_r) v_r, H_tr = sum_{r<=s<=t} (q_t.k_s) M_sr.
template <int D, int WM>
__device__ __forceinline__ void seam_ops_readout(const SeamArgs &a, const float (&Q)[WM][D / 64],
                                                 const float (&K)[WM][D / 64], const float (&V)[WM][D / 64],
                                                 float (&QK)[WM][WM + 1], float (&H)[WM][WM + 1],
                                                 const float (&M)[WM][WM + 1], const float *bq, const float *cl,
                                                 float *o)
{
    constexpr int C = D / 64, NQ = WM * (WM + 1) / 2;
    const int lane = threadIdx.x, w = a.w, wp = winop_wp(w);
    {   // q_t.k_s for s <= t, all reduced together
        float dot[NQ];
#pragma unroll
        for (int t = 0, p = 0; t < WM; ++t)
#pragma unroll
            for (int s = 0; s <= t; ++s, ++p) {
                dot[p] = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) dot[p] += Q[t][c] * K[s][c];
            }
#pragma unroll
        for (int p = 0; p < NQ; ++p) dot[p] = wave_sum(dot[p]);
        if (lane == 0) {
#pragma unroll
            for (int t = 0, p = 0; t < WM; ++t)
#pragma unroll
                for (int s = 0; s <= t; ++s, ++p) QK[t][s] = dot[p];
        }
    }
    __syncthreads();
    for (int e = lane; e < WM * WM; e += 64) {   // H_tr b_r gam_t / gam_r, r <= t
        const int t = e / WM, r = e % WM;
        float acc = 0.f;
        for (int s = r; s <= t; ++s) acc += QK[t][s] * M[s][r];
        H[t][r] = r <= t ? acc * bq[r] * exp2f(cl[t] - cl[r]) : 0.f;
    }
    __syncthreads();
    float *oA = o + (int64_t)3 * wp * D, *oC = o + (int64_t)4 * wp * D;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int d = lane + 64 * c;
        float Wd[WM];
#pragma unroll
        for (int t = 0; t < WM; ++t) {
            float sw = 0.f;
#pragma unroll
            for (int r = 0; r <= t; ++r) sw += M[t][r] * bq[r] * K[r][c];
            Wd[t] = sw;
        }
#pragma unroll
        for (int t = 0; t < WM; ++t) {
            float sa = Q[t][c], sc = 0.f;
#pragma unroll
            for (int s = 0; s <= t; ++s) sa -= QK[t][s] * Wd[s];
#pragma unroll
            for (int r = 0; r <= t; ++r) sc += H[t][r] * V[r][c];
            const bool in = t < w;
            if (t < wp) {
                oA[(int64_t)t * D + d] = in ? exp2f(cl[t]) * sa : 0.f;
                oC[(int64_t)t * D + d] = in ? sc : 0.f;
            }
        }
    }
}

// One wave per (window, value head): every operator of the window, with the
// key and value rows held in registers (C = D/64 columns per lane) and the
// small w x w factors in LDS.  WM (8 or 16) bounds w; every loop over tokens
// runs to WM with rows beyond w zero, so reductions interleave without branches.
template <int D, int WM, typename TIN, bool RO>
__global__ void __launch_bounds__(64) seam_ops_kernel(const SeamArgs a, float *ops)
{
    constexpr int C = D / 64, XR = WM + 3, NP = WM * (WM - 1) / 2;
    __shared__ float G[WM][WM + 1];   // b_r k_r.k_s, s < r
    __shared__ float M[WM][WM + 1];   // (I + G)^-1, unit lower triangular
    __shared__ float bq[WM], bd[WM];  // b_q and b_q dec_q
    __shared__ float QK[WM][WM + 1];  // q_t.k_s, s <= t (read-outs)
    __shared__ float H[WM][WM + 1];   // sum_{r<=s<=t} QK_ts M_sr b_r gam_t / gam_r (read-outs)
    __shared__ float cl[WM];          // log2 gam_t (read-outs)
    const int lane = threadIdx.x;
    const int win = blockIdx.x / a.h_v, h = blockIdx.x % a.h_v;
    const int w = a.w, Wc = a.conv_w, wp = winop_wp(w);
    const int kh = h / (a.h_v / a.h_k);
    const int64_t ldk = (int64_t)a.h_k * D, ldv = (int64_t)a.h_v * D;
    const TIN *xk = reinterpret_cast<const TIN *>(a.xk) + (int64_t)win * w * ldk + (int64_t)kh * D;
    const TIN *xv = reinterpret_cast<const TIN *>(a.xv) + (int64_t)win * w * ldv + (int64_t)h * D;
    const TIN *tk = Wc > 1 ? reinterpret_cast<const TIN *>(a.tail_k) + (int64_t)win * (Wc - 1) * ldk + (int64_t)kh * D : nullptr;
    const TIN *tv = Wc > 1 ? reinterpret_cast<const TIN *>(a.tail_v) + (int64_t)win * (Wc - 1) * ldv + (int64_t)h * D : nullptr;
    // RO: with the window's read-out operators (the records are laid out for them)
    constexpr bool ro = RO && WM <= 8;
    float *o = ops + ((int64_t)win * a.h_v + h) * winop_floats<D>(w, RO);

    // gates first (their loads overlap the row loads): b, suffix decay, window product
    float gb = 0.f, gl2 = 0.f;
    if (lane < w) {
        gb = ld1(reinterpret_cast<const TIN *>(a.beta) + ((int64_t)win * w + lane) * a.h_v + h);
        gl2 = log2f(ld1(reinterpret_cast<const TIN *>(a.alpha) + ((int64_t)win * w + lane) * a.h_v + h));
    }

    // final queries of the window (read-outs), loads in flight with the rows below
    float Q[WM][C];
#pragma unroll
    for (int t = 0; t < WM; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) Q[t][c] = 0.f;
    if constexpr (ro) {
        {
            const TIN *qp = reinterpret_cast<const TIN *>(a.q) + (int64_t)win * w * ldk + (int64_t)kh * D;
#pragma unroll
            for (int t = 0; t < WM; ++t)
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const float x = ld1(qp + (int64_t)(t < w ? t : 0) * ldk + lane + 64 * c);
                    Q[t][c] = t < w ? x : 0.f;
                }
        }
    }

    // keys and values after the causal conv: the extended rows (Wc - 1 tail rows,
    // then the window) are loaded once; x_s sits in extended row s + Wc - 1, so
    // tap j of output t reads row t + j
    float K[WM][C], V[WM][C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int d = lane + 64 * c;
        const int nh = Wc > 1 ? Wc - 1 : 0;
        float xk_[XR], xv_[XR];
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            // row address selected (no branch): tail row, window row, or past the
            // window (clamped to the last row and masked to 0)
            const int tt = r - nh;
            const bool in = tt < w;
            const int ti = in ? tt : w - 1;
            const TIN *pk = ti >= 0 ? xk + (int64_t)ti * ldk : tk + (int64_t)(nh + ti) * ldk;
            const TIN *pv = ti >= 0 ? xv + (int64_t)ti * ldv : tv + (int64_t)(nh + ti) * ldv;
            const float kx = ld1(pk + d), vx = ld1(pv + d);
            xk_[r] = in ? kx : 0.f;
            xv_[r] = in ? vx : 0.f;
        }
        // the taps as four independent loads (index clamped into the row, weight 0
        // past the conv width), so they are in flight together with the rows above
        float wk[4] = {0.f, 0.f, 0.f, 0.f}, wvv[4] = {0.f, 0.f, 0.f, 0.f};
        if (Wc > 0) {   // no weights without a conv (the pointers may be null)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int jj = min(j, Wc - 1);
                const float xk = a.conv_wk[((int64_t)kh * D + d) * Wc + jj];
                const float xv = a.conv_wv[((int64_t)h * D + d) * Wc + jj];
                wk[j] = j < Wc ? xk : 0.f;
                wvv[j] = j < Wc ? xv : 0.f;
            }
        }
#pragma unroll
        for (int t = 0; t < WM; ++t) {
            float yk = 0.f, yv = 0.f;
            if (Wc > 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    yk += wk[j] * xk_[t + j];   // taps beyond Wc have weight 0
                    yv += wvv[j] * xv_[t + j];
                }
            } else {
                yk = xk_[t];
                yv = xv_[t];
            }
            K[t][c] = t < w ? yk : 0.f;
            V[t][c] = t < w ? yv : 0.f;
        }
    }
    if (a.k_l2norm) {
        float ss[WM];
#pragma unroll
        for (int t = 0; t < WM; ++t) {
            ss[t] = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) ss[t] += K[t][c] * K[t][c];
        }
#pragma unroll
        for (int t = 0; t < WM; ++t) ss[t] = wave_sum(ss[t]);
#pragma unroll
        for (int t = 0; t < WM; ++t) {
            const float inv = ss[t] > 0.f ? 1.f / sqrtf(ss[t]) : 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) K[t][c] *= inv;
        }
    }
    {
        const float sfx = wave_suffix_excl(gl2);
        const double tot = wave_sum_f64((double)gl2);
        if (lane < WM) {
            bq[lane] = gb;
            bd[lane] = gb * exp2f(sfx);
        }
        if (lane == 0) o[winop_gw<D>(w, RO)] = scale_pow2(1.f, tot);
        if constexpr (ro) {   // log2 gam_t, inclusive prefix
            const float pre = wave_prefix_incl(gl2);
            if (lane < WM) cl[lane] = pre;
        }
    }
    // Gram pairs r > q, all reduced together
    {
        float dot[NP];
#pragma unroll
        for (int r = 1, p = 0; r < WM; ++r)
#pragma unroll
            for (int q = 0; q < r; ++q, ++p) {
                dot[p] = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) dot[p] += K[r][c] * K[q][c];
            }
#pragma unroll
        for (int p = 0; p < NP; ++p) dot[p] = wave_sum(dot[p]);
        __syncthreads();   // bq visible
        if (lane == 0) {
#pragma unroll
            for (int r = 1, p = 0; r < WM; ++r)
#pragma unroll
                for (int q = 0; q < r; ++q, ++p) G[r][q] = bq[r] * dot[p];
        }
    }
    __syncthreads();
    // M = (I + G)^-1: lane c < WM owns column c; rows of G are broadcast reads
    if (lane < WM) {
        const int c = lane;
        float mc[WM];
#pragma unroll
        for (int r = 0; r < WM; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) acc -= (q >= c ? G[r][q] : 0.f) * mc[q];
            mc[r] = r >= c ? acc : 0.f;
            M[r][c] = mc[r];
        }
    }
    __syncthreads();
    float *oW = o, *oK = o + (int64_t)wp * D, *oUT = o + (int64_t)2 * wp * D;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int d = lane + 64 * c;
        float Wd[WM], Ud[WM];
#pragma unroll
        for (int t = 0; t < WM; ++t) {
            float sw = 0.f, su = 0.f;
#pragma unroll
            for (int q = 0; q <= t; ++q) {
                const float m = M[t][q];
                sw += m * bq[q] * K[q][c];
                su += m * bd[q] * V[q][c];
            }
            Wd[t] = t < w ? sw : 0.f;
            Ud[t] = t < w ? su : 0.f;
        }
#pragma unroll
        for (int t = 0; t < WM; ++t)
            if (t < wp) {
                oW[(int64_t)t * D + d] = Wd[t];
                oK[(int64_t)t * D + d] = K[t][c];
            }
#pragma unroll
        for (int t4 = 0; t4 < WM; t4 += 4)
            if (t4 < wp)
                *reinterpret_cast<float4 *>(oUT + (int64_t)d * wp + t4) = make_float4(Ud[t4], Ud[t4 + 1], Ud[t4 + 2], Ud[t4 + 3]);
    }
    if constexpr (ro)   // read-outs ride on windows of up to 8 rows
        seam_ops_readout<D, WM>(a, Q, K, V, QK, H, M, bq, cl, o);
}

}  // namespace hy

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

// Window prep: everything that does not depend on the state (value columns
// [c0, c0 + NC) of head h).
template <int D, int WMAX, typename TIN, int NC = 16>
__device__ void seam_prep(WinSmem<D, WMAX, NC> &ws, const SeamArgs &a, int win, int h, int c0)
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

// Workspace record of one (window, head): the window's operators, fp32.
//   K  [w][D]  keys after conv and normalisation
//   W  [w][D]  M diag(b) K
//   UT [D][w]  (M diag(b dec) V)^T, value column-major
//   gw         gate product over the window
template <int D>
__host__ __device__ __forceinline__ int64_t winop_floats(int w) { return (int64_t)3 * w * D + 4; }

// One workgroup per (window, head): window operators into the workspace.
template <int D, typename TIN>
__global__ void __launch_bounds__(256) seam_ops_kernel(const SeamArgs a, float *ops)
{
    __shared__ WinSmem<D, 16, D> ws;
    const int win = blockIdx.x / a.h_v, h = blockIdx.x % a.h_v;
    seam_prep<D, 16, TIN, D>(ws, a, win, h, 0);
    const int w = a.w;
    float *o = ops + ((int64_t)win * a.h_v + h) * winop_floats<D>(w);
    for (int idx = threadIdx.x; idx < w * D; idx += blockDim.x) {
        const int t = idx / D, d = idx % D;
        o[idx] = ws.K[t][d];
        o[w * D + idx] = ws.W[t][d];
    }
    for (int idx = threadIdx.x; idx < w * D; idx += blockDim.x) {
        const int cc = idx / w, t = idx % w;
        o[2 * w * D + idx] = ws.U[t][cc];
    }
    if (threadIdx.x == 0) o[3 * w * D] = ws.gw;
}

}  // namespace hy

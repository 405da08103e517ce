// compose.hip -- folding cached pairs into a running state, S <- T_C S + S_{C|0}
// per segment in prompt order (HYPIC reading notes ch.2 sec.2, Eq. (6)), with
// the seam window of each inner segment applied first (ch.2 secs.5-6), and
// the standalone seam advance.
//
// Dense T (gated delta): one workgroup per (value head, 16-column block) of the
// state; the columns of S evolve independently under T*, so the chain is
// serial only in the segment index.  The block lives in LDS (double-buffered);
// each wave owns a band of rows and streams its rows of T straight from HBM
// into registers one segment ahead.  Products are fp32 (16x16x4) or fp32
// operands split into bf16 hi+lo with three products per term.
// Scalar / diagonal T: S <- t * S + S0 streamed element-wise, fp32 FMA.
#include "common.h"
#include "launch.h"
#include "seam.h"

namespace hy {

template <int D, bool SPLIT>
struct ComposeCfg {
    static constexpr int NW = D >= 64 ? 4 : D / 16;   // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int MTW = D / 16 / NW;           // 16-row tiles per wave
    static constexpr int LDS_ = D + 4;                // ST row stride (floats)
    static constexpr int AQ = D / 4;                  // A-operand floats per lane per tile
};

template <int D, bool SEAMS>
struct ComposeSmem {
    float ST[2][16][D + 4];
    WinSmem<D, SEAMS ? 16 : 1> win;
};

template <int D, bool SPLIT, bool SEAMS, typename TIN>
__global__ void __launch_bounds__((ComposeCfg<D, SPLIT>::NT))
compose_dense_kernel(const ComposeArgs a)
{
    using C = ComposeCfg<D, SPLIT>;
    constexpr int MTW = C::MTW, AQ = C::AQ, LD = C::LDS_;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ComposeSmem<D, SEAMS> &sm = *reinterpret_cast<ComposeSmem<D, SEAMS> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int nblk = D / 16;
    // the column blocks of one head run on one XCD and share T through its L2
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int h = lb / nblk, c0 = 16 * (lb % nblk);
    const int64_t hoff = (int64_t)h * D * D;

    for (int idx = tid; idx < 16 * D; idx += C::NT) {
        const int cc = idx / D, d = idx % D;
        sm.ST[0][cc][d] = a.S_in ? a.S_in[hoff + (int64_t)d * D + c0 + cc] : 0.f;
    }

    // this wave's rows: 16*(MTW*wv + mt) + (lane&15) for the A operand
    float Acur[MTW][AQ], Anext[MTW][AQ];
    float Scur[MTW][4], Snext[MTW][4];
    auto fetch = [&](int j, float (&A)[MTW][AQ], float (&S0)[MTW][4]) {
        const int slot = a.order[j];
        const float *T = a.T_pool + (int64_t)slot * a.h_v * D * D + hoff;
        const float *S0p = a.S0_pool + (int64_t)slot * a.h_v * D * D + hoff;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            const int row = 16 * (MTW * wv + mt) + r16;
            if constexpr (SPLIT) {
#pragma unroll
                for (int kb = 0; kb < D / 32; ++kb) {
                    const float4 *p = reinterpret_cast<const float4 *>(T + (int64_t)row * D + 32 * kb + 8 * g);
                    const float4 x0 = p[0], x1 = p[1];
                    A[mt][8 * kb + 0] = x0.x; A[mt][8 * kb + 1] = x0.y; A[mt][8 * kb + 2] = x0.z; A[mt][8 * kb + 3] = x0.w;
                    A[mt][8 * kb + 4] = x1.x; A[mt][8 * kb + 5] = x1.y; A[mt][8 * kb + 6] = x1.z; A[mt][8 * kb + 7] = x1.w;
                }
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(T + (int64_t)row * D + g * AQ);
#pragma unroll
                for (int q = 0; q < AQ / 4; ++q) {
                    const float4 x = p[q];
                    A[mt][4 * q + 0] = x.x; A[mt][4 * q + 1] = x.y; A[mt][4 * q + 2] = x.z; A[mt][4 * q + 3] = x.w;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S0[mt][i] = S0p[(int64_t)(16 * (MTW * wv + mt) + 4 * g + i) * D + c0 + r16];
        }
    };

    int cur = 0;
    if (a.n > 0) fetch(0, Acur, Scur);
    for (int j = 0; j < a.n; ++j) {
        if (j + 1 < a.n) fetch(j + 1, Anext, Snext);
        lds_barrier();
        if constexpr (SEAMS) {
            const int pos = a.first_pos + j;
            if (a.has_seams && pos >= 1) {
                if (a.seam.gate_diag) {
                    seam_apply_diag<D, 16, TIN>(sm.win, &sm.ST[cur][0][0], LD, a.seam, pos - 1, h, c0);
                } else {
                    seam_prep<D, 16, TIN>(sm.win, a.seam, pos - 1, h, c0);
                    seam_apply<D, 16, TIN>(sm.win, &sm.ST[cur][0][0], LD, a.seam, pos - 1, h, c0);
                }
            }
        }
        // S_next = T S + S0 for this wave's rows
        const float(*ST)[LD] = sm.ST[cur];
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            f4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = Scur[mt][i];
            if constexpr (SPLIT) {
#pragma unroll
                for (int kb = 0; kb < D / 32; ++kb) {
                    const float4 *bp = reinterpret_cast<const float4 *>(&ST[r16][32 * kb + 8 * g]);
                    const float4 y0 = bp[0], y1 = bp[1];
                    const float bx[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
                    b8 Ah, Al, Bh, Bl;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        __bf16 hi, lo;
                        split_bf16(Acur[mt][8 * kb + e], hi, lo);
                        Ah[e] = hi; Al[e] = lo;
                        split_bf16(bx[e], hi, lo);
                        Bh[e] = hi; Bl[e] = lo;
                    }
                    acc = mma(Al, Bh, acc);
                    acc = mma(Ah, Bl, acc);
                    acc = mma(Ah, Bh, acc);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < AQ; ++ks) acc = mma(Acur[mt][ks], ST[r16][g * AQ + ks], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.ST[cur ^ 1][r16][16 * (MTW * wv + mt) + 4 * g + i] = acc[i];
        }
        cur ^= 1;
        if (j + 1 < a.n) {
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
                for (int q = 0; q < AQ; ++q) Acur[mt][q] = Anext[mt][q];
#pragma unroll
                for (int i = 0; i < 4; ++i) Scur[mt][i] = Snext[mt][i];
            }
        }
    }
    lds_barrier();
    for (int idx = tid; idx < 16 * D; idx += C::NT) {
        const int cc = idx / D, d = idx % D;
        a.S_out[hoff + (int64_t)d * D + c0 + cc] = sm.ST[cur][cc][d];
    }
}

// Scalar / diagonal transitions: each thread owns 4 consecutive state columns.
template <int D, bool DIAG>
__global__ void __launch_bounds__(256) compose_decay_kernel(const ComposeArgs a)
{
    const int64_t total4 = (int64_t)a.h_v * D * D / 4;
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < total4;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = 4 * q;
        const int hh = (int)(e / (D * D));
        const int row = (int)((e / D) % D);
        float4 S = a.S_in ? reinterpret_cast<const float4 *>(a.S_in)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < a.n; ++j) {
            const int slot = a.order[j];
            const float t = DIAG ? a.T_pool[((int64_t)slot * a.h_v + hh) * D + row]
                                 : a.T_pool[(int64_t)slot * a.h_v + hh];
            const float4 s0 = reinterpret_cast<const float4 *>(a.S0_pool + (int64_t)slot * a.h_v * D * D)[q];
            S.x = fmaf(t, S.x, s0.x);
            S.y = fmaf(t, S.y, s0.y);
            S.z = fmaf(t, S.z, s0.z);
            S.w = fmaf(t, S.w, s0.w);
        }
        reinterpret_cast<float4 *>(a.S_out)[q] = S;
    }
}

// Standalone seam advance over windows 0..n_win-1 of a.seam, state in S (in place).
template <int D, typename TIN>
__global__ void __launch_bounds__(256) seam_kernel(const ComposeArgs a, float *S, int n_win)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    float(*ST)[D + 4] = reinterpret_cast<float(*)[D + 4]>(smem_raw);
    WinSmem<D, 64> &ws = *reinterpret_cast<WinSmem<D, 64> *>(smem_raw + sizeof(float) * 16 * (D + 4));
    const int tid = threadIdx.x;
    const int nblk = D / 16;
    const int h = blockIdx.x / nblk, c0 = 16 * (blockIdx.x % nblk);
    const int64_t hoff = (int64_t)h * D * D;
    for (int idx = tid; idx < 16 * D; idx += blockDim.x) {
        const int cc = idx / D, d = idx % D;
        ST[cc][d] = S[hoff + (int64_t)d * D + c0 + cc];
    }
    const SeamArgs &sa = a.seam;
    for (int win = 0; win < n_win; ++win) {
        lds_barrier();
        if (sa.gate_diag) {   // per-channel gates: token by token (no window pair)
            seam_apply_diag<D, 64, TIN>(ws, &ST[0][0], D + 4, sa, win, h, c0);
            continue;
        }
        seam_prep<D, 64, TIN>(ws, sa, win, h, c0);
        // window pair: T_w[:, cols of this block] and S_w0[:, cols]
        if (sa.T_w) {
            float *Tw = sa.T_w + ((int64_t)win * a.h_v + h) * D * D;
            for (int idx = tid; idx < D * 16; idx += blockDim.x) {
                const int d = idx / 16, cc = idx % 16;
                float acc = 0.f;
                for (int t = 0; t < sa.w; ++t) acc += ws.K[t][d] * ws.W[t][c0 + cc];
                Tw[(int64_t)d * D + c0 + cc] = ws.gw * (((d == c0 + cc) ? 1.f : 0.f) - acc);
            }
        }
        if (sa.S_w0) {
            float *Sw = sa.S_w0 + ((int64_t)win * a.h_v + h) * D * D;
            for (int idx = tid; idx < D * 16; idx += blockDim.x) {
                const int d = idx / 16, cc = idx % 16;
                float acc = 0.f;
                for (int t = 0; t < sa.w; ++t) acc += ws.K[t][d] * ws.U[t][cc];
                Sw[(int64_t)d * D + c0 + cc] = acc;
            }
        }
        seam_apply<D, 64, TIN>(ws, &ST[0][0], D + 4, sa, win, h, c0);
    }
    lds_barrier();
    for (int idx = tid; idx < 16 * D; idx += blockDim.x) {
        const int cc = idx / D, d = idx % D;
        S[hoff + (int64_t)d * D + c0 + cc] = ST[cc][d];
    }
}

template <int D, bool SPLIT, bool SEAMS, typename TIN>
static hipError_t launch_dense(const ComposeArgs &a, hipStream_t st)
{
    using C = ComposeCfg<D, SPLIT>;
    const size_t smem = sizeof(ComposeSmem<D, SEAMS>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&compose_dense_kernel<D, SPLIT, SEAMS, TIN>, smem, lds_set); e != hipSuccess)
        return e;
    hipLaunchKernelGGL((compose_dense_kernel<D, SPLIT, SEAMS, TIN>), dim3(a.h_v * (D / 16)),
                       dim3(C::NT), smem, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_compose_d(const ComposeArgs &a, int tform, int prec, int in_kind,
                                   hipStream_t st)
{
    if (tform == HYPIC_T_DENSE) {
        const bool split = (prec == HYPIC_PREC_SPLIT) && D >= 32;
        if (a.has_seams) {
            if (in_kind == IN_BF16)
                return split ? launch_dense<D, true, true, bf16_t>(a, st) : launch_dense<D, false, true, bf16_t>(a, st);
            return split ? launch_dense<D, true, true, float>(a, st) : launch_dense<D, false, true, float>(a, st);
        }
        return split ? launch_dense<D, true, false, float>(a, st) : launch_dense<D, false, false, float>(a, st);
    }
    const int64_t total4 = (int64_t)a.h_v * D * D / 4;
    const int grid = (int)((total4 + 255) / 256);
    if (tform == HYPIC_T_DIAG)
        hipLaunchKernelGGL((compose_decay_kernel<D, true>), dim3(grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((compose_decay_kernel<D, false>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_compose(const ComposeArgs &a, int D, int tform, int prec, int in_kind,
                          hipStream_t st)
{
    switch (D) {
    case 16: return launch_compose_d<16>(a, tform, prec, in_kind, st);
    case 32: return launch_compose_d<32>(a, tform, prec, in_kind, st);
    case 64: return launch_compose_d<64>(a, tform, prec, in_kind, st);
    case 128: return launch_compose_d<128>(a, tform, prec, in_kind, st);
    default: return hipErrorInvalidValue;
    }
}

template <int D, typename TIN>
static hipError_t launch_seam_t(const ComposeArgs &a, float *S, int n_win, hipStream_t st)
{
    const size_t smem = sizeof(float) * 16 * (D + 4) + sizeof(WinSmem<D, 64>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&seam_kernel<D, TIN>, smem, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL((seam_kernel<D, TIN>), dim3(a.h_v * (D / 16)), dim3(256), smem, st, a, S, n_win);
    return hipGetLastError();
}

hipError_t launch_seam(const ComposeArgs &a, int D, int in_kind, float *S, int n_win, hipStream_t st)
{
    const bool bf = in_kind == IN_BF16;
    switch (D) {
    case 16: return bf ? launch_seam_t<16, bf16_t>(a, S, n_win, st) : launch_seam_t<16, float>(a, S, n_win, st);
    case 32: return bf ? launch_seam_t<32, bf16_t>(a, S, n_win, st) : launch_seam_t<32, float>(a, S, n_win, st);
    case 64: return bf ? launch_seam_t<64, bf16_t>(a, S, n_win, st) : launch_seam_t<64, float>(a, S, n_win, st);
    case 128: return bf ? launch_seam_t<128, bf16_t>(a, S, n_win, st) : launch_seam_t<128, float>(a, S, n_win, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hy

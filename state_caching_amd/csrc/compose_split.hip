// compose_split.hip -- dense composition S <- T_C S + S_{C|0} over a prompt's
// segments (HYPIC reading notes ch.2 sec.2, Eq. (6)) with the seam window of
// every inner segment applied first (ch.2 secs.5-6), for d in {64, 128}:
// fp32 operands split into bf16 hi + lo, three matrix-core products per term.
//
// One workgroup (4 waves) per (value head, 16-column block) of the state;
// column blocks of a head share an XCD so T is fetched once into that L2.
// Each wave owns d/4 rows: its rows of T and S0 stream from memory through a
// 4-deep register ring, so several segments' operands are in flight while
// the serial chain advances.  The state block lives in LDS already split into
// bf16 hi/lo (every reader needs it split); each wave also keeps its own rows
// in fp32 registers for the seam update and the final write.
//
// Seam (window operators precomputed per (window, head) by seam_ops_kernel:
// K [w][d], W = M diag(b) K [w][d], U^T [d][w], gw):
//   P  = W S               (w x 16, every wave)
//   E  = U - gw P
//   S' = gw S + K^T E      (each wave its own rows)
//   S  <- T S' + S0
#include "common.h"
#include "launch.h"
#include "seam.h"

namespace hy {

template <int D>
struct CsCfg {
    static constexpr int NT = 256;
    static constexpr int MTW = D / 64;   // 16-row tiles per wave
    static constexpr int KB = D / 32;
    static constexpr int NST = 4;        // register ring depth (segments in flight)
    static constexpr int LDB = D + 8;    // split-state row stride (bf16)
    static constexpr int WMAXF = 16;     // window tokens held (zero-padded)
};

template <int D, bool SEAMS>
struct CsSmem {
    using C = CsCfg<D>;
    uint16_t SH[2][16][C::LDB];          // state hi, [column][row]
    uint16_t SL[2][16][C::LDB];          // state lo
    uint16_t WH[SEAMS ? 16 : 1][C::LDB]; // window W rows hi (token-major), zero beyond w
    uint16_t WL[SEAMS ? 16 : 1][C::LDB];
    float KT[SEAMS ? D : 1][20];         // window keys transposed [row][token]
    float UT[16][20];                    // window U of this column block [column][token]
    float gw;
};

__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 x8 -> bf16 hi/lo fragments
__device__ __forceinline__ void split8(const float (&x)[8], b8 &hi, b8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)x[e];
        hi[e] = h;
        lo[e] = (__bf16)(x[e] - (float)h);
    }
}
__device__ __forceinline__ f4 mma3(const b8 &ah, const b8 &al, const b8 &bh, const b8 &bl, f4 c) {
    c = mma(al, bh, c);
    c = mma(ah, bl, c);
    return mma(ah, bh, c);
}
__device__ __forceinline__ b8 ld_b8(const uint16_t *p) { return *reinterpret_cast<const b8 *>(p); }

template <int D, bool SEAMS>
__global__ void __launch_bounds__(256) compose_split_kernel(const ComposeArgs a, const float *ops)
{
    using C = CsCfg<D>;
    constexpr int MTW = C::MTW, KB = C::KB, NST = C::NST;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    CsSmem<D, SEAMS> &sm = *reinterpret_cast<CsSmem<D, SEAMS> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int h = lb / (D / 16), c0 = 16 * (lb % (D / 16));
    const int64_t hoff = (int64_t)h * D * D;
    const int w = SEAMS ? a.seam.w : 0;

    // initial state: split copy in LDS, own rows in fp32 registers
    f4 Sown[MTW];
    for (int idx = tid; idx < 16 * D; idx += C::NT) {
        const int cc = idx / D, d = idx % D;
        const float x = a.S_in ? a.S_in[hoff + (int64_t)d * D + c0 + cc] : 0.f;
        const uint16_t hb = bf16_bits(x);
        sm.SH[0][cc][d] = hb;
        sm.SL[0][cc][d] = bf16_bits(x - bf16_val(hb));
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * (MTW * wv + mt) + 4 * g + i;
            Sown[mt][i] = a.S_in ? a.S_in[hoff + (int64_t)row * D + c0 + r16] : 0.f;
        }
    if constexpr (SEAMS) {
        for (int idx = tid; idx < 16 * C::LDB; idx += C::NT) {
            (&sm.WH[0][0])[idx] = 0;
            (&sm.WL[0][0])[idx] = 0;
        }
        for (int idx = tid; idx < D * 20; idx += C::NT) (&sm.KT[0][0])[idx] = 0.f;
        for (int idx = tid; idx < 16 * 20; idx += C::NT) (&sm.UT[0][0])[idx] = 0.f;
    }

    // ---- register ring of T rows and S0 rows ---------------------------------
    float Tb[NST][MTW][D / 4];
    float S0b[NST][MTW][4];
    auto fetch = [&](int j, float (&T)[MTW][D / 4], float (&S0)[MTW][4]) {
        const int slot = a.order[j];
        const float *Tp = a.T_pool + (int64_t)slot * a.h_v * D * D + hoff;
        const float *Sp = a.S0_pool + (int64_t)slot * a.h_v * D * D + hoff;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            const int row = 16 * (MTW * wv + mt) + r16;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float4 *p = reinterpret_cast<const float4 *>(Tp + (int64_t)row * D + 32 * kb + 8 * g);
                const float4 x0 = p[0], x1 = p[1];
                T[mt][8 * kb + 0] = x0.x; T[mt][8 * kb + 1] = x0.y; T[mt][8 * kb + 2] = x0.z; T[mt][8 * kb + 3] = x0.w;
                T[mt][8 * kb + 4] = x1.x; T[mt][8 * kb + 5] = x1.y; T[mt][8 * kb + 6] = x1.z; T[mt][8 * kb + 7] = x1.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S0[mt][i] = Sp[(int64_t)(16 * (MTW * wv + mt) + 4 * g + i) * D + c0 + r16];
        }
    };
    // window operators: loaded into registers two steps ahead, stored to LDS one step ahead
    constexpr int WQ = (16 * D) / (4 * 256);   // float4 per thread for K and for W (w <= 16)
    float4 wK[2][WQ], wW[2][WQ];
    float4 wU[2];
    float wg[2] = {0.f, 0.f};
    auto fetch_win = [&](int pos, int st) {     // window of prompt position pos (>= 1)
        if constexpr (SEAMS) {
            const float *o = ops + ((int64_t)(pos - 1) * a.h_v + h) * winop_floats<D>(w);
#pragma unroll
            for (int q = 0; q < WQ; ++q) {
                const int idx = 4 * (tid + 256 * q);
                wK[st][q] = idx < w * D ? *reinterpret_cast<const float4 *>(o + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
                wW[st][q] = idx < w * D ? *reinterpret_cast<const float4 *>(o + w * D + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            const int uidx = 4 * tid;   // this column block's U^T: 16 columns x w tokens, contiguous
            wU[st] = uidx < 16 * w ? *reinterpret_cast<const float4 *>(o + 2 * w * D + c0 * w + uidx)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            wg[st] = o[3 * w * D];
        }
    };
    auto store_win = [&](int st) {
        if constexpr (SEAMS) {
#pragma unroll
            for (int q = 0; q < WQ; ++q) {
                const int idx = 4 * (tid + 256 * q);
                if (idx < w * D) {
                    const int t = idx / D, d = idx % D;
                    const float kx[4] = {wK[st][q].x, wK[st][q].y, wK[st][q].z, wK[st][q].w};
                    const float wx[4] = {wW[st][q].x, wW[st][q].y, wW[st][q].z, wW[st][q].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sm.KT[d + e][t] = kx[e];
                        const uint16_t hb = bf16_bits(wx[e]);
                        sm.WH[t][d + e] = hb;
                        sm.WL[t][d + e] = bf16_bits(wx[e] - bf16_val(hb));
                    }
                }
            }
            const int uidx = 4 * tid;
            if (uidx < 16 * w) {
                const float ux[4] = {wU[st].x, wU[st].y, wU[st].z, wU[st].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.UT[(uidx + e) / w][(uidx + e) % w] = ux[e];
            }
            if (tid == 0) sm.gw = wg[st];
        }
    };

    const int n = a.n;
#pragma unroll
    for (int s = 0; s < NST; ++s)
        if (s < n) fetch(s, Tb[s], S0b[s]);
    if constexpr (SEAMS) {
        if (a.first_pos + 0 >= 1) fetch_win(a.first_pos + 0, 0);
        if (n > 1 && a.first_pos + 1 >= 1) fetch_win(a.first_pos + 1, 1);
        if (a.first_pos + 0 >= 1) store_win(0);
    }

    int cur = 0;
    f4 acc[MTW];
    for (int j0 = 0; j0 < n; j0 += NST) {
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            const int j = j0 + s;
            if (j < n) {
                const int pos = a.first_pos + j;
                const bool seam = SEAMS && pos >= 1;
                lds_barrier();   // state S_j (buffer cur) and window pos complete
                if (seam) {
                    // P = W S (every wave), E = U - gw P; tokens in rows 4g + i
                    f4 p0 = zero4(), p1 = zero4();
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const int k0 = 32 * kb + 8 * g;
                        const b8 ah = ld_b8(&sm.WH[r16][k0]), al = ld_b8(&sm.WL[r16][k0]);
                        const b8 bh = ld_b8(&sm.SH[cur][r16][k0]), bl = ld_b8(&sm.SL[cur][r16][k0]);
                        p0 = mma(ah, bh, p0);
                        p1 = mma(al, bh, p1);
                        p1 = mma(ah, bl, p1);
                    }
                    const float gwv = sm.gw;
                    b8 eh, el;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = sm.UT[r16][4 * g + i] - gwv * (p0[i] + p1[i]);
                        const __bf16 hb = (__bf16)e;
                        eh[i] = hb; el[i] = (__bf16)(e - (float)hb);
                        eh[4 + i] = (__bf16)0.f; el[4 + i] = (__bf16)0.f;
                    }
                    // S' rows of this wave = gw S + K^T E, written split to the other buffer
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) {
                        const int row = 16 * (MTW * wv + mt) + r16;
                        const float4 kk = *reinterpret_cast<const float4 *>(&sm.KT[row][4 * g]);
                        const float kx[8] = {kk.x, kk.y, kk.z, kk.w, 0.f, 0.f, 0.f, 0.f};
                        b8 ah, al;
                        split8(kx, ah, al);
                        f4 sp = Sown[mt] * gwv;
                        sp = mma3(ah, al, eh, el, sp);
                        Sown[mt] = sp;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rr = 16 * (MTW * wv + mt) + 4 * g + i;
                            const uint16_t hb = bf16_bits(sp[i]);
                            sm.SH[cur ^ 1][r16][rr] = hb;
                            sm.SL[cur ^ 1][r16][rr] = bf16_bits(sp[i] - bf16_val(hb));
                        }
                    }
                    lds_barrier();   // S' complete
                    cur ^= 1;
                }
                // S_{j+1} = T S' + S0 for this wave's rows
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    f4 c1 = zero4();
                    acc[mt] = f4{S0b[s][mt][0], S0b[s][mt][1], S0b[s][mt][2], S0b[s][mt][3]};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const int k0 = 32 * kb + 8 * g;
                        float tx[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) tx[e] = Tb[s][mt][8 * kb + e];
                        b8 ah, al;
                        split8(tx, ah, al);
                        const b8 bh = ld_b8(&sm.SH[cur][r16][k0]), bl = ld_b8(&sm.SL[cur][r16][k0]);
                        acc[mt] = mma(ah, bh, acc[mt]);
                        c1 = mma(al, bh, c1);
                        c1 = mma(ah, bl, c1);
                    }
                    acc[mt] += c1;
                }
                // ring: segment j + NST into this stage (clamped, so the refill is
                // straight-line code: no branch between the products above and the
                // reads of their results below); window two positions ahead
                fetch(min(j + NST, n - 1), Tb[s], S0b[s]);
                if constexpr (SEAMS) {
                    if (j + 1 < n && pos + 1 >= 1) store_win((j + 1) & 1);
                    if (j + 2 < n && pos + 2 >= 1) fetch_win(pos + 2, j & 1);
                }
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    Sown[mt] = acc[mt];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 16 * (MTW * wv + mt) + 4 * g + i;
                        const uint16_t hb = bf16_bits(acc[mt][i]);
                        sm.SH[cur ^ 1][r16][rr] = hb;
                        sm.SL[cur ^ 1][r16][rr] = bf16_bits(acc[mt][i] - bf16_val(hb));
                    }
                }
                cur ^= 1;
            }
        }
    }
    // final state from the fp32 rows
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * (MTW * wv + mt) + 4 * g + i;
            a.S_out[hoff + (int64_t)row * D + c0 + r16] = Sown[mt][i];
        }
}

template <int D, typename TIN>
static hipError_t launch_ops(const ComposeArgs &a, int n_win, float *ops, hipStream_t st)
{
    if (n_win <= 0) return hipSuccess;
    hipLaunchKernelGGL((seam_ops_kernel<D, TIN>), dim3(n_win * a.h_v), dim3(256), 0, st, a.seam, ops);
    return hipGetLastError();
}

template <int D, bool SEAMS>
static hipError_t launch_cs(const ComposeArgs &a, const float *ops, hipStream_t st)
{
    const size_t smem = sizeof(CsSmem<D, SEAMS>);
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&compose_split_kernel<D, SEAMS>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL((compose_split_kernel<D, SEAMS>), dim3(a.h_v * (D / 16)), dim3(256), smem, st, a, ops);
    return hipGetLastError();
}

int64_t seam_ops_floats(int D, int w, int n_win, int h_v)
{
    const int64_t per = (D == 128) ? winop_floats<128>(w) : winop_floats<64>(w);
    return per * n_win * h_v;
}

hipError_t launch_seam_ops(const ComposeArgs &a, int D, int in_kind, int n_win, float *ops, hipStream_t st)
{
    const bool bf = in_kind == IN_BF16;
    if (D == 128) return bf ? launch_ops<128, bf16_t>(a, n_win, ops, st) : launch_ops<128, float>(a, n_win, ops, st);
    if (D == 64) return bf ? launch_ops<64, bf16_t>(a, n_win, ops, st) : launch_ops<64, float>(a, n_win, ops, st);
    return hipErrorInvalidValue;
}

hipError_t launch_compose_split(const ComposeArgs &a, int D, const float *ops, hipStream_t st)
{
    if (D == 128) return a.has_seams ? launch_cs<128, true>(a, ops, st) : launch_cs<128, false>(a, ops, st);
    if (D == 64) return a.has_seams ? launch_cs<64, true>(a, ops, st) : launch_cs<64, false>(a, ops, st);
    return hipErrorInvalidValue;
}

}  // namespace hy

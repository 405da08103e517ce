// build_delta_f16.hip -- chunkwise gated-delta build with fp16 matrix-core
// operands, for d_k = d_v in {64, 128} (HYPIC reading notes: the cached pair
// of a segment, ch.2 secs.2 and 4; the gated-delta family, ch.2 sec.3 Table 1).
//
// Same algebra as build_delta.hip (the compact-WY chunk update, carrying
// X = [Tbar | S] through chunks of 64 tokens), organised as a two-stage
// software pipeline inside one workgroup per (segment, value head):
//
//   prep waves  (4)    : chunk c+1 -- stage K, V, gates; diagonal Gram blocks and
//                        their inverses; W = M diag(b) K and U = M diag(b dec) V
//                        into LDS
//   state waves (d/32) : chunk c   -- E = U - W Xhat, Xhat += K^T E on the
//                        wave's four 16-column tiles of X (two of Tbar, two of S);
//                        the off-diagonal Gram tiles of chunk c+1 (matrix work the
//                        prep waves hand over)
//
// Three LDS barriers per chunk; the state waves spread their matrix work over
// the phases so the matrix cores stay busy while the prep waves run their
// latency-bound steps.  Xhat is kept in power-of-two units per
// column tile (renormalised every 4 chunks, or when the value scale runs
// ahead of the state), so every computed fp16 operand stays in range.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace hy {

template <int D>
struct F16Cfg {
    static constexpr int NS = D / 32;         // state waves, four column tiles each
    static constexpr int TPW = 4;             // column tiles of X per state wave
    static constexpr int NP = 4;              // prep waves
    static constexpr int NT = 64 * (NS + NP);
    static constexpr int MT = D / 16;
    static constexpr int KB = D / 32;
    static constexpr int LDT = 72;            // row stride (halves) of token-contiguous rows
    static constexpr int LDW = D + 8;         // Ks / Vs row stride (halves)
    static constexpr int LDU = 68;            // UT row stride (floats)
    static constexpr int LDG = 68;
    static constexpr int PASSES = D / 32;     // prep staging passes of 16 rows
};

template <int D>
struct F16Smem {
    using C = F16Cfg<D>;
    _Float16 Ks[2][64][C::LDW];  // keys, token-major, per pipeline slot (K^T operands
                                 // come from transposed loads of these rows)
    _Float16 nWT[D][C::LDT];     // -W^T = -(M diag(b) K)^T, token-contiguous rows
    float UT[D][C::LDU];         // U^T (value column-major), in units of 2^sv
    _Float16 Vs[64][C::LDW];     // diag(dec) V * 2^-sv, token-major
    float Gm[64][C::LDG];        // k_r.k_s for s < r in the off-diagonal blocks; each
                                 // diagonal block holds A' = b_r k_r.k_s transposed in
                                 // its upper triangle
    float Mi[4][16][20];         // M' = (I + A'_bb)^-1 diag(b_b) per diagonal block, row-major
    // 2x2 blocked inverse of each diagonal block (per prep wave): A21 row-major,
    // M11 transposed, M22 row-major, Y = A21 M11 transposed
    float A21s[4][8][12], M11t[4][8][12], M22s[4][8][12], Yt[4][8][12];
    float beta[2][64], dec[2][64];   // b_t and dec_t = prod_{s > t} a_s, per pipeline slot
    float gb[2];                 // chunk gate product, per pipeline slot
    int sv[2];                   // value scale exponent, per pipeline slot
    float wmax[4];
    double cl_tot;
};

typedef short s4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;

// Four consecutive reduction indices of a matrix-core operand whose lane index
// (row m of A or column n of B) runs along LDS rows: storage S[k][x], x
// contiguous.  The 16 lanes of each lane group receive S[k0 + e][x0 + lane%16],
// e = 0..3 (k0 may differ between groups), through the LDS transpose load:
// lane j of a group supplies the 4-element block at S[k0 + j/4][x0 + 4 (j%4)].
__device__ __forceinline__ h4 ld_tr4(const _Float16 *S, int ld, int k0, int x0, int lane)
{
    const int j = lane & 15;
    const _Float16 *p = S + (k0 + (j >> 2)) * ld + x0 + 4 * (j & 3);
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v *)p));
}
__device__ __forceinline__ h8 cat8(h4 lo, h4 hi) { return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; }


template <int D, typename TK, typename TV, typename TG>
__global__ void __launch_bounds__((F16Cfg<D>::NT))
build_delta_f16_kernel(const DeltaArgs a)
{
    using C = F16Cfg<D>;
    constexpr int NS = C::NS, MT = C::MT, KB = C::KB;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    F16Smem<D> &sm = *reinterpret_cast<F16Smem<D> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int unit = xcd_logical_block(blockIdx.x, gridDim.x);
    const int s = unit / a.h_v, h = unit % a.h_v;
    const int kh = h / (a.h_v / a.h_k);
    const int len = a.len[s];
    const int nch = (len + 63) / 64;
    const bool is_prep = w >= NS;


    // Warp-specialised roles.  Both loops run nch + 1 iterations of three
    // barriers each, so every barrier meets all waves; prep runs one chunk ahead.
    if (is_prep) {
        // ------------------------------------------------------------ prep state
        // the prep chain sets the pace: its waves issue ahead of the state waves
        // sharing their SIMDs, which fill the gaps
        __builtin_amdgcn_s_setprio(3);
        const int ptid = tid - 64 * NS, pw = w - NS;
        constexpr int CPR = D / 8;
        const int prow = (ptid >= 0 ? ptid : 0) / CPR, pcol = 8 * ((ptid >= 0 ? ptid : 0) % CPR);
        constexpr int RPP = 256 / CPR;             // rows per pass
        const TK *kp = reinterpret_cast<const TK *>(a.k) + a.tok0[s] * a.ldk + (int64_t)kh * D;
        const TV *vp = reinterpret_cast<const TV *>(a.v) + a.tok0[s] * a.ldv + (int64_t)h * D;
        const TG *bp = reinterpret_cast<const TG *>(a.beta) + a.gtok0[s] * a.h_v + h;
        const TG *ap = reinterpret_cast<const TG *>(a.alpha) + a.gtok0[s] * a.h_v + h;
        typename Raw8<TK>::type kraw[C::PASSES];
        typename Raw8<TV>::type vraw[C::PASSES];
        // fp16 value rows from the conv carry a power-of-two factor per (row, head)
        constexpr bool VSC = std::is_same<TV, _Float16>::value;
        float vrs[C::PASSES];
        const float *vsp = VSC ? a.vscale + a.tok0[s] * a.h_v + h : nullptr;
        double cl_lane = 0.0;
        // Prefetches are straight-line loads of rows clamped into the segment (rows
        // past its end are zeroed when staged), so the compiler's load waits stay
        // exact and the next chunk's rows remain in flight across the phases.
        TG braw, araw;   // gates of the next chunk (every prep wave loads them)
        // row addresses: a per-chunk base (uniform, 64-bit) plus the row within the
        // chunk (< 64, clamped to the segment's last row) times the pitch on 24-bit
        // multiplies
        auto fetch_k = [&](int c) {
            const int last = len - 1 - 64 * c;   // >= 0 for every chunk of the segment
            const TK *kc = kp + (int64_t)(64 * c) * a.ldk + pcol;
#pragma unroll
            for (int p = 0; p < C::PASSES; ++p)
                ld_raw8(kc + __umul24(min(prow + RPP * p, last), (unsigned)a.ldk), kraw[p]);
            const int tg = min(lane, last);
            braw = bp[(int64_t)(64 * c) * a.h_v + __umul24(tg, (unsigned)a.h_v)];
            araw = ap[(int64_t)(64 * c) * a.h_v + __umul24(tg, (unsigned)a.h_v)];
        };
        auto fetch_v = [&](int c) {
            const int last = len - 1 - 64 * c;
            const TV *vc = vp + (int64_t)(64 * c) * a.ldv + pcol;
#pragma unroll
            for (int p = 0; p < C::PASSES; ++p) {
                const int r = min(prow + RPP * p, last);
                ld_raw8(vc + __umul24(r, (unsigned)a.ldv), vraw[p]);
                if constexpr (VSC) vrs[p] = vsp[(int64_t)(64 * c) * a.h_v + __umul24(r, (unsigned)a.h_v)];
                else vrs[p] = 1.f;
            }
        };
        // gates of chunk c from braw/araw (every prep wave computes them, wave 0
        // writes them): b, dec, the chunk product; the log-gate total accumulates
        // when count is set
        auto gates = [&](int c, bool count) {
            const int bc = c & 1;
            const bool gin = 64 * c + lane < len;
            const float br = gin ? to_f32(braw) : 0.f, ar = gin ? to_f32(araw) : 1.f;
            const float l2 = log2f(ar);
            const float sfx = wave_suffix_excl(l2);
            cl_lane += count ? (double)l2 : 0.0;
            const float dcv = exp2f(sfx), gbv = exp2f(sfx + l2);
            if (pw == 0) {
                sm.beta[bc][lane] = br;
                sm.dec[bc][lane] = dcv;
                if (lane == 0) sm.gb[bc] = gbv;
            }
        };
        if (nch > 0) { fetch_k(0); fetch_v(0); gates(0, true); }
        constexpr int NTW = MT / 4;   // W (and U) column tiles per prep wave
        const h4 h4z = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
        h4 Xw[NTW][4], Xu[NTW][4];    // solved row blocks, fp16 B fragments


        // chunks 0 .. nch-1, every iteration the same straight-line load stream (the
        // last one refetches its own rows); then one idle round of barriers while the
        // state waves finish the last chunk
        for (int it = 0; it < nch; ++it) {
            const int cp = it;
            constexpr bool dop = true;
            const int bp_ = cp & 1;
            // ===================== phase 1: stage keys of cp | E of column tiles 0-1
            if (dop) {
                float vm = 0.f;
#pragma unroll
                for (int p = 0; p < C::PASSES; ++p) {
                    const int t = prow + RPP * p;
                    const bool in = 64 * cp + t < len;   // rows past the end were clamped: zero them
                    mask_raw8(kraw[p], in);
                    mask_raw8(vraw[p], in);
                    float kx[8], vx[8];
                    widen8(kraw[p], kx);
                    widen8(vraw[p], vx);
                    h8 kk;
                    float pm = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        kk[e] = (_Float16)kx[e];
                        pm = fmaxf(pm, fabsf(vx[e]));
                    }
                    vm = fmaxf(vm, VSC ? pm * vrs[p] : pm);
                    *reinterpret_cast<h8 *>(&sm.Ks[bp_][t][pcol]) = kk;
                }
                vm = wave_max(vm);
                if (lane == 0) sm.wmax[pw] = vm;
                fetch_k(min(cp + 1, nch - 1));
            }
            lds_barrier();
            // ===================== phase 2: V^, diagonal Gram blocks and inverses | off-diagonal Gram, E of column tiles 2-3
            if (dop) {
                // value scale of chunk cp; V^ = diag(dec) V * 2^-sv into Vs
                {
                    const float vm = fmaxf(fmaxf(sm.wmax[0], sm.wmax[1]), fmaxf(sm.wmax[2], sm.wmax[3]));
                    const int sv = pow2_exponent(vm);
                    if (pw == 0 && lane == 0) sm.sv[bp_] = sv;
                    const float vsc = exp2f(-(float)sv);
#pragma unroll
                    for (int p = 0; p < C::PASSES; ++p) {
                        float vx[8];
                        widen8(vraw[p], vx);   // zeroed past the end in phase 1
                        const int t = prow + RPP * p;
                        const float rsc = vsc * sm.dec[bp_][t] * (VSC ? vrs[p] : 1.f);
                        h8 vv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) vv[e] = (_Float16)(vx[e] * rsc);
                        *reinterpret_cast<h8 *>(&sm.Vs[t][pcol]) = vv;
                    }
                    fetch_v(min(cp + 1, nch - 1));
                }
                {
                    // diagonal block pw: Gram tile, A' = b_r k_r.k_s (s < r) written
                    // transposed into the block's upper triangle (column q of A' is then
                    // one contiguous row), then the inverse of I + A' by forward
                    // substitution, lane column c = r16 (the four lane groups repeat it)
                    const int o = 16 * pw;
                    f4 acc = zero4();
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const h8 A = *reinterpret_cast<const h8 *>(&sm.Ks[bp_][o + r16][32 * kb + 8 * g]);
                        acc = mma(A, A, acc);
                    }
                    const float4 bq = *reinterpret_cast<const float4 *>(&sm.beta[bp_][o + 4 * g]);
                    const float bqv[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 4 * g + i;   // A'[rr][r16] for r16 < rr, stored at [r16][rr]
                        const float av = bqv[i] * acc[i];
                        if (r16 < rr) sm.Gm[o + r16][o + rr] = av;
                        if (rr >= 8 && r16 < 8) sm.A21s[pw][rr - 8][r16] = av;   // A21 row-major
                    }
                    // (I + A')^-1 = [[M11, 0], [M21, M22]]: M11, M22 by forward substitution
                    // on the 8x8 diagonal halves, side by side (lane column c = r16: c < 8 a
                    // column of M11, c >= 8 one of M22; the four lane groups repeat it),
                    // then M21 = -M22 A21 M11 with one entry per lane.  LDS operations of a
                    // wave complete in order.
                    const int c = r16, bb = c & 8, cl = c & 7;
                    float x[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) x[r] = (r == cl) ? 1.f : 0.f;
                    float4 col[7][2];   // columns q of the half (rows q+1 .. 7 used)
#pragma unroll
                    for (int q = 0; q < 7; ++q) {
                        col[q][0] = *reinterpret_cast<const float4 *>(&sm.Gm[o + bb + q][o + bb]);
                        col[q][1] = *reinterpret_cast<const float4 *>(&sm.Gm[o + bb + q][o + bb + 4]);
                    }
#pragma unroll
                    for (int q = 0; q < 7; ++q) {
                        const float cv[8] = {col[q][0].x, col[q][0].y, col[q][0].z, col[q][0].w,
                                             col[q][1].x, col[q][1].y, col[q][1].z, col[q][1].w};
#pragma unroll
                        for (int r = q + 1; r < 8; ++r) x[r] -= cv[r] * x[q];
                    }
                    if (c < 8) {
                        *reinterpret_cast<float4 *>(&sm.M11t[pw][c][0]) = make_float4(x[0], x[1], x[2], x[3]);
                        *reinterpret_cast<float4 *>(&sm.M11t[pw][c][4]) = make_float4(x[4], x[5], x[6], x[7]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 8; ++r) sm.M22s[pw][r][cl] = x[r];
                    }
                    // Y = A21 M11, entry (yr, yc) per lane
                    const int yr = lane >> 3, yc = lane & 7;
                    const float4 a0 = *reinterpret_cast<const float4 *>(&sm.A21s[pw][yr][0]);
                    const float4 a1 = *reinterpret_cast<const float4 *>(&sm.A21s[pw][yr][4]);
                    const float4 m0 = *reinterpret_cast<const float4 *>(&sm.M11t[pw][yc][0]);
                    const float4 m1 = *reinterpret_cast<const float4 *>(&sm.M11t[pw][yc][4]);
                    const float yv = a0.x * m0.x + a0.y * m0.y + a0.z * m0.z + a0.w * m0.w +
                                     a1.x * m1.x + a1.y * m1.y + a1.z * m1.z + a1.w * m1.w;
                    sm.Yt[pw][yc][yr] = yv;
                    // M21 = -M22 Y
                    const float4 p0 = *reinterpret_cast<const float4 *>(&sm.M22s[pw][yr][0]);
                    const float4 p1 = *reinterpret_cast<const float4 *>(&sm.M22s[pw][yr][4]);
                    const float4 y0 = *reinterpret_cast<const float4 *>(&sm.Yt[pw][yc][0]);
                    const float4 y1 = *reinterpret_cast<const float4 *>(&sm.Yt[pw][yc][4]);
                    const float m21 = -(p0.x * y0.x + p0.y * y0.y + p0.z * y0.z + p0.w * y0.w +
                                        p1.x * y1.x + p1.y * y1.y + p1.z * y1.z + p1.w * y1.w);
                    // M' = (I + A')^-1 diag(b): column c (rows 0-7 M11 or zero, rows 8-15
                    // zero or M22), and M21 entry (8 + yr, yc)
                    const float bc = sm.beta[bp_][o + c];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        sm.Mi[pw][r][c] = c < 8 ? x[r] * bc : 0.f;
                        if (c >= 8) sm.Mi[pw][8 + r][c] = x[r] * bc;
                    }
                    sm.Mi[pw][8 + yr][yc] = m21 * sm.beta[bp_][o + yc];
                }
            }
            lds_barrier();
            // ===================== phase 3: W and U of chunk cp | update
            // (I + L) [W | U] = [diag(b) K | diag(b dec) V^], L = diag(b) strictlower(G),
            // G = K K^T, by block forward substitution over the four 16-row blocks.  With
            // M'_ii = (I + L_ii)^-1 diag(b_i) the row blocks are
            //   X_i = M'_ii (R_i - sum_{j<i} G_ij X_j),  R = [K | diag(dec) V^]
            // (diag(dec) is folded into V^ when it is staged).  Each wave owns the
            // key-column tiles {pw, pw + 4, ...} of W and the same value-column tiles
            // of U; the rows chain only through its own registers.  Products are 16 deep
            // on the matrix cores, B fragments from the accumulator tiles, k = 4g + e;
            // R_i rides the upper half of the first product (identity times the fp16 rows).
            h4 idq;   // identity fragment: I[r16][4g + e]
#pragma unroll
            for (int e = 0; e < 4; ++e) idq[e] = (_Float16)(r16 == 4 * g + e ? 1.f : 0.f);
            auto subst_row = [&](int i) {
                h4 kk[NTW], vv[NTW];   // R_i rows 16i + 4g + e, fp16 B fragments
#pragma unroll
                for (int q = 0; q < NTW; ++q) {
                    const int x0 = 16 * (pw + 4 * q);
                    kk[q] = ld_tr4(&sm.Ks[bp_][0][0], C::LDW, 16 * i + 4 * g, x0, lane);
                    vv[q] = ld_tr4(&sm.Vs[0][0], C::LDW, 16 * i + 4 * g, x0, lane);
                }
                h4 bw[NTW], bu[NTW];
                if (i == 0) {
#pragma unroll
                    for (int q = 0; q < NTW; ++q) { bw[q] = kk[q]; bu[q] = vv[q]; }
                } else {
                    f4 aw[NTW], au[NTW];
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        if (j < i) {
                            const float4 l = *reinterpret_cast<const float4 *>(&sm.Gm[16 * i + r16][16 * j + 4 * g]);
                            const h4 nl = {(_Float16)-l.x, (_Float16)-l.y, (_Float16)-l.z, (_Float16)-l.w};
                            const h8 A = cat8(nl, j == 0 ? idq : h4z);
#pragma unroll
                            for (int q = 0; q < NTW; ++q) {
                                if (j == 0) {
                                    aw[q] = mma(A, cat8(Xw[q][0], kk[q]), zero4());
                                    au[q] = mma(A, cat8(Xu[q][0], vv[q]), zero4());
                                } else {
                                    aw[q] = mma(A, cat8(Xw[q][j], h4z), aw[q]);
                                    au[q] = mma(A, cat8(Xu[q][j], h4z), au[q]);
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int q = 0; q < NTW; ++q) {
                        bw[q] = h4{(_Float16)aw[q][0], (_Float16)aw[q][1], (_Float16)aw[q][2], (_Float16)aw[q][3]};
                        bu[q] = h4{(_Float16)au[q][0], (_Float16)au[q][1], (_Float16)au[q][2], (_Float16)au[q][3]};
                    }
                }
                const float4 mi = *reinterpret_cast<const float4 *>(&sm.Mi[i][r16][4 * g]);
                const h8 A = {(_Float16)mi.x, (_Float16)mi.y, (_Float16)mi.z, (_Float16)mi.w,
                              (_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
#pragma unroll
                for (int q = 0; q < NTW; ++q) {
                    const f4 xw = mma(A, cat8(bw[q], h4z), zero4());
                    const f4 xu = mma(A, cat8(bu[q], h4z), zero4());
                    Xw[q][i] = h4{(_Float16)xw[0], (_Float16)xw[1], (_Float16)xw[2], (_Float16)xw[3]};
                    Xu[q][i] = h4{(_Float16)xu[0], (_Float16)xu[1], (_Float16)xu[2], (_Float16)xu[3]};
                    const int col = 16 * (pw + 4 * q) + r16;
                    // -W[16i + 4g + e][col] at nWT[col][16i + 4g + e]; U likewise at UT
                    *reinterpret_cast<h4 *>(&sm.nWT[col][16 * i + 4 * g]) = -Xw[q][i];
                    *reinterpret_cast<float4 *>(&sm.UT[col][16 * i + 4 * g]) = make_float4(xu[0], xu[1], xu[2], xu[3]);
                }
            };
            if (dop) { subst_row(0); subst_row(1); subst_row(2); subst_row(3); }
            // gates of the next chunk (its gate loads went out in phase 1); the last
            // iteration recomputes its own rows into the idle slot
            gates(cp + 1, cp + 1 < nch);
            lds_barrier();
        }
#pragma unroll
        for (int ph = 0; ph < 3; ++ph) lds_barrier();

        if (pw == 0) {
            const double tot = wave_sum_f64(cl_lane);
            if (lane == 0) sm.cl_tot = tot;
        }
        lds_barrier();
    } else {
        // ----------------------------------------------------------- state state
        // column tiles of X = [Tbar | S] held by this wave: Tbar tiles 2w, 2w + 1 and S
        // tiles MT + 2w, MT + 2w + 1 (every state wave carries the same share of the
        // S-only work: chunk-gate prescale and value terms)
        auto tile_n = [&](int jn) { return jn < 2 ? 2 * w + jn : MT + 2 * w + jn - 2; };
        f4 X[MT][C::TPW];
        float sig[C::TPW] = {0.f, 0.f, 0.f, 0.f};
        h8 Eb[C::TPW][2];  // E of the four column tiles as fp16 B operands (token blocks 0-31, 32-63)
        {
#pragma unroll
            for (int jn = 0; jn < C::TPW; ++jn) {
                const int n = tile_n(jn);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        X[mt][jn][i] = (jn < 2 && 16 * mt + 4 * g + i == 16 * n + r16) ? 1.f : 0.f;
            }
        }


        for (int it = 0; it <= nch; ++it) {
            const int cs = it - 1;
            const bool dos = cs >= 0;
            const int bs_ = cs & 1;
            // Xhat <- Xhat * 2^(sig - target): new unit from the block max, never below
            // 2^(sv - 4) for S (keeps E = U 2^(sv - sig) - W Xhat within fp16 range)
            auto renorm = [&](int jn, bool isS, float svs) {
                float xm = 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xm = fmaxf(xm, fabsf(X[mt][jn][i]));
                xm = wave_max(xm);
                float target = (float)pow2_exponent(xm) + sig[jn];
                if (xm == 0.f) target = isS ? svs : sig[jn];
                if (isS && target < svs - 4.f) target = svs - 4.f;
                const float f = exp2f(sig[jn] - target);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) X[mt][jn] *= f;
                sig[jn] = target;
            };
            // chunk gate on the S tiles, value-scale catch-up (before their E in phase 2)
            auto state_prescale = [&]() {
#pragma unroll
                for (int jn = 2; jn < C::TPW; ++jn) {
                    const float gbv = sm.gb[bs_];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) X[mt][jn] *= gbv;
                    if (cs == 0) sig[jn] = (float)sm.sv[bs_];   // S starts at 0: take the value scale
                    if ((float)sm.sv[bs_] > sig[jn] + 4.f) renorm(jn, true, (float)sm.sv[bs_]);
                }
            };
            // E = U 2^(sv - sig) - W Xhat for the column tiles {2 pp, 2 pp + 1}, all 64
            // tokens: each tile's Xhat is converted to fp16 fragments once per chunk
            auto state_e_pair = [&](int pp) {
                f4 E[2][4];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int jn = 2 * pp + q, n = tile_n(jn);
#pragma unroll
                    for (int tj = 0; tj < 4; ++tj) E[q][tj] = zero4();
                    if (jn >= 2) {
                        const float usc = exp2f((float)sm.sv[bs_] - sig[jn]);
                        const int cc = 16 * (n - MT) + r16;
#pragma unroll
                        for (int tj = 0; tj < 4; ++tj) {
                            const float4 u = *reinterpret_cast<const float4 *>(&sm.UT[cc][16 * tj + 4 * g]);
                            E[q][tj] = f4{u.x, u.y, u.z, u.w} * usc;
                        }
                    }
                }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    h8 B[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            B[q][i] = (_Float16)X[2 * kb][2 * pp + q][i];
                            B[q][4 + i] = (_Float16)X[2 * kb + 1][2 * pp + q][i];
                        }
#pragma unroll
                    for (int tj = 0; tj < 4; ++tj) {
                        // -W[16 tj + m][k], k = 32 kb + 4g + (e & 3) + 16 (e >> 2)
                        const h8 A = cat8(ld_tr4(&sm.nWT[0][0], C::LDT, 32 * kb + 4 * g, 16 * tj, lane),
                                          ld_tr4(&sm.nWT[0][0], C::LDT, 32 * kb + 16 + 4 * g, 16 * tj, lane));
#pragma unroll
                        for (int q = 0; q < 2; ++q) E[q][tj] = mma(A, B[q], E[q][tj]);
                    }
                }
                // token blocks of 32 as fp16 B operands of the update
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            Eb[2 * pp + q][hb][i] = (_Float16)E[q][2 * hb][i];
                            Eb[2 * pp + q][hb][4 + i] = (_Float16)E[q][2 * hb + 1][i];
                        }
            };
            // Xhat += K^T E for all four tiles, row tiles [m0, m1): every K^T fragment
            // read from LDS feeds the four tiles' products
            auto state_u4 = [&](int m0, int m1) {
#pragma unroll
                for (int mt = m0; mt < m1; ++mt) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        // K^T[16 mt + m][t], t = 32 kb + 4g + (e & 3) + 16 (e >> 2)
                        const h8 A = cat8(ld_tr4(&sm.Ks[bs_][0][0], C::LDW, 32 * kb + 4 * g, 16 * mt, lane),
                                          ld_tr4(&sm.Ks[bs_][0][0], C::LDW, 32 * kb + 16 + 4 * g, 16 * mt, lane));
#pragma unroll
                        for (int jn = 0; jn < C::TPW; ++jn) X[mt][jn] = mma(A, Eb[jn][kb], X[mt][jn]);
                    }
                }
            };
            auto state_u = [&](int jn) {   // periodic renormalisation
                if ((cs & 3) == 3) renorm(jn, jn >= 2, (float)sm.sv[bs_]);
            };
            // the off-diagonal Gram tiles G_ij = K_i K_j^T of the prep waves' chunk it
            // (staged in its phase 1, used by its phase 3): tile q -> (ti, tj), q = 0..5 ->
            // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2); state wave w takes q = w, w + NS, ...
            auto offdiag = [&](int q) {
                const int bp = it & 1;
                const int ti = q < 1 ? 1 : (q < 3 ? 2 : 3), tj = q - ti * (ti - 1) / 2;
                f4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const h8 A = *reinterpret_cast<const h8 *>(&sm.Ks[bp][16 * ti + r16][32 * kb + 8 * g]);
                    const h8 B = *reinterpret_cast<const h8 *>(&sm.Ks[bp][16 * tj + r16][32 * kb + 8 * g]);
                    acc = mma(A, B, acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.Gm[16 * ti + 4 * g + i][16 * tj + r16] = acc[i];
            };
            if (dos) state_e_pair(0);
            lds_barrier();
            if (it < nch) {
                for (int q = w; q < 6; q += NS) offdiag(q);
            }
            if (dos) {
                state_prescale();
                state_e_pair(1);
            }
            lds_barrier();
            if (dos) {
                state_u4(0, MT);
#pragma unroll
                for (int jn = 0; jn < C::TPW; ++jn) state_u(jn);
            }
            lds_barrier();
        }

        lds_barrier();
        {
            const double cl_tot = sm.cl_tot;
            float *Tu = a.T_out + (int64_t)unit * D * D;
            float *Su = a.S0_out + (int64_t)unit * D * D;
#pragma unroll
            for (int jn = 0; jn < C::TPW; ++jn) {
                const int n = tile_n(jn);
                const bool isS = jn >= 2;
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
    }
}

template <int D, typename TK, typename TV, typename TG>
hipError_t launch_f16_one(const DeltaArgs &a, int n_units, hipStream_t st)
{
    const size_t smem = sizeof(F16Smem<D>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&build_delta_f16_kernel<D, TK, TV, TG>, smem, lds_set); e != hipSuccess)
        return e;
    hipLaunchKernelGGL((build_delta_f16_kernel<D, TK, TV, TG>), dim3(n_units), dim3(F16Cfg<D>::NT), smem, st, a);
    return hipGetLastError();
}

// bf16 inputs (keys, values and gates), or the conv workspace of a bf16-input
// build (fp16 keys, fp16 values with a power of two per row) with bf16 gates
hipError_t launch_build_delta_f16(const DeltaArgs &a, int D, int kv_kind, int g_kind, int n_units,
                                  hipStream_t st)
{
    if (g_kind != IN_BF16) return hipErrorInvalidValue;
    if (D == 128) {
        if (kv_kind == IN_BF16) return launch_f16_one<128, bf16_t, bf16_t, bf16_t>(a, n_units, st);
        if (kv_kind == IN_F16K) return launch_f16_one<128, _Float16, _Float16, bf16_t>(a, n_units, st);
    } else if (D == 64) {
        if (kv_kind == IN_BF16) return launch_f16_one<64, bf16_t, bf16_t, bf16_t>(a, n_units, st);
        if (kv_kind == IN_F16K) return launch_f16_one<64, _Float16, _Float16, bf16_t>(a, n_units, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hy

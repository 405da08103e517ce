// compose_group.hip -- the dense composition of a prompt's segments as a
// two-level associative scan (HYPIC reading notes ch.2 sec.2, Eq. (6): pairs
// compose by (T2, S2) o (T1, S1) = (T2 T1, T2 S1 + S2); the seam window of an
// inner segment, ch.2 secs.5-6, is one more affine map of the state).
//
// Level 1 (this kernel): the positions of a launch are cut into groups of G
// consecutive ones, and every (group, value head) folds its maps into one pair
//   X = [T_g | S_g] <- A X + [0 | b]      from X = [I | 0],
// in prompt order: for a position p >= 1 first its window
//   X <- gw X + K^T (U~ - gw W X)         (U~ = U on the S half, 0 on the T half)
// then its pair X <- T_p X + [0 | S0_p].  All groups and heads run in
// parallel; level 2 is the ordinary serial fold over the group pairs (the
// no-seam compose kernel), G times shorter than the fold over the segments.
//
// One workgroup of d/16 waves (two per SIMD at d = 128, so one wave's VALU and
// LDS work overlaps the other's matrix products) per (group, value head).  A
// wave owns 32 columns of X (all d rows, fp32 in matrix-core accumulator
// layout): the first half of the waves the T half, the others the S half.  The products run on bf16 hi/lo splits (three matrix-core products
// per term), A operands from LDS, B operands from the wave's own accumulators,
// so X never leaves the registers until the group ends.  T of the next position
// is streamed through the T half's registers and split into the other LDS
// buffer while the current product runs (one barrier per position); the S
// half streams S0 the same way into its registers.  The window operators
// (W = M diag(b) K, K, U^T, gw; w <= 8) come from the per-(window, head)
// records that seam_ops_kernel writes.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "seam.h"

namespace hy {

// NN 16-column tiles of X per wave; the library instantiates NN = 2 (d/16
// waves, two per SIMD at d = 128)
template <int D, int NN_>
struct CgCfg {
    static constexpr int NN = NN_;
    static constexpr int NP = NN / 2;             // column pairs per wave
    static constexpr int NW = 2 * D / (16 * NN);  // waves
    static constexpr int NWH = NW / 2;            // waves per half
    static constexpr int NT = 64 * NW;
    static constexpr int MT = D / 16;             // 16-row tiles of X
    static constexpr int KB = D / 32;             // 32-deep k blocks of a product
    static constexpr int LDA = D + 8;             // split row stride (bf16 elements)
    static constexpr int WR = 8;                  // window rows held (w <= 8)
    static constexpr int TP = 2 * NP;             // parts of T's rows in the T half's ring
    static constexpr int QH = D * D / 4 / (64 * NWH * TP);   // float4 per lane per part
    static constexpr bool WK_SPLIT = NT >= 4 * D; // W and K staged by separate threads
};

template <int D, int NN, bool RO>
struct CgSmem {
    using C = CgCfg<D, NN>;
    // double-buffered by position parity
    uint16_t AH[2][D][C::LDA];       // T of the position, hi, k-permuted within 32-column blocks
    uint16_t AL[2][D][C::LDA];       // lo
    uint16_t WH[2][C::WR][C::LDA];   // window W, hi, k-permuted; rows >= w zero
    uint16_t WL[2][C::WR][C::LDA];
    uint16_t KH[2][C::WR][C::LDA];   // window K, hi, natural [t][d]; rows >= w zero
    uint16_t KL[2][C::WR][C::LDA];
    // window read-out rows A (with read-outs only), hi/lo, k-permuted; one buffer,
    // restaged after a barrier in the middle of each position
    uint16_t RH[RO ? C::WR : 0][C::LDA];
    uint16_t RL[RO ? C::WR : 0][C::LDA];
};

typedef __bf16 cg_bf2 __attribute__((ext_vector_type(2)));
typedef float cg_f2 __attribute__((ext_vector_type(2)));
typedef short cg_s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) cg_s4 cg_lds_s4;

// fp32 pair -> bf16 hi (nearest) and lo = bf16(x - hi), x - hi exact
__device__ __forceinline__ void cg_split2(float x0, float x1, uint32_t &h, uint32_t &l) {
    const cg_bf2 hv = __builtin_convertvector(cg_f2{x0, x1}, cg_bf2);
    h = __builtin_bit_cast(uint32_t, hv);
    const cg_bf2 lv = __builtin_convertvector(cg_f2{x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)}, cg_bf2);
    l = __builtin_bit_cast(uint32_t, lv);
}
__device__ __forceinline__ void cg_split4(const float4 &x, uint2 &h, uint2 &l) {
    cg_split2(x.x, x.y, h.x, l.x);
    cg_split2(x.z, x.w, h.y, l.y);
}
// B operand (32-deep, k = 4g + (e & 3) + 16 (e >> 2)) of one column tile from
// the accumulator tiles of rows 32 kb .. 32 kb + 15 (lo4) and + 16 .. + 31 (hi4)
__device__ __forceinline__ void cg_split_acc(const f4 &lo4, const f4 &hi4, b8 &bh, b8 &bl) {
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    cg_split2(lo4[0], lo4[1], h0, l0);
    cg_split2(lo4[2], lo4[3], h1, l1);
    cg_split2(hi4[0], hi4[1], h2, l2);
    cg_split2(hi4[2], hi4[3], h3, l3);
    bh = __builtin_bit_cast(b8, make_uint4(h0, h1, h2, h3));
    bl = __builtin_bit_cast(b8, make_uint4(l0, l1, l2, l3));
}
// position of column c (a multiple of 4) of a k-permuted row: within each block
// of 32 columns, lane group g reads the 8 elements k = 4g + (e & 3) + 16 (e >> 2)
// as one 16-byte piece
__device__ __forceinline__ int cg_perm(int c) {
    const int cc = c & 31;
    return (c & ~31) + 8 * ((cc & 15) >> 2) + 4 * (cc >> 4);
}
// four 16-bit elements S[k0 + e][x0 + lane % 16], e = 0..3, through the LDS
// transpose load (lane j of a group supplies the block at S[k0 + j/4][x0 + 4 (j%4)])
__device__ __forceinline__ uint2 cg_ld_tr4(const uint16_t *S, int ld, int k0, int x0, int lane) {
    const int j = lane & 15;
    const uint16_t *p = S + (k0 + (j >> 2)) * ld + x0 + 4 * (j & 3);
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((cg_lds_s4 *)p));
}
__device__ __forceinline__ f4 cg_mma3(const b8 &ah, const b8 &al, const b8 &bh, const b8 &bl, f4 c) {
    c = mma(al, bh, c);
    c = mma(ah, bl, c);
    return mma(ah, bh, c);
}

template <int D, bool SEAMS, int NN, bool RO>
__global__ void __launch_bounds__((CgCfg<D, NN>::NT)) compose_group_kernel(const ComposeArgs a, const float *ops,
                                                                           int G, float *gT, float *gS, float *Y)
{
    using C = CgCfg<D, NN>;
    constexpr int MT = C::MT, KB = C::KB, QH = C::QH, LDA = C::LDA, NWH = C::NWH, NP = C::NP, WR = C::WR,
                  TP = C::TP;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    CgSmem<D, NN, RO> &sm = *reinterpret_cast<CgSmem<D, NN, RO> *>(smem_raw);

    // the wave index as a scalar, so the branches on the wave's half are uniform
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int gi = blockIdx.x / a.h_v, h = blockIdx.x % a.h_v;
    const int j0 = gi * G, j1 = min(j0 + G, a.n);
    const int64_t hoff = (int64_t)h * D * D;
    const bool thalf = wv < NWH;
    const int cb = 16 * NN * (thalf ? wv : wv - NWH);   // first column of this wave within its half

    const int w = SEAMS ? a.seam.w : 0, wp = winop_wp(w);
    // W / K staging: one float4 of each per thread, or (WK_SPLIT) W by the first
    // 2D threads and K by the others
    const int wkt = C::WK_SPLIT ? tid % (2 * D) : tid;
    const bool do_w = !C::WK_SPLIT || tid < 2 * D, do_k = !C::WK_SPLIT || tid >= 2 * D;
    const int srow = wkt / (D / 4), scol = 4 * (wkt % (D / 4));
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    auto win_rec = [&](int pos) { return ops + ((int64_t)max(pos - 1, 0) * a.h_v + h) * winop_floats<D>(w, RO); };

    // The two halves run the same loop (one barrier per position) in separate
    // code, so that neither half's prefetch registers are live in the other's.
    auto run = [&](auto th) {
        constexpr bool TH = decltype(th)::value;
        // X = [I | 0]: lane (g, r16) of tile (mt, nt) holds row 16 mt + 4g + i,
        // column cb + 16 nt + r16 of its half
        f4 X[MT][NN];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NN; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    X[mt][nt][i] = (TH && 16 * mt + 4 * g + i == cb + 16 * nt + r16) ? 1.f : 0.f;

        // prefetch rings, refilled as they are consumed so that each load has about
        // half a column pair's work to land:
        //   T half: part hf of the next position's T rows (float4 f = tid + 64 NWH q
        //           + hf D*D/(4 TP) of the row-major matrix), fetched at the start
        //           (or the middle) of pair hf/2 and staged into the other buffer at
        //           its middle (or end);
        //   S half: the S0 tiles (mt, 2p + q) of the current pair, each slot
        //           reloaded with the next pair's tile once it is used.
        float4 tq[TH ? QH : 1];
        float4 s0q[TH ? 1 : MT][2];
        auto fetch_t = [&](int j, int hf) {
            if constexpr (TH) {
                const float *Tp = a.T_pool + (int64_t)a.order[j] * a.h_v * D * D + hoff + hf * (D * D / TP);
#pragma unroll
                for (int q = 0; q < QH; ++q) tq[q] = *reinterpret_cast<const float4 *>(Tp + 4 * (tid + 64 * NWH * q));
            }
        };
        auto stage_t = [&](int buf, int hf) {
            if constexpr (TH) {
#pragma unroll
                for (int q = 0; q < QH; ++q) {
                    const int f = tid + 64 * NWH * q + hf * (D * D / 4 / TP), row = f / (D / 4), c = 4 * (f % (D / 4));
                    uint2 hi, lo;
                    cg_split4(tq[q], hi, lo);
                    *reinterpret_cast<uint2 *>(&sm.AH[buf][row][cg_perm(c)]) = hi;
                    *reinterpret_cast<uint2 *>(&sm.AL[buf][row][cg_perm(c)]) = lo;
                }
            }
        };
        auto fetch_s0 = [&](int j, int p, int mt) {   // S0 tiles (mt, 2p), (mt, 2p + 1) of position j
            if constexpr (!TH) {
                const float *Sp = a.S0_pool + (int64_t)a.order[j] * a.h_v * D * D + hoff;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float *ps = Sp + (int64_t)(16 * mt + 4 * g) * D + cb + 16 * (2 * p + q) + r16;
                    s0q[mt][q] = make_float4(ps[0], ps[D], ps[2 * D], ps[3 * D]);
                }
            }
        };
        // window operators of position pos (pos >= 1) one position ahead of their
        // staging: this thread's float4 of W and of K (row tid / (D/4)), gw; the S
        // half's U^T slices are read at the start of the position's step
        float4 Wq = z4, Kq = z4, Rq = z4;
        float gwq = 1.f, gwc = 1.f;
        bool hwq = false, hwc = false;
        auto fetch_win = [&](int pos) {
            if constexpr (SEAMS) {
                hwq = pos >= 1;
                const float *o = win_rec(pos);
                const bool rin = hwq && srow < w;
                // this thread's offset inside a record, formed here (opaque) rather than held
                // across the position loop
                int ro = (rin ? srow : 0) * D + scol;
                asm volatile("" : "+v"(ro));
                if (do_w) Wq = *reinterpret_cast<const float4 *>(o + ro);
                if (do_k) Kq = *reinterpret_cast<const float4 *>(o + (int64_t)wp * D + ro);
                if constexpr (RO)
                    if (do_w) Rq = *reinterpret_cast<const float4 *>(o + (int64_t)3 * wp * D + ro);
                if (!rin) { Wq = z4; Kq = z4; Rq = z4; }
                gwq = hwq ? o[winop_gw<D>(w, RO)] : 1.f;
            }
        };
        auto stage_win = [&](int buf) {   // W, K of the fetched window into buffer buf; gw current
            if constexpr (SEAMS) {
                uint2 hi, lo;
                if (do_w) {
                    cg_split4(Wq, hi, lo);
                    *reinterpret_cast<uint2 *>(&sm.WH[buf][srow][cg_perm(scol)]) = hi;
                    *reinterpret_cast<uint2 *>(&sm.WL[buf][srow][cg_perm(scol)]) = lo;
                }
                if (do_k) {
                    cg_split4(Kq, hi, lo);
                    *reinterpret_cast<uint2 *>(&sm.KH[buf][srow][scol]) = hi;
                    *reinterpret_cast<uint2 *>(&sm.KL[buf][srow][scol]) = lo;
                }
                gwc = gwq;
                hwc = hwq;
            }
        };
        auto stage_r = [&]() {   // read-out rows of the fetched window (single buffer)
            if constexpr (RO) {
                if (do_w) {
                    uint2 hi, lo;
                    cg_split4(Rq, hi, lo);
                    *reinterpret_cast<uint2 *>(&sm.RH[srow][cg_perm(scol)]) = hi;
                    *reinterpret_cast<uint2 *>(&sm.RL[srow][cg_perm(scol)]) = lo;
                }
            }
        };
        // B operands of the column tiles 2 p, 2 p + 1 for the k block kb (rows
        // 32 kb .. 32 kb + 31 of X), from the accumulators
        auto split_kb = [&](int p, int kb, b8 (&bh)[2], b8 (&bl)[2]) {
#pragma unroll
            for (int q = 0; q < 2; ++q) cg_split_acc(X[2 * kb][2 * p + q], X[2 * kb + 1][2 * p + q], bh[q], bl[q]);
        };

        // prologue: position j0 staged in buffer 0 (T half), the S0 tiles of its
        // first pair in flight (S half), the window of j0 + 1 in flight
        if constexpr (TH) {
#pragma unroll
            for (int hf = 0; hf < TP; ++hf) { fetch_t(j0, hf); stage_t(0, hf); }
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) fetch_s0(j0, 0, mt);
        }
        fetch_win(a.first_pos + j0);
        stage_win(0);
        stage_r();
        fetch_win(a.first_pos + min(j0 + 1, j1 - 1));

#pragma unroll 1
        for (int j = j0; j < j1; ++j) {
            const int buf = (j - j0) & 1;
            lds_barrier();   // position j staged in buf; the reads of buf ^ 1 (position j - 1) done
            // U^T[column][t = 4g .. 4g + 3] of the S half's lanes (zero elsewhere)
            float4 Uc[NN];
#pragma unroll
            for (int nt = 0; nt < NN; ++nt) Uc[nt] = z4;
            if constexpr (SEAMS && !TH) {
                const bool uin = hwc && 4 * g < wp;
                const float *o = win_rec(a.first_pos + j) + (int64_t)2 * wp * D;
#pragma unroll
                for (int nt = 0; nt < NN; ++nt) {
                    const float4 u = *reinterpret_cast<const float4 *>(o + (int64_t)(cb + 16 * nt + r16) * wp +
                                                                       (uin ? 4 * g : 0));
                    Uc[nt] = uin ? u : z4;
                }
            }
            const int jn = min(j + 1, j1 - 1);
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                // scheduling regions per pair and per part: with one wave per SIMD the
                // scheduler would otherwise overlap the parts beyond the register file
                __builtin_amdgcn_sched_barrier(0);
                fetch_t(jn, 2 * p);
                if constexpr (SEAMS) {
                    // P = W X (window rows t = r16 < 8), E = U~ - gw P, X <- gw X + K^T E;
                    // branch-free: position 0 runs it with W = K = U = 0, gw = 1, which
                    // leaves X exactly as it is
                    const bool wl = r16 < WR;
                    f4 P[2] = {zero4(), zero4()};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        b8 bh[2], bl[2];
                        split_kb(p, kb, bh, bl);
                        b8 ah = *reinterpret_cast<const b8 *>(&sm.WH[buf][wl ? r16 : 0][32 * kb + 8 * g]);
                        b8 al = *reinterpret_cast<const b8 *>(&sm.WL[buf][wl ? r16 : 0][32 * kb + 8 * g]);
                        if constexpr (RO) {
                            // rows 8 .. 15 of the product: the read-out rows, Y = A X
                            if (!wl) {
                                ah = *reinterpret_cast<const b8 *>(&sm.RH[r16 - WR][32 * kb + 8 * g]);
                                al = *reinterpret_cast<const b8 *>(&sm.RL[r16 - WR][32 * kb + 8 * g]);
                            }
                        } else if (!wl) {
                            ah = b8{};
                            al = b8{};
                        }
#pragma unroll
                        for (int q = 0; q < 2; ++q) P[q] = cg_mma3(ah, al, bh[q], bl[q], P[q]);
                    }
                    if constexpr (RO) {
                        // rows 4g + i >= 8 of P are Y rows t = 4g + i - 8 (their E rows meet
                        // zero key columns below)
                        if (hwc && g >= 2) {
                            // the lane's offset is formed here (opaque), so the compiler does not
                            // hold a 64-bit lane address across the position loop
                            int yo = (4 * g - WR) * 2 * D + (TH ? 0 : D) + cb + r16;
                            asm volatile("" : "+v"(yo));
                            float *yp = Y + ((int64_t)(a.first_pos + j - 1) * a.h_v + h) * 8 * 2 * D + yo;
#pragma unroll
                            for (int q = 0; q < 2; ++q)
#pragma unroll
                                for (int i = 0; i < 4; ++i) yp[(int64_t)i * 2 * D + 16 * (2 * p + q)] = P[q][i];
                        }
                    }
                    b8 Eh[2], El[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float4 u = Uc[2 * p + q];
                        const float4 e = make_float4(u.x - gwc * P[q][0], u.y - gwc * P[q][1],
                                                     u.z - gwc * P[q][2], u.w - gwc * P[q][3]);
                        uint2 hi, lo;
                        cg_split4(e, hi, lo);   // E[t = 4g + e][column], k = 4g + e, upper half zero
                        Eh[q] = __builtin_bit_cast(b8, make_uint4(hi.x, hi.y, 0u, 0u));
                        El[q] = __builtin_bit_cast(b8, make_uint4(lo.x, lo.y, 0u, 0u));
                    }
                    const bool kl8 = g < WR / 4;   // token rows 4g .. 4g + 3 held
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        // K^T[16 mt + r16][t = 4g + e]
                        uint2 kh = cg_ld_tr4(&sm.KH[buf][0][0], LDA, 4 * (g & 1), 16 * mt, lane);
                        uint2 kl = cg_ld_tr4(&sm.KL[buf][0][0], LDA, 4 * (g & 1), 16 * mt, lane);
                        if (!kl8) { kh = make_uint2(0u, 0u); kl = kh; }
                        const b8 ah = __builtin_bit_cast(b8, make_uint4(kh.x, kh.y, 0u, 0u));
                        const b8 al = __builtin_bit_cast(b8, make_uint4(kl.x, kl.y, 0u, 0u));
#pragma unroll
                        for (int q = 0; q < 2; ++q)
                            X[mt][2 * p + q] = cg_mma3(ah, al, Eh[q], El[q], gwc * X[mt][2 * p + q]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // X <- T X (+ S0 on the S half) for the two column tiles: the new
                // values accumulate from S0 (or 0) over the k blocks, each k block's B
                // operands split from the old values just before use
                f4 acc[MT][2];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        if constexpr (TH) acc[mt][q] = zero4();
                        else acc[mt][q] = f4{s0q[mt][q].x, s0q[mt][q].y, s0q[mt][q].z, s0q[mt][q].w};
                    }
                // the S0 slots' next tiles: the other pair of this position, or the
                // first pair of the next one (clamped to the group)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (p + 1 < NP) fetch_s0(j, p + 1, mt);
                    else fetch_s0(jn, 0, mt);
                }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    if (kb == KB / 2) {
                        // the pair's first part of the next position's T into the other
                        // buffer (read only after the next barrier), the second in flight
                        __builtin_amdgcn_sched_barrier(0);
                        stage_t(buf ^ 1, 2 * p);
                        fetch_t(jn, 2 * p + 1);
                        if constexpr (RO) {
                            // every wave is past this position's window product: the
                            // read-out rows of the next position go into the one buffer
                            if (p == NP - 1) {
                                lds_barrier();
                                stage_r();
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    b8 bh[2], bl[2];
                    split_kb(p, kb, bh, bl);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const b8 ah = *reinterpret_cast<const b8 *>(&sm.AH[buf][16 * mt + r16][32 * kb + 8 * g]);
                        const b8 al = *reinterpret_cast<const b8 *>(&sm.AL[buf][16 * mt + r16][32 * kb + 8 * g]);
#pragma unroll
                        for (int q = 0; q < 2; ++q) acc[mt][q] = cg_mma3(ah, al, bh[q], bl[q], acc[mt][q]);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int q = 0; q < 2; ++q) X[mt][2 * p + q] = acc[mt][q];
                stage_t(buf ^ 1, 2 * p + 1);
            }
            stage_win(buf ^ 1);
            fetch_win(a.first_pos + min(j + 2, j1 - 1));
        }

        // the group pair, row-major [D][D] per (group, head)
        float *out = (TH ? gT : gS) + ((int64_t)gi * a.h_v + h) * D * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NN; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[(int64_t)(16 * mt + 4 * g + i) * D + cb + 16 * nt + r16] = X[mt][nt][i];
    };
    if (thalf) run(std::true_type{});
    else run(std::false_type{});
}

template <int D, bool SEAMS, int NN, bool RO>
static hipError_t launch_cg(const ComposeArgs &a, const float *ops, int G, int ng, float *gT, float *gS, float *Y,
                            hipStream_t st)
{
    const size_t smem = sizeof(CgSmem<D, NN, RO>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&compose_group_kernel<D, SEAMS, NN, RO>, smem, lds_set); e != hipSuccess)
        return e;
    hipLaunchKernelGGL((compose_group_kernel<D, SEAMS, NN, RO>), dim3(ng * a.h_v), dim3(CgCfg<D, NN>::NT), smem, st,
                       a, ops, G, gT, gS, Y);
    return hipGetLastError();
}

constexpr int kCgNN = 2;   // 16-column tiles of X per wave

hipError_t launch_compose_group(const ComposeArgs &a, int D, const float *ops, int G, int ng, float *gT,
                                float *gS, float *Y, hipStream_t st)
{
    if (G < 1 || ng < 1 || (int64_t)(ng - 1) * G >= a.n || (int64_t)ng * G < a.n) return hipErrorInvalidValue;
    if (a.has_seams && a.seam.w > CgCfg<128, kCgNN>::WR) return hipErrorInvalidValue;
    // the seam variant needs at least one window record in this launch
    const bool seams = a.has_seams && a.first_pos + a.n >= 2;
    // read-out records are laid out with the read-out rows: the kernel must match
    const bool ro = seams && a.seam.q != nullptr;
    if (ro && !Y) return hipErrorInvalidValue;
    if (D == 128) return ro ? launch_cg<128, true, kCgNN, true>(a, ops, G, ng, gT, gS, Y, st)
                    : seams ? launch_cg<128, true, kCgNN, false>(a, ops, G, ng, gT, gS, Y, st)
                            : launch_cg<128, false, kCgNN, false>(a, ops, G, ng, gT, gS, Y, st);
    if (D == 64) return ro ? launch_cg<64, true, kCgNN, true>(a, ops, G, ng, gT, gS, Y, st)
                   : seams ? launch_cg<64, true, kCgNN, false>(a, ops, G, ng, gT, gS, Y, st)
                           : launch_cg<64, false, kCgNN, false>(a, ops, G, ng, gT, gS, Y, st);
    return hipErrorInvalidValue;
}

}  // namespace hy

// compose_split.hip -- dense composition S <- T_C S + S_{C|0} over a prompt's
// segments (HYPIC reading notes ch.2 sec.2, Eq. (6)) with the seam window of
// every inner segment applied first (ch.2 secs.5-6), for d in {64, 128}:
// fp32 operands split into bf16 hi + lo, three matrix-core products per term.
//
// One workgroup (d/16 waves) per (value head, 16-column block) of the state;
// column blocks of a head share an XCD so T is fetched once into that L2.
// Each wave owns 16 rows of the state (fp32, in matrix-core accumulator
// layout).  Its rows of T and S0 stream from memory through a register ring a
// few segments deep, so several segments' operands are in flight while the
// serial chain advances.
//
// Seam of an inner segment (window operators precomputed per (window, head)
// by seam_ops_kernel: W = M diag(b) K, K, U^T, gw).  The window maps the state
// to S' = gw S + K^T E with E = U - gw W S, so the step is
//   S_new = T S' + S0 = gw (T S) + (T K^T) E + S0,
// one barrier per step: T S and W S both read the state S of this step (W S
// as per-wave parts formed from each wave's own rows at the end of the
// previous step), and T K^T needs only the segment's T and the window's keys,
// so it is formed beside T S from the same T fragments.
#include "common.h"
#include "launch.h"
#include "seam.h"

namespace hy {

template <int D, bool SEAMS>
struct CsCfg {
    static constexpr int NW = D / 16;    // waves, 16 state rows each
    static constexpr int NT = 64 * NW;
    static constexpr int KB = D / 32;    // 32-deep k blocks of the T S product
    // register ring depths: S0 rows and window records NST steps ahead (the
    // unroll factor of the step loop); raw T rows NTQ steps ahead of their
    // staging, which is itself one step ahead of their use.  The seam variant at
    // d = 128 keeps NST = 2, NTQ = 1 to stay within 256 registers (deeper T
    // rings measured no faster there)
    static constexpr int NST = (SEAMS && D == 128) ? 2 : 3;
    static constexpr int NTQ = (SEAMS && D == 128) ? 1 : NST;
    static constexpr int LDB = D + 8;    // split-state row stride (bf16)
};

template <int D, bool SEAMS>
struct CsSmem {
    using C = CsCfg<D, SEAMS>;
    // double-buffered by step parity: step j reads buffer j & 1 and writes the other
    uint16_t SH[2][16][C::LDB];                   // state hi, [column][row]
    uint16_t SL[2][16][C::LDB];                   // state lo
    f4 Ppart[SEAMS ? 2 : 1][SEAMS ? C::NW : 1][64];   // per-wave parts of W S, accumulator layout
    uint16_t KH[SEAMS ? 2 : 1][16][C::LDB];       // window keys hi, [token][dim], rows >= w zero
    uint16_t KL[SEAMS ? 2 : 1][16][C::LDB];       // window keys lo
    uint16_t TH[C::NW][16][C::LDB];               // each wave's 16 rows of T, split (wave-private)
    uint16_t TL[C::NW][16][C::LDB];
};

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 pair -> bf16 hi pair (rounded to nearest) and lo pair bf16(x - hi)
// (x - hi is exact), one conversion per pair
__device__ __forceinline__ void split2(float x0, float x1, bf2 &h, bf2 &l) {
    h = __builtin_convertvector(f2v{x0, x1}, bf2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    l = __builtin_convertvector(f2v{x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u)}, bf2);
}
// fp32 x8 -> bf16 hi/lo fragments
__device__ __forceinline__ void split8(const float (&x)[8], b8 &hi, b8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        bf2 h, l;
        split2(x[e], x[e + 1], h, l);
        hi[e] = h[0]; hi[e + 1] = h[1];
        lo[e] = l[0]; lo[e + 1] = l[1];
    }
}
// fp32 x4 into elements 0..3 of hi/lo fragments, elements 4..7 zero: the
// k-permuted operand k = 4g + e (e < 4) of a 16-deep product on 16x16x32
__device__ __forceinline__ void split4z(const float (&x)[4], b8 &hi, b8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
        bf2 h, l;
        split2(x[e], x[e + 1], h, l);
        hi[e] = h[0]; hi[e + 1] = h[1];
        lo[e] = l[0]; lo[e + 1] = l[1];
    }
#pragma unroll
    for (int e = 4; e < 8; ++e) {
        hi[e] = (__bf16)0.f;
        lo[e] = (__bf16)0.f;
    }
}
// fp32 x4 -> packed bf16 hi and lo (two 32-bit words each)
__device__ __forceinline__ void split4p(float x0, float x1, float x2, float x3, uint2 &hi, uint2 &lo) {
    bf2 h0, l0, h1, l1;
    split2(x0, x1, h0, l0);
    split2(x2, x3, h1, l1);
    hi = make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
    lo = make_uint2(__builtin_bit_cast(uint32_t, l0), __builtin_bit_cast(uint32_t, l1));
}
__device__ __forceinline__ f4 mma3(const b8 &ah, const b8 &al, const b8 &bh, const b8 &bl, f4 c) {
    c = mma(al, bh, c);
    c = mma(ah, bl, c);
    return mma(ah, bh, c);
}
__device__ __forceinline__ b8 ld_b8(const uint16_t *p) { return *reinterpret_cast<const b8 *>(p); }

template <int D, bool SEAMS>
__global__ void __launch_bounds__((CsCfg<D, SEAMS>::NT)) compose_split_kernel(const ComposeArgs a, const float *ops)
{
    using C = CsCfg<D, SEAMS>;
    constexpr int KB = C::KB, NST = C::NST, NTQ = C::NTQ;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    CsSmem<D, SEAMS> &sm = *reinterpret_cast<CsSmem<D, SEAMS> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int h = lb / (D / 16), c0 = 16 * (lb % (D / 16));
    const int64_t hoff = (int64_t)h * D * D;
    const int row0 = 16 * wv;                 // first state row of this wave
    const int n = a.n;

    // own rows of the state: lane (g, r16) holds S[row0 + 4g + i][c0 + r16]
    f4 Sown;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        Sown[i] = a.S_in ? a.S_in[hoff + (int64_t)(row0 + 4 * g + i) * D + c0 + r16] : 0.f;
    uint2 own_hi, own_lo;   // the split of the own rows last put into LDS
    auto put_state = [&](int buf, const f4 &x) {   // own rows, split, into the LDS block
        split4p(x[0], x[1], x[2], x[3], own_hi, own_lo);
        *reinterpret_cast<uint2 *>(&sm.SH[buf][r16][row0 + 4 * g]) = own_hi;
        *reinterpret_cast<uint2 *>(&sm.SL[buf][r16][row0 + 4 * g]) = own_lo;
    };

    // ---- register ring of T rows and S0 rows ---------------------------------
    // T rows load coalesced (whole rows per instruction: lane l takes row
    // RPI q + l / QPR, columns 4 (l % QPR) .. + 3 of load q), are split into bf16
    // hi/lo one step ahead of their use, off the serial chain, and parked in the
    // wave's own LDS rows TH/TL, from which the products read matrix-core
    // fragments T[row0 + r16][32 kb + 8 g .. + 7].  S0 rows: as Sown.
    constexpr int QPR = D / 4, RPI = 64 / QPR, NQ = 16 / RPI;
    float4 Tq[NTQ][NQ];
    f4 S0b[NST];
    auto fetch_t = [&](int j, float4 (&T)[NQ]) {
        const float *Tp = a.T_pool + (int64_t)a.order[j] * a.h_v * D * D + hoff +
                          (int64_t)(row0 + lane / QPR) * D + 4 * (lane % QPR);
#pragma unroll
        for (int q = 0; q < NQ; ++q) T[q] = *reinterpret_cast<const float4 *>(Tp + (int64_t)q * RPI * D);
    };
    auto stage_t = [&](const float4 (&T)[NQ]) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            uint2 hi, lo;
            split4p(T[q].x, T[q].y, T[q].z, T[q].w, hi, lo);
            const int r = RPI * q + lane / QPR, c = 4 * (lane % QPR);
            *reinterpret_cast<uint2 *>(&sm.TH[wv][r][c]) = hi;
            *reinterpret_cast<uint2 *>(&sm.TL[wv][r][c]) = lo;
        }
    };
    auto fetch_s0 = [&](int j, f4 &S0) {
        const float *Sp = a.S0_pool + (int64_t)a.order[j] * a.h_v * D * D + hoff;
#pragma unroll
        for (int i = 0; i < 4; ++i) S0[i] = Sp[(int64_t)(row0 + 4 * g + i) * D + c0 + r16];
    };
    // ring start: T of positions 0 .. NTQ-1 in slots 0 .. NTQ-1, position 0
    // staged and its slot refilled with position NTQ; S0 of positions 0 .. NST-1.
    // Afterwards the end of step j stages T of position j + 1 (slot (j + 1) % NTQ),
    // refills that slot with position j + 1 + NTQ, and refills the S0 slot of
    // step j with position j + NST.
    auto ring_start = [&]() {
#pragma unroll
        for (int s = 0; s < NTQ; ++s) fetch_t(min(s, n - 1), Tq[s]);
#pragma unroll
        for (int s = 0; s < NST; ++s) fetch_s0(min(s, n - 1), S0b[s]);
        stage_t(Tq[0]);
        fetch_t(min(NTQ, n - 1), Tq[0]);
    };
    auto ring_advance = [&](int j, int s) {   // end of step j, unroll slot s = j % NST
        const int s1 = (s + 1) % NTQ;
        stage_t(Tq[s1]);
        fetch_t(min(j + 1 + NTQ, n - 1), Tq[s1]);
    };
    // S_new = S0 + T S for this wave's rows, S split in LDS buffer `buf`
    auto product = [&](const f4 &S0, int buf) {
        f4 acc = S0, c1 = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int k0 = 32 * kb + 8 * g;
            const b8 ah = ld_b8(&sm.TH[wv][r16][k0]), al = ld_b8(&sm.TL[wv][r16][k0]);
            const b8 bh = ld_b8(&sm.SH[buf][r16][k0]), bl = ld_b8(&sm.SL[buf][r16][k0]);
            acc = mma(ah, bh, acc);
            c1 = mma(al, bh, c1);
            c1 = mma(ah, bl, c1);
        }
        return acc + c1;
    };

    if constexpr (!SEAMS) {
        // S_{j+1} = T_j S_j + S0_j; S_j split in buffer cur, one barrier per step
        ring_start();
        put_state(0, Sown);
        int cur = 0;
        auto step = [&](const int j, const int s) __attribute__((always_inline)) {
            if (a.S_steps) {   // the state entering step j, transposed ([column][row]), for the read-outs
                float *sp = a.S_steps + ((int64_t)j * a.h_v + h) * D * D + (int64_t)(c0 + r16) * D + row0 + 4 * g;
                *reinterpret_cast<float4 *>(sp) = make_float4(Sown[0], Sown[1], Sown[2], Sown[3]);
            }
            lds_barrier();   // S_j complete in buffer cur
            const f4 acc = product(S0b[s], cur);
            Sown = acc;
            put_state(cur ^ 1, acc);
            cur ^= 1;
            // off the chain, straight-line and clamped in range: next T staged,
            // ring refills
            ring_advance(j, s);
            fetch_s0(min(j + NST, n - 1), S0b[s]);
        };
        int j0 = 0;
        for (; j0 + NST <= n; j0 += NST) {
#pragma unroll
            for (int s = 0; s < NST; ++s) step(j0 + s, s);
        }
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (j0 + s < n) step(j0 + s, s);
    } else {
        // window operators of the step with prompt position pos (pos >= 1; step
        // position 0 has no window and runs with W = K = U = 0, gw = 1), this
        // lane's slices, one ring slot per step in flight:
        //   Wv: W[t = r16][row0 + 4g .. +3]   (A operand of this wave's part of W S)
        //   Uv: U^T[c0 + r16][4g .. +3]       (E layout: U[4g + i][c0 + r16])
        //   Kg: K[kt][kd .. kd + 3]           (this thread's piece of the keys, staged in LDS)
        const int w = a.seam.w, wp = winop_wp(w);
        const int win_hi = a.first_pos + n - 2;   // last window record of this launch
        constexpr int KPR = D / 4;                // key float4 pieces per token row
        const int kt = tid / KPR, kd = 4 * (tid % KPR);
        float4 Wv[NST], Uv[NST], Kg[NST];
        float gw[NST];
        bool hw[NST];
        const bool wrow = r16 < w, wtok = 4 * g < wp, ktok = kt < w;
        auto fetch_win = [&](int pos, int st) {
            const int wi = min(max(pos - 1, 0), win_hi);   // clamped: always in range
            const float *o = ops + ((int64_t)wi * a.h_v + h) * winop_floats<D>(w, a.seam.q != nullptr);
            Wv[st] = *reinterpret_cast<const float4 *>(o + (int64_t)(wrow ? r16 : 0) * D + row0 + 4 * g);
            Kg[st] = *reinterpret_cast<const float4 *>(o + (int64_t)wp * D + (int64_t)(ktok ? kt : 0) * D + kd);
            Uv[st] = *reinterpret_cast<const float4 *>(o + (int64_t)2 * wp * D + (int64_t)(c0 + r16) * wp + (wtok ? 4 * g : 0));
            gw[st] = o[winop_gw<D>(w, a.seam.q != nullptr)];
            hw[st] = pos >= 1;
        };
        // this wave's part of W S from its own rows (masked beyond the window)
        // this wave's part of W S from its own rows (masked beyond the window), with
        // the split of the own rows made when they were put into LDS
        auto part_p = [&](int st, int buf) {
            const bool m = wrow && hw[st];
            const float wx[4] = {m ? Wv[st].x : 0.f, m ? Wv[st].y : 0.f, m ? Wv[st].z : 0.f, m ? Wv[st].w : 0.f};
            b8 ah, al;
            split4z(wx, ah, al);
            const b8 bh = __builtin_bit_cast(b8, make_uint4(own_hi.x, own_hi.y, 0u, 0u));
            const b8 bl = __builtin_bit_cast(b8, make_uint4(own_lo.x, own_lo.y, 0u, 0u));
            sm.Ppart[buf][wv][lane] = mma3(ah, al, bh, bl, zero4());
        };
        // the window's keys, split, into LDS buffer buf (rows >= w zero)
        auto stage_k = [&](int st, int buf) {
            const bool m = ktok && hw[st];
            uint2 hi, lo;
            split4p(m ? Kg[st].x : 0.f, m ? Kg[st].y : 0.f, m ? Kg[st].z : 0.f, m ? Kg[st].w : 0.f, hi, lo);
            *reinterpret_cast<uint2 *>(&sm.KH[buf][kt][kd]) = hi;
            *reinterpret_cast<uint2 *>(&sm.KL[buf][kt][kd]) = lo;
        };

        // Load order: loads retire in issue order, so a wait for one load also waits
        // for every load issued before it.  The window of step m sits in slot
        // m % NST; each step issues the window NST steps ahead (into the slot it
        // has just used) before its ring refill, so the waits of step j drain only
        // what step j itself and the end of step j need.
#pragma unroll
        for (int s = 0; s < NST; ++s) fetch_win(a.first_pos + s, s);
        ring_start();
        // L2 warm-up: every workgroup of a head touches its own 1/8 of T (16 rows,
        // one float4 per thread) three positions ahead, so the HBM misses of a
        // position are spread over the head's workgroups before its rows are
        // streamed by all of them; the value is retired one step later
        float4 warm = make_float4(0.f, 0.f, 0.f, 0.f);
        const int cb = lb % (D / 16);
        auto touch_t = [&](int j) {
            warm = *reinterpret_cast<const float4 *>(a.T_pool + (int64_t)a.order[min(j, n - 1)] * a.h_v * D * D +
                                                     hoff + (int64_t)cb * 16 * D + 4 * tid);
        };
        touch_t(3);
        put_state(0, Sown);
        part_p(0, 0);
        stage_k(0, 0);
        int cur = 0;

        // step j: S, parts of W S and the keys of this step complete in buffer cur
        auto step = [&](const int j, const int s) __attribute__((always_inline)) {
            const int pos = a.first_pos + j;
            lds_barrier();
            // T S and P^T = K T^T (rows of T K^T as the lanes' columns) from the
            // same T fragments
            f4 ts = zero4(), ts1 = zero4(), pt = zero4(), pt1 = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int k0 = 32 * kb + 8 * g;
                const b8 ah = ld_b8(&sm.TH[wv][r16][k0]), al = ld_b8(&sm.TL[wv][r16][k0]);
                const b8 bh = ld_b8(&sm.SH[cur][r16][k0]), bl = ld_b8(&sm.SL[cur][r16][k0]);
                const b8 kh = ld_b8(&sm.KH[cur][r16][k0]), kl = ld_b8(&sm.KL[cur][r16][k0]);
                ts = mma(ah, bh, ts);
                ts1 = mma(al, bh, ts1);
                ts1 = mma(ah, bl, ts1);
                pt = mma(kh, ah, pt);
                pt1 = mma(kl, ah, pt1);
                pt1 = mma(kh, al, pt1);
            }
            // E = U - gw W S (token 4g + i, column r16)
            f4 ps = zero4();
#pragma unroll
            for (int q = 0; q < C::NW; ++q) ps += sm.Ppart[cur][q][lane];
            const bool mu = wtok && hw[s];
            const float gwv = hw[s] ? gw[s] : 1.f;
            const float ex[4] = {mu ? Uv[s].x - gwv * ps[0] : 0.f, mu ? Uv[s].y - gwv * ps[1] : 0.f,
                                 mu ? Uv[s].z - gwv * ps[2] : 0.f, mu ? Uv[s].w - gwv * ps[3] : 0.f};
            const f4 p = pt + pt1;
            const float px[4] = {p[0], p[1], p[2], p[3]};
            b8 ah, al, bh, bl;
            split4z(px, ah, al);   // (T K^T)[row0 + r16][t = 4g + e]
            split4z(ex, bh, bl);   // E[t = 4g + e][c0 + r16]
            const f4 acc = mma3(ah, al, bh, bl, S0b[s]) + gwv * (ts + ts1);
            Sown = acc;
            put_state(cur ^ 1, acc);
            // the next step's parts of W S and its keys
            part_p((s + 1) % NST, cur ^ 1);
            stage_k((s + 1) % NST, cur ^ 1);
            cur ^= 1;
            // off the chain, straight-line and clamped in range: next T staged and
            // its ring slot refilled; the window of step j + NST into the slot step j
            // used, and its S0
            ring_advance(j, s);
            fetch_win(pos + NST, s);
            asm volatile("" ::: "memory");
            fetch_s0(min(j + NST, n - 1), S0b[s]);
            asm volatile("" :: "v"(warm.x), "v"(warm.y), "v"(warm.z), "v"(warm.w));
            touch_t(j + 4);
        };
        int j0 = 0;
        for (; j0 + NST <= n; j0 += NST) {
#pragma unroll
            for (int s = 0; s < NST; ++s) step(j0 + s, s);
        }
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (j0 + s < n) step(j0 + s, s);
    }
    // final state from the fp32 rows
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a.S_out[hoff + (int64_t)(row0 + 4 * g + i) * D + c0 + r16] = Sown[i];
}

template <int D, typename TIN>
static hipError_t launch_ops(const ComposeArgs &a, int n_win, float *ops, hipStream_t st)
{
    if (n_win <= 0) return hipSuccess;
    const bool ro = a.seam.q != nullptr;
    if (ro && a.seam.w > 8) return hipErrorInvalidValue;   // read-out records hold windows of <= 8 rows
    if (ro)
        hipLaunchKernelGGL((seam_ops_kernel<D, 8, TIN, true>), dim3(n_win * a.h_v), dim3(64), 0, st, a.seam, ops);
    else if (a.seam.w <= 8)
        hipLaunchKernelGGL((seam_ops_kernel<D, 8, TIN, false>), dim3(n_win * a.h_v), dim3(64), 0, st, a.seam, ops);
    else
        hipLaunchKernelGGL((seam_ops_kernel<D, 16, TIN, false>), dim3(n_win * a.h_v), dim3(64), 0, st, a.seam, ops);
    return hipGetLastError();
}

// Window read-outs of a two-level compose: for the window of prompt position
// pos (launch-local j = pos - first_pos, group j / G) with state S_g entering
// its group, Y = A [P | Q] the read-out rows times the group-local prefix pair
// at the window (written by the group kernel), o = Y_P S_g + Y_Q + C.  One
// 256-thread workgroup per (group, value head, chunk of 4 windows of the
// group): the chunk's 32 rows (window, token) times S_g on the matrix cores,
// fp32 operands split into bf16 hi + lo (three products per term).  A
// fragments are 8 consecutive entries of a Y_P row, B fragments 8 consecutive
// rows of one column of S_g, which the fold stores transposed, so both load as
// whole vectors; wave w owns column tiles w, w + 4, ...
template <int D>
__global__ void __launch_bounds__(256) seam_readout_kernel(const ComposeArgs a, const float *ops, const float *Y,
                                                           int G, int j_begin)
{
    constexpr int CW = 4, RT = 2 * CW / 4, KB = D / 32, CTW = D / 16 / 4;   // row tiles, k blocks, column tiles per wave
    const int h = blockIdx.x % a.h_v, gi = blockIdx.x / a.h_v;
    const int jlo = gi * G + CW * (int)blockIdx.y, je = min(min(gi * G + G, a.n), jlo + CW);
    const int j0 = max(jlo, j_begin);
    if (j0 >= je) return;   // a chunk with no window
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g = lane >> 4;
    const int w = a.seam.w, wp = winop_wp(w);
    const int nwc = je - j0;
    // row r of the chunk = window j0 + r / 8 (clamped into the chunk), token r % 8
    auto yrow = [&](int r) {
        const int v = min(r / 8, nwc - 1);
        return Y + (((int64_t)(a.first_pos + j0 + v - 1) * a.h_v + h) * 8 + r % 8) * 2 * D;
    };
    const float *St = a.S_steps + ((int64_t)gi * a.h_v + h) * D * D;
    // the sums start from Y_Q + C of this lane's rows and columns (rows past the
    // chunk or the window read clamped ones and are never stored), fetched first
    // so that their loads overlap the products
    f4 acc[RT][CTW];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g + i, v = min(r / 8, nwc - 1), t = r % 8;
            const int win = a.first_pos + j0 + v - 1;
            const float *yq = Y + (((int64_t)win * a.h_v + h) * 8 + t) * 2 * D + D;
            const float *Cr = ops + ((int64_t)win * a.h_v + h) * winop_floats<D>(w, true) + (int64_t)4 * wp * D +
                              (int64_t)min(t, wp - 1) * D;
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
                const int col = 16 * (wv + 4 * c) + r16;
                acc[rt][c][i] = yq[col] + Cr[col];
            }
        }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int k0 = 32 * kb + 8 * g;
        b8 ah[RT], al[RT], bh[CTW], bl[CTW];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float *p = yrow(16 * rt + r16) + k0;
            const float4 u0 = *reinterpret_cast<const float4 *>(p), u1 = *reinterpret_cast<const float4 *>(p + 4);
            const float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            split8(x, ah[rt], al[rt]);
        }
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
            const float *p = St + (int64_t)(16 * (wv + 4 * c) + r16) * D + k0;
            const float4 u0 = *reinterpret_cast<const float4 *>(p), u1 = *reinterpret_cast<const float4 *>(p + 4);
            const float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            split8(x, bh[c], bl[c]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int c = 0; c < CTW; ++c) acc[rt][c] = mma3(ah[rt], al[rt], bh[c], bl[c], acc[rt][c]);
    }
    // lane (g, r16) of tile (rt, c) holds rows 16 rt + 4 g + i, column 16 (wv + 4 c) + r16
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g + i, v = r / 8, t = r % 8;
            if (v < nwc && t < w) {
                const int win = a.first_pos + j0 + v - 1;
                float *op = a.seam.o + (((int64_t)win * w + t) * a.h_v + h) * D;
#pragma unroll
                for (int c = 0; c < CTW; ++c) op[16 * (wv + 4 * c) + r16] = acc[rt][c][i];
            }
        }
}

hipError_t launch_seam_readout(const ComposeArgs &a, int D, const float *ops, const float *Y, int G,
                               hipStream_t st)
{
    // windows of this launch: positions first_pos + j >= 1
    const int j_begin = a.first_pos == 0 ? 1 : 0;
    if (a.n - j_begin <= 0) return hipSuccess;
    if (a.seam.w > 8 || G < 1 || !a.S_steps || !a.seam.o) return hipErrorInvalidValue;
    const int ng = (a.n + G - 1) / G;
    const dim3 grid((unsigned)(ng * a.h_v), (unsigned)((G + 3) / 4));
    if (D == 128) hipLaunchKernelGGL((seam_readout_kernel<128>), grid, dim3(256), 0, st, a, ops, Y, G, j_begin);
    else if (D == 64) hipLaunchKernelGGL((seam_readout_kernel<64>), grid, dim3(256), 0, st, a, ops, Y, G, j_begin);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D, bool SEAMS>
static hipError_t launch_cs(const ComposeArgs &a, const float *ops, hipStream_t st)
{
    const size_t smem = sizeof(CsSmem<D, SEAMS>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&compose_split_kernel<D, SEAMS>, smem, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL((compose_split_kernel<D, SEAMS>), dim3(a.h_v * (D / 16)), dim3(CsCfg<D, SEAMS>::NT), smem,
                       st, a, ops);
    return hipGetLastError();
}

int64_t seam_ops_floats(int D, int w, int n_win, int h_v, bool ro)
{
    const int64_t per = (D == 128) ? winop_floats<128>(w, ro) : winop_floats<64>(w, ro);
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
    // the seam variant needs at least one window record in this launch
    const bool seams = a.has_seams && a.first_pos + a.n >= 2;
    if (D == 128) return seams ? launch_cs<128, true>(a, ops, st) : launch_cs<128, false>(a, ops, st);
    if (D == 64) return seams ? launch_cs<64, true>(a, ops, st) : launch_cs<64, false>(a, ops, st);
    return hipErrorInvalidValue;
}

}  // namespace hy

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

// ---------------------------------------------------------------------------
// bf16 inputs at d in {64, 128}: the same contraction with the gate scan done
// by multiplication instead of in the log domain.  A wave reads whole rows of
// keys and gates (two key dims per lane, 64 / (d/2) rows per instruction), so
// every load is one contiguous row piece.  Thread (dp, b) owns dims 2 dp and
// 2 dp + 1 of the TPB consecutive tokens of block b of a 64-token chunk.
// Within a chunk the decay of token t is the product of the gates after it:
// the thread forms the products over its own later tokens, publishes its
// block product in LDS, and after a barrier multiplies the products of the
// later blocks.  Nothing but the chunk's gate product per dim is carried
// between chunks, so every factor stays a product of at most 64 gates.  T_C
// accumulates in the log domain per block (one log2 per block and dim), so it
// keeps its range however small it gets.  Khat = K * dec is split into bf16
// hi + lo and written dim-major; the raw value rows are staged untouched and
// read as matrix-core B fragments with the LDS transpose load.  The products
// of chunk c overlap the preparation of chunk c + 1 (double-buffered LDS, two
// barriers per chunk); two chunks of loads in flight.
template <int D>
struct DecayBCfg {
    static constexpr int NC = 64;            // value columns per workgroup
    static constexpr int NW = 8;             // waves; wave w owns columns 16 (w % 4) .. + 15
                                             // of the key-dim half w / 4 (two waves per SIMD)
    static constexpr int NT = 64 * NW;
    static constexpr int MT = D / 16;        // 16-row tiles of S
    static constexpr int MTW = MT / 2;       // row tiles per wave
    static constexpr int LPR = D / 2;        // lanes per key row (two dims each)
    static constexpr int NB = NT / LPR;      // token blocks of a chunk
    static constexpr int TPB = 64 / NB;      // tokens per block
    static constexpr int LDK = 64 + 8;       // Khat^T row stride (bf16; rows stay 16-byte aligned)
    static constexpr int LDV = NC + 8;       // value row stride
};

template <int D>
struct DecayBSmem {
    using C = DecayBCfg<D>;
    uint16_t KH[2][D][C::LDK];     // Khat^T hi, [key dim][token]
    uint16_t KL[2][D][C::LDK];     // lo
    uint16_t V[2][64][C::LDV];     // raw bf16 value rows of the column group
    float gam[2][D + 4];           // the chunk's gate product per key dim (+ a spare slot)
    float bp[C::NB][D];            // block gate products of the chunk being prepared
};

typedef short db_s4 __attribute__((ext_vector_type(4)));
typedef uint32_t db_u4 __attribute__((ext_vector_type(4)));
typedef uint32_t db_u2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) db_s4 db_lds_s4;

// fp32 pair -> bf16 hi (nearest) and lo = bf16(x - hi), x - hi exact
__device__ __forceinline__ void db_split2(float x0, float x1, uint32_t &h, uint32_t &l) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float fl2 __attribute__((ext_vector_type(2)));
    h = __builtin_bit_cast(uint32_t, __builtin_convertvector(fl2{x0, x1}, bf2));
    l = __builtin_bit_cast(uint32_t, __builtin_convertvector(
            fl2{x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)}, bf2));
}

template <int D, int GK>
__global__ void __launch_bounds__((DecayBCfg<D>::NT))
build_decay_bf16_kernel(const DecayArgs a)
{
    using C = DecayBCfg<D>;
    constexpr int MTW = C::MTW, NC = C::NC, LPR = C::LPR, NB = C::NB, TPB = C::TPB;
    constexpr bool DIAG = GK == HYPIC_GATE_DIAG;
    constexpr int NG = DIAG ? 2 : 1;          // gate values per token and thread
    extern __shared__ __align__(16) unsigned char smem_raw[];
    DecayBSmem<D> &sm = *reinterpret_cast<DecayBSmem<D> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int ct = w & 3, mt0 = (w >> 2) * MTW;   // this wave's column tile and first row tile
    const int dp = tid % LPR, blk = tid / LPR;    // scan role: dim pair, token block
    const int ngrp = D / NC;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);   // column groups of a unit share an XCD
    const int unit = lb / ngrp, grp = lb % ngrp;
    const int s = unit / a.h_v, h = unit % a.h_v;
    const int kh = h / (a.h_v / a.h_k);
    const int len = a.len[s];
    const int c0 = grp * NC;
    const unsigned ldk = (unsigned)(a.h_k * D), ldv = (unsigned)(a.h_v * D);
    const unsigned ldg = DIAG ? (unsigned)(a.h_v * D) : (unsigned)a.h_v;
    const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k) + (a.tok0[s] * a.h_k + kh) * D + 2 * dp;
    const uint16_t *vp = reinterpret_cast<const uint16_t *>(a.v) + (a.tok0[s] * a.h_v + h) * D + c0;
    const uint16_t *gp = nullptr;
    if constexpr (DIAG) gp = reinterpret_cast<const uint16_t *>(a.gate) + (a.tok0[s] * a.h_v + h) * D + 2 * dp;
    else if constexpr (GK == HYPIC_GATE_SCALAR) gp = reinterpret_cast<const uint16_t *>(a.gate) + a.tok0[s] * a.h_v + h;
    float gconst = 1.f;
    if constexpr (GK == HYPIC_GATE_HEAD_CONST) gconst = reinterpret_cast<const float *>(a.gate)[h];

    // value rows: thread (vrow, vpiece) moves 8 columns of row vrow
    const int vrow = tid >> 3, vcol = 8 * (tid & 7);

    // two chunks of raw loads in flight
    struct Buf {
        uint32_t k[TPB];                      // dims 2 dp, 2 dp + 1 of the block's tokens
        uint32_t g[DIAG ? TPB : 1];
        uint16_t gs[GK == HYPIC_GATE_SCALAR ? TPB : 1];
        db_u4 v;
    };
    Buf b0, b1;
    // rows are clamped into the segment (a chunk past its end re-reads the last
    // row, and its tokens are masked), so every fetch is unconditional; the loads
    // are issued in one fixed order on every path (scheduling fences), so the
    // compiler's load-counter waits stay exact across the loop
    // Addresses: a 64-bit base per chunk plus 32-bit row offsets inside it (a
    // clamped row lies at most a few chunks behind the base), so segments of any
    // length stay addressable.
    auto fetch = [&](int c, Buf &b) {
        const int last = len - 1 - 64 * c, t0 = TPB * blk;   // rows relative to the chunk
        const int64_t cb = (int64_t)(64 * c);
        const uint16_t *kc = kp + cb * ldk, *vc = vp + cb * ldv + vcol;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TPB; ++i) {
            b.k[i] = *reinterpret_cast<const uint32_t *>(kc + min(t0 + i, last) * (int)ldk);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DIAG) {
            const uint16_t *gc = gp + cb * ldg;
#pragma unroll
            for (int i = 0; i < TPB; ++i) {
                b.g[i] = *reinterpret_cast<const uint32_t *>(gc + min(t0 + i, last) * (int)ldg);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (GK == HYPIC_GATE_SCALAR) {
            const uint16_t *gc = gp + cb * ldg;
#pragma unroll
            for (int i = 0; i < TPB; ++i) {
                b.gs[i] = gc[min(t0 + i, last) * (int)ldg];
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        b.v = *reinterpret_cast<const db_u4 *>(vc + min(vrow, last) * (int)ldv);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto lo16 = [](uint32_t x) { return __uint_as_float(x << 16); };
    auto hi16 = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };

    f4 S[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) S[mt] = zero4();
    double cl[NG];   // log2 of this thread's share of the gate product over the segment
#pragma unroll
    for (int e = 0; e < NG; ++e) cl[e] = 0.0;
    const int nch = (len + 63) / 64;

    // suffix products of the gates within the thread's block (sl[i] = product of
    // the gates after token i of the block), carried from the first half of a
    // chunk's preparation to the second
    float sl[TPB][NG], pbk[NG];
    // first half: gates of the block (1 past the segment end), their suffix
    // products, the block product into LDS.  MASKED is false when the whole
    // chunk lies inside the segment.
    auto prep1 = [&](int c, Buf &b, auto MASKED) {
        constexpr bool MK = decltype(MASKED)::value;
        float gt[TPB][NG];
#pragma unroll
        for (int i = 0; i < TPB; ++i) {
            const bool in = !MK || 64 * c + TPB * blk + i < len;
#pragma unroll
            for (int e = 0; e < NG; ++e) {
                float x;
                if constexpr (DIAG) x = e ? hi16(b.g[i]) : lo16(b.g[i]);
                else if constexpr (GK == HYPIC_GATE_SCALAR) x = __uint_as_float((uint32_t)b.gs[i] << 16);
                else x = gconst;
                gt[i][e] = in ? x : 1.f;
            }
        }
#pragma unroll
        for (int e = 0; e < NG; ++e) {
            sl[TPB - 1][e] = 1.f;
#pragma unroll
            for (int i = TPB - 2; i >= 0; --i) sl[i][e] = sl[i + 1][e] * gt[i + 1][e];
            pbk[e] = sl[0][e] * gt[0][e];
            cl[e] += (double)log2f(pbk[e]);
        }
        if constexpr (DIAG) *reinterpret_cast<float2 *>(&sm.bp[blk][2 * dp]) = make_float2(pbk[0], pbk[1]);
        else *reinterpret_cast<float2 *>(&sm.bp[blk][2 * dp]) = make_float2(pbk[0], pbk[0]);
    };
    // second half (after a barrier): the products of the later blocks, Khat =
    // k * (decay to the chunk end), split, dim-major into LDS buffer p, the value
    // rows, and the chunk's gate product (block 0 holds it)
    auto prep2 = [&](int c, Buf &b, auto P, auto MASKED) {
        constexpr int p = decltype(P)::value;
        constexpr bool MK = decltype(MASKED)::value;
        float lat0 = 1.f, lat1 = 1.f;
#pragma unroll
        for (int bb = 1; bb < NB; ++bb) {
            if (bb > blk) {
                const float2 q = *reinterpret_cast<const float2 *>(&sm.bp[bb][2 * dp]);
                lat0 *= q.x;
                lat1 *= q.y;
            }
        }
        const float later[2] = {lat0, lat1};
        const float tot0 = lat0 * pbk[0], tot1 = lat1 * pbk[NG - 1];
        *reinterpret_cast<float2 *>(&sm.gam[p][blk == 0 ? 2 * dp : D]) = make_float2(tot0, tot1);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            constexpr int z = 0;
            const int eg = DIAG ? e : z;
            float kx[TPB];
#pragma unroll
            for (int i = 0; i < TPB; ++i) {
                const bool in = !MK || 64 * c + TPB * blk + i < len;
                kx[i] = in ? (e ? hi16(b.k[i]) : lo16(b.k[i])) * (sl[i][eg] * later[e]) : 0.f;
            }
            uint32_t hh[TPB / 2], ll[TPB / 2];
#pragma unroll
            for (int i = 0; i < TPB / 2; ++i) db_split2(kx[2 * i], kx[2 * i + 1], hh[i], ll[i]);
            if constexpr (TPB == 8) {
                *reinterpret_cast<db_u4 *>(&sm.KH[p][2 * dp + e][TPB * blk]) = db_u4{hh[0], hh[1], hh[2], hh[3]};
                *reinterpret_cast<db_u4 *>(&sm.KL[p][2 * dp + e][TPB * blk]) = db_u4{ll[0], ll[1], ll[2], ll[3]};
            } else {
                *reinterpret_cast<db_u2 *>(&sm.KH[p][2 * dp + e][TPB * blk]) = db_u2{hh[0], hh[1]};
                *reinterpret_cast<db_u2 *>(&sm.KL[p][2 * dp + e][TPB * blk]) = db_u2{ll[0], ll[1]};
            }
        }
        *reinterpret_cast<db_u4 *>(&sm.V[p][vrow][vcol]) = b.v;
    };
    // S <- diag(gam) S + Khat^T V over the k block kb, for this wave's 16
    // columns and MTW row tiles, from LDS buffer p (the gate factor with kb = 0)
    auto update = [&](auto P, int kb) {
        constexpr int p = decltype(P)::value;
        if (kb == 0) {
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                const float4 gm = *reinterpret_cast<const float4 *>(&sm.gam[p][16 * (mt0 + mt) + 4 * g]);
                S[mt][0] *= gm.x; S[mt][1] *= gm.y; S[mt][2] *= gm.z; S[mt][3] *= gm.w;
            }
        }
        // B[t][col] for t = 32 kb + 8 g + e: two transpose loads of 4 rows each
        const int j = lane & 15;
        const uint16_t *vb = &sm.V[p][32 * kb + 8 * g + (j >> 2)][16 * ct + 4 * (j & 3)];
        const uint2 v0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((db_lds_s4 *)vb));
        const uint2 v1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((db_lds_s4 *)(vb + 4 * C::LDV)));
        const b8 B = __builtin_bit_cast(b8, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            const b8 Ah = *reinterpret_cast<const b8 *>(&sm.KH[p][16 * (mt0 + mt) + r16][32 * kb + 8 * g]);
            const b8 Al = *reinterpret_cast<const b8 *>(&sm.KL[p][16 * (mt0 + mt) + r16][32 * kb + 8 * g]);
            S[mt] = mma(Ah, B, S[mt]);
            S[mt] = mma(Al, B, S[mt]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using FULL = std::false_type;
    using PART = std::true_type;
    // chunk c (LDS buffer p) is multiplied in while chunk c + 1 (raw loads in bn)
    // is prepared into the other buffer
    auto half = [&](int c, Buf &bn, auto P, auto Q) {
        lds_barrier();   // chunk c staged; the block products of chunk c may be overwritten
        if (64 * (c + 2) <= len) {
            update(P, 0);
            prep1(c + 1, bn, FULL{});
            lds_barrier();
            update(P, 1);
            prep2(c + 1, bn, Q, FULL{});
        } else {
            update(P, 0);
            prep1(c + 1, bn, PART{});
            lds_barrier();
            update(P, 1);
            prep2(c + 1, bn, Q, PART{});
        }
        fetch(c + 3, bn);
    };
    // chunks in pairs; the last pair may run one chunk past the segment end,
    // where every token is masked (gate 1, key 0) and the update leaves S as it is
    if (nch > 0) {
        fetch(0, b0);
        fetch(1, b1);
        if (64 <= len) {
            prep1(0, b0, FULL{});
            lds_barrier();
            prep2(0, b0, I0{}, FULL{});
        } else {
            prep1(0, b0, PART{});
            lds_barrier();
            prep2(0, b0, I0{}, PART{});
        }
        fetch(2, b0);
#pragma unroll 1
        for (int c = 0; c < nch; c += 2) {
            half(c, b1, I0{}, I1{});
            half(c + 1, b0, I1{}, I0{});
        }
    }

    float *Su = a.S0_out + (int64_t)unit * D * D;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Su[(16 * (mt0 + mt) + 4 * g + i) * D + c0 + 16 * ct + r16] = S[mt][i];
    // T_C: the block logs summed over the NB blocks of each dim, through LDS
    // (the value staging area is free once every wave is past its last update)
    if (grp == 0) {
        double *red = reinterpret_cast<double *>(&sm.KH[0][0][0]);   // [NB][D]
        lds_barrier();
        if constexpr (DIAG) {
            red[blk * D + 2 * dp] = cl[0];
            red[blk * D + 2 * dp + 1] = cl[1];
        } else {
            red[blk * D + 2 * dp] = cl[0];
        }
        lds_barrier();
        if (blk == 0) {
            if constexpr (DIAG) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    double t = 0.0;
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) t += red[bb * D + 2 * dp + e];
                    a.T_out[(int64_t)unit * D + 2 * dp + e] = scale_pow2(1.f, t);
                }
            } else if (dp == 0) {
                double t = 0.0;
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) t += red[bb * D];
                a.T_out[unit] = scale_pow2(1.f, t);
            }
        }
    }
}

template <int D, int GK>
static hipError_t launch_bf16(const DecayArgs &a, int n_units, hipStream_t st)
{
    const size_t smem = sizeof(DecayBSmem<D>);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&build_decay_bf16_kernel<D, GK>, smem, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL((build_decay_bf16_kernel<D, GK>), dim3(n_units * (D / DecayBCfg<D>::NC)),
                       dim3(DecayBCfg<D>::NT), smem, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bf16_d(const DecayArgs &a, int n_units, hipStream_t st)
{
    switch (a.gate_kind) {
    case HYPIC_GATE_HEAD_CONST: return launch_bf16<D, HYPIC_GATE_HEAD_CONST>(a, n_units, st);
    case HYPIC_GATE_SCALAR: return launch_bf16<D, HYPIC_GATE_SCALAR>(a, n_units, st);
    case HYPIC_GATE_DIAG: return launch_bf16<D, HYPIC_GATE_DIAG>(a, n_units, st);
    default: return hipErrorInvalidValue;
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
    if constexpr (D >= 64)
        if (in_kind == IN_BF16) return launch_bf16_d<D>(a, n_units, st);
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

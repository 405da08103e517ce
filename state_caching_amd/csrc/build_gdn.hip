// build_gdn.hip -- chunkwise gated-delta build with fp16 matrix-core operands
// for d_k = d_v = 128 (HYPIC reading notes: the cached pair of a segment,
// ch.2 secs.2 and 4; the gated-delta transition of ch.2 sec.3, Table 1).
//
// Algebra (ours; the pages give the recurrence and the two-run build).  For a
// chunk of 64 tokens with keys K, values V, write strengths b and gate
// suffix products dec_t = prod_{s>t} a_s, let G = K K^T and, per 16-row block
// i, M'_ii = (I + diag(b_i) strictlower(G_ii))^-1 diag(b_i).  Carry X = [Tbar | S]
// (Tbar the gate-free transition product, S the state).  One chunk is exactly
// (compact-WY / UT form of its 64 rank-one updates, published by Bischof & Van
// Loan; Schreiber & Van Loan; Joffrain et al.)
//   S <- gamma S                      (gamma = product of the chunk's gates)
//   P  = [0 | diag(dec) V] - K X      (64 x 256)
//   E_i = M'_ii (P_i - sum_{j<i} G_ij E_j)   for the 16-row blocks i = 0..3
//   X <- X + K^T E
// and T_C = (prod of all gates) Tbar.  The E step is block forward substitution
// on (I + diag(b) strictlower(G)) diag(b)^-1 E = P: only the four diagonal
// 16 x 16 inverses are formed, and everything the state side needs for a chunk
// (keys, values, G's lower blocks, the M'_ii) is ready a pipeline step ahead,
// so one barrier per chunk suffices.
//
// One workgroup of 8 waves per (segment, value head), two per SIMD: a state
// wave and a prep wave.  Between two barriers:
//   state waves 0-3  state(j-2): wave w owns column tiles 2w, 2w + 1 of Tbar and
//                    of S (fp32 in matrix-core accumulators): P (one half of its
//                    columns at a time; the value term scaled from the raw rows
//                    here), the block substitution for E, and X += K^T E
//   prep waves 4-7   chunk j: the raw value rows (prefetched into registers) to LDS;
//                    gates; 16 key rows per wave converted to fp16.  Chunk j-1:
//                    the transposed key copy; the Gram tiles below the diagonal
//                    (negated; waves 5-7) and, on wave 4, all four diagonal
//                    blocks' inverses (one block per lane row, the multipliers
//                    broadcast across the row by lane moves) and the M'_ii
// The two key operands reach the matrix cores through 16-byte LDS reads (twice
// the bandwidth of 8-byte and transposing reads): keys are stored with their
// order permuted inside each 32-key block so that one read yields the
// reduction order of the accumulator layout, and the transposed key copy
// permutes tokens the same way.
// X is kept in power-of-two units per column tile (renormalised every 4
// chunks, or when a chunk's values run ahead of the S unit), so every fp16
// operand stays in range.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace hy {
namespace {

constexpr int GD = 128;          // d_k = d_v
constexpr int GLK = GD + 8;      // Ks row stride (halves)
constexpr int GLT = 64 + 8;      // KT row stride (halves)
constexpr int GLP = 72;          // Mx row stride (halves)
constexpr int GLG = 20;          // Gd row stride (floats)

// Storage order inside a 32-wide block: position 8a + e holds index
// 4a + (e & 3) + 16 (e >> 2), so the 8 halves at 8a are the accumulator
// layout's reduction indices 4a + {0..3} and 16 + 4a + {0..3}.
__device__ __forceinline__ int perm32_index(int pos) { return 4 * ((pos & 31) >> 3) + (pos & 3) + 16 * ((pos >> 2) & 1) + (pos & ~31); }
// position of the four indices 4b .. 4b + 3 (b = 0..7 inside the block)
__device__ __forceinline__ int perm32_pos4(int idx) { return (idx & ~31) + 8 * ((idx & 15) >> 2) + 4 * ((idx >> 4) & 1); }

struct GdnSmem {
    _Float16 Ks[3][64][GLK];     // keys, token-major, key order permuted per 32-key block
    _Float16 KT[2][GD][GLT];     // keys transposed (key-major), token order permuted per 32 tokens
    unsigned short Vr[3][64][GD];   // raw value rows as stored (bf16 or fp16 bits); the 16-byte
                                    // piece p of row t sits at piece position p ^ (2 (t & 7))
    _Float16 Mx[2][64][GLP];     // per chunk slot: -G_ij in the blocks below the diagonal,
                                 // M'_ii on the diagonal blocks (upper blocks unused)
    float Gd[4][16][GLG];        // the four diagonal Gram blocks (inverting wave's scratch)
    float beta[3][64];           // b_t per slot
    float fac[3][64];            // value row factor dec_t (times the row scale of the conv
                                 // workspace), 0 past the segment end
    float gb[3];                 // chunk gate product per slot
    double cl_tot;               // log2 of the segment's gate product
};

typedef short s4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;

// Four consecutive reduction indices of a matrix-core operand whose lane index
// runs along shared-memory rows S[k][x] (x contiguous): lane group g receives
// S[k0 + e][x0 + lane % 16], e = 0..3, through the transposing LDS load.
__device__ __forceinline__ h4 tr4(const _Float16 *S, int ld, int k0, int x0, int lane)
{
    const int j = lane & 15;
    const _Float16 *p = S + (k0 + (j >> 2)) * ld + x0 + 4 * (j & 3);
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v *)p));
}
__device__ __forceinline__ h8 cat8(h4 lo, h4 hi) { return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; }
__device__ __forceinline__ h4 cvt4(f4 v) { return h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]}; }
// 16x16x16 product: lane holds A[l%16][4(l/16) + e], B[4(l/16) + e][l%16]
__device__ __forceinline__ f4 mma16(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); }
// LDS addressing for the per-chunk state loop: one base register per operand
// stream, made opaque each chunk so every constant offset folds into the load
// instruction (otherwise each offset is hoisted out of the loop as a register)
typedef __attribute__((address_space(3))) _Float16 lds_h;
typedef __attribute__((address_space(3))) h4 lds_h4;
typedef __attribute__((address_space(3))) h8 lds_h8;
typedef __attribute__((address_space(3))) f4 lds_f4;
__device__ __forceinline__ lds_h *lds_base(const void *p)
{
    lds_h *q = (lds_h *)p;
    asm volatile("" : "+v"(q));
    return q;
}
__device__ __forceinline__ h4 lds4h(lds_h *p) { return *(lds_h4 *)p; }
__device__ __forceinline__ h8 lds8h(lds_h *p) { return *(lds_h8 *)p; }
__device__ __forceinline__ f4 lds4f(lds_h *p) { return *(lds_f4 *)p; }
// transposing read at a precomputed lane address (see tr4)
__device__ __forceinline__ s4v lds_tr4s(lds_h *p) { return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v *)p); }
// 16-bit raw value to fp32
__device__ __forceinline__ float raw_f32(short x, bf16_t) { return __uint_as_float((uint32_t)(uint16_t)x << 16); }
__device__ __forceinline__ float raw_f32(short x, _Float16) { return (float)__builtin_bit_cast(_Float16, x); }
// maximum over the lanes of the wave, for x >= 0 (non-negative floats order
// like their bit patterns)
#define HY_DPPU(x, ctrl) __builtin_amdgcn_update_dpp(0u, (x), (ctrl), 0xf, 0xf, true)
__device__ __forceinline__ float wave_max_nn(float xf) {
    unsigned x = __float_as_uint(xf);
    x = max(x, (unsigned)HY_DPPU(x, 0xB1));
    x = max(x, (unsigned)HY_DPPU(x, 0x4E));
    x = max(x, (unsigned)HY_DPPU(x, 0x141));
    x = max(x, (unsigned)HY_DPPU(x, 0x140));
    const unsigned a = max((unsigned)__builtin_amdgcn_readlane(x, 0), (unsigned)__builtin_amdgcn_readlane(x, 16));
    const unsigned b = max((unsigned)__builtin_amdgcn_readlane(x, 32), (unsigned)__builtin_amdgcn_readlane(x, 48));
    return __uint_as_float(max(a, b));
}
// an opaque use of registers filled by an earlier load: the compiler places its
// wait for that load here
template <typename T>
__device__ __forceinline__ void claim(T &x)
{
    static_assert(sizeof(T) % 4 == 0 || sizeof(T) == 2, "register-sized values");
    if constexpr (sizeof(T) == 2) {
        uint16_t b = __builtin_bit_cast(uint16_t, x);
        uint32_t u = b;
        asm volatile("" : "+v"(u));
        x = __builtin_bit_cast(T, (uint16_t)u);
    } else {
        constexpr int n = sizeof(T) / 4;
        struct W { uint32_t w[n]; } v = __builtin_bit_cast(W, x);
#pragma unroll
        for (int i = 0; i < n; ++i) asm volatile("" : "+v"(v.w[i]));
        x = __builtin_bit_cast(T, v);
    }
}
// keeps the instruction scheduler from moving work across phases (register pressure)
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// orders this wave's LDS writes before its later LDS reads of what other lanes
// wrote (without it the compiler may move such a read above the write: for one
// lane alone the two addresses do not overlap)
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// x_r += (value of nv in lane Q of this lane's 16-lane row) * x_q: the row
// broadcast rides on the multiply-add.  The caller keeps two wait states
// between the last write of nv and the first use here (a lane move reads its
// source register that late).
template <int Q>
__device__ __forceinline__ void fmac_rowbcast(float &acc, float nv, float xq)
{
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc) : "v"(nv), "v"(xq), "n"(Q));
}
// forward substitution steps Q..14: x_r += N_r[lane Q] x_Q for r > Q
template <int Q>
__device__ __forceinline__ void subst_steps(float (&x)[16], const float (&n)[16])
{
#pragma unroll
    for (int r = Q + 1; r < 16; ++r) fmac_rowbcast<Q>(x[r], n[r], x[Q]);
    if constexpr (Q < 14) subst_steps<Q + 1>(x, n);
}

// the off-diagonal Gram tiles (row block, column block) of prep wave p = 1..3,
// two each: index 2 (p - 1) + q into (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
__device__ __forceinline__ int gram_ti(int idx) { return (0x333221u >> (4 * idx)) & 15; }
__device__ __forceinline__ int gram_tj(int idx) { return (0x210100u >> (4 * idx)) & 15; }

static_assert(sizeof(GdnSmem) <= 160 * 1024, "the build's LDS exceeds a workgroup's 160 KiB");

}  // namespace

template <typename TK, typename TV, typename TG>
__global__ void __launch_bounds__(512) build_gdn_kernel(const DeltaArgs a)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    GdnSmem &sm = *reinterpret_cast<GdnSmem *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int unit = xcd_logical_block(blockIdx.x, gridDim.x);
    const int s = unit / a.h_v, h = unit % a.h_v;
    const int kh = h / (a.h_v / a.h_k);
    const int len = a.len[s];
    const int nch = (len + 63) / 64;

    // The two roles keep their registers apart: every variable, lambda and loop
    // of a role lives inside its branch.  Both roles meet the same nch + 3 barriers.
    if (w >= 4) {
        // ------------------------------------------------------------ staging
        // prep lane (g, r16) stages key rows 16 pw + 4g + q (q = 0..3), columns 8 r16 .. 8 r16 + 7
        const int pw = w - 4;
        const int row0 = 16 * pw + 4 * g;
        // uniform row bases of the segment (64-bit) plus per-lane offsets inside a
        // chunk (32-bit: a chunk spans 64 rows)
        const TK *kb = reinterpret_cast<const TK *>(a.k) + a.tok0[s] * a.ldk + (int64_t)kh * GD;
        const unsigned char *vb = reinterpret_cast<const unsigned char *>(
            reinterpret_cast<const TV *>(a.v) + a.tok0[s] * a.ldv + (int64_t)h * GD);
        const uint32_t ldv_b = (uint32_t)(a.ldv * (int64_t)sizeof(TV));
        const TG *bp = reinterpret_cast<const TG *>(a.beta) + a.gtok0[s] * a.h_v + h;
        const TG *ap = reinterpret_cast<const TG *>(a.alpha) + a.gtok0[s] * a.h_v + h;
        constexpr bool VSC = std::is_same<TV, _Float16>::value;   // conv workspace: a power of two per row
        const float *vsp = VSC ? a.vscale + a.tok0[s] * a.h_v + h : nullptr;
        // register prefetch of the next chunk's key rows, value rows and gates,
        // double-buffered.  The value rows pass through registers rather than a direct
        // memory-to-LDS load: the compiler orders every later LDS read of the wave
        // behind such a load, which would expose the prefetch's memory latency.
        typename Raw8<TK>::type kraw[2][4];
        uint4 vraw[2][4];
        TG braw[2], araw[2];
        float vrs[2];
        auto fetch = [&](int c, auto pc) {
            constexpr int P = decltype(pc)::value;
            const int last = len - 1 - 64 * c;   // >= 0 for every chunk of the segment
            const TK *kc = kb + (int64_t)(64 * c) * a.ldk;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                ld_raw8(kc + (__umul24(min(row0 + q, last), (unsigned)a.ldk) + 8 * r16), kraw[P][q]);
            const uint32_t go = __umul24(min(lane, last), (unsigned)a.h_v);
            const int64_t gc = (int64_t)(64 * c) * a.h_v;
            braw[P] = bp[gc + go];
            araw[P] = ap[gc + go];
            if constexpr (VSC) vrs[P] = vsp[gc + go];
            else vrs[P] = 1.f;
            // raw value rows 16 pw + 4i + g, the 16-byte piece r16 ^ 2 (t & 7) of row t
            // (rows past the segment end repeat its last row; their factor is 0)
            const unsigned char *vc = vb + (int64_t)(64 * c) * ldv_b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * pw + 4 * i + g;
                const uint32_t off = (uint32_t)min(t, last) * ldv_b + 16 * (r16 ^ (2 * (t & 7)));
                vraw[P][i] = *reinterpret_cast<const uint4 *>(vc + off);
            }
        };

        double cl_lane = 0.0;
        // chunk c into slot c % 3 from prefetch buffer P: gates (every prep wave computes
        // all 64 and writes the same values) and this wave's 16 key rows.  TAIL: the
        // segment's last chunk, whose rows past the end read as zero.
        auto stage = [&](int c, auto pc, auto tail) {
            constexpr int P = decltype(pc)::value;
            const int sl = c % 3;
            const bool gin = 64 * c + lane < len;
            const float br = gin ? to_f32(braw[P]) : 0.f, ar = gin ? to_f32(araw[P]) : 1.f;
            const float l2 = log2f(ar);
            const float sfx = wave_suffix_excl(l2);   // log2 dec_t
            cl_lane += (double)l2;
            sm.beta[sl][lane] = br;
            sm.fac[sl][lane] = gin ? exp2f(sfx) * vrs[P] : 0.f;
            sm.gb[sl] = exp2f(lane_f(sfx + l2, 0));
            // value rows into slot sl: row 16 pw + 4i + g, piece position r16
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4 *>(&sm.Vr[sl][16 * pw + 4 * i + g][8 * r16]) = vraw[P][i];
            if constexpr (decltype(tail)::value) {
#pragma unroll
                for (int q = 0; q < 4; ++q) mask_raw8(kraw[P][q], 64 * c + row0 + q < len);
            }
            // keys 8 r16 .. 8 r16 + 7 = two runs of four, stored at their permuted positions
            const int kpos = perm32_pos4(8 * r16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float kx[8];
                widen8(kraw[P][q], kx);
                h4 k0, k1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    k0[e] = (_Float16)kx[e];
                    k1[e] = (_Float16)kx[4 + e];
                }
                *reinterpret_cast<h4 *>(&sm.Ks[sl][row0 + q][kpos]) = k0;
                *reinterpret_cast<h4 *>(&sm.Ks[sl][row0 + q][kpos + 8]) = k1;
            }
        };
        // keys of chunk c transposed into KT slot c & 1, by prep waves 1-3 (key blocks
        // xb = 3 (p - 1) .. , all 64 tokens): a transposing read gives lane (g, r16)
        // tokens 16 tb + 4g .. + 3 of stored key column 16 xb + r16, written as one run at
        // the tokens' permuted position
        auto store_kt = [&](int c) {
            const int sl = c % 3, s2 = c & 1;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int xb = 3 * (pw - 1) + i;
                if (xb < 8) {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        const h4 v = tr4(&sm.Ks[sl][0][0], GLK, 16 * tb + 4 * g, 16 * xb, lane);
                        *reinterpret_cast<h4 *>(&sm.KT[s2][perm32_index(16 * xb + r16)][perm32_pos4(16 * tb + 4 * g)]) = v;
                    }
                }
            }
        };

        // ------------------------------------------------------- prep: Gram, M'
        // 16x16 Gram tile K_i K_j^T of slot sl (lane (g, r16), register i: row 4g + i,
        // column r16); the stored key order is the same for both operands
        auto gram_tile = [&](int sl, int ti, int tj) {
            f4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const h8 A = *reinterpret_cast<const h8 *>(&sm.Ks[sl][16 * ti + r16][32 * kb + 8 * g]);
                const h8 B = *reinterpret_cast<const h8 *>(&sm.Ks[sl][16 * tj + r16][32 * kb + 8 * g]);
                acc = mma(A, B, acc);
            }
            return acc;
        };
        // chunk c, prep waves 1-3: two off-diagonal Gram tiles each, negated, into Mx
        auto prep_offgram = [&](int c) {
            const int ms = c & 1, sl = c % 3;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int idx = 2 * (pw - 1) + q, ti = gram_ti(idx), tj = gram_tj(idx);
                const f4 acc = gram_tile(sl, ti, tj);
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.Mx[ms][16 * ti + 4 * g + i][16 * tj + r16] = (_Float16)(-acc[i]);
            }
        };
        // chunk c, prep wave 0: the four diagonal blocks.  Their Gram tiles go through
        // LDS so that lane row g holds block g with one column per lane (G is
        // symmetric); the inverse of I + A'_gg (A' = diag(b) strictlower(G)) follows by
        // forward substitution, x_r += (-A'[r][q]) x_q, the multiplier taken from lane
        // q of the row; M'_gg[r][c] = x_r b_c into the chunk's Mx slot
        auto prep_diag = [&](int c) {
            const int sl = c % 3, ms = c & 1;
            h8 kf[4][4];   // [block][k block]: rows 16 b + r16 (each is both operands of its tile)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    kf[b][kb] = *reinterpret_cast<const h8 *>(&sm.Ks[sl][16 * b + r16][32 * kb + 8 * g]);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f4 acc = zero4();   // lane (g, r16), register i: G_b[4g + i][r16]
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc = mma(kf[b][kb], kf[b][kb], acc);
                *reinterpret_cast<float4 *>(&sm.Gd[b][r16][4 * g]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
            wave_lds_fence();
            // lane (g, c): G_g[r][c] = Gd[g][c][r], r = 0..15; the rows' write strengths
            float n[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 gv = *reinterpret_cast<const float4 *>(&sm.Gd[g][r16][4 * r4]);
                const float4 bv = *reinterpret_cast<const float4 *>(&sm.beta[sl][16 * g + 4 * r4]);
                n[4 * r4 + 0] = -bv.x * gv.x;
                n[4 * r4 + 1] = -bv.y * gv.y;
                n[4 * r4 + 2] = -bv.z * gv.z;
                n[4 * r4 + 3] = -bv.w * gv.w;
            }
            const float bc = sm.beta[sl][16 * g + r16];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = r == r16 ? 1.f : 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(n[r]));   // n complete here
            asm volatile("s_nop 1");   // the two wait states before the lane moves read n
            subst_steps<0>(x, n);
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.Mx[ms][16 * g + r][16 * g + r16] = (_Float16)(x[r] * bc);
        };

        const std::false_type full;
        const std::true_type tail;
        const std::integral_constant<int, 0> p0;
        const std::integral_constant<int, 1> p1;
        if (nch > 0) fetch(0, p0);
        // iteration j: the prefetch of chunk j + 1 first (in flight across the barrier,
        // waited for where the next step first uses it), then chunk j's gates, keys and
        // value rows, then chunk j-1's transposed keys, Gram tiles and inverses
        auto iter = [&](int j, auto pc) {
            constexpr int P = decltype(pc)::value;
            lds_barrier();
            // this chunk's prefetch landed before the barrier: claim its registers now,
            // so no later wait covers the loads issued below
#pragma unroll
            for (int q = 0; q < 4; ++q) claim(kraw[P][q]);
#pragma unroll
            for (int i = 0; i < 4; ++i) claim(vraw[P][i]);
            claim(braw[P]);
            claim(araw[P]);
            claim(vrs[P]);
            if (j + 1 < nch) fetch(j + 1, std::integral_constant<int, P ^ 1>());
            if (j < nch - 1) stage(j, pc, full);
            else if (j == nch - 1) stage(j, pc, tail);
            if (j >= 1 && j <= nch) {
                if (pw == 0) {
                    prep_diag(j - 1);
                } else {
                    prep_offgram(j - 1);
                    store_kt(j - 1);
                }
            }
        };
        for (int j = 0; j < nch + 2; j += 2) {
            iter(j, p0);
            if (j + 1 < nch + 2) iter(j + 1, p1);
        }
        if (w == 4) {   // the prep waves accumulate the log-gates
            const double tot = wave_sum_f64(cl_lane);
            if (lane == 0) sm.cl_tot = tot;
        }
        lds_barrier();
    } else {
        // ---------------------------------------------------------------- state
        // column tiles of X = [Tbar | S] held by state wave w: n = 0, 1 the Tbar
        // tiles 2w, 2w + 1; n = 2, 3 the S tiles 2w, 2w + 1
        f4 X[8][4];
        float sig[4] = {0.f, 0.f, 0.f, 0.f};
        int svq[2] = {0, 0};   // value exponent of the last chunk per S tile
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    X[mt][n][i] = (n < 2 && 16 * mt + 4 * g + i == 16 * (2 * w + n) + r16) ? 1.f : 0.f;

        // Xhat <- Xhat 2^(sig - target): the unit follows the tile's largest entry,
        // never below 2^(ev - 4) for S (keeps the value term of P within fp16 range)
        auto renorm = [&](int n, bool isS, int ev) {
            float xm = 0.f;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) xm = fmaxf(xm, fabsf(X[mt][n][i]));
            xm = wave_max(xm);
            float target = (float)pow2_exponent(xm) + sig[n];
            if (xm == 0.f) target = isS ? (float)ev : sig[n];
            if (isS && target < (float)ev - 4.f) target = (float)ev - 4.f;
            // an integer shift, exact, and finite however far the tile has decayed
            const int sh = (int)(sig[n] - target);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) X[mt][n][i] = ldexpf(X[mt][n][i], sh);
            sig[n] = target;
        };
        // chunk c, before its products: the chunk gate on S
        // chunk c, before its products: the chunk gate on S
        auto state_pre = [&](int c) {
            const float gbv = sm.gb[c % 3];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                X[mt][2] *= gbv;
                X[mt][3] *= gbv;
            }
        };
        h4 Eh[4][2];   // [token block][column tile of the half]
        // chunk c, column half hf (tiles 2 hf, 2 hf + 1): P = [0 | diag(dec) V 2^-sig] - K Xhat,
        // E by block forward substitution, E_i = M'_ii (P_i - sum_{j<i} G_ij E_j), kept
        // as fp16 (accumulator layout: rows 16 i + 4g + e, column r16), then X += K^T E
        // for the half's tiles (the halves are independent columns of X)
        auto state_half = [&](int c, auto hfc) {
            constexpr int hf = decltype(hfc)::value;
            const int sl = c % 3, s2 = c & 1;
            // bases: K rows (P's A operand, 16 bytes per lane), K^T rows (the update's
            // A operand, 16 bytes per lane), the Mx rows
            lds_h *kA = lds_base(&sm.Ks[sl][r16][8 * g]);
            lds_h *kT = lds_base(&sm.KT[s2][r16][8 * g]);
            lds_h *mx = lds_base(&sm.Mx[s2][r16][4 * g]);
            // Software pipeline: every LDS fragment is requested one step before
            // the products that use it (the scheduling fences keep the requests
            // ahead), so a single wave keeps the matrix core fed.
            h8 Ak[2][4];   // K rows 16 tt + r16, keys 32 kb + 4g + (e & 3) + 16 (e >> 2)
            auto load_k = [&](int kb, h8 (&dst)[4]) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) dst[tt] = lds8h(kA + 16 * tt * GLK + 32 * kb);
            };
            h4 Am[10];     // Mx fragments: -G_ij (j < i) and M'_ii, in use order
            auto load_m = [&]() {
                int n = 0;
#pragma unroll
                for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                    for (int jb = 0; jb <= ib; ++jb) Am[n++] = lds4h(mx + 16 * ib * GLP + 16 * jb);
            };
            h8 At[2][2];   // K^T rows 16 mt + r16, tokens 32 jb + 4g + (e & 3) + 16 (e >> 2)
            auto load_t = [&](int mt, h8 (&dst)[2]) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) dst[jb] = lds8h(kT + 16 * mt * GLT + 32 * jb);
            };

            f4 P[4][2];    // [token block][column tile of the half]
            load_k(0, Ak[0]);
            if constexpr (hf == 0) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) P[tt][0] = P[tt][1] = zero4();
            } else {
                // value term: lane (g, r16) reads V[16 tt + 4g + e][16 (2w + q) + r16], e = 0..3,
                // through the transposing load (lane j's 8 bytes: row 4g + (j >> 2) of the
                // block, piece 4w + 2q + ((j >> 1) & 1) at its swizzled position, half j & 1)
                const int t4 = 4 * g + (r16 >> 2);
                lds_h *vb[2];
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    vb[q] = lds_base(&sm.Vr[sl][t4][8 * ((4 * w + 2 * q + ((r16 >> 1) & 1)) ^ (2 * (t4 & 7))) + 4 * (r16 & 1)]);
                lds_h *fb = lds_base(&sm.fac[sl][4 * g]);
                float vmax[2] = {0.f, 0.f};
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const f4 f = lds4f(fb + 32 * tt);   // fac[16 tt + 4g + e] (floats: 2 halves each)
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const s4v v = lds_tr4s(vb[q] + 16 * tt * GD);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            P[tt][q][e] = raw_f32(v[e], TV()) * f[e];
                            vmax[q] = fmaxf(vmax[q], fabsf(P[tt][q][e]));
                        }
                    }
                }
                // the S unit: the chunk's value scale on the first chunk (S is zero),
                // renormalised when the values run more than 2^4 ahead of it
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    svq[q] = pow2_exponent(wave_max_nn(vmax[q]));
                    if (c == 0) sig[2 + q] = (float)svq[q];
                    else if ((float)svq[q] > sig[2 + q] + 4.f) renorm(2 + q, true, svq[q]);
                    const int isg = (int)sig[2 + q];
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) P[tt][q][e] = ldexpf(P[tt][q][e], -isg);
                }
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                if (kb < 3) load_k(kb + 1, Ak[(kb + 1) & 1]);
                else load_m();
                sched_fence();
                h8 B[2];   // -Xhat, keys 32 kb + 4g + (e & 3) + 16 (e >> 2)
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        B[q][i] = (_Float16)(-X[2 * kb][2 * hf + q][i]);
                        B[q][4 + i] = (_Float16)(-X[2 * kb + 1][2 * hf + q][i]);
                    }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int q = 0; q < 2; ++q) P[tt][q] = mma(Ak[kb & 1][tt], B[q], P[tt][q]);
                sched_fence();
            }
            load_t(0, At[0]);
            sched_fence();
            {
                int n = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int jb = 0; jb < i; ++jb, ++n)
#pragma unroll
                        for (int q = 0; q < 2; ++q) P[i][q] = mma16(Am[n], Eh[jb][q], P[i][q]);
#pragma unroll
                    for (int q = 0; q < 2; ++q) Eh[i][q] = cvt4(mma16(Am[n], cvt4(P[i][q]), zero4()));
                    ++n;
                }
            }
            sched_fence();
            // X += K^T E for the half's two tiles
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                if (mt < 7) load_t(mt + 1, At[(mt + 1) & 1]);
                sched_fence();
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        X[mt][2 * hf + q] = mma(At[mt & 1][jb], cat8(Eh[2 * jb][q], Eh[2 * jb + 1][q]), X[mt][2 * hf + q]);
                sched_fence();
            }
        };
        // periodic renormalisation of the four tiles, every 4 chunks
        auto state_post = [&](int c) {
            if ((c & 3) == 3) {
#pragma unroll
                for (int n = 0; n < 4; ++n) renorm(n, n >= 2, n >= 2 ? svq[n - 2] : 0);
            }
        };
        auto state = [&](int c) {
            state_pre(c);
            state_half(c, std::integral_constant<int, 0>());
            state_half(c, std::integral_constant<int, 1>());
            state_post(c);
        };

        for (int j = 0; j < nch + 2; ++j) {
            lds_barrier();
            if (j >= 2) state(j - 2);
        }
        lds_barrier();
        const double cl_tot = sm.cl_tot;
        float *Tu = a.T_out + (int64_t)unit * GD * GD;
        float *Su = a.S0_out + (int64_t)unit * GD * GD;
        int g4 = 4 * g;   // opaque: keeps the row indices from being computed before the loop
        asm volatile("" : "+v"(g4));
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const bool isS = n >= 2;
            const int col = 16 * (2 * w + (n & 1)) + r16;
            const double e = (double)sig[n] + (isS ? 0.0 : cl_tot);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * mt + g4 + i;
                    const float val = scale_pow2(X[mt][n][i], e);
                    if (isS) Su[row * GD + col] = val;
                    else     Tu[row * GD + col] = val;
                }
        }
    }
}

template <typename TK, typename TV, typename TG>
static hipError_t launch_gdn_one(const DeltaArgs &a, int n_units, hipStream_t st)
{
    const size_t smem = sizeof(GdnSmem);
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = allow_dyn_lds(&build_gdn_kernel<TK, TV, TG>, smem, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL((build_gdn_kernel<TK, TV, TG>), dim3(n_units), dim3(512), smem, st, a);
    return hipGetLastError();
}

// d = 128, bf16 inputs (keys, values, gates), or the conv workspace of a
// bf16-input build (fp16 keys, fp16 values with a power of two per row) with
// bf16 gates
hipError_t launch_build_gdn(const DeltaArgs &a, int kv_kind, int g_kind, int n_units, hipStream_t st)
{
    if (g_kind != IN_BF16) return hipErrorInvalidValue;
    if (kv_kind == IN_BF16) return launch_gdn_one<bf16_t, bf16_t, bf16_t>(a, n_units, st);
    if (kv_kind == IN_F16K) return launch_gdn_one<_Float16, _Float16, bf16_t>(a, n_units, st);
    return hipErrorInvalidValue;
}

}  // namespace hy

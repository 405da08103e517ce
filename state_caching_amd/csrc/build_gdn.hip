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
// The substitution runs over two 32-row blocks: M'_00 and M'_11 are the
// inverses of the two 32 x 32 diagonal blocks (times diag(b)), each assembled
// from two 16-row inverses as [[M'_a, 0], [-M'_b G_ba M'_a, M'_b]], and G_10 is
// the 32 x 32 block of G below the diagonal, so
//   E_0 = M'_00 P_0,   E_1 = M'_11 (P_1 - G_10 E_0).
//
// One workgroup of 8 waves per (segment, value head), two per SIMD: a state
// wave and a prep wave.  Between two barriers:
//   state waves 0-3  state(j-2): wave w owns the 32-column tile w of Tbar and
//                    of S (fp32 in matrix-core accumulators, 32 x 32 x 16
//                    products): P (one tile at a time; the value term scaled
//                    from the raw rows here), the two-block substitution for E,
//                    and X += K^T E
//   prep waves 4-7   chunk j (waves 6 and 7, 32 rows each): the raw value rows
//                    and the key rows (prefetched into registers, keys converted
//                    to fp16) to LDS; gates (wave 7).  Chunk j-1: waves 4 and 5 each one
//                    32-row inverse M'_ii (its two 16-row diagonal inverses, one
//                    block per lane row with the multipliers broadcast across the
//                    row by lane moves, joined by -M'_b G_ba M'_a); wave 6 the
//                    32 x 32 block -G_10 in one 32 x 32 x 16 product
// The reduction order of a 32 x 32 accumulator tile, read as an operand, runs
// over rows 4a + {0..3} and 8 + 4a + {0..3} of each 16-block (lane half a), so
// every operand fragment is two runs of four: the P product reads its key
// fragments as two 8-byte runs of a key row, and the M tiles (stored transposed,
// token-major) and K^T (the key rows themselves) reach their products through
// two transposing loads per fragment.
// X is kept in power-of-two units per column tile (renormalised every 4
// chunks, or when a chunk's values run ahead of the S unit), so every fp16
// operand stays in range.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace hy {
namespace {

// fourth word of a raw buffer resource: 32-bit data format, so untyped loads
// return data and loads past the resource's size return zero
#define HY_BUF_DW3 0x00020000
constexpr int GD = 128;          // d_k = d_v
constexpr int GLK = GD + 8;      // Ks row stride (halves)
constexpr int GLM = 32 + 8;      // Mx row stride (halves)
constexpr int GLG = 20;          // Gd row stride (floats)

struct GdnSmem {
    _Float16 Ks[3][64][GLK];     // keys in fp16, token-major, natural key order
    unsigned short Vr[3][64][GD];   // raw value rows as stored (bf16 or fp16 bits); the 16-byte
                                    // piece p of row t sits at piece position p ^ (2 (t & 7))
    _Float16 Mx[2][3][32][GLM];  // per chunk slot: M'_00, M'_11 and -G_10 (32 x 32 each), stored
                                 // transposed, Mx[.][.][token][row]; the upper right 16 x 16
                                 // blocks of the two inverses stay zero
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
typedef float f16v __attribute__((ext_vector_type(16)));
// registers o .. o + 7 of a 32 x 32 accumulator tile as an fp16 operand
__device__ __forceinline__ h8 cvt8(const f16v &v, int o)
{
    h8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)v[o + e];
    return r;
}
// 32x32x16 product: lane holds A[l%32][8(l/32) + e], B[8(l/32) + e][l%32]; the
// result register i is row 8 (i >> 2) + 4 (l/32) + (i & 3), column l%32
__device__ __forceinline__ f16v mma32(h8 a, h8 b, f16v c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
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

    // the upper right 16 x 16 blocks of the two 32-row inverses are never written:
    // zero all M tiles once (the roles' first barrier orders this)
    {
        uint32_t *mz = reinterpret_cast<uint32_t *>(&sm.Mx[0][0][0][0]);
        for (int i = tid; i < (int)(sizeof(sm.Mx) / 4); i += 512) mz[i] = 0u;
    }
    // The two roles keep their registers apart: every variable, lambda and loop
    // of a role lives inside its branch.  Both roles meet the same nch + 3 barriers.
    if (w >= 4) {
        // ------------------------------------------------------------ staging
        // Prep waves 2 and 3 stage the chunk, rows 0-31 and 32-63 (wave 3 also the
        // gates); waves 0 and 1 form the inverses.  Lane (g, r16) stages key rows
        // rbase + MR g + q, columns 8 r16 .. 8 r16 + 7, and value rows rbase + 4i + g.
        constexpr int MR = 8;
        const int pw = w - 4;
        const bool stager = pw >= 2;
        const int rbase = pw == 3 ? 32 : 0;
        const int row0 = rbase + MR * g;
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
        typename Raw8<TK>::type kraw[2][MR];
        uint4 vraw[2][MR];
        TG braw[2], araw[2];
        float vrs[2];
        // Key and value rows through buffer loads: per chunk, a resource whose base is the
        // chunk's first row and whose size covers only its rows inside the segment, so
        // rows past the segment end read as zero; each lane's byte offsets inside a chunk
        // are fixed
        const uint32_t ldk_b = (uint32_t)(a.ldk * (int64_t)sizeof(TK));
        uint32_t koff[MR], voff[MR];
#pragma unroll
        for (int q = 0; q < MR; ++q) {
            koff[q] = (uint32_t)(row0 + q) * ldk_b + (uint32_t)(16 * r16);
            const int t = rbase + 4 * q + g;
            voff[q] = (uint32_t)t * ldv_b + 16 * (r16 ^ (2 * (t & 7)));
        }
        auto fetch = [&](int c, auto pc) {
            constexpr int P = decltype(pc)::value;
            const int last = len - 1 - 64 * c;   // >= 0 for every chunk of the segment
            const int rows = min(last + 1, 64);
            const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(reinterpret_cast<const unsigned char *>(kb) + (int64_t)(64 * c) * ldk_b), (short)0,
                (int)((uint32_t)rows * ldk_b), HY_BUF_DW3);
            const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(vb + (int64_t)(64 * c) * ldv_b), (short)0, (int)((uint32_t)rows * ldv_b), HY_BUF_DW3);
#pragma unroll
            for (int q = 0; q < MR; ++q)
                kraw[P][q].u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)koff[q], 0, 0));
            if (pw == 3) {   // the gate wave
                const uint32_t go = __umul24(min(lane, last), (unsigned)a.h_v);
                const int64_t gc = (int64_t)(64 * c) * a.h_v;
                braw[P] = bp[gc + go];
                araw[P] = ap[gc + go];
                if constexpr (VSC) vrs[P] = vsp[gc + go];
                else vrs[P] = 1.f;
            }
            // raw value rows rbase + 4i + g, the 16-byte piece r16 ^ 2 (t & 7) of row t
#pragma unroll
            for (int i = 0; i < MR; ++i)
                vraw[P][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, (int)voff[i], 0, 0));
        };

        double cl_lane = 0.0;
        // chunk c into slot c % 3 from prefetch buffer P: gates (prep wave 3 alone) and this
        // wave's 16 key rows.  TAIL: the segment's last chunk, whose rows past the end read
        // as zero.
        auto stage = [&](int c, auto pc, auto tail) {
            constexpr int P = decltype(pc)::value;
            const int sl = c % 3;
            if (pw == 3) {
                const bool gin = 64 * c + lane < len;
                const float br = gin ? to_f32(braw[P]) : 0.f, ar = gin ? to_f32(araw[P]) : 1.f;
                const float l2 = log2f(ar);
                const float sfx = wave_suffix_excl(l2);   // log2 dec_t
                cl_lane += (double)l2;
                sm.beta[sl][lane] = br;
                sm.fac[sl][lane] = gin ? exp2f(sfx) * vrs[P] : 0.f;
                sm.gb[sl] = exp2f(lane_f(sfx + l2, 0));
            }
            // value rows into slot sl: row rbase + 4i + g, piece position r16
#pragma unroll
            for (int i = 0; i < MR; ++i)
                *reinterpret_cast<uint4 *>(&sm.Vr[sl][rbase + 4 * i + g][8 * r16]) = vraw[P][i];
            if constexpr (decltype(tail)::value) {
#pragma unroll
                for (int q = 0; q < MR; ++q) mask_raw8(kraw[P][q], 64 * c + row0 + q < len);
            }
            // keys 8 r16 .. 8 r16 + 7 in fp16, one 16-byte store per row
#pragma unroll
            for (int q = 0; q < MR; ++q) {
                float kx[8];
                widen8(kraw[P][q], kx);
                h8 k8;
#pragma unroll
                for (int e = 0; e < 8; ++e) k8[e] = (_Float16)kx[e];
                *reinterpret_cast<h8 *>(&sm.Ks[sl][row0 + q][8 * r16]) = k8;
            }
        };
        // ------------------------------------------------------- prep: Gram, M'
        // chunk c, prep wave 2: -G_10, the 32 x 32 Gram block of tokens 32..63 against
        // 0..31, in one 32 x 32 x 16 product (lane (l32, hh) of the result holds rows
        // 8j + 4hh + e of column l32), written transposed, four rows per store
        auto prep_g10 = [&](int c) {
            const int sl = c % 3, ms = c & 1;
            const int l32 = lane & 31, hh = lane >> 5;
            f16v acc = f16v{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const h8 A = *reinterpret_cast<const h8 *>(&sm.Ks[sl][32 + l32][16 * ks + 8 * hh]);
                const h8 B = *reinterpret_cast<const h8 *>(&sm.Ks[sl][l32][16 * ks + 8 * hh]);
                acc = mma32(A, B, acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<h4 *>(&sm.Mx[ms][2][l32][8 * j + 4 * hh]) =
                    h4{(_Float16)(-acc[4 * j]), (_Float16)(-acc[4 * j + 1]), (_Float16)(-acc[4 * j + 2]), (_Float16)(-acc[4 * j + 3])};
        };
        // chunk c, prep wave p (0 or 1): the 32-row inverse M'_pp from the 16-row blocks
        // a = 2p, b = 2p + 1.  Their Gram tiles go through LDS so that lane row g holds
        // block 2p + (g & 1) with one column per lane (G is symmetric; rows 2 and 3
        // repeat rows 0 and 1); the inverse of I + A'_bb (A' = diag(b) strictlower(G))
        // follows by forward substitution, x_r += (-A'[r][q]) x_q, the multiplier taken
        // from lane q of the row; M'_bb[r][c] = x_r b_c into the chunk's Mx slot.  Then
        // the lower left 16 x 16 block, -M'_b G_ba M'_a.
        auto prep_diag = [&](int c) {
            const int sl = c % 3, ms = c & 1, p = pw;
            h8 kf[2][4];   // [block a or b][k block]: rows 16 (2p + e) + r16
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    kf[e][kb] = *reinterpret_cast<const h8 *>(&sm.Ks[sl][16 * (2 * p + e) + r16][32 * kb + 8 * g]);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                f4 acc = zero4();   // lane (g, r16), register i: G_b[4g + i][r16]
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc = mma(kf[e][kb], kf[e][kb], acc);
                *reinterpret_cast<float4 *>(&sm.Gd[2 * p + e][r16][4 * g]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
            // G_ab: lane (g, r16) holds G_ab[4g + i][r16] = G_ba[r16][4g + i], which is
            // G_ba's operand layout on the left of a product
            h4 Gba;
            {
                f4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc = mma(kf[0][kb], kf[1][kb], acc);
                Gba = cvt4(acc);
            }
            wave_lds_fence();
            // lane (g, c): G_blk[r][c] = Gd[blk][c][r], r = 0..15; the rows' write strengths
            const int e = g & 1, blk = 2 * p + e;
            float n[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 gv = *reinterpret_cast<const float4 *>(&sm.Gd[blk][r16][4 * r4]);
                const float4 bv = *reinterpret_cast<const float4 *>(&sm.beta[sl][16 * blk + 4 * r4]);
                n[4 * r4 + 0] = -bv.x * gv.x;
                n[4 * r4 + 1] = -bv.y * gv.y;
                n[4 * r4 + 2] = -bv.z * gv.z;
                n[4 * r4 + 3] = -bv.w * gv.w;
            }
            const float bc = sm.beta[sl][16 * blk + r16];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = r == r16 ? 1.f : 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(n[r]));   // n complete here
            asm volatile("s_nop 1");   // the two wait states before the lane moves read n
            subst_steps<0>(x, n);
            if (g < 2) {
                // column r16 of block blk, rows 0..15: one contiguous run of the transposed tile
                const int off = 16 * e;
                h8 lo, hi;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    lo[r] = (_Float16)(x[r] * bc);
                    hi[r] = (_Float16)(x[8 + r] * bc);
                }
                *reinterpret_cast<h8 *>(&sm.Mx[ms][p][off + r16][off]) = lo;
                *reinterpret_cast<h8 *>(&sm.Mx[ms][p][off + r16][off + 8]) = hi;
            }
            wave_lds_fence();
            // T = G_ba M'_a: lane (g, j) holds M'_a[4g .. 4g + 3][j], contiguous in the
            // transposed tile, and so T
            const h4 Ma = *reinterpret_cast<const h4 *>(&sm.Mx[ms][p][r16][4 * g]);
            const f4 T = mma16(Gba, Ma, zero4());
            // L = -M'_b T: lane (r16, g) holds M'_b[r16][4g .. 4g + 3] through the
            // transposing load; lane (g, j) writes L[4g .. 4g + 3][j] as one run
            const h4 Mb = tr4(&sm.Mx[ms][p][0][0], GLM, 16 + 4 * g, 16, lane);
            const f4 L = mma16(Mb, cvt4(T), zero4());
            *reinterpret_cast<h4 *>(&sm.Mx[ms][p][r16][16 + 4 * g]) = cvt4(-L);
        };

        const std::false_type full;
        const std::true_type tail;
        const std::integral_constant<int, 0> p0;
        if (stager && nch > 0) fetch(0, p0);
        // iteration j: chunk j's gates, keys and value rows from the registers, then the
        // prefetch of chunk j + 1 into them (in flight across the barrier, waited for where
        // the next step first uses it), then chunk j-1's transposed keys, Gram tiles and
        // inverses
        auto iter = [&](int j, auto pc) {
            constexpr int P = decltype(pc)::value;
            lds_barrier();
            // this chunk's prefetch landed before the barrier: claim its registers now,
            // so no later wait covers the loads issued below
            if (stager) {
#pragma unroll
                for (int q = 0; q < MR; ++q) claim(kraw[P][q]);
#pragma unroll
                for (int i = 0; i < MR; ++i) claim(vraw[P][i]);
            }
            if (pw == 3) {
                claim(braw[P]);
                claim(araw[P]);
                claim(vrs[P]);
            }
            if (stager) {
                if (j < nch - 1) stage(j, pc, full);
                else if (j == nch - 1) stage(j, pc, tail);
            }
            // the next chunk's prefetch reuses the registers just staged (one buffer:
            // the loads still have the rest of this step and the barrier to land)
            if (stager && j + 1 < nch) fetch(j + 1, pc);
            if (j >= 1 && j <= nch) {
                if (pw < 2) prep_diag(j - 1);
                else if (pw == 2) prep_g10(j - 1);
            }
        };
        for (int j = 0; j < nch + 2; ++j) iter(j, p0);
        if (w == 7) {   // the gate wave accumulates the log-gates
            const double tot = wave_sum_f64(cl_lane);
            if (lane == 0) sm.cl_tot = tot;
        }
        lds_barrier();
    } else {
        // ---------------------------------------------------------------- state
        // column tiles of X = [Tbar | S] held by state wave w: n = 0 the Tbar tile w,
        // n = 1 the S tile w (32 columns each), as four 32-row tiles.  Lane (l32, hh),
        // register i of a tile: row 32 rt + 8 (i >> 2) + 4 hh + (i & 3), column 32 w + l32
        const int l32 = lane & 31, hh = lane >> 5;
        f16v X[4][2];
        float sig[2] = {0.f, 0.f};
        int svq = 0;   // value exponent of the last chunk (S tile)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    X[rt][n][i] = (n == 0 && 32 * rt + 8 * (i >> 2) + 4 * hh + (i & 3) == 32 * w + l32) ? 1.f : 0.f;

        // Xhat <- Xhat 2^(sig - target): the unit follows the tile's largest entry,
        // never below 2^(ev - 4) for S (keeps the value term of P within fp16 range)
        auto renorm = [&](int n, bool isS, int ev) {
            float xm = 0.f;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 16; ++i) xm = fmaxf(xm, fabsf(X[rt][n][i]));
            xm = wave_max(xm);
            float target = (float)pow2_exponent(xm) + sig[n];
            if (xm == 0.f) target = isS ? (float)ev : sig[n];
            if (isS && target < (float)ev - 4.f) target = (float)ev - 4.f;
            // an integer shift, exact, and finite however far the tile has decayed
            const int sh = (int)(sig[n] - target);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 16; ++i) X[rt][n][i] = ldexpf(X[rt][n][i], sh);
            sig[n] = target;
        };
        // chunk c, before its products: the chunk gate on S
        auto state_pre = [&](int c) {
            const float gbv = sm.gb[c % 3];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) X[rt][1] *= gbv;
        };
        // chunk c: P = [0 | diag(dec) V 2^-sig] - K Xhat for both tiles (two 32-token
        // tiles each), E by the two-block substitution E_0 = M'_00 P_0, E_1 = M'_11 (P_1 -
        // G_10 E_0) (fp16 operands from the accumulators: registers 8m .. 8m + 7 of a
        // 32-row tile are its rows 16m + {4hh .. 4hh + 3, 8 + 4hh .. 8 + 4hh + 3}, the
        // stored order of the operands' 16-blocks), then X += K^T E.  Every key and M
        // fragment read from LDS feeds both tiles, and the two tiles' substitutions
        // interleave.
        auto state_chunk = [&](int c) {
            const int sl = c % 3, s2 = c & 1;
            // bases: K rows (P's left operand: keys 4hh .. 4hh + 3 of a 16-key block, and 8
            // more on), the K^T and M fragments (the left operands of the update and of the
            // substitution: in lane row G of the wave, lane j supplies the 8 bytes of row
            // 4 hh + (j >> 2), columns 16 (G & 1) + 4 (j & 3) .. of the transposing load)
            const int G = lane >> 4, lj = lane & 15;
            lds_h *kA = lds_base(&sm.Ks[sl][l32][4 * hh]);
            lds_h *kT = lds_base(&sm.Ks[sl][4 * hh + (lj >> 2)][16 * (G & 1) + 4 * (lj & 3)]);
            lds_h *mx = lds_base(&sm.Mx[s2][0][4 * hh + (lj >> 2)][16 * (G & 1) + 4 * (lj & 3)]);
            // Software pipeline: every LDS fragment is requested one step before
            // the products that use it (the scheduling fences keep the requests
            // ahead), so a single wave keeps the matrix core fed.
            h8 Ak[2][2];   // [buffer][token tile]: K rows 32 tt + l32, keys of block ks
            auto load_k = [&](int ks, h8 (&dst)[2]) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    dst[tt] = cat8(lds4h(kA + 32 * tt * GLK + 16 * ks), lds4h(kA + 32 * tt * GLK + 16 * ks + 8));
            };
            h8 Am[2];      // one 32 x 32 tile of Mx (M'_00, M'_11 or -G_10), token blocks m = 0, 1
            auto load_m = [&](int b) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    lds_h *p = mx + 32 * b * GLM + 16 * m * GLM;
                    Am[m] = cat8(__builtin_bit_cast(h4, lds_tr4s(p)), __builtin_bit_cast(h4, lds_tr4s(p + 8 * GLM)));
                }
            };
            h8 At[2][2];   // [buffer][token block of the pair]: K^T rows 32 rt + l32
            auto load_t = [&](int rt, int kp, h8 (&dst)[2]) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    lds_h *p = kT + 16 * (2 * kp + q) * GLK + 32 * rt;
                    dst[q] = cat8(__builtin_bit_cast(h4, lds_tr4s(p)), __builtin_bit_cast(h4, lds_tr4s(p + 8 * GLK)));
                }
            };

            f16v P[2][2];  // [tile][token tile 0-31, 32-63]
            load_k(0, Ak[0]);
            P[0][0] = P[0][1] = f16v{};
            {
                // value term of the S tile: lane (l32, hh) reads V[32 tt + 8j + 4hh + e][32 w + l32],
                // e = 0..3, through the transposing load: in lane row G = lane >> 4, lane j reads
                // 8 bytes of row 32 tt + 8j + 4 (G >> 1) + (j >> 2), piece 4w + 2 (G & 1) +
                // ((j >> 1) & 1) at its swizzled position, half j & 1
                const int G = lane >> 4, lj = lane & 15;
                const int t4 = 4 * (G >> 1) + (lj >> 2);
                lds_h *vb = lds_base(&sm.Vr[sl][t4][8 * ((4 * w + 2 * (G & 1) + ((lj >> 1) & 1)) ^ (2 * (t4 & 7))) + 4 * (lj & 1)]);
                lds_h *fb = lds_base(&sm.fac[sl][4 * hh]);
                float vmax = 0.f;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f4 f = lds4f(fb + 2 * (32 * tt + 8 * j));   // fac[32 tt + 8j + 4hh + e]
                        const s4v v = lds_tr4s(vb + (32 * tt + 8 * j) * GD);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            P[1][tt][4 * j + e] = raw_f32(v[e], TV()) * f[e];
                            vmax = fmaxf(vmax, fabsf(P[1][tt][4 * j + e]));
                        }
                    }
                // the S unit: the chunk's value scale on the first chunk (S is zero),
                // renormalised when the values run more than 2^4 ahead of it
                svq = pow2_exponent(wave_max_nn(vmax));
                if (c == 0) sig[1] = (float)svq;
                else if ((float)svq > sig[1] + 4.f) renorm(1, true, svq);
                const int isg = (int)sig[1];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) P[1][tt][i] = ldexpf(P[1][tt][i], -isg);
            }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks < 7) load_k(ks + 1, Ak[(ks + 1) & 1]);
                else load_m(0);
                sched_fence();
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    h8 B;   // -Xhat, keys 16 ks + the stored order of the block
#pragma unroll
                    for (int e = 0; e < 8; ++e) B[e] = (_Float16)(-X[ks >> 1][n][8 * (ks & 1) + e]);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) P[n][tt] = mma32(Ak[ks & 1][tt], B, P[n][tt]);
                }
                sched_fence();
            }
            h8 Eh[2][4];   // [tile] E as fp16, token blocks of 16
            {
                // each Mx tile is requested while the products before its use run
                f16v E[2];
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    E[n] = mma32(Am[0], cvt8(P[n][0], 0), f16v{});
                    E[n] = mma32(Am[1], cvt8(P[n][0], 8), E[n]);
                }
                sched_fence();
                load_m(2);
                sched_fence();
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    Eh[n][0] = cvt8(E[n], 0);
                    Eh[n][1] = cvt8(E[n], 8);
                    P[n][1] = mma32(Am[0], Eh[n][0], P[n][1]);
                    P[n][1] = mma32(Am[1], Eh[n][1], P[n][1]);
                }
                sched_fence();
                load_m(1);
                sched_fence();
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const h8 Pa = cvt8(P[n][1], 0), Pb = cvt8(P[n][1], 8);
                    E[n] = mma32(Am[0], Pa, f16v{});
                    E[n] = mma32(Am[1], Pb, E[n]);
                }
                sched_fence();
                load_t(0, 0, At[0]);
                sched_fence();
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    Eh[n][2] = cvt8(E[n], 0);
                    Eh[n][3] = cvt8(E[n], 8);
                }
            }
            sched_fence();
            // X += K^T E for both tiles: row tile rt, token block pairs kp = 0, 1
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const int rt = st >> 1, kp = st & 1;
                if (st < 7) load_t((st + 1) >> 1, (st + 1) & 1, At[(st + 1) & 1]);
                sched_fence();
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int q = 0; q < 2; ++q) X[rt][n] = mma32(At[st & 1][q], Eh[n][2 * kp + q], X[rt][n]);
                sched_fence();
            }
        };
        // periodic renormalisation of the two tiles, every 4 chunks
        auto state_post = [&](int c) {
            if ((c & 3) == 3) {
                renorm(0, false, 0);
                renorm(1, true, svq);
            }
        };
        auto state = [&](int c) {
            state_pre(c);
            state_chunk(c);
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
        int h4r = 4 * hh;   // opaque: keeps the row indices from being computed before the loop
        asm volatile("" : "+v"(h4r));
        const int col = 32 * w + l32;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const bool isS = n == 1;
            // 2^e split into an integer exponent and a factor in [1, 2) (0 once the tile
            // has decayed below the float range), the same for the whole tile
            const double e = (double)sig[n] + (isS ? 0.0 : cl_tot);
            const double fl = floor(e);
            const int ie = e < -400.0 ? 0 : (int)fl;
            const float fr = e < -400.0 ? 0.f : exp2f((float)(e - fl));
            float *dst = isS ? Su : Tu;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 32 * rt + 8 * (i >> 2) + h4r + (i & 3);
                    dst[row * GD + col] = ldexpf(X[rt][n][i] * fr, ie);
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

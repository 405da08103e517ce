/*
 * hypic.h -- C ABI of the MI355X (gfx950) linear-attention state-caching library.
 *
 * The library implements the linear-layer hot path of HYPIC's
 * position-independent caching (page "HYPIC ... reading notes"):
 *
 *   hypic_segment_build  the cached pair (T_C, S_{C|0}) of each cold segment:
 *                        T_C = T_m ... T_1 and S_{C|0} = sum_t T_m...T_{t+1} u_t,
 *                        the end state of S_i = T_i S_{i-1} + u_i from S_0 = 0
 *                        (ch.1 sec.2 Eq. (2); ch.2 sec.2; ch.2 sec.4)
 *   hypic_compose        S <- T_C S + S_{C|0} over the segments of a prompt, in
 *                        prompt order (ch.2 sec.2, Eq. (6)), optionally with the
 *                        seam window of every inner segment folded in first
 *                        (ch.2 secs.5-6)
 *   hypic_seam_advance   advance running states over a seam window: the first w
 *                        tokens of an inner segment recomputed from the prefix
 *                        state, with the causal-conv warm-up from the previous
 *                        segment's tail rows (ch.2 secs.5-6)
 *   hypic_rope_rerotate  move cached full-attention keys to their positions in
 *                        the request, K_b = R(b - a) K_a (ch.2 sec.6, Eq. (8));
 *                        hypic_rope_rerotate_state moves a scalar-transition
 *                        state the same way (Eq. (7))
 *
 * Transition families (ch.2 sec.3, Table 1), chosen by (rule, gate_kind):
 *   DECAY + HEAD_CONST : T_i = gamma_h I,      u_i = k_i v_i^T  (RetNet)     T_C scalar
 *   DECAY + SCALAR     : T_i = a_i I,          u_i = k_i v_i^T  (Mamba2)     T_C scalar
 *   DECAY + DIAG       : T_i = diag(g_i),      u_i = k_i v_i^T  (GLA)        T_C diagonal
 *   DELTA + SCALAR     : T_i = a_i(I - b_i k_i k_i^T), u_i = b_i k_i v_i^T
 *                        (GDN; DeltaNet is a_i = 1)                           T_C dense
 *   DELTA + DIAG       : T_i = (I - b_i k_i k_i^T) diag(g_i), u_i = b_i k_i v_i^T
 *                        (KDA)                                                T_C dense
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller; arrays are
 *     contiguous, row-major, leading index first.  Tables named "HOST" are
 *     host arrays read before the call returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise.  The library never allocates or frees
 *     device memory; scratch is the caller's workspace (hypic_workspace_size),
 *     except for hypic_compose_noalloc, which uses a static device array.
 *   - Argument errors are returned synchronously as negative hypic_status and
 *     nothing is launched.  Launch failures return HYPIC_E_HIP.  A device fault
 *     surfaces at the caller's next synchronisation.
 *   - Nothing is printed and no exception crosses the boundary.  Calls are
 *     thread-safe; calls that overlap on one device write only their own
 *     outputs.
 *   - Supported head dimensions: d_k = d_v in {16, 32, 64, 128}.  Other shapes
 *     return HYPIC_E_UNSUPPORTED.  Pointers must be 16-byte aligned.
 *   - States, transitions and pair pools are fp32.  Inputs are fp32 or bf16.
 *     Precision: fp32 inputs are computed with fp32 matrix products (relative
 *     Frobenius error ~1e-6).  bf16 inputs of the delta rule (scalar gate, and
 *     per-channel gate at d >= 64) use fp16 matrix-core operands with fp32
 *     accumulation and power-of-two block scaling (~3e-4 on S, <=1.7e-3 on
 *     dense T_C for 4096-token segments; the per-channel gate's Gram matrix and
 *     triangular inverse stay fp32); delta-rule segments longer than 4096
 *     tokens are built with fp32 products whatever the input dtype (the fp16
 *     rounding of every 64-token chunk would add up past 2e-3 on T_C).  bf16
 *     inputs of the decay family take bf16 hi + lo key products against the
 *     exact bf16 values (<= 5e-6 in the tests); factors below 2^-126 of a chunk's own
 *     contributions flush to zero.
 *   - Delta rule keys enter the matrix products as given: they are meant to be
 *     L2-normalised (k_l2norm = 1, or by the caller), with b_t |k_t|^2 <= 2 so
 *     that no transition expands.  With bf16 inputs the keys, b and the solved
 *     pseudo-keys are fp16 operands: key entries must stay below 2^15 in
 *     magnitude (larger ones overflow to non-finite pairs), and nonzero entries
 *     below 2^-14 lose relative precision.  Keys of norm 2^-4 .. 2^4 with
 *     b scaled by the inverse square are tested at the bf16 bound.
 */
#ifndef HYPIC_H
#define HYPIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HYPIC_OK = 0,
    HYPIC_E_INVALID = -1,      /* null pointer, negative or inconsistent size     */
    HYPIC_E_UNSUPPORTED = -2,  /* valid request this build does not implement    */
    HYPIC_E_WORKSPACE = -3,    /* workspace missing or smaller than required     */
    HYPIC_E_HIP = -4,          /* a HIP runtime call or kernel launch failed     */
    HYPIC_E_DEVICE = -5,       /* current device is not a gfx950 GPU             */
    HYPIC_E_TOO_LARGE = -6     /* hypic_compose_noalloc: the request needs more
                                  scratch than HYPIC_NOALLOC_SCRATCH_BYTES        */
} hypic_status;

typedef enum { HYPIC_F32 = 0, HYPIC_BF16 = 1 } hypic_dtype;
typedef enum { HYPIC_RULE_DECAY = 0, HYPIC_RULE_DELTA = 1 } hypic_rule;
typedef enum {
    HYPIC_GATE_HEAD_CONST = 0, /* gate [h_v] fp32, one constant per value head   */
    HYPIC_GATE_SCALAR = 1,     /* gate [N, h_v], one scalar per token and head   */
    HYPIC_GATE_DIAG = 2        /* gate [N, h_v, d_k], one vector per token, head */
} hypic_gate;
typedef enum { HYPIC_T_SCALAR = 0, HYPIC_T_DIAG = 1, HYPIC_T_DENSE = 2 } hypic_tform;
typedef enum {
    HYPIC_PREC_FP32 = 0,       /* fp32 matrix products                           */
    HYPIC_PREC_SPLIT = 1       /* fp32 operands split into bf16 hi+lo, three
                                  products per term (relative error ~1e-5)       */
} hypic_prec;

/* Segments per kernel launch; longer tables are processed in several launches. */
#define HYPIC_MAX_SEG_PER_LAUNCH 128

/*
 * hypic_segment_build -- the cached pair of each segment (ch.2 secs.2 and 4).
 *
 * Token arrays hold N rows in token order; each pair covers the tokens
 * [seg_start[s], seg_start[s] + seg_len[s]) of those rows.  For an inner
 * segment the range is the body after the seam window; for the first segment
 * of a prompt it is the whole segment.
 *
 *   k      [N, h_k, d_k]  keys (raw conv inputs when conv_w > 0), in_dtype
 *   v      [N, h_v, d_v]  values (raw conv inputs when conv_w > 0), in_dtype
 *   beta   [N, h_v]       write strength in [0,1] (DELTA only, else NULL), in_dtype
 *   gate   per gate_kind, values in (0,1]; in_dtype, except HEAD_CONST: fp32
 *   GQA: value head h reads key head h / (h_v / h_k); h_v % h_k == 0.
 *
 *   conv_w     0: k, v are final.  2..4: k, v are raw rows of a depthwise causal
 *              conv of width conv_w (y_t = sum_j w[c][j] x_{t-conv_w+1+j}, no bias,
 *              no activation, weights conv_wk [h_k*d_k, conv_w] and
 *              conv_wv [h_v*d_v, conv_w] fp32).  Rows before conv_from[s] read
 *              as zero (a segment prefilled on its own).
 *   conv_from  HOST [n_seg] (conv_w > 0 only): first row the conv may read.
 *   k_l2norm   1: divide each key (after the conv) by its L2 norm.
 *
 *   T_out   [n_seg, h_v, 1 | d_k | d_k*d_k] fp32 by T form (scalar / diag / dense)
 *   S0_out  [n_seg, h_v, d_k, d_v] fp32
 *
 * Workspace: hypic_workspace_size(desc, HYPIC_WS_BUILD) bytes (0 without conv
 * or key normalisation; ws may then be NULL).  Empty ranges give T = I, S0 = 0.
 * Errors: HYPIC_E_INVALID (null pointers, negative lengths, h_v % h_k != 0),
 * HYPIC_E_UNSUPPORTED (dimensions, h_v * d_k >= 2^24, DECAY+DIAG with conv),
 * HYPIC_E_WORKSPACE, HYPIC_E_HIP.  DELTA+DIAG: a gate below 2^-126 is taken
 * as 2^-126.
 */
typedef struct {
    int32_t rule, gate_kind, in_dtype;
    int32_t n_seg;
    const int64_t *seg_start;  /* HOST [n_seg] */
    const int64_t *seg_len;    /* HOST [n_seg] */
    int32_t h_k, h_v, d_k, d_v;
    const void *k, *v, *beta, *gate;
    int32_t conv_w, k_l2norm;
    const int64_t *conv_from;  /* HOST [n_seg] or NULL when conv_w == 0 */
    const float *conv_wk, *conv_wv;
    float *T_out, *S0_out;
} hypic_build_desc;

hypic_status hypic_segment_build(const hypic_build_desc *d, void *ws, size_t ws_bytes,
                                 void *stream);

/*
 * Seam windows (ch.2 secs.5-6).  Window i holds the first w tokens of an inner
 * segment and the conv_w-1 raw rows that end the previous segment (its cached
 * tail conv state).  The delta rule only (rule DELTA): the gated delta rule
 * with one gate per token and head (gate_diag 0), or the delta rule with a
 * gate per key channel, KDA (gate_diag 1; ch.2 sec.3, Table 1:
 * T_t = (I - b_t k_t k_t^T) diag(g_t)).  Per-channel windows are applied token
 * by token in fp32 (in hypic_compose on the serial dense path) and have no
 * window pair (T_w, S_w0 must be NULL).
 *
 *   xk     [n_win, w, h_k, d_k]  raw (conv_w > 0) or final keys, in_dtype
 *   xv     [n_win, w, h_v, d_v]  raw or final values, in_dtype
 *   tail_k [n_win, conv_w-1, h_k, d_k], tail_v [n_win, conv_w-1, h_v, d_v]
 *          (conv_w > 1 only), in_dtype
 *   conv_wk [h_k*d_k, conv_w], conv_wv [h_v*d_v, conv_w] fp32 (conv_w > 0)
 *   beta   [n_win, w, h_v] in_dtype
 *   alpha  [n_win, w, h_v] (gate_diag 0) or [n_win, w, h_v, d_k] (gate_diag 1),
 *          in_dtype, values in (0, 1]
 *   q      optional [n_win, w, h_k, d_k] final queries (in_dtype);
 *   o      optional [n_win, w, h_v, d_v] fp32 read-outs o_t = q_t^T S_t with the
 *          post-update state (Eq. (2)); q and o are both set or both NULL.
 *   T_w    optional [n_win, h_v, d_k, d_k] fp32 window transition
 *   S_w0   optional [n_win, h_v, d_k, d_v] fp32 window zero-initial end state
 *   1 <= w <= 64.
 */
typedef struct {
    int32_t rule, in_dtype;
    int32_t w, conv_w, k_l2norm;
    int32_t h_k, h_v, d_k, d_v;
    int32_t n_win;
    const void *xk, *xv, *tail_k, *tail_v;
    const float *conv_wk, *conv_wv;
    const void *beta, *alpha;
    const void *q;
    float *o, *T_w, *S_w0;
    int32_t gate_diag;          /* 0: alpha per token and head; 1: per key channel (KDA) */
} hypic_seam_desc;

/*
 * hypic_seam_advance -- S_inout [h_v, d_k, d_v] fp32 advances over windows
 * 0..n_win-1 in order (normally n_win = 1).  Computes the window's transition
 * and zero-initial state and folds them into S (equal, up to rounding, to
 * running the w tokens one by one).  Errors: HYPIC_E_INVALID,
 * HYPIC_E_UNSUPPORTED (rule, dimensions, w > 64), HYPIC_E_HIP.
 */
hypic_status hypic_seam_advance(const hypic_seam_desc *d, float *S_inout, void *stream);

/*
 * hypic_rope_rerotate -- move cached full-attention keys to new positions
 * (ch.2 sec.6, Eq. (8): K_b = R(b - a) K_a).  Keys stored from a segment-local
 * start a are turned by R(delta) with delta = b - a, the segment's start in the
 * request: for every row t in [seg_start[s], seg_start[s] + seg_len[s]) and head
 *   x_out[t, head, :] = R(delta[s]) x_in[t, head, :].
 * R(delta) turns pair i of the leading rot_dim entries by delta * theta_i,
 * theta_i = base^(-2 i / rot_dim); pairing HYPIC_ROPE_HALF pairs entries
 * (i, i + rot_dim/2), HYPIC_ROPE_INTERLEAVED pairs (2i, 2i + 1).  Entries past
 * rot_dim are copied (x_out != x_in) or left as they are (in place).  The angle
 * is reduced modulo 2 pi in double precision; cos and sin are then rounded to
 * fp32 (relative error ~1e-7 per element; bf16 data is rounded once on output).
 *
 *   x_in, x_out [N, h, d], dtype HYPIC_F32 or HYPIC_BF16; x_out may equal x_in
 *   seg_start, seg_len, delta  HOST [n_seg]
 *   d in 8 .. 512, d % 8 == 0; rot_dim % 8 == 0, 8 <= rot_dim <= d; base > 0
 *
 * Rows of different segments must not overlap.  Errors: HYPIC_E_INVALID,
 * HYPIC_E_UNSUPPORTED (d, rot_dim), HYPIC_E_HIP.
 */
typedef enum { HYPIC_ROPE_HALF = 0, HYPIC_ROPE_INTERLEAVED = 1 } hypic_rope_pairing;

typedef struct {
    int32_t n_seg;
    const int64_t *seg_start;   /* HOST [n_seg] */
    const int64_t *seg_len;     /* HOST [n_seg] */
    const int64_t *delta;       /* HOST [n_seg]: new start minus cached start */
    int32_t h, d, rot_dim, pairing;
    int32_t dtype;              /* hypic_dtype of x_in and x_out */
    double base;
    const void *x_in;
    void *x_out;
} hypic_rope_desc;

hypic_status hypic_rope_rerotate(const hypic_rope_desc *d, void *stream);

/*
 * hypic_rope_rerotate_state -- the state of a scalar-transition layer whose
 * keys carry RoPE, moved from start a to b (ch.2 sec.6, Eq. (7)):
 *   S_out[head] = R(delta) S_in[head]   (R acting on the d_k rows)
 * with R(delta) as in hypic_rope_rerotate.  The identity holds for a scalar
 * transition (gamma I commutes with R); a diagonal gate does not commute with
 * R, and the identity does not hold there (the caller's responsibility).
 *
 *   S_in, S_out [h, d_k, d_v] fp32 (S_out may equal S_in); d_v % 4 == 0,
 *   rot_dim % 8 == 0, 8 <= rot_dim <= d_k, d_k <= 512
 *
 * Errors: HYPIC_E_INVALID, HYPIC_E_UNSUPPORTED, HYPIC_E_HIP.
 */
hypic_status hypic_rope_rerotate_state(int32_t h, int32_t d_k, int32_t d_v, int32_t rot_dim,
                                       int32_t pairing, double base, int64_t delta,
                                       const float *S_in, float *S_out, void *stream);

/*
 * hypic_compose -- fold cached pairs into a running state (Eq. (6)):
 *   S = S_init (or 0);  for i in 0..n-1:  [seam window i-1 if i >= 1]
 *                                         S <- T[order[i]] S + S0[order[i]]
 *
 *   T_pool   [n_slots, h_v, 1 | d_k | d_k*d_k] fp32 by tform
 *   S0_pool  [n_slots, h_v, d_k, d_v] fp32
 *   order    HOST [n]: pool slot of the i-th segment in prompt order
 *   S_init   [h_v, d_k, d_v] fp32, or NULL for the zero state
 *   S_out    [h_v, d_k, d_v] fp32; may equal S_init
 *   seams    NULL, or windows for positions 1..n-1 (seams->n_win == n-1,
 *            seams->w <= 16), dense tform only; seams->T_w/S_w0 must be NULL
 *            here.  seams->q and seams->o (both or neither) ask for the
 *            read-outs of every window token from the true prefix state it
 *            sees (ch.2 sec.5; Eq. (2): o_t = q_t^T S_t after token t),
 *            o [n-1, w, h_v, d_v] fp32, written for tokens t < w only.  On the
 *            split path they need w <= 8 (else HYPIC_E_UNSUPPORTED) and always
 *            take the group route (group_len 1: groups of one position).
 *   prec     HYPIC_PREC_FP32 or HYPIC_PREC_SPLIT for the dense product
 *   group_len  dense split compose with d_k in {64, 128} only (ignored
 *            otherwise): 1 folds the positions one after another; G >= 2
 *            folds every G consecutive positions (windows included) into one
 *            pair in parallel, then folds those pairs in order (composition is
 *            associative, ch.2 sec.2); 0 picks G from n and h_v.  The result
 *            is the same fold up to rounding.  Negative: HYPIC_E_INVALID.
 *
 * Workspace: hypic_workspace_size(desc, HYPIC_WS_COMPOSE) bytes, 16-byte
 * aligned.  It is 0 except for a dense split-precision compose with d_k in
 * {64, 128}:
 *   - with seams and n >= 2, the operators of all n-1 windows are computed
 *     first and staged there, (3 wp d_k + 4) floats per (window, value head)
 *     with wp = w rounded up to a multiple of 4 (rounded up to 256 bytes);
 *   - with groups, two pools of group pairs follow, [ng, h_v, d_k, d_v] fp32
 *     each, ng = ceil(min(n, HYPIC_MAX_SEG_PER_LAUNCH) / G);
 *   - with read-outs, the window records hold (5 wp d_k + 4) floats, and
 *     two more arrays follow: the read-out rows times the group-local prefix
 *     pair, [n-1, h_v, 8, 2 d_k] fp32 (rounded up to 256 bytes), and the
 *     state entering each group, [ng, h_v, d_k, d_v] fp32.
 * Errors: HYPIC_E_INVALID, HYPIC_E_UNSUPPORTED, HYPIC_E_WORKSPACE, HYPIC_E_HIP.
 */
typedef struct {
    int32_t tform, prec;
    int32_t h_v, d_k, d_v;
    int32_t n;
    int32_t n_slots;           /* slots in the pools; every order[i] < n_slots */
    const int32_t *order;      /* HOST [n] */
    const float *T_pool, *S0_pool;
    const float *S_init;
    float *S_out;
    const hypic_seam_desc *seams;
    int32_t group_len;         /* 0 automatic, 1 serial, G >= 2 groups of G positions */
} hypic_compose_desc;

hypic_status hypic_compose(const hypic_compose_desc *d, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * hypic_compose_noalloc -- hypic_compose for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same descriptor, same kernels and the same result
 * bit for bit as hypic_compose; the workspace is a static device array inside
 * the library instead of the caller's buffer, so the call allocates nothing.
 *
 *   - The array holds HYPIC_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the
 *     library runs on, from the first kernel launch on that GPU until the
 *     process ends.  A request whose hypic_workspace_size(d, HYPIC_WS_COMPOSE)
 *     exceeds it returns HYPIC_E_TOO_LARGE and launches nothing.  (For
 *     example, 100 positions with w = 8 seams at h_v = 32, d = 128 need 73 MB:
 *     split such a prompt into two calls, or use hypic_compose.)
 *   - Every call on one GPU uses that GPU's one array.  Calls that overlap on
 *     one GPU (two streams, or two host threads without ordering) race on it:
 *     the caller orders them.  Each call writes every scratch byte it reads
 *     before reading it, so nothing needs to start at zero and leftovers of an
 *     earlier call are harmless.
 * Errors: those of hypic_compose, with HYPIC_E_TOO_LARGE in place of
 * HYPIC_E_WORKSPACE.
 */
#define HYPIC_NOALLOC_SCRATCH_BYTES (64u << 20)
hypic_status hypic_compose_noalloc(const hypic_compose_desc *d, void *stream);

#define HYPIC_WS_BUILD 0
#define HYPIC_WS_COMPOSE 1
/* Workspace bytes a call with this descriptor needs (0 if none). */
size_t hypic_workspace_size(const void *desc, int which);

/* Static description of a status code. */
const char *hypic_status_string(hypic_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t hypic_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HYPIC_H */

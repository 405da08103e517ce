"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (relative Frobenius error per (segment, head) unit, on T_C and on
S): 1e-5 for fp32 inputs, 2e-3 for bf16 inputs with fp32 state.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, case, expand_T, head_relF, max_relF, need_gpu, np64

pytestmark = pytest.mark.gpu


def _lib():
    import state_caching_amd as sca
    from state_caching_amd.runner import DeviceWorkload
    return sca, DeviceWorkload


def _check_build(wl, segs=None, heads=None, tol=None, T=None, S0=None, label=""):
    """GPU pairs (all segments) against oracle pairs on the sampled units."""
    sca, DW = _lib()
    tol = TOL[wl.dtype] if tol is None else tol
    dw = DW(wl)
    case(f"build {wl.name} {label}")
    if T is None:
        T, S0 = dw.build()
        torch.cuda.synchronize()
    segs = list(range(wl.n_seg)) if segs is None else segs
    heads = list(range(wl.h_v)) if heads is None else heads
    Tr, Sr = oracle.build_pairs(wl, segs=segs, heads=heads)
    Tg = expand_T(np64(T), dw.tform, wl.d_k)[segs][:, heads]
    Sg = np64(S0)[segs][:, heads]
    eT = max_relF(Tg, Tr, 2)
    eS = max_relF(Sg, Sr, 2)
    print(f"  {wl.name}: max relF T {eT:.3e}  S {eS:.3e}", flush=True)
    assert eS <= tol, (eS, tol)
    assert eT <= tol, (eT, tol)
    return dw, T, S0


# ----------------------------------------------------------- reference configs

def test_gdn_d16_fp32_build_compose():
    need_gpu()
    wl = synth.workload("gdn_d16_2x64_fp32")
    dw, T, S0 = _check_build(wl)
    case("compose gdn d16 fp32")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    Tr, Sr = oracle.build_pairs(wl)
    S_or = oracle.compose(Tr, Sr)
    full = oracle.full_recompute(wl)
    e = head_relF(np64(S), S_or)
    print(f"  compose relF {e:.3e}; oracle compose vs full {oracle.relF(S_or, full):.1e}")
    assert e <= 1e-5
    assert head_relF(np64(S), full) <= 1e-5


def test_retnet_fp32_build_compose_naive():
    need_gpu()
    wl = synth.workload("retnet_d64_8h_4x256_fp32")
    dw, T, S0 = _check_build(wl)
    case("compose retnet (scalar T)")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    Tr, Sr = oracle.build_pairs(wl)
    S_or = oracle.compose(Tr, Sr)
    assert head_relF(np64(S), S_or) <= 1e-5
    naive = oracle.naive_sum(np64(S0))
    err = oracle.relF(naive, S_or)
    print(f"  naive-sum error vs composed state: {err:.4f}")
    # head 5 (gamma = 1 - 2^-10): Table 2's ratio at 256 tokens from the GPU pairs
    S1 = np64(S0)[0, 5]
    two = np64(T)[1, 5] * S1 + np64(S0)[1, 5]
    r = np.linalg.norm(two - (S1 + np64(S0)[1, 5])) / np.linalg.norm(S1)
    assert round(r, 3) == 0.221


def test_gla_bf16_build():
    need_gpu()
    wl = synth.workload("gla_d128_16h_8x512_bf16")
    dw, T, S0 = _check_build(wl)
    case("compose gla (diag T)")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    Tr, Sr = oracle.build_pairs(wl)
    assert head_relF(np64(S), oracle.compose(Tr, Sr)) <= 2e-3


def test_gla_slow_build():
    need_gpu()
    _check_build(synth.workload("gla_d128_16h_8x512_bf16_slow"), segs=[0, 5], heads=[0, 7, 15])


def test_gdn_gqa_32k_prompt_sampled():
    need_gpu()
    wl = synth.workload("gdn_gqa_d128_8x4096_bf16")
    dw, T, S0 = _check_build(wl, segs=[0, 7], heads=[0, 1, 31], label="(sampled units)")
    case("compose gdn gqa 32k prompt")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    heads = [3]
    Tr, Sr = oracle.build_pairs(wl, heads=heads)
    S_or = oracle.compose(Tr, Sr)
    e = head_relF(np64(S)[heads], S_or)
    print(f"  compose relF (head 3) {e:.3e}")
    assert e <= 2e-3


def test_gdn_gqa_slow_sampled():
    need_gpu()
    _check_build(synth.workload("gdn_gqa_d128_8x4096_bf16_slow"), segs=[2], heads=[4, 5], label="(sampled units)")


# ------------------------------------------------------------- shape coverage

@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_delta_shapes_ragged(d, dtype):
    need_gpu()
    wl = synth.gdn(20 + d, [0, 1, 63, 65, 130, 200], 2, 4, d, dtype, alpha_div=32.0)
    _check_build(wl, label=f"d={d}")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["retnet", "gla", "gla_slow"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decay_shapes_ragged(d, kind, dtype):
    need_gpu()
    lens = [0, 1, 63, 65, 130, 257]
    if kind == "retnet":
        wl = synth.retnet(30 + d, lens, 3, d, dtype=dtype)
    else:
        wl = synth.gla(40 + d, lens, 3, d, dtype=dtype, literal=(kind == "gla"))
    _check_build(wl, label=f"d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_mamba2_scalar_gate(d):
    """Per-token scalar gate with the decay rule (Mamba2 form)."""
    need_gpu()
    import dataclasses
    base = synth.gdn(50, [100, 77], 2, 2, d, torch.bfloat16, alpha_div=8.0)
    wl = dataclasses.replace(base, rule="decay", beta=None, name="mamba2-like")
    _check_build(wl)


def test_deltanet_no_decay():
    """DeltaNet: gate 1 everywhere; T_C is the pure product of the rank-one erases."""
    need_gpu()
    import dataclasses
    base = synth.gdn(51, [300, 129], 2, 2, 64, torch.bfloat16)
    wl = dataclasses.replace(base, gate=torch.ones_like(base.gate), name="deltanet")
    _check_build(wl)


# ------------------------------------------- builds over more than one launch

def _multi_launch_lens(n, seed):
    """Ragged segment lengths (30..61 tokens) for builds of n > 128 segments, so
    that a wrong row offset in a later launch reads another segment's rows."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(30, 62, size=n)]


@pytest.mark.parametrize("kind,d,dtype,conv", [
    ("delta", 64, torch.bfloat16, 0), ("delta", 64, torch.bfloat16, 4),
    ("delta", 128, torch.bfloat16, 4), ("delta", 32, torch.float32, 4),
    ("retnet", 32, torch.float32, 0), ("gla", 64, torch.bfloat16, 0)],
    ids=["gdn-bf16-d64", "gdn-bf16-d64-conv", "gdn-bf16-d128-conv", "gdn-f32-d32-conv",
         "retnet-f32-d32", "gla-bf16-d64"])
def test_build_multi_launch(kind, d, dtype, conv):
    """A build of 150 segments runs as two launches (128 + 22).  The pairs of
    the first and last segments of each launch, and of segments inside both,
    are compared with the oracle's own pairs: a wrong segment table, output
    offset or packed conv-workspace offset in the second launch fails here.
    With conv, inner segments have seam windows, so every body starts after its
    conv history (rows the second launch must read from the right place)."""
    need_gpu()
    n = 150
    lens = _multi_launch_lens(n, 600 + d + conv)
    if kind == "delta":
        wl = synth.gdn(601 + d + conv, lens, 1, 2, d, dtype, alpha_div=16.0, conv_w=conv,
                       seam_w=8 if conv else 0, name=f"gdn-150seg-d{d}-conv{conv}")
    elif kind == "retnet":
        wl = synth.retnet(602 + d, lens, 2, d, dtype=dtype, name="retnet-150seg")
    else:
        wl = synth.gla(603 + d, lens, 2, d, dtype=dtype, literal=False, name="gla-150seg")
    _check_build(wl, segs=[0, 1, 77, 126, 127, 128, 129, 148, 149], label="(two launches)")


# ------------------------------------------------------ long segments, key scale

def test_gdn_slow_16k_segment():
    """One 16384-token segment per head (bf16, d = 128, slow decay as the 32k
    prompt's slow companion, so the gate-free transition product decays only by
    the erases): T_C and S0 against the oracle at the bf16 contract bound.  The
    fp16 operands' rounding would add up over 256 chunks past the bound (3.3e-3
    on T_C); segments longer than 4096 tokens take the fp32-operand build."""
    need_gpu()
    wl = synth.gdn(610, [16384], 1, 2, 128, torch.bfloat16, alpha_div=4096.0, name="gdn-slow-16k")
    _check_build(wl, label="(16384-token segment)")


@pytest.mark.parametrize("conv", [0, 4])
def test_gdn_mixed_segment_lengths(conv):
    """A build whose segments alternate between the fp16-operand class (up to
    4096 tokens) and the fp32-operand class (longer), with and without conv:
    each run of one class is its own launch, with its own conv workspace
    layout.  Every pair against the oracle; the long ones at the fp32 path's
    precision."""
    need_gpu()
    lens = [4096, 4105, 300, 5008, 64, 4108]   # bodies (after 8-token windows) 4096, 4097, ...: both classes
    wl = synth.gdn(611 + conv, lens, 1, 2, 128, torch.bfloat16, alpha_div=512.0, conv_w=conv,
                   seam_w=8 if conv else 0, name=f"gdn-mixed-lengths-conv{conv}")
    dw, T, S0 = _check_build(wl, label="(mixed operand classes)")
    long_segs = [j for j, (s, e) in enumerate(wl.body_ranges()) if e - s > 4096]
    Tr, Sr = oracle.build_pairs(wl, segs=long_segs)
    eT = max_relF(expand_T(np64(T), dw.tform, 128)[long_segs], Tr, 2)
    eS = max_relF(np64(S0)[long_segs], Sr, 2)
    print(f"  segments over 4096 tokens: max relF T {eT:.3e}  S {eS:.3e}")
    assert eT <= 2e-5 and eS <= 2e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("log2r", [-4, 0, 4])
def test_delta_key_scale(d, log2r):
    """Keys of norm r = 2^log2r with write strengths beta / r^2 (bf16 inputs,
    fp16 matrix-core operands): every transition I - beta' k' k'^T equals the
    one of the unit-norm keys, and the writes scale by 1/r.  Against the oracle
    at the contract bound, for keys far from unit norm in both directions."""
    need_gpu()
    import dataclasses
    base = synth.gdn(620 + d, [200, 130, 64], 1, 2, d, torch.bfloat16, alpha_div=32.0)
    r = 2.0 ** log2r
    wl = dataclasses.replace(base, k=(base.k.float() * r).to(torch.bfloat16),
                             beta=(base.beta.float() / (r * r)).to(torch.bfloat16),
                             name=f"gdn-keys-2^{log2r}")
    _check_build(wl, label=f"key norm 2^{log2r}")


def test_delta_value_scale_jumps():
    """Values whose scale jumps between 64-token chunks by exact powers of two
    (bf16, d = 128): up 2^12 (the state's unit follows the values), down 2^20,
    up 2^70 (far past the unit), and a segment whose first chunk is at 2^80.
    Every change of the state's unit is an exact power-of-two rescaling, so
    T_C and S0 stay within the contract bound of the oracle."""
    need_gpu()
    import dataclasses
    base = synth.gdn(630, [1024, 300, 200], 1, 2, 128, torch.bfloat16, alpha_div=32.0)
    ex = np.zeros(sum(base.seg_len))
    for c, e in enumerate([0, 0, 12, 12, -8, -8, 62, 62, 62, 70, 70, 70, 70, 70, 70, 70]):
        ex[64 * c:64 * (c + 1)] = e
    ex[1024:1088] = 80
    ex[1324:1524] = 20
    f = torch.tensor(np.exp2(ex), dtype=torch.float32)[:, None, None]
    wl = dataclasses.replace(base, v=(base.v.float() * f).to(torch.bfloat16), name="gdn-value-jumps")
    _check_build(wl, label="value scale jumps")


# ---------------------------------------------------------------- compose only

@pytest.mark.parametrize("tform,prec", [("dense", 0), ("dense", 1), ("diag", 0), ("scalar", 0)])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_compose_prebuilt_pairs(tform, prec, d):
    need_gpu()
    sca, _ = _lib()
    T, S0 = synth.random_pairs(60 + d, 9, 3, d, d, tform=tform)
    S_init = synth.random_state(61, 3, d, d)
    order = [4, 0, 8, 2, 2, 7, 1]
    tf = {"scalar": 0, "diag": 1, "dense": 2}[tform]
    case(f"compose prebuilt {tform} prec={prec} d={d}")
    S = sca.compose(T.cuda(), S0.cuda(), order, S_init=S_init.cuda(), tform=tf, prec=prec)
    torch.cuda.synchronize()
    Td = expand_T(np64(T), tf, d)
    ref = oracle.compose(Td[order], np64(S0)[order], np64(S_init))
    e = head_relF(np64(S), ref)
    print(f"  relF {e:.3e}")
    assert e <= 1e-5   # fp32 pairs: the fp32 contract bound, per head, for both product forms


def test_compose_in_place_and_long_chain():
    """S_out aliasing S_init, and more segments than one launch holds."""
    need_gpu()
    sca, _ = _lib()
    d = 64
    T, S0 = synth.random_pairs(70, 5, 2, d, d, tform="dense", rho=0.95)
    order = [i % 5 for i in range(300)]
    S = synth.random_state(71, 2, d, d).cuda()
    S_ref_init = np64(S)
    case("compose in place, 300 segments")
    sca.compose(T.cuda(), S0.cuda(), order, S_init=S, S_out=S, tform=2, prec=0)
    torch.cuda.synchronize()
    ref = oracle.compose(np64(T)[order], np64(S0)[order], S_ref_init)
    assert head_relF(np64(S), ref) <= 1e-5


def test_compose_empty():
    need_gpu()
    sca, _ = _lib()
    T, S0 = synth.random_pairs(72, 2, 2, 32, 32)
    S_init = synth.random_state(73, 2, 32, 32).cuda()
    S = sca.compose(T.cuda(), S0.cuda(), [], S_init=S_init)
    assert torch.equal(S, S_init)
    S = sca.compose(T.cuda(), S0.cuda(), [])
    assert float(S.abs().max()) == 0.0


# ------------------------------------------------------------------- seams

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_seam_standalone_outputs(dtype):
    need_gpu()
    sca, DW = _lib()
    d, h = 64, 2
    wl = synth.gdn(80, [40, 30], 1, h, d, dtype, alpha_div=16.0, conv_w=4, seam_w=8)
    dw = DW(wl)
    rng = np.random.default_rng(81)
    S_init = synth.random_state(82, h, d, d)
    q = synth._round(rng.standard_normal((1, 8, 1, d)) / np.sqrt(d), dtype)
    sm = dw.seams
    sm.q = q.cuda()
    sm.o = torch.zeros((1, 8, h, d), dtype=torch.float32, device="cuda")
    sm.T_w = torch.zeros((1, h, d, d), dtype=torch.float32, device="cuda")
    sm.S_w0 = torch.zeros((1, h, d, d), dtype=torch.float32, device="cuda")
    S = S_init.clone().cuda()
    case(f"seam standalone {dtype}")
    sca.seam_advance(S, sm)
    torch.cuda.synchronize()
    s, e = wl.window_ranges()[0]
    sl = oracle.Slice(wl, s, e)
    u = sl.units()
    S_ref = np64(S_init).copy()
    o_ref = np.zeros((8, h, d))
    qa = np64(q)[0]
    oracle.recur_units(wl.rule, sl.gate_kind, u, d, d, sl.k, sl.v, sl.beta, sl.g, S_ref,
                       q=np.ascontiguousarray(qa), o=o_ref, off_q=u.off_k, ldq=u.ldk,
                       off_o=u.off_v, ldo=u.ldv)
    Tw, Sw = oracle.build_units(wl.rule, sl.gate_kind, u, d, d, sl.k, sl.v, sl.beta, sl.g)
    tol = 1e-5   # the window runs in fp32 arithmetic for every input dtype
    errs = (head_relF(np64(S), S_ref), oracle.relF(np64(sm.o)[0], o_ref),
            max_relF(np64(sm.T_w)[0], Tw, 1), max_relF(np64(sm.S_w0)[0], Sw, 1))
    print("  seam relF S %.2e o %.2e T_w %.2e S_w0 %.2e" % errs)
    assert max(errs) <= tol


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_seam_pipeline_small(dtype):
    """Conv + seams, small: pairs built from raw rows, composed with seams, against
    the oracle's composition and against full recompute."""
    need_gpu()
    wl = synth.gdn(90, [70, 64, 100, 65, 90], 2, 2, 32, dtype, alpha_div=64.0, conv_w=4,
                   seam_w=8)
    dw, T, S0 = _check_build(wl)
    case(f"compose with seams {dtype}")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    Tr, Sr = oracle.build_pairs(wl)
    S_or = oracle.compose(Tr, Sr, wl=wl, seams=True)
    full = oracle.full_recompute(wl)
    e1, e2 = head_relF(np64(S), S_or), head_relF(np64(S), full)
    print(f"  compose relF vs oracle {e1:.3e}, vs full recompute {e2:.3e}")
    assert e1 <= TOL[dtype] and e2 <= TOL[dtype]


@pytest.mark.parametrize("d", [64, 128])
def test_split_compose_with_seams(d):
    """The split-precision compose with fused seam windows (d in {64, 128}) on
    non-degenerate gates: against the oracle's composition of the same GPU-built
    pairs (isolates the compose and window arithmetic), and against full
    recompute of the prompt."""
    need_gpu()
    wl = synth.gdn(95 + d, [70, 64, 100, 65, 90, 33, 80], 1, 2, d, torch.bfloat16,
                   alpha_div=64.0, conv_w=4, seam_w=8)
    dw, T, S0 = _check_build(wl)
    S_init = synth.random_state(96 + d, 2, d, d)
    case(f"split compose with seams d={d}")
    S = dw.compose(T, S0, S_init=S_init.cuda())
    torch.cuda.synchronize()
    S_or = oracle.compose(np64(T), np64(S0), S_init=np64(S_init), wl=wl, seams=True)
    full = oracle.full_recompute(wl, S_init=np64(S_init))
    e1, e2 = head_relF(np64(S), S_or), head_relF(np64(S), full)
    print(f"  relF vs oracle compose of the same pairs {e1:.3e}, vs full recompute {e2:.3e}")
    assert e1 <= 2e-5 and e2 <= TOL[torch.bfloat16]


def test_split_compose_seams_across_launches():
    """More segments than one compose launch holds, with seams: windows are
    indexed by prompt position across launches."""
    need_gpu()
    wl = synth.gdn(97, [12] * 150, 1, 1, 64, torch.bfloat16, alpha_div=16.0, conv_w=4,
                   seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    case("split compose with seams, 150 segments")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    S_or = oracle.compose(np64(T), np64(S0), wl=wl, seams=True)
    e = head_relF(np64(S), S_or)
    print(f"  relF vs oracle compose of the same pairs {e:.3e}")
    assert e <= 2e-5


@pytest.mark.parametrize("d,G", [(64, 2), (64, 5), (128, 3), (128, 7)])
def test_group_compose_with_seams(d, G):
    """The two-level compose (groups of G consecutive positions folded in
    parallel, then the group pairs in order) with seams and a random prefix
    state, ragged last group: against the oracle's sequential composition of
    the same pairs, against the serial GPU fold, and against full recompute."""
    need_gpu()
    lens = [40, 64, 33, 70, 21, 64, 50, 90, 17, 64, 45, 80, 66, 29, 55, 64, 38]
    wl = synth.gdn(110 + d + G, lens, 1, 2, d, torch.bfloat16, alpha_div=64.0, conv_w=4,
                   seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    S_init = synth.random_state(111 + d, 2, d, d)
    case(f"group compose with seams d={d} G={G} n={len(lens)}")
    S = dw.compose(T, S0, S_init=S_init.cuda(), group_len=G)
    S_ser = dw.compose(T, S0, S_init=S_init.cuda(), group_len=1)
    torch.cuda.synchronize()
    S_or = oracle.compose(np64(T), np64(S0), S_init=np64(S_init), wl=wl, seams=True)
    full = oracle.full_recompute(wl, S_init=np64(S_init))
    e1, e2, e3 = (head_relF(np64(S), S_or), head_relF(np64(S), np64(S_ser)),
                  head_relF(np64(S), full))
    print(f"  relF vs oracle compose {e1:.3e}, vs serial GPU fold {e2:.3e}, vs full recompute {e3:.3e}")
    assert e1 <= 2e-5 and e2 <= 2e-5 and e3 <= TOL[torch.bfloat16]


@pytest.mark.parametrize("d", [64, 128])
def test_group_compose_no_seams(d):
    """The two-level compose without seams (automatic and fixed group lengths,
    and a group length beyond n), dense random pairs: against the oracle."""
    need_gpu()
    sca, _ = _lib()
    n, h = 37, 3
    T, S0 = synth.random_pairs(120 + d, n, h, d, d, tform="dense", rho=0.95)
    S_init = synth.random_state(121 + d, h, d, d)
    order = list(np.random.default_rng(122 + d).permutation(n))
    ref = oracle.compose(np64(T)[order], np64(S0)[order], np64(S_init))
    for G in (0, 4, 9, 64):
        case(f"group compose no seams d={d} G={G}")
        S = sca.compose(T.cuda(), S0.cuda(), order, S_init=S_init.cuda(), group_len=G)
        torch.cuda.synchronize()
        e = head_relF(np64(S), ref)
        print(f"  G={G}: relF vs oracle {e:.3e}")
        assert e <= 2e-5


def test_group_compose_seams_across_launches():
    """The two-level compose over more positions than one launch holds, with
    seams: group pairs per launch, windows by prompt position, the running
    state carried between launches."""
    need_gpu()
    wl = synth.gdn(131, [12] * 150, 1, 1, 64, torch.bfloat16, alpha_div=16.0, conv_w=4,
                   seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    case("group compose with seams, 150 segments, G=6")
    S = dw.compose(T, S0, group_len=6)
    torch.cuda.synchronize()
    S_or = oracle.compose(np64(T), np64(S0), wl=wl, seams=True)
    e = head_relF(np64(S), S_or)
    print(f"  relF vs oracle compose of the same pairs {e:.3e}")
    assert e <= 2e-5


def test_gdn_100_segments_seams_slow_group_compose():
    """The 100-segment prompt with slow decay (alpha = exp(-softplus(z)/1024), so
    T_C stays far from 0 and every group pair carries the earlier positions):
    the automatic two-level compose, in the bench's launch configuration, against
    the oracle's sequential composition of the same GPU-built pairs with the same
    windows, on sampled heads; and against the serial GPU fold on all heads."""
    need_gpu()
    wl = synth.workload("gdn_d128_32h_100x1024_seams_bf16_slow")
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    case("100-segment slow-decay compose, two-level (automatic) and serial")
    S = dw.compose(T, S0)
    S_ser = dw.compose(T, S0, group_len=1)
    torch.cuda.synchronize()
    heads = [3, 30]
    Tn, Sn = np64(T)[:, heads], np64(S0)[:, heads]
    S_or = oracle.compose(Tn, Sn, wl=wl, heads=heads, seams=True)
    e1 = head_relF(np64(S)[heads], S_or)
    e2 = head_relF(np64(S), np64(S_ser))
    tn = float(np.linalg.norm(np64(T)[-1, heads[0]]))
    print(f"  ||T_C|| (last segment, head {heads[0]}) {tn:.3e}; relF vs oracle compose {e1:.3e}, "
          f"vs serial GPU fold {e2:.3e}")
    assert tn > 1e-3
    assert e1 <= 2e-5 and e2 <= 2e-5


# ------------------------------------------------ window read-outs in the compose

def _attach_queries(dw, seed):
    """Seeded final queries for every seam window (the workload's dtype) and a
    zeroed fp32 read-out buffer, on the device seams; returns q as fp64."""
    wl = dw.wl
    n_win, w = len(wl.window_ranges()), wl.seam_w
    rng = np.random.default_rng(seed)
    q = synth._round(rng.standard_normal((n_win, w, wl.h_k, wl.d_k)) / np.sqrt(wl.d_k), wl.dtype)
    dw.seams.q = q.cuda()
    dw.seams.o = torch.full((n_win, w, wl.h_v, wl.d_v), float("nan"), dtype=torch.float32,
                            device="cuda")
    return np64(q)


def _readout_errs(o_gpu, o_ref):
    """Largest relF of one head's read-outs over all windows, and the largest
    relF of one (window, head) unit (o is [n_win, w, h, d_v])."""
    heads = range(o_ref.shape[2])
    per_head = max(oracle.relF(o_gpu[:, :, h], o_ref[:, :, h]) for h in heads)
    per = max(oracle.relF(o_gpu[j, :, h], o_ref[j, :, h])
              for j in range(o_ref.shape[0]) for h in heads)
    return per_head, per


@pytest.mark.parametrize("d,G", [(64, 1), (64, 2), (64, 5), (128, 0), (128, 1), (128, 3), (128, 7),
                                 (128, 64)])
def test_group_compose_readouts(d, G):
    """Window read-outs o_t = q_t^T S_t inside the two-level compose (ch.2 sec.5:
    the recomputed window tokens produce their outputs from the true prefix
    state), ragged segments, a random prefix state: o and the final state against
    the oracle's composition of the same pairs with the same windows."""
    need_gpu()
    lens = [40, 64, 33, 70, 21, 64, 50, 90, 17, 64, 45, 80, 66, 29, 55, 64, 38]
    wl = synth.gdn(140 + d + G, lens, 1, 2, d, torch.bfloat16, alpha_div=64.0, conv_w=4,
                   seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    S_init = synth.random_state(141 + d, 2, d, d)
    q = _attach_queries(dw, 142 + d + G)
    case(f"group compose with read-outs d={d} G={G} n={len(lens)}")
    S = dw.compose(T, S0, S_init=S_init.cuda(), group_len=G)
    torch.cuda.synchronize()
    S_or, o_or = oracle.compose(np64(T), np64(S0), S_init=np64(S_init), wl=wl, seams=True, q=q)
    eS = head_relF(np64(S), S_or)
    eo, eo_win = _readout_errs(np64(dw.seams.o), o_or)
    print(f"  relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
    assert eS <= 2e-5 and eo <= 2e-5 and eo_win <= 1e-4


@pytest.mark.parametrize("n", [2, 5])
def test_compose_readouts_short_chain(n):
    """Read-outs on a chain shorter than the automatic grouping threshold (one
    group holds every position) and with windows narrower than 8 rows."""
    need_gpu()
    wl = synth.gdn(160 + n, [30 + 7 * i for i in range(n)], 2, 4, 64, torch.bfloat16, alpha_div=32.0,
                   conv_w=4, seam_w=5)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    q = _attach_queries(dw, 161 + n)
    case(f"compose with read-outs, short chain n={n}, w=5")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    S_or, o_or = oracle.compose(np64(T), np64(S0), wl=wl, seams=True, q=q)
    eS = head_relF(np64(S), S_or)
    eo, eo_win = _readout_errs(np64(dw.seams.o), o_or)
    print(f"  relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
    assert eS <= 2e-5 and eo <= 2e-5 and eo_win <= 1e-4


@pytest.mark.parametrize("d", [16, 32])
def test_compose_readouts_small_heads(d):
    """Read-outs with bf16 inputs at d = 16 and 32 (the dense compose kernel,
    whose window code reads out itself), against the oracle."""
    need_gpu()
    wl = synth.gdn(170 + d, [40, 64, 33, 70], 1, 2, d, torch.bfloat16, alpha_div=32.0, conv_w=4,
                   seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    q = _attach_queries(dw, 171 + d)
    case(f"compose with read-outs, d={d}, bf16")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    S_or, o_or = oracle.compose(np64(T), np64(S0), wl=wl, seams=True, q=q)
    eS = head_relF(np64(S), S_or)
    eo, eo_win = _readout_errs(np64(dw.seams.o), o_or)
    print(f"  relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
    assert eS <= 2e-5 and eo <= 2e-5 and eo_win <= 1e-4


def test_compose_readouts_fp32_path():
    """Read-outs on the fp32 compose path (fp32 inputs, windows in fp32
    arithmetic), a window wider than 8 rows: against the oracle."""
    need_gpu()
    wl = synth.gdn(150, [40, 64, 33, 70, 21], 2, 2, 64, torch.float32, alpha_div=16.0, conv_w=4,
                   seam_w=12)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    q = _attach_queries(dw, 151)
    case("compose with read-outs, fp32 path, w=12")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    S_or, o_or = oracle.compose(np64(T), np64(S0), wl=wl, seams=True, q=q)
    eS = head_relF(np64(S), S_or)
    eo, eo_win = _readout_errs(np64(dw.seams.o), o_or)
    print(f"  relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
    assert eS <= 1e-5 and eo <= 1e-5 and eo_win <= 1e-4


def test_compose_readouts_twice():
    """Two read-out composes in a row with different queries and one workspace
    (the records, Y and the group-start states are rewritten by the second call):
    each against the oracle."""
    need_gpu()
    import state_caching_amd as sca_mod
    lens = [40, 64, 33, 70, 21, 64, 50, 90, 17, 64, 45, 80, 66, 29, 55, 64, 38, 70]
    wl = synth.gdn(180, lens, 1, 2, 128, torch.bfloat16, alpha_div=64.0, conv_w=4, seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    order = list(range(wl.n_seg))
    for call, seed in enumerate((181, 182)):
        q = _attach_queries(dw, seed)
        case(f"compose with read-outs, call {call} of two, one workspace")
        S = sca_mod.compose(T, S0, order, tform=dw.tform, prec=dw.prec, seams=dw.seams, workspace=ws)
        torch.cuda.synchronize()
        S_or, o_or = oracle.compose(np64(T), np64(S0), wl=wl, seams=True, q=q)
        eS = head_relF(np64(S), S_or)
        eo, eo_win = _readout_errs(np64(dw.seams.o), o_or)
        print(f"  call {call}: relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
        assert eS <= 2e-5 and eo <= 2e-5 and eo_win <= 1e-4


def test_group_compose_readouts_across_launches():
    """Read-outs over more positions than one launch holds: windows indexed by
    prompt position, group-start states per launch."""
    need_gpu()
    wl = synth.gdn(152, [12] * 150, 1, 1, 64, torch.bfloat16, alpha_div=16.0, conv_w=4,
                   seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    q = _attach_queries(dw, 153)
    case("group compose with read-outs, 150 segments, G=6")
    S = dw.compose(T, S0, group_len=6)
    torch.cuda.synchronize()
    S_or, o_or = oracle.compose(np64(T), np64(S0), wl=wl, seams=True, q=q)
    eS = head_relF(np64(S), S_or)
    eo, eo_win = _readout_errs(np64(dw.seams.o), o_or)
    print(f"  relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
    assert eS <= 2e-5 and eo <= 2e-5 and eo_win <= 1e-4


def test_gdn_100_segments_readouts_slow():
    """The 100-segment slow-decay prompt with read-outs at all 99 windows, in the
    bench's launch configuration (automatic groups): o on sampled heads against
    the oracle's composition of the same GPU-built pairs, and the final state
    against the compose without read-outs."""
    need_gpu()
    wl = synth.workload("gdn_d128_32h_100x1024_seams_bf16_slow")
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    S_plain = dw.compose(T, S0)
    q = _attach_queries(dw, 154)
    case("100-segment slow-decay compose with read-outs")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    heads = [3, 30]
    _, o_or = oracle.compose(np64(T)[:, heads], np64(S0)[:, heads], wl=wl, heads=heads,
                             seams=True, q=q)
    eo, eo_win = _readout_errs(np64(dw.seams.o)[:, :, heads], o_or)
    eS = head_relF(np64(S), np64(S_plain))
    print(f"  relF o (heads {heads}) {eo:.3e} (worst window {eo_win:.3e}); S vs compose without "
          f"read-outs {eS:.3e}")
    assert eo <= 2e-5 and eo_win <= 1e-4 and eS <= 1e-6


# --------------------------------------------- delta rule with a diagonal gate (KDA)

@pytest.mark.parametrize("d,dtype", [(16, torch.float32), (32, torch.bfloat16), (64, torch.float32),
                                     (64, torch.bfloat16), (128, torch.float32), (128, torch.bfloat16)])
def test_kda_build_compose(d, dtype):
    """KDA pairs (T dense) on ragged and empty segments with GQA, against the
    oracle's two-run pairs; their composition from a random state against full
    recompute of the prompt."""
    need_gpu()
    lens = [0, 1, 63, 65, 130, 200]
    wl = synth.kda(400 + d, lens, 2, 4, d, dtype, gate_div=32.0, name=f"kda-d{d}")
    # bf16 inputs at d >= 64 take fp16 state products: the contract's bf16 bound;
    # below that the fp32-product kernel holds its own much tighter figure
    tol = 1e-5 if dtype == torch.float32 else (TOL[dtype] if d >= 64 else 2e-5)
    dw, T, S0 = _check_build(wl, tol=tol)
    S_init = synth.random_state(401 + d, 4, d, d)
    case(f"compose kda d={d}")
    S = dw.compose(T, S0, S_init=S_init.cuda())
    torch.cuda.synchronize()
    full = oracle.full_recompute(wl, S_init=np64(S_init))
    e = head_relF(np64(S), full)
    print(f"  compose relF vs full recompute {e:.3e}")
    assert e <= TOL[dtype]


def test_kda_build_fast_gates():
    """KDA with the unscaled gate draw (g = exp(-softplus(N(0,1))), strong
    per-channel decay): the chunk's tile references keep every decay factor in
    range; T_C decays towards 0 and S0 rests on the last tokens."""
    need_gpu()
    wl = synth.kda(410, [64, 100, 300], 1, 2, 64, torch.float32, gate_div=1.0, name="kda-fast")
    _check_build(wl, tol=1e-5)


def test_kda_build_conv():
    """KDA with a width-4 causal conv and key L2 normalisation before the build."""
    need_gpu()
    wl = synth.kda(420, [70, 64, 129], 2, 2, 64, torch.bfloat16, gate_div=16.0, conv_w=4,
                   name="kda-conv")
    _check_build(wl, tol=2e-5)


def test_kda_sampled_4096():
    """KDA at a long segment length (2 x 4096 tokens, 32 value / 16 key heads,
    d = 128, bf16), sampled (segment, head) units."""
    need_gpu()
    wl = synth.kda(430, [4096, 4096], 16, 32, 128, torch.bfloat16, gate_div=256.0,
                   name="kda-gqa-2x4096")
    _check_build(wl, segs=[1], heads=[0, 31], label="(sampled units)")


def test_kda_32k_prompt_sampled():
    """The bench's KDA workload in its launch configuration (8 x 4096 tokens, 32
    value / 16 key heads, d = 128, bf16; all 256 units built in one launch), the
    first and last segments of two heads against the oracle.  Its gates are
    fast, so T_C underflows to zero on both sides after 4096 tokens; the slower
    gates of test_kda_sampled_4096 keep a non-trivial T_C at this length."""
    need_gpu()
    wl = synth.workload("kda_gqa_d128_8x4096_bf16")
    _check_build(wl, segs=[0, 7], heads=[0, 31], label="(sampled units)")


# ------------------------------------------------------------- rotary re-rotation

@pytest.mark.parametrize("dtype,pairing,rot,inplace", [
    (torch.float32, 0, 128, False), (torch.float32, 1, 128, True), (torch.bfloat16, 0, 128, True),
    (torch.bfloat16, 1, 64, False), (torch.float32, 0, 96, False), (torch.bfloat16, 0, 8, True)])
def test_rope_keys(dtype, pairing, rot, inplace):
    """Cached keys moved to new positions (Eq. (8)) against the oracle: several
    segments with their own shifts (negative, zero, 1e5), an empty one, partial
    rotary width, both pairings, in place and out of place."""
    need_gpu()
    import state_caching_amd as sca
    rng = np.random.default_rng(500 + rot + pairing)
    h, d = 3, 128
    starts, lens, deltas = [0, 37, 37, 300], [37, 0, 263, 129], [4096, 11, -250, 100000]
    x64 = rng.standard_normal((429, h, d))
    x = torch.from_numpy(x64).to(torch.float32).to(dtype)
    xin = x.cuda()
    out = None if inplace else torch.empty_like(xin)
    case(f"rope keys {dtype} pairing={pairing} rot={rot} inplace={inplace}")
    y = sca.rope_rerotate(xin, starts, lens, deltas, rot_dim=rot, pairing=pairing, out=out)
    torch.cuda.synchronize()
    xr = np64(x)
    ref = xr.copy()
    for s0, n, dl in zip(starts, lens, deltas):
        ref[s0:s0 + n] = oracle.rope_rotate(xr[s0:s0 + n], float(dl), rot_dim=rot, pairing=pairing)
    got = np64(y)
    if dtype == torch.float32:
        e = oracle.relF(got, ref)
        print(f"  relF {e:.3e}")
        assert e <= 1e-6
    else:
        # bf16: the oracle's value rounded once; an fp32 computation may land on the
        # other side of a rounding boundary, one unit in the last place at most
        rb = np64(torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16))
        # one bf16 unit in the last place of the larger of the two values, plus the
        # fp32 arithmetic of the rotation (cos, sin and the two products rounded):
        # at most 2^-22 (|x1| + |x2|) for a rotated entry whose pair is (x1, x2)
        mag = np.maximum(np.maximum(np.abs(rb), np.abs(got)), 2.0 ** -126)
        ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
        idx = np.arange(d)
        part = np.where(idx < rot, (idx + rot // 2) % rot if pairing == 0 else idx ^ 1, idx)
        arith = np.where(idx < rot, 2.0 ** -22, 0.0) * (np.abs(xr) + np.abs(xr[..., part]))
        diff = np.abs(got - rb)
        frac = np.mean(diff > 0)
        print(f"  elements differing from the rounded oracle: {frac:.2e}, "
              f"max {np.max(diff / (ulp + arith)):.2f} of the bound")
        assert np.all(diff <= ulp + arith) and frac < 1e-3
        assert oracle.relF(got, ref) <= 2e-3
    if rot < d:
        assert np.array_equal(got[..., rot:], xr[..., rot:])


def test_rope_keys_32k_prompt():
    """The bench's workload in its launch configuration: the 32k-token prompt's
    keys (8 segments x 4096, 16 heads, d = 128, bf16) moved out of place, every
    element against the oracle (rounded once to bf16, the bound of
    test_rope_keys)."""
    need_gpu()
    import state_caching_amd as sca
    r = synth.ROPE_32K
    x = synth.rope_keys(r["seed"], r["n_tokens"], r["h"], r["d"])
    xin = x.cuda()
    out = torch.empty_like(xin)
    case("rope keys, 32k-token prompt, 16 heads, bf16, out of place")
    sca.rope_rerotate(xin, r["seg_start"], r["seg_len"], r["delta"], out=out)
    torch.cuda.synchronize()
    got = np64(out)
    del xin, out
    xr = np64(x)
    ref = np.empty_like(xr)
    for s0, n, dl in zip(r["seg_start"], r["seg_len"], r["delta"]):
        ref[s0:s0 + n] = oracle.rope_rotate(xr[s0:s0 + n], float(dl))
    rb = np64(torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16))
    d = r["d"]
    mag = np.maximum(np.maximum(np.abs(rb), np.abs(got)), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    part = (np.arange(d) + d // 2) % d
    bound = ulp + 2.0 ** -22 * (np.abs(xr) + np.abs(xr[..., part]))
    diff = np.abs(got - rb)
    frac = np.mean(diff > 0)
    print(f"  elements differing from the rounded oracle: {frac:.2e}, "
          f"max {np.max(diff / bound):.2f} of the bound; relF {oracle.relF(got, ref):.3e}")
    assert np.all(diff <= bound) and frac < 1e-3
    assert oracle.relF(got, ref) <= 2e-3


@pytest.mark.parametrize("pairing,rot", [(0, 128), (1, 64)])
def test_rope_state(pairing, rot):
    """A state moved along its key dimension (Eq. (7)) against the oracle."""
    need_gpu()
    import state_caching_amd as sca
    S = synth.random_state(510 + rot, 4, 128, 128)
    out = torch.empty_like(S).cuda()
    case(f"rope state pairing={pairing} rot={rot}")
    sca.rope_rerotate_state(S.cuda(), 77777, rot_dim=rot, pairing=pairing, out=out)
    torch.cuda.synchronize()
    ref = oracle.rope_rotate_state(np64(S), 77777.0, rot_dim=rot, pairing=pairing)
    e = oracle.relF(np64(out), ref)
    print(f"  relF {e:.3e}")
    assert e <= 1e-6


def test_rope_state_identity_on_gpu():
    """Eq. (7) end to end on the GPU: a scalar-decay segment whose keys carry RoPE
    from start a, built; the same segment moved to start b (its keys re-rotated
    by the key kernel), built again; the first state moved by the state kernel
    equals the second."""
    need_gpu()
    import state_caching_amd as sca
    from state_caching_amd.runner import DeviceWorkload
    wl = synth.retnet(520, [200], 4, 64)
    dw = DeviceWorkload(wl)
    pos = list(range(200))
    ka = sca.rope_rerotate(dw.k.clone(), [p for p in pos], [1] * 200, [1000 + p for p in pos])
    kb = sca.rope_rerotate(ka.clone(), [0], [200], [5000 - 1000])
    case("rope state identity, scalar decay")

    def build(k):
        T, S0 = sca.segment_build(dw.rule, dw.gate_kind, k, dw.v, None, dw.gate, [0], [200])
        return S0

    Sa, Sb = build(ka), build(kb)
    Sm = sca.rope_rerotate_state(Sa[0].clone(), 4000)
    torch.cuda.synchronize()
    e = oracle.relF(np64(Sm), np64(Sb[0]))
    print(f"  relF {e:.3e}")
    assert e <= 1e-5


def test_gdn_100_segments_seams_sampled():
    need_gpu()
    wl = synth.workload("gdn_d128_32h_100x1024_seams_bf16")
    dw, T, S0 = _check_build(wl, segs=[0, 1, 99], heads=[0, 17], label="(sampled units)")
    case("compose 100 segments with 99 seams")
    S = dw.compose(T, S0)
    torch.cuda.synchronize()
    heads = [9]
    Tr, Sr = oracle.build_pairs(wl, heads=heads)
    S_or = oracle.compose(Tr, Sr, wl=wl, heads=heads, seams=True)
    e = head_relF(np64(S)[heads], S_or)
    print(f"  compose relF (head 9) {e:.3e}")
    assert e <= 2e-3


@pytest.mark.parametrize("conv_w", [0, 4])
def test_multilayer_seam_stack(conv_w):
    """Three layers composed bottom to top (ch.2 sec.5, Figs. 7-8): each layer's
    seam-window inputs (raw keys and values, write strengths, gates, queries)
    are seeded projections of the layer below's window read-outs.  The device
    runs one compose with read-outs per layer on its own pairs; the oracle runs
    every layer token by token over its windows from its own pairs and its own
    read-outs.  Every layer's read-outs and end state per head against it."""
    need_gpu()
    sca, DW = _lib()
    from state_caching_amd.runner import compose_layers
    from stack_util import project_np, project_torch
    h_k, h_v, d, w, n_layers = 2, 4, 32, 8, 3
    lens = [48, 40, 56, 36, 44]
    wls = [synth.gdn(700 + 10 * conv_w + l, lens, h_k, h_v, d, torch.float32, alpha_div=8.0,
                     conv_w=conv_w, seam_w=w) for l in range(n_layers)]
    P = [synth.layer_projection(720 + l, h_k, h_v, d) for l in range(n_layers - 1)]
    q0 = synth.window_queries(730 + conv_w, len(lens) - 1, w, h_k, d)
    layers = []
    for wl in wls:
        dw = DW(wl)
        T, S0 = dw.build()
        layers.append((T, S0, range(wl.n_seg), dw.seams, dw.tform, dw.prec))
    layers[0][3].q = q0.cuda()
    case(f"multi-layer seam stack: {n_layers} layers, conv_w={conv_w}, fp32, d={d}")
    got = compose_layers(layers, project_torch(P, h_k, h_v, d, norm_k=conv_w == 0, device="cuda"))
    torch.cuda.synchronize()
    pairs = [oracle.build_pairs(wl) for wl in wls]
    ref = oracle.compose_layers(wls, [p[0] for p in pairs], [p[1] for p in pairs],
                                np64(q0), project_np(P, h_k, h_v, d, norm_k=conv_w == 0))
    for l in range(n_layers):
        eS = head_relF(np64(got[l][0]), ref[l][0])
        eo, eo_win = _readout_errs(np64(got[l][1]), ref[l][1])
        print(f"  layer {l}: relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
        assert eS <= 1e-5 and eo <= 1e-5 and eo_win <= 1e-4, l


@pytest.mark.parametrize("d,conv_w,dtype", [(64, 4, torch.bfloat16), (128, 4, torch.bfloat16),
                                            (128, 0, torch.bfloat16), (32, 4, torch.float32),
                                            (16, 0, torch.float32)],
                         ids=["bf16-64-conv", "bf16-128-conv", "bf16-128", "f32-32-conv", "f32-16"])
def test_kda_seams_compose(d, conv_w, dtype):
    """KDA prompts on the reuse path (ch.2 sec.3 Table 1, KDA row; ch.2 sec.5):
    pairs built on the device, composed with per-channel-gate seam windows that
    read out at every window token, GQA, ragged segments: the end state per head
    and the read-outs against the oracle's composition of its own pairs."""
    need_gpu()
    lens = [40, 57, 33, 70, 21, 64, 45]
    wl = synth.kda(740 + d + conv_w, lens, 1, 2, d, dtype, gate_div=16.0, conv_w=conv_w, seam_w=8)
    sca, DW = _lib()
    dw = DW(wl)
    T, S0 = dw.build()
    S_init = synth.random_state(741 + d, 2, d, d)
    q = _attach_queries(dw, 742 + d + conv_w)
    case(f"KDA compose with seams and read-outs d={d} conv_w={conv_w} {dtype}")
    S = dw.compose(T, S0, S_init=S_init.cuda())
    torch.cuda.synchronize()
    Tr, S0r = oracle.build_pairs(wl)
    S_or, o_or = oracle.compose(Tr, S0r, S_init=np64(S_init), wl=wl, seams=True, q=q)
    eS = head_relF(np64(S), S_or)
    eo, eo_win = _readout_errs(np64(dw.seams.o), o_or)
    print(f"  relF S {eS:.3e}, o {eo:.3e} (worst head), {eo_win:.3e} (worst window and head)")
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    # a single window's read-out: 1e-4 where the pairs come from fp32 products, the
    # bf16 bound where the build took fp16 state products (bf16, no conv, d >= 64)
    win_tol = 2e-3 if (dtype == torch.bfloat16 and conv_w == 0 and d >= 64) else 1e-4
    assert eS <= tol and eo <= tol and eo_win <= win_tol


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_kda_seam_standalone(dtype):
    """hypic_seam_advance over one KDA window (per-channel gates) with read-outs,
    from a random state, against the oracle's token recurrence; a window pair
    is not available for per-channel gates and is refused."""
    need_gpu()
    sca, DW = _lib()
    d, h = 64, 2
    wl = synth.kda(750, [40, 30], 1, h, d, dtype, gate_div=8.0, conv_w=4, seam_w=8)
    dw = DW(wl)
    rng = np.random.default_rng(751)
    S_init = synth.random_state(752, h, d, d)
    q = synth._round(rng.standard_normal((1, 8, 1, d)) / np.sqrt(d), dtype)
    sm = dw.seams
    sm.q = q.cuda()
    sm.o = torch.zeros((1, 8, h, d), dtype=torch.float32, device="cuda")
    S = S_init.clone().cuda()
    case(f"KDA seam standalone {dtype}")
    sca.seam_advance(S, sm)
    torch.cuda.synchronize()
    s, e = wl.window_ranges()[0]
    sl = oracle.Slice(wl, s, e)
    u = sl.units()
    S_ref = np64(S_init).copy()
    o_ref = np.zeros((8, h, d))
    oracle.recur_units(wl.rule, sl.gate_kind, u, d, d, sl.k, sl.v, sl.beta, sl.g, S_ref,
                       q=np.ascontiguousarray(np64(q)[0]), o=o_ref, off_q=u.off_k, ldq=u.ldk,
                       off_o=u.off_v, ldo=u.ldv)
    errs = (head_relF(np64(S), S_ref), oracle.relF(np64(sm.o)[0], o_ref))
    print("  KDA seam relF S %.2e o %.2e" % errs)
    assert max(errs) <= 1e-5   # fp32 window arithmetic for every input dtype
    sm.T_w = torch.zeros((1, h, d, d), dtype=torch.float32, device="cuda")
    with pytest.raises(sca.HypicError):
        sca.seam_advance(S, sm)

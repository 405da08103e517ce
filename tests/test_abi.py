"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments synchronously with the documented status codes (CPU only: every
call below fails validation before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hypic.h")


@pytest.fixture(scope="module")
def sca():
    import state_caching_amd as m
    m.library()
    return m


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const\s+)?\w+\s*\*?\s*(hypic_\w+)\s*\(", text, re.M)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("hypic_segment_build", "hypic_compose", "hypic_seam_advance",
              "hypic_workspace_size", "hypic_status_string", "hypic_version"):
        assert n in names, names


def test_library_exports_every_declared_symbol(sca):
    out = subprocess.run(["nm", "-D", "--defined-only", sca.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(hypic_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_status_strings(sca):
    L = sca.library()
    assert L.hypic_status_string(0) == b"ok"
    assert b"invalid" in L.hypic_status_string(-1)
    assert L.hypic_version() >= 100


def _build_desc(sca, **over):
    ss = (ctypes.c_int64 * 2)(0, 64)
    sl = (ctypes.c_int64 * 2)(64, 64)
    kw = dict(rule=sca.RULE_DELTA, gate_kind=sca.GATE_SCALAR, in_dtype=sca.BF16, n_seg=2,
              seg_start=ctypes.cast(ss, sca._pi64), seg_len=ctypes.cast(sl, sca._pi64),
              h_k=2, h_v=4, d_k=128, d_v=128, k=16, v=16, beta=16, gate=16,
              conv_w=0, k_l2norm=0, conv_from=None, conv_wk=None, conv_wv=None,
              T_out=16, S0_out=16)
    kw.update(over)
    d = sca.BuildDesc(**kw)
    d._keep = (ss, sl)
    return d


@pytest.mark.parametrize("over,code", [
    (dict(h_v=3), -1),                       # h_v % h_k != 0
    (dict(k=None), -1),
    (dict(beta=None), -1),                   # delta rule needs beta
    (dict(d_k=96, d_v=96), -2),
    (dict(d_k=64, d_v=128), -2),
    (dict(gate_kind=0), -2),                 # delta rule with a per-head constant gate
    (dict(in_dtype=7), -1),
    (dict(k=8), -1),                         # misaligned pointer
    (dict(conv_w=5), -1),
    (dict(conv_w=4), -1),                    # conv without conv_from / weights
    (dict(rule=0, conv_w=0, k_l2norm=1), -2),  # decay family with key normalisation
])
def test_build_validation(sca, over, code):
    d = _build_desc(sca, **over)
    assert sca.library().hypic_segment_build(ctypes.byref(d), None, 0, None) == code


def test_build_negative_length(sca):
    d = _build_desc(sca)
    sl = (ctypes.c_int64 * 2)(64, -1)
    d.seg_len = ctypes.cast(sl, sca._pi64)
    assert sca.library().hypic_segment_build(ctypes.byref(d), None, 0, None) == -1


def test_build_workspace_required_for_conv(sca):
    cf = (ctypes.c_int64 * 2)(0, 64)
    d = _build_desc(sca, conv_w=4, conv_from=ctypes.cast(cf, sca._pi64), conv_wk=16, conv_wv=16,
                    k_l2norm=1)
    need = sca.library().hypic_workspace_size(ctypes.byref(d), sca.WS_BUILD)
    assert need == 128 * 2 * 128 * 4 + 128 * 4 * 128 * 4
    assert sca.library().hypic_segment_build(ctypes.byref(d), None, 0, None) == -3
    assert sca.library().hypic_workspace_size(ctypes.byref(_build_desc(sca)), sca.WS_BUILD) == 0


def _compose_desc(sca, order=(0, 1), **over):
    o = (ctypes.c_int32 * max(1, len(order)))(*order)
    kw = dict(tform=sca.T_DENSE, prec=sca.PREC_SPLIT, h_v=4, d_k=128, d_v=128, n=len(order),
              n_slots=2, order=ctypes.cast(o, sca._pi32), T_pool=16, S0_pool=16, S_init=None,
              S_out=16, seams=None)
    kw.update(over)
    d = sca.ComposeDesc(**kw)
    d._keep = o
    return d


@pytest.mark.parametrize("over,code", [
    (dict(tform=5), -1), (dict(prec=3), -1), (dict(h_v=0), -1), (dict(n=-1), -1),
    (dict(S_out=None), -1), (dict(T_pool=None), -1), (dict(n_slots=1), -1),
    (dict(d_k=48, d_v=48), -2), (dict(S_out=20), -1),
])
def test_compose_validation(sca, over, code):
    d = _compose_desc(sca, **over)
    assert sca.library().hypic_compose(ctypes.byref(d), None, 0, None) == code


def test_compose_seam_validation(sca):
    sd = sca.SeamDesc(rule=sca.RULE_DELTA, in_dtype=sca.BF16, w=8, conv_w=4, k_l2norm=1, h_k=4,
                      h_v=4, d_k=128, d_v=128, n_win=1, xk=16, xv=16, tail_k=16, tail_v=16,
                      conv_wk=16, conv_wv=16, beta=16, alpha=16)
    L = sca.library()
    d = _compose_desc(sca, seams=ctypes.pointer(sd))
    sd.w = 17                                     # fused windows hold at most 16 tokens
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -2
    sd.w = 8
    sd.n_win = 2                                  # must be n - 1
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -1
    sd.n_win = 1
    sd.tail_k = None                              # conv of width 4 needs the tail rows
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -1
    sd.tail_k = 16
    sd.rule = sca.RULE_DECAY
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -2
    d2 = _compose_desc(sca, tform=sca.T_DIAG, seams=ctypes.pointer(sd))
    sd.rule = sca.RULE_DELTA
    assert L.hypic_compose(ctypes.byref(d2), None, 0, None) == -2
    sd.q = 16                                     # read-outs: q and o together
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -1
    sd.o = 16
    sd.w = 12                                     # split-path read-outs hold windows of <= 8 rows
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -2
    sd.w = 8
    sd.T_w = 16                                   # window pairs are a standalone-call output
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -1
    sd.T_w = None
    # a valid read-out request that only lacks its workspace
    assert L.hypic_compose(ctypes.byref(d), None, 0, None) == -3
    need = L.hypic_workspace_size(ctypes.byref(d), sca.WS_COMPOSE)
    sd.q = sd.o = None
    assert need > L.hypic_workspace_size(ctypes.byref(d), sca.WS_COMPOSE)


def test_compose_workspace_sizes(sca):
    """Workspace of the 100-segment compose with seams (h_v = 32, d = 128, w = 8),
    without and with window read-outs, against the layout the header states:
    window records of (3 wp d + 4) floats, or (5 wp d + 4) with read-outs, then
    two pools of group pairs, then (read-outs) the rows Y [n-1, h_v, 8, 2d] and
    the states entering the groups; each array rounded up to 256 bytes."""
    L = sca.library()
    n, h, d, w = 100, 32, 128, 8
    sd = sca.SeamDesc(rule=sca.RULE_DELTA, in_dtype=sca.BF16, w=w, conv_w=4, k_l2norm=1, h_k=h,
                      h_v=h, d_k=d, d_v=d, n_win=n - 1, xk=16, xv=16, tail_k=16, tail_v=16,
                      conv_wk=16, conv_wv=16, beta=16, alpha=16)
    dsc = _compose_desc(sca, order=list(range(n)), h_v=h, n_slots=n, seams=ctypes.pointer(sd))
    al = lambda b: (b + 255) // 256 * 256
    wp = (w + 3) // 4 * 4
    G = -(-n // (256 // h))              # automatic group length: one (group, head) per CU
    ng = -(-n // G)
    pool = ng * h * d * d * 4
    plain = al((3 * wp * d + 4) * (n - 1) * h * 4) + 2 * pool
    assert L.hypic_workspace_size(ctypes.byref(dsc), sca.WS_COMPOSE) == plain
    sd.q, sd.o = 16, 16
    ro = al((5 * wp * d + 4) * (n - 1) * h * 4) + 2 * pool + al((n - 1) * h * 8 * 2 * d * 4) + pool
    assert L.hypic_workspace_size(ctypes.byref(dsc), sca.WS_COMPOSE) == ro
    # the fp32 path keeps its windows in the kernel: no workspace either way
    d32 = _compose_desc(sca, order=list(range(n)), h_v=h, n_slots=n, prec=sca.PREC_FP32,
                        seams=ctypes.pointer(sd))
    assert L.hypic_workspace_size(ctypes.byref(d32), sca.WS_COMPOSE) == 0


def test_seam_validation(sca):
    L = sca.library()
    sd = sca.SeamDesc(rule=sca.RULE_DELTA, in_dtype=sca.F32, w=65, conv_w=0, k_l2norm=0, h_k=1,
                      h_v=2, d_k=64, d_v=64, n_win=1, xk=16, xv=16, beta=16, alpha=16)
    assert L.hypic_seam_advance(ctypes.byref(sd), 16, None) == -2      # w > 64
    sd.w = 8
    assert L.hypic_seam_advance(ctypes.byref(sd), None, None) == -1
    sd.q = 16                                                            # q without o
    assert L.hypic_seam_advance(ctypes.byref(sd), 16, None) == -1
    sd.q = None
    sd.gate_diag = 2                                                     # neither gate form
    assert L.hypic_seam_advance(ctypes.byref(sd), 16, None) == -1
    sd.gate_diag = 1                                                     # KDA windows have no pair
    sd.T_w = 16
    assert L.hypic_seam_advance(ctypes.byref(sd), 16, None) == -2


def test_kda_seams_take_serial_compose(sca):
    """Per-channel window gates need no workspace: the compose runs them token
    by token in the serial dense kernel (the split path's window records hold
    scalar-gate operators only)."""
    L = sca.library()
    n, h, d, w = 100, 32, 128, 8
    sd = sca.SeamDesc(rule=sca.RULE_DELTA, in_dtype=sca.BF16, w=w, conv_w=4, k_l2norm=1, h_k=h,
                      h_v=h, d_k=d, d_v=d, n_win=n - 1, xk=16, xv=16, tail_k=16, tail_v=16,
                      conv_wk=16, conv_wv=16, beta=16, alpha=16)
    dsc = _compose_desc(sca, order=list(range(n)), h_v=h, n_slots=n, seams=ctypes.pointer(sd))
    assert L.hypic_workspace_size(ctypes.byref(dsc), sca.WS_COMPOSE) > 0
    sd.gate_diag = 1
    assert L.hypic_workspace_size(ctypes.byref(dsc), sca.WS_COMPOSE) == 0


def test_binding_rejects_out_of_range_rows(sca):
    k = torch.zeros(10, 1, 16)
    with pytest.raises(ValueError):
        sca.segment_build(sca.RULE_DELTA, sca.GATE_SCALAR, k, torch.zeros(10, 1, 16),
                          torch.zeros(10, 1), torch.ones(10, 1), [5], [6])


def _rope_desc(sca, **over):
    ss = (ctypes.c_int64 * 1)(0)
    sl = (ctypes.c_int64 * 1)(4)
    dl = (ctypes.c_int64 * 1)(7)
    f = dict(n_seg=1, seg_start=ctypes.cast(ss, ctypes.POINTER(ctypes.c_int64)),
             seg_len=ctypes.cast(sl, ctypes.POINTER(ctypes.c_int64)),
             delta=ctypes.cast(dl, ctypes.POINTER(ctypes.c_int64)), h=2, d=64, rot_dim=64,
             pairing=0, dtype=sca.BF16, base=10000.0, x_in=ctypes.c_void_p(4096),
             x_out=ctypes.c_void_p(4096))
    f.update(over)
    d = sca.RopeDesc(**f)
    d._keep = (ss, sl, dl)
    return d


@pytest.mark.parametrize("over,code", [
    (dict(d=60, rot_dim=56), -2),            # d not a multiple of 8
    (dict(rot_dim=12), -2),                  # rot_dim not a multiple of 8
    (dict(rot_dim=72), -2),                  # rot_dim > d
    (dict(d=1024, rot_dim=64), -2),
    (dict(pairing=2), -1),
    (dict(dtype=7), -1),
    (dict(base=0.0), -1),
    (dict(base=float("inf")), -1),
    (dict(h=0), -1),
    (dict(x_in=ctypes.c_void_p(4100)), -1),  # misaligned
    (dict(x_out=None), -1),
    (dict(seg_len=None), -1),
])
def test_rope_validation(sca, over, code):
    d = _rope_desc(sca, **over)
    assert sca.library().hypic_rope_rerotate(ctypes.byref(d), None) == code


def test_rope_state_validation(sca):
    L = sca.library()
    p = ctypes.c_void_p(4096)
    assert L.hypic_rope_rerotate_state(2, 64, 62, 64, 0, 10000.0, 5, p, p, None) == -2   # d_v % 4
    assert L.hypic_rope_rerotate_state(2, 64, 64, 20, 0, 10000.0, 5, p, p, None) == -2   # rot_dim % 8
    assert L.hypic_rope_rerotate_state(2, 64, 64, 64, 3, 10000.0, 5, p, p, None) == -1   # pairing
    assert L.hypic_rope_rerotate_state(2, 64, 64, 64, 0, -1.0, 5, p, p, None) == -1     # base
    assert L.hypic_rope_rerotate_state(2, 64, 64, 64, 0, 10000.0, 5, None, p, None) == -1


def test_compose_noalloc_validation(sca):
    """The allocation-free compose checks its arguments like hypic_compose and
    refuses, before touching a device, a request whose workspace exceeds its
    static scratch: the 100-segment prompt with w = 8 seams at h_v = 32,
    d = 128 needs 73 MB of the 64 MiB, so it returns HYPIC_E_TOO_LARGE; the
    same request at h_v = 16 fits and gets past that check."""
    L = sca.library()
    assert L.hypic_compose_noalloc(None, None) == -1
    d = _compose_desc(sca, tform=5)
    assert L.hypic_compose_noalloc(ctypes.byref(d), None) == -1
    n, d_ = 100, 128
    for h, fits in ((32, False), (16, True)):
        sd = sca.SeamDesc(rule=sca.RULE_DELTA, in_dtype=sca.BF16, w=8, conv_w=4, k_l2norm=1, h_k=h,
                          h_v=h, d_k=d_, d_v=d_, n_win=n - 1, xk=16, xv=16, tail_k=16, tail_v=16,
                          conv_wk=16, conv_wv=16, beta=16, alpha=16)
        dsc = _compose_desc(sca, order=list(range(n)), h_v=h, n_slots=n, seams=ctypes.pointer(sd))
        need = L.hypic_workspace_size(ctypes.byref(dsc), sca.WS_COMPOSE)
        assert (need <= sca.NOALLOC_SCRATCH_BYTES) == fits
        if not fits:
            assert L.hypic_compose_noalloc(ctypes.byref(dsc), None) == -6
            assert b"scratch" in L.hypic_status_string(-6)

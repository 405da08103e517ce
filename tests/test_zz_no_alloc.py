"""The allocation-free compose (hypic_compose_noalloc) against hypic_compose:
two calls in a row on one GPU, the second smaller, each compared with the
workspace entry point (the same kernels: bit-identical) and with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import case, head_relF, need_gpu, np64

pytestmark = pytest.mark.gpu


def _first_windows(sm, n_win):
    """The first n_win windows of a Seams (a prompt cut after n_win + 1 segments)."""
    import dataclasses
    cut = lambda t: None if t is None else t[:n_win].contiguous()
    return dataclasses.replace(sm, xk=cut(sm.xk), xv=cut(sm.xv), beta=cut(sm.beta), alpha=cut(sm.alpha),
                               tail_k=cut(sm.tail_k), tail_v=cut(sm.tail_v), q=cut(sm.q), o=cut(sm.o))


def test_compose_noalloc_matches_compose():
    need_gpu()
    import state_caching_amd as sca
    from state_caching_amd.runner import DeviceWorkload
    lens = [40, 64, 33, 70, 21, 64, 50, 90, 17, 64, 45, 80, 66, 29, 55, 64, 38, 70, 41, 52]
    wl = synth.gdn(700, lens, 2, 4, 128, torch.bfloat16, alpha_div=64.0, conv_w=4, seam_w=8)
    dw = DeviceWorkload(wl)
    T, S0 = dw.build()
    S_init = synth.random_state(701, 4, 128, 128).cuda()
    rng = np.random.default_rng(702)
    n_win = wl.n_seg - 1
    q = synth._round(rng.standard_normal((n_win, 8, wl.h_k, 128)) / np.sqrt(128), wl.dtype)
    order_all = list(range(wl.n_seg))
    # call 1: all 20 positions, 19 windows with read-outs; call 2: the first 9 positions,
    # no read-outs (a smaller workspace footprint on the same static scratch)
    for call, (n, ro) in enumerate(((wl.n_seg, True), (9, False))):
        sm = _first_windows(dw.seams, n - 1)
        sm.q = q[:n - 1].cuda() if ro else None
        sm_ref = _first_windows(dw.seams, n - 1)
        sm_ref.q = sm.q
        if ro:
            sm.o = torch.full((n - 1, 8, 4, 128), float("nan"), device="cuda")
            sm_ref.o = torch.full_like(sm.o, float("nan"))
        else:
            sm.o = sm_ref.o = None
        order = order_all[:n]
        S_ref = torch.empty((4, 128, 128), device="cuda")
        S_na = torch.full((4, 128, 128), float("nan"), device="cuda")
        case(f"compose_noalloc call {call}: n={n}, read-outs={ro}")
        sca.compose(T, S0, order, S_init=S_init, tform=dw.tform, prec=dw.prec, seams=sm_ref, S_out=S_ref)
        sca.compose_noalloc(T, S0, order, S_na, S_init=S_init, tform=dw.tform, prec=dw.prec, seams=sm)
        torch.cuda.synchronize()
        assert torch.equal(S_na, S_ref), "state differs from hypic_compose"
        if ro:
            assert torch.equal(sm.o, sm_ref.o), "read-outs differ from hypic_compose"
        Tn, Sn = np64(T)[:n], np64(S0)[:n]
        if ro:
            S_or, o_or = oracle.compose(Tn, Sn, S_init=np64(S_init), wl=wl, seams=True, q=np64(q))
        else:
            S_or = oracle.compose(Tn, Sn, S_init=np64(S_init), wl=wl, seams=True)
        e = head_relF(np64(S_na), S_or)
        msg = f"  call {call}: relF S vs oracle {e:.3e}"
        if ro:
            eo = max(oracle.relF(np64(sm.o)[:, :, h], o_or[:, :, h]) for h in range(4))
            msg += f", o {eo:.3e}"
            assert eo <= 2e-5
        print(msg, flush=True)
        assert e <= 2e-5

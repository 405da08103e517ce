"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc.build())


def test_retnet_head5_naive_ratio(orc):
    """The reference RetNet workload: head 5 has gamma = 1 - 2^-10, so the
    two-segment naive-addition ratio at 256 tokens is 1 - gamma^256 = 0.2213."""
    import synth
    wl = synth.workload("retnet_d64_8h_4x256_fp32")
    T, S0 = orc.build_pairs(wl, segs=[0, 1], heads=[5])
    true = orc.compose(T, S0)[0]
    delta = true - orc.naive_sum(S0)[0]
    r = np.linalg.norm(delta) / np.linalg.norm(S0[0, 0])
    gamma = 1.0 - 2.0 ** -10
    assert abs(r - (1 - gamma ** 256)) < 1e-6       # fp32-rounded gamma
    assert round(r, 4) == 0.2213


def test_relF_metric(orc):
    assert orc.relF(np.zeros(3), np.zeros(3)) == 0.0
    assert orc.relF(np.ones(4), np.ones(4) * 2) == pytest.approx(0.5)
    assert orc.relF(np.array([1e-40]), np.array([0.0])) == pytest.approx(1e-40 / 2.0 ** -126)
    # angle ~ relative error in radians for small perpendicular errors
    x = np.array([1.0, 6e-5])
    assert orc.angle_deg(x, np.array([1.0, 0.0])) == pytest.approx(np.degrees(6e-5), rel=1e-6)


def test_oracle_threads(orc):
    assert orc.threads() >= 1

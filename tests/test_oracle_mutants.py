"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant is a one-line textual change to oracle.c (a dropped term, a
wrong sign, a transposed operand, a reversed index), compiled to a scratch
library; the pins of tests/pins.py then run against it.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    "erase_sign": ("S[i * dv + j] -= b * k[i] * p[j];", "S[i * dv + j] += b * k[i] * p[j];"),
    "write_drops_beta": ("S[i * dv + j] += b * k[i] * v[j];", "S[i * dv + j] += k[i] * v[j];"),
    "scalar_gate_dropped": ("for (i = 0; i < dk * dv; ++i) S[i] *= g[0];",
                            "for (i = 0; i < dk * dv; ++i) S[i] *= 1.0;"),
    "diag_gate_transposed": ("for (j = 0; j < dv; ++j) S[i * dv + j] *= g[i];",
                             "for (j = 0; j < dv; ++j) S[i * dv + j] *= g[j];"),
    "decay_write_dropped": ("for (j = 0; j < dv; ++j) S[i * dv + j] += k[i] * v[j];",
                            "for (j = 0; j < dv; ++j) S[i * dv + j] += 0.0 * v[j];"),
    "erase_uses_ungated_dot": ("for (i = 0; i < dk; ++i) acc += k[i] * S[i * dv + j];",
                               "for (i = 0; i < dk; ++i) acc += k[i] * S[j * dk + i];"),
    "readout_transposed": ("for (i = 0; i < dk; ++i) acc += q[i] * S[i * dv + j];",
                           "for (i = 0; i < dk; ++i) acc += q[i] * S[i * dv + (dv - 1 - j)];"),
    "pair_transposed": ("acc += Tu[i * dk + l] * Su[l * dv + j];",
                        "acc += Tu[l * dk + i] * Su[l * dv + j];"),
    "pair_drops_S0": ("tmp[i * dv + j] = acc + S0u[i * dv + j];", "tmp[i * dv + j] = acc;"),
    "conv_reversed": ("int src = t - (W - 1) + j;", "int src = t - j;"),
    "l2norm_no_sqrt": ("double inv = 1.0 / sqrt(s);", "double inv = 1.0 / s;"),
    "transition_init_not_identity": ("T[u * (long)dk * dk + (long)i * dk + i] = 1.0;",
                                     "T[u * (long)dk * dk + (long)i * dk + i] = 0.5;"),
    "rope_sin_sign": ("v[a] = x1 * c - x2 * sn;", "v[a] = x1 * c + x2 * sn;"),
    "rope_frequency_exponent": ("pow(base, -2.0 * (double)i / (double)rot_dim)",
                                "pow(base, -1.0 * (double)i / (double)rot_dim)"),
    "rope_half_pairing_offset": ("int b = pairing == 0 ? i + half : 2 * i + 1;",
                                 "int b = pairing == 0 ? i + half - 1 : 2 * i + 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut_src = tmp_path / "oracle_mut.c"
    mut_src.write_text(src.replace(old, new))
    so = str(tmp_path / f"liboracle_{name}.so")
    import subprocess
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    str(mut_src), "-o", so, "-lm"], check=True)
    failed = []
    for pin in pins.ALL:
        try:
            pin(so)
        except (AssertionError, FloatingPointError, ValueError, IndexError) as e:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

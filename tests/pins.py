"""Pins of the fp64 oracle against what the HYPIC pages and plain mathematics fix.

Every check takes the path of an oracle build, so the same checks run on the
real oracle (tests/test_oracle_pins.py) and on builds with a planted mistake
(tests/test_oracle_mutants.py), where at least one of them must fail.

Sources (page "HYPIC ... reading notes" unless noted):
  worked example ..... ch.2 sec.2, the 1-D teaching example
  Table 2 ............ ch.1 sec.2, Eqs. (4)-(5), Table 2
  22 % ............... aibase news article (page 2)
  affine summary ..... ch.2 sec.2 (T_C, S_{C|0}, F_C)
  composition law .... ch.2 sec.2 (pairwise law, associative, not commutative)
  Eq. (6) ............ ch.2 sec.2
  T_i = I reduction .. ch.1 sec.2
  family forms ....... ch.2 sec.3, Table 1
  conv warm-up ....... ch.2 sec.6
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- helpers

def one_unit(path, rule, gate_kind, k, v, beta, g, S_init=None):
    """Pair (T, S0) and, if S_init is given, the end state from S_init,
    for a single unit given as k [m, dk], v [m, dv], beta [m], g [m] / [m, dk]."""
    k = np.ascontiguousarray(k, dtype=np.float64)[:, None, :]
    v = np.ascontiguousarray(v, dtype=np.float64)[:, None, :]
    m, _, dk = k.shape
    dv = v.shape[2]
    b = np.ascontiguousarray(beta if beta is not None else np.zeros(m), dtype=np.float64)[:, None]
    g = np.asarray(g, dtype=np.float64)
    g = np.ascontiguousarray(g[:, None, :] if gate_kind == "diag" else g[:, None])
    u = oracle.Units([(0, m, 0, 0)], 1, 1, dk, dv, gate_kind)
    T, S0 = oracle.build_units(rule, gate_kind, u, dk, dv, k, v, b, g, path)
    end = None
    if S_init is not None:
        S = np.array(S_init, dtype=np.float64, copy=True)[None]
        oracle.recur_units(rule, gate_kind, u, dk, dv, k, v, b, g, S, path=path)
        end = S[0]
    return T[0], S0[0], end


def dense_transition(rule, gate_kind, k, beta, g):
    dk = k.shape[0]
    G = np.diag(g) if gate_kind == "diag" else g * np.eye(dk)
    if rule == "decay":
        return G
    P = np.eye(dk) - beta * np.outer(k, k)
    return P @ G if gate_kind == "diag" else g * P


def dense_write(rule, k, v, beta):
    return np.outer(k, v) * (beta if rule == "delta" else 1.0)


def rand_unit(rng, rule, gate_kind, m, dk, dv, slow=False):
    k = rng.standard_normal((m, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((m, dv))
    beta = rng.uniform(0.1, 0.9, m) if rule == "delta" else None
    lo = 0.9 if slow else 0.3
    g = rng.uniform(lo, 1.0, (m, dk) if gate_kind == "diag" else m)
    return k, v, beta, g


FAMILIES = [("decay", "scalar"), ("decay", "diag"), ("delta", "scalar"), ("delta", "diag")]


# ------------------------------------------------------------------- pins

def pin_worked_example(path):
    gx = _golden("worked_example.json")
    m = len(gx["token_decay"])
    T, S0, end = one_unit(path, "decay", "scalar", np.ones((m, 1)),
                          np.array(gx["token_write"])[:, None], None,
                          np.array(gx["token_decay"]), S_init=[[gx["prefix_state"]]])
    assert abs(T[0, 0] - gx["T_C"]) < 1e-15, T
    assert abs(S0[0, 0] - gx["S_C0"]) < 1e-15, S0
    S = oracle.compose(T[None, None], S0[None, None], np.array([[[gx["prefix_state"]]]]),
                       path=path)
    assert abs(S[0, 0, 0] - gx["composed"]) < 1e-14, S
    assert abs(end[0, 0] - gx["composed"]) < 1e-14, end
    parts = np.stack([np.full((1, 1, 1), gx["prefix_state"]), S0[None]])
    naive = oracle.naive_sum(parts)
    assert abs(naive[0, 0, 0] - gx["naive_sum"]) < 1e-14


def _two_segment_ratio(path, gamma, n1, n2, d=8, seed=0):
    """||Delta|| / ||S_{C1|0}|| with Delta = true - naive, from oracle runs."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n1 + n2, d))
    v = rng.standard_normal((n1 + n2, d))
    g = np.full(n1 + n2, gamma)
    _, S1, _ = one_unit(path, "decay", "scalar", k[:n1], v[:n1], None, g[:n1])
    T2, S2, _ = one_unit(path, "decay", "scalar", k[n1:], v[n1:], None, g[n1:])
    _, true, _ = one_unit(path, "decay", "scalar", k, v, None, g)
    delta = true - (S1 + S2)
    return np.linalg.norm(delta) / np.linalg.norm(S1), delta, T2, S1


def pin_table2(path):
    gx = _golden("table2_naive_error.json")
    gamma = 1.0 - 2.0 ** -gx["gamma_exponent"]
    for n2, printed in zip(gx["C2_len"], gx["ratio_printed"]):
        r, _, _, _ = _two_segment_ratio(path, gamma, 300, n2)
        assert round(r, gx["printed_decimals"]) == printed, (n2, r, printed)
        assert abs(r - (1.0 - gamma ** n2)) < 1e-10, (n2, r)


def pin_news_22pct(path):
    gx = _golden("news_slow_decay_22pct.json")
    gamma = 1.0 - 2.0 ** -gx["gamma_exponent"]
    r, _, _, _ = _two_segment_ratio(path, gamma, 256, gx["C2_len"], seed=1)
    assert round(100 * r) == gx["ratio_percent_printed"], r


def pin_naive_error_identity(path):
    """Delta = (T_{C2} - I) S_{C1|0} (Eq. (4)), for every family."""
    rng = np.random.default_rng(2)
    for rule, gk in FAMILIES:
        k, v, b, g = rand_unit(rng, rule, gk, 24, 5, 3, slow=True)
        _, S1, _ = one_unit(path, rule, gk, k[:10], v[:10], None if b is None else b[:10], g[:10])
        T2, S2, _ = one_unit(path, rule, gk, k[10:], v[10:], None if b is None else b[10:], g[10:])
        _, true, _ = one_unit(path, rule, gk, k, v, b, g)
        delta = true - (S1 + S2)
        assert np.allclose(delta, (T2 - np.eye(5)) @ S1, atol=1e-12, rtol=0), (rule, gk)


def pin_brute_force(path):
    """Dense products of explicitly formed T_i (ch.2 sec.2 expansion)."""
    rng = np.random.default_rng(3)
    for rule, gk in FAMILIES:
        for m, dk, dv in [(1, 2, 3), (5, 3, 2), (8, 4, 4)]:
            k, v, b, g = rand_unit(rng, rule, gk, m, dk, dv)
            Ts = [dense_transition(rule, gk, k[t], None if b is None else b[t], g[t])
                  for t in range(m)]
            us = [dense_write(rule, k[t], v[t], None if b is None else b[t]) for t in range(m)]
            T_ref = np.eye(dk)
            for t in range(m):
                T_ref = Ts[t] @ T_ref
            S_ref = np.zeros((dk, dv))
            for t in range(m):
                P = np.eye(dk)
                for s in range(m - 1, t, -1):   # T_m ... T_{t+1}
                    P = P @ Ts[s]
                S_ref += P @ us[t]
            if m >= 2:
                assert np.allclose(np.linalg.multi_dot(Ts[::-1]), T_ref, atol=1e-14)
            T, S0, _ = one_unit(path, rule, gk, k, v, b, g)
            assert np.allclose(T, T_ref, atol=1e-13, rtol=0), (rule, gk, m)
            assert np.allclose(S0, S_ref, atol=1e-13, rtol=0), (rule, gk, m)


def pin_affine(path):
    """Recurrence from any S_init equals T_C S_init + S_{C|0} (F_C)."""
    rng = np.random.default_rng(4)
    for rule, gk in FAMILIES:
        k, v, b, g = rand_unit(rng, rule, gk, 40, 6, 5, slow=True)
        S_init = rng.standard_normal((6, 5))
        T, S0, end = one_unit(path, rule, gk, k, v, b, g, S_init=S_init)
        assert np.allclose(end, T @ S_init + S0, atol=1e-12, rtol=0), (rule, gk)


def pin_decay_closed_forms(path):
    """Scalar decay: T = gamma^m I, S0 = K^T diag(gamma^(m-t)) V.
    Diagonal gate: T = diag(exp(cl_m)), S0 = (K * exp(cl_m - cl_t))^T V."""
    rng = np.random.default_rng(5)
    m, dk, dv = 50, 6, 4
    k = rng.standard_normal((m, dk))
    v = rng.standard_normal((m, dv))
    gamma = 0.97
    T, S0, _ = one_unit(path, "decay", "scalar", k, v, None, np.full(m, gamma))
    w = gamma ** (m - 1 - np.arange(m))
    assert np.allclose(T, gamma ** m * np.eye(dk), rtol=1e-13, atol=0)
    assert np.allclose(S0, k.T @ (w[:, None] * v), rtol=1e-12, atol=1e-13)
    g = rng.uniform(0.8, 1.0, (m, dk))
    cl = np.cumsum(np.log(g), axis=0)
    T, S0, _ = one_unit(path, "decay", "diag", k, v, None, g)
    assert np.allclose(T, np.diag(np.exp(cl[-1])), rtol=1e-12, atol=0)
    assert np.allclose(S0, (k * np.exp(cl[-1] - cl)).T @ v, rtol=1e-12, atol=1e-13)


def pin_identity_transition(path):
    """With T_i = I the zero-initial end states simply add (ch.1 sec.2)."""
    rng = np.random.default_rng(6)
    k = rng.standard_normal((30, 4))
    v = rng.standard_normal((30, 3))
    one = np.ones(30)
    T, S0, _ = one_unit(path, "decay", "scalar", k, v, None, one)
    _, S1, _ = one_unit(path, "decay", "scalar", k[:12], v[:12], None, one[:12])
    _, S2, _ = one_unit(path, "decay", "scalar", k[12:], v[12:], None, one[12:])
    assert np.allclose(T, np.eye(4), atol=0, rtol=0)
    assert np.allclose(S0, k.T @ v, atol=1e-12)
    assert np.allclose(S0, S1 + S2, atol=1e-12)


def pin_composition_laws(path):
    """Pairwise law, associativity, Eq. (6) and non-commutativity."""
    rng = np.random.default_rng(7)
    for rule, gk in FAMILIES:
        parts = []
        for m in (9, 13, 7):
            k, v, b, g = rand_unit(rng, rule, gk, m, 4, 3, slow=True)
            parts.append(one_unit(path, rule, gk, k, v, b, g)[:2])
        (TA, BA), (TB, BB), (TC, BC) = parts
        S_s = rng.standard_normal((4, 3))
        seq = oracle.compose(np.array([[TA], [TB], [TC]]), np.array([[BA], [BB], [BC]]),
                             S_s[None], path=path)[0]
        # (C o B) o A  vs  C o (B o A), pair law (T_B T_A, T_B B_A + B_B)
        TBA, BBA = TB @ TA, TB @ BA + BB
        left = TC @ (TBA @ S_s + BBA) + BC
        TCB, BCB = TC @ TB, TC @ BB + BC
        right = TCB @ (TA @ S_s + BA) + BCB
        eq6 = (TC @ TB @ TA) @ S_s + (TC @ TB) @ BA + TC @ BB + BC
        for x in (left, right, eq6):
            assert np.allclose(seq, x, atol=1e-12), (rule, gk)
        swapped = oracle.compose(np.array([[TB], [TA], [TC]]), np.array([[BB], [BA], [BC]]),
                                 S_s[None], path=path)[0]
        assert np.linalg.norm(swapped - seq) > 1e-3 * np.linalg.norm(seq), (rule, gk)


def pin_gdn_bounds(path):
    """||k|| = 1, beta in [0,1]: ||T_i||_2 = alpha_i, hence ||T_C||_2 <= prod alpha.
    DeltaNet with beta = 1 makes T_i a projector that annihilates k."""
    rng = np.random.default_rng(8)
    k, v, b, g = rand_unit(rng, "delta", "scalar", 30, 8, 4)
    T, _, _ = one_unit(path, "delta", "scalar", k, v, b, g)
    assert np.linalg.norm(T, 2) <= np.prod(g) * (1 + 1e-12)
    T1, _, _ = one_unit(path, "delta", "scalar", k[:1], v[:1], np.ones(1), np.ones(1))
    assert np.allclose(T1 @ T1, T1, atol=1e-14)
    assert np.allclose(T1 @ k[0], 0.0, atol=1e-14)
    assert abs(np.trace(T1) - 7.0) < 1e-13


def pin_key_scale(path):
    """The delta transition depends on beta and k only through beta k k^T
    (ch.2 sec.3, Table 1): keys scaled by r = 2^6 with beta / r^2 give the same
    T_C, and the writes beta k v^T, hence S_{C|0}, scale by 1/r.  Powers of two
    keep the scaled inputs exact."""
    rng = np.random.default_rng(12)
    k, v, b, g = rand_unit(rng, "delta", "scalar", 40, 8, 5)
    T, S0, _ = one_unit(path, "delta", "scalar", k, v, b, g)
    for r in (2.0 ** 6, 2.0 ** -6):
        Tr, S0r, _ = one_unit(path, "delta", "scalar", k * r, v, b / (r * r), g)
        assert np.allclose(Tr, T, rtol=0, atol=1e-13 * np.abs(T).max())
        assert np.allclose(S0r * r, S0, rtol=0, atol=1e-13 * np.abs(S0).max())


def pin_kda_reductions(path):
    """Delta rule with a diagonal gate (KDA row of Table 1), against the other
    families and the norm bound:
    - equal gates on every channel (g_i = a_i 1) give the gated-delta pair;
    - b = 0 gives the gate-only product diag(prod g) and S0 = 0 (the diagonal
      gate's closed form, T = diag(exp(cl_m)));
    - ||k|| = 1, b in [0,1]: ||T_i||_2 <= max_d g_i[d], hence ||T_C||_2 <= prod max g;
    - the gate acts before the erase: T_1 = (I - b k k^T) diag(g), not diag(g)(I - b k k^T)."""
    rng = np.random.default_rng(15)
    m, dk, dv = 21, 6, 5
    k, v, b, _ = rand_unit(rng, "delta", "scalar", m, dk, dv)
    a = rng.uniform(0.5, 1.0, m)
    T1, S1, _ = one_unit(path, "delta", "diag", k, v, b, np.repeat(a[:, None], dk, axis=1))
    T2, S2, _ = one_unit(path, "delta", "scalar", k, v, b, a)
    assert np.allclose(T1, T2, rtol=0, atol=1e-14) and np.allclose(S1, S2, rtol=0, atol=1e-13)
    g = rng.uniform(0.3, 1.0, (m, dk))
    T0, S0, _ = one_unit(path, "delta", "diag", k, v, np.zeros(m), g)
    assert np.allclose(T0, np.diag(np.exp(np.log(g).sum(axis=0))), rtol=1e-13, atol=0)
    assert np.all(S0 == 0.0)
    T, _, _ = one_unit(path, "delta", "diag", k, v, b, g)
    assert np.linalg.norm(T, 2) <= np.prod(g.max(axis=1)) * (1 + 1e-12)
    Tf, _, _ = one_unit(path, "delta", "diag", k[:1], v[:1], b[:1], g[:1])
    P = np.eye(dk) - b[0] * np.outer(k[0], k[0])
    assert np.allclose(Tf, P @ np.diag(g[0]), rtol=0, atol=1e-15)
    assert not np.allclose(Tf, np.diag(g[0]) @ P, rtol=0, atol=1e-6)


def pin_rope(path):
    """Rotary re-rotation (ch.2 sec.6, Eq. (8): K_b = R(b - a) K_a), against the
    rotation's own algebra and a direct 2x2 construction:
    - R(0) = I, R(b) R(a) = R(a + b), R(-a) R(a) = I, every pair keeps its norm;
    - relative positions: <R(m) q, R(n) k> = <R(m - n) q, k>;
    - the first pair turns by exactly delta radians (theta_0 = 1) and the last
      by delta base^(-(rot-2)/rot), written out as 2x2 rotations;
    - the interleaved pairing is the half pairing conjugated by the permutation
      that interleaves the two halves; entries past rot_dim pass through;
    - a key encoded at a + p and moved by b - a equals the key encoded at b + p."""
    rng = np.random.default_rng(16)
    d, base = 16, 10000.0
    x = rng.standard_normal((5, d))
    assert np.array_equal(oracle.rope_rotate(x, 0.0, path=path), x)
    a, b = 37.0, -1250.0
    xa = oracle.rope_rotate(x, a, path=path)
    assert np.allclose(oracle.rope_rotate(xa, b, path=path), oracle.rope_rotate(x, a + b, path=path), atol=1e-12)
    assert np.allclose(oracle.rope_rotate(xa, -a, path=path), x, atol=1e-13)
    h = d // 2
    n0 = x[:, :h] ** 2 + x[:, h:] ** 2
    n1 = xa[:, :h] ** 2 + xa[:, h:] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in ((3.0, 11.0), (1000.0, 7.0)):
        lhs = oracle.rope_rotate(q, m, path=path) @ oracle.rope_rotate(k, n, path=path)
        assert abs(lhs - oracle.rope_rotate(q, m - n, path=path) @ k) < 1e-12
    th_last = 5.0 * base ** (-(d - 2) / d)
    for i, th in ((0, 5.0), (h - 1, th_last)):
        c, s_ = np.cos(th), np.sin(th)
        y = oracle.rope_rotate(x, 5.0, path=path)
        assert np.allclose(y[:, i], c * x[:, i] - s_ * x[:, i + h], atol=1e-14)
        assert np.allclose(y[:, i + h], s_ * x[:, i] + c * x[:, i + h], atol=1e-14)
    perm = np.empty(d, dtype=int)
    perm[0::2], perm[1::2] = np.arange(h), np.arange(h) + h     # interleaved slot -> half slot
    yi = oracle.rope_rotate(x[:, perm], 5.0, pairing=1, path=path)
    assert np.allclose(yi, oracle.rope_rotate(x, 5.0, path=path)[:, perm], atol=1e-14)
    yp = oracle.rope_rotate(x, 5.0, rot_dim=8, path=path)
    assert np.array_equal(yp[:, 8:], x[:, 8:])
    assert np.allclose(yp[:, :8], oracle.rope_rotate(x[:, :8], 5.0, path=path), atol=0)
    pos = np.arange(6, dtype=np.float64)
    kx = rng.standard_normal((6, d))
    ka = oracle.rope_rotate(kx, 40.0 + pos, path=path)
    kb = oracle.rope_rotate(kx, 900.0 + pos, path=path)
    assert np.allclose(oracle.rope_rotate(ka, 860.0, path=path), kb, atol=1e-12)


def pin_rope_state(path):
    """Eq. (7), S_{C|b} = R(b - a) S_{C|a}: a segment whose keys carry RoPE at
    positions a + p, moved to b + p.  Holds for the scalar transition (gamma I
    commutes with R) and for the gated delta rule, whose transition is built
    from the moved keys (T_C -> R T_C R^T); fails for a diagonal gate, which
    does not commute with R."""
    rng = np.random.default_rng(17)
    m, d, dv = 9, 8, 3
    k0 = rng.standard_normal((m, d))
    k0 /= np.linalg.norm(k0, axis=1, keepdims=True)
    v = rng.standard_normal((m, dv))
    beta = rng.uniform(0.1, 0.9, m)
    pa, pb = 100.0 + np.arange(m), 4321.0 + np.arange(m)
    ka = oracle.rope_rotate(k0, pa, path=path)
    kb = oracle.rope_rotate(k0, pb, path=path)
    dlt = 4321.0 - 100.0
    _, Sa, _ = one_unit(path, "decay", "scalar", ka, v, None, np.full(m, 0.97))
    _, Sb, _ = one_unit(path, "decay", "scalar", kb, v, None, np.full(m, 0.97))
    assert np.allclose(oracle.rope_rotate_state(Sa, dlt, path=path), Sb, atol=1e-12)
    alpha = rng.uniform(0.6, 1.0, m)
    Ta, Sa, _ = one_unit(path, "delta", "scalar", ka, v, beta, alpha)
    Tb, Sb, _ = one_unit(path, "delta", "scalar", kb, v, beta, alpha)
    assert np.allclose(oracle.rope_rotate_state(Sa, dlt, path=path), Sb, atol=1e-12)
    R = oracle.rope_rotate_state(np.eye(d), dlt, path=path)
    assert np.allclose(R @ Ta @ R.T, Tb, atol=1e-12)
    g = rng.uniform(0.3, 1.0, (m, d))
    _, Sa, _ = one_unit(path, "decay", "diag", ka, v, None, g)
    _, Sb, _ = one_unit(path, "decay", "diag", kb, v, None, g)
    assert not np.allclose(oracle.rope_rotate_state(Sa, dlt, path=path), Sb, atol=1e-6)


def pin_conv(path):
    """Depthwise causal conv against numpy's full convolution, with history."""
    rng = np.random.default_rng(9)
    n, C, W = 11, 5, 4
    x = rng.standard_normal((n, C))
    w = rng.standard_normal((C, W))
    hist = rng.standard_normal((W - 1, C))
    y = oracle.causal_conv(x, w, hist, path)
    y0 = oracle.causal_conv(x, w, None, path)
    xe = np.concatenate([hist, x])
    for c in range(C):
        full = np.convolve(xe[:, c], w[c, ::-1])          # y_t = sum_j w_j x_{t-(W-1)+j}
        assert np.allclose(y[:, c], full[W - 1:W - 1 + n], atol=1e-13)
        full0 = np.convolve(x[:, c], w[c, ::-1])
        assert np.allclose(y0[:, c], full0[:n], atol=1e-13)


def pin_l2norm(path):
    rng = np.random.default_rng(10)
    x = rng.standard_normal((7, 3, 9))
    y = oracle.l2norm_rows(x, path)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x, atol=1e-14)


def pin_compose_equals_full(path):
    """Composition = full recompute, with conv warm-up and seams (w >= W-1),
    and differs when the seam is narrower than the conv history (ch.2 sec.6)."""
    import synth
    import torch
    for seam_w, should_match in ((8, True), (3, True), (0, False), (2, False)):
        wl = synth.gdn(11, [40, 37, 45], 2, 2, 8, torch.float32, alpha_div=64.0,
                       conv_w=4, seam_w=seam_w)
        T, S0 = oracle.build_pairs(wl, path=path)
        S = oracle.compose(T, S0, wl=wl, seams=seam_w > 0, path=path)
        F = oracle.full_recompute(wl, path=path)
        err = oracle.relF(S, F)
        if should_match:
            assert err < 1e-12, (seam_w, err)
        else:
            assert err > 1e-4, (seam_w, err)
    # per-channel gates (KDA windows), GQA, read-outs at the window tokens
    wl = synth.kda(17, [30, 26, 35, 22], 1, 2, 8, torch.float32, gate_div=16.0, conv_w=4, seam_w=6)
    q_all = np.random.default_rng(18).standard_normal((wl.n_tokens, 1, 8))
    wins = wl.window_ranges()
    T, S0 = oracle.build_pairs(wl, path=path)
    S, o = oracle.compose(T, S0, wl=wl, seams=True, path=path,
                          q=np.stack([q_all[s:e] for s, e in wins]))
    F, o_full = oracle.recur_range(wl, 0, wl.n_tokens, np.zeros((2, 8, 8)), path=path, q=q_all)
    assert oracle.relF(S, F) < 1e-12
    for j, (s, e) in enumerate(wins):
        assert oracle.relF(o[j], o_full[s:e]) < 1e-12, j
    wl = synth.gdn(12, [33, 50, 21, 64], 1, 2, 8, torch.float32, alpha_div=16.0)
    S_init = np.random.default_rng(13).standard_normal((2, 8, 8))
    T, S0 = oracle.build_pairs(wl, path=path)
    S = oracle.compose(T, S0, S_init, path=path)
    F = oracle.full_recompute(wl, S_init, path=path)
    assert oracle.relF(S, F) < 1e-12


def pin_readout(path):
    """o_t = q_t^T S_t with the post-update state (Eq. (2))."""
    rng = np.random.default_rng(14)
    for rule, gk in FAMILIES:
        m, dk, dv = 6, 4, 3
        k, v, b, g = rand_unit(rng, rule, gk, m, dk, dv)
        q = rng.standard_normal((m, 1, dk))
        S_ref = rng.standard_normal((dk, dv))
        S = S_ref.copy()[None]
        o = np.zeros((m, 1, dv))
        bb = np.zeros((m, 1)) if b is None else b[:, None].copy()
        gg = g[:, None, :].copy() if gk == "diag" else g[:, None].copy()
        u = oracle.Units([(0, m, 0, 0)], 1, 1, dk, dv, gk)
        oracle.recur_units(rule, gk, u, dk, dv, np.ascontiguousarray(k[:, None]),
                           np.ascontiguousarray(v[:, None]), bb, gg, S, q=q, o=o,
                           off_q=[0], ldq=dk, off_o=[0], ldo=dv, path=path)
        for t in range(m):
            Tt = dense_transition(rule, gk, k[t], None if b is None else b[t], g[t])
            S_ref = Tt @ S_ref + dense_write(rule, k[t], v[t], None if b is None else b[t])
            assert np.allclose(o[t, 0], q[t, 0] @ S_ref, atol=1e-13), (rule, gk, t)
        assert np.allclose(S[0], S_ref, atol=1e-13)


def pin_compose_readouts(path):
    """Read-outs of the seam windows along a composed chain equal the read-outs
    of the full token recurrence at the same tokens (ch.2 sec.5: the recomputed
    window tokens see the true prefix state; Eq. (2)), GQA heads and a subset
    of value heads included."""
    import synth
    import torch
    rng = np.random.default_rng(15)
    for seam_w, heads in ((8, None), (3, [1])):
        wl = synth.gdn(16, [40, 37, 45, 30], 1, 2, 8, torch.float32, alpha_div=32.0,
                       conv_w=4, seam_w=seam_w)
        q_all = rng.standard_normal((wl.n_tokens, wl.h_k, wl.d_k))
        hs = list(range(wl.h_v)) if heads is None else heads
        _, o_full = oracle.recur_range(wl, 0, wl.n_tokens, np.zeros((len(hs), wl.d_k, wl.d_v)),
                                       heads=hs, path=path, q=q_all)
        wins = wl.window_ranges()
        q_win = np.stack([q_all[s:e] for s, e in wins])
        T, S0 = oracle.build_pairs(wl, heads=hs, path=path)
        S, o = oracle.compose(T, S0, wl=wl, heads=hs, seams=True, path=path, q=q_win)
        assert o.shape == (len(wins), seam_w, len(hs), wl.d_v)
        for j, (s, e) in enumerate(wins):
            assert oracle.relF(o[j], o_full[s:e]) < 1e-12, (seam_w, j)
        S_full = oracle.recur_range(wl, 0, wl.n_tokens, np.zeros((len(hs), wl.d_k, wl.d_v)),
                                    heads=hs, path=path)
        assert oracle.relF(S, S_full) < 1e-12


def pin_compose_layers(path):
    """A stack of three layers whose seam-window inputs are projections of the
    layer below's window read-outs (ch.2 sec.5, Figs. 7-8) equals, layer by
    layer, the full token recurrence over the whole prompt with those window
    rows substituted: read-outs at the window tokens and the end state, GQA
    heads included (no conv, so the cached bodies never read the windows)."""
    import synth
    import torch
    from stack_util import project_np
    h_k, h_v, d, w = 1, 2, 8, 4
    lens = [20, 17, 23, 15]
    wls = [synth.gdn(30 + l, lens, h_k, h_v, d, torch.float32, alpha_div=8.0, seam_w=w)
           for l in range(3)]
    P = [synth.layer_projection(40 + l, h_k, h_v, d) for l in range(2)]
    proj = project_np(P, h_k, h_v, d, norm_k=True)
    wins = wls[0].window_ranges()
    q0 = synth.window_queries(50, len(wins), w, h_k, d).double().numpy()
    pairs = [oracle.build_pairs(wl, path=path) for wl in wls]
    got = oracle.compose_layers(wls, [p[0] for p in pairs], [p[1] for p in pairs], q0, proj,
                                path=path)
    win, q = None, q0
    for l, wl in enumerate(wls):
        wl_l = wl if win is None else oracle._with_window_rows(wl, win)
        q_all = np.zeros((wl.n_tokens, h_k, d))
        for j, (s, e) in enumerate(wins):
            q_all[s:e] = q[j]
        S_full, o_full = oracle.recur_range(wl_l, 0, wl.n_tokens, np.zeros((h_v, d, d)), path=path,
                                            q=q_all)
        o_win = np.stack([o_full[s:e] for s, e in wins])
        S, o = got[l]
        assert oracle.relF(S, S_full) < 1e-12, l
        assert oracle.relF(o, o_win) < 1e-12, l
        if l + 1 < len(wls):
            win = proj(l, o_win)
            q = win["q"]
    # the layers differ: the upper layers' windows do not see layer 0's rows
    assert oracle.relF(got[1][1], got[0][1]) > 0.1


ALL = [pin_readout, pin_compose_readouts, pin_compose_layers, pin_worked_example, pin_table2, pin_news_22pct, pin_naive_error_identity,
       pin_brute_force, pin_affine, pin_decay_closed_forms, pin_identity_transition,
       pin_composition_laws, pin_gdn_bounds, pin_key_scale, pin_kda_reductions, pin_rope, pin_rope_state, pin_conv, pin_l2norm, pin_compose_equals_full]

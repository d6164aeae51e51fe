"""Pins for the fp64 oracle: it is checked against hand-derived values,
closed forms, special cases and invariants before anything is compared to it."""
import json
import math
import os

import numpy as np
import pytest

import kda_inputs
from oracle import kda_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _chain(seed, L, lb=-2.0, K=D, V=D, H=1):
    """Post-activation inputs for the core recurrence."""
    r = _rng(seed)
    qh = _unit(r.standard_normal((L, H, K)))
    kh = _unit(r.standard_normal((L, H, K)))
    v = r.standard_normal((L, H, V))
    lam = lb * r.uniform(0.0, 1.0, (L, H, K))
    beta = r.uniform(0.0, 1.0, (L, H))
    S0 = 0.1 * r.standard_normal((H, K, V))
    return qh, kh, v, lam, beta, S0


# --------------------------------------------------------------------------- golden
def test_golden_two_token_k2v2():
    """Hand-derived two-token example: fixes the decay-then-delta order, the
    inclusive output and the orientation of S (tests/golden/delta_rule_k2v2.json)."""
    gd = json.load(open(os.path.join(GOLD, "delta_rule_k2v2.json")))
    qh = np.asarray(gd["q"])[:, None, :]
    kh = np.asarray(gd["k"])[:, None, :]
    v = np.asarray(gd["v"])[:, None, :]
    lam = np.log(np.asarray(gd["alpha"]))[:, None, :]
    beta = np.asarray(gd["beta"])[:, None]
    S0 = np.asarray(gd["S0"])[None]
    o, S = O.delta_rule_recurrence(qh, kh, v, lam, beta, gd["scale"], S0)
    np.testing.assert_allclose(o[:, 0], gd["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[0], gd["S_final"], rtol=0, atol=1e-12)
    # the chunked form reproduces the same two tokens in one chunk and in two
    for C in (1, 2):
        o2, S2, _ = O.chunked_recurrence(qh[:, 0], kh[:, 0], v[:, 0], lam[:, 0], beta[:, 0], gd["scale"], S0[0], C=C)
        np.testing.assert_allclose(o2, gd["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(S2, gd["S_final"], rtol=0, atol=1e-12)


def test_golden_index_tables():
    gd = json.load(open(os.path.join(GOLD, "index_tables.json")))
    for case in gd["cases"]:
        t = O.index_tables(case["seqlens"], 16, case["seg_chunks"])
        assert list(np.diff(t["seq_chunk_off"])) == case["chunks_per_seq"]
        assert list(t["seq_chunk_off"]) == case["seq_chunk_off"]
        assert list(t["seq_seg_off"]) == case["seq_seg_off"]
        if "chunk_tab" in case:
            assert t["chunk_tab"].tolist() == case["chunk_tab"]
        if "seg_tab" in case:
            assert t["seg_tab"].tolist() == case["seg_tab"]
        for r, row in case.get("seg_rows", {}).items():
            assert t["seg_tab"][int(r)].tolist() == row
        for r, row in case.get("chunk_rows", {}).items():
            assert t["chunk_tab"][int(r)].tolist() == row
        assert t["chunk_tab"].shape[0] == t["seq_chunk_off"][-1]
        assert t["seg_tab"].shape[0] == t["seq_seg_off"][-1]


# --------------------------------------------------------------------------- activations
def test_gate_closed_forms():
    lb = -4.0
    dt = np.zeros((1, D))
    # g + dt_bias = 0 -> sigmoid(0) = 1/2 -> l = lb/2 exactly
    g = np.zeros((3, 1, D))
    assert np.all(O.log_decay(g, np.array([0.7]), dt, lb) == lb / 2)
    # exp(A_log) multiplies (g + dt): A_log = ln 2, g = ln(3)/2 -> sigmoid(ln 3) = 3/4
    g = np.full((1, 1, D), math.log(3.0) / 2)
    np.testing.assert_allclose(O.log_decay(g, np.array([math.log(2.0)]), dt, lb), 0.75 * lb, rtol=1e-15)
    # dt_bias adds to g: g = 0, dt = -ln 3, A_log = 0 -> sigmoid(-ln 3) = 1/4
    np.testing.assert_allclose(O.log_decay(np.zeros((1, 1, D)), np.array([0.0]), np.full((1, D), -math.log(3.0)), lb),
                               0.25 * lb, rtol=1e-15)
    # range (lb, 0] and lb = 0 gives exactly 0
    r = _rng(7)
    lam = O.log_decay(r.standard_normal((50, 2, D)) * 3, r.standard_normal(2), r.standard_normal((2, D)), -5.0)
    assert lam.max() <= 0 and lam.min() >= -5.0
    assert np.all(O.log_decay(r.standard_normal((5, 2, D)), np.zeros(2), np.zeros((2, D)), 0.0) == 0)


def test_sigmoid_and_norm():
    np.testing.assert_allclose(O.sigmoid(np.array([math.log(3.0), 0.0, -math.log(3.0)])), [0.75, 0.5, 0.25], rtol=1e-15)
    assert O.sigmoid(np.array([-1e308]))[0] == 0.0 and O.sigmoid(np.array([1e308]))[0] == 1.0
    x = _rng(3).standard_normal((4, D))
    n = np.linalg.norm(O.l2_normalize(x), axis=-1)
    s = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(n, np.sqrt(s / (s + O.EPS_L2)), rtol=1e-14)
    assert np.all(O.l2_normalize(np.zeros((2, D))) == 0)


def test_widen_and_round():
    bits = kda_inputs.f32_to_bf16_bits(np.array([1.0, -2.5, 3.140625, 1.0 + 2 ** -8], dtype=np.float32))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    np.testing.assert_array_equal(O.widen(bits), [1.0, -2.5, 3.140625, 1.0])
    np.testing.assert_array_equal(O.round_to_bf16(np.array([1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9])), [1.0 + 2 ** -7, 1.0])


# --------------------------------------------------------------------------- special cases of the recurrence
def test_lower_bound_zero_is_textbook_delta_rule():
    """lb = 0 makes every decay exactly 1; the call must then equal the plain
    delta rule S <- S + b k (v - S^T k)^T, o = scale S^T q, written here per head."""
    w = kda_inputs.custom(B=1, T=40, H=2, lower_bound=0.0, scale=0.3, seed=11)
    x = kda_inputs.make_inputs(w)
    outs, finals = O.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                                 x["scale"], x["lower_bound"], x["initial_state"])
    for h in range(2):
        S = O.widen(x["initial_state"][0, h]).T.copy()
        for t in range(40):
            q = O.widen(x["q"][0, t, h])
            k = O.widen(x["k"][0, t, h])
            q = q / math.sqrt(q @ q + 1e-6)
            k = k / math.sqrt(k @ k + 1e-6)
            b = 1.0 / (1.0 + math.exp(-float(O.widen(x["beta"][0, t, h]))))
            S = S + b * np.outer(k, O.widen(x["v"][0, t, h]) - S.T @ k)
            np.testing.assert_allclose(outs[0][t, h], x["scale"] * S.T @ q, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(finals[0, h], S.T, rtol=1e-12, atol=1e-12)


def test_beta_zero_only_decays():
    """b = 0: S_t = Diag(exp(G_t)) S_0 and o_t = scale (Diag(exp G_t) S_0)^T q_t."""
    qh, kh, v, lam, beta, S0 = _chain(5, 30, lb=-0.7, H=2)
    o, S = O.delta_rule_recurrence(qh, kh, v, lam, 0 * beta, 0.5, S0)
    G = np.cumsum(lam, axis=0)
    for t in range(30):
        ref = 0.5 * np.einsum("hk,hkv->hv", qh[t] * np.exp(G[t]), S0)
        np.testing.assert_allclose(o[t], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, np.exp(G[-1])[:, :, None] * S0, rtol=1e-12, atol=1e-16)


def test_beta_zero_through_interface_state_layout():
    """Same closed form through the interface with an asymmetric initial state:
    the state tensor holds S^T ([v][k]), so only column v=3 of o is non-zero."""
    w = kda_inputs.custom(B=1, T=6, H=1, lower_bound=-2.0, scale=0.25, seed=12)
    x = kda_inputs.make_inputs(w)
    x["beta"][:] = kda_inputs.f32_to_bf16_bits(np.full(x["beta"].shape, -3e38, dtype=np.float32))
    st = np.zeros((1, 1, D, D), dtype=np.float32)
    st[0, 0, 3, 9] = 2.0  # element [v=3][k=9] -> S[9][3]
    outs, finals = O.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                                 x["scale"], x["lower_bound"], st)
    q = O.l2_normalize(O.widen(x["q"][0, :, 0]))
    lam = O.log_decay(O.widen(x["g"][0]), x["A_log"], x["dt_bias"], x["lower_bound"])[:, 0]
    G = np.cumsum(lam, axis=0)
    expect = np.zeros((6, D))
    expect[:, 3] = 0.25 * q[:, 9] * np.exp(G[:, 9]) * 2.0
    np.testing.assert_allclose(outs[0][:, 0], expect, rtol=1e-12, atol=1e-15)
    fin = np.zeros((D, D))
    fin[3, 9] = 2.0 * np.exp(G[-1, 9])
    np.testing.assert_allclose(finals[0, 0], fin, rtol=1e-12, atol=1e-15)


def test_unit_key_write_reads_back():
    """b = 1, a = 1, |k| = 1: after token t the memory returns v_t for key k_t."""
    qh, kh, v, lam, beta, S0 = _chain(6, 12, H=1)
    S = S0
    for t in range(12):
        _, S = O.delta_rule_recurrence(qh[t:t + 1], kh[t:t + 1], v[t:t + 1], 0 * lam[t:t + 1],
                                       np.ones((1, 1)), 1.0, S)
        np.testing.assert_allclose(S[0].T @ kh[t, 0], v[t, 0], rtol=0, atol=1e-12)


def test_one_token_from_zero_state():
    """T = 1, S_0 = 0: o = scale sigmoid(b) (k^ . q^) v, through the interface."""
    w = kda_inputs.custom(B=1, T=1, H=3, lower_bound=-5.0, scale=0.7, init_std=None, seed=13)
    x = kda_inputs.make_inputs(w)
    outs, finals = O.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                                 x["scale"], x["lower_bound"], None)
    for h in range(3):
        q = O.widen(x["q"][0, 0, h])
        k = O.widen(x["k"][0, 0, h])
        b = O.widen(x["beta"][0, 0, h])
        vv = O.widen(x["v"][0, 0, h])
        coef = (q @ k) / math.sqrt((q @ q + 1e-6) * (k @ k + 1e-6)) / (1 + math.exp(-b))
        np.testing.assert_allclose(outs[0][0, h], np.float32(0.7) * coef * vv, rtol=1e-12, atol=1e-15)
        # the final state is the rank-one write b k^ v^T, stored as [v][k]
        kn = k / math.sqrt(k @ k + 1e-6)
        np.testing.assert_allclose(finals[0, h], np.outer(vv, kn) / (1 + math.exp(-b)), rtol=1e-12, atol=1e-15)


def test_linearity_and_scale():
    """o and S are jointly linear in (v, S_0); o is degree-1 homogeneous in scale."""
    qh, kh, v1, lam, beta, S01 = _chain(8, 25, H=2)
    _, _, v2, _, _, S02 = _chain(9, 25, H=2)
    o1, s1 = O.delta_rule_recurrence(qh, kh, v1, lam, beta, 0.4, S01)
    o2, s2 = O.delta_rule_recurrence(qh, kh, v2, lam, beta, 0.4, S02)
    o3, s3 = O.delta_rule_recurrence(qh, kh, 2 * v1 - 3 * v2, lam, beta, 0.4, 2 * S01 - 3 * S02)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s3, 2 * s1 - 3 * s2, rtol=1e-10, atol=1e-12)
    o4, s4 = O.delta_rule_recurrence(qh, kh, v1, lam, beta, 1.2, S01)
    np.testing.assert_allclose(o4, 3 * o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(s4, s1)


# --------------------------------------------------------------------------- chunked form
@pytest.mark.parametrize("C", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("lb", [-0.5, -5.0])
def test_chunked_equals_token_form(C, lb):
    L = 37  # not a multiple of any C > 1 above
    qh, kh, v, lam, beta, S0 = _chain(20 + C, L, lb=lb)
    o, S = O.delta_rule_recurrence(qh, kh, v, lam, beta, 0.3, S0)
    oc, Sc, _ = O.chunked_recurrence(qh[:, 0], kh[:, 0], v[:, 0], lam[:, 0], beta[:, 0], 0.3, S0[0], C=C)
    scale_o = np.abs(o).max()
    np.testing.assert_allclose(oc, o[:, 0], rtol=0, atol=1e-11 * scale_o)
    np.testing.assert_allclose(Sc, S[0], rtol=0, atol=1e-11 * np.abs(S).max())


def test_chunked_form_through_interface():
    w = kda_inputs.custom(seqlens=[5, 33, 16], H=2, lower_bound=-5.0, seed=14)
    x = kda_inputs.make_inputs(w)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"], x["scale"], x["lower_bound"],
            x["initial_state"], x["cu_seqlens"])
    o1, f1 = O.kda_forward(*args)
    o2, f2 = O.kda_forward(*args, chunked=16)
    for a, b in zip(o1, o2):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-11)
    np.testing.assert_allclose(f2, f1, rtol=0, atol=1e-11)


def test_chunk_quantities_closed_forms():
    qh, kh, v, lam, beta, _ = _chain(31, 16, lb=-3.0)
    c = O.chunk_quantities(qh[:, 0], kh[:, 0], v[:, 0], lam[:, 0], beta[:, 0], 0.6)
    # decays cancel on the diagonal: Aqk_rr = scale q^_r . k^_r
    np.testing.assert_allclose(np.diag(c["Aqk"]), 0.6 * np.sum(qh[:, 0] * kh[:, 0], axis=1), rtol=1e-12)
    assert np.all(np.triu(c["A"]) == 0) and np.all(np.triu(c["Aqk"], 1) == 0)
    np.testing.assert_allclose(c["gamma_C"], np.exp(lam[:, 0].sum(0)), rtol=1e-12)
    # first row of the WY factors has no correction
    np.testing.assert_allclose(c["W"][0], beta[0, 0] * kh[0, 0] * np.exp(lam[0, 0]), rtol=1e-12)
    np.testing.assert_allclose(c["Ut"][0], beta[0, 0] * v[0, 0], rtol=1e-12)
    # Khat of the last row is the plain key
    np.testing.assert_allclose(c["Khat"][-1], kh[-1, 0], rtol=1e-12)


def test_forward_substitution_matches_solve():
    r = _rng(40)
    for m in (1, 2, 7, 16):
        A = np.tril(r.uniform(-1, 1, (m, m)), -1)
        T = O.forward_substitution_inverse(A)
        np.testing.assert_allclose(T, np.linalg.solve(np.eye(m) + A, np.eye(m)), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(T @ (np.eye(m) + A), np.eye(m), atol=1e-12)
        assert np.all(np.triu(T, 1) == 0) and np.all(np.diag(T) == 1)


# --------------------------------------------------------------------------- invariants of the interface
def test_varlen_equals_separate_calls():
    lens = [17, 1, 40, 16]
    w = kda_inputs.custom(seqlens=lens, H=2, lower_bound=-3.0, seed=15)
    x = kda_inputs.make_inputs(w)
    outs, finals = O.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                                 x["scale"], x["lower_bound"], x["initial_state"], x["cu_seqlens"])
    cu = x["cu_seqlens"]
    for i, L in enumerate(lens):
        sl = slice(cu[i], cu[i + 1])
        o1, f1 = O.kda_forward(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl], x["beta"][:, sl],
                               x["A_log"], x["dt_bias"], x["scale"], x["lower_bound"], x["initial_state"][i:i + 1])
        np.testing.assert_array_equal(o1[0], outs[i])
        np.testing.assert_array_equal(f1[0], finals[i])


def test_state_chaining():
    """fwd(x1 || x2) equals fwd(x2) started from the final state of fwd(x1)."""
    w = kda_inputs.custom(B=1, T=50, H=2, lower_bound=-1.0, seed=16)
    x = kda_inputs.make_inputs(w)
    args = lambda sl: (x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl], x["beta"][:, sl],
                       x["A_log"], x["dt_bias"], x["scale"], x["lower_bound"])
    o, f = O.kda_forward(*args(slice(0, 50)), x["initial_state"])
    o1, f1 = O.kda_forward(*args(slice(0, 21)), x["initial_state"])
    o2, f2 = O.kda_forward(*args(slice(21, 50)), f1)
    np.testing.assert_allclose(np.concatenate([o1[0], o2[0]]), o[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f2, f, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("lb", [0.0, -1.0, -5.0])
def test_segment_merge_is_exact(lb):
    """Pre-scan + merge: M_i S_i + R_i reproduces the serial state at every
    segment boundary (segments of 3 chunks over a 150-token chain)."""
    qh, kh, v, lam, beta, S0 = _chain(50, 150, lb=lb)
    _, _, chunks = O.chunked_recurrence(qh[:, 0], kh[:, 0], v[:, 0], lam[:, 0], beta[:, 0], 0.3, S0[0], keep=True)
    S_serial = [S0[0]]
    for c in chunks:
        S_serial.append(O.chunk_step(c, S_serial[-1])[1])
    S = S0[0]
    for b in range(0, len(chunks), 3):
        M, R = O.segment_transition(chunks[b:b + 3])
        S = O.merge(M, R, S)
        ref = S_serial[min(b + 3, len(chunks))]
        np.testing.assert_allclose(S, ref, rtol=0, atol=1e-10 * max(1.0, np.abs(ref).max()))


def test_input_generator_is_deterministic():
    w = kda_inputs.custom(B=2, T=8, H=2, seed=99)
    a = kda_inputs.make_inputs(w)
    b = kda_inputs.make_inputs(w)
    for key in ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "initial_state"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["q"].dtype == np.uint16 and a["A_log"].dtype == np.float32

"""Pins of the decode oracle's building blocks against closed forms, invariants and special cases.

The pages print no worked example, so every pin here is mathematics: each is
chosen so a plausible slip in oracle.c (a dropped term, a wrong sign or index,
a transposed operand, the wrong RoPE pairing) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
import synth

RNG = np.random.default_rng(1234)


def bf(x):
    return oracle.bf16(np.asarray(x, np.float32))


def f32(bits):
    return synth.bf16_to_f32(np.asarray(bits, np.uint16))


# ------------------------------------------------------------------ bf16
def test_bf16_rounding_nearest_even():
    assert oracle.lib().orc_f32_to_bf16(1.0) == 0x3F80
    # 1 + 2^-8 is exactly halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert oracle.lib().orc_f32_to_bf16(1.0 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even): rounds up to even
    assert oracle.lib().orc_f32_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82
    assert oracle.lib().orc_f32_to_bf16(-2.0) == 0xC000
    for h in (0x0000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F):
        assert oracle.lib().orc_f32_to_bf16(oracle.lib().orc_bf16_to_f32(h)) == h


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    for c in (0.5, 3.0, -2.0):
        x = np.full(64, c, np.float32)
        g = bf(np.linspace(0.5, 1.5, 64))
        y = oracle.rmsnorm(x, g, 1e-6)
        want = f32(g) * c / math.sqrt(c * c + 1e-6)
        np.testing.assert_allclose(y, want, rtol=1e-6)


def test_rmsnorm_known_vector_and_scale_invariance():
    y = oracle.rmsnorm(np.array([3.0, 4.0], np.float32), None, 0.0)
    np.testing.assert_allclose(y, np.array([3, 4]) / math.sqrt(12.5), rtol=1e-7)
    x = RNG.standard_normal(512).astype(np.float32)
    np.testing.assert_allclose(oracle.rmsnorm(x, None, 1e-6), oracle.rmsnorm(8 * x, None, 1e-6), rtol=1e-5)


# ------------------------------------------------------------------ GEMV
def test_matvec_small_integers_exact_and_orientation():
    rows, cols = 37, 300                       # not square: a transposed operand cannot pass
    Wi = RNG.integers(-8, 9, size=(rows, cols))
    xi = RNG.integers(-8, 9, size=cols)
    y = oracle.matvec(bf(Wi), xi.astype(np.float32))
    want = [sum(int(Wi[r, k]) * int(xi[k]) for k in range(cols)) for r in range(rows)]
    assert y.tolist() == [float(v) for v in want]


# ------------------------------------------------------------------ RoPE
def test_rope_identity_at_position_zero():
    u = RNG.standard_normal(128).astype(np.float32)
    assert np.array_equal(oracle.rope(u, 0, 1e4), u)


def test_rope_rotate_half_pairing_and_frequency():
    # d = 4: pairs (0, 2) at angle pos * base^0 and (1, 3) at angle pos * base^(-1/2)
    base, pos = 100.0, 3
    u = np.array([1.0, 1.0, 0.0, 0.0], np.float32)
    y = oracle.rope(u, pos, base)
    t0, t1 = pos * 1.0, pos * base ** -0.5
    np.testing.assert_allclose(y, [math.cos(t0), math.cos(t1), math.sin(t0), math.sin(t1)], atol=1e-7)


def test_rope_preserves_pair_norms_and_relative_positions():
    d = 128
    q = RNG.standard_normal(d).astype(np.float32)
    k = RNG.standard_normal(d).astype(np.float32)
    y = oracle.rope(q, 777, 5e5)
    h = d // 2
    np.testing.assert_allclose(y[:h] ** 2 + y[h:] ** 2, q[:h] ** 2 + q[h:] ** 2, rtol=1e-5)
    a = np.dot(oracle.rope(q, 10, 1e4).astype(np.float64), oracle.rope(k, 3, 1e4))
    b = np.dot(oracle.rope(q, 110, 1e4).astype(np.float64), oracle.rope(k, 103, 1e4))
    assert abs(a - b) < 1e-4 * (1 + abs(a))


# ------------------------------------------------------------------ attention
def test_attention_single_key_returns_its_value():
    d = 128
    q = RNG.standard_normal(d).astype(np.float32)
    K = bf(RNG.standard_normal((1, d)))
    V = bf(RNG.standard_normal((1, d)))
    o, p = oracle.attend(q, K, V)
    assert np.array_equal(o, f32(V[0]))
    assert p.tolist() == [1.0]


def test_attention_softmax_normalised_and_two_key_closed_form():
    d, n = 64, 50
    q = RNG.standard_normal(d).astype(np.float32)
    K = bf(RNG.standard_normal((n, d)))
    V = bf(RNG.standard_normal((n, d)))
    o, p = oracle.attend(q, K, V)
    assert (p >= 0).all() and abs(p.sum() - 1.0) < 1e-12
    # two keys: p0 = 1 / (1 + exp(s1 - s0)), s_j = q.k_j / sqrt(d)
    o2, p2 = oracle.attend(q, K[:2], V[:2])
    s = [float(np.dot(q.astype(np.float64), f32(K[j]))) / math.sqrt(d) for j in range(2)]
    assert abs(p2[0] - 1.0 / (1.0 + math.exp(s[1] - s[0]))) < 1e-12
    np.testing.assert_allclose(o2, p2[0] * f32(V[0]) + p2[1] * f32(V[1]), rtol=1e-6, atol=1e-7)


def test_attention_identical_keys_mean_dominant_key_and_ones():
    d, n = 128, 33
    q = RNG.standard_normal(d).astype(np.float32)
    K = np.repeat(bf(RNG.standard_normal((1, d))), n, axis=0)
    V = bf(RNG.standard_normal((n, d)))
    o, _ = oracle.attend(q, K, V)
    np.testing.assert_allclose(o, f32(V).astype(np.float64).mean(axis=0), rtol=1e-5, atol=1e-6)
    # one key scoring 50 above all others returns (to fp32 precision) that key's value
    q1 = np.zeros(d, np.float32); q1[0] = 1.0
    Kd = np.zeros((n, d), np.float32); Kd[7, 0] = 50.0 * math.sqrt(d)
    o, p = oracle.attend(q1, bf(Kd), V)
    assert p[7] >= 1 - 1e-15 and np.delete(p, 7).max() < 1e-20
    np.testing.assert_allclose(o, f32(V[7]), rtol=1e-6)
    o, _ = oracle.attend(q, bf(RNG.standard_normal((n, d))), bf(np.ones((n, d))))
    np.testing.assert_allclose(o, 1.0, rtol=1e-6)


def test_attention_shift_invariance():
    # adding the same component along q to every key shifts all scores by one constant
    d, n = 64, 20
    q = np.zeros(d, np.float32); q[5] = 2.0
    K = RNG.standard_normal((n, d)); K[:, 5] = np.round(K[:, 5] * 4) / 4
    V = bf(RNG.standard_normal((n, d)))
    o1, p1 = oracle.attend(q, bf(K), V)
    K2 = K.copy(); K2[:, 5] += 3.0
    o2, p2 = oracle.attend(q, bf(K2), V)
    np.testing.assert_allclose(p1, p2, rtol=1e-9)


# ------------------------------------------------------------------ SwiGLU pieces
def test_silu_and_sigmoid():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert oracle.sigmoid(0.0) == 0.5


# ------------------------------------------------------------------ conv
def test_conv_taps_and_rolling_state():
    C, W = 6, 4
    st = RNG.standard_normal((C, W - 1)).astype(np.float32)
    u = RNG.standard_normal(C).astype(np.float32)
    # one-hot taps pick the oldest cached input / the current input
    w_old = np.zeros((C, W)); w_old[:, 0] = 1
    y, st2 = oracle.conv_step(u, bf(w_old), st)
    np.testing.assert_allclose(y, [oracle.silu(float(v)) for v in st[:, 0]], rtol=1e-6)
    w_cur = np.zeros((C, W)); w_cur[:, W - 1] = 1
    y, st2 = oracle.conv_step(u, bf(w_cur), st)
    np.testing.assert_allclose(y, [oracle.silu(float(v)) for v in u], rtol=1e-6)
    # the state is the last W-1 inputs, bitwise, oldest first
    assert np.array_equal(st2[:, :-1], st[:, 1:]) and np.array_equal(st2[:, -1], u)


def test_conv_matches_full_sequence_convolution():
    C, W, T = 5, 4, 12
    w = bf(RNG.standard_normal((C, W)))
    U = RNG.standard_normal((T, C)).astype(np.float32)
    st = np.zeros((C, W - 1), np.float32)
    ys = []
    for t in range(T):
        y, st = oracle.conv_step(U[t], w, st)
        ys.append(y)
    for c in range(C):
        full = np.convolve(U[:, c].astype(np.float64), f32(w[c])[::-1].astype(np.float64))[:T]  # zero left pad
        pre = [oracle.silu(float(v)) for v in full]
        np.testing.assert_allclose([ys[t][c] for t in range(T)], pre, rtol=2e-6, atol=1e-7)
    # after every step the state holds the last W-1 inputs
    assert np.array_equal(st.T, U[-(W - 1):])


# ------------------------------------------------------------------ delta rule
def _unit(v):
    return (v / np.linalg.norm(v)).astype(np.float32)


def test_delta_from_zero_state():
    dk, dv = 16, 12
    q = RNG.standard_normal(dk).astype(np.float32)
    k = _unit(RNG.standard_normal(dk))
    v = RNG.standard_normal(dv).astype(np.float32)
    st, o = oracle.delta_step(np.zeros((dv, dk)), q, k, v, 0.7, 0.4)
    np.testing.assert_allclose(st, 0.4 * np.outer(v, k), rtol=1e-6)          # S' = beta k v^T
    np.testing.assert_allclose(o, 0.4 * float(np.dot(k, q)) * v, rtol=1e-5)  # o = beta (k.q) v


def test_delta_retrieval_with_unit_gates():
    dk, dv = 32, 32
    st0 = RNG.standard_normal((dv, dk)).astype(np.float32)
    k = _unit(RNG.standard_normal(dk))
    v = RNG.standard_normal(dv).astype(np.float32)
    st, _ = oracle.delta_step(st0, np.zeros(dk), k, v, 1.0, 1.0)
    np.testing.assert_allclose(st.astype(np.float64) @ k, v, atol=2e-5)     # S'^T k = v


def test_delta_zero_gate_pins_update_order():
    dk, dv = 8, 8
    st0 = RNG.standard_normal((dv, dk)).astype(np.float32)
    k = _unit(RNG.standard_normal(dk))
    v = RNG.standard_normal(dv).astype(np.float32)
    lit, _ = oracle.delta_step(st0, np.zeros(dk), k, v, 0.0, 0.5, decay_first=0)
    dec, _ = oracle.delta_step(st0, np.zeros(dk), k, v, 0.0, 0.5, decay_first=1)
    kS = st0.astype(np.float64) @ k                                          # (k^T S)_j
    np.testing.assert_allclose(lit, 0.5 * np.outer(v - kS, k), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dec, 0.5 * np.outer(v, k), rtol=1e-6)


def test_delta_matches_product_form():
    dk, dv, T = 8, 6, 7
    st = RNG.standard_normal((dv, dk)).astype(np.float32)
    S0 = st.T.astype(np.float64)
    ks = [_unit(RNG.standard_normal(dk)) for _ in range(T)]
    vs = [RNG.standard_normal(dv).astype(np.float32) for _ in range(T)]
    gs = RNG.uniform(0.2, 0.95, T)
    bs = RNG.uniform(0.1, 0.9, T)
    for t in range(T):
        st, _ = oracle.delta_step(st, np.zeros(dk), ks[t], vs[t], gs[t], bs[t])
    # S_T = sum_t (A_T..A_{t+1}) b_t k_t v_t^T + (A_T..A_1) S_0,  A_s = g_s I - b_s k_s k_s^T
    A = [gs[s] * np.eye(dk) - bs[s] * np.outer(ks[s], ks[s]) for s in range(T)]
    S = np.zeros((dk, dv))
    for t in range(T):
        Pm = np.eye(dk)
        for s in range(T - 1, t, -1):
            Pm = Pm @ A[s]
        S += Pm @ (bs[t] * np.outer(ks[t], vs[t]))
    Pm = np.eye(dk)
    for s in range(T - 1, -1, -1):
        Pm = Pm @ A[s]
    S += Pm @ S0
    np.testing.assert_allclose(st.T, S, rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------------ greedy
def test_argmax_ties_to_lowest_index():
    v = np.array([0.1, 0.7, 0.3, 0.7, 0.7], np.float32)
    assert oracle.argmax(v) == 1
    assert oracle.argmax(np.zeros(10, np.float32)) == 0

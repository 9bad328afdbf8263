"""Pins for the fp64 oracle: closed forms, invariants and special cases that
the mathematics fixes, chosen so that a dropped term, a wrong sign, a wrong
index or a transposed operand anywhere in the oracle fails one of them.

The recurrence pinned is the gated delta rule of Yang, Kautz and
Hatamizadeh, "Gated Delta Networks" (ICLR 2025):
    S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.chunked import chunk_affine_map, delta_rule_chunked


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---- scalar pieces --------------------------------------------------------

def test_silu_limits_and_symmetry():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(50.0) - 50.0) < 1e-18 * 50 + 1e-15
    assert abs(oracle.silu(-50.0)) < 1e-19
    # SiLU(x) - SiLU(-x) = x  (x*s(x) - (-x)*s(-x) = x (s(x)+s(-x)) = x)
    for x in (-3.0, -0.7, 0.3, 2.5):
        assert abs(oracle.silu(x) - oracle.silu(-x) - x) < 1e-15


def test_softplus_identities():
    assert abs(oracle.softplus(0.0) - math.log(2.0)) < 1e-16
    for x in (-30.0, -2.0, -0.1, 0.0, 0.4, 3.0, 30.0):
        # softplus(x) - softplus(-x) = x
        assert abs(oracle.softplus(x) - oracle.softplus(-x) - x) < 1e-14
        assert oracle.softplus(x) > 0.0
    assert abs(oracle.softplus(800.0) - 800.0) < 1e-12       # no overflow
    # d/dx softplus = sigmoid (central difference)
    for x in (-1.5, 0.2, 2.0):
        h = 1e-5
        fd = (oracle.softplus(x + h) - oracle.softplus(x - h)) / (2 * h)
        assert abs(fd - oracle.sigmoid(x)) < 1e-9


def test_sigmoid_identities():
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(oracle.sigmoid(40.0) - 1.0) < 1e-17
    assert 0.0 < oracle.sigmoid(-40.0) < 5e-18
    for x in (-4.0, -0.3, 1.7):
        assert abs(oracle.sigmoid(x) + oracle.sigmoid(-x) - 1.0) < 1e-15


def test_gates_special_cases():
    # a + dt_bias = 0  =>  g = -e^{A_log} ln 2
    g, beta = oracle.gates(0.3, 0.0, math.log(5.0), -0.3)
    assert abs(g + 5.0 * math.log(2.0)) < 1e-14
    assert beta == 0.5
    # A_log = -100: g ~ -4e-44 so exp(g) is exactly 1 in fp64
    g, _ = oracle.gates(1.0, 0.0, -100.0, 0.0)
    assert g < 0.0 and math.exp(g) == 1.0
    # decay is monotone in A_log and in a, and never positive
    g1, _ = oracle.gates(0.5, 0.0, 0.0, 0.1)
    g2, _ = oracle.gates(0.5, 0.0, 1.0, 0.1)
    g3, _ = oracle.gates(1.5, 0.0, 1.0, 0.1)
    assert g2 < g1 < 0.0 and g3 < g2


# ---- norms ----------------------------------------------------------------

def test_l2norm_onehot_and_invariant():
    x = np.zeros(16)
    x[5] = 8.0
    y = oracle.l2norm(x, 1e-6)
    assert np.count_nonzero(y) == 1 and abs(y[5] - 8.0 / math.sqrt(64 + 1e-6)) < 1e-15
    x = _rng(0).standard_normal(37)
    eps = 0.3
    y = oracle.l2norm(x, eps, scale=2.5)
    n2 = float(x @ x)
    assert abs(float(y @ y) - 6.25 * n2 / (n2 + eps)) < 1e-12
    # direction preserved
    assert np.allclose(y / np.linalg.norm(y), x / np.linalg.norm(x), atol=1e-15)


def test_rmsnorm_gate_closed_forms():
    o = _rng(1).standard_normal(64)
    w = np.ones(64)
    z = np.full(64, 40.0)
    eps = 1e-3
    y = oracle.rmsnorm_gate(o, z, w, eps)
    m = float(np.mean(o * o))
    silu40 = 40.0 / (1.0 + math.exp(-40.0))
    rms_y = math.sqrt(float(np.mean(y * y)))
    assert abs(rms_y / silu40 - math.sqrt(m / (m + eps))) < 1e-14
    # scale invariance in o (eps -> 0 limit) and elementwise w
    w2 = _rng(2).standard_normal(64)
    z2 = _rng(3).standard_normal(64)
    y1 = oracle.rmsnorm_gate(o, z2, w2, 0.0)
    y2 = oracle.rmsnorm_gate(7.0 * o, z2, w2, 0.0)
    assert np.allclose(y1, y2, rtol=1e-14, atol=1e-15)
    # zero gate -> zero output (SiLU(0) = 0)
    assert np.all(oracle.rmsnorm_gate(o, np.zeros(64), w2, eps) == 0.0)


def test_rmsnorm_gate_weight_is_elementwise():
    """The norm weight scales each output element by its own entry: the
    output is linear in w element by element, y(w) = w (.) y(1), so dropping
    w, broadcasting one entry, or shifting its index all fail here."""
    n = 48
    o = _rng(4).standard_normal(n)
    z = _rng(5).standard_normal(n)
    eps = 1e-6
    y1 = oracle.rmsnorm_gate(o, z, np.ones(n), eps)
    # a non-uniform weight, every entry distinct and of both signs
    w = np.linspace(-1.5, 2.5, n)
    yw = oracle.rmsnorm_gate(o, z, w, eps)
    assert np.allclose(yw, w * y1, rtol=1e-15, atol=0)
    # a one-hot weight keeps exactly one element, the others are exactly 0
    for j in (0, 17, n - 1):
        e = np.zeros(n)
        e[j] = 3.0
        ye = oracle.rmsnorm_gate(o, z, e, eps)
        assert np.all(ye[np.arange(n) != j] == 0.0)
        assert ye[j] == pytest.approx(3.0 * y1[j], rel=1e-15)
    # the closed form for w = 1, elementwise: o / rms(o) * SiLU(z)
    rms = math.sqrt(float(np.mean(o * o)) + eps)
    silu_z = z / (1.0 + np.exp(-z))
    assert np.allclose(y1, o / rms * silu_z, rtol=1e-14, atol=0)


# ---- the recurrence -------------------------------------------------------

def test_beta0_g0_leaves_state_unchanged():
    r = _rng(4)
    T, dk, dv = 9, 6, 5
    S0 = r.standard_normal((dv, dk))
    q, k = r.standard_normal((T, dk)), _unit_rows(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    o, S = oracle.delta_rule(q, k, v, np.zeros(T), np.zeros(T), S0)
    assert np.array_equal(S, S0)
    assert np.allclose(o, q @ S0.T, rtol=0, atol=1e-14)


def test_beta0_pure_decay_nonsymmetric_state():
    r = _rng(5)
    T, dk, dv = 7, 3, 8
    S0 = r.standard_normal((dv, dk))
    q, k = r.standard_normal((T, dk)), r.standard_normal((T, dk))
    v = r.standard_normal((T, dv))
    g = -r.uniform(0.0, 0.5, T)
    o, S = oracle.delta_rule(q, k, v, g, np.zeros(T), S0)
    gam = np.cumsum(g)
    assert np.allclose(S, math.exp(gam[-1]) * S0, rtol=1e-14, atol=0)
    assert np.allclose(o, np.exp(gam)[:, None] * (q @ S0.T), rtol=1e-13, atol=1e-15)


def test_g0_beta1_unit_key_writes_value():
    r = _rng(6)
    T, dk, dv = 12, 8, 6
    k = _unit_rows(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    q = r.standard_normal((T, dk))
    S = r.standard_normal((dv, dk))
    for t in range(T):
        _, S = oracle.delta_rule(q[t:t + 1], k[t:t + 1], v[t:t + 1],
                                 np.zeros(1), np.ones(1), S)
        assert np.allclose(S @ k[t], v[t], rtol=0, atol=1e-14)


def test_retrieval_invariant_random_gates():
    """For unit k: S_t k_t = e^{g}(1 - beta) S_{t-1} k_t + beta v_t."""
    r = _rng(7)
    T, dk, dv = 20, 5, 7
    k = _unit_rows(r.standard_normal((T, dk)))
    v, q = r.standard_normal((T, dv)), r.standard_normal((T, dk))
    g = -r.uniform(0.0, 2.0, T)
    beta = r.uniform(0.0, 1.0, T)
    S = r.standard_normal((dv, dk))
    for t in range(T):
        Sprev = S
        o, S = oracle.delta_rule(q[t:t + 1], k[t:t + 1], v[t:t + 1],
                                 g[t:t + 1], beta[t:t + 1], Sprev)
        lhs = S @ k[t]
        rhs = math.exp(g[t]) * (1 - beta[t]) * (Sprev @ k[t]) + beta[t] * v[t]
        assert np.allclose(lhs, rhs, rtol=0, atol=1e-13)
        # directions orthogonal to k are only decayed
        w = r.standard_normal(dk)
        w -= (w @ k[t]) * k[t]
        assert np.allclose(S @ w, math.exp(g[t]) * (Sprev @ w), atol=1e-13)
        # output is the read-out of the new state
        assert np.allclose(o[0], S @ q[t], atol=1e-14)


def test_associative_recall_onehot():
    r = _rng(8)
    dk, dv, T = 6, 4, 25
    slots = r.integers(0, dk, T)
    k = np.eye(dk)[slots]
    v = r.standard_normal((T, dv))
    qslots = r.integers(0, dk, T)
    q = np.eye(dk)[qslots]
    S0 = r.standard_normal((dv, dk))
    o, S = oracle.delta_rule(q, k, v, np.zeros(T), np.ones(T), S0)
    for t in range(T):
        written = [s for s in range(t + 1) if slots[s] == qslots[t]]
        exp = v[written[-1]] if written else S0[:, qslots[t]]
        assert np.allclose(o[t], exp, atol=1e-15)


def test_single_token_from_zero_state():
    r = _rng(9)
    dk, dv = 7, 3
    q, k = r.standard_normal((1, dk)), r.standard_normal((1, dk))
    v = r.standard_normal((1, dv))
    g, beta = np.array([-0.8]), np.array([0.37])
    o, S = oracle.delta_rule(q, k, v, g, beta, None)
    assert np.allclose(o[0], beta[0] * float(k[0] @ q[0]) * v[0], atol=1e-15)
    assert np.allclose(S, beta[0] * np.outer(v[0], k[0]), atol=1e-15)


@pytest.mark.parametrize("T,dk,dv,C", [(37, 6, 5, 8), (40, 4, 4, 16),
                                       (5, 3, 9, 16), (33, 8, 2, 1),
                                       (64, 5, 6, 64), (17, 2, 3, 4)])
def test_chunked_equals_sequential(T, dk, dv, C):
    r = _rng(100 + T + C)
    q = r.standard_normal((T, dk))
    k = _unit_rows(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    g = -np.exp(r.uniform(-3, 1.5, T))
    beta = r.uniform(0, 1, T)
    S0 = r.standard_normal((dv, dk))
    o1, S1 = oracle.delta_rule(q, k, v, g, beta, S0)
    o2, S2 = delta_rule_chunked(q, k, v, g, beta, S0, C=C)
    assert np.max(np.abs(o1 - o2)) < 1e-12 * max(1, np.max(np.abs(o1)))
    assert np.max(np.abs(S1 - S2)) < 1e-12 * max(1, np.max(np.abs(S1)))


def test_chunked_strong_decay_underflow():
    """Cumulative decay far below exp(-745): only differences are formed."""
    r = _rng(11)
    T, dk, dv = 48, 4, 3
    q = r.standard_normal((T, dk))
    k = _unit_rows(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    g = np.full(T, -40.0)
    beta = r.uniform(0, 1, T)
    o1, S1 = oracle.delta_rule(q, k, v, g, beta, None)
    o2, S2 = delta_rule_chunked(q, k, v, g, beta, None, C=48)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(S2))
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(S1, S2, atol=1e-12)


def test_chunk_map_is_affine():
    r = _rng(12)
    L, dk, dv = 11, 5, 4
    q = r.standard_normal((L, dk))
    k = _unit_rows(r.standard_normal((L, dk)))
    v = r.standard_normal((L, dv))
    g = -r.uniform(0, 1, L)
    beta = r.uniform(0, 1, L)
    P, R = chunk_affine_map(k, v, g, beta)
    for _ in range(3):
        S0 = r.standard_normal((dv, dk))
        _, S = oracle.delta_rule(q, k, v, g, beta, S0)
        assert np.allclose(S, S0 @ P.T + R, atol=1e-13)

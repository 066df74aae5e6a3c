"""Pins of the KDA oracle against what the LeapQuant page fixes (section "The state,
from the update rule up": eq. 1 with a per-key-channel decay, and KDA's own form
(I - beta k k^T) Diag(alpha) S + beta k v^T, which the page says expands to it) and
against exact arithmetic.

Each test would fail under a plausible slip in ``oracle.kda``: the decay missing
from the correction (S k instead of S (alpha o k)), the decay on value channels
instead of key channels, a transposed state, or an exclusive read-out."""
from fractions import Fraction

import numpy as np

from oracle import gdn, kda


def _rand(rng, N, T, d, unit=True):
    q = rng.standard_normal((N, T, d))
    k = rng.standard_normal((N, T, d))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, T, d))
    a = 1 / (1 + np.exp(-rng.normal(2, 1, (N, T, d))))
    b = 1 / (1 + np.exp(-rng.normal(0, 1, (N, T))))
    return q, k, v, a, b


def test_exact_rational_against_kda_own_form():
    """Brute force in exact rationals on 4x4 states through KDA's own matrices in
    the page's orientation (keys index rows): S_t = (I - b k k^T) Diag(a) S + b k v^T,
    o_t = S_t^T q_t. The oracle (eq. 1 / eq. 3 in the transposed layout) must agree
    to fp64 rounding."""
    rng = np.random.default_rng(11)
    d, T = 4, 8

    def rat(x):
        return Fraction(int(round(x * 16)), 16)

    q = [[rat(x) for x in rng.standard_normal(d)] for _ in range(T)]
    k = [[rat(x) for x in rng.standard_normal(d)] for _ in range(T)]
    v = [[rat(x) for x in rng.standard_normal(d)] for _ in range(T)]
    a = [[Fraction(int(rng.integers(9, 16)), 16) for _ in range(d)] for _ in range(T)]
    b = [Fraction(int(rng.integers(1, 16)), 16) for _ in range(T)]
    S = [[rat(x) for x in rng.standard_normal(d)] for _ in range(d)]      # page orientation [k][v]
    S0_page = [row[:] for row in S]
    outs = []
    for t in range(T):
        DS = [[a[t][i] * S[i][j] for j in range(d)] for i in range(d)]        # Diag(a) S
        kDS = [sum(k[t][i] * DS[i][j] for i in range(d)) for j in range(d)]   # k^T Diag(a) S
        S = [[DS[i][j] - b[t] * k[t][i] * kDS[j] + b[t] * k[t][i] * v[t][j] for j in range(d)]
             for i in range(d)]
        outs.append([sum(S[i][j] * q[t][i] for i in range(d)) for j in range(d)])
    f = lambda M: np.array([[float(x) for x in r] for r in M])
    o, Sd = kda.kda_recurrent(f(q)[None], f(k)[None], f(v)[None], f(a)[None],
                              np.array([[float(x) for x in b]]), f(S0_page).T[None])
    np.testing.assert_allclose(o[0], f(outs), rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sd[0], f(S).T, rtol=0, atol=1e-13)


def test_eq1_form_equals_kda_own_form_in_fp64():
    rng = np.random.default_rng(3)
    q, k, v, a, b = _rand(rng, 2, 7, 6)
    S0 = rng.standard_normal((2, 6, 6))
    o1, S1 = kda.kda_recurrent(q, k, v, a, b, S0)
    o2, S2 = kda.kda_recurrent_explicit(q, k, v, a, b, S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-12)


def test_equal_channel_decays_are_gated_deltanet():
    """A decay vector with every entry alpha_t is GDN's scalar decay (the GDN
    oracle is pinned on its own)."""
    rng = np.random.default_rng(4)
    q, k, v, _, b = _rand(rng, 3, 10, 8)
    a = 1 / (1 + np.exp(-rng.normal(2, 1, (3, 10))))
    S0 = rng.standard_normal((3, 8, 8))
    o1, S1 = kda.kda_recurrent(q, k, v, np.repeat(a[:, :, None], 8, axis=2), b, S0)
    o2, S2 = gdn.gdn_recurrent(q, k, v, a, b, S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-12)


def test_beta_zero_is_per_key_channel_decay():
    """beta = 0: S_t = S_0 Diag(prod_{i<=t} alpha_i), each key column decaying at its
    own rate, and o_t = S_t q_t."""
    rng = np.random.default_rng(5)
    N, T, d = 2, 9, 6
    q, k, v, a, _ = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    o, ST = kda.kda_recurrent(q, k, v, a, np.zeros((N, T)), S0)
    G = np.cumprod(a, axis=1)                          # [N][T][d_k]
    np.testing.assert_allclose(ST, S0 * G[:, -1][:, None, :], rtol=1e-13, atol=0)
    for t in range(T):
        St = S0 * G[:, t][:, None, :]
        np.testing.assert_allclose(o[:, t], np.einsum("nvk,nk->nv", St, q[:, t]), rtol=0, atol=1e-12)


def test_beta_one_unit_key_stores_value_along_key():
    """beta = 1 with a unit key: S_t k_t = S_{t-1}(alpha o k) + u (k.k) = v_t, so
    reading with q = k returns v, whatever the per-channel decays."""
    rng = np.random.default_rng(6)
    N, T, d = 3, 12, 16
    _, k, v, a, _ = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    o, _ = kda.kda_recurrent(k, k, v, a, np.ones((N, T)), S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_unit_decay_is_the_delta_rule():
    """alpha = 1 on every channel: S_t = S_{t-1} + beta (v - S_{t-1} k) k^T."""
    rng = np.random.default_rng(8)
    N, T, d = 2, 6, 5
    q, k, v, _, b = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    o, ST = kda.kda_recurrent(q, k, v, np.ones((N, T, d)), b, S0)
    S = S0.copy()
    for t in range(T):
        u = b[:, t][:, None] * (v[:, t] - np.einsum("nvk,nk->nv", S, k[:, t]))
        S = S + u[:, :, None] * k[:, t][:, None, :]
        np.testing.assert_allclose(o[:, t], np.einsum("nvk,nk->nv", S, q[:, t]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ST, S, rtol=0, atol=1e-12)


def test_chunk_form_equals_recurrence():
    """The UT-transform chunk reading with per-channel decays inside the products
    equals the token-by-token recurrence for several chunk sizes, from zero and
    from a nonzero state."""
    rng = np.random.default_rng(31)
    N, T, d = 2, 64, 16
    q, k, v, a, b = _rand(rng, N, T, d)
    S0 = 0.3 * rng.standard_normal((N, d, d))
    o_r, S_r = kda.kda_recurrent(q, k, v, a, b, S0)
    for C in (1, 16, 64):
        o_c, S_c = kda.kda_chunk_wy(q, k, v, a, b, S0, chunk=C)
        np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-11 * np.abs(o_r).max())
        np.testing.assert_allclose(S_c, S_r, rtol=0, atol=1e-11 * np.abs(S_r).max())

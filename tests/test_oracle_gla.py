"""Pins of the GLA oracle against the ZeCO summary page's statements and
against the textbook masked form of linear attention."""
import numpy as np
import pytest

from oracle import gla


def _rand(rng, N, T, d, mu=3.0):
    q, k, v = rng.standard_normal((3, N, T, d))
    lg = -np.log1p(np.exp(-rng.normal(mu, 1, (N, T, d))))     # logsigmoid
    return q, k, v, lg


def test_zero_gates_is_causal_linear_attention():
    """g = 0: o_t = sum_{j<=t} (q_t . k_j) v_j + S0 q_t, i.e. tril(Q K^T) V + Q S0^T."""
    rng = np.random.default_rng(1)
    N, T, d = 2, 20, 8
    q, k, v, _ = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    o, S = gla.gla_recurrent(q, k, v, np.zeros((N, T, d)), S0)
    ref = np.tril(np.einsum("ntk,njk->ntj", q, k)) @ v + np.einsum("ntk,nvk->ntv", q, S0)
    np.testing.assert_allclose(o, ref, atol=1e-12)
    np.testing.assert_allclose(S, S0 + np.einsum("ntv,ntk->nvk", v, k), atol=1e-12)


def test_incoming_state_decomposition_eq6():
    """ZeCO eq. 6: the state from S0 equals exp(sum g) o S0 (key columns) plus
    the state from zero; outputs differ by (q_t o exp(b_t)) read through S0."""
    rng = np.random.default_rng(2)
    N, T, d = 2, 48, 8
    q, k, v, lg = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    o1, S1 = gla.gla_recurrent(q, k, v, lg, S0)
    o0, Sz = gla.gla_recurrent(q, k, v, lg, None)
    b = np.cumsum(lg, axis=1)
    np.testing.assert_allclose(S1, np.exp(b[:, -1])[:, None, :] * S0 + Sz, atol=1e-12)
    np.testing.assert_allclose(o1, o0 + np.einsum("ntk,nvk->ntv", q * np.exp(b), S0), atol=1e-12)


def test_decay_acts_on_key_columns():
    rng = np.random.default_rng(3)
    N, T, d = 1, 5, 6
    lg = -rng.uniform(0.1, 1.0, (N, T, d))
    S0 = rng.standard_normal((N, d, d))
    j = 2
    q = np.zeros((N, T, d))
    q[..., j] = 1.0
    o, _ = gla.gla_recurrent(q, np.zeros((N, T, d)), np.zeros((N, T, d)), lg, S0)
    b = np.cumsum(lg, axis=1)
    np.testing.assert_allclose(o[0], np.exp(b[0, :, j])[:, None] * S0[0][:, j][None, :], atol=1e-13)


def test_single_token_from_zero():
    rng = np.random.default_rng(4)
    q, k, v, lg = _rand(rng, 1, 1, 7)
    o, S = gla.gla_recurrent(q, k, v, lg, None)
    np.testing.assert_allclose(o[0, 0], v[0, 0] * (k[0, 0] @ q[0, 0]), atol=1e-13)
    np.testing.assert_allclose(S[0], np.outer(v[0, 0], k[0, 0]), atol=1e-14)


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunk_form_equals_recurrence(C):
    rng = np.random.default_rng(5 + C)
    N, T, d = 2, 128, 16
    q, k, v, lg = _rand(rng, N, T, d)
    S0 = 0.1 * rng.standard_normal((N, d, d))
    o1, S1 = gla.gla_recurrent(q, k, v, lg, S0)
    o2, S2 = gla.gla_chunk(q, k, v, lg, S0, chunk=C)
    scale = np.abs(o1).max()
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-12 * np.abs(S1).max())


def test_printed_intra_chunk_key_scaling_is_not_the_recurrence():
    """The section prints the intra-chunk keys as K o Gamma; with that form the
    chunk output is far from the recurrence, which is why the K / Lambda reading
    (the forward algorithm's) is used."""
    rng = np.random.default_rng(6)
    N, T, d, C = 1, 64, 8, 64
    q, k, v, lg = _rand(rng, N, T, d, mu=1.0)
    o1, _ = gla.gla_recurrent(q, k, v, lg, None)
    b = np.cumsum(lg[:, :C], axis=1)
    Qt = q * np.exp(b)
    Kg = k * np.exp(b[:, -1:, :] - b)
    A = np.einsum("nrk,njk->nrj", Qt, Kg) * np.tril(np.ones((C, C)))
    o_printed = A @ v
    assert np.abs(o_printed - o1).max() > 0.1 * np.abs(o1).max()


def test_shards_chain_like_one_call():
    rng = np.random.default_rng(7)
    N, T, d = 2, 96, 8
    q, k, v, lg = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    o, S = gla.gla_recurrent(q, k, v, lg, S0)
    h = 32
    oa, Sa = gla.gla_recurrent(q[:, :h], k[:, :h], v[:, :h], lg[:, :h], S0)
    ob, Sb = gla.gla_recurrent(q[:, h:], k[:, h:], v[:, h:], lg[:, h:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, atol=1e-12)
    np.testing.assert_allclose(Sb, S, atol=1e-12)

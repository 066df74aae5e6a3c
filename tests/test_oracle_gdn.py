"""Pins of the Gated DeltaNet oracle against what the LeapQuant page fixes
(section "The state, from the update rule up") and against exact arithmetic.

Each test would fail under a plausible slip in ``oracle.gdn``: a dropped decay,
the decay on the wrong term, a sign flip in the erase, a transposed state, an
exclusive instead of inclusive read-out, or a wrong chunk-form index."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gdn


def _rand(rng, N, T, d, unit=True):
    q = rng.standard_normal((N, T, d))
    k = rng.standard_normal((N, T, d))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, T, d))
    a = 1 / (1 + np.exp(-rng.normal(2, 1, (N, T))))
    b = 1 / (1 + np.exp(-rng.normal(0, 1, (N, T))))
    return q, k, v, a, b


def test_expanded_equals_explicit_matrix_form():
    rng = np.random.default_rng(1)
    q, k, v, a, b = _rand(rng, 3, 9, 6)
    S0 = rng.standard_normal((3, 6, 6))
    o1, S1 = gdn.gdn_recurrent(q, k, v, a, b, S0)
    o2, S2 = gdn.gdn_recurrent_explicit(q, k, v, a, b, S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-12)


def test_exact_rational_against_page_dk_by_dv_form():
    """Brute force in exact rationals on 4x4 states, written in the page's own
    orientation (keys index rows) and its eq. 1 with a scalar decay:
    S_t = a S + b k (v - S^T (a k))^T, o_t = S_t^T q. The oracle stores the
    transpose and must agree to fp64 rounding."""
    rng = np.random.default_rng(7)
    d, T = 4, 8

    def rat(x):
        return Fraction(int(round(x * 16)), 16)

    q = [[rat(x) for x in rng.standard_normal(d)] for _ in range(T)]
    k = [[rat(x) for x in rng.standard_normal(d)] for _ in range(T)]
    v = [[rat(x) for x in rng.standard_normal(d)] for _ in range(T)]
    a = [Fraction(int(rng.integers(9, 16)), 16) for _ in range(T)]
    b = [Fraction(int(rng.integers(1, 16)), 16) for _ in range(T)]
    S = [[Fraction(0)] * d for _ in range(d)]        # page orientation [k][v]
    outs = []
    for t in range(T):
        ak = [a[t] * x for x in k[t]]
        StAk = [sum(S[i][j] * ak[i] for i in range(d)) for j in range(d)]   # S^T (a k)
        corr = [b[t] * (v[t][j] - StAk[j]) for j in range(d)]
        S = [[a[t] * S[i][j] + k[t][i] * corr[j] for j in range(d)] for i in range(d)]
        outs.append([sum(S[i][j] * q[t][i] for i in range(d)) for j in range(d)])
    f = lambda M: np.array([[float(x) for x in r] for r in M])
    o, Sd = gdn.gdn_recurrent(f(q)[None], f(k)[None], f(v)[None],
                              np.array([[float(x) for x in a]]), np.array([[float(x) for x in b]]))
    np.testing.assert_allclose(o[0], f(outs), rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sd[0], f(S).T, rtol=0, atol=1e-13)


def test_beta_one_unit_key_stores_value_along_key():
    """With beta = 1 and a unit-norm key, the old association along k is erased
    and replaced: S_t k_t = v_t for any decay; reading with q = k returns v."""
    rng = np.random.default_rng(2)
    N, T, d = 4, 12, 16
    _, k, v, a, _ = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    b = np.ones((N, T))
    o, _ = gdn.gdn_recurrent(k, k, v, a, b, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_alpha_one_beta_zero_leaves_state_unchanged():
    rng = np.random.default_rng(3)
    N, T, d = 2, 10, 8
    q, k, v, _, _ = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    o, S = gdn.gdn_recurrent(q, k, v, np.ones((N, T)), np.zeros((N, T)), S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, np.einsum("nvk,ntk->ntv", S0, q), atol=1e-13)


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(4)
    N, T, d = 2, 10, 8
    q, k, v, a, _ = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    _, S = gdn.gdn_recurrent(q, k, v, a, np.zeros((N, T)), S0)
    np.testing.assert_allclose(S, np.prod(a, axis=1)[:, None, None] * S0, rtol=1e-13)


def test_orthonormal_keys_recall_every_value():
    """alpha = beta = 1 from zero with orthonormal keys: later writes do not
    disturb earlier ones, so S k_j = v_j for every stored pair. A transposed
    state (S^T k_j) fails this."""
    rng = np.random.default_rng(5)
    d = 12
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T[None, :, :]                        # rows orthonormal
    v = rng.standard_normal((1, d, d))
    _, S = gdn.gdn_recurrent(k, k, v, np.ones((1, d)), np.ones((1, d)))
    np.testing.assert_allclose(S[0] @ k[0].T, v[0].T, atol=1e-12)
    assert np.abs(S[0].T @ k[0].T - v[0].T).max() > 0.1


def test_delta_rule_first_form_alpha_one():
    """alpha = 1 is the plain delta rule, page form (I - b k k^T) S + b k v^T in
    d_k x d_v orientation, read with S^T q."""
    rng = np.random.default_rng(6)
    N, T, d = 1, 7, 5
    q, k, v, _, b = _rand(rng, N, T, d, unit=False)
    S = np.zeros((d, d))
    outs = []
    for t in range(T):
        kt = k[0, t][:, None]
        S = (np.eye(d) - b[0, t] * kt @ kt.T) @ S + b[0, t] * kt @ v[0, t][None, :]
        outs.append(S.T @ q[0, t])
    o, Sd = gdn.gdn_recurrent(q, k, v, np.ones((N, T)), b)
    np.testing.assert_allclose(o[0], np.array(outs), atol=1e-12)
    np.testing.assert_allclose(Sd[0], S.T, atol=1e-12)


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunk_wy_form_equals_recurrence(C):
    rng = np.random.default_rng(10 + C)
    N, T, d = 2, 128, 16
    q, k, v, a, b = _rand(rng, N, T, d)
    a = 1 / (1 + np.exp(-rng.normal(4, 1, (N, T))))
    S0 = 0.1 * rng.standard_normal((N, d, d))
    o1, S1 = gdn.gdn_recurrent(q, k, v, a, b, S0)
    o2, S2 = gdn.gdn_chunk_wy(q, k, v, a, b, S0, chunk=C)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-10)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-10)


def test_chunk_wy_affine_in_incoming_state():
    """run(S0) - run(0) is linear in S0 (the map is affine)."""
    rng = np.random.default_rng(11)
    N, T, d = 1, 64, 8
    q, k, v, a, b = _rand(rng, N, T, d)
    A1, A2 = rng.standard_normal((2, N, d, d))
    f = lambda S0: gdn.gdn_chunk_wy(q, k, v, a, b, S0, chunk=16)
    o0, S0_ = f(np.zeros((N, d, d)))
    o1, S1 = f(A1)
    o2, S2 = f(A2)
    o3, S3 = f(2 * A1 - 3 * A2)
    np.testing.assert_allclose(o3 - o0, 2 * (o1 - o0) - 3 * (o2 - o0), atol=1e-10)
    np.testing.assert_allclose(S3 - S0_, 2 * (S1 - S0_) - 3 * (S2 - S0_), atol=1e-10)


# ------------------------------------------------------------------ backward

def _torch_grads(q, k, v, a, b, S0, dO, dST):
    """Gradients by torch autograd (float64, CPU) of a separately written forward:
    the explicit matrix form S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T."""
    import torch
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, a, b, S0)]
    tq, tk, tv, ta, tb, tS = t
    S = tS
    eye = torch.eye(q.shape[2], dtype=torch.float64)
    outs = []
    for i in range(q.shape[1]):
        kt = tk[:, i][:, :, None]
        P = eye - tb[:, i][:, None, None] * (kt @ kt.transpose(1, 2))
        S = ta[:, i][:, None, None] * (S @ P) + tb[:, i][:, None, None] * (tv[:, i][:, :, None] @ kt.transpose(1, 2))
        outs.append((S @ tq[:, i][:, :, None])[..., 0])
    o = torch.stack(outs, 1)
    L = (o * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    L.backward()
    return [x.grad.numpy() for x in t]


def _bwd_case(rng, N, T, d):
    q, k, v, a, b = _rand(rng, N, T, d)
    S0, dST = rng.standard_normal((2, N, d, d))
    dO = rng.standard_normal((N, T, d))
    return q, k, v, a, b, S0, dO, dST


NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def test_backward_equals_autograd_of_explicit_form():
    rng = np.random.default_rng(51)
    q, k, v, a, b, S0, dO, dST = _bwd_case(rng, 2, 40, 8)
    got = gdn.gdn_recurrent_bwd(q, k, v, a, b, S0, dO, dST, ckpt=16)
    ref = _torch_grads(q, k, v, a, b, S0, dO, dST)
    for g_, r_, name in zip(got, ref, NAMES):
        np.testing.assert_allclose(g_, r_, rtol=0, atol=1e-10 * np.abs(r_).max(), err_msg=name)


def test_backward_finite_differences():
    """Central differences of L = sum(dO o o) + sum(dST o S_T) on a tiny case."""
    rng = np.random.default_rng(52)
    q, k, v, a, b, S0, dO, dST = _bwd_case(rng, 1, 6, 3)

    def L(*args):
        o, ST = gdn.gdn_recurrent(*args)
        return float((o * dO).sum() + (ST * dST).sum())

    args = [q, k, v, a, b, S0]
    grads = gdn.gdn_recurrent_bwd(q, k, v, a, b, S0, dO, dST)
    h = 1e-6
    for ai, g_ in enumerate(grads):
        x = args[ai]
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[ai], am[ai] = xp, xm
            num[idx] = (L(*ap) - L(*am)) / (2 * h)
        np.testing.assert_allclose(g_, num, rtol=0, atol=1e-6 * max(1.0, np.abs(num).max()), err_msg=NAMES[ai])


def test_backward_constant_state_closed_form():
    """alpha = 1, beta = 0: S_t = S0 and o_t = S0 q_t, so with D_t = dST + sum_{s>=t}
    do_s q_s^T: dq_t = S0^T do_t, dk = dv = 0, dbeta_t = (D_t k_t) . (v_t - S0 k_t),
    dalpha_t = sum(D_t o S0), dS0 = D_0."""
    rng = np.random.default_rng(53)
    N, T, d = 2, 12, 5
    q, k, v, _, _, S0, dO, dST = _bwd_case(rng, N, T, d)
    dq, dk, dv, da, db, dS0 = gdn.gdn_recurrent_bwd(q, k, v, np.ones((N, T)), np.zeros((N, T)), S0, dO, dST)
    D = dST[:, None] + np.cumsum(np.einsum("ntv,ntk->ntvk", dO, q)[:, ::-1], axis=1)[:, ::-1]
    np.testing.assert_allclose(dq, np.einsum("nvk,ntv->ntk", S0, dO), atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)
    np.testing.assert_allclose(dv, 0, atol=1e-12)
    Dk = np.einsum("ntvk,ntk->ntv", D, k)
    np.testing.assert_allclose(db, np.einsum("ntv,ntv->nt", Dk, v - np.einsum("nvk,ntk->ntv", S0, k)), atol=1e-11)
    np.testing.assert_allclose(da, np.einsum("ntvk,nvk->nt", D, S0), atol=1e-11)
    np.testing.assert_allclose(dS0, D[:, 0], atol=1e-12)


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunk_backward_equals_reverse_mode(C):
    """The chunk-form backward (WY gradients, the state-gradient scan and the gate
    gradient from q . dq - v . dv) equals reverse mode through the recurrence."""
    rng = np.random.default_rng(60 + C)
    q, k, v, a, b, S0, dO, dST = _bwd_case(rng, 2, 128, 8)
    ref = gdn.gdn_recurrent_bwd(q, k, v, a, b, S0, dO, dST, ckpt=32)
    got = gdn.gdn_chunk_wy_bwd(q, k, v, a, b, S0, dO, dST, chunk=C)
    for g_, r_, name in zip(got, ref, NAMES):
        np.testing.assert_allclose(g_, r_, rtol=0, atol=1e-11 * np.abs(r_).max(), err_msg=name)
    got = gdn.gdn_chunk_wy_bwd(q, k, v, a, b, None, dO, None, chunk=C)
    ref = gdn.gdn_recurrent_bwd(q, k, v, a, b, None, dO, None)
    for g_, r_, name in zip(got, ref, NAMES):
        np.testing.assert_allclose(g_, r_, rtol=0, atol=1e-11 * np.abs(r_).max(), err_msg=name)


def test_decay_gradient_sums_and_state_boundary_identity():
    """d log alpha_t (reverse mode, alpha_t dalpha_t) equals the reverse sum over s >= t
    of q_s . dq_s - v_s . dv_s (+ sum(dST o S_T)), and its part beyond any token
    boundary equals sum(dS o S) of the state there and its gradient: scaling alpha_t
    is scaling the state that token t starts from."""
    rng = np.random.default_rng(54)
    N, T, d = 2, 40, 6
    q, k, v, a, b, S0, dO, dST = _bwd_case(rng, N, T, d)
    dq, dk, dv, da, db, dS0 = gdn.gdn_recurrent_bwd(q, k, v, a, b, S0, dO, dST)
    _, ST = gdn.gdn_recurrent(q, k, v, a, b, S0)
    dB = np.einsum("ntk,ntk->nt", q, dq) - np.einsum("ntv,ntv->nt", v, dv)
    dB[:, -1] += np.einsum("nvk,nvk->n", dST, ST)
    dlog = a * da
    np.testing.assert_allclose(dlog, np.cumsum(dB[:, ::-1], axis=1)[:, ::-1], rtol=0, atol=1e-10 * np.abs(dlog).max())
    for t0 in (1, 17, 39):   # boundary before token t0: state S_{t0-1} and its gradient
        _, S_mid = gdn.gdn_recurrent(q[:, :t0], k[:, :t0], v[:, :t0], a[:, :t0], b[:, :t0], S0)
        *_, dS_mid = gdn.gdn_recurrent_bwd(q[:, t0:], k[:, t0:], v[:, t0:], a[:, t0:], b[:, t0:], S_mid,
                                           dO[:, t0:], dST)
        np.testing.assert_allclose(dlog[:, t0], np.einsum("nvk,nvk->n", dS_mid, S_mid), rtol=0,
                                   atol=1e-10 * np.abs(dlog).max())

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


# ------------------------------------------------------------------ backward

def _loss_grads_torch(q, k, v, lg, S0, dO, dST):
    """Gradients by torch autograd (float64, CPU) of a separately written torch
    forward of the recurrence: an independent derivation of the same gradients."""
    import torch
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, lg, S0)]
    tq, tk, tv, tg, tS = t
    S = tS
    outs = []
    for i in range(q.shape[1]):
        S = torch.exp(tg[:, i])[:, None, :] * S + tv[:, i][:, :, None] * tk[:, i][:, None, :]
        outs.append(torch.einsum("nvk,nk->nv", S, tq[:, i]))
    o = torch.stack(outs, 1)
    L = (o * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    L.backward()
    return [x.grad.numpy() for x in t]


def test_backward_equals_autograd():
    rng = np.random.default_rng(41)
    N, T, d = 2, 40, 8
    q, k, v, lg = _rand(rng, N, T, d)
    S0, dST = rng.standard_normal((2, N, d, d))
    dO = rng.standard_normal((N, T, d))
    got = gla.gla_recurrent_bwd(q, k, v, lg, S0, dO, dST, ckpt=16)
    ref = _loss_grads_torch(q, k, v, lg, S0, dO, dST)
    for g_, r_, name in zip(got, ref, ("dq", "dk", "dv", "dg", "dS0")):
        np.testing.assert_allclose(g_, r_, rtol=0, atol=1e-10 * np.abs(r_).max(), err_msg=name)


def test_backward_finite_differences():
    """Central differences of L = sum(dO o o) + sum(dST o S_T) on a tiny case."""
    rng = np.random.default_rng(42)
    N, T, d = 1, 6, 3
    q, k, v, lg = _rand(rng, N, T, d)
    S0, dST = rng.standard_normal((2, N, d, d))
    dO = rng.standard_normal((N, T, d))

    def L(q_, k_, v_, g_, S_):
        o, ST = gla.gla_recurrent(q_, k_, v_, g_, S_)
        return float((o * dO).sum() + (ST * dST).sum())

    grads = gla.gla_recurrent_bwd(q, k, v, lg, S0, dO, dST)
    args = [q, k, v, lg, S0]
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
        np.testing.assert_allclose(g_, num, rtol=0, atol=1e-6 * max(1.0, np.abs(num).max()))


def test_backward_zero_gates_textbook():
    """g = 0: O = tril(Q K^T) V + Q S0^T, so dQ = tril(dO V^T) K + dO S0,
    dK = tril(dO V^T)^T Q, dV = tril(Q K^T)^T dO, dS0 = dO^T Q (dST = 0)."""
    rng = np.random.default_rng(43)
    N, T, d = 2, 24, 8
    q, k, v, _ = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    dO = rng.standard_normal((N, T, d))
    dq, dk, dv, dg, dS0 = gla.gla_recurrent_bwd(q, k, v, np.zeros((N, T, d)), S0, dO)
    P = np.tril(np.einsum("ntv,njv->ntj", dO, v))
    np.testing.assert_allclose(dq, P @ k + np.einsum("ntv,nvk->ntk", dO, S0), atol=1e-10)
    np.testing.assert_allclose(dk, np.swapaxes(P, 1, 2) @ q, atol=1e-10)
    np.testing.assert_allclose(dv, np.swapaxes(np.tril(np.einsum("ntk,njk->ntj", q, k)), 1, 2) @ dO, atol=1e-10)
    np.testing.assert_allclose(dS0, np.einsum("ntv,ntk->nvk", dO, q), atol=1e-10)


def test_backward_zeco_chunk_state_gradient():
    """ZeCO's backward, phase 1: per chunk in reverse, dS <- gamma o dS + Q~^T dO
    (in this orientation dS <- exp(b_C) o dS + dO^T (Q o exp(b))) gives the
    gradient with respect to the incoming state; and the gate gradient follows
    from dq and dk: with b the cumulative log-gate over the sequence, q o exp(b)
    and k o exp(-b) are what b enters, so dL/db_t = q_t o dq_t - k_t o dk_t
    (+ sum_v dST o S_T at the last token) and dg is its reverse cumulative sum."""
    rng = np.random.default_rng(44)
    N, T, d, C = 2, 128, 8, 32
    q, k, v, lg = _rand(rng, N, T, d)
    S0, dST = rng.standard_normal((2, N, d, d))
    dO = rng.standard_normal((N, T, d))
    dq, dk, dv, dg, dS0 = gla.gla_recurrent_bwd(q, k, v, lg, S0, dO, dST)
    dS = dST.copy()
    for c0 in range(T - C, -1, -C):
        sl = slice(c0, c0 + C)
        b = np.cumsum(lg[:, sl], axis=1)
        dS = np.exp(b[:, -1])[:, None, :] * dS + np.einsum("ntv,ntk->nvk", dO[:, sl], q[:, sl] * np.exp(b))
    np.testing.assert_allclose(dS0, dS, rtol=0, atol=1e-10 * np.abs(dS).max())
    _, ST = gla.gla_recurrent(q, k, v, lg, S0)
    db = q * dq - k * dk
    db[:, -1] += np.einsum("nvk,nvk->nk", dST, ST)
    np.testing.assert_allclose(dg, np.cumsum(db[:, ::-1], axis=1)[:, ::-1], rtol=0,
                               atol=1e-9 * np.abs(dg).max())


def test_backward_gate_gradient_beyond_a_boundary():
    """The part of d log_g_t from tokens after a boundary equals sum_v dS o S (per key
    channel) of the state there and its gradient: shifting the cumulative log-gate of
    one channel on every later token scales that key column of the state."""
    rng = np.random.default_rng(45)
    N, T, d = 2, 48, 6
    q, k, v, lg = _rand(rng, N, T, d)
    S0, dST = rng.standard_normal((2, N, d, d))
    dO = rng.standard_normal((N, T, d))
    dq, dk, dv, dg, dS0 = gla.gla_recurrent_bwd(q, k, v, lg, S0, dO, dST)
    for t0 in (1, 16, 47):
        _, S_mid = gla.gla_recurrent(q[:, :t0], k[:, :t0], v[:, :t0], lg[:, :t0], S0)
        *_, dS_mid = gla.gla_recurrent_bwd(q[:, t0:], k[:, t0:], v[:, t0:], lg[:, t0:], S_mid, dO[:, t0:], dST)
        np.testing.assert_allclose(dg[:, t0], np.einsum("nvk,nvk->nk", dS_mid, S_mid), rtol=0,
                                   atol=1e-10 * np.abs(dg).max())


@pytest.mark.parametrize("devices,blocks", [(1, 1), (2, 1), (4, 4), (3, 2)])
def test_zeco_forward_equals_recurrence(devices, blocks):
    """ZeCO's three phases over several devices (local states from zero, All-Scan
    in device order with the state cut into key blocks, outputs from the received
    state) give the recurrence over the whole sequence, from a nonzero S0."""
    rng = np.random.default_rng(46)
    N, C, d = 2, 16, 8
    T = devices * 2 * C
    q, k, v, lg = _rand(rng, N, T, d, mu=1.0)
    S0 = rng.standard_normal((N, d, d))
    o_ref, S_ref = gla.gla_recurrent(q, k, v, lg, S0)
    o, S = gla.zeco_forward(q, k, v, lg, devices, S0, chunk=C, blocks=blocks)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12 * np.abs(o_ref).max())
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12 * np.abs(S_ref).max())


def test_zeco_local_states_and_decays():
    """Phase 1: S_[n] is the state from zero after n chunks (the recurrence cut
    there), and gamma~_[n] is exp of the log-gates summed over those tokens."""
    rng = np.random.default_rng(47)
    N, T, d, C = 2, 64, 6, 16
    q, k, v, lg = _rand(rng, N, T, d)
    Ss, gam = gla.zeco_local(k, v, lg, C)
    assert Ss.shape == (N, T // C + 1, d, d) and gam.shape == (N, T // C + 1, d)
    np.testing.assert_array_equal(Ss[:, 0], 0.0)
    np.testing.assert_array_equal(gam[:, 0], 1.0)
    for n in range(1, T // C + 1):
        _, S_n = gla.gla_recurrent(q[:, :n * C], k[:, :n * C], v[:, :n * C], lg[:, :n * C], None)
        np.testing.assert_allclose(Ss[:, n], S_n, rtol=0, atol=1e-12 * np.abs(S_n).max())
        np.testing.assert_allclose(gam[:, n], np.exp(lg[:, :n * C].sum(axis=1)), rtol=1e-13)


def test_zeco_all_scan_step_blocks_and_start_device():
    """All-Scan's update is elementwise along the key channels: cutting the state
    into 1, 2 or 8 blocks gives the same result bit for bit, and the start device
    sends its local state unchanged."""
    rng = np.random.default_rng(48)
    N, d = 3, 8
    S_loc, S_recv = rng.standard_normal((2, N, d, d))
    gam = rng.uniform(0.1, 1.0, (N, d))
    ref = gam[:, None, :] * S_recv + S_loc
    for blocks in (1, 2, 8):
        np.testing.assert_array_equal(gla.zeco_all_scan_step(S_loc, gam, S_recv, blocks), ref)
    np.testing.assert_array_equal(gla.zeco_all_scan_step(S_loc, gam, None), S_loc)


@pytest.mark.parametrize("devices,blocks,zero_ends", [(1, 1, False), (2, 4, False), (3, 2, True), (4, 1, False)])
def test_zeco_backward_equals_reverse_mode(devices, blocks, zero_ends):
    """ZeCO's backward over several devices (phase 1 from zero, the backward
    All-Scan from the last device, gradients from the received state gradient)
    gives the gradients of the recurrence over the whole sequence."""
    rng = np.random.default_rng(49)
    N, C, d = 2, 16, 6
    T = devices * 2 * C
    q, k, v, lg = _rand(rng, N, T, d, mu=1.0)
    S0, dST = (None, None) if zero_ends else rng.standard_normal((2, N, d, d))
    dO = rng.standard_normal((N, T, d))
    ref = gla.gla_recurrent_bwd(q, k, v, lg, S0, dO, dST)
    got = gla.zeco_backward(q, k, v, lg, dO, devices, S0, dST, chunk=C, blocks=blocks)
    for name, a, b in zip(("dq", "dk", "dv", "dlog_g", "dS0"), got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * np.abs(b).max(), err_msg=name)


def test_zeco_bwd_local_state_is_the_incoming_state_gradient():
    """Phase 1's dS_[0] is the gradient with respect to S0 when nothing arrives from
    later tokens (reverse mode with dST = 0), and it does not depend on S0, k or v."""
    rng = np.random.default_rng(50)
    N, T, d, C = 2, 64, 6, 16
    q, k, v, lg = _rand(rng, N, T, d)
    S0 = rng.standard_normal((N, d, d))
    dO = rng.standard_normal((N, T, d))
    *_, dS0 = gla.gla_recurrent_bwd(q, k, v, lg, S0, dO, None)
    np.testing.assert_allclose(gla.zeco_bwd_local_state(q, lg, dO, C), dS0, rtol=0, atol=1e-12 * np.abs(dS0).max())

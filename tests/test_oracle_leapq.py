"""Pins of the LeapQuant oracle against what the LeapQuant page fixes."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import gdn, leapq

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(rng, T, N, d, amu=4.0):
    q = rng.standard_normal((T, N, d))
    k = rng.standard_normal((T, N, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, N, d))
    a = 1 / (1 + np.exp(-rng.normal(amu, 1, (T, N))))
    b = 1 / (1 + np.exp(-rng.normal(0, 1, (T, N))))
    return q, k, v, a, b


def _tn(x):   # [T][N][d] -> [N][T][d]
    return np.swapaxes(x, 0, 1)


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_window_one_no_extras_equals_per_token_rounding_eq2(bits):
    """Eq. 2 rounding after every token, written separately, must equal the
    windowed scheme with W = 1, no compensator tokens and no smoothing, at every
    code width."""
    rng = np.random.default_rng(1)
    T, N, d = 24, 3, 16
    q, k, v, a, b = _inputs(rng, T, N, d)
    S0 = 0.05 * rng.standard_normal((N, d, d))
    o1, Z1, s1 = leapq.per_step_int8(q, k, v, a, b, S0, bits=bits)
    r = leapq.decode_run(q, k, v, a, b, S0, None, window=1, rank=0, smooth_mode=2,
                         buf_dtype=np.float64, bits=bits)
    np.testing.assert_array_equal(r["st"]["Z"], Z1)
    np.testing.assert_array_equal(r["st"]["s"], s1)
    np.testing.assert_allclose(r["o"], o1, rtol=0, atol=1e-12)


def test_eq10_readout_equals_dense_eq4_state():
    rng = np.random.default_rng(2)
    N, d, m = 3, 16, 9
    S0 = rng.standard_normal((N, d, d))
    Q0 = rng.standard_normal((d, 4))
    st = leapq.flush(S0, Q0, rank=4)
    buf = [(rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.uniform(0.5, 1, N))
           for _ in range(m)]
    x = rng.standard_normal((N, d))
    dense = leapq.rebuild(st, buf)
    np.testing.assert_allclose(leapq.readout(st, buf, x), np.einsum("nvk,nk->nv", dense, x),
                               atol=1e-12)
    # the rebuild itself: decayed stored state plus decayed rank-one writes
    g = np.prod(np.stack([bb[2] for bb in buf]), axis=0)
    ref = g[:, None, None] * leapq.dequant(st)
    for j, (kj, uj, _) in enumerate(buf):
        gj = np.prod(np.stack([bb[2] for bb in buf[j + 1:]] + [np.ones(N)]), axis=0)
        ref += gj[:, None, None] * uj[:, :, None] * kj[:, None, :]
    np.testing.assert_allclose(dense, ref, atol=1e-12)


def test_rank_r_state_is_caught_by_compensators():
    """A state of rank <= r lies in the fitted subspace after one round from a
    generic start, so the unquantised residual S - (S Q) Q^T vanishes."""
    rng = np.random.default_rng(3)
    N, d, r = 2, 32, 4
    S = np.einsum("nvr,nkr->nvk", rng.standard_normal((N, d, r)), rng.standard_normal((N, d, r)))
    Q0 = rng.standard_normal((d, r))
    Q = leapq.fit_compensators(S, Q0, r, iters=1)
    np.testing.assert_allclose(np.swapaxes(Q, -1, -2) @ Q, np.broadcast_to(np.eye(r), (N, r, r)),
                               atol=1e-5)
    # the subspace is exact: project onto an exactly orthonormal basis of it
    Qh = np.linalg.qr(Q)[0]
    R = S - (S @ Qh) @ np.swapaxes(Qh, -1, -2)
    assert np.abs(R).max() < 1e-10 * np.abs(S).max()
    # the Gram shift leaves the fitted columns short of unit norm by ~1e-6 only
    R = S - (S @ Q) @ np.swapaxes(Q, -1, -2)
    assert np.abs(R).max() < 2e-5 * np.abs(S).max()
    st = leapq.flush(S, Q0, rank=r)
    # what is left after subtracting the fp16 pieces is fp16 rounding only
    R16 = S - np.swapaxes(st["ut"], -1, -2) @ st["kt"]
    assert np.abs(R16).max() < 4e-3 * np.abs(S).max()


def test_subspace_iteration_reaches_eckart_young_bound():
    """With a spectral gap and enough rounds, the fitted pieces achieve the
    Eckart-Young minimum ||S - S_r||_F^2 = sum_{i>r} sigma_i^2; the SVD mode
    achieves it exactly."""
    rng = np.random.default_rng(4)
    d, r = 24, 4
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    sig = np.concatenate([[40, 30, 20, 10], np.linspace(1, 0.1, d - r)])
    S = (U * sig) @ V.T
    tail = np.sum(sig[r:] ** 2)
    for Q in (leapq.fit_compensators(S[None], rng.standard_normal((d, r)), r, iters=40),
              leapq.fit_compensators(S[None], None, r, svd=True)):
        R = S - (S @ Q[0]) @ Q[0].T
        np.testing.assert_allclose(np.sum(R ** 2), tail, rtol=1e-8)
    # one round from a random start is worse than the bound but far below ||S||^2
    Q1 = leapq.fit_compensators(S[None], rng.standard_normal((d, r)), r, iters=1)
    R1 = S - (S @ Q1[0]) @ Q1[0].T
    assert tail <= np.sum(R1 ** 2) < 0.2 * np.sum(sig ** 2)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_reconstruction_within_half_a_step(mode):
    rng = np.random.default_rng(5)
    N, d = 3, 32
    S = rng.standard_normal((N, d, d))
    S[:, :, 3] *= 50
    st = leapq.flush(S, rng.standard_normal((d, 4)), rank=4, smooth_mode=mode)
    err = np.abs(leapq.dequant(st) - S)
    step = st["s"][:, :, None] / 127.0 * st["c"][:, None, :]
    assert np.all(err <= 0.5 * step * (1 + 1e-5) + 1e-12)


def test_smoothing_statistic_and_quant_scale_orientation():
    """Smoothing is one factor per key channel (page: per key row), the root of
    the mean magnitude over the value channels; the quantisation scale is one
    per value channel, its largest smoothed magnitude, which maps to +-127."""
    d = 8
    m = np.arange(1, d + 1, dtype=np.float64)               # column magnitudes
    signs = np.where(np.add.outer(np.arange(d), np.arange(d)) % 2 == 0, 1.0, -1.0)
    S = (signs * m[None, :])[None]                          # |S[v,k]| = m_k
    st = leapq.flush(S, None, rank=0, smooth_mode=0)
    np.testing.assert_allclose(st["c"][0], np.sqrt(m), rtol=1e-7)
    st1 = leapq.flush(S, None, rank=0, smooth_mode=1)
    np.testing.assert_allclose(st1["c"][0], m, rtol=1e-7)          # root mean square of a constant column
    np.testing.assert_allclose(st["s"][0], np.full(d, np.sqrt(m[-1])), rtol=1e-7)
    assert np.all(np.abs(st["Z"][0][:, -1]) == 127)
    # a column that is not constant separates the two statistics
    S2 = S.copy()
    S2[0, 0, 0] = 9.0
    c0 = leapq.flush(S2, None, rank=0, smooth_mode=0)["c"][0, 0]
    c1 = leapq.flush(S2, None, rank=0, smooth_mode=1)["c"][0, 0]
    np.testing.assert_allclose(c0, np.sqrt((9 + 7) / 8), rtol=1e-7)
    np.testing.assert_allclose(c1, np.sqrt((81 + 7) / 8), rtol=1e-7)


def test_codes_invariant_under_power_of_four_scaling():
    rng = np.random.default_rng(6)
    S = rng.standard_normal((2, 16, 16))
    Q0 = rng.standard_normal((16, 4))
    base = leapq.flush(S, Q0, rank=0, smooth_mode=0)
    for f in (4.0, 1 / 16):
        st = leapq.flush(f * S, Q0, rank=0, smooth_mode=0)
        np.testing.assert_array_equal(st["Z"], base["Z"])
        np.testing.assert_allclose(st["s"], np.sqrt(f) * base["s"], rtol=0)


def test_zero_state_is_finite_and_zero():
    st = leapq.flush(np.zeros((2, 16, 16)), np.ones((16, 4)), rank=4, smooth_mode=0)
    for key in ("s", "c", "kt", "ut"):
        assert np.all(np.isfinite(st[key]))
    assert np.all(st["Z"] == 0)
    assert np.all(leapq.dequant(st) == 0)


def test_stored_bytes_match_page_layout():
    with open(os.path.join(GOLD, "leapq_layout.json")) as f:
        g = json.load(f)
    n = leapq.stored_bytes(g["d_v"], g["d_k"], g["rank"])
    assert n == g["bytes"]
    assert n / (g["d_v"] * g["d_k"]) == g["bytes_per_element"]


def test_decay_freezing_counts_of_the_roundings():
    """The page's exhaustive count of values that never decay when re-rounded,
    reproduced with the bf16 cast of the input generator (torch) and the fp16
    cast of the compensator tokens (numpy)."""
    with open(os.path.join(GOLD, "decay_freeze.json")) as f:
        g = json.load(f)
    lo, hi = np.log10(g["range"][0]), np.log10(g["range"][1])
    x = 10.0 ** np.linspace(lo, hi, 200001)
    xb = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
    for a, want in g["bf16"].items():
        y = (xb.float() * torch.tensor(float(a))).to(torch.bfloat16)
        assert abs((y == xb).float().mean().item() - want) <= g["tol"], a
    xh = leapq.fp16(x)
    for a, want in g["fp16"].items():
        y = leapq.fp16(np.float32(xh) * np.float32(a))
        assert abs(np.mean(y == xh) - want) <= g["tol"], a


def test_windowed_run_tracks_exact_trajectory():
    """With the window, compensators and smoothing, the read-outs stay close
    to the exact fp64 recurrence on a 128-dim head with outlier channels."""
    rng = np.random.default_rng(8)
    T, N, d = 64, 2, 128
    q, k, v, a, b = _inputs(rng, T, N, d)
    S0 = 0.05 * rng.standard_normal((N, d, d))
    S0[:, :, [5, 77]] *= 50
    Q0 = rng.standard_normal((d, 4))
    r = leapq.decode_run(q, k, v, a, b, S0, Q0)
    o_ex, _ = gdn.gdn_recurrent(_tn(q), _tn(k), _tn(v), a.T, b.T, S0)
    err = np.abs(r["o"] - _tn(o_ex)).max() / np.abs(o_ex).max()
    assert err < 2e-2


def test_error_ordering_trend_on_a_toy_head():
    """Trend only (parity unpinned): on a toy head in the spirit of the page's
    simulator, the relative state error orders as per-token INT8 > window >
    window with compensator tokens and smoothing."""
    rng = np.random.default_rng(9)
    T, N, d = 512, 1, 32
    k = rng.standard_normal((T, N, d))
    k[..., :2] += 2.0
    k[..., 2:6] *= 3.0
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = k[::-1].copy()
    v = rng.standard_normal((T, N, d))
    v[..., :2] += 4.0
    a = np.full((T, N), 0.995)
    b = rng.uniform(0.05, 0.15, (T, N))
    S0 = np.zeros((N, d, d))
    _, S_ex = gdn.gdn_recurrent(_tn(q), _tn(k), _tn(v), a.T, b.T, S0)

    def final_dense(r):
        return leapq.rebuild(r["st"], r["buf"])

    e = {}
    _, Zp, sp = leapq.per_step_int8(q, k, v, a, b, S0)
    e["step"] = np.linalg.norm(sp[:, :, None] * Zp / 127.0 - S_ex) / np.linalg.norm(S_ex)
    r = leapq.decode_run(q, k, v, a, b, S0, None, window=16, rank=0, smooth_mode=2)
    e["window"] = np.linalg.norm(final_dense(r) - S_ex) / np.linalg.norm(S_ex)
    r = leapq.decode_run(q, k, v, a, b, S0, rng.standard_normal((d, 4)), window=16, rank=4,
                         smooth_mode=0)
    e["full"] = np.linalg.norm(final_dense(r) - S_ex) / np.linalg.norm(S_ex)
    assert e["step"] > e["window"] > e["full"], e


# ------------------------------------------------------------------ narrower codes, BF16

@pytest.mark.parametrize("bits", [6, 4])
def test_narrow_grid_codes_and_half_step_bound(bits):
    """At b bits the codes stay in [-Q, Q], Q = 2^(b-1) - 1, every nonzero value
    channel reaches +-Q, and each entry is within half a step s_v / Q c_k."""
    rng = np.random.default_rng(15)
    N, d = 3, 32
    S = rng.standard_normal((N, d, d))
    S[:, :, 3] *= 50
    st = leapq.flush(S, rng.standard_normal((d, 6)), rank=6, smooth_mode=0, bits=bits)
    Q = (1 << (bits - 1)) - 1
    assert st["Q"] == Q and np.abs(st["Z"]).max() == Q
    assert np.all(np.abs(st["Z"]).max(axis=-1) == Q)
    err = np.abs(leapq.dequant(st) - S)
    step = st["s"][:, :, None] / Q * st["c"][:, None, :]
    assert np.all(err <= 0.5 * step * (1 + 1e-5) + 1e-12)


def test_bf16_rounding_is_torch_bfloat16():
    rng = np.random.default_rng(16)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.5]])
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(leapq.bf16(x), ref)


def test_per_step_bf16_state_freezes_slow_decays():
    """The page's count: a BF16 state re-rounded after every token does not move
    under a decay of 0.999 (all values), 0.998 (most) or 0.997 (about a third),
    for log-uniform values in [0.01, 10] -- through the per-step BF16 baseline with
    no writes (beta = 0)."""
    with open(os.path.join(GOLD, "decay_freeze.json")) as f:
        g = json.load(f)
    lo, hi = np.log10(g["range"][0]), np.log10(g["range"][1])
    N, d = 4, 64
    S0 = leapq.bf16(10.0 ** np.linspace(lo, hi, N * d * d)).reshape(N, d, d)
    z = np.zeros((1, N, d))
    for a, want in g["bf16"].items():
        _, S1 = leapq.per_step_bf16(z, z, z, np.full((1, N), float(a)), np.zeros((1, N)), S0)
        assert abs(np.mean(S1 == S0) - want) <= 2 * g["tol"] + 2e-3, a
    _, S100 = leapq.per_step_bf16(np.zeros((100, N, d)), np.zeros((100, N, d)), np.zeros((100, N, d)),
                                  np.full((100, N), 0.999), np.zeros((100, N)), S0)
    np.testing.assert_array_equal(S100, S0)


@pytest.mark.parametrize("bits", [6, 4])
def test_error_ordering_trend_at_narrow_widths(bits):
    """Trend only (parity unpinned): at 6 and 4 bits, with 6 compensator tokens
    (the paper's pairing), the relative state error still orders as per-token
    rounding > window > window with compensator tokens and smoothing."""
    rng = np.random.default_rng(9)
    T, N, d = 512, 1, 32
    k = rng.standard_normal((T, N, d))
    k[..., :2] += 2.0
    k[..., 2:6] *= 3.0
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = k[::-1].copy()
    v = rng.standard_normal((T, N, d))
    v[..., :2] += 4.0
    a = np.full((T, N), 0.995)
    b = rng.uniform(0.05, 0.15, (T, N))
    S0 = np.zeros((N, d, d))
    _, S_ex = gdn.gdn_recurrent(_tn(q), _tn(k), _tn(v), a.T, b.T, S0)
    rel = lambda X: np.linalg.norm(X - S_ex) / np.linalg.norm(S_ex)
    _, Zp, mp = leapq.per_step_int8(q, k, v, a, b, S0, bits=bits)
    e_step = rel(mp[:, :, None] * Zp / leapq.qmax(bits))
    r = leapq.decode_run(q, k, v, a, b, S0, None, window=16, rank=0, smooth_mode=2, bits=bits)
    e_win = rel(leapq.rebuild(r["st"], r["buf"]))
    r = leapq.decode_run(q, k, v, a, b, S0, rng.standard_normal((d, 6)), window=16, rank=6,
                         smooth_mode=0, bits=bits)
    e_full = rel(leapq.rebuild(r["st"], r["buf"]))
    assert e_step > e_win > e_full, (e_step, e_win, e_full)


def test_window_run_from_exact_grid_state_is_the_gdn_recurrence():
    """Teacher-forced window of the windowed scheme (section "Fix one: leap over a
    window", eq. 4 and eq. 10). A stored state the INT8 grid holds exactly (codes,
    scales and smoothing factors chosen, fp16 compensator pieces given) dequantises
    to S_hat_0 with no rounding, so one window of read-outs from it with an fp64
    buffer must be the exact Gated DeltaNet recurrence from S_hat_0 (itself pinned by
    exact rationals in test_oracle_gdn.py), and the eq. 4 rebuild its final state.
    Fails if u is formed from the state after the token instead of before it, or if
    alpha is applied twice or not at all in the correction."""
    rng = np.random.default_rng(31)
    T, N, d, r = 16, 3, 16, 4
    q, k, v, a, b = _inputs(rng, T, N, d, amu=2.0)
    st = dict(Z=rng.integers(-127, 128, (N, d, d)).astype(np.int8),
              s=rng.uniform(0.5, 2.0, (N, d)), c=rng.uniform(0.25, 1.0, (N, d)),
              kt=leapq.fp16(rng.standard_normal((N, r, d))),
              ut=leapq.fp16(rng.standard_normal((N, r, d))))
    S0 = leapq.dequant(st)
    o, buf = leapq.window_run(st, q, k, v, a, b, buf_dtype=np.float64)
    o_ex, S_ex = gdn.gdn_recurrent(_tn(q), _tn(k), _tn(v), a.T, b.T, S0)
    scale = np.abs(o_ex).max()
    np.testing.assert_allclose(o, _tn(o_ex), rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(leapq.rebuild(st, buf), S_ex, rtol=0,
                               atol=1e-12 * np.abs(S_ex).max())
    # each record's correction is u_t = beta_t (v_t - alpha_t S_{t-1} k_t): recover
    # S_{t-1} from the recurrence's own prefix and check the buffer term by term
    for t in range(T):
        _, S_prev = gdn.gdn_recurrent(_tn(q[:t]), _tn(k[:t]), _tn(v[:t]), a[:t].T, b[:t].T, S0)
        u_ref = b[t][:, None] * (v[t] - a[t][:, None] * np.einsum("nvk,nk->nv", S_prev, k[t]))
        np.testing.assert_allclose(buf[t][1], u_ref, rtol=0, atol=1e-12 * np.abs(u_ref).max())
        np.testing.assert_array_equal(buf[t][2], a[t])


def test_window_run_on_the_first_window_equals_decode_run():
    """The teacher-forced window from the encoded initial state is the first window
    of the whole windowed run (same fp32 buffer, same flush)."""
    rng = np.random.default_rng(32)
    T, N, d = 24, 2, 32
    q, k, v, a, b = _inputs(rng, T, N, d)
    S0 = 0.05 * rng.standard_normal((N, d, d))
    Q0 = rng.standard_normal((d, 4))
    run = leapq.decode_run(q, k, v, a, b, S0, Q0, window=8, rank=4, collect=True)
    for w in range(3):
        sl = slice(8 * w, 8 * w + 8)
        o, buf = leapq.window_run(run["starts"][w], q[sl], k[sl], v[sl], a[sl], b[sl])
        np.testing.assert_array_equal(o, run["o"][sl])
        if w < 2:
            nxt = leapq.flush(leapq.rebuild(run["starts"][w], buf), Q0, rank=4)
            np.testing.assert_array_equal(nxt["Z"], run["starts"][w + 1]["Z"])

"""Pins of the KDA windowed-INT8 oracle (``oracle.kda_leapq``) against what the
LeapQuant page fixes: eq. 4 and eq. 10 with diagonal decays, the per-token
rounding of eq. 2, and the exact KDA recurrence of eq. 1 / eq. 3 (itself pinned
by exact rationals in test_oracle_kda.py).

A plausible slip fails one of them: the decay of a record counted from its own
token instead of the one after it, the decay applied to value channels, the
smoothing or Gamma_{1:m} left out of the integer read, the correction formed
from S k instead of S (alpha o k)."""
import numpy as np

from oracle import kda, kda_leapq, leapq


def _inputs(rng, T, N, d, amu=3.0):
    q = rng.standard_normal((T, N, d))
    k = rng.standard_normal((T, N, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, N, d))
    a = 1 / (1 + np.exp(-rng.normal(amu, 1, (T, N, d))))
    b = 1 / (1 + np.exp(-rng.normal(0, 1, (T, N))))
    return q, k, v, a, b


def _tn(x):   # [T][N][..] -> [N][T][..]
    return np.swapaxes(x, 0, 1)


def test_exact_grid_state_reproduces_the_kda_recurrence():
    """A stored state the INT8 grid holds exactly (codes, scales and smoothing
    factors chosen, compensator pieces given) is S_hat_0 itself; one window of
    read-outs from it (fp64 buffer) must then be the exact KDA recurrence from
    S_hat_0, token by token, and the eq. 4 rebuild its final state."""
    rng = np.random.default_rng(21)
    T, N, d, r = 16, 3, 16, 2
    q, k, v, a, b = _inputs(rng, T, N, d)
    st = dict(Z=rng.integers(-127, 128, (N, d, d)).astype(np.int8),
              s=rng.uniform(0.5, 2.0, (N, d)), c=rng.uniform(0.25, 1.0, (N, d)),
              kt=leapq.fp16(rng.standard_normal((N, r, d))), ut=leapq.fp16(rng.standard_normal((N, r, d))))
    S0 = leapq.dequant(st)
    o, buf = kda_leapq.window_run(st, q, k, v, a, b, buf_dtype=np.float64)
    o_ex, S_ex = kda.kda_recurrent(_tn(q), _tn(k), _tn(v), _tn(a), b.T, S0)
    scale = np.abs(o_ex).max()
    np.testing.assert_allclose(o, _tn(o_ex), rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(kda_leapq.rebuild(st, buf), S_ex, rtol=0, atol=1e-12 * np.abs(S_ex).max())


def test_eq10_readout_equals_dense_eq4_state():
    rng = np.random.default_rng(22)
    N, d, m = 3, 16, 9
    S0 = rng.standard_normal((N, d, d))
    st = leapq.flush(S0, rng.standard_normal((d, 4)), rank=4)
    buf = [(rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.uniform(0.5, 1, (N, d)))
           for _ in range(m)]
    y = rng.standard_normal((N, d))
    dense = kda_leapq.rebuild(st, buf)
    np.testing.assert_allclose(kda_leapq.readout(st, buf, y), np.einsum("nvk,nk->nv", dense, y),
                               atol=1e-12)
    # eq. 4 term by term: S_hat_0 Gamma_{1:m} + sum_j u_j k_j^T Gamma_{j+1:m}
    prod = lambda recs: np.prod(np.stack([bb[2] for bb in recs] + [np.ones((N, d))]), axis=0)
    ref = leapq.dequant(st) * prod(buf)[:, None, :]
    for j, (kj, uj, _) in enumerate(buf):
        ref += uj[:, :, None] * (kj * prod(buf[j + 1:]))[:, None, :]
    np.testing.assert_allclose(dense, ref, atol=1e-12)


def test_equal_channel_decays_are_the_gdn_windowed_scheme():
    """KDA with alpha_t equal on every channel is Gated DeltaNet: the whole
    windowed scheme (flushes, compensators, smoothing) must match oracle.leapq."""
    rng = np.random.default_rng(23)
    T, N, d = 40, 3, 32
    q, k, v, a, b = _inputs(rng, T, N, d)
    a1 = a[..., 0]                                     # one decay per (token, head)
    av = np.repeat(a1[..., None], d, axis=-1)
    S0 = 0.1 * rng.standard_normal((N, d, d))
    Q0 = rng.standard_normal((d, 4))
    ref = leapq.decode_run(q, k, v, a1, b, S0, Q0, window=8, rank=4)
    got = kda_leapq.decode_run(q, k, v, av, b, S0, Q0, window=8, rank=4)
    np.testing.assert_allclose(got["o"], ref["o"], rtol=0, atol=1e-10 * np.abs(ref["o"]).max())
    np.testing.assert_array_equal(got["st"]["Z"], ref["st"]["Z"])


def test_window_one_no_extras_equals_per_token_rounding_eq2():
    rng = np.random.default_rng(24)
    T, N, d = 24, 3, 16
    q, k, v, a, b = _inputs(rng, T, N, d)
    S0 = 0.05 * rng.standard_normal((N, d, d))
    o1, Z1, s1 = kda_leapq.per_step_int8(q, k, v, a, b, S0)
    r = kda_leapq.decode_run(q, k, v, a, b, S0, None, window=1, rank=0, smooth_mode=2,
                             buf_dtype=np.float64)
    np.testing.assert_array_equal(r["st"]["Z"], Z1)
    np.testing.assert_array_equal(r["st"]["s"], s1)
    np.testing.assert_allclose(r["o"], o1, rtol=0, atol=1e-12)


def test_windowed_error_stays_near_the_exact_recurrence():
    """Trend on a small head with decays near 1 (parity unpinned: a statement
    about accuracy, not an identity): rounding once per window keeps the read-outs
    within a few percent of the exact recurrence, and per-token rounding of the
    same state does worse."""
    rng = np.random.default_rng(25)
    T, N, d = 128, 4, 32
    q, k, v, a, b = _inputs(rng, T, N, d, amu=5.0)
    S0 = 0.2 * rng.standard_normal((N, d, d))
    Q0 = rng.standard_normal((d, 4))
    o_ex, _ = kda.kda_recurrent(_tn(q), _tn(k), _tn(v), _tn(a), b.T, S0)
    o_ex = _tn(o_ex)
    win = kda_leapq.decode_run(q, k, v, a, b, S0, Q0, window=16, rank=4)["o"]
    step = kda_leapq.per_step_int8(q, k, v, a, b, S0)[0]
    e_win = np.abs(win - o_ex).max() / np.abs(o_ex).max()
    e_step = np.abs(step - o_ex).max() / np.abs(o_ex).max()
    assert e_win < 0.05
    assert e_win < e_step

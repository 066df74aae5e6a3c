"""GPU parity of gdn_chunk_bwd (the chunk-form backward of the GDN UT forward: state
and state-gradient scans, WY gradients, the decay gradient from q.dq - v.dv) against
the fp64 reverse-mode oracle ``oracle.gdn.gdn_recurrent_bwd``.

bf16 inputs and gradient outputs, bf16 MFMA operands (states, state gradients, the
WY factors and the intermediate gradients rounded to bf16) with fp32 accumulation:
max-abs error <= 2e-2 of max|ref| for dq, dk, dv, dalpha, dbeta and dS0."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gdn
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def _case(N, T, seed, S0_std=0.05):
    inp = synth.gdn_prefill(B=N, H=1, T=T, device="cpu", seed=seed, S0_std=S0_std)
    g = torch.Generator().manual_seed(seed + 1)
    dO = torch.randn((N, T, 128), generator=g).to(torch.bfloat16)
    dST = 0.1 * torch.randn((N, 128, 128), generator=g)
    return inp, dO, dST


def _check(out, inp, dO, dST, idx, what, S0=True, cond=False):
    """dalpha is compared as alpha * dalpha = d log alpha: the kernels form d log alpha and
    divide it by alpha exactly, so an absolute error in it grows by 1/alpha in dalpha and
    a check normalised by max|dalpha| would measure the smallest alpha of the input."""
    ref = gdn.gdn_recurrent_bwd(*(np64(inp[n][idx]) for n in ("q", "k", "v", "alpha", "beta")),
                                np64(inp["S0"][idx]) if S0 else None, np64(dO[idx]),
                                np64(dST[idx]) if dST is not None else None)
    a = np64(inp["alpha"][idx])
    errs = []
    for got, r, name in zip(out, ref, NAMES):
        g_ = np64(got[idx])
        if name == "dalpha":
            g_, r = a * g_, a * r
            if cond:
                errs.append(_check_dlog(g_, r, inp, ref, idx, what))
                continue
        errs.append(assert_rel(g_, r, TOL, f"{what} {name}"))
    say(f"  {what}: " + " ".join(f"{n} {e:.1e}" for n, e in zip(NAMES, errs)))


def _check_dlog(got, ref, inp, grads, idx, what):
    """d log alpha_t is the reverse sum over the rest of its chunk of q.dq - v.dv (plus
    the chunk-boundary term): where those terms nearly cancel, a relative error e of
    each term gives at most e sum_{s >= t} (|q_s.dq_s| + |v_s.dv_s|). Checked with e =
    5e-3, the accuracy of dq and dv themselves; returns the error relative to
    max |d log alpha| for the log."""
    q, v = np64(inp["q"][idx]), np64(inp["v"][idx])
    terms = np.abs(np.einsum("ntk,ntk->nt", q, grads[0])) + np.abs(np.einsum("ntv,ntv->nt", v, grads[2]))
    N, T = terms.shape
    c = terms.reshape(N, T // 64, 64)
    bound = 5e-3 * np.cumsum(c[..., ::-1], axis=-1)[..., ::-1].reshape(N, T) + 1e-6 * np.abs(ref).max()
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{what} d log alpha: {np.max(err / bound):.2f}x the conditioning bound"
    return float(err.max() / np.abs(ref).max())


@pytest.mark.parametrize("N,T", [(3, 192), (1, 64), (8, 128)])
def test_small_against_reverse_mode(N, T):
    """N = 8 takes the XCD-grouped scan blocks, the others the plain mapping."""
    dev = need_gpu()
    say(f"gdn_chunk_bwd: N={N} T={T}")
    inp, dO, dST = _case(N, T, 1100 + N)
    d = {k_: t.to(dev) for k_, t in inp.items()}
    out = m.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO.to(dev), S0=d["S0"],
                          dST=dST.to(dev))
    torch.cuda.synchronize()
    _check(out, inp, dO, dST, slice(None), f"N={N} T={T}")


def test_no_state_and_no_final_state_gradient():
    dev = need_gpu()
    inp, dO, _ = _case(2, 128, 1150, S0_std=0.0)
    d = {k_: t.to(dev) for k_, t in inp.items()}
    out = m.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO.to(dev))
    torch.cuda.synchronize()
    _check(out, inp, dO, None, slice(None), "S0 = dST = 0", S0=False)


def test_empty_sequence_passes_the_state_gradient():
    dev = need_gpu()
    e = torch.empty((2, 0, 128), dtype=torch.bfloat16, device=dev)
    s = torch.empty((2, 0), device=dev)
    dST = torch.randn((2, 128, 128), device=dev)
    *_, dS0 = m.gdn_chunk_bwd(e, e, e, s, s, e, S0=torch.randn((2, 128, 128), device=dev), dST=dST)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dST)


def test_full_size_config_sampled():
    """B=1 x H=32 heads of 16,384 tokens (the GDN prefill workload, zero initial
    state), in the benchmark's launch configuration; two heads checked against the
    reverse-mode oracle."""
    dev = need_gpu()
    say("gdn_chunk_bwd: B=1 H=32 T=16384")
    inp = synth.gdn_prefill(device=dev)
    g = torch.Generator(device=dev).manual_seed(91)
    dO = torch.randn(inp["q"].shape, generator=g, device=dev).to(torch.bfloat16)
    ws = m.gdn_chunk_bwd_workspace(32, 16384)
    out = m.gdn_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dO, workspace=ws)
    torch.cuda.synchronize()
    idx = torch.tensor([0, 21])
    host = {k_: t.cpu() for k_, t in inp.items()}
    _check(tuple(t.cpu() for t in out), host, dO.cpu(), None, idx, "full", S0=False)


@pytest.mark.parametrize("case", ["no_decay_no_write", "fast_decay_full_write"])
def test_degenerate_gates(case):
    """alpha = 1 with beta = 0 on half the tokens (pure state carry, no decay), and
    alpha down to 0.02 with beta = 1 (the state forgets within a few tokens and every
    write replaces the value along k): the gradients still match reverse mode."""
    dev = need_gpu()
    say(f"gdn_chunk_bwd: degenerate gates, {case}")
    N, T = 2, 128
    inp, dO, dST = _case(N, T, 1170)
    if case == "no_decay_no_write":
        inp["alpha"] = torch.ones_like(inp["alpha"])
        inp["beta"][:, ::2] = 0.0
    else:
        g = torch.Generator().manual_seed(1171)
        inp["alpha"] = 0.02 + 0.5 * torch.rand(inp["alpha"].shape, generator=g)
        inp["beta"] = torch.ones_like(inp["beta"])
    d = {k_: t.to(dev) for k_, t in inp.items()}
    out = m.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO.to(dev), S0=d["S0"],
                          dST=dST.to(dev))
    torch.cuda.synchronize()
    # fast decays with beta = 1: q.dq and v.dv nearly cancel within a chunk
    _check(out, inp, dO, dST, slice(None), case, cond=case == "fast_decay_full_write")

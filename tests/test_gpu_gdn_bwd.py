"""GPU parity of gdn_chunk_bwd (the chunk-form backward of the GDN UT forward: state
and state-gradient scans, WY gradients, the decay gradient from q.dq - v.dv) against
the fp64 reverse-mode oracle ``oracle.gdn.gdn_recurrent_bwd``.

bf16 inputs and gradient outputs, bf16 MFMA operands (states, state gradients, the
WY factors and the intermediate gradients rounded to bf16) with fp32 accumulation:
max-abs error <= 2e-2 of max|ref| for dq, dk, dv, dalpha, dbeta and dS0."""
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


def _check(out, inp, dO, dST, idx, what, S0=True):
    ref = gdn.gdn_recurrent_bwd(*(np64(inp[n][idx]) for n in ("q", "k", "v", "alpha", "beta")),
                                np64(inp["S0"][idx]) if S0 else None, np64(dO[idx]),
                                np64(dST[idx]) if dST is not None else None)
    errs = [assert_rel(np64(got[idx]), r, TOL, f"{what} {name}") for got, r, name in zip(out, ref, NAMES)]
    say(f"  {what}: " + " ".join(f"{n} {e:.1e}" for n, e in zip(NAMES, errs)))


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

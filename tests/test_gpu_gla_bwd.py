"""GPU parity of gla_chunk_bwd (ZeCO's chunkwise backward: reverse state-gradient
scan plus per-chunk intra/inter gradients) against the fp64 reverse-mode oracle
``oracle.gla.gla_recurrent_bwd``.

bf16 inputs and gradient outputs, bf16 MFMA operands (states, state gradients and
gate-scaled keys and queries rounded to bf16) with fp32 accumulation: max-abs error
<= 2e-2 of max|ref| for dq, dk, dv, d log_g and dS0."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gla
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _grads(N, T, dev, seed, full=False):
    inp = synth.gla_prefill(B=N, H=1, T=T, device="cpu", seed=seed) if not full else None
    g = torch.Generator().manual_seed(seed + 1)
    dO = torch.randn((N, T, 128), generator=g).to(torch.bfloat16)
    dST = 0.1 * torch.randn((N, 128, 128), generator=g)
    return inp, dO, dST


def _check(out, inp, dO, dST, idx, what):
    ref = gla.gla_recurrent_bwd(*(np64(inp[n][idx]) for n in ("q", "k", "v", "log_g", "S0")),
                                np64(dO[idx]), np64(dST[idx]))
    errs = []
    for got, r, name in zip(out, ref, ("dq", "dk", "dv", "dlog_g", "dS0")):
        errs.append(assert_rel(np64(got[idx]), r, TOL, f"{what} {name}"))
    say(f"  {what}: " + " ".join(f"{n} {e:.1e}" for n, e in zip(("dq", "dk", "dv", "dg", "dS0"), errs)))


@pytest.mark.parametrize("N,T", [(3, 192), (1, 64), (4, 128)])
def test_small_against_reverse_mode(N, T):
    dev = need_gpu()
    say(f"gla_chunk_bwd: N={N} T={T}")
    inp, dO, dST = _grads(N, T, dev, 900 + N)
    d = {k_: t.to(dev) for k_, t in inp.items()}
    out = m.gla_chunk_bwd(d["q"], d["k"], d["v"], d["log_g"], dO.to(dev), S0=d["S0"], dST=dST.to(dev))
    torch.cuda.synchronize()
    _check(out, inp, dO, dST, slice(None), f"N={N} T={T}")


def test_no_final_state_gradient_and_zero_state():
    dev = need_gpu()
    N, T = 2, 128
    inp, dO, _ = _grads(N, T, dev, 950)
    d = {k_: t.to(dev) for k_, t in inp.items()}
    dq, dk, dv, dg, dS0 = m.gla_chunk_bwd(d["q"], d["k"], d["v"], d["log_g"], dO.to(dev))
    torch.cuda.synchronize()
    ref = gla.gla_recurrent_bwd(*(np64(inp[n]) for n in ("q", "k", "v", "log_g")), None, np64(dO))
    for got, r, name in zip((dq, dk, dv, dg, dS0), ref, ("dq", "dk", "dv", "dlog_g", "dS0")):
        assert_rel(np64(got), r, TOL, name)


def test_empty_sequence_passes_the_state_gradient():
    dev = need_gpu()
    e = torch.empty((2, 0, 128), dtype=torch.bfloat16, device=dev)
    eg = torch.empty((2, 0, 128), device=dev)
    dST = torch.randn((2, 128, 128), device=dev)
    S0 = torch.randn((2, 128, 128), device=dev)
    *_, dS0 = m.gla_chunk_bwd(e, e, e, eg, e, S0=S0, dST=dST)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dST)


def test_full_size_config_sampled():
    """B=4 x H=16 sequences of 4096 tokens (the GLA prefill workload) with its
    incoming state, in the benchmark's launch configuration; two sequences checked
    against the reverse-mode oracle."""
    dev = need_gpu()
    say("gla_chunk_bwd: B=4 H=16 T=4096")
    inp = synth.gla_prefill(device=dev)
    g = torch.Generator(device=dev).manual_seed(77)
    dO = torch.randn(inp["q"].shape, generator=g, device=dev).to(torch.bfloat16)
    dST = 0.1 * torch.randn(inp["S0"].shape, generator=g, device=dev)
    ws = m.gla_chunk_bwd_workspace(64, 4096)
    out = m.gla_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_g"], dO, S0=inp["S0"], dST=dST,
                          workspace=ws)
    torch.cuda.synchronize()
    idx = torch.tensor([5, 50])
    cpu = {k_: t[idx].cpu() for k_, t in inp.items()}
    ref = gla.gla_recurrent_bwd(*(np64(cpu[n]) for n in ("q", "k", "v", "log_g", "S0")),
                                np64(dO[idx]), np64(dST[idx]))
    for got, r, name in zip(out, ref, ("dq", "dk", "dv", "dlog_g", "dS0")):
        e = assert_rel(np64(got[idx]), r, TOL, name)
        say(f"  {name} err {e:.2e}")


@pytest.mark.parametrize("case", ["no_decay", "fast_decay"])
def test_degenerate_gates(case):
    """log-gates 0 (plain linear attention, nothing forgotten) and log-gates down to
    log 0.05 on every channel (the state forgets within a few tokens)."""
    dev = need_gpu()
    say(f"gla_chunk_bwd: degenerate gates, {case}")
    N, T = 2, 128
    inp, dO, dST = _grads(N, T, dev, 960)
    if case == "no_decay":
        inp["log_g"] = torch.zeros_like(inp["log_g"])
    else:
        g = torch.Generator().manual_seed(961)
        inp["log_g"] = torch.log(0.05 + 0.5 * torch.rand(inp["log_g"].shape, generator=g))
    d = {k_: t.to(dev) for k_, t in inp.items()}
    out = m.gla_chunk_bwd(d["q"], d["k"], d["v"], d["log_g"], dO.to(dev), S0=d["S0"], dST=dST.to(dev))
    torch.cuda.synchronize()
    _check(out, inp, dO, dST, slice(None), case)

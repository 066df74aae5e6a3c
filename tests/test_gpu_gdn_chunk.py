"""GPU parity of gdn_chunk_fwd (UT / WY chunk form) against the fp64 per-token
Gated DeltaNet recurrence.

bf16 inputs and outputs, bf16 MFMA operands with fp32 accumulation and an fp32
carried state: max-abs error <= 2e-2 of max|ref| for o and the final state."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gdn
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _ref(inp, idx, S0=True):
    return gdn.gdn_recurrent(np64(inp["q"][idx]), np64(inp["k"][idx]), np64(inp["v"][idx]),
                             np64(inp["alpha"][idx]), np64(inp["beta"][idx]),
                             np64(inp["S0"][idx]) if S0 else None)


@pytest.mark.parametrize("N,T", [(3, 192), (1, 64), (64, 128)])
def test_small_with_incoming_state(N, T):
    """N = 64 takes the 32-wide value-tile path, the others the 16-wide one."""
    dev = need_gpu()
    say(f"gdn_chunk_fwd: N={N} T={T}")
    inp = synth.gdn_prefill(B=N, H=1, T=T, device="cpu", seed=600 + N, S0_std=0.05)
    g = {k_: t.to(dev) for k_, t in inp.items()}
    o, ST = m.gdn_chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(inp, slice(None))
    e1 = assert_rel(np64(o), o_ref, TOL, "o")
    e2 = assert_rel(np64(ST), S_ref, TOL, "S_T")
    say(f"  o err {e1:.2e}  S err {e2:.2e}")


def test_full_size_config_sampled():
    """B=1 x H=32 heads of 16,384 tokens from a zero state, in the benchmark's
    launch configuration; 3 heads checked against the per-token recurrence."""
    dev = need_gpu()
    say("gdn_chunk_fwd: B=1 H=32 T=16384")
    inp = synth.gdn_prefill(device=dev)
    ws = m.gdn_chunk_workspace(32, 16384)
    o, ST = m.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None,
                            workspace=ws)
    torch.cuda.synchronize()
    idx = torch.tensor([0, 17, 31])
    o_ref, S_ref = _ref(inp, idx, S0=False)
    e1 = assert_rel(np64(o[idx]), o_ref, TOL, "o")
    e2 = assert_rel(np64(ST[idx]), S_ref, TOL, "S_T")
    say(f"  o err {e1:.2e}  S err {e2:.2e}")


def test_in_place_empty_and_shards():
    dev = need_gpu()
    inp = synth.gdn_prefill(B=2, H=2, T=384, device=dev, seed=21, S0_std=0.05)
    args = [inp[n] for n in ("q", "k", "v", "alpha", "beta")]
    o, S_full = m.gdn_chunk_fwd(*args, inp["S0"])
    # in place
    S = inp["S0"].clone()
    m.gdn_chunk_fwd(*args, S, ST=S)
    torch.cuda.synchronize()
    assert torch.equal(S, S_full)
    # T = 0 keeps the incoming state
    e = torch.empty((4, 0, 128), dtype=torch.bfloat16, device=dev)
    g0 = torch.empty((4, 0), device=dev)
    _, S_e = m.gdn_chunk_fwd(e, e, e, g0, g0, inp["S0"])
    torch.cuda.synchronize()
    assert torch.equal(S_e, inp["S0"])
    # shards split on a chunk boundary chain bitwise
    part = lambda x, s: x[:, s].contiguous()
    o1, S1 = m.gdn_chunk_fwd(*(part(x, slice(0, 128)) for x in args), inp["S0"])
    o2, S2 = m.gdn_chunk_fwd(*(part(x, slice(128, None)) for x in args), S1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], 1), o) and torch.equal(S2, S_full)


def test_workspace_and_shape_errors():
    dev = need_gpu()
    inp = synth.gdn_prefill(B=1, H=1, T=128, device=dev)
    args = [inp[n] for n in ("q", "k", "v", "alpha", "beta")]
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(m.GdnrtError) as ei:
        m.gdn_chunk_fwd(*args, None, workspace=small)
    assert ei.value.status == 1
    bad = synth.gdn_prefill(B=1, H=1, T=96, device=dev)
    with pytest.raises(m.GdnrtError) as ei:
        m.gdn_chunk_fwd(*(bad[n] for n in ("q", "k", "v", "alpha", "beta")))
    assert ei.value.status == 2


@pytest.mark.parametrize("case", ["no_decay_no_write", "fast_decay_full_write"])
def test_degenerate_gates(case):
    """alpha = 1 with beta = 0 on alternate tokens (the state carried unchanged
    through every other token) and alpha down to 0.02 with beta = 1 (the state forgets
    within a few tokens; each write replaces the value along k). The chunk form's
    decay ratios g_r / g_j span 0.02^63 within a chunk there."""
    dev = need_gpu()
    say(f"gdn_chunk_fwd: degenerate gates, {case}")
    N, T = 4, 192
    inp = synth.gdn_prefill(B=N, H=1, T=T, device="cpu", seed=1180, S0_std=0.05)
    if case == "no_decay_no_write":
        inp["alpha"] = torch.ones_like(inp["alpha"])
        inp["beta"][:, ::2] = 0.0
    else:
        g = torch.Generator().manual_seed(1181)
        inp["alpha"] = 0.02 + 0.5 * torch.rand(inp["alpha"].shape, generator=g)
        inp["beta"] = torch.ones_like(inp["beta"])
    d = {k_: t.to(dev) for k_, t in inp.items()}
    o, ST = m.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(inp, slice(None))
    e1 = assert_rel(np64(o), o_ref, TOL, "o")
    e2 = assert_rel(np64(ST), S_ref, TOL, "S_T")
    say(f"  o err {e1:.2e}  S err {e2:.2e}")

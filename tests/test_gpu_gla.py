"""GPU parity of gla_chunk_fwd against the fp64 per-token GLA recurrence.

bf16 inputs and outputs: max-abs error <= 2e-2 of max|ref| for o and for the
final state (the state is carried in fp32; its per-chunk updates go through
bf16 operands)."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gla
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _run_ref(inp, idx, T=None):
    sl = slice(None) if T is None else slice(0, T)
    return gla.gla_recurrent(np64(inp["q"][idx, sl]), np64(inp["k"][idx, sl]), np64(inp["v"][idx, sl]),
                             np64(inp["log_g"][idx, sl]), np64(inp["S0"][idx]))


@pytest.mark.parametrize("N,T", [(3, 320), (8, 128), (1, 64), (64, 192)])
def test_small_ragged(N, T):
    """Ragged sequence counts (XCD placement only when N % 8 == 0)."""
    dev = need_gpu()
    say(f"gla_chunk_fwd: N={N} T={T}")
    inp = synth.gla_prefill(B=N, H=1, T=T, device="cpu", seed=500 + N)
    g = {k_: t.to(dev) for k_, t in inp.items()}
    o, ST = m.gla_chunk_fwd(g["q"], g["k"], g["v"], g["log_g"], g["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = _run_ref(inp, slice(None))
    e1 = assert_rel(np64(o), o_ref, TOL, "o")
    e2 = assert_rel(np64(ST), S_ref, TOL, "S_T")
    say(f"  o err {e1:.2e}  S err {e2:.2e}")


def test_full_size_config_sampled():
    """B=4 x H=16 sequences of 4096 tokens with a nonzero incoming state, in the
    launch configuration the benchmark times; 4 sequences checked."""
    dev = need_gpu()
    say("gla_chunk_fwd: B=4 H=16 T=4096")
    inp = synth.gla_prefill(device=dev)
    o, ST = m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["S0"])
    torch.cuda.synchronize()
    idx = torch.tensor([0, 13, 38, 63])
    o_ref, S_ref = _run_ref(inp, idx)
    e1 = assert_rel(np64(o[idx]), o_ref, TOL, "o")
    e2 = assert_rel(np64(ST[idx]), S_ref, TOL, "S_T")
    say(f"  o err {e1:.2e}  S err {e2:.2e}")


def test_zero_and_in_place_state_and_empty():
    dev = need_gpu()
    inp = synth.gla_prefill(B=2, H=1, T=128, device=dev, seed=9)
    o0, S_a = m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], None)
    torch.cuda.synchronize()
    o_ref, S_ref = gla.gla_recurrent(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["log_g"]), None)
    assert_rel(np64(o0), o_ref, TOL, "o from zero")
    # in place: ST is S0
    S = inp["S0"].clone()
    m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], S, ST=S)
    torch.cuda.synchronize()
    _, S_ref = gla.gla_recurrent(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["log_g"]),
                                 np64(inp["S0"]))
    assert_rel(np64(S), S_ref, TOL, "in-place state")
    # T = 0: the final state is the incoming state
    e = torch.empty((2, 0, 128), dtype=torch.bfloat16, device=dev)
    _, S_e = m.gla_chunk_fwd(e, e, e, torch.empty((2, 0, 128), device=dev), inp["S0"])
    torch.cuda.synchronize()
    assert torch.equal(S_e, inp["S0"])


def test_shards_chain():
    """Two shards split on a chunk boundary, the second starting from the first's
    final state (one device's local computation from its incoming state), match the
    recurrence over the whole sequence. Each call cuts its sequences into segments by
    its own length, so the chained run rounds differently from a single call: both are
    checked against the recurrence."""
    dev = need_gpu()
    inp = synth.gla_prefill(B=2, H=4, T=512, device=dev, seed=11)
    o, S = m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["S0"])
    h = 192
    sl1, sl2 = slice(0, h), slice(h, None)
    part = lambda x, s: x[:, s].contiguous()
    o1, S1 = m.gla_chunk_fwd(*(part(inp[n], sl1) for n in ("q", "k", "v", "log_g")), inp["S0"])
    o2, S2 = m.gla_chunk_fwd(*(part(inp[n], sl2) for n in ("q", "k", "v", "log_g")), S1)
    torch.cuda.synchronize()
    o_ref, S_ref = gla.gla_recurrent(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["log_g"]),
                                     np64(inp["S0"]))
    assert_rel(np64(torch.cat([o1, o2], 1)), o_ref, TOL, "chained o")
    assert_rel(np64(S2), S_ref, TOL, "chained S_T")
    assert_rel(np64(o), o_ref, TOL, "one-call o")
    assert_rel(np64(S), S_ref, TOL, "one-call S_T")


def test_bad_shapes_rejected():
    dev = need_gpu()
    inp = synth.gla_prefill(B=1, H=1, T=100, device=dev)
    with pytest.raises(m.GdnrtError) as ei:
        m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["S0"])
    assert ei.value.status == 2

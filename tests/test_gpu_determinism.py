"""Run-twice bitwise determinism of the kernels that reduce across waves or blocks
(the race check): each call runs twice on the same inputs, into fresh outputs (and
from copies of any state it updates), and every result must be the same bits.

Covered: the LeapQuant decode step, flush and fused last-token flush (GDN and KDA),
whose blocks exchange partial sums through LDS across a barrier; the chunkwise
forwards (GLA, GDN, KDA) and backwards (GLA, GDN), whose preparation and serial
passes hand operands through a workspace and LDS."""
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from helpers import need_gpu, say

pytestmark = pytest.mark.gpu

FIELDS = ("codes", "vscale", "ksmooth", "ct_k", "ct_u", "buf_k", "buf_u", "buf_a")


def _copy(st):
    c = m.LeapqBuffers(st.N, rank=st.rank, window=st.window, kda=st.kda, bits=st.bits)
    for n in FIELDS:
        getattr(c, n).copy_(getattr(st, n))
    c.pos = st.pos
    return c


def _same(a, b, what):
    assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"{what} differs between runs"


def _same_state(a, b, what):
    for n in FIELDS:
        _same(getattr(a, n), getattr(b, n), f"{what}: {n}")


@pytest.mark.parametrize("kda", [False, True])
def test_leapq_kernels_run_twice(kda):
    dev = need_gpu()
    say(f"determinism: leapq kernels, kda={kda}")
    B, H, W = 16, 32, 16
    N = B * H
    gen = synth.kda_leapq_decode if kda else synth.leapq_decode
    inp = gen(B=B, H=H, steps=2 * W, device=dev)
    Q0 = inp["Q0"].to(dev)
    step = m.kda_leapq_decode_step if kda else m.leapq_decode_step
    flush = m.kda_leapq_window_flush if kda else m.leapq_window_flush
    fused = m.kda_leapq_decode_flush if kda else m.leapq_decode_flush
    tok = lambda t: [inp[n][t] for n in ("q", "k", "v", "alpha", "beta")]
    st = m.LeapqBuffers(N, rank=4, window=W, kda=kda)
    pre = [torch.empty((N, 128, 128), device=dev) for _ in range(2)]
    runs = []
    for r in range(2):                                       # encode the initial state twice
        s_ = m.LeapqBuffers(N, rank=4, window=W, kda=kda)
        flush(s_, Q0, dense=inp["S0"], pre_round=pre[r])
        runs.append(s_)
    torch.cuda.synchronize()
    _same_state(runs[0], runs[1], "encode")
    _same(pre[0], pre[1], "encode pre-rounding values")
    st = runs[0]
    for t in range(W - 1):                                   # every window position
        a, b = _copy(st), _copy(st)
        oa, ob = step(a, *tok(t)), step(b, *tok(t))
        torch.cuda.synchronize()
        _same(oa, ob, f"decode output at pos {t}")
        _same_state(a, b, f"decode at pos {t}")
        st = a
    a, b = _copy(st), _copy(st)
    oa, ob = fused(a, *tok(W - 1), Q0), fused(b, *tok(W - 1), Q0)      # last token + flush
    torch.cuda.synchronize()
    _same(oa, ob, "fused last-token output")
    _same_state(a, b, "fused flush")
    c, d = _copy(st), _copy(st)
    step(c, *tok(W - 1))
    step(d, *tok(W - 1))
    flush(c, Q0)                                             # the plain flush of a full window
    flush(d, Q0)
    torch.cuda.synchronize()
    _same_state(c, d, "flush")


def _twice(fn):
    outs = [fn() for _ in range(2)]
    torch.cuda.synchronize()
    return outs


def test_chunk_forwards_run_twice():
    dev = need_gpu()
    say("determinism: gla / gdn / kda chunk forwards")
    inp = synth.gla_prefill(B=4, H=4, T=512, device=dev)
    a, b = _twice(lambda: m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["S0"]))
    for x, y, n in zip(a, b, ("o", "ST")):
        _same(x, y, f"gla_chunk_fwd {n}")
    for kda in (False, True):
        gen = synth.kda_prefill if kda else synth.gdn_prefill
        fwd = m.kda_chunk_fwd if kda else m.gdn_chunk_fwd
        inp = gen(B=2, H=8, T=512, device=dev, S0_std=0.05)
        a, b = _twice(lambda: fwd(*(inp[n] for n in ("q", "k", "v", "alpha", "beta", "S0"))))
        for x, y, n in zip(a, b, ("o", "ST")):
            _same(x, y, f"{'kda' if kda else 'gdn'}_chunk_fwd {n}")


def test_chunk_backwards_run_twice():
    dev = need_gpu()
    say("determinism: gla / gdn chunk backwards")
    g = torch.Generator(device=dev).manual_seed(5)
    inp = synth.gla_prefill(B=4, H=4, T=512, device=dev)
    dO = torch.randn(inp["q"].shape, generator=g, device=dev).to(torch.bfloat16)
    dST = 0.1 * torch.randn(inp["S0"].shape, generator=g, device=dev)
    a, b = _twice(lambda: m.gla_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_g"], dO, inp["S0"], dST))
    for x, y, n in zip(a, b, ("dq", "dk", "dv", "dlog_g", "dS0")):
        _same(x, y, f"gla_chunk_bwd {n}")
    inp = synth.gdn_prefill(B=2, H=8, T=512, device=dev, S0_std=0.05)
    dO = torch.randn(inp["q"].shape, generator=g, device=dev).to(torch.bfloat16)
    dST = 0.1 * torch.randn(inp["S0"].shape, generator=g, device=dev)
    a, b = _twice(lambda: m.gdn_chunk_bwd(*(inp[n] for n in ("q", "k", "v", "alpha", "beta")), dO,
                                          S0=inp["S0"], dST=dST))
    for x, y, n in zip(a, b, ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")):
        _same(x, y, f"gdn_chunk_bwd {n}")

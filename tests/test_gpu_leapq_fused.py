"""GPU parity of leapq_decode_flush / kda_leapq_decode_flush: the window's last
token decoded inside the flush.

Against the fp64 oracle, teacher-forced on the GPU's own state: S_{W-1} is the
oracle's eq. 4 rebuild of the stored state and the W - 1 records the GPU buffered,
the last token is one step of the exact recurrence (oracle.gdn / oracle.kda) from
it, and the flush result is checked with the bounds of ``compare_flush``, widened by
the fp32 rounding of the token's update (the correction's 128-term dot product and
the rank-one add: 128 ulps of the terms they sum). Outputs 1e-4 of max|ref| (fp32
io), 2e-2 (bf16). Against the two-launch path (decode step, then flush): outputs as
above, and the two dequantised states within half a code step of each side."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gdn, kda, kda_leapq, leapq
from helpers import assert_rel, need_gpu, np64, say
from test_gpu_leapq import buffer, compare_flush, rebuild_error, stored, token_update_error

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def _copy(st):
    c = m.LeapqBuffers(st.N, rank=st.rank, window=st.window, kda=st.kda, bits=st.bits)
    for n in ("codes", "vscale", "ksmooth", "ct_k", "ct_u", "buf_k", "buf_u", "buf_a"):
        getattr(c, n).copy_(getattr(st, n))
    c.pos = st.pos
    return c


@pytest.mark.parametrize("kda_mode", [False, True])
@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_last_token_and_flush(kda_mode, io):
    dev = need_gpu()
    say(f"leapq decode+flush: kda={kda_mode} io={io}")
    B, H, W, windows = 8, 8, 16, 2
    N = B * H
    gen = synth.kda_leapq_decode if kda_mode else synth.leapq_decode
    inp = gen(B=B, H=H, steps=W * windows, device="cpu")
    if io == torch.float32:
        for n in ("q", "k", "v"):
            inp[n] = inp[n].float()
    st = m.LeapqBuffers(N, rank=4, window=W, kda=kda_mode)
    Q0 = inp["Q0"].to(dev)
    step = m.kda_leapq_decode_step if kda_mode else m.leapq_decode_step
    (m.kda_leapq_window_flush if kda_mode else m.leapq_window_flush)(st, Q0, dense=inp["S0"].to(dev))
    tol = TOL_F32 if io == torch.float32 else TOL_BF16
    for w in range(windows):
        start = stored(st)
        t0, tl = w * W, w * W + W - 1
        for t in range(t0, tl):
            step(st, *(inp[n][t].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
        two = _copy(st)
        tok = [inp[n][tl].to(dev) for n in ("q", "k", "v", "alpha", "beta")]
        if kda_mode:
            o = m.kda_leapq_decode_flush(st, *tok, Q0)
            o2 = m.kda_leapq_decode_step(two, *tok)
            m.kda_leapq_window_flush(two, Q0)
        else:
            o = m.leapq_decode_flush(st, *tok, Q0)
            o2 = m.leapq_decode_step(two, *tok)
            m.leapq_window_flush(two, Q0)
        torch.cuda.synchronize()
        assert st.pos == 0
        # oracle: rebuild S_{W-1} from the GPU's buffer, one exact step of the recurrence
        S_prev = (kda_leapq.rebuild if kda_mode else leapq.rebuild)(start, buffer(st, W - 1))
        q1, k1, v1 = (np64(inp[n][tl])[:, None] for n in ("q", "k", "v"))
        a1, b1 = np64(inp["alpha"][tl])[:, None], np64(inp["beta"][tl])[:, None]
        o_ref, S_w = (kda.kda_recurrent if kda_mode else gdn.gdn_recurrent)(q1, k1, v1, a1, b1, S_prev)
        assert_rel(np64(o), o_ref[:, 0], tol, f"window {w} last output")
        assert_rel(np64(o2), o_ref[:, 0], tol, f"window {w} last output (two launches)")
        # the bound on the GPU's fp32 S_{W-1} and on the token's update applied to it
        dS = token_update_error(S_prev, rebuild_error(start, buffer(st, W - 1), kda=kda_mode),
                                k1[:, 0], v1[:, 0], np64(inp["alpha"][tl]), b1[:, 0])
        ref = leapq.flush(S_w, np64(inp["Q0"]), rank=4)
        flips, _, _ = compare_flush(st, ref, f"window {w} fused flush", S_w, dS=dS)
        rec, rec2 = leapq.dequant(stored(st)), leapq.dequant(stored(two))
        half = lambda s_: 0.5 * np64(s_.vscale)[:, :, None] / 127.0 * np64(s_.ksmooth)[:, None, :]
        gap = np.abs(rec - rec2) - (half(st) + half(two)) * (1 + 1e-4)
        assert gap.max() <= 1e-5 * np.abs(S_w).max(), f"window {w}: fused and two-launch states differ"
        say(f"  window {w}: code flips vs oracle {flips}")
    # the next window starts from the fused flush's state
    o = step(st, *(inp[n][0].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("bits", [6, 4])
def test_packed_widths_last_token_and_flush(bits):
    """The fused launch on packed 6- and 4-bit codes (rank 6, as the bench's rows): the
    last token against one exact step from the oracle's rebuild of the GPU's stored
    state, the fused flush against the oracle's flush at Q = 2^(b-1) - 1 within the
    bounds of ``compare_flush``, and against the two-launch path within half a code step
    of each side."""
    dev = need_gpu()
    say(f"leapq decode+flush at {bits} bits, rank 6")
    Q = (1 << (bits - 1)) - 1
    B, H, W = 4, 8, 16
    N = B * H
    inp = synth.leapq_decode(B=B, H=H, steps=W, device="cpu")
    Q0 = synth.compensator_start(r=6).to(dev)
    st = m.LeapqBuffers(N, rank=6, window=W, bits=bits)
    m.leapq_window_flush(st, Q0, dense=inp["S0"].to(dev))
    start = stored(st)
    start["Q"] = Q
    for t in range(W - 1):
        m.leapq_decode_step(st, *(inp[n][t].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
    two = _copy(st)
    tok = [inp[n][W - 1].to(dev) for n in ("q", "k", "v", "alpha", "beta")]
    o = m.leapq_decode_flush(st, *tok, Q0)
    o2 = m.leapq_decode_step(two, *tok)
    m.leapq_window_flush(two, Q0)
    torch.cuda.synchronize()
    S_prev = leapq.rebuild(start, buffer(st, W - 1))
    q1, k1, v1 = (np64(inp[n][W - 1])[:, None] for n in ("q", "k", "v"))
    a1, b1 = np64(inp["alpha"][W - 1])[:, None], np64(inp["beta"][W - 1])[:, None]
    o_ref, S_w = gdn.gdn_recurrent(q1, k1, v1, a1, b1, S_prev)
    assert_rel(np64(o), o_ref[:, 0], TOL_BF16, "last output")
    assert_rel(np64(o2), o_ref[:, 0], TOL_BF16, "last output (two launches)")
    dS = token_update_error(S_prev, rebuild_error(start, buffer(st, W - 1)), k1[:, 0], v1[:, 0],
                            np64(inp["alpha"][W - 1]), b1[:, 0])
    ref = leapq.flush(S_w, np64(Q0.cpu()), rank=6, bits=bits)
    flips, _, _ = compare_flush(st, ref, f"{bits}-bit fused flush", S_w, Q=Q, dS=dS)
    s1, s2 = stored(st), stored(two)
    s1["Q"] = s2["Q"] = Q
    rec, rec2 = leapq.dequant(s1), leapq.dequant(s2)
    half = lambda s_: 0.5 * np64(s_.vscale)[:, :, None] / Q * np64(s_.ksmooth)[:, None, :]
    gap = np.abs(rec - rec2) - (half(st) + half(two)) * (1 + 1e-4)
    assert gap.max() <= 1e-5 * np.abs(S_w).max(), "fused and two-launch states differ"
    say(f"  code flips vs oracle {flips}")


def test_edge_cases():
    dev = need_gpu()
    say("leapq decode+flush: window 1, rank 0, wrong position")
    inp = synth.leapq_decode(B=2, H=2, steps=2, device=dev)
    N = 4
    for rank, W in ((0, 1), (4, 1), (0, 4)):
        st = m.LeapqBuffers(N, rank=rank, window=W)
        Q0 = inp["Q0"].to(dev) if rank else torch.zeros((128, 0), device=dev)
        m.leapq_window_flush(st, Q0, dense=inp["S0"])
        for t in range(W - 1):
            m.leapq_decode_step(st, inp["q"][0], inp["k"][0], inp["v"][0], inp["alpha"][0], inp["beta"][0])
        start = stored(st)
        o = m.leapq_decode_flush(st, inp["q"][1], inp["k"][1], inp["v"][1], inp["alpha"][1], inp["beta"][1], Q0)
        torch.cuda.synchronize()
        S_prev = leapq.rebuild(start, buffer(st, W - 1)) if W > 1 else leapq.dequant(start)
        o_ref, S_w = gdn.gdn_recurrent(*(np64(inp[n][1])[:, None] for n in ("q", "k", "v")),
                                       np64(inp["alpha"][1])[:, None], np64(inp["beta"][1])[:, None], S_prev)
        assert_rel(np64(o), o_ref[:, 0], TOL_BF16, f"rank {rank} window {W} output")
        rec = leapq.dequant(stored(st))
        step = np64(st.vscale)[:, :, None] / 127.0 * np64(st.ksmooth)[:, None, :]
        assert np.all(np.abs(rec - S_w) <= 0.5 * step * (1 + 1e-3) + 1e-4 * np.abs(S_w).max())
    st = m.LeapqBuffers(N, rank=0, window=4)
    with pytest.raises(ValueError):
        m.leapq_decode_flush(st, inp["q"][0], inp["k"][0], inp["v"][0], inp["alpha"][0], inp["beta"][0],
                             torch.zeros((128, 0), device=dev))

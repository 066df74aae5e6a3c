"""GPU parity of kda_leapq_decode_step / kda_leapq_window_flush (Kimi Delta
Attention, one decay per key channel, in the windowed 8-bit state) against the
fp64 oracle ``oracle.kda_leapq``.

Tolerances as for the Gated DeltaNet windowed state: read-outs and corrections
1e-4 of max|ref| (fp32 io) when the oracle starts each window from the GPU's own
stored state; 2e-2 for bf16 outputs; flush results through the bounds of
``compare_flush`` (the compensator fit is ill-conditioned on outlier states)."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import kda, kda_leapq, leapq
from helpers import assert_rel, need_gpu, np64, rel_err, say, codes_of, pack_codes
from test_gpu_leapq import buffer, compare_flush, rebuild_error, stored

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_teacher_forced_windows(io):
    """Each window's read-outs from the GPU's stored state at the window start,
    then the flush of the GPU's own buffer against the oracle's flush of the same
    eq. 4 rebuild."""
    dev = need_gpu()
    say(f"kda_leapq decode: teacher-forced windows, io={io}")
    B, H, W, windows = 8, 8, 16, 3
    N = B * H
    inp = synth.kda_leapq_decode(B=B, H=H, steps=W * windows, device="cpu")
    if io == torch.float32:
        for n in ("q", "k", "v"):
            inp[n] = inp[n].float()
    st = m.LeapqBuffers(N, rank=4, window=W, kda=True)
    Q0 = inp["Q0"].to(dev)
    m.kda_leapq_window_flush(st, Q0, dense=inp["S0"].to(dev))
    for w in range(windows):
        start = stored(st)
        outs = []
        for t in range(w * W, (w + 1) * W):
            outs.append(m.kda_leapq_decode_step(st, *(inp[n][t].to(dev) for n in ("q", "k", "v", "alpha", "beta"))))
        o = torch.stack(outs)
        torch.cuda.synchronize()
        sl = slice(w * W, (w + 1) * W)
        o_ref, buf_ref = kda_leapq.window_run(start, np64(inp["q"][sl]), np64(inp["k"][sl]),
                                              np64(inp["v"][sl]), np64(inp["alpha"][sl]),
                                              np64(inp["beta"][sl]))
        u_gpu = np64(st.buf_u).transpose(1, 0, 2)
        u_ref = np.stack([b[1] for b in buf_ref])
        assert_rel(u_gpu, u_ref, TOL_F32, f"window {w} corrections")
        assert_rel(np64(o), o_ref, TOL_F32 if io == torch.float32 else TOL_BF16, f"window {w} outputs")
        # the buffer holds the token's keys and per-channel decays as given
        assert np.array_equal(np64(st.buf_a).transpose(1, 0, 2), np64(inp["alpha"][sl]))
        S_w = kda_leapq.rebuild(start, buffer(st, W))
        ref = leapq.flush(S_w, np64(inp["Q0"]), rank=4)
        dS = rebuild_error(start, buffer(st, W), kda=True)
        m.kda_leapq_window_flush(st, Q0)
        torch.cuda.synchronize()
        flips, _, _ = compare_flush(st, ref, f"window {w} flush", S_w, dS=dS)
        say(f"  window {w}: u err {rel_err(u_gpu, u_ref):.2e}, code flips {flips}")


@pytest.mark.parametrize("bits", [6, 4])
def test_packed_widths_window(bits):
    """Per-channel decays on packed 6- and 4-bit codes (rank 6): the encode (stored
    bytes equal to the host packer applied to the host-unpacked codes; codes within the
    flush bounds at Q = 2^(b-1) - 1), one teacher-forced window of read-outs and
    corrections (bf16 io), and the flush that closes it."""
    dev = need_gpu()
    say(f"kda_leapq at {bits} bits, rank 6: flush + window")
    Q = (1 << (bits - 1)) - 1
    B, H, W = 4, 8, 16
    N = B * H
    inp = synth.kda_leapq_decode(B=B, H=H, steps=W, device="cpu")
    Q0 = synth.compensator_start(r=6)
    st = m.LeapqBuffers(N, rank=6, window=W, kda=True, bits=bits)
    m.kda_leapq_window_flush(st, Q0.to(dev), dense=inp["S0"].to(dev))
    torch.cuda.synchronize()
    Z = codes_of(st)
    assert np.abs(Z).max() <= Q
    assert np.array_equal(st.codes.cpu().numpy().view(np.uint8), pack_codes(Z, bits))
    ref = leapq.flush(np64(inp["S0"]), np64(Q0), rank=6, bits=bits)
    compare_flush(st, ref, f"{bits}-bit encode", np64(inp["S0"]), Q=Q)
    start = stored(st)
    start["Q"] = Q
    outs = [m.kda_leapq_decode_step(st, *(inp[n][t].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
            for t in range(W)]
    torch.cuda.synchronize()
    o_ref, buf_ref = kda_leapq.window_run(start, *(np64(inp[n]) for n in ("q", "k", "v", "alpha", "beta")))
    u_gpu = np64(st.buf_u).transpose(1, 0, 2)
    assert_rel(u_gpu, np.stack([b_[1] for b_ in buf_ref]), TOL_F32, "corrections")
    e = assert_rel(np64(torch.stack(outs)), o_ref, TOL_BF16, "outputs")
    S_w = kda_leapq.rebuild(start, buffer(st, W))
    ref = leapq.flush(S_w, np64(Q0), rank=6, bits=bits)
    dS = rebuild_error(start, buffer(st, W), kda=True)
    m.kda_leapq_window_flush(st, Q0.to(dev))
    torch.cuda.synchronize()
    flips, _, _ = compare_flush(st, ref, f"{bits}-bit window flush", S_w, Q=Q, dS=dS)
    say(f"  outputs {e:.2e}, code flips {flips}")


def test_flush_mid_window():
    """A flush after fewer than W tokens rebuilds from the records it has."""
    dev = need_gpu()
    N, W, m_ = 16, 16, 5
    inp = synth.kda_leapq_decode(B=2, H=8, steps=m_, device="cpu")
    for n in ("q", "k", "v"):
        inp[n] = inp[n].float()
    st = m.LeapqBuffers(N, rank=4, window=W, kda=True)
    Q0 = inp["Q0"].to(dev)
    m.kda_leapq_window_flush(st, Q0, dense=inp["S0"].to(dev))
    start = stored(st)
    for t in range(m_):
        m.kda_leapq_decode_step(st, *(inp[n][t].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
    torch.cuda.synchronize()
    S_w = kda_leapq.rebuild(start, buffer(st, m_))
    ref = leapq.flush(S_w, np64(inp["Q0"]), rank=4)
    m.kda_leapq_window_flush(st, Q0)
    torch.cuda.synchronize()
    compare_flush(st, ref, "mid-window flush", S_w, dS=rebuild_error(start, buffer(st, m_), kda=True))


def test_free_running_full_head_count():
    """512 streams x 32 heads in the benchmark's launch configuration, 48 tokens
    (three windows); sampled heads against the oracle's own windowed run and the
    exact KDA recurrence."""
    dev = need_gpu()
    B, H, steps = 512, 32, 48
    N = B * H
    say(f"kda_leapq decode: free running B={B} H={H} steps={steps}")
    inp = synth.kda_leapq_decode(B=B, H=H, steps=steps, device=dev)
    st = m.LeapqBuffers(N, rank=4, window=16, kda=True)
    Q0 = inp["Q0"].to(dev)
    m.kda_leapq_window_flush(st, Q0, dense=inp["S0"])
    outs = torch.empty((steps, N, 128), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        m.kda_leapq_decode_step(st, inp["q"][t], inp["k"][t], inp["v"][t], inp["alpha"][t],
                                inp["beta"][t], outs[t])
        if st.pos == st.window:
            m.kda_leapq_window_flush(st, Q0)
    torch.cuda.synchronize()
    heads = torch.tensor([0, 5, 16, 31, 32 * 77 + 9, 32 * 200 + 25, N - 1])
    sel = lambda x: np64(x[:, heads])
    ref = kda_leapq.decode_run(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["alpha"]),
                               sel(inp["beta"]), np64(inp["S0"][heads]), np64(inp["Q0"]))
    e = assert_rel(sel(outs), ref["o"], TOL_BF16, "outputs vs oracle windowed run")
    o_ex, _ = kda.kda_recurrent(*(np.swapaxes(sel(inp[n]), 0, 1) for n in ("q", "k", "v", "alpha")),
                                sel(inp["beta"]).T, np64(inp["S0"][heads]))
    e2 = rel_err(sel(outs), np.swapaxes(o_ex, 0, 1))
    assert e2 < 5e-2
    say(f"  vs oracle windowed {e:.2e}, vs exact recurrence {e2:.2e}")


def test_edge_cases():
    dev = need_gpu()
    st = m.LeapqBuffers(4, rank=4, window=4, kda=True)
    Q0 = torch.randn((128, 4), device=dev)
    m.kda_leapq_window_flush(st, Q0, dense=torch.zeros((4, 128, 128), device=dev))
    torch.cuda.synchronize()
    assert torch.all(st.codes == 0) and torch.isfinite(st.vscale).all()
    # tiny per-channel decays: the flush of a fully decayed window stays finite
    x = torch.zeros((4, 128), device=dev)
    g = torch.full((4, 128), 1e-30, device=dev)
    for _ in range(4):
        m.kda_leapq_decode_step(st, x, x, x + 1, g, torch.full((4,), 0.5, device=dev))
    with pytest.raises(m.GdnrtError) as ei:
        m.kda_leapq_decode_step(st, x, x, x, g, torch.full((4,), 0.5, device=dev))
    assert ei.value.status == 5
    m.kda_leapq_window_flush(st, Q0)
    torch.cuda.synchronize()
    for t in (st.vscale, st.ksmooth, st.ct_k.float(), st.ct_u.float()):
        assert torch.isfinite(t).all()
    # the GDN entry points refuse buffers laid out for per-channel decays
    with pytest.raises(ValueError):
        m.leapq_decode_step(st, x, x, x, g[:, 0], g[:, 0])

"""GPU parity of the LeapQuant variants against the fp64 oracle: the windowed state
at 6 and 4 bits with 6 compensator tokens, and the per-step BF16 and b-bit baselines
(the state re-rounded after every token; a run of tokens in one launch must equal the
same tokens in one-token launches bit for bit).

Tolerances: windowed read-outs as the 8-bit path (teacher forced from the GPU's own
stored state; outputs bf16: 2e-2, corrections fp32: 1e-4); flush pieces, scales and
codes within the propagated bounds of the 8-bit tests with the step s_v c_k / Q. Per
step: one token from a given stored state is exact up to the fp32-vs-fp64 decision at
a rounding tie (bf16 entries within one bf16 step, codes within one code step, on
< 1e-3 of the entries). Longer runs: the b-bit state is checked token by token from the
GPU's own stored state with the same criteria (a free run parts from the oracle's at
the first code flip, a whole code step, 1/7 of a row's range at 4 bits); the BF16
state, whose flips are one bf16 step, free-runs 64 tokens within 1e-2 of max|ref|."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gdn, leapq
from helpers import assert_rel, need_gpu, np64, rel_err, say, codes_of, pack_codes
from test_gpu_leapq import compare_flush, rebuild_error, stored

pytestmark = pytest.mark.gpu
TOL_F32, TOL_BF16 = 1e-4, 2e-2


@pytest.mark.parametrize("bits", [6, 4])
def test_narrow_width_flush_and_window(bits):
    """Encode the outlier initial state at b bits with 6 compensator tokens, then one
    window of 16 decode steps (teacher forced) and the flush that closes it."""
    dev = need_gpu()
    say(f"leapq {bits}-bit, rank 6: flush + window")
    Q = (1 << (bits - 1)) - 1
    B, H, W = 4, 8, 16
    N = B * H
    inp = synth.leapq_decode(B=B, H=H, steps=W, device="cpu")
    Q0 = synth.compensator_start(r=6)
    st = m.LeapqBuffers(N, rank=6, window=W, bits=bits)
    pre = torch.empty((N, 128, 128), device=dev)
    m.leapq_window_flush(st, Q0.to(dev), dense=inp["S0"].to(dev), pre_round=pre)
    torch.cuda.synchronize()
    ref = leapq.flush(np64(inp["S0"]), np64(Q0), rank=6, bits=bits)
    Z = codes_of(st)
    assert np.abs(Z).max() == Q
    # the stored bytes are the documented packing of those codes
    assert np.array_equal(st.codes.cpu().numpy().view(np.uint8), pack_codes(Z, bits))
    assert np.array_equal(leapq.round_codes(pre.cpu().numpy(), bits), Z)
    flips, _, _ = compare_flush(st, ref, f"{bits}-bit encode", np64(inp["S0"]), Q=Q)
    start = stored(st)
    start["Q"] = Q
    outs = [m.leapq_decode_step(st, *(inp[n][t].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
            for t in range(W)]
    torch.cuda.synchronize()
    o_ref, buf_ref = leapq.window_run(start, *(np64(inp[n]) for n in ("q", "k", "v", "alpha", "beta")))
    u_gpu = np64(st.buf_u).transpose(1, 0, 2)
    assert_rel(u_gpu, np.stack([b[1] for b in buf_ref]), TOL_F32, "corrections")
    e = assert_rel(np64(torch.stack(outs)), o_ref, TOL_BF16, "outputs")
    recs = [(np64(st.buf_k)[:, j], np64(st.buf_u)[:, j], np64(st.buf_a)[:, j]) for j in range(W)]
    S_w = leapq.rebuild(start, recs)
    ref = leapq.flush(S_w, np64(Q0), rank=6, bits=bits)
    m.leapq_window_flush(st, Q0.to(dev))
    torch.cuda.synchronize()
    f2, _, _ = compare_flush(st, ref, f"{bits}-bit window flush", S_w, Q=Q, dS=rebuild_error(start, recs))
    say(f"  outputs {e:.2e}, code flips {flips} / {f2}")


def _tokens(N, T, seed, io=torch.float32):
    g = torch.Generator().manual_seed(seed)
    q = torch.nn.functional.normalize(torch.randn((N, T, 128), generator=g), dim=-1).to(io)
    k = torch.nn.functional.normalize(torch.randn((N, T, 128), generator=g), dim=-1).to(io)
    v = torch.randn((N, T, 128), generator=g).to(io)
    a = torch.sigmoid(torch.randn((N, T), generator=g) + 4.0)
    b = torch.sigmoid(torch.randn((N, T), generator=g))
    return q, k, v, a, b


def test_per_step_bf16_one_token_and_run():
    dev = need_gpu()
    say("per-step bf16 state")
    N = 8
    q, k, v, a, b = _tokens(N, 64, 31)
    S0 = (0.05 * torch.randn((N, 128, 128), generator=torch.Generator().manual_seed(32))).to(torch.bfloat16)
    # one token: the stored state after it equals the oracle's bf16 rounding
    S = S0.to(dev).clone()
    o1 = m.gdn_decode_step_bf16_state(S, *(x[:, :1].contiguous().to(dev) for x in (q, k, v, a, b)))
    torch.cuda.synchronize()
    ref_o, ref_S = leapq.per_step_bf16(*(np.swapaxes(np64(x[:, :1]), 0, 1) for x in (q, k, v)),
                                       np64(a[:, :1]).T, np64(b[:, :1]).T, np64(S0))
    assert_rel(np64(o1), np.swapaxes(ref_o, 0, 1), 1e-5, "one-token outputs")
    got = np64(S)
    diff = got != ref_S
    # one bf16 step of the entry, or the fp32 rounding of a * s + u * k where the two
    # terms cancel (a few 2^-24 of the state's scale)
    ulp = np.maximum(np.abs(ref_S) * 2.0 ** -7, 8 * 2.0 ** -24 * np.abs(ref_S).max())
    bad = diff & (np.abs(got - ref_S) > ulp * 1.01)
    assert diff.mean() < 1e-3 and not bad.any(), (diff.mean(), got[bad][:4], ref_S[bad][:4])
    # 64 tokens free running: outputs and final state against the oracle's run
    S = S0.to(dev).clone()
    o = m.gdn_decode_step_bf16_state(S, *(x.to(dev) for x in (q, k, v, a, b)))
    torch.cuda.synchronize()
    ref_o, ref_S = leapq.per_step_bf16(*(np.swapaxes(np64(x), 0, 1) for x in (q, k, v)), np64(a).T,
                                       np64(b).T, np64(S0))
    e1 = assert_rel(np64(o), np.swapaxes(ref_o, 0, 1), 1e-2, "outputs over 64 tokens")
    e2 = assert_rel(np64(S), ref_S, 1e-2, "state after 64 tokens")
    # the same 64 tokens in one-token launches: bit for bit the run above
    S1 = S0.to(dev).clone()
    outs = [m.gdn_decode_step_bf16_state(S1, *(x[:, t:t + 1].contiguous().to(dev) for x in (q, k, v, a, b)))
            for t in range(64)]
    torch.cuda.synchronize()
    assert torch.equal(S, S1) and torch.equal(o, torch.cat(outs, dim=1)), "one launch differs from 64"
    say(f"  64 tokens: outputs {e1:.1e}, state {e2:.1e}")


@pytest.mark.parametrize("bits", [8, 4])
def test_per_step_int_one_token_and_run(bits):
    dev = need_gpu()
    say(f"per-step {bits}-bit state")
    Q = (1 << (bits - 1)) - 1
    N = 8
    q, k, v, a, b = _tokens(N, 64, 41 + bits)
    S0 = 0.05 * torch.randn((N, 128, 128), generator=torch.Generator().manual_seed(42))
    m0 = S0.abs().amax(dim=-1)
    Z0 = torch.clamp(torch.round(S0 * (Q / m0[:, :, None])), -Q, Q).to(torch.int8)
    Sd = np64(m0)[:, :, None] * Z0.numpy().astype(np.float64) / Q     # the stored state
    # one token from the stored state
    Z, mx = Z0.to(dev).clone(), m0.to(dev).clone()
    o1 = m.gdn_decode_step_int_state(Z, mx, bits, *(x[:, :1].contiguous().to(dev) for x in (q, k, v, a, b)))
    torch.cuda.synchronize()
    ref_o, ref_Z, ref_m = leapq.per_step_int8(*(np.swapaxes(np64(x[:, :1]), 0, 1) for x in (q, k, v)),
                                              np64(a[:, :1]).T, np64(b[:, :1]).T, Sd, bits=bits)
    assert_rel(np64(o1), np.swapaxes(ref_o, 0, 1), 1e-5, "one-token outputs")
    assert_rel(np64(mx), ref_m, 1e-6, "row maxima")
    dz = Z.cpu().numpy().astype(np.int32) - ref_Z.astype(np.int32)
    assert np.abs(dz).max() <= 1 and (dz != 0).mean() < 1e-3, (dz != 0).mean()
    # 64 tokens in one launch (the row stays in registers between tokens) equal 64
    # one-token launches bit for bit: the same step from the same stored state
    Z, mx = Z0.to(dev).clone(), m0.to(dev).clone()
    o = m.gdn_decode_step_int_state(Z, mx, bits, *(x.to(dev) for x in (q, k, v, a, b)))
    Z1, mx1 = Z0.to(dev).clone(), m0.to(dev).clone()
    outs, flips = [], 0
    for t in range(64):
        Zp, mp = Z1.cpu().numpy().astype(np.float64), np64(mx1)
        ot = m.gdn_decode_step_int_state(Z1, mx1, bits, *(x[:, t:t + 1].contiguous().to(dev) for x in (q, k, v, a, b)))
        torch.cuda.synchronize()
        outs.append(ot)
        # every step against the oracle's step from the GPU's own stored state (teacher
        # forcing): at these widths a code flip at a rounding tie changes an entry by a
        # whole code step, so free-running trajectories part at the first one
        ref_o, ref_Z, ref_m = leapq.per_step_int8(*(np.swapaxes(np64(x[:, t:t + 1]), 0, 1) for x in (q, k, v)),
                                                  np64(a[:, t:t + 1]).T, np64(b[:, t:t + 1]).T,
                                                  mp[:, :, None] * Zp / Q, bits=bits)
        assert_rel(np64(ot), np.swapaxes(ref_o, 0, 1), 1e-5, f"token {t} outputs")
        assert_rel(np64(mx1), ref_m, 1e-6, f"token {t} row maxima")
        dz = Z1.cpu().numpy().astype(np.int32) - ref_Z.astype(np.int32)
        assert np.abs(dz).max() <= 1 and (dz != 0).mean() < 1e-3, (t, (dz != 0).mean())
        flips += int((dz != 0).sum())
    torch.cuda.synchronize()
    assert torch.equal(Z, Z1) and torch.equal(mx, mx1), "64 tokens in one launch differ from 64 launches"
    assert torch.equal(o, torch.cat(outs, dim=1)), "outputs of one launch differ from 64 launches"
    say(f"  64 teacher-forced steps: {flips} code flips at ties")


def test_per_step_baselines_full_decode_shape_sampled():
    """512 streams x 32 heads, one token per launch as the benchmark times them:
    sampled heads of the BF16 and INT8 per-step states after 4 steps against the
    oracle's per-step schemes run from the same stored states."""
    dev = need_gpu()
    B, H, steps = 512, 32, 4
    N = B * H
    say(f"per-step baselines: B={B} H={H} steps={steps}")
    inp = synth.gdn_decode(B=B, H=H, steps=steps, device=dev)
    heads = torch.tensor([0, 7, 31, 32 * 100 + 3, 32 * 333 + 17, N - 1])
    S_bf = inp["S0"].to(torch.bfloat16)
    mx = inp["S0"].abs().amax(dim=-1)
    Z = torch.clamp(torch.round(inp["S0"] * (127.0 / mx)[..., None]), -127, 127).to(torch.int8)
    start_bf, start_Z, start_m = S_bf[heads].cpu(), Z[heads].cpu(), mx[heads].cpu()
    o_bf, o_i8 = [], []
    for t in range(steps):
        args = [inp[n_][t, :, None] for n_ in ("q", "k", "v", "alpha", "beta")]
        o_bf.append(m.gdn_decode_step_bf16_state(S_bf, *args)[:, 0])
        o_i8.append(m.gdn_decode_step_int_state(Z, mx, 8, *args)[:, 0])
    torch.cuda.synchronize()
    sel = lambda x: np64(x[:, heads])
    ins = [sel(inp[n_]) for n_ in ("q", "k", "v", "alpha", "beta")]
    ref_o, ref_S = leapq.per_step_bf16(*ins, np64(start_bf))
    assert_rel(np64(torch.stack(o_bf)[:, heads]), ref_o, TOL_BF16, "bf16 state outputs")
    assert_rel(np64(S_bf[heads]), ref_S, 1e-2, "bf16 state")
    Sd = np64(start_m)[:, :, None] * start_Z.numpy().astype(np.float64) / 127.0
    ref_o, ref_Z, ref_m = leapq.per_step_int8(*ins, Sd)
    assert_rel(np64(torch.stack(o_i8)[:, heads]), ref_o, TOL_BF16, "int8 state outputs")
    S_gpu = np64(mx[heads])[:, :, None] * Z[heads].cpu().numpy().astype(np.float64) / 127.0
    assert_rel(S_gpu, ref_m[:, :, None] * ref_Z.astype(np.float64) / 127.0, 2e-2, "int8 state")


def test_error_study_trend_long_memory():
    """Trend only (parity unpinned): the GPU error study on 1 stream x 32 heads over
    512 tokens in the long-memory regime orders per-token rounding above the window
    and the window above the window with compensator tokens and smoothing (8 bits)."""
    need_gpu()
    from delta_rule_recurrent_amd import error_study
    res = error_study.run(streams=1, heads=32, steps=512, every=256, regime="long", log=lambda s: None)
    e = {k_: v_["ordinary"][-1] for k_, v_ in res["schemes"].items()}
    say("  " + ", ".join(f"{k_} {100 * v_:.2f}%" for k_, v_ in e.items()))
    assert e["per-step int8"] > e["window int8"] > e["window int8 + 4 CT + smooth"], e
    assert e["per-step int4"] > e["window int4 + 6 CT + smooth"], e

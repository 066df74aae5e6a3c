"""Parity of the LeapQuant windowed INT8 decode at its own workload, horizon and
launch sequence: 512 streams x 32 heads (d = 128, two outlier key channels x50 per
head), 4,096 tokens = 256 windows of 16, every window run as the benchmark times it:
15 leapq_decode_step launches, then leapq_decode_flush (the last token decoded inside
the flush). The run is free: every window starts from the GPU's own stored state.

At windows spread over the horizon, sampled heads (slow and fast, across the batch)
are checked teacher-forced against the fp64 oracle ("LeapQuant" page, section "Fix
one: leap over a window", eq. 4 and eq. 10):
  * the 15 corrections u_t (fp32 in the buffer) within 1e-4 and the bf16 outputs
    within 2e-2 of max|ref|, from the GPU's stored state at the window start
    (oracle.leapq.window_run);
  * the last token: one exact step of the recurrence (oracle.gdn) from the oracle's
    eq. 4 rebuild of that state and the GPU's 15 records, output within 2e-2;
  * the flush against oracle.leapq.flush of that state, with the bounds of
    compare_flush propagated from the fp32 rebuild and update (no slack factor);
  * the codes against the oracle's quantiser applied to the residual the GPU's own
    fp16 compensators leave: these are the code flips of the run, each within one
    step wherever the propagated fp32 error is under a step.
The flip counts are printed."""
import types

import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gdn, leapq
from helpers import assert_rel, need_gpu, np64, rel_err, say
from test_gpu_leapq import EPS, buffer, compare_flush, rebuild_error, stored, token_update_error

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
CHECK_WINDOWS = (0, 1, 64, 128, 255)


def _snap(st, heads):
    """Copies of the sampled heads' stored state, shaped like LeapqBuffers' fields."""
    return types.SimpleNamespace(rank=st.rank, bits=st.bits, **{n: getattr(st, n)[heads].clone()
                                                  for n in ("codes", "vscale", "ksmooth", "ct_k", "ct_u")})


def test_config4_full_run_bench_launch_sequence():
    dev = need_gpu()
    B, H, W, steps = 512, 32, 16, 4096
    N = B * H
    say(f"leapq config 4: B={B} H={H} {steps} tokens, 15 decode steps + leapq_decode_flush per window")
    inp = synth.leapq_decode(B=B, H=H, steps=steps, device=dev)
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    st = m.LeapqBuffers(N, rank=4, window=W)
    Q0 = inp["Q0"].to(dev)
    Q0h = np64(inp["Q0"])
    m.leapq_window_flush(st, Q0, dense=inp["S0"])
    o = torch.empty((N, 128), dtype=torch.bfloat16, device=dev)
    heads = torch.tensor([0, 7, 15, 16, 23, 31, 32 * 100 + 3, 32 * 255 + 20, 32 * 400 + 17, N - 1],
                         device=dev)
    hc = heads.cpu()
    flips_oracle = flips_own = gt1_own = 0
    max_own = 0
    n_codes = 0
    for w in range(steps // W):
        check = w in CHECK_WINDOWS
        if check:
            start = stored(st, heads)
            outs = []
        for j in range(W - 1):
            t = w * W + j
            m.leapq_decode_step(st, q[t], k[t], v[t], a[t], b[t], o)
            if check:
                outs.append(o[heads].clone())
        t = w * W + W - 1
        if check:
            recs = buffer(st, W - 1, heads)            # synchronises; the 15 records
        m.leapq_decode_flush(st, q[t], k[t], v[t], a[t], b[t], Q0, o)
        if not check:
            continue
        o_last = o[heads].clone()
        snap = _snap(st, heads)
        torch.cuda.synchronize()
        sl = slice(w * W, w * W + W - 1)
        sel = lambda x: np64(x[sl][:, hc])
        o_ref, buf_ref = leapq.window_run(start, *(sel(x) for x in (q, k, v, a, b)))
        u_ref = np.stack([r_[1] for r_ in buf_ref])
        u_gpu = np.stack([r_[1] for r_ in recs])
        e_u = assert_rel(u_gpu, u_ref, TOL_F32, f"window {w} corrections")
        e_o = assert_rel(np64(torch.stack(outs)), o_ref, TOL_BF16, f"window {w} outputs")
        # the last token, one exact step from the eq. 4 rebuild of the GPU's records
        S_prev = leapq.rebuild(start, recs)
        one = lambda x: np64(x[t][hc])
        o1_ref, S_w = gdn.gdn_recurrent(one(q)[:, None], one(k)[:, None], one(v)[:, None],
                                        one(a)[:, None], one(b)[:, None], S_prev)
        e_l = assert_rel(np64(o_last), o1_ref[:, 0], TOL_BF16, f"window {w} last output")
        dS = token_update_error(S_prev, rebuild_error(start, recs), one(k), one(v), one(a), one(b))
        ref = leapq.flush(S_w, Q0h, rank=4)
        f1, mx1, g1 = compare_flush(snap, ref, f"window {w} flush", S_w, dS=dS)
        # code flips: the oracle's quantiser on the residual the GPU's own pieces leave
        ug, kg = np.swapaxes(np64(snap.ct_u), -1, -2), np64(snap.ct_k)
        R = S_w - ug @ kg
        enc = leapq.encode_residual(R)
        Z = snap.codes.cpu().numpy().astype(np.int32)
        dZ = np.abs(Z - enc["Z"].astype(np.int32))
        # |Z_gpu - Z| <= 1 + |R_gpu - R| / step_gpu + Q |1 - step / step_gpu| + 5 Q eps, with
        # |R_gpu - R| <= dS + (r + 1) eps (|S| + sum_r |u_r| |k_r|) (as in compare_flush)
        step = np64(snap.vscale)[:, :, None] * np64(snap.ksmooth)[:, None, :] / 127.0
        step_r = enc["s"][:, :, None] * enc["c"][:, None, :] / 127.0
        dR = dS + 5 * EPS * (np.abs(S_w) + np.abs(ug) @ np.abs(kg))
        with np.errstate(divide="ignore", invalid="ignore"):
            allow = np.where(step > 0, 1 + dR / step + 127 * np.abs(1 - step_r / step) + 127 * 5 * EPS, 1)
        assert np.all(dZ <= allow), f"window {w}: a code flip beyond its propagated bound"
        assert np.all(dZ[allow < 2] <= 1), f"window {w}: a code flip of more than one step"
        flips_oracle += f1
        flips_own += int((dZ > 0).sum())
        gt1_own += int((dZ > 1).sum())
        max_own = max(max_own, int(dZ.max()))
        n_codes += dZ.size
        say(f"  window {w}: u {e_u:.1e}, o {e_o:.1e}, last o {e_l:.1e}; flips vs oracle flush {f1} "
            f"(max {mx1}, >1: {g1}); flips on the GPU's own pieces {int((dZ > 0).sum())} (max {int(dZ.max())})")
    say(f"  code flips over {len(CHECK_WINDOWS)} checked windows x {len(hc)} heads ({n_codes} codes): "
        f"{flips_own} on the GPU's own compensators (largest {max_own}, {gt1_own} beyond one step); "
        f"{flips_oracle} against the oracle's own fit")
    assert flips_own <= 1e-3 * n_codes
    assert torch.isfinite(o.float()).all()

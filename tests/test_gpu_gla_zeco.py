"""GPU parity of the per-device calls of ZeCO's sequence-parallel GLA forward
(gla_shard_decay, gla_all_scan_step, gla_shard_output_correct) and backward
(gla_shard_bwd_state, the All-Scan step run backward, gla_chunk_bwd from the
received state gradient) against the fp64 oracle of ZeCO's phases and against the
per-token recurrence (and reverse mode through it) over the whole sequence.

The devices of a sequence-parallel run are played one after the other on the one
GPU: every device runs its shard's forward from a zero state and its cumulative
decays; the All-Scan then passes the state along the devices in order, key block
by key block; each device adds the received state's share to its outputs.

Tolerances: o and the final state 2e-2 of max|ref| (bf16 inputs and outputs, as
gla_chunk_fwd). The cumulative decays are products of fp32 chunk decays e^{b_C},
each formed from an fp32 sum of 64 log-gates: relative error within
4e-6 |log gamma~| + 1e-5 (a dropped or repeated chunk is off by a factor e^{b_C},
about e^-3 here). The All-Scan update is one fp32 fused multiply-add per element:
within 2^-23 (|gamma S_recv| + |S_local|) of the fp64 value of the same inputs."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gla
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
D = 128


def _edges(blocks):
    return [int(x) for x in np.linspace(0, D, blocks + 1).astype(int)]


def _chain(g, devices, blocks, S0):
    """The devices one after the other: local phase on each, then All-Scan in order
    (key blocks), then each device's output correction."""
    N, T, _ = g["q"].shape
    L = T // devices
    local = []
    for p in range(devices):
        sl = slice(p * L, (p + 1) * L)
        local.append(m.gla_shard_local(*(g[n][:, sl].contiguous() for n in ("q", "k", "v", "log_g"))))
    S_recv, outs, sent = S0, [], []
    e = _edges(blocks)
    for o, S_loc, gam, ws in local:
        S_send = torch.empty_like(S_loc)
        for k0, k1 in zip(e[:-1], e[1:]):
            m.gla_all_scan_step(S_loc, gam[:, -1], S_recv, S_send, k0, k1)
        m.gla_shard_output_correct(ws, gam, S_recv, o)
        outs.append(o)
        sent.append(S_send)
        S_recv = S_send
    return torch.cat(outs, 1), S_recv, local, sent


def _check_gamma(gam, log_g, C=64):
    """gam [N][nc+1][128] against exp of the log-gates summed over whole chunks."""
    lg = np.asarray(log_g, np.float64)
    N, T, _ = lg.shape
    ref = np.exp(np.concatenate([np.zeros((N, 1, D)), np.cumsum(lg.reshape(N, T // C, C, D).sum(2), axis=1)], 1))
    got = np64(gam)
    big = ref > 1e-30
    tol = 4e-6 * np.abs(np.log(np.where(big, ref, 1.0))) + 1e-5
    err = np.abs(got - ref) / np.where(big, ref, 1.0)
    assert np.all(err[big] <= tol[big]), f"gamma: worst relative error {err[big].max():.2e}"
    assert np.all((got[~big] >= 0) & (got[~big] <= 1e-29)), "gamma: underflowing decays not near zero"
    return float(err[big].max()) if big.any() else 0.0


@pytest.mark.parametrize("N,devices,L,blocks,zero_s0", [(3, 3, 192, 4, False), (8, 2, 256, 1, False),
                                                      (2, 4, 64, 2, True), (16, 2, 128, 8, False)])
def test_chain_small(N, devices, L, blocks, zero_s0):
    """Several devices (L tokens each) from a nonzero or zero incoming state; XCD
    placement of the correction only when N % 8 == 0."""
    dev = need_gpu()
    say(f"zeco chain: N={N} devices={devices} L={L} blocks={blocks} zero_s0={zero_s0}")
    inp = synth.gla_prefill(B=N, H=1, T=devices * L, device="cpu", seed=700 + N)
    g = {k_: t.to(dev) for k_, t in inp.items()}
    S0 = None if zero_s0 else g["S0"]
    o, ST, local, sent = _chain(g, devices, blocks, S0)
    torch.cuda.synchronize()
    f = {k_: np64(t) for k_, t in inp.items()}
    s0 = None if zero_s0 else f["S0"]
    o_ref, S_ref = gla.gla_recurrent(f["q"], f["k"], f["v"], f["log_g"], s0)
    e1 = assert_rel(np64(o), o_ref, TOL, "o")
    e2 = assert_rel(np64(ST), S_ref, TOL, "S_T")
    # per device: the decays, the local final state and the state it sends
    S_recv, eg = s0, 0.0
    for p, ((_, S_loc, gam, _), S_send) in enumerate(zip(local, sent)):
        sl = slice(p * L, (p + 1) * L)
        Ss, gam_ref = gla.zeco_local(f["k"][:, sl], f["v"][:, sl], f["log_g"][:, sl])
        eg = max(eg, _check_gamma(gam, f["log_g"][:, sl]))
        assert_rel(np64(S_loc), Ss[:, -1], TOL, f"device {p} local state")
        S_recv = gla.zeco_all_scan_step(Ss[:, -1], gam_ref[:, -1], S_recv, blocks)
        assert_rel(np64(S_send), S_recv, TOL, f"device {p} sent state")
    say(f"  o err {e1:.2e}  S err {e2:.2e}  gamma rel err {eg:.2e}")


def test_all_scan_step_elementwise():
    """One fp32 fma per element against fp64, key blocks touching only their
    channels, S_send in place of S_local, and the first device (nothing received)."""
    dev = need_gpu()
    gen = torch.Generator(device=dev).manual_seed(5)
    N = 5
    S_loc, S_recv = (torch.randn((N, D, D), generator=gen, device=dev) for _ in range(2))
    gam_full = torch.rand((N, 3, D), generator=gen, device=dev)
    gam = gam_full[:, 1]                                       # strided view: stride 3 * 128
    ref = np64(gam)[:, None, :] * np64(S_recv) + np64(S_loc)
    bound = 2.0 ** -23 * (np.abs(np64(gam)[:, None, :] * np64(S_recv)) + np.abs(np64(S_loc))) + 1e-30
    out = torch.full_like(S_loc, 7.0)
    m.gla_all_scan_step(S_loc, gam, S_recv, out, 32, 96)
    torch.cuda.synchronize()
    got = np64(out)
    assert np.all(np.abs(got[:, :, 32:96] - ref[:, :, 32:96]) <= bound[:, :, 32:96])
    assert np.all(got[:, :, :32] == 7.0) and np.all(got[:, :, 96:] == 7.0)
    inpl = S_loc.clone()
    for k0, k1 in zip(_edges(4)[:-1], _edges(4)[1:]):
        m.gla_all_scan_step(inpl, gam, S_recv, inpl, k0, k1)
    torch.cuda.synchronize()
    assert np.all(np.abs(np64(inpl) - ref) <= bound)
    first = m.gla_all_scan_step(S_loc, None, None)
    torch.cuda.synchronize()
    assert torch.equal(first, S_loc)


def test_full_size_shard_sampled():
    """One device's shard at the prefill workload's shape (B=4 x H=16 sequences of
    4096 tokens) receiving the workload's incoming state, in the launch
    configuration the benchmark times: local phase, an All-Scan step in 4 key
    blocks, the output correction. Against one gla_chunk_fwd from that state on
    every output, and against the oracle on 4 sampled sequences."""
    dev = need_gpu()
    say("zeco shard: B=4 H=16 T=4096")
    inp = synth.gla_prefill(device=dev)
    o, S_loc, gam, ws = m.gla_shard_local(inp["q"], inp["k"], inp["v"], inp["log_g"])
    S_send = torch.empty_like(S_loc)
    for k0, k1 in zip(_edges(4)[:-1], _edges(4)[1:]):
        m.gla_all_scan_step(S_loc, gam[:, -1], inp["S0"], S_send, k0, k1)
    m.gla_shard_output_correct(ws, gam, inp["S0"], o)
    o1, S1 = m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["S0"])
    torch.cuda.synchronize()
    e0 = assert_rel(np64(o), np64(o1), TOL, "o against one call")
    assert_rel(np64(S_send), np64(S1), TOL, "sent state against one call")
    idx = torch.tensor([0, 13, 38, 63])
    f = {k_: np64(inp[k_][idx]) for k_ in ("q", "k", "v", "log_g", "S0")}
    o_ref, S_ref = gla.gla_recurrent(f["q"], f["k"], f["v"], f["log_g"], f["S0"])
    e1 = assert_rel(np64(o[idx]), o_ref, TOL, "o")
    e2 = assert_rel(np64(S_send[idx]), S_ref, TOL, "S_T")
    eg = _check_gamma(gam[idx], f["log_g"])
    say(f"  vs one call {e0:.2e}  o err {e1:.2e}  S err {e2:.2e}  gamma rel err {eg:.2e}")


def test_empty_and_no_incoming_state():
    """T = 0: the decays are the ones row; no incoming state leaves o unchanged."""
    dev = need_gpu()
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    gam = m.gla_shard_decay(ws, 3, 0)
    torch.cuda.synchronize()
    assert gam.shape == (3, 1, D) and torch.equal(gam, torch.ones_like(gam))
    inp = synth.gla_prefill(B=2, H=1, T=128, device=dev, seed=11)
    o, S_loc, gam, ws = m.gla_shard_local(inp["q"], inp["k"], inp["v"], inp["log_g"])
    before = o.clone()
    m.gla_shard_output_correct(ws, gam, None, o)
    torch.cuda.synchronize()
    assert torch.equal(o, before)


# ------------------------------------------------------------------ backward

def _bwd_chain(g, dO, dST, devices, blocks, S0):
    """The backward over the devices played in turn: the forward chain for each
    device's incoming state, phase 1 on every device, the backward All-Scan from
    the last device, then each device's gradients from its incoming state and the
    state gradient it received. Returns the concatenated gradients, the state
    gradient the first device sends, and each device's (dS0 of its gradient pass,
    state gradient it sent)."""
    N, T, _ = g["q"].shape
    L = T // devices
    _, _, local, sent = _chain(g, devices, blocks, S0)
    S_in = [S0] + sent[:-1]
    sls = [slice(p * L, (p + 1) * L) for p in range(devices)]
    sh = [{n: g[n][:, sl].contiguous() for n in ("q", "k", "v", "log_g")} for sl in sls]
    dOs = [dO[:, sl].contiguous() for sl in sls]
    wss = [m.gla_chunk_bwd_workspace(N, L) for _ in range(devices)]
    dS_loc = [m.gla_shard_bwd_state(x["q"], x["k"], x["log_g"], d, workspace=w) for x, d, w in zip(sh, dOs, wss)]
    e = _edges(blocks)
    recv, send, d = [None] * devices, [None] * devices, dST
    for p in range(devices - 1, -1, -1):
        recv[p] = d
        out = torch.empty_like(dS_loc[p])
        for k0, k1 in zip(e[:-1], e[1:]):
            m.gla_all_scan_step(dS_loc[p], local[p][2][:, -1], d, out, k0, k1)
        send[p] = d = out
    grads = [m.gla_shard_bwd_grads(x["q"], x["k"], x["v"], x["log_g"], dOs[p], wss[p], S0=S_in[p], dST=recv[p])
             for p, x in enumerate(sh)]
    cat = [torch.cat([gr[i] for gr in grads], 1) for i in range(4)]
    return cat, d, [(gr[4], send[p]) for p, gr in enumerate(grads)]


@pytest.mark.parametrize("N,devices,L,blocks,zero_ends", [(3, 3, 128, 4, False), (8, 2, 192, 2, False),
                                                        (2, 4, 64, 1, True)])
def test_backward_chain_small(N, devices, L, blocks, zero_ends):
    """ZeCO's backward with the devices played in turn against reverse mode through
    the recurrence over the whole sequence; each device's gradient pass reproduces
    the state gradient its backward All-Scan step sent."""
    dev = need_gpu()
    say(f"zeco backward chain: N={N} devices={devices} L={L} blocks={blocks} zero_ends={zero_ends}")
    inp = synth.gla_prefill(B=N, H=1, T=devices * L, device="cpu", seed=740 + N)
    gen = torch.Generator().manual_seed(741 + N)
    dO = torch.randn((N, devices * L, D), generator=gen).to(torch.bfloat16)
    dST = 0.1 * torch.randn((N, D, D), generator=gen)
    g = {k_: t.to(dev) for k_, t in inp.items()}
    S0, dST_d = (None, None) if zero_ends else (g["S0"], dST.to(dev))
    cat, dS0, per = _bwd_chain(g, dO.to(dev), dST_d, devices, blocks, S0)
    torch.cuda.synchronize()
    f = {k_: np64(t) for k_, t in inp.items()}
    ref = gla.gla_recurrent_bwd(f["q"], f["k"], f["v"], f["log_g"], None if zero_ends else f["S0"], np64(dO),
                                None if zero_ends else np64(dST))
    errs = [assert_rel(np64(a), r, TOL, n) for a, r, n in zip(cat + [dS0], ref, ("dq", "dk", "dv", "dlog_g", "dS0"))]
    for p, (from_pass, sent) in enumerate(per):
        assert_rel(np64(from_pass), np64(sent), TOL, f"device {p}: gradient pass dS0 vs All-Scan send")
    say("  " + " ".join(f"{n} {e_:.1e}" for n, e_ in zip(("dq", "dk", "dv", "dg", "dS0"), errs)))


def test_bwd_state_against_oracle_at_shard_shape():
    """Phase 1 at the prefill shard's shape (64 x 4096 tokens) against the oracle's
    chunk recurrence on 4 sampled sequences, and against the dS0 of gla_chunk_bwd
    from the same incoming state with no state gradient arriving; the gradient pass
    in phase 1's workspace gives the same bits as gla_chunk_bwd."""
    dev = need_gpu()
    say("zeco bwd phase 1: B=4 H=16 T=4096")
    inp = synth.gla_prefill(device=dev)
    gen = torch.Generator(device=dev).manual_seed(77)
    dO = torch.randn(inp["q"].shape, generator=gen, device=dev).to(torch.bfloat16)
    ws = m.gla_chunk_bwd_workspace(64, 4096)
    dS_loc = m.gla_shard_bwd_state(inp["q"], inp["k"], inp["log_g"], dO, workspace=ws)
    dST = 0.1 * torch.randn(inp["S0"].shape, generator=gen, device=dev)
    reused = m.gla_shard_bwd_grads(inp["q"], inp["k"], inp["v"], inp["log_g"], dO, ws, S0=inp["S0"], dST=dST)
    full = m.gla_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_g"], dO, S0=inp["S0"], dST=dST)
    *_, dS0 = m.gla_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_g"], dO, S0=inp["S0"])
    torch.cuda.synchronize()
    for a, b, name in zip(reused, full, ("dq", "dk", "dv", "dlog_g", "dS0")):
        assert torch.equal(a, b), f"gla_shard_bwd_grads {name} differs from gla_chunk_bwd"
    e0 = assert_rel(np64(dS_loc), np64(dS0), TOL, "phase 1 vs gradient pass")
    idx = torch.tensor([0, 21, 42, 63])
    ref = gla.zeco_bwd_local_state(np64(inp["q"][idx]), np64(inp["log_g"][idx]), np64(dO[idx]))
    e1 = assert_rel(np64(dS_loc[idx]), ref, TOL, "phase 1 vs oracle")
    say(f"  vs gradient pass {e0:.1e}  vs oracle {e1:.1e}")

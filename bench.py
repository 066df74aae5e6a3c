"""Benchmark of the gated delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows decode,bf16_state,int8_state,kda,leapq,
                     leapq6,leapq4,kda_leapq,gla,zeco,gla_bwd,gdn,gdn_bwd,kda_chunk]

Headline (`value`): Gated DeltaNet decode of one layer, 512 streams x 32 heads,
d_k = d_v = 128, fp32 state resident in HBM, bf16 q/k/v; one step = one token for
every stream (one gdn_decode_step launch over 16,384 heads); `value` is
stream-tokens per second over K timed steps. The other rows of the hot path are
measured in the same run and reported under "rows".

Timing: W untimed warm-up steps, then K steps bracketed by synchronisation;
HIP events recorded on the stream the kernels run on give the per-launch time. The
prefill and backward rows take warm-up calls of their own on the buffers they then time:
10, and 30 for the GDN and KDA chunk calls, which reach their steady time only after some
tens of calls on fresh buffers (GDN: 540-555 us per call after 2 warm-up calls, 492 after
10, 474 after 30). The CPU baseline runs after every GPU row, so that no row follows the
tens of seconds the GPU idles meanwhile.
The CPU baseline times the fp64 oracle on a bounded sample of heads.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import delta_rule_recurrent_amd as m  # noqa: E402
from delta_rule_recurrent_amd import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA, published
D = 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed(fn, K, W):
    """Run fn(i) W times untimed, then K times between events on the current
    stream. Returns (ms per call, wall seconds)."""
    for i in range(W):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for i in range(K):
        fn(W + i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K, time.perf_counter() - t0


def per_step_median(fn, n=64, start=0):
    """Median over n consecutive calls of fn, each between its own pair of events on
    the current stream (the calls still run back to back)."""
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(s)
    for i in range(n):
        fn(start + i)
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    ts = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
    return ts[n // 2]


def timed_graph(fn, K, reps=20):
    """GPU time per call of a launch-bound call: ``reps`` calls captured in one HIP
    graph, the graph replayed K times between events (the host's launch cost per call
    would otherwise exceed the kernels' own time). Returns (ms per call, wall s)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    ms, wall = timed(lambda i: g.replay(), K, 2)
    del g
    return ms / reps, wall


# ------------------------------------------------------------------- decode

DECODE_B, DECODE_H = 512, 32
DECODE_WORKLOAD = "gdn_decode B=512 H=32 d_k=d_v=128 fp32 state, bf16 q/k/v, T=1 per launch"


def decode_bytes_per_head_step(io_bytes=2):
    # fp32 state read + written, q/k/v in, o out, alpha/beta in
    return 2 * D * D * 4 + 3 * D * io_bytes + D * io_bytes + 2 * 4


def bench_decode(K, W, gen_steps=256):
    B, H = DECODE_B, DECODE_H
    N = B * H
    log(f"[decode] generating B={B} H={H} steps={gen_steps}")
    inp = synth.gdn_decode(B=B, H=H, steps=gen_steps, device="cuda")
    S = inp["S0"].clone()
    o = torch.empty((N, 1, D), dtype=torch.bfloat16, device="cuda")
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))

    def step(i):
        t = i % gen_steps
        m.gdn_decode_step(S, q[t, :, None], k[t, :, None], v[t, :, None],
                          a[t, :, None], b[t, :, None], o)

    ms, wall = timed(step, K, W)
    med = per_step_median(step, 64, W + K)
    bytes_launch = decode_bytes_per_head_step() * N
    gbs = bytes_launch / (ms * 1e-3) / 1e9
    return dict(workload=DECODE_WORKLOAD,
                ms_per_step=ms, ms_per_step_median_of_64=med, tokens_per_s=B / (ms * 1e-3), head_steps=N,
                bytes_per_launch=bytes_launch, achieved_gbs=gbs, frac_hbm=gbs / PEAK_HBM_GBS,
                wall_s=wall), inp


def bench_decode_lowp(K, W, bits, gen_steps=256):
    """The per-step baselines at the GDN decode shape: the state stored in bf16
    (bits = 16) or as b-bit codes with one fp32 maximum per value row, re-rounded
    after every token; one launch over 16,384 heads per step."""
    B, H = DECODE_B, DECODE_H
    N = B * H
    name = "bf16_state" if bits == 16 else f"int{bits}_state"
    log(f"[{name}] generating B={B} H={H} steps={gen_steps}")
    inp = synth.gdn_decode(B=B, H=H, steps=gen_steps, device="cuda")
    o = torch.empty((N, 1, D), dtype=torch.bfloat16, device="cuda")
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    if bits == 16:
        S = inp["S0"].to(torch.bfloat16)
        state_bytes = D * D * 2

        def step(i):
            t = i % gen_steps
            m.gdn_decode_step_bf16_state(S, q[t, :, None], k[t, :, None], v[t, :, None],
                                         a[t, :, None], b[t, :, None], o)
    else:
        Qm = (1 << (bits - 1)) - 1
        mx = inp["S0"].abs().amax(dim=-1)
        Z = torch.clamp(torch.round(inp["S0"] * (Qm / mx)[..., None]), -Qm, Qm).to(torch.int8)
        state_bytes = D * D + D * 4

        def step(i):
            t = i % gen_steps
            m.gdn_decode_step_int_state(Z, mx, bits, q[t, :, None], k[t, :, None], v[t, :, None],
                                        a[t, :, None], b[t, :, None], o)
    ms, wall = timed(step, K, W)
    per_head = 2 * state_bytes + decode_bytes_per_head_step() - 2 * D * D * 4
    gbs = per_head * N / (ms * 1e-3) / 1e9
    del inp, q, k, v, a, b
    return dict(workload=f"gdn_decode B=512 H=32 d=128, state {'bf16' if bits == 16 else f'int{bits} + fp32 row max'}"
                         f" re-rounded every token, bf16 q/k/v, T=1 per launch",
                ms_per_step=ms, tokens_per_s=B / (ms * 1e-3), bytes_per_head_step=per_head,
                achieved_gbs=gbs, frac_hbm=gbs / PEAK_HBM_GBS, wall_s=wall)


def bench_kda(K, W, gen_steps=256):
    """Kimi Delta Attention decode (one decay per key channel) at the GDN decode
    shape: one kda_decode_step launch over 16,384 heads per step."""
    B, H = DECODE_B, DECODE_H
    N = B * H
    log(f"[kda] generating B={B} H={H} steps={gen_steps}")
    inp = synth.kda_decode(B=B, H=H, steps=gen_steps, device="cuda")
    S = inp["S0"].clone()
    o = torch.empty((N, 1, D), dtype=torch.bfloat16, device="cuda")
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))

    def step(i):
        t = i % gen_steps
        m.kda_decode_step(S, q[t, :, None], k[t, :, None], v[t, :, None],
                          a[t, :, None], b[t, :, None], o)

    ms, wall = timed(step, K, W)
    per_head = decode_bytes_per_head_step() + (D - 1) * 4     # alpha is a d_k vector
    bytes_launch = per_head * N
    gbs = bytes_launch / (ms * 1e-3) / 1e9
    del inp, S, q, k, v, a, b
    return dict(workload="kda_decode B=512 H=32 d_k=d_v=128 fp32 state, bf16 q/k/v, fp32 per-key-channel "
                         "decays, T=1 per launch",
                ms_per_step=ms, tokens_per_s=B / (ms * 1e-3), head_steps=N,
                bytes_per_launch=bytes_launch, achieved_gbs=gbs, frac_hbm=gbs / PEAK_HBM_GBS,
                wall_s=wall)


def cpu_baseline_decode(inp, target_s=15.0):
    """The fp64 oracle recurrence on a bounded sample of heads (every 8th head of
    the batch, slow and fast heads alike) over all generated steps, reported as
    stream-tokens per second (head-steps per second / 32 heads). The sample is cut
    into slices run by one thread per host core (numpy releases the interpreter
    lock inside its array loops); ``cores`` is the thread count used."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import gdn
    steps = inp["q"].shape[0]
    H = DECODE_H
    N = inp["q"].shape[1]
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    threads = max(1, min(16, threads))
    host = {n: inp[n].to("cpu", torch.float64).numpy() for n in ("q", "k", "v", "alpha", "beta")}

    def one(heads):
        args = [np.ascontiguousarray(np.swapaxes(host[n][:, heads], 0, 1))
                for n in ("q", "k", "v", "alpha", "beta")]
        gdn.gdn_recurrent(*args, inp["S0"][heads].to("cpu", torch.float64).numpy())

    def run(heads):
        parts = [p for p in np.array_split(heads, threads * 2) if len(p)]
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, parts))
        return time.perf_counter() - t0

    sample = np.arange(0, N, 8)
    probe = sample[:4 * threads]                       # calibration at the full step count
    per_head = run(probe) / len(probe)
    n_heads = int(min(len(sample), max(8 * threads, target_s / max(per_head, 1e-12))))
    heads = sample[:n_heads]
    dt = run(heads)
    return dict(value=n_heads * steps / dt / H, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{n_heads} heads (every 8th of 16,384) x {steps} decode steps of the "
                       f"B=512 H=32 workload in {dt:.1f} s on {threads} threads; "
                       f"stream-tokens/s = head-steps/s / 32")


# ------------------------------------------------------------------- LeapQuant

def leapq_bytes_per_head_window(W=16, rank=4, kda=False, fused=True, bits=8):
    """Algorithmic bytes of one head over one window. A decode step at position m
    reads codes 16,384 (8 bits; 12,288 at 6 bits, 8,192 at 4, packed) + scales 1,024 + compensators 4*r*128 + m buffered records
    (k, u fp32 and a) + q, k, v (bf16) and alpha, beta; it writes one record and o
    (bf16). With ``fused`` (the window's last token decoded inside its flush) the
    window is W - 1 such steps and one launch that reads the stored state, the
    W - 1 records and the token's inputs and writes o and the stored state; without
    it, W steps and a flush that reads the stored state and the W records and
    writes the stored state. With ``kda`` every decay is a 128-long fp32 vector
    (the token's alpha and each record's)."""
    stored = D * m.code_row_bytes(bits) + 2 * D * 4 + rank * 2 * D * 2   # 19,456 at r = 4, 8 bits
    a_b = D * 4 if kda else 4
    rec = 2 * D * 4 + a_b                                 # 1,028 (KDA 1,536)
    io_in, io_out = 3 * D * 2 + a_b + 4, D * 2
    step = lambda m: stored + m * rec + io_in + rec + io_out
    if fused:
        return sum(step(m) for m in range(W - 1)) + stored + (W - 1) * rec + io_in + io_out + stored
    return sum(step(m) for m in range(W)) + stored + W * rec + stored


def bench_leapq(tokens=4096, B=DECODE_B, H=DECODE_H, W=16, rank=4, kda=False, bits=8):
    """The windowed INT8 state over ``tokens`` decode steps (every window: W - 1
    decode launches, then the window's last token and its flush in one launch; the
    two-launch form, W decode launches and a flush, is timed beside it). With
    ``kda``: one decay per key channel (inputs are drawn for 256 steps and reused
    cyclically). ``bits`` 6 or 4: the codes stored packed at that width."""
    N = B * H
    tag = ("kda_leapq" if kda else "leapq") + (str(bits) if bits != 8 else "")
    gen = min(tokens, 256) if kda else tokens
    log(f"[{tag}] generating B={B} H={H} steps={gen}")
    inp = (synth.kda_leapq_decode if kda else synth.leapq_decode)(B=B, H=H, steps=gen, device="cuda")
    st = m.LeapqBuffers(N, rank=rank, window=W, kda=kda, bits=bits)
    Q0 = (inp["Q0"] if rank == inp["Q0"].shape[1] else synth.compensator_start(r=rank)).cuda()
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    o = torch.empty((N, D), dtype=torch.bfloat16, device="cuda")
    step = m.kda_leapq_decode_step if kda else m.leapq_decode_step
    flush = m.kda_leapq_window_flush if kda else m.leapq_window_flush
    last = m.kda_leapq_decode_flush if kda else m.leapq_decode_flush

    def run_window(w):
        for j in range(W - 1):
            t = (w * W + j) % gen
            step(st, q[t], k[t], v[t], a[t], b[t], o)
        t = (w * W + W - 1) % gen
        last(st, q[t], k[t], v[t], a[t], b[t], Q0, o)

    def run_window_two_launch(w):
        for j in range(W):
            t = (w * W + j) % gen
            step(st, q[t], k[t], v[t], a[t], b[t], o)
        flush(st, Q0)

    flush(st, Q0, dense=inp["S0"])      # encode the initial state
    n_win = tokens // W
    ms_win, wall = timed(run_window, n_win, 1)
    ms_win2, _ = timed(run_window_two_launch, n_win, 1)
    ms_step = ms_win / W
    bpw = leapq_bytes_per_head_window(W, rank, kda, bits=bits) * N
    bpw2 = leapq_bytes_per_head_window(W, rank, kda, fused=False, bits=bits) * N
    # per-kernel split from events around each launch of one window
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(W + 2)]
    ev[0].record(s)
    for j in range(W):
        step(st, q[j], k[j], v[j], a[j], b[j], o)
        ev[j + 1].record(s)
    flush(st, Q0)
    ev[W + 1].record(s)
    for j in range(W - 1):
        step(st, q[j], k[j], v[j], a[j], b[j], o)
    ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev2[0].record(s)
    last(st, q[W - 1], k[W - 1], v[W - 1], a[W - 1], b[W - 1], Q0, o)
    ev2[1].record(s)
    torch.cuda.synchronize()
    dec_ms = ev[0].elapsed_time(ev[W]) / W
    flush_ms = ev[W].elapsed_time(ev[W + 1])
    last_ms = ev2[0].elapsed_time(ev2[1])
    width = "INT8" if bits == 8 else f"{bits}-bit packed"
    res = dict(workload=f"{tag}_decode B={B} H={H} d=128, {width} residual + fp32 scales + {rank} fp16 "
                        f"compensators, {W}-token fp32 buffer"
                        f"{' with per-channel fp32 decays' if kda else ''}, {tokens} tokens",
               ms_per_step=ms_step, tokens_per_s=B / (ms_step * 1e-3),
               bytes_per_head_step=bpw / N / W, achieved_gbs=bpw / (ms_win * 1e-3) / 1e9,
               decode_kernel_ms=dec_ms, flush_kernel_ms=flush_ms, decode_flush_kernel_ms=last_ms,
               two_launch_ms_per_step=ms_win2 / W, two_launch_bytes_per_head_step=bpw2 / N / W,
               two_launch_achieved_gbs=bpw2 / (ms_win2 * 1e-3) / 1e9, wall_s=wall, decode_kernel_gbs=None)
    res["frac_hbm"] = res["achieved_gbs"] / PEAK_HBM_GBS
    del inp
    return res


# ------------------------------------------------------------------- prefill

def gla_chunk_work(C=64):
    """Algorithmic FLOPs (multiply-add = 2) of one chunk of one sequence, with the
    causal products at triangular size, and the dense-tile count MFMA executes."""
    tri = C * (C + 1) // 2
    alg = 2 * tri * D + 2 * C * D * D + 2 * tri * D + 2 * D * D * C   # QK^T, QS^T, AV, V^T K
    dense = 2 * C * C * D + 2 * C * D * D + 2 * C * C * D + 2 * D * D * C
    return alg, dense


def bench_gla(K=20, W=10, B=4, H=16, T=4096):
    N = B * H
    log(f"[gla] generating B={B} H={H} T={T}")
    inp = synth.gla_prefill(B=B, H=H, T=T, device="cuda")
    ws = m.gla_chunk_workspace(N, T)
    ST = torch.empty_like(inp["S0"])
    o = torch.empty_like(inp["q"])

    def run(i):
        m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["S0"], ST, o, ws)

    ms, wall = timed(run, K, W)
    alg, dense = gla_chunk_work()
    chunks = N * T // 64
    flops, dflops = alg * chunks, dense * chunks
    byts = N * T * D * (3 * 2 + 4 + 2) + 2 * N * D * D * 4    # q,k,v bf16, gates fp32, o bf16, S0, ST
    res = dict(workload=f"gla_chunk_fwd B={B} H={H} T={T} d=128 chunk 64, bf16 q/k/v, fp32 gates, "
                        f"fp32 incoming state",
               ms=ms, tokens_per_s=B * T / (ms * 1e-3), gflop=flops / 1e9, gflop_dense=dflops / 1e9,
               tflops=flops / (ms * 1e-3) / 1e12, tflops_dense=dflops / (ms * 1e-3) / 1e12,
               bytes=byts, achieved_gbs=byts / (ms * 1e-3) / 1e9,
               workspace_bytes=int(ws.numel()), wall_s=wall)
    res["frac_hbm"] = res["achieved_gbs"] / PEAK_HBM_GBS
    res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
    res["frac_mfma_dense"] = res["tflops_dense"] / PEAK_BF16_TFLOPS
    res["roofline_bound"] = "hbm"
    del inp, ws
    return res


def bench_zeco(K=20, W=10, B=4, H=16, T=4096, blocks=4):
    """The per-device work that ZeCO's sequence parallelism adds to a GLA prefill
    shard (one device's share at the prefill shape, receiving the workload's
    incoming state): the cumulative decays after the local forward, one All-Scan
    step in ``blocks`` key blocks, and the output correction. Each is timed on its
    own (the two small ones as graphs of 20 calls, their host launch cost excluded);
    the local forward from a zero state is timed beside them, and the backward's
    phase 1 (the local state gradient) after them."""
    N = B * H
    log(f"[zeco] generating B={B} H={H} T={T}")
    inp = synth.gla_prefill(B=B, H=H, T=T, device="cuda")
    o, S_loc, gam, ws = m.gla_shard_local(inp["q"], inp["k"], inp["v"], inp["log_g"])
    S_send = torch.empty_like(S_loc)
    edges = [int(x) for x in np.linspace(0, D, blocks + 1)]

    def local(i):
        m.gla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_g"], None, S_loc, o, ws, shard=True)

    def decay(i):
        m.gla_shard_decay(ws, N, T, gam)

    def scan(i):
        for k0, k1 in zip(edges[:-1], edges[1:]):
            m.gla_all_scan_step(S_loc, gam[:, -1], inp["S0"], S_send, k0, k1)

    def correct(i):
        m.gla_shard_output_correct(ws, gam, inp["S0"], o)

    ms_local, _ = timed(local, K, W)
    ms_decay, _ = timed_graph(decay, K)
    ms_scan, _ = timed_graph(scan, K)
    ms_corr, wall = timed(correct, K, W)
    del ws
    # backward phase 1: the local state gradient from the shard's own outputs
    g = torch.Generator(device="cuda").manual_seed(77)
    dO = torch.randn(inp["q"].shape, generator=g, device="cuda").to(torch.bfloat16)
    bws = m.gla_chunk_bwd_workspace(N, T)
    dS_loc = torch.empty_like(S_loc)

    def bwd_state(i):
        m.gla_shard_bwd_state(inp["q"], inp["k"], inp["log_g"], dO, dS_loc, bws)

    ms_bstate, _ = timed(bwd_state, K, W)
    gout = (torch.empty_like(inp["q"]), torch.empty_like(inp["k"]), torch.empty_like(inp["v"]),
            torch.empty_like(inp["log_g"]), torch.empty_like(S_loc))
    dS_recv = 0.1 * torch.randn(S_loc.shape, generator=g, device="cuda")

    def bwd_grads(i):   # the gradient pass in phase 1's workspace (its preparation reused)
        m.gla_shard_bwd_grads(inp["q"], inp["k"], inp["v"], inp["log_g"], dO, bws, inp["S0"], dS_recv, gout)

    ms_bgrads, _ = timed(bwd_grads, K, W)
    del bws, dO, gout
    nc = T // 64
    # correction: per chunk Q o e^b (bf16) and o in and out, one decay row; the state once per sequence
    corr_bytes = N * nc * (64 * D * 2 * 3 + D * 4) + N * D * D * 4
    corr_flops = 2 * N * T * D * D
    scan_bytes = 3 * N * D * D * 4 + N * D * 4
    decay_bytes = N * nc * D * 4 + N * (nc + 1) * D * 4
    res = dict(workload=f"ZeCO per-device steps on a gla_chunk_fwd shard B={B} H={H} T={T} d=128 chunk 64 "
                        f"(bf16 q/k/v, fp32 gates), incoming state fp32, All-Scan step in {blocks} key blocks",
               local_fwd_ms=ms_local, decay_ms=ms_decay, all_scan_step_ms=ms_scan, correct_ms=ms_corr,
               bwd_local_state_ms=ms_bstate, bwd_grads_reusing_prep_ms=ms_bgrads,
               extra_ms=ms_decay + ms_scan + ms_corr, exposed_after_receive_ms=ms_scan + ms_corr,
               overhead_vs_local=(ms_decay + ms_scan + ms_corr) / ms_local,
               correct_bytes=corr_bytes, correct_gbs=corr_bytes / (ms_corr * 1e-3) / 1e9,
               correct_tflops=corr_flops / (ms_corr * 1e-3) / 1e12,
               decay_gbs=decay_bytes / (ms_decay * 1e-3) / 1e9,
               all_scan_step_gbs=scan_bytes / (ms_scan * 1e-3) / 1e9, wall_s=wall)
    res["correct_frac_hbm"] = res["correct_gbs"] / PEAK_HBM_GBS
    res["roofline_bound"] = "hbm"
    del inp, o
    return res


def gla_bwd_work(C=64):
    """Algorithmic FLOPs of one chunk of the GLA backward: the forward state recompute
    (V^T K^) and the state-gradient scan (dO^T Q^), then A and dA (lower), dQ^ = dO S_b,
    dQ~ = dA K~ and dK~ = dA^T Q~ (triangular), dK^ = V dS_a, dV = A^T dO + K^ dS_a^T."""
    tri = C * (C + 1) // 2
    full, low = 2 * C * D * D, 2 * tri * D
    return 2 * full + (2 * low + full + 2 * low + full + low + full)


def bench_gla_bwd(K=10, W=10, B=4, H=16, T=4096):
    N = B * H
    log(f"[gla_bwd] generating B={B} H={H} T={T}")
    inp = synth.gla_prefill(B=B, H=H, T=T, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    dO = torch.randn(inp["q"].shape, generator=g, device="cuda").to(torch.bfloat16)
    dST = 0.1 * torch.randn(inp["S0"].shape, generator=g, device="cuda")
    ws = m.gla_chunk_bwd_workspace(N, T)
    out = (torch.empty_like(inp["q"]), torch.empty_like(inp["k"]), torch.empty_like(inp["v"]),
           torch.empty_like(inp["log_g"]), torch.empty_like(inp["S0"]))

    def run(i):
        m.gla_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_g"], dO, inp["S0"], dST, ws, out)

    ms, wall = timed(run, K, W)
    chunks = N * T // 64
    flops = gla_bwd_work() * chunks
    # reads q, k, v, dO (bf16), gates (fp32), S0, dST; writes dq, dk, dv (bf16), d gates, dS0
    byts = N * T * D * (4 * 2 + 4 + 3 * 2 + 4) + 3 * N * D * D * 4
    res = dict(workload=f"gla_chunk_bwd B={B} H={H} T={T} d=128 chunk 64: gradients of q, k, v, log-gates "
                        f"and the incoming state, bf16 in and out, fp32 gates",
               ms=ms, tokens_per_s=B * T / (ms * 1e-3), gflop=flops / 1e9,
               tflops=flops / (ms * 1e-3) / 1e12, bytes=byts, achieved_gbs=byts / (ms * 1e-3) / 1e9,
               workspace_bytes=int(ws.numel()), wall_s=wall)
    res["frac_hbm"] = res["achieved_gbs"] / PEAK_HBM_GBS
    res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
    res["roofline_bound"] = "hbm"
    del inp, ws, out
    return res


def gdn_bwd_work(C=64):
    """Algorithmic FLOPs of one chunk of one head in the GDN chunk-form backward: the
    forward's chunk operands (as gdn_chunk_work, without the state products), the state
    recompute (W S^T, U^T K^), the state-gradient scan (K^ dS^T, dO^T Q', dU^T W), then
    A and dA (lower), U, dU = A^T dO + K^ dS^T, dq = dA' K + dO S_b, dA'^T Q + U dS_a,
    dW = dU S_b, T^T dW and T^T dU (lower T), dL (strict lower, with the Gram matrix)
    and (dL' + dL'^T) K."""
    tri, stri = C * (C + 1) // 2, C * (C - 1) // 2
    full, low, slow = 2 * C * D * D, 2 * tri * D, 2 * stri * D
    fwd_ops = slow + 2 * C ** 3 // 3 + low + 2 * low + low   # Gram, inverse, A, W and U~, Q' (A W)
    scans = 2 * full + 3 * full
    grad1 = low + full + (low + full) + low + (low + full) + (low + full)
    grad2 = full + 2 * low + 3 * slow + 2 * C * C * D
    return fwd_ops + scans + grad1 + grad2


def bench_gdn_bwd(K=10, W=10, B=1, H=32, T=16384):
    N = B * H
    log(f"[gdn_bwd] generating B={B} H={H} T={T}")
    inp = synth.gdn_prefill(B=B, H=H, T=T, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(91)
    dO = torch.randn(inp["q"].shape, generator=g, device="cuda").to(torch.bfloat16)
    ws = m.gdn_chunk_bwd_workspace(N, T)
    out = (torch.empty_like(inp["q"]), torch.empty_like(inp["k"]), torch.empty_like(inp["v"]),
           torch.empty_like(inp["alpha"]), torch.empty_like(inp["beta"]), torch.empty_like(inp["S0"]))

    def run(i):
        m.gdn_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dO, None, None, ws, out)

    ms, wall = timed(run, K, W)
    flops = gdn_bwd_work() * (N * T // 64)
    # reads q, k, v, dO (bf16), alpha, beta; writes dq, dk, dv (bf16), dalpha, dbeta, dS0
    byts = N * T * (D * 4 * 2 + 2 * 4 + D * 3 * 2 + 2 * 4) + N * D * D * 4
    res = dict(workload=f"gdn_chunk_bwd B={B} H={H} T={T} d=128 chunk 64: gradients of q, k, v, alpha, beta "
                        f"and the incoming state, bf16 in and out, fp32 gates, zero initial state",
               ms=ms, tokens_per_s=B * T / (ms * 1e-3), gflop=flops / 1e9,
               tflops=flops / (ms * 1e-3) / 1e12, bytes=byts, achieved_gbs=byts / (ms * 1e-3) / 1e9,
               workspace_bytes=int(ws.numel()), wall_s=wall)
    res["frac_hbm"] = res["achieved_gbs"] / PEAK_HBM_GBS
    res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
    res["roofline_bound"] = "mfma (at the knee)"
    del inp, ws, out
    return res


def gdn_chunk_work(C=64):
    """Algorithmic FLOPs of one chunk of one head in the UT / WY form: Gram k.k
    (strict lower), triangular inverse (C^3/3 multiply-adds), scores q.k (lower),
    W and U~ (lower-triangular T times K, V), W S^T, Q S^T, A U (lower), U^T K;
    and the dense-tile count."""
    tri, stri = C * (C + 1) // 2, C * (C - 1) // 2
    alg = (2 * stri * D + 2 * C ** 3 // 3 + 2 * tri * D + 2 * 2 * tri * D
           + 2 * C * D * D * 2 + 2 * tri * D + 2 * D * D * C)
    dense = (2 * C * C * D * 2 + 2 * C ** 3 // 3 + 2 * 2 * C * C * D
             + 2 * C * D * D * 2 + 2 * C * C * D + 2 * D * D * C)
    return alg, dense


def bench_gdn_chunk(K=10, W=30, B=1, H=32, T=16384, kda=False):
    """Chunkwise prefill of the Gated DeltaNet workload; with ``kda`` the same shape
    with one decay per key channel and token (kda_chunk_fwd). The FLOP count is the
    GDN one (the per-channel decays only rescale operands)."""
    N = B * H
    tag = "kda_chunk" if kda else "gdn_chunk"
    log(f"[{tag}] generating B={B} H={H} T={T}")
    inp = (synth.kda_prefill if kda else synth.gdn_prefill)(B=B, H=H, T=T, device="cuda")
    ws = (m.kda_chunk_workspace if kda else m.gdn_chunk_workspace)(N, T)
    fwd = m.kda_chunk_fwd if kda else m.gdn_chunk_fwd
    ST = torch.empty((N, D, D), device="cuda")
    o = torch.empty_like(inp["q"])

    def run(i):
        fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, ST, o, ws)

    ms, wall = timed(run, K, W)
    alg, dense = gdn_chunk_work()
    chunks = N * T // 64
    flops, dflops = alg * chunks, dense * chunks
    a_b = D * 4 if kda else 4
    byts = N * T * (3 * D * 2 + a_b + 4 + D * 2) + N * D * D * 4   # q,k,v, alpha,beta, o, ST
    res = dict(workload=f"{tag}_fwd B={B} H={H} T={T} d=128 chunk 64, bf16 q/k/v (q, k "
                        f"L2-normalised), fp32 {'per-channel ' if kda else ''}gates, zero initial state",
               ms=ms, tokens_per_s=B * T / (ms * 1e-3), gflop=flops / 1e9, gflop_dense=dflops / 1e9,
               tflops=flops / (ms * 1e-3) / 1e12, tflops_dense=dflops / (ms * 1e-3) / 1e12,
               bytes=byts, achieved_gbs=byts / (ms * 1e-3) / 1e9,
               workspace_bytes=int(ws.numel()), wall_s=wall)
    res["frac_hbm"] = res["achieved_gbs"] / PEAK_HBM_GBS
    res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
    res["frac_mfma_dense"] = res["tflops_dense"] / PEAK_BF16_TFLOPS
    res["roofline_bound"] = "hbm (at the knee)"
    del inp, ws
    return res


GLA_FWD_KERNELS = ("gla_fused_kernel<pass1>", "gla_seg_combine_kernel", "gla_fused_kernel<pass2>")
GLA_BWD_KERNELS = ("gla_bwd_prep_kernel", "gla_bwd_scans_kernel", "gla_bwd_grad_kernel")


GDN_BWD_KERNELS = ("gdn_chunk_prep_kernel<bwd>", "gdn_bwd_scans_kernel", "gdn_bwd_grad1_kernel",
                   "gdn_bwd_grad2_kernel")


def counter_traffic(kernel):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/counters.json),
    or None if the kernel's sources changed since they were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    for path, want in rec["sources"].items():
        with open(os.path.join(ROOT, path), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != want:
                return None
    return rec["traffic_bytes"]


# ------------------------------------------------------------------- ceilings

def measure_ceilings(reps=20):
    """Ceilings measured on this GPU, reported beside the published peaks. HBM: the
    library's streaming kernel (gdnrt_hbm_stream: 16-byte non-temporal loads and
    stores, one read and one write of every byte) over 2 GiB of fp32, in place (as the
    decode updates its state) and as a copy, 1, 2 and 4 pieces per thread; the best
    rate is the ceiling. MFMA: an 8192^3 bf16 matrix product through torch's BLAS.
    Neither is part of the hot path."""
    n = 1 << 29
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sweep = {}
    for vec in (1, 2, 4):
        for name, d in (("inplace", src), ("copy", dst)):
            ms, _ = timed(lambda i: m.hbm_stream(d, src, vec), reps, 3)
            sweep[f"{name}_vec{vec}"] = 2 * n * 4 / (ms * 1e-3) / 1e9
    ms, _ = timed(lambda i: dst.copy_(src), reps, 3)
    torch_copy_gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    M = 8192
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn((M, M), generator=g, device="cuda").to(torch.bfloat16).contiguous()
    b = torch.randn((M, M), generator=g, device="cuda").to(torch.bfloat16).contiguous()
    ms, _ = timed(lambda i: torch.matmul(a, b), reps, 3)
    gemm_tflops = 2 * M ** 3 / (ms * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    best = max(sweep, key=sweep.get)
    return {"hbm_stream_gbs": sweep[best], "hbm_stream_best": best, "hbm_stream_sweep": sweep,
            "torch_copy_gbs": torch_copy_gbs, "bf16_gemm_tflops": gemm_tflops,
            "how": "gdnrt_hbm_stream over 2 GiB fp32 (bytes read + written; best of in-place / copy x "
                   "1, 2, 4 pieces per thread); torch copy_ of the same for reference; torch.matmul "
                   "8192^3 bf16 (hipBLASLt), not a dense-MFMA ceiling but what a library GEMM reaches",
            "published_hbm_gbs": PEAK_HBM_GBS, "published_bf16_tflops": PEAK_BF16_TFLOPS}


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rows", default="decode,bf16_state,int8_state,kda,leapq,leapq6,leapq4,kda_leapq,gla,zeco,gla_bwd,gdn,gdn_bwd,"
                                      "kda_chunk")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured HBM-copy and bf16-GEMM ceilings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    m.lib()
    rows = [r.strip() for r in args.rows.split(",") if r.strip()]
    out_rows = {}
    res, cpu, decode_inp = None, None, None
    if "decode" in rows:
        res, inp = bench_decode(args.steps, args.warmup)
        log(f"[decode] {res['ms_per_step']*1e3:.1f} us/step  {res['achieved_gbs']:.0f} GB/s  "
            f"{res['tokens_per_s']/1e6:.3f} M tok/s")
        out_rows["decode"] = res
        if args.copy_probe:
            # a plain copy of known size: 1 GiB read + 1 GiB written per launch
            src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        # the oracle runs on the CPU after the GPU rows (the GPU would idle meanwhile)
        decode_inp = None if args.no_cpu_baseline else inp
        del inp
        torch.cuda.empty_cache()
    for bits, key in ((16, "bf16_state"), (8, "int8_state")):
        if key in rows:
            r = bench_decode_lowp(args.steps, args.warmup, bits)
            r["speedup_vs_fp32_decode"] = res["ms_per_step"] / r["ms_per_step"] if res else None
            out_rows[key] = r
            log(f"[{key}] {r['ms_per_step']*1e3:.1f} us/step  {r['achieved_gbs']:.0f} GB/s  "
                f"{r['tokens_per_s']/1e6:.3f} M tok/s")
            torch.cuda.empty_cache()
    if "kda" in rows:
        r = bench_kda(args.steps, args.warmup)
        r["traffic_bytes"] = counter_traffic("gdn_decode_kernel<kda>")
        out_rows["kda"] = r
        log(f"[kda] {r['ms_per_step']*1e3:.1f} us/step  {r['achieved_gbs']:.0f} GB/s  "
            f"{r['tokens_per_s']/1e6:.3f} M tok/s")
        torch.cuda.empty_cache()
    if "gla" in rows:
        r = bench_gla()
        parts = [counter_traffic(k) for k in GLA_FWD_KERNELS]
        r["traffic_bytes"] = sum(parts) if None not in parts else None
        out_rows["gla"] = r
        log(f"[gla] {r['ms']*1e3:.1f} us  {r['tflops']:.1f} TFLOP/s ({r['frac_mfma']*100:.1f}% MFMA)  "
            f"{r['achieved_gbs']:.0f} GB/s ({r['frac_hbm']*100:.1f}% HBM)  {r['tokens_per_s']/1e6:.2f} M tok/s")
        torch.cuda.empty_cache()
    if "gdn" in rows:
        r = bench_gdn_chunk()
        tp, ts = counter_traffic("gdn_chunk_prep_kernel"), counter_traffic("gdn_chunk_seq_kernel")
        r["traffic_bytes"] = tp + ts if tp is not None and ts is not None else None
        out_rows["gdn_chunk"] = r
        log(f"[gdn_chunk] {r['ms']*1e3:.1f} us  {r['tflops']:.1f} TFLOP/s ({r['frac_mfma']*100:.1f}% MFMA)  "
            f"{r['achieved_gbs']:.0f} GB/s ({r['frac_hbm']*100:.1f}% HBM)  {r['tokens_per_s']/1e6:.2f} M tok/s")
        torch.cuda.empty_cache()
    if "zeco" in rows:
        r = bench_zeco()
        r["traffic_bytes_correct_kernel"] = counter_traffic("gla_shard_correct_kernel")
        out_rows["zeco"] = r
        log(f"[zeco] local fwd {r['local_fwd_ms']*1e3:.1f} us; decay {r['decay_ms']*1e3:.1f} us, "
            f"All-Scan step {r['all_scan_step_ms']*1e3:.1f} us, correction {r['correct_ms']*1e3:.1f} us "
            f"({r['correct_gbs']:.0f} GB/s, {r['correct_frac_hbm']*100:.1f}% HBM); "
            f"backward phase 1 {r['bwd_local_state_ms']*1e3:.1f} us, gradient pass after it "
            f"{r['bwd_grads_reusing_prep_ms']*1e3:.1f} us")
        torch.cuda.empty_cache()
    if "gla_bwd" in rows:
        r = bench_gla_bwd()
        parts = [counter_traffic(k) for k in GLA_BWD_KERNELS]
        r["traffic_bytes"] = sum(parts) if None not in parts else None
        out_rows["gla_bwd"] = r
        log(f"[gla_bwd] {r['ms']*1e3:.1f} us  {r['tflops']:.1f} TFLOP/s ({r['frac_mfma']*100:.1f}% MFMA)  "
            f"{r['achieved_gbs']:.0f} GB/s ({r['frac_hbm']*100:.1f}% HBM)  {r['tokens_per_s']/1e6:.2f} M tok/s")
        torch.cuda.empty_cache()
    if "gdn_bwd" in rows:
        r = bench_gdn_bwd()
        parts = [counter_traffic(k) for k in GDN_BWD_KERNELS]
        r["traffic_bytes"] = sum(parts) if None not in parts else None
        out_rows["gdn_bwd"] = r
        log(f"[gdn_bwd] {r['ms']*1e3:.1f} us  {r['tflops']:.1f} TFLOP/s ({r['frac_mfma']*100:.1f}% MFMA)  "
            f"{r['achieved_gbs']:.0f} GB/s ({r['frac_hbm']*100:.1f}% HBM)  {r['tokens_per_s']/1e6:.2f} M tok/s")
        torch.cuda.empty_cache()
    if "kda_chunk" in rows:
        r = bench_gdn_chunk(kda=True)
        tp, ts = counter_traffic("gdn_chunk_prep_kernel<kda>"), counter_traffic("gdn_chunk_seq_kernel<kda>")
        r["traffic_bytes"] = tp + ts if tp is not None and ts is not None else None
        out_rows["kda_chunk"] = r
        log(f"[kda_chunk] {r['ms']*1e3:.1f} us  {r['tflops']:.1f} TFLOP/s ({r['frac_mfma']*100:.1f}% MFMA)  "
            f"{r['achieved_gbs']:.0f} GB/s ({r['frac_hbm']*100:.1f}% HBM)  {r['tokens_per_s']/1e6:.2f} M tok/s")
        torch.cuda.empty_cache()
    if "leapq" in rows:
        r = bench_leapq()
        r["traffic_bytes_decode_kernel"] = counter_traffic("leapq_decode_kernel")
        r["traffic_bytes_flush_kernel"] = counter_traffic("leapq_flush_kernel")
        r["traffic_bytes_decode_flush_kernel"] = counter_traffic("leapq_decode_flush_kernel")
        r["speedup_vs_fp32_decode"] = res["ms_per_step"] / r["ms_per_step"] if res else None
        out_rows["leapq"] = r
        log(f"[leapq] {r['ms_per_step']*1e3:.1f} us/step ({r['decode_kernel_ms']*1e3:.1f} us decode, "
            f"{r['decode_flush_kernel_ms']*1e3:.1f} us last token + flush per window; two launches "
            f"{r['two_launch_ms_per_step']*1e3:.1f} us/step)  {r['achieved_gbs']:.0f} GB/s  "
            f"{r['tokens_per_s']/1e6:.3f} M tok/s")
        torch.cuda.empty_cache()
    for bits in (6, 4):
        if f"leapq{bits}" not in rows:
            continue
        r = bench_leapq(bits=bits, rank=6)
        r["traffic_bytes_decode_kernel"] = counter_traffic(f"leapq_decode_kernel<{bits}bit>")
        r["speedup_vs_int8"] = out_rows["leapq"]["ms_per_step"] / r["ms_per_step"] if "leapq" in out_rows else None
        out_rows[f"leapq{bits}"] = r
        log(f"[leapq{bits}] {r['ms_per_step']*1e3:.1f} us/step ({r['decode_kernel_ms']*1e3:.1f} us decode, "
            f"{r['decode_flush_kernel_ms']*1e3:.1f} us last token + flush per window)  "
            f"{r['achieved_gbs']:.0f} GB/s  {r['tokens_per_s']/1e6:.3f} M tok/s")
        torch.cuda.empty_cache()
    if "kda_leapq" in rows:
        r = bench_leapq(tokens=256, kda=True)
        r["traffic_bytes_decode_kernel"] = counter_traffic("leapq_decode_kernel<kda>")
        r["traffic_bytes_flush_kernel"] = counter_traffic("leapq_flush_kernel<kda>")
        r["traffic_bytes_decode_flush_kernel"] = counter_traffic("leapq_decode_flush_kernel<kda>")
        kda_row = out_rows.get("kda")
        r["speedup_vs_fp32_kda_decode"] = kda_row["ms_per_step"] / r["ms_per_step"] if kda_row else None
        out_rows["kda_leapq"] = r
        log(f"[kda_leapq] {r['ms_per_step']*1e3:.1f} us/step ({r['decode_kernel_ms']*1e3:.1f} us decode, "
            f"{r['decode_flush_kernel_ms']*1e3:.1f} us last token + flush per window; two launches "
            f"{r['two_launch_ms_per_step']*1e3:.1f} us/step)  {r['achieved_gbs']:.0f} GB/s  "
            f"{r['tokens_per_s']/1e6:.3f} M tok/s")
        torch.cuda.empty_cache()
    ceil = None
    if decode_inp is not None:
        log("[cpu] timing the oracle on a sample")
        cpu = cpu_baseline_decode(decode_inp)
        del decode_inp
        torch.cuda.empty_cache()
    if not args.no_ceilings:
        ceil = measure_ceilings()
        log(f"[ceilings] HBM stream {ceil['hbm_stream_gbs']:.0f} GB/s ({ceil['hbm_stream_best']}), "
            f"torch copy {ceil['torch_copy_gbs']:.0f} GB/s, bf16 GEMM {ceil['bf16_gemm_tflops']:.0f} TFLOP/s")
        for r in out_rows.values():
            if "achieved_gbs" in r:
                r["frac_hbm_of_measured_stream"] = r["achieved_gbs"] / ceil["hbm_stream_gbs"]
            if "tflops" in r:
                r["frac_of_library_gemm"] = r["tflops"] / ceil["bf16_gemm_tflops"]
    line = {
        "metric": "GDN decode tokens/s at B=512 (one layer, 32 heads, d=128)",
        "value": res["tokens_per_s"] if res else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"] if res else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": DECODE_WORKLOAD, "streams": DECODE_B, "heads": DECODE_H,
                   "d_k": D, "d_v": D},
        "roofline": ({"bound": "hbm", "achieved": res["achieved_gbs"], "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": res["frac_hbm"],
                      "traffic": counter_traffic("gdn_decode_kernel")} if res else None),
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "rows": out_rows,
        "host": {"cpus": os.cpu_count(), "machine": platform.processor() or platform.machine(),
                 "torch": torch.__version__, "hip": torch.version.hip},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

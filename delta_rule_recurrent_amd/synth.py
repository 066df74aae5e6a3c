"""Seeded synthetic inputs for the gated delta-rule workloads.

This module only draws random tensors with the shapes and distributions of the
workloads; it contains none of the recurrence, chunking or quantisation
arithmetic. Both the HIP path (through its tests and the benchmark) and the CPU
reference draw their inputs from here, on the same seeds.

Conventions shared by every generator
-------------------------------------
* ``N(mu, sigma)``: sigma is the standard deviation.
* Draw order is fixed: q, k, v, then the gate (alpha or log-gate), then beta,
  then the initial state, then anything extra (outlier channels).
* q and k are L2-normalised in fp32 over the key dimension where the workload
  says so, then cast to bf16 with round-to-nearest-even; the stored bf16 bits are
  the inputs (k is then only approximately unit norm).
* Per-token tensors of a sequence workload are ``[N][T][d]`` (N = batch x heads,
  head-major inside a batch entry). Decode workloads are ``[steps][N][d]`` so
  that one step's slice is contiguous.
* States are ``[N][d_v][d_k]`` fp32: rows are value channels, columns key
  channels.

Generation runs on ``device`` with a ``torch.Generator`` seeded per workload, so
a workload is reproducible on one device type (CPU and GPU streams differ).
"""
from __future__ import annotations

import torch

D = 128


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, mean=0.0, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x


def _l2n(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def gdn_small(T=64, d=D, device="cpu", seed=1000):
    """One Gated DeltaNet head, fp32 throughout, zero initial state."""
    g = _gen(device, seed)
    q = _l2n(_randn((1, T, d), g, device))
    k = _l2n(_randn((1, T, d), g, device))
    v = _randn((1, T, d), g, device)
    alpha = torch.sigmoid(_randn((1, T), g, device, 4.0, 1.0))
    beta = torch.sigmoid(_randn((1, T), g, device, 0.0, 1.0))
    S0 = torch.zeros((1, d, d), device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


def gla_prefill(B=4, H=16, T=4096, d=D, device="cpu", seed=1001):
    """Gated linear attention prefill shard: bf16 q/k/v, fp32 per-key-dim
    log-gates logsigmoid(N(3,1)), nonzero fp32 incoming state N(0, 0.1)."""
    g = _gen(device, seed)
    N = B * H
    q = _randn((N, T, d), g, device).to(torch.bfloat16)
    k = _randn((N, T, d), g, device).to(torch.bfloat16)
    v = _randn((N, T, d), g, device).to(torch.bfloat16)
    log_g = torch.nn.functional.logsigmoid(_randn((N, T, d), g, device, 3.0, 1.0))
    S0 = _randn((N, d, d), g, device, 0.0, 0.1)
    return dict(q=q, k=k, v=v, log_g=log_g, S0=S0)


def gdn_prefill(B=1, H=32, T=16384, d=D, device="cpu", seed=1002, S0_std=0.0):
    """Gated DeltaNet prefill: bf16 q/k/v (q, k L2-normalised), alpha =
    sigmoid(N(4,1)), beta = sigmoid(N(0,1)), zero initial state unless
    ``S0_std`` > 0 (used by tests of the incoming-state path)."""
    g = _gen(device, seed)
    N = B * H
    q = _l2n(_randn((N, T, d), g, device)).to(torch.bfloat16)
    k = _l2n(_randn((N, T, d), g, device)).to(torch.bfloat16)
    v = _randn((N, T, d), g, device).to(torch.bfloat16)
    alpha = torch.sigmoid(_randn((N, T), g, device, 4.0, 1.0))
    beta = torch.sigmoid(_randn((N, T), g, device, 0.0, 1.0))
    if S0_std > 0:
        S0 = _randn((N, d, d), g, device, 0.0, S0_std)
    else:
        S0 = torch.zeros((N, d, d), device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


CHUNK_STEPS = 256


def kda_prefill(B=1, H=32, T=16384, d=D, device="cpu", seed=1008, S0_std=0.0):
    """Kimi Delta Attention chunkwise prefill: the GDN prefill workload's shape and
    draws, with one decay per key channel and token, alpha = sigmoid(N(4,1))
    ([N][T][d_k] fp32, drawn 1024 tokens at a time)."""
    g = _gen(device, seed)
    N = B * H
    q = torch.empty((N, T, d), dtype=torch.bfloat16, device=device)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    for x, norm in ((q, True), (k, True), (v, False)):
        for t0 in range(0, T, 1024):
            t1 = min(T, t0 + 1024)
            c = _randn((N, t1 - t0, d), g, device)
            x[:, t0:t1] = (_l2n(c) if norm else c).to(torch.bfloat16)
    alpha = torch.empty((N, T, d), dtype=torch.float32, device=device)
    for t0 in range(0, T, 1024):
        t1 = min(T, t0 + 1024)
        alpha[:, t0:t1] = torch.sigmoid(_randn((N, t1 - t0, d), g, device, 4.0, 1.0))
    beta = torch.sigmoid(_randn((N, T), g, device, 0.0, 1.0))
    S0 = (_randn((N, d, d), g, device, 0.0, S0_std) if S0_std > 0
          else torch.zeros((N, d, d), device=device, dtype=torch.float32))
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


def _decode_tokens(steps, N, d, g, device, io):
    """q, k (L2-normalised) and v for ``steps`` decode steps, drawn in chunks of
    256 steps (q chunks, then k chunks, then v chunks) so that long runs need no
    full-size fp32 temporaries."""
    out = []
    for norm in (True, True, False):
        x = torch.empty((steps, N, d), dtype=io, device=device)
        for s0 in range(0, steps, CHUNK_STEPS):
            s1 = min(steps, s0 + CHUNK_STEPS)
            c = _randn((s1 - s0, N, d), g, device)
            x[s0:s1] = (_l2n(c) if norm else c).to(io)
        out.append(x)
    return out


def _decode_gates(steps, B, H, g, device):
    """Heads h < H/2 are slow heads with alpha = 0.999 on every token; the
    rest draw alpha = sigmoid(N(2,1)) per (stream, token)."""
    N = B * H
    a = torch.sigmoid(_randn((steps, N), g, device, 2.0, 1.0))
    slow = (torch.arange(N, device=device) % H) < (H // 2)
    a[:, slow] = 0.999
    return a


def gdn_decode(B=512, H=32, steps=256, d=D, device="cpu", seed=1003, io=torch.bfloat16):
    """Gated DeltaNet decode of one layer: B streams x H heads, fp32 state
    N(0, 0.05) resident on the device, one token per stream per step."""
    g = _gen(device, seed)
    N = B * H
    q, k, v = _decode_tokens(steps, N, d, g, device, io)
    alpha = _decode_gates(steps, B, H, g, device)
    beta = torch.sigmoid(_randn((steps, N), g, device, 0.0, 1.0))
    S0 = _randn((N, d, d), g, device, 0.0, 0.05)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


def _decode_gates_vec(steps, B, H, d, g, device):
    """Per-key-channel decays: heads h < H/2 are slow heads with alpha = 0.999 on
    every channel and token; the rest draw alpha = sigmoid(N(2,1)) per (stream,
    token, key channel), in chunks of 256 steps."""
    N = B * H
    a = torch.empty((steps, N, d), device=device, dtype=torch.float32)
    for s0 in range(0, steps, CHUNK_STEPS):
        s1 = min(steps, s0 + CHUNK_STEPS)
        a[s0:s1] = torch.sigmoid(_randn((s1 - s0, N, d), g, device, 2.0, 1.0))
    slow = (torch.arange(N, device=device) % H) < (H // 2)
    a[:, slow] = 0.999
    return a


def kda_decode(B=512, H=32, steps=256, d=D, device="cpu", seed=1005, io=torch.bfloat16):
    """Kimi Delta Attention decode of one layer: the GDN decode workload's shape and
    draws, with one decay per key channel (``alpha`` is ``[steps][N][d_k]``)."""
    g = _gen(device, seed)
    N = B * H
    q, k, v = _decode_tokens(steps, N, d, g, device, io)
    alpha = _decode_gates_vec(steps, B, H, d, g, device)
    beta = torch.sigmoid(_randn((steps, N), g, device, 0.0, 1.0))
    S0 = _randn((N, d, d), g, device, 0.0, 0.05)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


def kda_small(T=64, d=D, device="cpu", seed=1006):
    """One KDA head, fp32 throughout: q, k L2-normalised, alpha = sigmoid(N(4,1))
    per key channel and token, beta = sigmoid(N(0,1)), zero initial state."""
    g = _gen(device, seed)
    q = _l2n(_randn((1, T, d), g, device))
    k = _l2n(_randn((1, T, d), g, device))
    v = _randn((1, T, d), g, device)
    alpha = torch.sigmoid(_randn((1, T, d), g, device, 4.0, 1.0))
    beta = torch.sigmoid(_randn((1, T), g, device, 0.0, 1.0))
    S0 = torch.zeros((1, d, d), device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


def leapq_decode(B=512, H=32, steps=4096, d=D, device="cpu", seed=1004,
                 outlier_scale=50.0, n_outliers=2):
    """LeapQuant windowed 8-bit decode: the decode workload above plus two
    outlier key channels per head in the initial state, scaled by 50 so their
    median magnitude is 50x the state's. Also returns the fixed start block
    ``Q0`` ([d_k][4], N(0,1), its own seed) of the compensator fit."""
    g = _gen(device, seed)
    N = B * H
    q, k, v = _decode_tokens(steps, N, d, g, device, torch.bfloat16)
    alpha = _decode_gates(steps, B, H, g, device)
    beta = torch.sigmoid(_randn((steps, N), g, device, 0.0, 1.0))
    S0 = _randn((N, d, d), g, device, 0.0, 0.05)
    # two distinct outlier key channels per head
    cols = torch.argsort(torch.rand((N, d), generator=g, device=device), dim=1)[:, :n_outliers]
    scale = torch.ones((N, d), device=device)
    scale.scatter_(1, cols, outlier_scale)
    S0.mul_(scale[:, None, :])
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0, outlier_cols=cols,
                Q0=compensator_start(d))


def kda_leapq_decode(B=512, H=32, steps=256, d=D, device="cpu", seed=1007,
                     outlier_scale=50.0, n_outliers=2):
    """KDA in the windowed 8-bit state: the KDA decode workload (one decay per key
    channel, slow heads at 0.999) with the LeapQuant initial state's two outlier key
    channels per head at 50x, and the compensator start block ``Q0``."""
    g = _gen(device, seed)
    N = B * H
    q, k, v = _decode_tokens(steps, N, d, g, device, torch.bfloat16)
    alpha = _decode_gates_vec(steps, B, H, d, g, device)
    beta = torch.sigmoid(_randn((steps, N), g, device, 0.0, 1.0))
    S0 = _randn((N, d, d), g, device, 0.0, 0.05)
    cols = torch.argsort(torch.rand((N, d), generator=g, device=device), dim=1)[:, :n_outliers]
    scale = torch.ones((N, d), device=device)
    scale.scatter_(1, cols, outlier_scale)
    S0.mul_(scale[:, None, :])
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0, outlier_cols=cols,
                Q0=compensator_start(d))


def compensator_start(d=D, r=4, seed=0):
    """Fixed random start block of the compensator-token subspace iteration:
    ``[d_k][r]`` fp32 entries N(0,1) from seed 0 (always drawn on the CPU)."""
    g = _gen("cpu", seed)
    return torch.randn((d, r), generator=g, dtype=torch.float32)

"""State error of the low-precision schemes against the exact fp32 recurrence, on the
GPU, over the LeapQuant decode workload (the analog of the state-error-vs-time figure
of "LeapQuant: an 8-bit recurrent state that stops rounding every token", section "Fix
one: leap over a window", on synthetic inputs).

Schemes (every one on the same seeded inputs, one decode token per step):
  per-step BF16 / INT8 / INT4  the state re-rounded after every token (eq. 2);
  window W=16 at b bits        the LeapQuant state (eq. 4 / eq. 10), flushed every 16
                               tokens, with or without compensator tokens (rank 4 at
                               8 bits, 6 at 6 and 4 bits) and smoothing (eq. 7).
The reference is gdn_decode_step with its fp32 state. Every ``--every`` tokens the
dense state of each scheme (dequantised codes, compensators, right after a flush) is
compared with it: relative Frobenius error over all heads, over the key channels
other than the two outlier channels of each head (which otherwise dominate the norm),
and over the slow heads alone.

Regimes: ``workload`` is the decode workload as drawn (half the heads at alpha = 0.999,
the rest sigmoid(N(2,1)); beta = sigmoid(N(0,1))); ``long`` sets alpha = 0.999 on every
head and scales beta by 1/10, so each write is small next to the state -- the long-
memory case in which the page's per-step rounding discards part of every update.

    python -m delta_rule_recurrent_amd.error_study [--streams 16] [--steps 4096] [--regime long]
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import torch

from . import binding as m
from . import synth

D = 128


def _per_step_state(S0, bits):
    Q = (1 << (bits - 1)) - 1
    mx = S0.abs().amax(dim=-1)
    Z = torch.clamp(torch.round(S0 * (Q / torch.where(mx > 0, mx, 1.0))[..., None]), -Q, Q).to(torch.int8)
    return Z, mx, Q


def _windowed_dense(st, Q):
    S = st.vscale[:, :, None] * (st.code_values().float() / Q) * st.ksmooth[:, None, :]
    if st.rank > 0:
        S = S + st.ct_u.float().transpose(1, 2) @ st.ct_k.float()
    return S


def run(streams=16, heads=32, steps=4096, every=256, regime="workload", device="cuda", log=print):
    inp = synth.leapq_decode(B=streams, H=heads, steps=steps, device=device)
    N = streams * heads
    slow = torch.arange(N, device=device) % heads < heads // 2
    q, k, v, a, b, S0 = (inp[n] for n in ("q", "k", "v", "alpha", "beta", "S0"))
    if regime == "long":
        a.fill_(0.999)
        b.mul_(0.1)
        slow[:] = True
    elif regime != "workload":
        raise ValueError(f"regime {regime!r}")
    ordinary = torch.ones((N, D), dtype=torch.bool, device=device)
    ordinary.scatter_(1, inp["outlier_cols"], False)
    ordinary = ordinary[:, None, :].expand(N, D, D)
    Q0 = {r: synth.compensator_start(r=r).to(device) for r in (4, 6)}

    def block(x, t0, t1):   # [T][N][..] -> [N][t1 - t0][..] contiguous
        return x[t0:t1].transpose(0, 1).contiguous()

    schemes = {}
    exact = S0.clone()
    bf = S0.to(torch.bfloat16)
    ints = {bits: _per_step_state(S0, bits) for bits in (8, 4)}
    ints = {bits: (Z.clone(), mx.clone(), Q) for bits, (Z, mx, Q) in ints.items()}
    wins = {}
    for name, bits, rank, mode in (("window int8", 8, 0, 2), ("window int8 + 4 CT + smooth", 8, 4, 0),
                                   ("window int6 + 6 CT + smooth", 6, 6, 0), ("window int4", 4, 0, 2),
                                   ("window int4 + 6 CT + smooth", 4, 6, 0)):
        st = m.LeapqBuffers(N, rank=rank, window=16, device=device, bits=bits)
        q0 = Q0[rank] if rank else torch.zeros((D, 0), device=device)
        m.leapq_window_flush(st, q0, dense=S0, smooth_mode=mode)
        wins[name] = (st, q0, mode, (1 << (bits - 1)) - 1)
    names = (["per-step bf16", "per-step int8", "per-step int4"] + list(wins))
    for n_ in names:
        schemes[n_] = {"all": [], "ordinary": [], "slow": []}
    marks = []

    def rel(d, ref, mask=None):
        if mask is not None:
            d, ref = d[mask], ref[mask]
        return math.sqrt(float((d * d).sum()) / float((ref * ref).sum()))

    def record(t, dense):
        ex = exact.double()
        for n_, S in dense.items():
            d = (S - exact).double()
            schemes[n_]["all"].append(rel(d, ex))
            schemes[n_]["ordinary"].append(rel(d, ex, ordinary))
            schemes[n_]["slow"].append(rel(d[slow], ex[slow], ordinary[slow]))
        marks.append(t)

    for t0 in range(0, steps, every):
        t1 = min(steps, t0 + every)
        args = [block(x, t0, t1) for x in (q, k, v, a, b)]
        m.gdn_decode_step(exact, *args)
        m.gdn_decode_step_bf16_state(bf, *args)
        for bits, (Z, mx, Q) in ints.items():
            m.gdn_decode_step_int_state(Z, mx, bits, *args)
        for t in range(t0, t1):
            for st, q0, mode, _ in wins.values():
                m.leapq_decode_step(st, q[t], k[t], v[t], a[t], b[t])
                if st.pos == st.window:
                    m.leapq_window_flush(st, q0, smooth_mode=mode)
        dense = {"per-step bf16": bf.float()}
        for bits, (Z, mx, Q) in ints.items():
            dense[f"per-step int{bits}"] = mx[:, :, None] * (Z.float() / Q)
        for n_, (st, _, _, Q) in wins.items():
            assert st.pos == 0
            dense[n_] = _windowed_dense(st, Q)
        record(t1, dense)
        log(f"[error_study] t={t1}: " + ", ".join(f"{n_} {schemes[n_]['all'][-1]:.2e}" for n_ in names))
    return {"workload": f"leapq_decode B={streams} H={heads} (half the heads at alpha 0.999), {steps} tokens, "
                        f"bf16 q/k/v, S0 ~ N(0, 0.05) with two key channels x50",
            "regime": regime, "tokens": marks, "schemes": schemes}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--streams", type=int, default=16)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--every", type=int, default=256)
    ap.add_argument("--regime", default="workload", choices=("workload", "long"))
    ap.add_argument("--out", default=None, help="write the JSON result here")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("error_study needs a GPU", file=sys.stderr)
        return 1
    res = run(args.streams, 32, args.steps, args.every, args.regime,
              log=lambda s: print(s, file=sys.stderr, flush=True))
    if args.out:
        with open(args.out, "w") as f:
            json.dump(res, f, indent=1)
    cols = [i for i, t in enumerate(res["tokens"]) if t in (256, 1024, 4096) or i == len(res["tokens"]) - 1]
    last = res["tokens"][-1]
    print(f"regime: {res['regime']}")
    print("| scheme | " + " | ".join(f"all, t={res['tokens'][i]}" for i in cols) +
          f" | ordinary channels, t={last} | slow heads, ordinary, t={last} |")
    print("|---" * (len(cols) + 3) + "|")
    for n_, e in res["schemes"].items():
        print(f"| {n_} | " + " | ".join(f"{100 * e['all'][i]:.2f}%" for i in cols) +
              f" | {100 * e['ordinary'][-1]:.2f}% | {100 * e['slow'][-1]:.2f}% |")
    return 0


if __name__ == "__main__":
    sys.exit(main())

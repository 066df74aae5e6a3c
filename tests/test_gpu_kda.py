"""GPU parity of kda_decode_step (one decay per key channel) against the fp64 KDA
oracle recurrence."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import kda
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4    # fp32-state paths: max-abs error / max|ref|
TOL_BF16 = 2e-2   # bf16 outputs


def _to_nt(x):       # [steps][N][...] -> [N][steps][...]
    return x.transpose(0, 1).contiguous()


def test_single_head_fp32_T64():
    dev = need_gpu()
    inp = synth.kda_small(device="cpu")
    say("kda_decode_step: single head T=64 fp32")
    S = inp["S0"].to(dev).clone()
    o = m.kda_decode_step(S, *(inp[n].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
    torch.cuda.synchronize()
    o_ref, S_ref = kda.kda_recurrent(*(np64(inp[n]) for n in ("q", "k", "v", "alpha", "beta")),
                                     np64(inp["S0"]))
    e1 = assert_rel(np64(o), o_ref, TOL_F32, "o")
    e2 = assert_rel(np64(S), S_ref, TOL_F32, "S_T")
    say(f"  o err {e1:.2e}  S err {e2:.2e}")


@pytest.mark.parametrize("N,T,dt", [(37, 5, torch.bfloat16), (300, 3, torch.float32),
                                    (2049, 2, torch.bfloat16), (1, 1, torch.float32)])
def test_ragged_head_counts_and_dtypes(N, T, dt):
    dev = need_gpu()
    say(f"kda_decode_step: N={N} T={T} {dt}")
    inp = synth.kda_decode(B=N, H=1, steps=T, device="cpu", io=dt, seed=91 + N)
    q, k, v, a = (_to_nt(inp[n]) for n in ("q", "k", "v", "alpha"))
    b = inp["beta"].t().contiguous()
    S = inp["S0"].to(dev).clone()
    o = m.kda_decode_step(S, q.to(dev), k.to(dev), v.to(dev), a.to(dev), b.to(dev))
    torch.cuda.synchronize()
    o_ref, S_ref = kda.kda_recurrent(np64(q), np64(k), np64(v), np64(a), np64(b), np64(inp["S0"]))
    tol_o = TOL_F32 if dt == torch.float32 else TOL_BF16
    assert_rel(np64(o), o_ref, tol_o, "o")
    assert_rel(np64(S), S_ref, TOL_F32, "S_T")


def test_equal_channel_decays_match_gdn_kernel():
    """With every channel's decay equal to alpha_t the KDA step is the GDN step. The
    two kernels group the row sums differently (decay inside or outside the dot
    product), so they agree to fp32 rounding, not bit for bit."""
    dev = need_gpu()
    inp = synth.gdn_decode(B=64, H=2, steps=4, device="cpu", io=torch.bfloat16, seed=5)
    q, k, v = (_to_nt(inp[n]).to(dev) for n in ("q", "k", "v"))
    a = inp["alpha"].t().contiguous().to(dev)
    b = inp["beta"].t().contiguous().to(dev)
    S1, S2 = inp["S0"].to(dev).clone(), inp["S0"].to(dev).clone()
    o1 = m.gdn_decode_step(S1, q, k, v, a, b)
    o2 = m.kda_decode_step(S2, q, k, v, a[:, :, None].expand(-1, -1, 128).contiguous(), b)
    torch.cuda.synchronize()
    assert_rel(np64(S2), np64(S1), 1e-5, "S_T")
    assert_rel(np64(o2), np64(o1), TOL_BF16, "o")


def test_full_size_512x32_256_steps_sampled_heads():
    """The KDA decode workload at its real size (512 streams x 32 heads, fp32 state,
    256 consecutive T=1 calls in the launch configuration the benchmark times);
    sampled heads (slow and fast) checked against the oracle."""
    dev = need_gpu()
    B, H, steps = 512, 32, 256
    say(f"kda_decode_step: full size B={B} H={H} steps={steps}")
    inp = synth.kda_decode(B=B, H=H, steps=steps, device=dev)
    S = inp["S0"].clone()
    N = B * H
    o_all = torch.empty((steps, N, 128), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        m.kda_decode_step(S, inp["q"][t, :, None], inp["k"][t, :, None], inp["v"][t, :, None],
                          inp["alpha"][t, :, None], inp["beta"][t, :, None], o_all[t, :, None])
    torch.cuda.synchronize()
    heads = torch.tensor([0, 1, 15, 16, 17, 31, 32 * 100 + 3, 32 * 255 + 20, N - 1])
    sel = lambda x: np64(x[:, heads].transpose(0, 1))
    o_ref, S_ref = kda.kda_recurrent(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["alpha"]),
                                     np64(inp["beta"][:, heads].t()), np64(inp["S0"][heads]))
    e1 = assert_rel(np64(S[heads]), S_ref, TOL_F32, "S_T")
    e2 = assert_rel(sel(o_all), o_ref, TOL_BF16, "o")
    d = np.abs(sel(o_all) - o_ref)
    assert np.all(d <= 2.0 ** -8 * np.abs(o_ref) + 1e-4 * np.abs(o_ref).max())
    say(f"  S err {e1:.2e}  o err {e2:.2e}")

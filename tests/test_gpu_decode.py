"""GPU parity of gdn_decode_step against the fp64 oracle recurrence."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import synth
from oracle import gdn
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4    # fp32-state paths: max-abs error / max|ref|
TOL_BF16 = 2e-2   # bf16 outputs


def _to_nt(x):       # [steps][N][...] -> [N][steps][...]
    return x.transpose(0, 1).contiguous()


def test_single_head_fp32_T64():
    dev = need_gpu()
    inp = synth.gdn_small(device="cpu")
    say("gdn_decode_step: single head T=64 fp32")
    S = inp["S0"].to(dev).clone()
    o = m.gdn_decode_step(S, *(inp[n].to(dev) for n in ("q", "k", "v", "alpha", "beta")))
    torch.cuda.synchronize()
    o_ref, S_ref = gdn.gdn_recurrent(*(np64(inp[n]) for n in ("q", "k", "v", "alpha", "beta")),
                                     np64(inp["S0"]))
    e1 = assert_rel(np64(o), o_ref, TOL_F32, "o")
    e2 = assert_rel(np64(S), S_ref, TOL_F32, "S_T")
    say(f"  o err {e1:.2e}  S err {e2:.2e}")


@pytest.mark.parametrize("N,T,dt", [(37, 5, torch.bfloat16), (300, 3, torch.float32),
                                    (2049, 2, torch.bfloat16), (1, 1, torch.float32)])
def test_ragged_head_counts_and_dtypes(N, T, dt):
    """Head counts that hit each rows-per-wave variant, not multiples of anything."""
    dev = need_gpu()
    say(f"gdn_decode_step: N={N} T={T} {dt}")
    inp = synth.gdn_decode(B=N, H=1, steps=T, device="cpu", io=dt, seed=77 + N)
    q, k, v = (_to_nt(inp[n]) for n in ("q", "k", "v"))
    a, b = (inp[n].t().contiguous() for n in ("alpha", "beta"))
    S = inp["S0"].to(dev).clone()
    o = m.gdn_decode_step(S, q.to(dev), k.to(dev), v.to(dev), a.to(dev), b.to(dev))
    torch.cuda.synchronize()
    o_ref, S_ref = gdn.gdn_recurrent(np64(q), np64(k), np64(v), np64(a), np64(b), np64(inp["S0"]))
    tol_o = TOL_F32 if dt == torch.float32 else TOL_BF16
    assert_rel(np64(o), o_ref, tol_o, "o")
    assert_rel(np64(S), S_ref, TOL_F32, "S_T")


def test_full_size_512x32_256_steps_sampled_heads():
    """The decode workload at its real size (512 streams x 32 heads, fp32 state,
    256 consecutive T=1 calls in the same launch configuration the benchmark
    times); sampled heads (slow and fast) checked against the oracle."""
    dev = need_gpu()
    B, H, steps = 512, 32, 256
    say(f"gdn_decode_step: full size B={B} H={H} steps={steps}")
    inp = synth.gdn_decode(B=B, H=H, steps=steps, device=dev)
    S = inp["S0"].clone()
    N = B * H
    o_all = torch.empty((steps, N, 128), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        m.gdn_decode_step(S, inp["q"][t, :, None], inp["k"][t, :, None], inp["v"][t, :, None],
                          inp["alpha"][t, :, None], inp["beta"][t, :, None], o_all[t, :, None])
    torch.cuda.synchronize()
    heads = torch.tensor([0, 1, 15, 16, 17, 31, 32 * 100 + 3, 32 * 255 + 20, N - 1])
    sel = lambda x: np64(x[:, heads].transpose(0, 1))
    o_ref, S_ref = gdn.gdn_recurrent(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]),
                                     np64(inp["alpha"][:, heads].t()), np64(inp["beta"][:, heads].t()),
                                     np64(inp["S0"][heads]))
    e1 = assert_rel(np64(S[heads]), S_ref, TOL_F32, "S_T")
    e2 = assert_rel(sel(o_all), o_ref, TOL_BF16, "o")
    # o is bf16: each entry within bf16 rounding of the reference plus fp32 noise
    d = np.abs(sel(o_all) - o_ref)
    assert np.all(d <= 2.0 ** -8 * np.abs(o_ref) + 1e-4 * np.abs(o_ref).max())
    say(f"  S err {e1:.2e}  o err {e2:.2e}")


def test_run_twice_bitwise_identical():
    dev = need_gpu()
    inp = synth.gdn_decode(B=64, H=32, steps=1, device=dev)
    outs = []
    for _ in range(2):
        S = inp["S0"].clone()
        o = m.gdn_decode_step(S, *(inp[n][0, :, None] for n in ("q", "k", "v", "alpha", "beta")))
        torch.cuda.synchronize()
        outs.append((S.cpu(), o.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_degenerate_cases():
    dev = need_gpu()
    # empty work launches nothing
    S = torch.zeros((0, 128, 128), device=dev)
    z = torch.zeros((0, 1, 128), device=dev)
    g = torch.zeros((0, 1), device=dev)
    m.gdn_decode_step(S, z, z, z, g, g)
    # alpha tiny: finite, state collapses onto the write
    inp = synth.gdn_decode(B=4, H=2, steps=1, device=dev, io=torch.float32)
    q, k, v = (inp[n][0, :, None].contiguous() for n in ("q", "k", "v"))
    a = torch.full((8, 1), 1e-30, device=dev)
    b = inp["beta"][0, :, None].contiguous()
    S = inp["S0"].clone()
    o = m.gdn_decode_step(S, q, k, v, a, b)
    torch.cuda.synchronize()
    assert torch.isfinite(S).all() and torch.isfinite(o).all()
    o_ref, S_ref = gdn.gdn_recurrent(np64(q), np64(k), np64(v), np64(a), np64(b), np64(inp["S0"]))
    assert_rel(np64(S), S_ref, TOL_F32, "S tiny alpha")
    # NaN in one head stays in that head
    S = inp["S0"].clone()
    v2 = v.clone()
    v2[3, 0, 5] = float("nan")
    o = m.gdn_decode_step(S, q, k, v2, inp["alpha"][0, :, None].contiguous(), b)
    torch.cuda.synchronize()
    assert torch.isnan(S[3]).any()
    mask = torch.ones(8, dtype=torch.bool)
    mask[3] = False
    assert torch.isfinite(S[mask]).all() and torch.isfinite(o[mask]).all()


def test_erase_and_replace_and_carry():
    """The page's special cases on the GPU: beta = 1 with a unit key stores v_t along
    k_t exactly (S_t k_t = v_t, whatever was there: "erase and replace"), whatever
    the decay; alpha = 1 with beta = 0 leaves the state unchanged and reads it out,
    o_t = S q_t. fp32 throughout, 1e-4 of max|ref|."""
    dev = need_gpu()
    say("gdn_decode_step: beta = 1 unit key; alpha = 1 beta = 0")
    inp = synth.gdn_decode(B=8, H=4, steps=3, device=dev, io=torch.float32)
    N = 32
    S0 = inp["S0"].clone()
    k = inp["k"][0].double()
    k = (k / k.norm(dim=-1, keepdim=True)).float()          # unit norm in fp32
    q, v, a = inp["q"][0], inp["v"][0], inp["alpha"][0]
    S = S0.clone()
    m.gdn_decode_step(S, q[:, None].contiguous(), k[:, None].contiguous(), v[:, None].contiguous(),
                      a[:, None].contiguous(), torch.ones((N, 1), device=dev))
    torch.cuda.synchronize()
    Sk = torch.einsum("nvk,nk->nv", S.double(), k.double())
    assert_rel(np64(Sk), np64(v), TOL_F32, "S_t k_t = v_t")
    # alpha = 1, beta = 0: state bitwise unchanged, o = S q
    S = S0.clone()
    o = m.gdn_decode_step(S, q[:, None].contiguous(), k[:, None].contiguous(), v[:, None].contiguous(),
                          torch.ones((N, 1), device=dev), torch.zeros((N, 1), device=dev))
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    assert_rel(np64(o[:, 0]), np64(torch.einsum("nvk,nk->nv", S0.double(), q.double())), TOL_F32, "o = S q")

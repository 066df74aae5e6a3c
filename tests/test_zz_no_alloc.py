"""gdn_chunk_fwd_noalloc, the allocation-free form of gdn_chunk_fwd (its operands in
the library's fixed per-GPU scratch), called through the C ABI: two calls in a row,
the second on a smaller input, each equal bit for bit to gdn_chunk_fwd with a caller
workspace on the same inputs (the same kernels), and the first also against the fp64
recurrence at the bf16 tolerance; sizes beyond the scratch are refused."""
import ctypes

import pytest
import torch

import delta_rule_recurrent_amd as m
from delta_rule_recurrent_amd import binding, synth
from oracle import gdn
from helpers import assert_rel, need_gpu, np64, say

pytestmark = pytest.mark.gpu


def _call(inp, S0):
    N, T = inp["alpha"].shape
    o = torch.empty((N, T, 128), dtype=torch.bfloat16, device=inp["q"].device)
    ST = torch.empty((N, 128, 128), dtype=torch.float32, device=inp["q"].device)
    m.gdn_chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0, ST, o)
    return o, ST


def test_noalloc_matches_workspace_entry_twice():
    dev = need_gpu()
    lib = binding.lib()
    assert lib.gdn_chunk_fwd_noalloc_max_bytes() == 128 << 20
    for i, (N, T, seed) in enumerate(((8, 1024, 1190), (2, 256, 1191))):
        say(f"gdn_chunk_fwd_noalloc call {i + 1}: N={N} T={T}")
        inp = synth.gdn_prefill(B=N, H=1, T=T, device=dev, seed=seed, S0_std=0.05)
        o, ST = _call(inp, inp["S0"])
        o_ws, ST_ws = m.gdn_chunk_fwd(*(inp[n] for n in ("q", "k", "v", "alpha", "beta", "S0")))
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ws.view(torch.int16)), f"call {i + 1}: o"
        assert torch.equal(ST, ST_ws), f"call {i + 1}: ST"
        if i == 0:
            h = [0, N - 1]
            o_ref, S_ref = gdn.gdn_recurrent(*(np64(inp[n][h]) for n in ("q", "k", "v", "alpha", "beta", "S0")))
            assert_rel(np64(o[h]), o_ref, 2e-2, "o vs oracle")
            assert_rel(np64(ST[h]), S_ref, 2e-2, "ST vs oracle")


def test_noalloc_refuses_beyond_the_scratch():
    need_gpu()
    lib = binding.lib()
    p = ctypes.c_void_p(1 << 30)
    # 32 heads x 16,384 tokens: 8,192 chunks, far beyond 128 MiB; refused before any launch
    rc = lib.gdn_chunk_fwd_noalloc(p, p, p, p, p, None, p, p, 32, 16384, 128, 128, 64, 1, None)
    assert rc == binding.ESHAPE
    assert "maximum" in lib.gdnrt_last_error().decode()
    assert lib.gdn_chunk_fwd_noalloc(p, p, p, p, p, None, p, p, 0, 64, 128, 128, 64, 1, None) == binding.OK

"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments with the documented status before touching
the GPU (no GPU is needed for these calls)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdnrt.h")
# GDNRT_ABI_LIB: another build of the library to check (the host-sanitized one)
LIB = os.environ.get("GDNRT_ABI_LIB") or os.path.join(ROOT, "delta_rule_recurrent_amd", "libgdnrt.so")

OK, EINVAL, ESHAPE, EALIGN, EDTYPE, ESTATE = range(6)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from delta_rule_recurrent_amd import build
        build.build()
    from delta_rule_recurrent_amd import binding
    if binding._LIB is None:
        binding.LIB_PATH = LIB
    return binding.lib()


def declared():
    text = open(HEADER).read()
    return re.findall(r"GDNRT_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(declared())
    for n in ("gdn_decode_step", "gla_chunk_fwd", "gdn_chunk_fwd", "leapq_decode_step",
              "leapq_window_flush", "gdnrt_last_error", "gdn_chunk_fwd_workspace_bytes",
              "gla_chunk_fwd_workspace_bytes", "kda_decode_step", "kda_leapq_decode_step",
              "kda_leapq_window_flush", "kda_chunk_fwd", "kda_chunk_fwd_workspace_bytes",
              "gla_chunk_bwd", "gla_chunk_bwd_workspace_bytes", "gdn_chunk_bwd",
              "gdn_chunk_bwd_workspace_bytes", "gdn_decode_step_bf16_state",
              "gdn_decode_step_int_state", "gla_shard_decay", "gla_all_scan_step",
              "gla_shard_output_correct", "gla_shard_bwd_state", "gla_shard_bwd_grads",
              "leapq_decode_flush", "kda_leapq_decode_flush"):
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in declared():
        assert n in exported, n
        assert getattr(lib, n) is not None


def _err(lib):
    return lib.gdnrt_last_error().decode()


def test_decode_validation(lib):
    f = lib.gdn_decode_step
    p = ctypes.c_void_p(4096)   # never dereferenced: every call below fails validation
    assert f(p, p, p, p, p, p, p, 4, 1, 64, 128, 1, None) == ESHAPE and "128" in _err(lib)
    assert f(p, p, p, p, p, p, p, -1, 1, 128, 128, 1, None) == ESHAPE
    assert f(p, p, p, p, p, p, p, 4, 1, 128, 128, 7, None) == EDTYPE
    assert f(None, p, p, p, p, p, p, 4, 1, 128, 128, 1, None) == EINVAL
    assert f(p, ctypes.c_void_p(4098), p, p, p, p, p, 4, 1, 128, 128, 1, None) == EALIGN
    assert f(p, p, p, p, p, p, p, 0, 1, 128, 128, 1, None) == OK          # empty: no launch
    big = ctypes.c_void_p(1 << 40)
    # o overlapping the state
    assert f(big, p, p, p, p, p, big, 4, 1, 128, 128, 1, None) == EINVAL


def test_kda_decode_validation(lib):
    f = lib.kda_decode_step
    p = ctypes.c_void_p(4096)
    assert f(p, p, p, p, p, p, p, 4, 1, 128, 64, 1, None) == ESHAPE and "kda_decode_step" in _err(lib)
    assert f(p, p, p, p, p, p, p, 4, 1, 128, 128, 3, None) == EDTYPE
    assert f(p, p, p, p, None, p, p, 4, 1, 128, 128, 1, None) == EINVAL
    # the per-channel decays are read 16 bytes at a time: 4-byte alignment is not enough
    assert f(p, p, p, p, ctypes.c_void_p(4100), p, p, 4, 1, 128, 128, 1, None) == EALIGN
    assert lib.gdn_decode_step(p, p, p, p, ctypes.c_void_p(4100), p, ctypes.c_void_p(1 << 40),
                               4, 1, 128, 128, 1, None) != EALIGN
    # alpha spans N*T*d_k floats: an o placed inside that span overlaps it
    assert f(p, ctypes.c_void_p(1 << 41), p, p, ctypes.c_void_p(1 << 40), p,
             ctypes.c_void_p((1 << 40) + 1024), 4, 1, 128, 128, 1, None) == EINVAL


def test_chunk_validation(lib):
    p = ctypes.c_void_p(4096)
    g = lib.gla_chunk_fwd
    assert g(p, p, p, p, None, p, p, 2, 100, 128, 128, 64, 1, p, 1 << 30, None) == ESHAPE  # T % 64
    assert g(p, p, p, p, None, p, p, 2, 128, 128, 128, 32, 1, p, 1 << 30, None) == ESHAPE  # chunk
    assert g(p, p, p, p, None, p, p, 2, 128, 128, 128, 64, 0, p, 1 << 30, None) == EDTYPE  # fp32 io
    assert g(p, p, p, p, None, p, p, 2, 128, 128, 128, 64, 0x100, p, 1 << 30, None) == EDTYPE  # shard, fp32
    assert g(p, p, p, p, None, p, p, 2, 128, 128, 128, 64, 0x201, p, 1 << 30, None) == EDTYPE  # unknown flag
    assert g(p, p, p, p, None, p, p, 2, 128, 128, 128, 64, 0x101, p, 10, None) == EINVAL    # shard, workspace
    assert g(p, p, p, p, None, p, p, 2, 128, 128, 128, 64, 1, p, 10, None) == EINVAL       # workspace
    # per chunk Q o e^b and e^{b_C} (16,896 B); 4 segments of 16 chunks per sequence: the
    # end states and decays of the 2 halves of each of the first 3, the start states of 4
    assert lib.gla_chunk_fwd_workspace_bytes(64, 4096, 128, 128, 64) == \
        64 * 64 * 16896 + 64 * 3 * 2 * (65536 + 512) + 64 * 4 * 65536
    assert lib.gla_chunk_fwd_workspace_bytes(64, 100, 128, 128, 64) == 0
    d = lib.gdn_chunk_fwd
    assert lib.gdn_chunk_fwd_workspace_bytes(32, 16384, 128, 128, 64) == 32 * 256 * 81984
    assert lib.gdn_chunk_fwd_workspace_bytes(32, 100, 128, 128, 64) == 0
    assert d(p, p, p, p, p, None, p, p, 2, 128, 128, 128, 64, 1, p, 10, None) == EINVAL  # workspace


def _state(lib, **kw):
    from delta_rule_recurrent_amd.binding import LeapqState
    a = dict(codes=4096, vscale=4096, ksmooth=4096, ct_k=4096, ct_u=4096, buf_k=4096,
             buf_u=4096, buf_a=4096, N=8, dk=128, dv=128, rank=4, window=16)
    a.update(kw)
    return LeapqState(**a)


def test_leapq_validation(lib):
    p = ctypes.c_void_p(4096)
    st = _state(lib)
    f = lib.leapq_decode_step
    assert f(ctypes.byref(st), 16, p, p, p, p, p, p, 1, None) == ESTATE     # window full
    assert f(ctypes.byref(st), -1, p, p, p, p, p, p, 1, None) == ESTATE
    assert f(ctypes.byref(_state(lib, rank=9)), 0, p, p, p, p, p, p, 1, None) == ESHAPE
    assert f(ctypes.byref(_state(lib, window=17)), 0, p, p, p, p, p, p, 1, None) == ESHAPE
    assert f(ctypes.byref(_state(lib, codes=4097)), 0, p, p, p, p, p, p, 1, None) == EALIGN
    assert f(None, 0, p, p, p, p, p, p, 1, None) == EINVAL
    fl = lib.leapq_window_flush
    assert fl(ctypes.byref(st), 17, None, p, 1, 0, None, None) == ESTATE
    assert fl(ctypes.byref(st), 0, None, p, 1, 3, None, None) == EINVAL      # smooth_mode
    assert fl(ctypes.byref(st), 0, None, None, 1, 0, None, None) == EINVAL   # q0 missing
    for bad in (1, 9, -1):                                                    # code width
        assert fl(ctypes.byref(_state(lib, bits=bad)), 0, None, p, 1, 0, None, None) == ESHAPE
        assert f(ctypes.byref(_state(lib, bits=bad)), 0, p, p, p, p, p, p, 1, None) == ESHAPE


def test_per_step_state_validation(lib):
    p = ctypes.c_void_p(4096)
    fb, fi = lib.gdn_decode_step_bf16_state, lib.gdn_decode_step_int_state
    assert fb(p, p, p, p, p, p, p, 2, 4, 96, 128, 1, None) == ESHAPE          # d_k
    assert fb(p, p, p, p, p, p, p, 2, 4, 128, 128, 7, None) == EDTYPE
    assert fb(ctypes.c_void_p(4104), p, p, p, p, p, p, 2, 4, 128, 128, 1, None) == EALIGN
    assert fb(p, p, p, p, p, p, p, 2, 4, 128, 128, 1, None) == EINVAL         # all overlap
    assert fi(p, p, 9, p, p, p, p, p, p, 2, 4, 128, 128, 1, None) == ESHAPE   # bits
    assert fi(p, None, 8, p, p, p, p, p, p, 2, 4, 128, 128, 1, None) == EINVAL
    assert fi(p, p, 4, p, p, p, p, p, p, 0, 4, 128, 128, 1, None) == OK        # empty


def test_kda_leapq_validation(lib):
    """The KDA windowed entry points validate as the GDN ones, and read the
    per-channel decays 16 bytes at a time."""
    p = ctypes.c_void_p(4096)
    st = _state(lib)
    f = lib.kda_leapq_decode_step
    assert f(ctypes.byref(st), 16, p, p, p, p, p, p, 1, None) == ESTATE
    assert f(ctypes.byref(_state(lib, rank=9)), 0, p, p, p, p, p, p, 1, None) == ESHAPE
    assert f(ctypes.byref(st), 0, p, p, p, ctypes.c_void_p(4100), p, p, 1, None) == EALIGN
    assert "kda_leapq_decode_step" in _err(lib)
    assert f(None, 0, p, p, p, p, p, p, 1, None) == EINVAL
    fl = lib.kda_leapq_window_flush
    assert fl(ctypes.byref(st), 17, None, p, 1, 0, None, None) == ESTATE
    assert fl(ctypes.byref(st), 0, None, None, 1, 0, None, None) == EINVAL   # q0 missing
    assert fl(ctypes.byref(_state(lib, buf_a=4100)), 0, None, p, 1, 0, None, None) == EALIGN


def test_leapq_decode_flush_validation(lib):
    """The window-closing entry points check the token as the decode step and the
    flush arguments as the flush, and launch nothing on an error."""
    q, k, v, a, b, q0 = (ctypes.c_void_p(x << 20) for x in range(1, 7))
    o = ctypes.c_void_p(1 << 40)
    st = _state(lib)
    for name in ("leapq_decode_flush", "kda_leapq_decode_flush"):
        f = getattr(lib, name)
        assert f(None, q, k, v, a, b, o, 1, q0, 1, 0, None) == EINVAL
        assert f(ctypes.byref(_state(lib, rank=9)), q, k, v, a, b, o, 1, q0, 1, 0, None) == ESHAPE
        assert f(ctypes.byref(_state(lib, window=0)), q, k, v, a, b, o, 1, q0, 1, 0, None) == ESHAPE
        assert f(ctypes.byref(st), q, k, v, a, b, o, 7, q0, 1, 0, None) == EDTYPE
        assert f(ctypes.byref(st), q, k, v, a, b, o, 1, q0, 1, 3, None) == EINVAL     # smooth_mode
        assert f(ctypes.byref(st), q, k, v, a, b, o, 1, q0, 65, 0, None) == EINVAL    # iters
        assert f(ctypes.byref(st), q, k, v, a, b, o, 1, None, 1, 0, None) == EINVAL   # q0 missing
        assert f(ctypes.byref(st), q, None, v, a, b, o, 1, q0, 1, 0, None) == EINVAL
        assert f(ctypes.byref(st), q, k, v, a, b, ctypes.c_void_p((1 << 40) + 2), 1, q0, 1, 0, None) == EALIGN
        assert f(ctypes.byref(st), q, k, v, a, b, q, 1, q0, 1, 0, None) == EINVAL     # o is q
        assert name in _err(lib)
        # o against the state the launch writes, and against the buffer it reads
        far = dict(codes=1 << 41, vscale=(1 << 41) + (1 << 22), ksmooth=(1 << 41) + (2 << 22),
                   ct_k=(1 << 41) + (3 << 22), ct_u=(1 << 41) + (4 << 22), buf_k=(1 << 41) + (5 << 22),
                   buf_u=(1 << 41) + (6 << 22), buf_a=(1 << 41) + (7 << 22))
        for field in ("vscale", "ksmooth", "buf_a", "ct_u"):
            kw = dict(far)
            kw[field] = 1 << 40
            assert f(ctypes.byref(_state(lib, **kw)), q, k, v, a, b, o, 1, q0, 1, 0, None) == EINVAL, field
            assert "o overlaps" in _err(lib)
        # a token input inside the stored state the launch rewrites (a cross-block race)
        for field, arg in (("codes", 0), ("vscale", 4), ("ksmooth", 3), ("ct_k", 1), ("ct_u", 2)):
            kw = dict(far)
            kw[field] = (arg + 1) << 20
            assert f(ctypes.byref(_state(lib, **kw)), q, k, v, a, b, o, 1, q0, 1, 0, None) == EINVAL, field
            assert "token input overlaps" in _err(lib)
        assert f(ctypes.byref(_state(lib, N=0, **far)), q, k, v, a, b, o, 1, q0, 1, 0, None) == OK
        assert f(ctypes.byref(_state(lib, N=0)), q, k, v, a, b, o, 1, q0, 1, 0, None) == OK


def test_kda_chunk_validation(lib):
    p = ctypes.c_void_p(4096)
    f = lib.kda_chunk_fwd
    assert lib.kda_chunk_fwd_workspace_bytes(32, 16384, 128, 128, 64) == 32 * 256 * 82432
    assert lib.kda_chunk_fwd_workspace_bytes(32, 100, 128, 128, 64) == 0
    assert f(p, p, p, p, p, None, p, p, 2, 128, 128, 128, 64, 1, p, 10, None) == EINVAL      # workspace
    assert f(p, p, p, p, p, None, p, p, 2, 96, 128, 128, 64, 1, p, 1 << 30, None) == ESHAPE  # T % 64
    # the per-channel decays are read 16 bytes at a time
    assert f(p, p, p, ctypes.c_void_p(4100), p, None, p, p, 2, 128, 128, 128, 64, 1, p, 1 << 30,
             None) == EALIGN
    assert "kda_chunk_fwd" in _err(lib)


def test_gla_bwd_validation(lib):
    p = ctypes.c_void_p(4096)
    f = lib.gla_chunk_bwd
    assert lib.gla_chunk_bwd_workspace_bytes(64, 4096, 128, 128, 64) == 64 * 64 * 132608
    assert lib.gla_chunk_bwd_workspace_bytes(64, 100, 128, 128, 64) == 0
    args = lambda T, ws_bytes, **kw: [kw.get(n, p) for n in ("q", "k", "v", "g", "S0", "dO", "dST", "dq", "dk",
                                                          "dv", "dg", "dS0")] + [2, T, 128, 128, 64, 1, p,
                                                                                 ws_bytes, None]
    assert f(*args(128, 10)) == EINVAL                                   # workspace too small
    assert f(*args(96, 1 << 34)) == ESHAPE                               # T % 64
    assert f(*args(128, 1 << 34, q=ctypes.c_void_p(4098))) == EALIGN
    assert f(*args(128, 1 << 34, dS0=None)) == EINVAL
    assert "gla_chunk_bwd" in _err(lib)


def test_gdn_bwd_validation(lib):
    p = ctypes.c_void_p(4096)
    f = lib.gdn_chunk_bwd
    per_chunk = 81984 + 8192 + 2 * 32768 + 16384 + 16384 + 256 + 4
    assert lib.gdn_chunk_bwd_workspace_bytes(32, 16384, 128, 128, 64) == 32 * 256 * per_chunk
    assert lib.gdn_chunk_bwd_workspace_bytes(32, 100, 128, 128, 64) == 0
    names = ("q", "k", "v", "a", "b", "S0", "dO", "dST", "dq", "dk", "dv", "da", "db", "dS0")
    args = lambda T, ws_bytes, **kw: [kw.get(n, p) for n in names] + [2, T, 128, 128, 64, 1, p, ws_bytes, None]
    assert f(*args(128, 10)) == EINVAL                                   # workspace too small
    assert f(*args(96, 1 << 34)) == ESHAPE                               # T % 64
    assert f(*args(128, 1 << 34, k=ctypes.c_void_p(4104))) == EALIGN
    assert f(*args(128, 1 << 34, dS0=None)) == EINVAL
    assert f(*args(128, 1 << 34)) == EINVAL                              # outputs overlap inputs
    assert "gdn_chunk_bwd" in _err(lib)


def test_gla_shard_validation(lib):
    p = ctypes.c_void_p(4096)
    ws_need = 2 * 2 * 16896
    # gla_shard_decay(workspace, ws_bytes, gamma, N, T, dk, chunk, stream)
    f = lib.gla_shard_decay
    assert f(p, ws_need - 1, ctypes.c_void_p(1 << 30), 2, 128, 128, 64, None) == EINVAL
    assert f(p, ws_need, ctypes.c_void_p(1 << 30), 2, 96, 128, 64, None) == ESHAPE
    assert f(p, ws_need, ctypes.c_void_p((1 << 30) + 4), 2, 128, 128, 64, None) == EALIGN
    assert f(p, ws_need, None, 2, 128, 128, 64, None) == EINVAL
    assert f(p, ws_need, p, 2, 128, 128, 64, None) == EINVAL           # gamma overlaps the workspace
    assert "gla_shard_decay" in _err(lib)
    assert f(p, 0, None, 0, 128, 128, 64, None) == OK                  # nothing to do
    # gla_all_scan_step(S_recv, gamma, gamma_stride, S_local, S_send, N, dk, dv, k0, k1, stream)
    f = lib.gla_all_scan_step
    a, b, c, g = (ctypes.c_void_p(x << 30) for x in (1, 2, 3, 4))
    assert f(a, g, 128, b, c, 2, 128, 128, 0, 129, None) == ESHAPE      # key block past d_k
    assert f(a, g, 128, b, c, 2, 128, 128, 64, 32, None) == ESHAPE     # k1 < k0
    assert f(a, None, 128, b, c, 2, 128, 128, 0, 128, None) == EINVAL  # S_recv without gamma
    assert f(a, g, 64, b, c, 2, 128, 128, 0, 128, None) == ESHAPE      # gamma_stride < d_k
    assert f(a, g, 128, b, ctypes.c_void_p((2 << 30) + 256), 2, 128, 128, 0, 128, None) == EINVAL
    assert "gla_all_scan_step" in _err(lib)
    assert f(a, g, 128, b, c, 2, 128, 128, 16, 16, None) == OK          # empty key block
    assert f(a, g, 128, b, c, 0, 128, 128, 0, 128, None) == OK
    # gla_shard_output_correct(workspace, ws_bytes, gamma, S_in, o, N, T, dk, dv, chunk, io, stream)
    f = lib.gla_shard_output_correct
    assert f(a, ws_need, g, b, c, 2, 128, 128, 128, 64, 0, None) == EDTYPE
    assert f(a, ws_need, g, None, c, 2, 128, 128, 128, 64, 1, None) == OK   # no incoming state
    assert f(a, ws_need - 1, g, b, c, 2, 128, 128, 128, 64, 1, None) == EINVAL
    assert f(a, ws_need, g, b, ctypes.c_void_p((3 << 30) + 8), 2, 128, 128, 128, 64, 1, None) == EALIGN
    assert f(a, ws_need, g, b, ctypes.c_void_p((1 << 30) + 1024), 2, 128, 128, 128, 64, 1, None) == EINVAL
    assert f(a, ws_need, g, b, c, 2, 100, 128, 128, 64, 1, None) == ESHAPE
    assert "gla_shard_output_correct" in _err(lib)


def test_gla_shard_bwd_state_validation(lib):
    p = ctypes.c_void_p(4096)
    f = lib.gla_shard_bwd_state
    q, k, g, dO, dS0, ws = (ctypes.c_void_p(x << 30) for x in (1, 2, 3, 4, 5, 6))
    need = 2 * 2 * 132608
    assert f(q, k, g, dO, dS0, 2, 128, 128, 128, 64, 1, ws, need - 1, None) == EINVAL
    assert "gla_shard_bwd_state" in _err(lib)
    assert f(q, k, g, dO, dS0, 2, 96, 128, 128, 64, 1, ws, need, None) == ESHAPE
    assert f(q, k, g, dO, dS0, 2, 128, 128, 128, 64, 0, ws, need, None) == EDTYPE
    assert f(q, ctypes.c_void_p((2 << 30) + 8), g, dO, dS0, 2, 128, 128, 128, 64, 1, ws, need, None) == EALIGN
    assert f(q, k, g, dO, None, 2, 128, 128, 128, 64, 1, ws, need, None) == EINVAL
    assert f(q, k, g, dO, ctypes.c_void_p((1 << 30) + 4096), 2, 128, 128, 128, 64, 1, ws, need, None) == EINVAL
    assert f(q, k, g, dO, dS0, 0, 128, 128, 128, 64, 1, ws, need, None) == OK


def test_hbm_stream_validation(lib):
    f = lib.gdnrt_hbm_stream
    p = ctypes.c_void_p(4096)
    assert f(p, p, 0, 1, 1.0, None) == OK                                      # empty
    assert f(None, p, 16, 1, 1.0, None) == EINVAL
    assert f(p, p, 18, 1, 1.0, None) == ESHAPE                                 # n % 4
    assert f(p, p, 16, 3, 1.0, None) == ESHAPE                                 # vec
    assert f(ctypes.c_void_p(4100), p, 16, 1, 1.0, None) == EALIGN
    assert f(ctypes.c_void_p(4096 + 32), p, 64, 1, 1.0, None) == EINVAL        # partial overlap
    assert "gdnrt_hbm_stream" in _err(lib)

"""Thin Python binding of the gdnrt C ABI (include/gdnrt.h).

Argument marshalling only: every step of the computation runs in the HIP kernels
of ``libgdnrt.so``. torch supplies device memory and the current stream. If the
library has not been built, or no GPU is visible, calls raise; there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdnrt.so")

OK, EINVAL, ESHAPE, EALIGN, EDTYPE, ESTATE, ELAUNCH = range(7)
F32, BF16 = 0, 1
GLA_SHARD = 0x100   # or-ed into gla_chunk_fwd's io: keep what the shard calls read
D = 128
CHUNK = 64

_c_int, _vp, _fp = ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p


class LeapqState(ctypes.Structure):
    """Mirror of ``leapq_state`` (device pointers + sizes)."""
    _fields_ = [("codes", _vp), ("vscale", _vp), ("ksmooth", _vp), ("ct_k", _vp),
                ("ct_u", _vp), ("buf_k", _vp), ("buf_u", _vp), ("buf_a", _vp),
                ("N", _c_int), ("dk", _c_int), ("dv", _c_int), ("rank", _c_int),
                ("window", _c_int), ("bits", _c_int)]


# exported symbol -> (argtypes, restype); mirrors include/gdnrt.h
SIGNATURES = {
    "gdn_decode_step": ([_vp] * 7 + [_c_int] * 5 + [_vp], _c_int),
    "kda_decode_step": ([_vp] * 7 + [_c_int] * 5 + [_vp], _c_int),
    "gla_chunk_fwd": ([_vp] * 7 + [_c_int] * 6 + [_vp, ctypes.c_size_t, _vp], _c_int),
    "gla_chunk_fwd_workspace_bytes": ([_c_int] * 5, ctypes.c_size_t),
    "gla_shard_decay": ([_vp, ctypes.c_size_t, _vp] + [_c_int] * 4 + [_vp], _c_int),
    "gla_all_scan_step": ([_vp, _vp, ctypes.c_size_t, _vp, _vp] + [_c_int] * 5 + [_vp], _c_int),
    "gla_shard_output_correct": ([_vp, ctypes.c_size_t, _vp, _vp, _vp] + [_c_int] * 6 + [_vp], _c_int),
    "gdn_chunk_fwd": ([_vp] * 8 + [_c_int] * 6 + [_vp, ctypes.c_size_t, _vp], _c_int),
    "gdn_chunk_fwd_workspace_bytes": ([_c_int] * 5, ctypes.c_size_t),
    "kda_chunk_fwd": ([_vp] * 8 + [_c_int] * 6 + [_vp, ctypes.c_size_t, _vp], _c_int),
    "gla_chunk_bwd": ([_vp] * 12 + [_c_int] * 6 + [_vp, ctypes.c_size_t, _vp], _c_int),
    "gla_chunk_bwd_workspace_bytes": ([_c_int] * 5, ctypes.c_size_t),
    "gla_shard_bwd_state": ([_vp] * 5 + [_c_int] * 6 + [_vp, ctypes.c_size_t, _vp], _c_int),
    "gla_shard_bwd_grads": ([_vp] * 12 + [_c_int] * 6 + [_vp, ctypes.c_size_t, _vp], _c_int),
    "gdn_decode_step_bf16_state": ([_vp] * 7 + [_c_int] * 5 + [_vp], _c_int),
    "gdn_decode_step_int_state": ([_vp, _vp, _c_int] + [_vp] * 6 + [_c_int] * 5 + [_vp], _c_int),
    "gdn_chunk_bwd": ([_vp] * 14 + [_c_int] * 6 + [_vp, ctypes.c_size_t, _vp], _c_int),
    "gdn_chunk_bwd_workspace_bytes": ([_c_int] * 5, ctypes.c_size_t),
    "kda_chunk_fwd_workspace_bytes": ([_c_int] * 5, ctypes.c_size_t),
    "leapq_decode_step": ([ctypes.POINTER(LeapqState), _c_int] + [_vp] * 6 + [_c_int, _vp], _c_int),
    "leapq_window_flush": ([ctypes.POINTER(LeapqState), _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp],
                           _c_int),
    "kda_leapq_decode_step": ([ctypes.POINTER(LeapqState), _c_int] + [_vp] * 6 + [_c_int, _vp], _c_int),
    "leapq_decode_flush": ([ctypes.POINTER(LeapqState)] + [_vp] * 6 + [_c_int, _vp, _c_int, _c_int, _vp],
                           _c_int),
    "kda_leapq_decode_flush": ([ctypes.POINTER(LeapqState)] + [_vp] * 6 + [_c_int, _vp, _c_int, _c_int, _vp],
                               _c_int),
    "kda_leapq_window_flush": ([ctypes.POINTER(LeapqState), _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp],
                               _c_int),
    "gdn_chunk_fwd_noalloc": ([_vp] * 8 + [_c_int] * 6 + [_vp], _c_int),
    "gdn_chunk_fwd_noalloc_max_bytes": ([], ctypes.c_size_t),
    "gdnrt_hbm_stream": ([_vp, _vp, ctypes.c_size_t, _c_int, ctypes.c_float, _vp], _c_int),
    "gdnrt_last_error": ([], ctypes.c_char_p),
}

_LIB = None


class GdnrtError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """Load libgdnrt.so (built in-tree) and declare every exported signature."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m delta_rule_recurrent_amd.build` "
                "(the HIP library is required; there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (argt, rest) in SIGNATURES.items():
            f = getattr(L, name, None)
            if f is None:
                continue
            f.argtypes = argt
            f.restype = rest
        _LIB = L
    return _LIB


def _check(fn, status):
    if status != OK:
        raise GdnrtError(fn, status, lib().gdnrt_last_error().decode())


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, shape=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _io(dtype):
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {dtype}")


# ---------------------------------------------------------------- entry points

def gdn_decode_step(S, q, k, v, alpha, beta, o=None):
    """Gated DeltaNet recurrent step(s), state updated in place.

    S [N][128][128] fp32; q, k, v [N][T][128] (fp32 or bf16, one dtype);
    alpha, beta [N][T] fp32. Returns o [N][T][128] in the dtype of q."""
    N, T, _ = q.shape
    io = _io(q.dtype)
    _need(S, "S", torch.float32, (N, D, D))
    for n_, t_ in (("q", q), ("k", k), ("v", v)):
        _need(t_, n_, q.dtype, (N, T, D))
    _need(alpha, "alpha", torch.float32, (N, T))
    _need(beta, "beta", torch.float32, (N, T))
    if o is None:
        o = torch.empty((N, T, D), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (N, T, D))
    _check("gdn_decode_step", lib().gdn_decode_step(
        _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o),
        N, T, D, D, io, _stream()))
    return o


def gdn_decode_step_bf16_state(S, q, k, v, alpha, beta, o=None):
    """Per-step BF16 baseline: gdn_decode_step with S [N][128][128] stored in bf16 and
    re-rounded after every token (in place). Returns o."""
    return _lowp_decode("gdn_decode_step_bf16_state", S, None, 0, q, k, v, alpha, beta, o)


def gdn_decode_step_int_state(codes, rowmax, bits, q, k, v, alpha, beta, o=None):
    """Per-step b-bit baseline: the state is rowmax[v] * codes[v,k] / Q (Q = 2^(bits-1)
    - 1), requantised after every token (codes int8 [N][128][128], rowmax fp32
    [N][128], in place). Returns o."""
    return _lowp_decode("gdn_decode_step_int_state", codes, rowmax, bits, q, k, v, alpha, beta, o)


def _lowp_decode(name, S, rowmax, bits, q, k, v, alpha, beta, o):
    N, T = q.shape[0], q.shape[1]
    _need(S, "S", torch.bfloat16 if rowmax is None else torch.int8, (N, D, D))
    if rowmax is not None:
        _need(rowmax, "rowmax", torch.float32, (N, D))
    for n_, t_ in (("q", q), ("k", k), ("v", v)):
        _need(t_, n_, q.dtype, (N, T, D))
    for n_, t_ in (("alpha", alpha), ("beta", beta)):
        _need(t_, n_, torch.float32, (N, T))
    if o is None:
        o = torch.empty_like(v)
    _need(o, "o", q.dtype, (N, T, D))
    io = _io(q.dtype)
    args = (_ptr(S),) if rowmax is None else (_ptr(S), _ptr(rowmax), bits)
    _check(name, getattr(lib(), name)(*args, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o),
                                      N, T, D, D, io, _stream()))
    return o


def kda_decode_step(S, q, k, v, alpha, beta, o=None):
    """Kimi Delta Attention recurrent step(s) (one decay per key channel), state
    updated in place.

    S [N][128][128] fp32; q, k, v [N][T][128] (fp32 or bf16, one dtype);
    alpha [N][T][128] fp32; beta [N][T] fp32. Returns o [N][T][128] in the dtype of q."""
    N, T, _ = q.shape
    io = _io(q.dtype)
    _need(S, "S", torch.float32, (N, D, D))
    for n_, t_ in (("q", q), ("k", k), ("v", v)):
        _need(t_, n_, q.dtype, (N, T, D))
    _need(alpha, "alpha", torch.float32, (N, T, D))
    _need(beta, "beta", torch.float32, (N, T))
    if o is None:
        o = torch.empty((N, T, D), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (N, T, D))
    _check("kda_decode_step", lib().kda_decode_step(
        _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o),
        N, T, D, D, io, _stream()))
    return o


def gla_chunk_workspace(N, T, device="cuda", chunk=CHUNK):
    """Allocate the workspace gla_chunk_fwd needs for N sequences of T tokens."""
    nb = lib().gla_chunk_fwd_workspace_bytes(N, T, D, D, chunk)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device)


def gla_chunk_fwd(q, k, v, log_g, S0=None, ST=None, o=None, workspace=None, chunk=CHUNK, shard=False):
    """Gated linear attention chunkwise forward from an incoming state.

    q, k, v [N][T][128] bf16; log_g [N][T][128] fp32; S0 [N][128][128] fp32 or
    None; workspace from gla_chunk_workspace (allocated here if None); shard: also
    leave in the workspace what gla_shard_decay / gla_shard_output_correct read.
    Returns (o [N][T][128] bf16, ST [N][128][128] fp32)."""
    N, T, _ = q.shape
    for n_, t_ in (("q", q), ("k", k), ("v", v)):
        _need(t_, n_, torch.bfloat16, (N, T, D))
    _need(log_g, "log_g", torch.float32, (N, T, D))
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, D, D))
    if ST is None:
        ST = torch.empty((N, D, D), dtype=torch.float32, device=q.device)
    _need(ST, "ST", torch.float32, (N, D, D))
    if o is None:
        o = torch.empty((N, T, D), dtype=torch.bfloat16, device=q.device)
    _need(o, "o", torch.bfloat16, (N, T, D))
    if workspace is None:
        workspace = gla_chunk_workspace(N, T, q.device, chunk)
    _need(workspace, "workspace", torch.uint8)
    _check("gla_chunk_fwd", lib().gla_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(S0), _ptr(ST), _ptr(o),
        N, T, D, D, chunk, BF16 | (GLA_SHARD if shard else 0), _ptr(workspace), workspace.numel(), _stream()))
    return o, ST


def gla_shard_decay(workspace, N, T, gamma=None, chunk=CHUNK):
    """ZeCO's cumulative decays of a shard from the workspace its gla_chunk_fwd call
    left: gamma [N][T/chunk + 1][128] fp32, gamma[n][c] = product of the chunk decays
    e^{b_C} of chunks 0..c-1."""
    _need(workspace, "workspace", torch.uint8)
    if gamma is None:
        gamma = torch.empty((N, T // chunk + 1, D), dtype=torch.float32, device=workspace.device)
    _need(gamma, "gamma", torch.float32, (N, T // chunk + 1, D))
    _check("gla_shard_decay", lib().gla_shard_decay(
        _ptr(workspace), workspace.numel(), _ptr(gamma), N, T, D, chunk, _stream()))
    return gamma


def gla_all_scan_step(S_local, gamma_total=None, S_recv=None, S_send=None, k0=0, k1=D):
    """One device's All-Scan update of key channels [k0, k1):
    S_send = gamma_total o S_recv + S_local (S_recv None: S_send = S_local).
    gamma_total [N][128] fp32 with unit stride along the keys (a view such as
    gamma[:, -1] of gla_shard_decay's output is accepted). Returns S_send."""
    N = S_local.shape[0]
    _need(S_local, "S_local", torch.float32, (N, D, D))
    if S_send is None:
        S_send = torch.empty_like(S_local)
    _need(S_send, "S_send", torch.float32, (N, D, D))
    stride = D
    if S_recv is not None:
        _need(S_recv, "S_recv", torch.float32, (N, D, D))
        if not isinstance(gamma_total, torch.Tensor) or gamma_total.dtype != torch.float32 or \
                tuple(gamma_total.shape) != (N, D) or gamma_total.stride(1) != 1 or not gamma_total.is_cuda:
            raise ValueError("gamma_total must be a [N][128] float32 GPU tensor with unit stride along keys")
        stride = gamma_total.stride(0) if N > 1 else D
    _check("gla_all_scan_step", lib().gla_all_scan_step(
        _ptr(S_recv), None if S_recv is None else gamma_total.data_ptr(), stride, _ptr(S_local),
        _ptr(S_send), N, D, D, k0, k1, _stream()))
    return S_send


def gla_shard_output_correct(workspace, gamma, S_in, o, chunk=CHUNK):
    """Adds the received state's share to a shard's outputs (o from gla_chunk_fwd with
    a zero state, updated in place): o_t += S_in (q_t o e^{b_t} o gamma[c(t)])."""
    N, T, _ = o.shape
    _need(o, "o", torch.bfloat16, (N, T, D))
    _need(workspace, "workspace", torch.uint8)
    _need(gamma, "gamma", torch.float32, (N, T // chunk + 1, D))
    if S_in is not None:
        _need(S_in, "S_in", torch.float32, (N, D, D))
    _check("gla_shard_output_correct", lib().gla_shard_output_correct(
        _ptr(workspace), workspace.numel(), _ptr(gamma), _ptr(S_in), _ptr(o), N, T, D, D, chunk, BF16,
        _stream()))
    return o


def gla_shard_local(q, k, v, log_g, workspace=None, chunk=CHUNK):
    """ZeCO's first phase on one device: gla_chunk_fwd from a zero state and the
    cumulative decays. Returns (o_local, S_local, gamma, workspace); the workspace
    is read again by gla_shard_output_correct."""
    N, T, _ = q.shape
    if workspace is None:
        workspace = gla_chunk_workspace(N, T, q.device, chunk)
    o, S_local = gla_chunk_fwd(q, k, v, log_g, None, None, None, workspace, chunk, shard=True)
    gamma = gla_shard_decay(workspace, N, T, chunk=chunk)
    return o, S_local, gamma, workspace


def gdn_chunk_workspace(N, T, device="cuda", chunk=CHUNK):
    """Allocate the workspace gdn_chunk_fwd needs for N sequences of T tokens."""
    nb = lib().gdn_chunk_fwd_workspace_bytes(N, T, D, D, chunk)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device)


def gla_chunk_bwd_workspace(N, T, device="cuda", chunk=CHUNK):
    """Allocate the workspace gla_chunk_bwd needs for N sequences of T tokens."""
    nb = lib().gla_chunk_bwd_workspace_bytes(N, max(T, CHUNK), D, D, chunk)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device)


def gla_chunk_bwd(q, k, v, log_g, dO, S0=None, dST=None, workspace=None, out=None, chunk=CHUNK,
                  _entry="gla_chunk_bwd"):
    """Gated linear attention chunkwise backward: gradients of
    sum(dO * o) + sum(dST * S_T) for the forward of gla_chunk_fwd.

    q, k, v, dO [N][T][128] bf16; log_g [N][T][128] fp32; S0, dST [N][128][128]
    fp32 or None. Returns (dq, dk, dv (bf16), dlog_g (fp32), dS0 (fp32))."""
    N, T, _ = q.shape
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        _need(t_, n_, torch.bfloat16, (N, T, D))
    _need(log_g, "log_g", torch.float32, (N, T, D))
    for n_, t_ in (("S0", S0), ("dST", dST)):
        if t_ is not None:
            _need(t_, n_, torch.float32, (N, D, D))
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(log_g),
               torch.empty((N, D, D), dtype=torch.float32, device=q.device))
    dq, dk, dv, dg, dS0 = out
    if workspace is None:
        workspace = gla_chunk_bwd_workspace(N, T, q.device, chunk)
    _need(workspace, "workspace", torch.uint8)
    _check(_entry, getattr(lib(), _entry)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(S0), _ptr(dO), _ptr(dST), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dg), _ptr(dS0), N, T, D, D, chunk, BF16, _ptr(workspace), workspace.numel(),
        _stream()))
    return dq, dk, dv, dg, dS0


def gla_shard_bwd_state(q, k, log_g, dO, dS0=None, workspace=None, chunk=CHUNK):
    """ZeCO's backward phase 1 on one device: the gradient with respect to the
    shard's incoming state from its own outputs alone (dS = 0 at the shard's end).
    q, k, dO [N][T][128] bf16; log_g fp32; workspace as for gla_chunk_bwd (allocated
    here if None). Returns dS0 [N][128][128] fp32."""
    N, T, _ = q.shape
    for n_, t_ in (("q", q), ("k", k), ("dO", dO)):
        _need(t_, n_, torch.bfloat16, (N, T, D))
    _need(log_g, "log_g", torch.float32, (N, T, D))
    if dS0 is None:
        dS0 = torch.empty((N, D, D), dtype=torch.float32, device=q.device)
    _need(dS0, "dS0", torch.float32, (N, D, D))
    if workspace is None:
        workspace = gla_chunk_bwd_workspace(N, T, q.device, chunk)
    _need(workspace, "workspace", torch.uint8)
    _check("gla_shard_bwd_state", lib().gla_shard_bwd_state(
        _ptr(q), _ptr(k), _ptr(log_g), _ptr(dO), _ptr(dS0), N, T, D, D, chunk, BF16, _ptr(workspace),
        workspace.numel(), _stream()))
    return dS0


def gla_shard_bwd_grads(q, k, v, log_g, dO, workspace, S0=None, dST=None, out=None, chunk=CHUNK):
    """gla_chunk_bwd in a workspace where gla_shard_bwd_state has just run on the same
    q, k, log_g (its per-chunk preparation is reused). Returns as gla_chunk_bwd."""
    return gla_chunk_bwd(q, k, v, log_g, dO, S0, dST, workspace, out, chunk, _entry="gla_shard_bwd_grads")


def gdn_chunk_bwd_workspace(N, T, device="cuda", chunk=CHUNK):
    """Allocate the workspace gdn_chunk_bwd needs for N sequences of T tokens."""
    nb = lib().gdn_chunk_bwd_workspace_bytes(N, max(T, CHUNK), D, D, chunk)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device)


def gdn_chunk_bwd(q, k, v, alpha, beta, dO, S0=None, dST=None, workspace=None, out=None, chunk=CHUNK):
    """Gated DeltaNet chunkwise backward: gradients of sum(dO * o) + sum(dST * S_T)
    for the forward of gdn_chunk_fwd.

    q, k, v, dO [N][T][128] bf16; alpha, beta [N][T] fp32; S0, dST [N][128][128]
    fp32 or None. Returns (dq, dk, dv (bf16), dalpha, dbeta, dS0 (fp32))."""
    N, T, _ = q.shape
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        _need(t_, n_, torch.bfloat16, (N, T, D))
    for n_, t_ in (("alpha", alpha), ("beta", beta)):
        _need(t_, n_, torch.float32, (N, T))
    for n_, t_ in (("S0", S0), ("dST", dST)):
        if t_ is not None:
            _need(t_, n_, torch.float32, (N, D, D))
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(alpha),
               torch.empty_like(beta), torch.empty((N, D, D), dtype=torch.float32, device=q.device))
    dq, dk, dv, da, db, dS0 = out
    if workspace is None:
        workspace = gdn_chunk_bwd_workspace(N, T, q.device, chunk)
    _need(workspace, "workspace", torch.uint8)
    _check("gdn_chunk_bwd", lib().gdn_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dST), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(da), _ptr(db), _ptr(dS0), N, T, D, D, chunk, BF16, _ptr(workspace),
        workspace.numel(), _stream()))
    return dq, dk, dv, da, db, dS0


def kda_chunk_workspace(N, T, device="cuda", chunk=CHUNK):
    """Allocate the workspace kda_chunk_fwd needs for N sequences of T tokens."""
    nb = lib().kda_chunk_fwd_workspace_bytes(N, T, D, D, chunk)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device)


def kda_chunk_fwd(q, k, v, alpha, beta, S0=None, ST=None, o=None, workspace=None, chunk=CHUNK):
    """Kimi Delta Attention chunkwise forward (prefill), one decay per key channel.

    q, k, v [N][T][128] bf16; alpha [N][T][128] fp32; beta [N][T] fp32; S0
    [N][128][128] fp32 or None; workspace from kda_chunk_workspace (allocated here
    if None). Returns (o [N][T][128] bf16, ST [N][128][128] fp32)."""
    return _chunk_fwd("kda_chunk_fwd", kda_chunk_workspace, (q.shape[0], q.shape[1], D),
                      q, k, v, alpha, beta, S0, ST, o, workspace, chunk)


def gdn_chunk_fwd(q, k, v, alpha, beta, S0=None, ST=None, o=None, workspace=None, chunk=CHUNK):
    """Gated DeltaNet chunkwise forward (prefill).

    q, k, v [N][T][128] bf16; alpha, beta [N][T] fp32; S0 [N][128][128] fp32 or
    None; workspace from gdn_chunk_workspace (allocated here if None).
    Returns (o [N][T][128] bf16, ST [N][128][128] fp32)."""
    return _chunk_fwd("gdn_chunk_fwd", gdn_chunk_workspace, (q.shape[0], q.shape[1]),
                      q, k, v, alpha, beta, S0, ST, o, workspace, chunk)


def gdn_chunk_fwd_noalloc(q, k, v, alpha, beta, S0, ST, o):
    """gdn_chunk_fwd through the allocation-free entry point (the library's fixed
    scratch instead of a workspace). Every tensor, outputs included, is the caller's:
    o [N][T][128] bf16 and ST [N][128][128] fp32 must be passed in."""
    N, T, _ = q.shape
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t_, n_, torch.bfloat16, (N, T, D))
    _need(alpha, "alpha", torch.float32, (N, T))
    _need(beta, "beta", torch.float32, (N, T))
    _need(ST, "ST", torch.float32, (N, D, D))
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, D, D))
    _check("gdn_chunk_fwd_noalloc", lib().gdn_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(ST), _ptr(o),
        N, T, D, D, CHUNK, BF16, _stream()))
    return o, ST


def _chunk_fwd(name, alloc, alpha_shape, q, k, v, alpha, beta, S0, ST, o, workspace, chunk):
    N, T, _ = q.shape
    for n_, t_ in (("q", q), ("k", k), ("v", v)):
        _need(t_, n_, torch.bfloat16, (N, T, D))
    _need(alpha, "alpha", torch.float32, alpha_shape)
    _need(beta, "beta", torch.float32, (N, T))
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, D, D))
    if ST is None:
        ST = torch.empty((N, D, D), dtype=torch.float32, device=q.device)
    _need(ST, "ST", torch.float32, (N, D, D))
    if o is None:
        o = torch.empty((N, T, D), dtype=torch.bfloat16, device=q.device)
    _need(o, "o", torch.bfloat16, (N, T, D))
    if workspace is None:
        workspace = alloc(N, T, q.device, chunk)
    _need(workspace, "workspace", torch.uint8)
    _check(name, getattr(lib(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(ST), _ptr(o),
        N, T, D, D, chunk, BF16, _ptr(workspace), workspace.numel(), _stream()))
    return o, ST


def code_row_bytes(bits):
    """Bytes of one value row of LeapQuant codes (128 codes) at this width."""
    return 16 * bits if bits in (4, 6) else D


class LeapqBuffers:
    """Caller-owned device memory of a LeapQuant state for N heads (see
    ``leapq_state`` in include/gdnrt.h). Allocated once by torch."""

    def __init__(self, N, rank=4, window=16, device="cuda", kda=False, bits=8):
        self.N, self.rank, self.window, self.kda, self.bits = N, rank, window, kda, bits
        f = dict(dtype=torch.float32, device=device)
        # one value row of codes: packed at 4 and 6 bits (include/gdnrt.h), a byte per code otherwise
        self.codes = torch.zeros((N, D, code_row_bytes(bits)), dtype=torch.int8, device=device)
        self.vscale = torch.zeros((N, D), **f)
        self.ksmooth = torch.ones((N, D), **f)
        # fp16 bit patterns; view as torch.float16 for reading
        self.ct_k = torch.zeros((N, max(rank, 1), D), dtype=torch.float16, device=device)
        self.ct_u = torch.zeros((N, max(rank, 1), D), dtype=torch.float16, device=device)
        self.buf_k = torch.zeros((N, window, D), **f)
        self.buf_u = torch.zeros((N, window, D), **f)
        # Gated DeltaNet: one decay per buffered token; KDA: one per key channel
        self.buf_a = torch.zeros((N, window, D) if kda else (N, window), **f)
        self.pos = 0
        self._st = LeapqState(
            _ptr(self.codes), _ptr(self.vscale), _ptr(self.ksmooth), _ptr(self.ct_k),
            _ptr(self.ct_u), _ptr(self.buf_k), _ptr(self.buf_u), _ptr(self.buf_a),
            N, D, D, rank, window, bits)

    @property
    def struct(self):
        return self._st

    def code_values(self):
        """The signed codes [N][128][128] as int8, unpacked from the stored rows by
        torch ops on the codes' device (for inspection and studies, not the decode
        path): at 4 bits byte j holds codes 2j and 2j+1 in its low and high nibble, at 6
        bits each 3 bytes hold four codes in 6-bit fields of a little-endian 24-bit
        word, two's complement."""
        raw = self.codes.view(torch.uint8).to(torch.int32)
        if self.bits == 4:
            z = torch.stack((raw & 15, raw >> 4), dim=-1).reshape(self.N, D, D)
            return torch.where(z >= 8, z - 16, z).to(torch.int8)
        if self.bits == 6:
            g = raw.reshape(self.N, D, 32, 3)
            w = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
            z = torch.stack([(w >> (6 * i)) & 63 for i in range(4)], dim=-1).reshape(self.N, D, D)
            return torch.where(z >= 32, z - 64, z).to(torch.int8)
        return self.codes


def _flush(name, st, q0, dense, iters, smooth_mode, pre_round):
    _need(q0, "q0", torch.float32, (D, st.rank) if st.rank > 0 else None)
    if dense is not None:
        _need(dense, "dense", torch.float32, (st.N, D, D))
    if pre_round is not None:
        _need(pre_round, "pre_round", torch.float32, (st.N, D, D))
    _check(name, getattr(lib(), name)(
        ctypes.byref(st.struct), st.pos, _ptr(dense), _ptr(q0), iters, smooth_mode,
        _ptr(pre_round), _stream()))
    st.pos = 0


def _decode(name, st, q, k, v, alpha, beta, o, alpha_shape):
    N = st.N
    io = _io(q.dtype)
    for n_, t_ in (("q", q), ("k", k), ("v", v)):
        _need(t_, n_, q.dtype, (N, D))
    _need(alpha, "alpha", torch.float32, alpha_shape)
    _need(beta, "beta", torch.float32, (N,))
    if o is None:
        o = torch.empty((N, D), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (N, D))
    _check(name, getattr(lib(), name)(
        ctypes.byref(st.struct), st.pos, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(o), io, _stream()))
    st.pos += 1
    return o


def leapq_window_flush(st: LeapqBuffers, q0, dense=None, iters=1, smooth_mode=0, pre_round=None):
    """Rebuild (or take ``dense``), fit compensator tokens, smooth, round once.
    Resets the window position to 0."""
    if st.kda:
        raise ValueError("leapq_window_flush: the buffers hold per-channel decays (use kda_leapq_window_flush)")
    _flush("leapq_window_flush", st, q0, dense, iters, smooth_mode, pre_round)


def leapq_decode_step(st: LeapqBuffers, q, k, v, alpha, beta, o=None):
    """One token per head inside the open window; appends its record."""
    if st.kda:
        raise ValueError("leapq_decode_step: the buffers hold per-channel decays (use kda_leapq_decode_step)")
    return _decode("leapq_decode_step", st, q, k, v, alpha, beta, o, (st.N,))


def kda_leapq_window_flush(st: LeapqBuffers, q0, dense=None, iters=1, smooth_mode=0, pre_round=None):
    """KDA windowed state: rebuild with per-channel decays (or take ``dense``),
    fit compensator tokens, smooth, round once. Resets the window position to 0."""
    if not st.kda:
        raise ValueError("kda_leapq_window_flush: allocate the buffers with kda=True")
    _flush("kda_leapq_window_flush", st, q0, dense, iters, smooth_mode, pre_round)


def kda_leapq_decode_step(st: LeapqBuffers, q, k, v, alpha, beta, o=None):
    """KDA windowed state: one token per head (alpha [N][128], one decay per key
    channel) inside the open window; appends its record."""
    if not st.kda:
        raise ValueError("kda_leapq_decode_step: allocate the buffers with kda=True")
    return _decode("kda_leapq_decode_step", st, q, k, v, alpha, beta, o, (st.N, D))


def _decode_flush(name, st, q, k, v, alpha, beta, o, alpha_shape, q0, iters, smooth_mode):
    N = st.N
    if st.pos != st.window - 1:
        raise ValueError(f"{name}: {st.pos} records buffered, the window's last token needs {st.window - 1}")
    io = _io(q.dtype)
    for n_, t_ in (("q", q), ("k", k), ("v", v)):
        _need(t_, n_, q.dtype, (N, D))
    _need(alpha, "alpha", torch.float32, alpha_shape)
    _need(beta, "beta", torch.float32, (N,))
    _need(q0, "q0", torch.float32, (D, st.rank) if st.rank > 0 else None)
    if o is None:
        o = torch.empty((N, D), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (N, D))
    _check(name, getattr(lib(), name)(
        ctypes.byref(st.struct), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), io,
        _ptr(q0), iters, smooth_mode, _stream()))
    st.pos = 0
    return o


def leapq_decode_flush(st: LeapqBuffers, q, k, v, alpha, beta, q0, o=None, iters=1, smooth_mode=0):
    """The window's last token and the flush in one launch (window - 1 records
    buffered). Returns o; resets the window position to 0."""
    if st.kda:
        raise ValueError("leapq_decode_flush: the buffers hold per-channel decays (use kda_leapq_decode_flush)")
    return _decode_flush("leapq_decode_flush", st, q, k, v, alpha, beta, o, (st.N,), q0, iters, smooth_mode)


def kda_leapq_decode_flush(st: LeapqBuffers, q, k, v, alpha, beta, q0, o=None, iters=1, smooth_mode=0):
    """KDA form of leapq_decode_flush (alpha [N][128])."""
    if not st.kda:
        raise ValueError("kda_leapq_decode_flush: allocate the buffers with kda=True")
    return _decode_flush("kda_leapq_decode_flush", st, q, k, v, alpha, beta, o, (st.N, D), q0, iters, smooth_mode)


def hbm_stream(dst, src, vec=1, scale=1.0):
    """Streaming read + write of an fp32 array (``dst`` may be ``src``): the HBM
    ceiling kernel. Not a step of the method."""
    _need(src, "src", torch.float32)
    _need(dst, "dst", torch.float32, src.shape)
    _check("gdnrt_hbm_stream", lib().gdnrt_hbm_stream(_ptr(dst), _ptr(src), src.numel(), vec,
                                                      float(scale), _stream()))
    return dst

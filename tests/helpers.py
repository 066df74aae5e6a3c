"""Shared test utilities: device checks, tolerances, host copies."""
import numpy as np
import torch


def need_gpu():
    """GPU tests fail (not skip) without a GPU: the HIP path must be the one run."""
    assert torch.cuda.is_available(), "this test needs an MI355X GPU"
    import delta_rule_recurrent_amd as m
    m.lib()
    return torch.device("cuda:0")


def np64(t):
    """Exact fp64 host copy of a tensor (bf16 and fp16 upcast bit-exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_err(got, ref):
    """max |got - ref| / max |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def assert_rel(got, ref, tol, what=""):
    e = rel_err(got, ref)
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{what}: non-finite values"
    assert e <= tol, f"{what}: max-abs error {e:.3e} of max|ref| exceeds {tol:.1e}"
    return e


def say(*a):
    print(*a, flush=True)


def unpack_codes(raw, bits):
    """int8 LeapQuant codes [..., 128] from value rows as stored: packed at 4 and 6 bits
    (at 4 bits byte j holds codes 2j, 2j+1 in its low and high nibble; at 6 bits each 3
    bytes hold codes 4c+i in bits [6i, 6i+6) of a little-endian 24-bit group; two's
    complement), a byte per code otherwise. Written from that description of the
    layout, independently of the kernels."""
    raw = np.ascontiguousarray(np.asarray(raw)).view(np.uint8)
    lead = raw.shape[:-1]
    if bits == 4:
        z = np.stack([raw & 15, raw >> 4], axis=-1).reshape(*lead, 128).astype(np.int16)
        return np.where(z >= 8, z - 16, z).astype(np.int8)
    if bits == 6:
        g = raw.reshape(*lead, 32, 3).astype(np.uint32)
        word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
        z = np.stack([(word >> (6 * i)) & 63 for i in range(4)], axis=-1).reshape(*lead, 128).astype(np.int16)
        return np.where(z >= 32, z - 64, z).astype(np.int8)
    return raw.view(np.int8)


def pack_codes(z, bits):
    """The stored bytes of int8 codes [..., 128] (the inverse of unpack_codes)."""
    z = np.asarray(z).astype(np.int64)
    lead = z.shape[:-1]
    if bits == 4:
        u = (z & 15).reshape(*lead, 64, 2)
        return (u[..., 0] | (u[..., 1] << 4)).astype(np.uint8)
    if bits == 6:
        u = (z & 63).reshape(*lead, 32, 4)
        word = u[..., 0] | (u[..., 1] << 6) | (u[..., 2] << 12) | (u[..., 3] << 18)
        return np.stack([word & 255, (word >> 8) & 255, (word >> 16) & 255], axis=-1).reshape(*lead, 96).astype(np.uint8)
    return z.astype(np.int8).view(np.uint8)


def codes_of(st, heads=None):
    """The int8 codes [N][128][128] of a LeapqBuffers state (unpacked on the host)."""
    raw = st.codes if heads is None else st.codes[heads]
    return unpack_codes(raw.cpu().numpy(), st.bits)

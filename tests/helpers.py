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

"""Helpers shared by the GPU parity tests (not a test module)."""
import numpy as np
import torch

EPS32 = 2.0 ** -24


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def empty(shape, dtype=torch.float32, fill=float("nan")):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if dtype.is_floating_point:
        t.fill_(fill)
    return t


def assert_close_bound(got, ref, bound, what=""):
    """Elementwise |got - ref| <= bound (bound broadcastable)."""
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} exceed bound; worst at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r} bound {np.broadcast_to(bound, err.shape)[i]!r}")


def assert_rel(got, ref, rtol, atol=0.0, what=""):
    assert_close_bound(got, ref, atol + rtol * np.abs(ref), what)


def normwise(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))

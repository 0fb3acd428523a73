"""Shared test helpers: tolerance checks and GPU availability."""
import numpy as np


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def rel_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    nr = np.linalg.norm(ref.ravel())
    mr = np.abs(ref).max() if ref.size else 0.0
    l2 = np.linalg.norm(d.ravel()) / nr if nr > 0 else np.linalg.norm(d.ravel())
    linf = np.abs(d).max() / mr if mr > 0 else (np.abs(d).max() if d.size else 0.0)
    return l2, linf


def assert_close(got, ref, tol, what=""):
    """Per-tensor relative L2 and relative max-abs error both within tol."""
    l2, linf = rel_errors(got, ref)
    assert l2 <= tol and linf <= tol, f"{what}: rel_l2={l2:.3e} rel_linf={linf:.3e} tol={tol:g}"
    return l2, linf

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


def assert_close_local(got, ref, tol, what="", block_rows=64, block_cols=None):
    """assert_close on the whole tensor, plus the same relative L2 bound on
    every block of block_rows rows x block_cols columns (all columns when
    None; e.g. one attention head's 64 rows), so that an error confined to a
    small-magnitude region (one head, the first causal rows, one layer's
    bias gradient) cannot hide under the tensor's norm.  A block whose
    reference is far below the tensor's RMS -- a structural zero such as the
    key-bias gradient of softmax attention, which is exactly zero -- is held
    to tol times half the RMS norm of a typical block instead."""
    assert_close(got, ref, tol, what)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return
    if ref.ndim == 1:
        got, ref = got[:, None], ref[:, None]
    got = got.reshape(ref.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:  # an exactly zero reference: the absolute whole-tensor check above decides
        return
    rows, cols = ref.shape
    bc = cols if block_cols is None else block_cols
    for r0 in range(0, rows, block_rows):
        for c0 in range(0, cols, bc):
            rb, gb = ref[r0:r0 + block_rows, c0:c0 + bc], got[r0:r0 + block_rows, c0:c0 + bc]
            nr = max(np.linalg.norm(rb), 0.5 * rms * np.sqrt(rb.size))
            e = np.linalg.norm(gb - rb) / nr
            assert e <= tol, f"{what}: block rows {r0}.. cols {c0}..: rel_l2={e:.3e} tol={tol:g}"

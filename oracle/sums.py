"""The AllReduce-point sum in the storage type (test infrastructure only).

Oases (arXiv 2305.16121), Section IV: the AllReduce output is y = sum of the
inputs x_i over the w ranks.  On one GPU the w-1 peer inputs are resident
buffers.  This is the sum exactly as the storage-type path defines it:
accumulator = float32(x_0); then accumulator += float32(x_k) for k = 1..w-1,
each add rounded to float32 (plain adds, no fused operations); the result is
rounded to the storage type (float32: unchanged; bf16: round to nearest even
on the float32 bit pattern).  numpy's float32 adds are IEEE round-to-nearest,
so this is exactly reproducible.
"""
from __future__ import annotations

import numpy as np


def _bf16_decode(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_encode_rne(v: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    keep_odd = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + keep_odd) >> np.uint32(16)).astype(np.uint16)


def allreduce_point_storage(own: np.ndarray, peers, is_bf16: bool) -> np.ndarray:
    """own, peers[k]: storage arrays (float32, or uint16 bf16 bit patterns)."""
    dec = _bf16_decode if is_bf16 else (lambda a: a.astype(np.float32))
    acc = dec(own).copy()
    for pk in peers:
        acc = (acc + dec(pk)).astype(np.float32)
    return _bf16_encode_rne(acc) if is_bf16 else acc

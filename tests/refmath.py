"""Independent numpy views of the packed inputs, used to pin the oracle.

Nothing here calls the oracle: these are separate, vectorised readings of the packed
layout (unpack, dequantize) and dense brute-force products, so that a mistake in the
oracle's loops (an index, a dropped term, a transposed operand) shows up as a mismatch.
"""
from __future__ import annotations

import numpy as np


def unpack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """uint32 [E][nb][rows][bits] -> int64 codes [E][rows][nb*32] (column order)."""
    E, nb, rows, nw = codes.shape
    assert nw == bits
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint64) * bits)
    q = (codes.astype(np.uint64)[..., None] >> shifts) & np.uint64((1 << bits) - 1)
    q = q.reshape(E, nb, rows, 32).astype(np.int64)
    return q.transpose(0, 2, 1, 3).reshape(E, rows, nb * 32)


def scales_mins(sm: np.ndarray):
    """uint16 [E][nb][rows][2] -> (scale, min) float64 [E][rows][nb]."""
    h = np.ascontiguousarray(sm).view(np.float16).astype(np.float64)
    return h[..., 0].transpose(0, 2, 1), h[..., 1].transpose(0, 2, 1)


def dequant(codes: np.ndarray, sm: np.ndarray, bits: int) -> np.ndarray:
    """Dense float64 weights [E][rows][cols] = scale*q + min per 32-column block."""
    q = unpack_codes(codes, bits).astype(np.float64)
    s, m = scales_mins(sm)
    return q * np.repeat(s, 32, axis=2) + np.repeat(m, 32, axis=2)


def dequant_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """int8 codes [..., L] with block scales [..., L/32] -> float64 values."""
    return q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=-1)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

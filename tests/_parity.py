"""Shared helpers for comparing librope results with the CPU oracle.

Tolerances (stated once, used by every parity test):
  - float32 outputs: |gpu - oracle| <= 2e-6 on every element;
  - float16 / bfloat16 outputs: at most 1 unit apart in the monotone integer
    order of the 16-bit patterns (+0 and -0 are the same point), i.e. the
    GPU value is the oracle's or one of its two neighbours;
  - dims >= R and tokens whose index is < 0 or >= table_rows: bit-exact with
    the input (and hence with the oracle, which copies them).
The 1-unit allowance covers the one extra rounding of the float32 pipeline
(exact value -> float32 -> 16 bits) against the oracle's single rounding of
the binary64 value; the float32 bound is about 4 ulps at |y| ~ 4.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

import oracle as orc
import workloads as W

F32_ATOL = 2e-6
ORD_TOL = 1


def storage(t: torch.Tensor) -> np.ndarray:
    return orc.torch_to_storage(t)


def ord16(bits: np.ndarray) -> np.ndarray:
    """Monotone integer order of 16-bit float patterns (+0 == -0)."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def oracle_rope(w: W.Workload, x: torch.Tensor, direction: int,
                pos: Optional[torch.Tensor], pos_batch_stride: Optional[int] = None,
                table_rows: Optional[int] = None,
                interpolate_factor: float = 1.0) -> np.ndarray:
    return orc.rope(storage(x), w.dtype, layout=w.layout, pairing=w.pairing,
                    direction=direction, rotary_dim=w.rotary_dim, theta=w.theta,
                    pos=None if pos is None else pos.numpy(),
                    pos_batch_stride=w.pos_batch_stride if pos_batch_stride is None
                    else pos_batch_stride,
                    table_rows=w.table_rows if table_rows is None else table_rows,
                    interpolate_factor=interpolate_factor)


def masked_tokens(w: W.Workload, pos: Optional[torch.Tensor], table_rows=None,
                  pos_batch_stride=None) -> np.ndarray:
    """[B, S] bool: tokens that pass through unchanged."""
    rows = w.table_rows if table_rows is None else table_rows
    if pos is None:
        return np.zeros((w.batch, w.seq_len), bool)
    bs = w.pos_batch_stride if pos_batch_stride is None else pos_batch_stride
    p = pos.numpy().astype(np.int64)
    idx = np.arange(w.batch)[:, None] * bs + np.arange(w.seq_len)[None, :]
    pv = p[idx]
    return (pv < 0) | (pv >= rows)


def _token_axis(layout):
    return 2 if layout == "bhsd" else 1


def assert_parity(got: np.ndarray, ref: np.ndarray, inp: np.ndarray, dtype: str,
                  layout: str, rotary_dim: int, masked: Optional[np.ndarray] = None,
                  what: str = "") -> dict:
    """GPU (or emulated) storage array vs oracle storage array; returns stats."""
    assert got.shape == ref.shape == inp.shape, (got.shape, ref.shape, inp.shape)
    R = rotary_dim
    gb = got.view(np.uint32) if dtype == "f32" else got
    ib = inp.view(np.uint32) if dtype == "f32" else inp
    # pass-through dims: bit-exact
    assert np.array_equal(gb[..., R:], ib[..., R:]), f"{what}: dims >= R changed"
    if masked is not None and masked.any():
        ax = _token_axis(layout)
        m = masked[:, None, :] if ax == 2 else masked[:, :, None]
        m = np.broadcast_to(m, got.shape[:3])
        assert np.array_equal(gb[m], ib[m]), f"{what}: masked tokens changed"
    stats = {}
    if dtype == "f32":
        diff = np.abs(got[..., :R].astype(np.float64) - ref[..., :R].astype(np.float64))
        mx = float(diff.max()) if diff.size else 0.0
        stats = {"max_abs": mx, "n": int(diff.size)}
        assert mx <= F32_ATOL, f"{what}: max |diff| {mx:.3g} > {F32_ATOL}"
    else:
        d = np.abs(ord16(got[..., :R]) - ord16(ref[..., :R]))
        mx = int(d.max()) if d.size else 0
        stats = {"max_ord": mx, "n_off_by_one": int((d == 1).sum()), "n": int(d.size)}
        assert mx <= ORD_TOL, f"{what}: max ord distance {mx} > {ORD_TOL}"
    return stats

"""CPU oracle for rotary position embedding -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never loads it and shares no code with
it; the two meet only in the seeded inputs of `workloads`.

The arithmetic lives in `rope_oracle.c` (plain scalar binary64 loops, compiled
with gcc by `build()`); this module only moves numpy arrays in and out. See
the C file's header for what is computed and which passage of the pages each
step follows.

Parity status: every function here is pinned by tests/test_oracle_pins.py
against closed forms, invariants of rotations, brute force and exact rational
arithmetic; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rope_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Codes of the oracle's own C interface.
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
LAYOUTS = {"bhsd": 0, "bshd": 1}
PAIRINGS = {"split_half": 0, "interleaved": 1}
NP_STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}

_lib = None


def build(out: str = _LIB, src: str = _SRC, extra=()) -> str:
    """Compile the oracle into a shared object with gcc (no contraction, no fast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", *extra, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_I64 = ctypes.c_int64
_P = ctypes.c_void_p


def _bind(lib):
    lib.oracle_freq.restype = ctypes.c_double
    lib.oracle_freq.argtypes = [ctypes.c_double, _I64, _I64]
    lib.oracle_table.restype = None
    lib.oracle_table.argtypes = [ctypes.c_double, ctypes.c_double, _I64, _I64, _P, _P]
    lib.oracle_rope.restype = ctypes.c_int
    lib.oracle_rope.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, _I64, _I64, _I64, _I64, _I64,
                                ctypes.c_double, ctypes.c_double, _P, _I64, _I64]
    lib.oracle_rope_exact.restype = ctypes.c_int
    lib.oracle_rope_exact.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _I64, _I64, _I64, _I64, _I64, ctypes.c_double,
                                      ctypes.c_double, _P, _I64, _I64]
    lib.oracle_rope_attention.restype = ctypes.c_int
    lib.oracle_rope_attention.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                          _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                          ctypes.c_double, ctypes.c_double, _P, _I64, _P, _I64,
                                          _I64, ctypes.c_int, ctypes.c_double]
    lib.oracle_xpos_zeta.restype = ctypes.c_double
    lib.oracle_xpos_zeta.argtypes = [ctypes.c_double, _I64, _I64]
    lib.oracle_xpos_table.restype = None
    lib.oracle_xpos_table.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, _I64,
                                      _I64, _P, _P]
    xpos_args = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                 _I64, _I64, _I64, _I64, _I64, ctypes.c_double, ctypes.c_double, _P, _I64,
                 _I64, ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.oracle_rope_xpos.restype = ctypes.c_int
    lib.oracle_rope_xpos.argtypes = [_P, _P, ctypes.c_int] + xpos_args
    lib.oracle_rope_xpos_exact.restype = ctypes.c_int
    lib.oracle_rope_xpos_exact.argtypes = [_P, _P] + xpos_args
    lib.oracle_to_bf16_bits.restype = ctypes.c_uint16
    lib.oracle_to_bf16_bits.argtypes = [ctypes.c_double]
    lib.oracle_to_f16_bits.restype = ctypes.c_uint16
    lib.oracle_to_f16_bits.argtypes = [ctypes.c_double]
    lib.oracle_from_bits.restype = ctypes.c_double
    lib.oracle_from_bits.argtypes = [ctypes.c_uint32, ctypes.c_int]
    return lib


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library; cached for the default path."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None and os.environ.get("ROPE_ORACLE_LIB"):
        # a deliberately altered oracle built by the mutation tests
        _lib = _bind(ctypes.CDLL(os.environ["ROPE_ORACLE_LIB"]))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _dims(shape, layout):
    if len(shape) != 4:
        raise ValueError("expected a 4-d tensor")
    if layout == "bhsd":
        B, H, S, D = shape
    else:
        B, S, H, D = shape
    return B, H, S, D


def _pos_arr(pos):
    if pos is None:
        return None
    return np.ascontiguousarray(np.asarray(pos, dtype=np.int32))


def freq(theta: float, rotary_dim: int, i: int, lib=None) -> float:
    """freq_i = theta^(-2i/R) in binary64."""
    return (lib or load()).oracle_freq(theta, rotary_dim, i)


def table(theta: float, rotary_dim: int, rows: int, interpolate_factor: float = 1.0,
          lib=None):
    """The oracle's own fp32 cos/sin tables, each [rows, R/2]: row p holds
    cos/sin of (p / interpolate_factor) * freq_i."""
    half = rotary_dim // 2
    c = np.empty((rows, half), np.float32)
    s = np.empty((rows, half), np.float32)
    (lib or load()).oracle_table(theta, interpolate_factor, rotary_dim, rows, _ptr(c), _ptr(s))
    return c, s


def rope(x: np.ndarray, dtype: str, *, layout: str = "bhsd", pairing: str = "split_half",
         direction: int = 1, rotary_dim: Optional[int] = None, theta: float = 10000.0,
         pos=None, pos_batch_stride: int = 0, table_rows: Optional[int] = None,
         interpolate_factor: float = 1.0, lib=None) -> np.ndarray:
    """Table-mode RoPE of storage array `x` (float32, or uint16 bits for f16/bf16).

    Positions are divided by `interpolate_factor` before the angle is formed.
    Returns a new array of the same storage type and shape.
    """
    x = np.ascontiguousarray(x, dtype=NP_STORAGE[dtype])
    B, H, S, D = _dims(x.shape, layout)
    R = D if rotary_dim is None else rotary_dim
    rows = S if table_rows is None else table_rows
    p = _pos_arr(pos)
    y = np.empty_like(x)
    rc = (lib or load()).oracle_rope(_ptr(x), _ptr(y), DTYPES[dtype], LAYOUTS[layout],
                                     PAIRINGS[pairing], direction, B, H, S, D, R, theta,
                                     interpolate_factor, _ptr(p), pos_batch_stride, rows)
    if rc:
        raise OracleError(f"oracle_rope rejected its arguments (code {rc})")
    return y


def rope_exact(x: np.ndarray, *, layout: str = "bhsd", pairing: str = "split_half",
               direction: int = 1, rotary_dim: Optional[int] = None,
               theta: float = 10000.0, pos=None, pos_batch_stride: int = 0,
               table_rows: Optional[int] = None, interpolate_factor: float = 1.0,
               lib=None) -> np.ndarray:
    """Exact-mode RoPE in binary64 (unrounded cos/sin), for invariant checks."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    B, H, S, D = _dims(x.shape, layout)
    R = D if rotary_dim is None else rotary_dim
    rows = S if table_rows is None else table_rows
    p = _pos_arr(pos)
    y = np.empty_like(x)
    rc = (lib or load()).oracle_rope_exact(_ptr(x), _ptr(y), LAYOUTS[layout],
                                           PAIRINGS[pairing], direction, B, H, S, D, R,
                                           theta, interpolate_factor, _ptr(p),
                                           pos_batch_stride, rows)
    if rc:
        raise OracleError(f"oracle_rope_exact rejected its arguments (code {rc})")
    return y


def xpos_zeta(gamma: float, rotary_dim: int, i: int, lib=None) -> float:
    """zeta_i = (i / (R/2) + gamma) / (1 + gamma) in binary64 (xPos)."""
    return (lib or load()).oracle_xpos_zeta(gamma, rotary_dim, i)


def xpos_table(rotary_dim: int, rows: int, scale_base: float = 512.0, gamma: float = 0.4,
               center: float = 0.0, lib=None):
    """The oracle's own fp32 XPOS factor tables (query, key), each [rows, R/2]:
    row p holds zeta_i^((p - center)/B) and its reciprocal power."""
    half = rotary_dim // 2
    zq = np.empty((rows, half), np.float32)
    zk = np.empty((rows, half), np.float32)
    (lib or load()).oracle_xpos_table(scale_base, gamma, center, rotary_dim, rows, _ptr(zq),
                                      _ptr(zk))
    return zq, zk


def rope_xpos(x: np.ndarray, dtype: str, *, is_key: bool, layout: str = "bhsd",
              pairing: str = "split_half", direction: int = 1,
              rotary_dim: Optional[int] = None, theta: float = 10000.0, pos=None,
              pos_batch_stride: int = 0, table_rows: Optional[int] = None,
              interpolate_factor: float = 1.0, scale_base: float = 512.0, gamma: float = 0.4,
              center: float = 0.0, lib=None) -> np.ndarray:
    """Table-mode RoPE with XPOS factors (query rows, or key rows when
    is_key) of storage array `x`. Returns a new array."""
    x = np.ascontiguousarray(x, dtype=NP_STORAGE[dtype])
    B, H, S, D = _dims(x.shape, layout)
    R = D if rotary_dim is None else rotary_dim
    rows = S if table_rows is None else table_rows
    p = _pos_arr(pos)
    y = np.empty_like(x)
    rc = (lib or load()).oracle_rope_xpos(_ptr(x), _ptr(y), DTYPES[dtype], LAYOUTS[layout],
                                          PAIRINGS[pairing], direction, int(is_key), B, H, S,
                                          D, R, theta, interpolate_factor, _ptr(p),
                                          pos_batch_stride, rows, scale_base, gamma, center)
    if rc:
        raise OracleError(f"oracle_rope_xpos rejected its arguments (code {rc})")
    return y


def rope_xpos_exact(x: np.ndarray, *, is_key: bool, layout: str = "bhsd",
                    pairing: str = "split_half", direction: int = 1,
                    rotary_dim: Optional[int] = None, theta: float = 10000.0, pos=None,
                    pos_batch_stride: int = 0, table_rows: Optional[int] = None,
                    interpolate_factor: float = 1.0, scale_base: float = 512.0,
                    gamma: float = 0.4, center: float = 0.0, lib=None) -> np.ndarray:
    """Exact-mode RoPE with XPOS factors in binary64, for invariant checks."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    B, H, S, D = _dims(x.shape, layout)
    R = D if rotary_dim is None else rotary_dim
    rows = S if table_rows is None else table_rows
    p = _pos_arr(pos)
    y = np.empty_like(x)
    rc = (lib or load()).oracle_rope_xpos_exact(_ptr(x), _ptr(y), LAYOUTS[layout],
                                                PAIRINGS[pairing], direction, int(is_key), B,
                                                H, S, D, R, theta, interpolate_factor,
                                                _ptr(p), pos_batch_stride, rows, scale_base,
                                                gamma, center)
    if rc:
        raise OracleError(f"oracle_rope_xpos_exact rejected its arguments (code {rc})")
    return y


def rope_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: str, *,
                   pairing: str = "split_half", rotary_dim: Optional[int] = None,
                   theta: float = 10000.0, interpolate_factor: float = 1.0, qpos=None,
                   qpos_batch_stride: int = 0, kpos=None, kpos_batch_stride: int = 0,
                   table_rows: Optional[int] = None, causal: bool = False,
                   scale: Optional[float] = None, lib=None) -> np.ndarray:
    """Attention over RoPE-rotated Q and K (see rope_oracle.c), binary64 output.

    q [B,Hq,Sq,D], k and v [B,Hk,Sk,D] storage arrays (float32, or uint16 bits
    for f16/bf16). scale defaults to 1/sqrt(D); positions default to s for
    keys and s + Sk - Sq for queries.
    """
    st = NP_STORAGE[dtype]
    q, k, v = (np.ascontiguousarray(a, dtype=st) for a in (q, k, v))
    B, Hq, Sq, D = q.shape
    _, Hk, Sk, _ = k.shape
    R = D if rotary_dim is None else rotary_dim
    rows = max(Sq, Sk) if table_rows is None else table_rows
    sc = 1.0 / np.sqrt(D) if scale is None else scale
    o = np.empty((B, Hq, Sq, D), np.float64)
    qp, kp = _pos_arr(qpos), _pos_arr(kpos)
    rc = (lib or load()).oracle_rope_attention(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), DTYPES[dtype], PAIRINGS[pairing], B, Hq, Hk, Sq,
        Sk, D, R, theta, interpolate_factor, _ptr(qp), qpos_batch_stride, _ptr(kp),
        kpos_batch_stride, rows, int(causal), float(sc))
    if rc:
        raise OracleError(f"oracle_rope_attention rejected its arguments (code {rc})")
    return o


def to_bits(y: float, dtype: str, lib=None) -> int:
    lib = lib or load()
    if dtype == "bf16":
        return int(lib.oracle_to_bf16_bits(y))
    if dtype == "f16":
        return int(lib.oracle_to_f16_bits(y))
    raise ValueError(dtype)


def from_bits(bits: int, dtype: str, lib=None) -> float:
    return float((lib or load()).oracle_from_bits(bits, DTYPES[dtype]))


def torch_to_storage(t) -> np.ndarray:
    """CPU torch tensor -> numpy storage array (float32, or uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)

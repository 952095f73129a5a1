"""Python binding of librope (fused RoPE for MI355X): argument marshalling only.

Each function below has the name of a C entry point in include/librope.h,
builds its rope_desc_t from torch tensors (shapes, dtype, data pointers and
the current HIP stream) and calls it. No arithmetic of the method happens
here, and there is no fallback: if librope.so is not built, or a call is
rejected, this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librope.so")

ROPE_OK = 0
STATUS_NAMES = {0: "ROPE_OK", -1: "ROPE_ERR_NULL", -2: "ROPE_ERR_SHAPE",
                -3: "ROPE_ERR_DTYPE", -4: "ROPE_ERR_LAYOUT", -5: "ROPE_ERR_ALIGN",
                -6: "ROPE_ERR_ALIAS", -7: "ROPE_ERR_HIP"}
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
LAYOUTS = {"bhsd": 0, "bshd": 1}
PAIRINGS = {"split_half": 0, "interleaved": 1}
LAUNCHES = {"auto": 0, "rows": 1, "token": 2}


class RopeDesc(ctypes.Structure):
    """rope_desc_t of include/librope.h."""
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("n_heads_q", ctypes.c_int64),
        ("n_heads_k", ctypes.c_int64),
        ("seq_len", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("rotary_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("pairing", ctypes.c_int32),
        ("launch", ctypes.c_int32),
        ("cos", ctypes.c_void_p),
        ("sin", ctypes.c_void_p),
        ("table_rows", ctypes.c_int64),
        ("pos", ctypes.c_void_p),
        ("pos_batch_stride", ctypes.c_int64),
    ]


class RopeView(ctypes.Structure):
    """rope_view_t: data pointer and element strides of the batch, head and
    sequence dims (the head_dim axis is contiguous)."""
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_s", ctypes.c_int64)]


class RopeApplyDesc(ctypes.Structure):
    """rope_apply_desc_t of include/librope.h."""
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seq_len", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("rotary_dim", ctypes.c_int64),
        ("n_heads_q", ctypes.c_int64),
        ("n_heads_k", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("pairing", ctypes.c_int32),
        ("launch", ctypes.c_int32),
        ("direction", ctypes.c_int32),
        ("q_in", RopeView),
        ("k_in", RopeView),
        ("q_out", RopeView),
        ("k_out", RopeView),
        ("cos", ctypes.c_void_p),
        ("sin", ctypes.c_void_p),
        ("table_rows", ctypes.c_int64),
        ("table_row_stride", ctypes.c_int64),
        ("table_col_stride", ctypes.c_int64),
        ("pos", ctypes.c_void_p),
        ("pos_batch_stride", ctypes.c_int64),
        ("theta", ctypes.c_double),
        ("interpolate_factor", ctypes.c_double),
        ("angles", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


ANGLES_TABLE, ANGLES_THETA = 0, 1


class RopeAttnDesc(ctypes.Structure):
    """rope_attn_desc_t of include/librope.h."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("n_heads_q", ctypes.c_int64),
        ("n_heads_k", ctypes.c_int64), ("seq_len_q", ctypes.c_int64),
        ("seq_len_k", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("rotary_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("pairing", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("rotate", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p),
        ("table_rows", ctypes.c_int64),
        ("q_pos", ctypes.c_void_p), ("q_pos_batch_stride", ctypes.c_int64),
        ("k_pos", ctypes.c_void_p), ("k_pos_batch_stride", ctypes.c_int64),
        ("scale", ctypes.c_double),
        ("k_rotated", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class RopeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({status_string(status)})")


_lib = None


def lib():
    """The loaded librope.so with argument types set. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"librope.so is not built ({LIB_PATH}); run "
                              "`python -m rotary_position_embedding_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, D = ctypes.c_void_p, ctypes.POINTER(RopeDesc)
        for name in ("rope_fwd_qk", "rope_bwd_qk"):
            getattr(L, name).argtypes = [P, P, D, P]
            getattr(L, name).restype = ctypes.c_int
        for name in ("rope_fwd_q", "rope_bwd_q"):
            getattr(L, name).argtypes = [P, D, P]
            getattr(L, name).restype = ctypes.c_int
        L.rope_apply.argtypes = [ctypes.POINTER(RopeApplyDesc), P]
        L.rope_apply.restype = ctypes.c_int
        L.rope_build_table.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                       ctypes.c_double]
        L.rope_build_table.restype = ctypes.c_int
        L.rope_apply_xpos.argtypes = [ctypes.POINTER(RopeApplyDesc), P, P, P]
        L.rope_apply_xpos.restype = ctypes.c_int
        L.rope_build_xpos_table.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_double, ctypes.c_double, ctypes.c_double]
        L.rope_build_xpos_table.restype = ctypes.c_int
        L.rope_attention_fwd.argtypes = [ctypes.POINTER(RopeAttnDesc), P]
        L.rope_attention_fwd_k_once.argtypes = [ctypes.POINTER(RopeAttnDesc), P, P]
        L.rope_attention_fwd_k_once.restype = ctypes.c_int
        L.rope_attention_fwd_k_once_noalloc.argtypes = [ctypes.POINTER(RopeAttnDesc), P]
        L.rope_attention_fwd_k_once_noalloc.restype = ctypes.c_int
        L.rope_attention_fwd.restype = ctypes.c_int
        L.rope_describe.argtypes = [P, P, D, ctypes.c_int, ctypes.c_char_p, ctypes.c_int64]
        L.rope_describe.restype = ctypes.c_int
        L.rope_status_string.argtypes = [ctypes.c_int]
        L.rope_status_string.restype = ctypes.c_char_p
        L.rope_version.argtypes = []
        L.rope_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().rope_status_string(status).decode()


def rope_status_string(status: int) -> str:
    return status_string(status)


def rope_version() -> int:
    return int(lib().rope_version())


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _dims(t, layout: str):
    if t.dim() != 4:
        raise ValueError("q/k must be 4-d")
    if layout == "bhsd":
        B, H, S, D = t.shape
    else:
        B, S, H, D = t.shape
    return B, H, S, D


def make_desc(q, k, cos, sin, *, layout: str = "bhsd", pairing: str = "split_half",
              rotary_dim: Optional[int] = None, pos=None,
              pos_batch_stride: Optional[int] = None, launch: str = "auto") -> RopeDesc:
    """rope_desc_t for torch tensors q (and k, or None) and device tables cos/sin."""
    B, Hq, S, D = _dims(q, layout)
    Hk = 0
    if k is not None:
        Bk, Hk, Sk, Dk = _dims(k, layout)
        if (Bk, Sk, Dk) != (B, S, D) or k.dtype != q.dtype:
            raise ValueError("k must match q in batch, seq_len, head_dim and dtype")
    for name, t in (("q", q), ("k", k)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (it is rotated in place)")
    R = D if rotary_dim is None else int(rotary_dim)
    if cos.dtype != sin.dtype or cos.shape != sin.shape or cos.dim() != 2:
        raise ValueError("cos and sin must be matching 2-d float32 tables")
    import torch
    if cos.dtype != torch.float32 or not cos.is_contiguous() or not sin.is_contiguous():
        raise ValueError("cos and sin must be contiguous float32 [table_rows, R/2]")
    if cos.shape[1] != R // 2:
        raise ValueError(f"tables have {cos.shape[1]} columns, expected R/2 = {R // 2}")
    d = RopeDesc()
    d.batch, d.n_heads_q, d.n_heads_k, d.seq_len, d.head_dim = B, Hq, Hk, S, D
    d.rotary_dim = R
    d.dtype = _dtype_code(q)
    d.layout = LAYOUTS[layout]
    d.pairing = PAIRINGS[pairing]
    d.launch = LAUNCHES[launch]
    d.cos, d.sin = cos.data_ptr(), sin.data_ptr()
    d.table_rows = cos.shape[0]
    if pos is not None:
        if pos.dtype != torch.int32 or not pos.is_contiguous():
            raise ValueError("pos must be a contiguous int32 tensor")
        if pos_batch_stride is None:
            if pos.dim() == 2:
                pos_batch_stride = pos.stride(0)
            elif pos.numel() == S:
                pos_batch_stride = 0
            elif pos.numel() == B * S:
                pos_batch_stride = S
            else:
                raise ValueError("pos must hold seq_len or batch*seq_len indices")
        need = (B - 1) * pos_batch_stride + S if B > 0 and S > 0 else 0
        if pos.numel() < need:
            raise ValueError(f"pos holds {pos.numel()} indices, needs {need}")
        d.pos = pos.data_ptr()
        d.pos_batch_stride = pos_batch_stride
    return d


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != ROPE_OK:
        raise RopeError(status, where)


def _on_one_device(where: str, *tensors):
    """Every tensor a call hands to librope must be GPU memory of one device:
    the library cannot tell a host pointer from a device pointer without
    touching the GPU, and a kernel that dereferences a host pointer faults.
    None entries (absent optional operands) are skipped."""
    ts = [t for t in tensors if t is not None]
    if not ts:
        return
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError(f"{where}: every tensor must be on the GPU, got one on {t.device}")
        if t.device != dev:
            raise ValueError(f"{where}: tensors on {dev} and {t.device}; use one device")


def rope_fwd_qk(q, k, cos, sin, *, stream=None, **kw):
    """Forward RoPE on q and k in place (one launch). See make_desc for options."""
    _on_one_device("rope_fwd_qk", q, k, cos, sin, kw.get("pos"))
    d = make_desc(q, k, cos, sin, **kw)
    _check(lib().rope_fwd_qk(q.data_ptr(), k.data_ptr(), ctypes.byref(d), _stream(stream)),
           "rope_fwd_qk")
    return q, k


def rope_bwd_qk(dq, dk, cos, sin, *, stream=None, **kw):
    """Backward RoPE on gradients dq and dk in place."""
    _on_one_device("rope_bwd_qk", dq, dk, cos, sin, kw.get("pos"))
    d = make_desc(dq, dk, cos, sin, **kw)
    _check(lib().rope_bwd_qk(dq.data_ptr(), dk.data_ptr(), ctypes.byref(d), _stream(stream)),
           "rope_bwd_qk")
    return dq, dk


def rope_fwd_q(q, cos, sin, *, stream=None, **kw):
    """Forward RoPE on q only, in place."""
    _on_one_device("rope_fwd_q", q, cos, sin, kw.get("pos"))
    d = make_desc(q, None, cos, sin, **kw)
    _check(lib().rope_fwd_q(q.data_ptr(), ctypes.byref(d), _stream(stream)), "rope_fwd_q")
    return q


def rope_bwd_q(dq, cos, sin, *, stream=None, **kw):
    """Backward RoPE on dq only, in place."""
    _on_one_device("rope_bwd_q", dq, cos, sin, kw.get("pos"))
    d = make_desc(dq, None, cos, sin, **kw)
    _check(lib().rope_bwd_q(dq.data_ptr(), ctypes.byref(d), _stream(stream)), "rope_bwd_q")
    return dq


def rope_describe(q, k, cos, sin, **kw) -> str:
    """The kernel and grid rope_fwd_qk(q, k, ...) (or rope_fwd_q when k is
    None) would launch on the current device; nothing is enqueued."""
    _on_one_device("rope_describe", q, k, cos, sin, kw.get("pos"))
    d = make_desc(q, k, cos, sin, **kw)
    buf = ctypes.create_string_buffer(512)
    _check(lib().rope_describe(q.data_ptr(), None if k is None else k.data_ptr(),
                               ctypes.byref(d), int(k is not None), buf, len(buf)),
           "rope_describe")
    return buf.value.decode()


TABLE_LAYOUTS = ("half", "duplicated", "interleaved")


def _view(t, layout: str) -> RopeView:
    """RopeView of a 4-d torch tensor in `layout` order with a contiguous last dim."""
    if t.dim() != 4:
        raise ValueError("q/k views must be 4-d")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the head_dim axis must be contiguous (stride 1)")
    if layout == "bhsd":
        sb, sh, ss = t.stride(0), t.stride(1), t.stride(2)
    else:
        sb, ss, sh = t.stride(0), t.stride(1), t.stride(2)
    return RopeView(t.data_ptr(), sb, sh, ss)


def make_apply_desc(q, k, cos, sin, *, q_out=None, k_out=None, direction: int = 1,
                    layout: str = "bhsd", pairing: str = "split_half",
                    rotary_dim: Optional[int] = None, pos=None,
                    pos_batch_stride: Optional[int] = None, launch: str = "auto",
                    table_layout: str = "half", theta: Optional[float] = None,
                    interpolate_factor: float = 1.0,
                    max_positions: Optional[int] = None) -> RopeApplyDesc:
    """rope_apply_desc_t for (possibly strided) torch views q, k (k may be None)
    and optional outputs q_out, k_out of the same shapes.

    table_layout: "half" = [rows, R/2]; "duplicated" = [rows, R] holding
    cat(f, f); "interleaved" = [rows, R] holding each value twice in a row.
    The table's row stride is taken from the tensor, so row-sliced views work.

    theta: compute cos/sin in the kernel from theta and interpolate_factor
    instead of reading tables (cos and sin must then be None);
    max_positions bounds the positions as table_rows does (default: seq_len
    without an index, else 2^31 - 1).
    """
    B, Hq, S, D = _dims(q, layout)
    Hk = 0
    if k is not None:
        Bk, Hk, Sk, Dk = _dims(k, layout)
        if (Bk, Sk, Dk) != (B, S, D) or k.dtype != q.dtype:
            raise ValueError("k must match q in batch, seq_len, head_dim and dtype")
    for name, o, x in (("q_out", q_out, q), ("k_out", k_out, k)):
        if o is not None and (x is None or o.shape != x.shape or o.dtype != x.dtype):
            raise ValueError(f"{name} must match its input's shape and dtype")
    R = D if rotary_dim is None else int(rotary_dim)
    import torch
    if theta is not None:
        if cos is not None or sin is not None:
            raise ValueError("pass either cos/sin tables or theta, not both")
    else:
        if cos is None or sin is None:
            raise ValueError("cos and sin tables are required unless theta is given")
        if cos.dtype != torch.float32 or sin.dtype != torch.float32 or cos.shape != sin.shape:
            raise ValueError("cos and sin must be matching float32 tables")
        if (cos.dim() != 2 or cos.stride(1) != 1 or sin.stride(1) != 1 or
                cos.stride(0) != sin.stride(0)):
            raise ValueError("cos/sin must be 2-d with contiguous rows and equal strides")
        if table_layout not in TABLE_LAYOUTS:
            raise ValueError(f"table_layout must be one of {TABLE_LAYOUTS}")
        want = R // 2 if table_layout == "half" else R
        if cos.shape[1] != want:
            raise ValueError(f"a {table_layout!r} table has {want} columns, got {cos.shape[1]}")
    d = RopeApplyDesc()
    d.batch, d.seq_len, d.head_dim, d.rotary_dim = B, S, D, R
    d.n_heads_q, d.n_heads_k = Hq, Hk
    d.dtype = _dtype_code(q)
    d.pairing = PAIRINGS[pairing]
    d.launch = LAUNCHES[launch]
    d.direction = int(direction)
    d.q_in = _view(q, layout)
    if k is not None:
        d.k_in = _view(k, layout)
    if q_out is not None:
        d.q_out = _view(q_out, layout)
    if k_out is not None:
        d.k_out = _view(k_out, layout)
    if theta is not None:
        d.angles = ANGLES_THETA
        d.theta, d.interpolate_factor = float(theta), float(interpolate_factor)
        if max_positions is None:
            max_positions = S if pos is None else 2 ** 31 - 1
        d.table_rows = int(max_positions)
        d.table_col_stride = 1
    else:
        d.cos, d.sin = cos.data_ptr(), sin.data_ptr()
        d.table_rows = cos.shape[0]
        d.table_row_stride = cos.stride(0)
        d.table_col_stride = 2 if table_layout == "interleaved" else 1
    if pos is not None:
        if pos.dtype != torch.int32 or not pos.is_contiguous():
            raise ValueError("pos must be a contiguous int32 tensor")
        if pos_batch_stride is None:
            if pos.dim() == 2:
                pos_batch_stride = pos.stride(0)
            elif pos.numel() == S:
                pos_batch_stride = 0
            elif pos.numel() == B * S:
                pos_batch_stride = S
            else:
                raise ValueError("pos must hold seq_len or batch*seq_len indices")
        need = (B - 1) * pos_batch_stride + S if B > 0 and S > 0 else 0
        if pos.numel() < need:
            raise ValueError(f"pos holds {pos.numel()} indices, needs {need}")
        d.pos = pos.data_ptr()
        d.pos_batch_stride = pos_batch_stride
    return d


def rope_apply(q, k, cos, sin, *, stream=None, **kw):
    """General call: strided views, optional outputs (q_out, k_out), direction
    +1/-1, table layouts. Returns the tensors that hold the result."""
    _on_one_device("rope_apply", q, k, cos, sin, kw.get("pos"), kw.get("q_out"), kw.get("k_out"))
    d = make_apply_desc(q, k, cos, sin, **kw)
    _check(lib().rope_apply(ctypes.byref(d), _stream(stream)), "rope_apply")
    qo = kw.get("q_out")
    ko = kw.get("k_out")
    return (q if qo is None else qo), (k if ko is None else ko)


def _xpos_ptrs(xpos_q, xpos_k, cos):
    import torch
    out = []
    for name, z in (("xpos_q", xpos_q), ("xpos_k", xpos_k)):
        if z is None:
            out.append(None)
            continue
        if z.dtype != torch.float32 or z.shape != cos.shape or z.stride() != cos.stride():
            raise ValueError(f"{name} must be a float32 table laid out like cos")
        out.append(z.data_ptr())
    return out


def rope_apply_xpos(q, k, cos, sin, xpos_q, xpos_k, *, stream=None, **kw):
    """rope_apply with XPOS factors: after the rotation, pair i of a query row
    at position p is multiplied by xpos_q[p, i], of a key row by xpos_k[p, i]
    (tables laid out like cos and sin, e.g. from rope_build_xpos_table).
    Same keywords as rope_apply, tables only (no theta). Returns the tensors
    that hold the result."""
    if kw.get("theta") is not None:
        raise ValueError("XPOS factors come with cos/sin tables, not theta")
    _on_one_device("rope_apply_xpos", q, k, cos, sin, xpos_q, xpos_k, kw.get("pos"),
                   kw.get("q_out"), kw.get("k_out"))
    d = make_apply_desc(q, k, cos, sin, **kw)
    zq, zk = _xpos_ptrs(xpos_q, xpos_k, cos)
    _check(lib().rope_apply_xpos(ctypes.byref(d), zq, zk, _stream(stream)), "rope_apply_xpos")
    qo = kw.get("q_out")
    ko = kw.get("k_out")
    return (q if qo is None else qo), (k if ko is None else ko)


class Prepared:
    """A call whose descriptor is built once: for loops that issue the same
    rotation many times (benchmarks, decode steps). Holds the tensors alive;
    each method only forwards cached pointers to the C entry point."""

    def __init__(self, q, k, cos, sin, stream=None, **kw):
        self._keep = (q, k, cos, sin, kw.get("pos"))
        _on_one_device("prepare", q, k, cos, sin, kw.get("pos"))
        self.desc = make_desc(q, k, cos, sin, **kw)
        self._q = q.data_ptr()
        self._k = k.data_ptr() if k is not None else None
        self._stream = _stream(stream)
        self._pdesc = ctypes.byref(self.desc)
        self._lib = lib()

    def rope_fwd_qk(self):
        _check(self._lib.rope_fwd_qk(self._q, self._k, self._pdesc, self._stream), "rope_fwd_qk")

    def rope_bwd_qk(self):
        _check(self._lib.rope_bwd_qk(self._q, self._k, self._pdesc, self._stream), "rope_bwd_qk")

    def rope_fwd_q(self):
        _check(self._lib.rope_fwd_q(self._q, self._pdesc, self._stream), "rope_fwd_q")

    def rope_bwd_q(self):
        _check(self._lib.rope_bwd_q(self._q, self._pdesc, self._stream), "rope_bwd_q")


class PreparedApplyXpos:
    """A rope_apply_xpos call whose descriptor is built once (see Prepared)."""

    def __init__(self, q, k, cos, sin, xpos_q, xpos_k, stream=None, **kw):
        self._keep = (q, k, cos, sin, xpos_q, xpos_k, kw.get("pos"), kw.get("q_out"),
                      kw.get("k_out"))
        if kw.get("theta") is not None:
            raise ValueError("XPOS factors come with cos/sin tables, not theta")
        _on_one_device("prepare_apply_xpos", q, k, cos, sin, xpos_q, xpos_k, kw.get("pos"),
                       kw.get("q_out"), kw.get("k_out"))
        self.desc = make_apply_desc(q, k, cos, sin, **kw)
        self._zq, self._zk = _xpos_ptrs(xpos_q, xpos_k, cos)
        self._stream = _stream(stream)
        self._pdesc = ctypes.byref(self.desc)
        self._lib = lib()

    def rope_apply_xpos(self):
        _check(self._lib.rope_apply_xpos(self._pdesc, self._zq, self._zk, self._stream),
               "rope_apply_xpos")


def prepare_apply_xpos(q, k, cos, sin, xpos_q, xpos_k, *, stream=None,
                       **kw) -> PreparedApplyXpos:
    """Build the descriptor of a rope_apply_xpos call once."""
    return PreparedApplyXpos(q, k, cos, sin, xpos_q, xpos_k, stream=stream, **kw)


class PreparedApply:
    """A rope_apply call whose descriptor is built once (see Prepared)."""

    def __init__(self, q, k, cos, sin, stream=None, **kw):
        self._keep = (q, k, cos, sin, kw.get("pos"), kw.get("q_out"), kw.get("k_out"))
        _on_one_device("prepare_apply", q, k, cos, sin, kw.get("pos"), kw.get("q_out"),
                       kw.get("k_out"))
        self.desc = make_apply_desc(q, k, cos, sin, **kw)
        self._stream = _stream(stream)
        self._pdesc = ctypes.byref(self.desc)
        self._lib = lib()

    def rope_apply(self):
        _check(self._lib.rope_apply(self._pdesc, self._stream), "rope_apply")


def prepare_apply(q, k, cos, sin, *, stream=None, **kw) -> PreparedApply:
    """Build the descriptor of a rope_apply call once."""
    return PreparedApply(q, k, cos, sin, stream=stream, **kw)


def prepare(q, k, cos, sin, *, stream=None, **kw) -> Prepared:
    """Build the descriptor of a rope_*_qk / rope_*_q call once (see Prepared)."""
    return Prepared(q, k, cos, sin, stream=stream, **kw)


def rope_build_table(table_rows: int, rotary_dim: int, theta: float = 10000.0,
                     interpolate_factor: float = 1.0):
    """Host float32 cos/sin tables [table_rows, R/2] (CPU torch tensors); row p
    holds the angles of position p / interpolate_factor."""
    import torch
    half = rotary_dim // 2
    cos = torch.empty((table_rows, half), dtype=torch.float32)
    sin = torch.empty((table_rows, half), dtype=torch.float32)
    _check(lib().rope_build_table(cos.data_ptr(), sin.data_ptr(), table_rows, rotary_dim,
                                  float(theta), float(interpolate_factor)), "rope_build_table")
    return cos, sin


def rope_build_xpos_table(table_rows: int, rotary_dim: int, scale_base: float = 512.0,
                          gamma: float = 0.4, center: float = 0.0):
    """Host float32 XPOS factor tables (query, key), each [table_rows, R/2]:
    zeta_i^((p - center)/scale_base) and its reciprocal power,
    zeta_i = (2i/R + gamma) / (1 + gamma)."""
    import torch
    half = rotary_dim // 2
    zq = torch.empty((table_rows, half), dtype=torch.float32)
    zk = torch.empty((table_rows, half), dtype=torch.float32)
    _check(lib().rope_build_xpos_table(zq.data_ptr(), zk.data_ptr(), table_rows, rotary_dim,
                                       float(scale_base), float(gamma), float(center)),
           "rope_build_xpos_table")
    return zq, zk


def _index(pos, batch: int, seq: int, batch_stride: Optional[int], what: str):
    """(pointer, batch stride) of an optional int32 index of `seq` entries per batch."""
    if pos is None:
        return None, 0
    import torch
    if pos.dtype != torch.int32 or not pos.is_contiguous():
        raise ValueError(f"{what} must be a contiguous int32 tensor")
    bs = (seq if pos.numel() >= batch * seq else 0) if batch_stride is None else batch_stride
    need = (batch - 1) * bs + seq if batch > 0 and seq > 0 else 0
    if pos.numel() < need:
        raise ValueError(f"{what} holds {pos.numel()} indices, needs {need}")
    return pos.data_ptr(), bs


def make_attn_desc(q, k, v, cos, sin, o, *, pairing: str = "split_half",
                   rotary_dim: Optional[int] = None, causal: bool = False,
                   rotate: bool = True, q_pos=None, k_pos=None,
                   q_pos_batch_stride: Optional[int] = None,
                   k_pos_batch_stride: Optional[int] = None, scale: float = 0.0,
                   k_rotated: bool = False) -> RopeAttnDesc:
    """rope_attn_desc_t for q [B,Hq,Sq,D], k and v [B,Hk,Sk,D], o like q (all
    contiguous bf16). rotary_dim defaults to 2 * cos.shape[1]; positions
    default to key j at j and query i at i + Sk - Sq. An index with at least
    B*S entries is taken per batch (stride S), otherwise shared (stride 0)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d tensor")
    B, Hq, Sq, D = q.shape
    Hk, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hk, Sk, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hk, Sk, D] with q's B and D")
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    d = RopeAttnDesc()
    d.batch, d.n_heads_q, d.n_heads_k = B, Hq, Hk
    d.seq_len_q, d.seq_len_k, d.head_dim = Sq, Sk, D
    d.dtype = _dtype_code(q)
    for t in (k, v, o):
        if _dtype_code(t) != d.dtype:
            raise ValueError("q, k, v and o must share one dtype")
    d.pairing = PAIRINGS[pairing]
    d.causal = int(bool(causal))
    d.rotate = int(bool(rotate))
    d.q, d.k, d.v, d.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    if cos is not None:
        import torch
        if sin is None or cos.dim() != 2 or tuple(sin.shape) != tuple(cos.shape):
            raise ValueError("cos and sin must be [table_rows, R/2]")
        if cos.dtype != torch.float32 or sin.dtype != torch.float32:
            raise ValueError("cos and sin must be float32")
        if not cos.is_contiguous() or not sin.is_contiguous():
            raise ValueError("cos and sin must be contiguous [table_rows, R/2] tables")
        R = 2 * cos.shape[1] if rotary_dim is None else int(rotary_dim)
        if cos.shape[1] != R // 2 or R % 2:
            raise ValueError(f"tables have {cos.shape[1]} columns, rotary_dim {R} needs "
                             f"{R // 2}")
        d.rotary_dim = R
        d.cos, d.sin = cos.data_ptr(), sin.data_ptr()
        d.table_rows = cos.shape[0]
    else:
        d.rotary_dim = 0 if rotary_dim is None else rotary_dim
    d.q_pos, d.q_pos_batch_stride = _index(q_pos, B, Sq, q_pos_batch_stride, "q_pos")
    d.k_pos, d.k_pos_batch_stride = _index(k_pos, B, Sk, k_pos_batch_stride, "k_pos")
    d.scale = float(scale)
    d.k_rotated = int(bool(k_rotated))
    return d


def _k_workspace(k_workspace, k):
    if k_workspace is None:
        return None
    if (k_workspace.dtype != k.dtype or tuple(k_workspace.shape) != tuple(k.shape) or
            not k_workspace.is_contiguous()):
        raise ValueError("k_workspace must be a contiguous tensor like k")
    return k_workspace.data_ptr()


def rope_attention(q, k, v, cos, sin, *, o=None, stream=None, k_workspace=None, **kw):
    """Attention over RoPE-rotated q and k (rope_attention_fwd):
    softmax(scale * rope(q) rope(k)^T [causal]) v, GQA by head groups, in one
    launch, the rotated q and k never written. With k_workspace (a tensor
    like k), rope(k) is written there once and the attention rotates only q
    (rope_attention_fwd_k_once): the same result, faster on long sequences.
    Returns o (allocated if not given)."""
    import torch
    if o is None:
        o = torch.empty_like(q)
    _on_one_device("rope_attention", q, k, v, cos, sin, o, kw.get("q_pos"), kw.get("k_pos"),
                   k_workspace)
    d = make_attn_desc(q, k, v, cos, sin, o, **kw)
    ws = _k_workspace(k_workspace, k)
    if ws is None:
        _check(lib().rope_attention_fwd(ctypes.byref(d), _stream(stream)), "rope_attention_fwd")
    else:
        _check(lib().rope_attention_fwd_k_once(ctypes.byref(d), ws, _stream(stream)),
               "rope_attention_fwd_k_once")
    return o


def rope_attention_noalloc(q, k, v, cos, sin, o, *, stream=None, **kw):
    """rope_attention with K rotated once into the library's own device array
    (rope_attention_fwd_k_once_noalloc): the same result as passing a
    k_workspace, for callers that cannot allocate. o must be given (nothing
    is allocated here either). Calls that overlap on one device race."""
    _on_one_device("rope_attention_noalloc", q, k, v, cos, sin, o, kw.get("q_pos"),
                   kw.get("k_pos"))
    d = make_attn_desc(q, k, v, cos, sin, o, **kw)
    _check(lib().rope_attention_fwd_k_once_noalloc(ctypes.byref(d), _stream(stream)),
           "rope_attention_fwd_k_once_noalloc")
    return o


class PreparedAttention:
    """A rope_attention_fwd call whose descriptor is built once (see Prepared)."""

    def __init__(self, q, k, v, cos, sin, o, stream=None, k_workspace=None, **kw):
        self._keep = (q, k, v, cos, sin, o, kw.get("q_pos"), kw.get("k_pos"), k_workspace)
        _on_one_device("prepare_attention", q, k, v, cos, sin, o, kw.get("q_pos"),
                       kw.get("k_pos"), k_workspace)
        self.desc = make_attn_desc(q, k, v, cos, sin, o, **kw)
        self._ws = _k_workspace(k_workspace, k)
        self._stream = _stream(stream)
        self._pdesc = ctypes.byref(self.desc)
        self._lib = lib()

    def rope_attention_fwd(self):
        """The fused call, or with a workspace the K-once call."""
        if self._ws is None:
            _check(self._lib.rope_attention_fwd(self._pdesc, self._stream), "rope_attention_fwd")
        else:
            _check(self._lib.rope_attention_fwd_k_once(self._pdesc, self._ws, self._stream),
                   "rope_attention_fwd_k_once")


def prepare_attention(q, k, v, cos, sin, o, *, stream=None, **kw) -> PreparedAttention:
    """Build the descriptor of a rope_attention_fwd call once."""
    return PreparedAttention(q, k, v, cos, sin, o, stream=stream, **kw)

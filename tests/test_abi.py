"""The librope C ABI on the CPU: exports, validation, tables, status strings.

No test here launches GPU work. Validation runs before any HIP call and never
dereferences a device pointer, so the descriptors below use fake addresses.
The one call with valid arguments runs only where no GPU is visible, where it
must fail with ROPE_ERR_HIP instead of crashing.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import rotary_position_embedding_fwd_amd as rp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "librope.h")

OK, NULL, SHAPE, DTYPE, LAYOUT, ALIGN, ALIAS, HIP = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[a-z_][a-z_0-9 ]*?[ *](rope_[a-z_0-9]+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert {"rope_fwd_qk", "rope_bwd_qk", "rope_fwd_q", "rope_bwd_q", "rope_build_table",
            "rope_status_string", "rope_version"} <= names


def test_library_exports_every_declared_symbol():
    L = rp.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (rope_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    # the C ABI exports no C++ (mangled) names of its own
    assert not re.search(r" T _ZN4rope", out)


def test_desc_layout_matches_header():
    assert ctypes.sizeof(rp.RopeDesc) == 6 * 8 + 4 * 4 + 8 + 8 + 8 + 8 + 8
    assert rp.RopeDesc.cos.offset == 64 and rp.RopeDesc.pos_batch_stride.offset == 96


def test_version_and_status_strings():
    assert rp.rope_version() >= 10000
    for code in (OK, NULL, SHAPE, DTYPE, LAYOUT, ALIGN, ALIAS, HIP):
        assert rp.status_string(code) and rp.status_string(code) != "unknown status"
    assert rp.status_string(-99) == "unknown status"


A16 = 1 << 20  # a fake, 16-byte aligned device address (never dereferenced)


def good_desc(**kw):
    d = rp.RopeDesc()
    d.batch, d.n_heads_q, d.n_heads_k, d.seq_len, d.head_dim, d.rotary_dim = 2, 4, 2, 8, 64, 64
    d.dtype, d.layout, d.pairing, d.launch = 2, 0, 0, 0
    d.cos, d.sin, d.table_rows = A16 * 64, A16 * 65, 8
    d.pos, d.pos_batch_stride = None, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def call_qk(d, q=A16, k=A16 * 16, fn="rope_fwd_qk"):
    return getattr(rp.lib(), fn)(q, k, ctypes.byref(d) if d is not None else None, None)


@pytest.mark.parametrize("fn", ["rope_fwd_qk", "rope_bwd_qk"])
@pytest.mark.parametrize("change,expected", [
    (dict(dtype=3), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(layout=2), LAYOUT), (dict(pairing=2), LAYOUT), (dict(launch=3), LAYOUT),
    (dict(rotary_dim=63), SHAPE), (dict(rotary_dim=66), SHAPE),
    (dict(n_heads_k=5), SHAPE), (dict(batch=-1), SHAPE), (dict(seq_len=-2), SHAPE),
    (dict(head_dim=-64), SHAPE), (dict(table_rows=7), SHAPE), (dict(n_heads_k=-1), SHAPE),
    (dict(cos=None), NULL), (dict(sin=None), NULL),
    (dict(cos=A16 * 64 + 4), ALIGN), (dict(sin=A16 * 65 + 8), ALIGN),
    (dict(pos=A16 * 70 + 2, table_rows=4), ALIGN),
    (dict(pos=A16 * 70, pos_batch_stride=-1), SHAPE),
])
def test_validation_errors(fn, change, expected):
    assert call_qk(good_desc(**change), fn=fn) == expected


def test_null_and_alias_and_alignment():
    assert call_qk(None) == NULL
    assert call_qk(good_desc(), q=None) == NULL
    assert call_qk(good_desc(), k=None) == NULL
    assert call_qk(good_desc(), q=A16 + 1) == ALIGN  # bf16 needs 2-byte alignment
    assert call_qk(good_desc(dtype=0), k=A16 * 16 + 2) == ALIGN  # f32 needs 4
    q_bytes = 2 * 4 * 8 * 64 * 2
    assert call_qk(good_desc(), q=A16, k=A16 + q_bytes - 2) == ALIAS
    k_bytes = 2 * 2 * 8 * 64 * 2
    assert call_qk(good_desc(), q=A16, k=A16 - k_bytes + 16) == ALIAS  # k ends inside q
    assert call_qk(good_desc(), q=A16, k=A16 + q_bytes) != ALIAS  # adjacent is fine


def test_q_only_ignores_k_heads():
    L = rp.lib()
    d = good_desc(n_heads_k=99, dtype=7)
    assert L.rope_fwd_q(A16, ctypes.byref(d), None) == DTYPE
    d = good_desc(n_heads_k=99, rotary_dim=3)
    assert L.rope_bwd_q(A16, ctypes.byref(d), None) == SHAPE


@pytest.mark.parametrize("change", [dict(batch=0), dict(seq_len=0), dict(rotary_dim=0),
                                    dict(n_heads_q=0, n_heads_k=0)])
def test_empty_work_is_ok_without_touching_the_gpu(change):
    # even with NULL data pointers: nothing is enqueued
    assert call_qk(good_desc(**change), q=None, k=None) == OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks behaviour with no GPU present")
def test_valid_call_without_gpu_reports_hip_error():
    assert call_qk(good_desc()) == HIP
    assert rp.lib().rope_fwd_q(A16, ctypes.byref(good_desc()), None) == HIP


@pytest.mark.parametrize("theta,R,rows,interp", [(10000.0, 64, 128, 1.0),
                                                 (10000.0, 128, 4096, 1.0),
                                                 (10000.0, 32, 9216, 1.0),
                                                 (500000.0, 128, 32768, 1.0),
                                                 (500000.0, 128, 131072, 1.0), (3.0, 6, 17, 1.0),
                                                 (10000.0, 64, 3000, 3.0),
                                                 (500000.0, 128, 8192, 0.25)])
def test_host_table_matches_oracle_bitexact(orc, theta, R, rows, interp):
    """The product's table builder and the oracle's own table are two separate
    implementations of RN32(cos/sin((p / s) * theta^(-2i/R))); they must agree."""
    c, s = rp.rope_build_table(rows, R, theta, interp)
    oc, os_ = orc.table(theta, R, rows, interp)
    assert np.array_equal(c.numpy().view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(s.numpy().view(np.uint32), os_.view(np.uint32))


def test_table_builder_errors():
    L = rp.lib()
    buf = (ctypes.c_float * 8)()
    assert L.rope_build_table(buf, buf, 2, 3, 10000.0, 1.0) == SHAPE
    assert L.rope_build_table(buf, buf, -1, 4, 10000.0, 1.0) == SHAPE
    assert L.rope_build_table(buf, buf, 2, 4, 0.0, 1.0) == SHAPE
    for bad in (0.0, -2.0, float("inf"), float("nan")):
        assert L.rope_build_table(buf, buf, 2, 4, 10000.0, bad) == SHAPE
        assert L.rope_build_table(buf, buf, 2, 4, bad if bad != 0.0 else -1.0, 1.0) == SHAPE
    assert L.rope_build_table(None, None, 2, 4, 10000.0, 1.0) == NULL
    assert L.rope_build_table(None, None, 0, 4, 10000.0, 1.0) == OK


def test_binding_marshals_shapes():
    q = torch.zeros(2, 32, 100, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 8, 100, 128, dtype=torch.bfloat16)
    cos = torch.zeros(100, 64)
    sin = torch.zeros(100, 64)
    d = rp.make_desc(q, k, cos, sin)
    assert (d.batch, d.n_heads_q, d.n_heads_k, d.seq_len, d.head_dim, d.rotary_dim) == \
        (2, 32, 8, 100, 128, 128)
    assert d.dtype == 2 and d.layout == 0 and d.table_rows == 100 and not d.pos
    qs = torch.zeros(2, 100, 32, 64, dtype=torch.float16)
    ks = torch.zeros(2, 100, 8, 64, dtype=torch.float16)
    pos = torch.zeros(100, dtype=torch.int32)
    d = rp.make_desc(qs, ks, cos[:, :16].contiguous(), sin[:, :16].contiguous(),
                     layout="bshd", pairing="interleaved", rotary_dim=32, pos=pos)
    assert (d.n_heads_q, d.n_heads_k, d.seq_len, d.head_dim, d.rotary_dim) == (32, 8, 100, 64, 32)
    assert d.dtype == 1 and d.layout == 1 and d.pairing == 1 and d.pos_batch_stride == 0
    dec = torch.zeros(7, 4, 1, 64, dtype=torch.bfloat16)
    d = rp.make_desc(dec, None, cos[:, :32].contiguous(), sin[:, :32].contiguous(),
                     pos=torch.zeros(7, dtype=torch.int32))
    assert d.pos_batch_stride == 1 and d.n_heads_k == 0
    with pytest.raises(ValueError):
        rp.make_desc(q.transpose(1, 2), None, cos, sin)
    with pytest.raises(ValueError):
        rp.make_desc(q, k, cos[:, :10].contiguous(), sin[:, :10].contiguous())


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(rp, "_lib", None)
    monkeypatch.setattr(rp, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        rp.lib()


def test_struct_layouts_match_the_c_compiler(tmp_path):
    """ctypes mirrors of rope_desc_t and rope_apply_desc_t have the C layout."""
    src = tmp_path / "layout.c"
    src.write_text('''#include <stddef.h>
#include <stdio.h>
#include "librope.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(rope_desc_t), offsetof(rope_desc_t, cos),
         offsetof(rope_desc_t, pos_batch_stride), sizeof(rope_apply_desc_t),
         offsetof(rope_apply_desc_t, q_in), offsetof(rope_apply_desc_t, k_out),
         offsetof(rope_apply_desc_t, cos), offsetof(rope_apply_desc_t, pos_batch_stride));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", f"-I{os.path.join(ROOT, 'include')}", "-o", str(exe),
                    str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    D, A = rp.RopeDesc, rp.RopeApplyDesc
    assert got == [ctypes.sizeof(D), D.cos.offset, D.pos_batch_stride.offset,
                   ctypes.sizeof(A), A.q_in.offset, A.k_out.offset, A.cos.offset,
                   A.pos_batch_stride.offset]


def apply_desc(**kw):
    d = rp.RopeApplyDesc()
    d.batch, d.seq_len, d.head_dim, d.rotary_dim, d.n_heads_q, d.n_heads_k = 2, 8, 64, 64, 4, 2
    d.dtype, d.pairing, d.launch, d.direction = 2, 0, 0, 1
    W = (4 + 2 * 2) * 64  # packed [B, S, (Hq + 2Hk) * D]
    d.q_in = rp.RopeView(A16, 8 * W, 64, W)
    d.k_in = rp.RopeView(A16 + 4 * 64 * 2, 8 * W, 64, W)
    d.cos, d.sin, d.table_rows = A16 * 64, A16 * 65, 8
    d.table_row_stride, d.table_col_stride = 0, 1
    for key, v in kw.items():
        setattr(d, key, v)
    return d


def call_apply(d):
    return rp.lib().rope_apply(ctypes.byref(d) if d is not None else None, None)


@pytest.mark.parametrize("change,expected", [
    (dict(direction=0), LAYOUT), (dict(direction=2), LAYOUT), (dict(table_col_stride=3), LAYOUT),
    (dict(table_row_stride=31), SHAPE), (dict(table_row_stride=-1), SHAPE),
    (dict(table_col_stride=2, table_row_stride=62), SHAPE),
    (dict(q_in=rp.RopeView(A16 + 1, 8 * 512, 64, 512)), ALIGN),
    (dict(q_out=rp.RopeView(A16 * 3 + 1, 0, 0, 0)), ALIGN),
    (dict(k_in=rp.RopeView(A16 + 3 * 64 * 2, 8 * 512, 64, 512)), ALIAS),   # K inside Q's heads
    (dict(q_in=rp.RopeView(A16, 8 * 512, 0, 512)), ALIAS),                  # heads share rows
    (dict(q_out=rp.RopeView(A16 + 4 * 64 * 2, 8 * 512, 64, 512)), ALIAS),  # Q out onto K in
    (dict(k_in=rp.RopeView(A16 + 4 * 64 * 2, 8 * 512, 64, -512)), SHAPE),
    (dict(k_in=rp.RopeView(None, 0, 0, 0)), NULL),
    (dict(pos=A16 + 1024, pos_batch_stride=8), ALIAS),   # index entries inside written Q
    (dict(cos=A16 + 2 * 512 * 2), ALIAS),                # cos table inside written rows
    (dict(sin=A16 - 16), ALIAS),                         # sin table runs into written Q
])
def test_apply_validation_errors(change, expected):
    assert call_apply(apply_desc(**change)) == expected


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks behaviour with no GPU present")
@pytest.mark.parametrize("change", [
    dict(),                                                        # packed QKV, in place
    dict(q_out=rp.RopeView(A16 * 8, 4 * 8 * 64, 8 * 64, 64),       # out of place, [B,H,S,D]
         k_out=rp.RopeView(A16 * 9, 2 * 8 * 64, 8 * 64, 64)),
    dict(table_row_stride=64, table_col_stride=2),                 # repeat-interleaved table
    dict(n_heads_k=0, k_in=rp.RopeView(None, 0, 0, 0),             # broadcast input, Q only
         q_in=rp.RopeView(A16, 0, 64, 512), q_out=rp.RopeView(A16 * 8, 4 * 8 * 64, 8 * 64, 64)),
    dict(q_out=rp.RopeView(A16 * 8, 4 * 8 * 64, 8 * 64, 64),       # tables and index may share
         k_out=rp.RopeView(A16 * 9, 2 * 8 * 64, 8 * 64, 64),       # memory with inputs that are
         cos=A16 + 2 * 512 * 2, pos=A16 + 1024, pos_batch_stride=8),  # only read
])
def test_apply_accepts_valid_views(change):
    """Accepted descriptors get past validation; with no GPU the call then
    fails at the HIP runtime instead."""
    assert call_apply(apply_desc(**change)) == HIP


def test_apply_empty_and_null():
    assert call_apply(None) == NULL
    assert call_apply(apply_desc(batch=0, q_in=rp.RopeView(None, 0, 0, 0))) == OK


def test_binding_marshals_strided_views():
    B, S, Hq, Hk, D = 2, 16, 8, 2, 128
    qkv = torch.zeros(B, S, (Hq + 2 * Hk) * D, dtype=torch.bfloat16)
    q = qkv[..., :Hq * D].view(B, S, Hq, D)
    k = qkv[..., Hq * D:(Hq + Hk) * D].view(B, S, Hk, D)
    c = torch.zeros(S, D)  # duplicated halves, [S, R]
    d = rp.make_apply_desc(q, k, c, c, layout="bshd", table_layout="duplicated", direction=-1)
    W = (Hq + 2 * Hk) * D
    assert (d.q_in.stride_b, d.q_in.stride_h, d.q_in.stride_s) == (S * W, D, W)
    assert d.k_in.data == q.data_ptr() + Hq * D * 2
    assert d.table_row_stride == D and d.table_col_stride == 1 and d.direction == -1
    assert not d.q_out.data and not d.k_out.data
    d = rp.make_apply_desc(q, k, c, c, layout="bshd", table_layout="interleaved",
                           q_out=torch.empty(B, S, Hq, D, dtype=torch.bfloat16))
    assert d.table_col_stride == 2 and d.q_out.data
    with pytest.raises(ValueError):
        rp.make_apply_desc(q, k, c[:, :64].contiguous(), c[:, :64].contiguous(), layout="bshd",
                           table_layout="duplicated")
    with pytest.raises(ValueError):
        rp.make_apply_desc(q.transpose(2, 3), None, c, c, table_layout="duplicated")


# ------------------------------------------------- attention with RoPE fused
def attn_desc(**kw):
    d = rp.RopeAttnDesc()
    d.batch, d.n_heads_q, d.n_heads_k, d.seq_len_q, d.seq_len_k = 2, 8, 2, 100, 100
    d.head_dim, d.rotary_dim, d.dtype, d.pairing, d.causal, d.rotate = 128, 128, 2, 0, 1, 1
    qb, kb = 2 * 8 * 100 * 128 * 2, 2 * 2 * 100 * 128 * 2
    d.q, d.k, d.v, d.o = A16 * 1024, A16 * 1024 + qb, A16 * 1024 + qb + kb, A16 * 4096
    d.cos, d.sin, d.table_rows = A16 * 8192, A16 * 9000, 100
    for key, v in kw.items():
        setattr(d, key, v)
    return d


def call_attn(d):
    return rp.lib().rope_attention_fwd(ctypes.byref(d) if d is not None else None, None)


@pytest.mark.parametrize("change,expected", [
    (dict(dtype=1), DTYPE), (dict(dtype=0), DTYPE), (dict(dtype=7), DTYPE),
    (dict(pairing=2), LAYOUT),
    (dict(head_dim=96, rotary_dim=96), SHAPE), (dict(head_dim=256, rotary_dim=128), SHAPE),
    (dict(rotary_dim=48), SHAPE),                     # split-half R % 32
    (dict(pairing=1, rotary_dim=20), SHAPE),          # interleaved R % 8
    (dict(rotary_dim=130), SHAPE), (dict(rotary_dim=-2), SHAPE),
    (dict(n_heads_k=3), SHAPE), (dict(n_heads_k=0), SHAPE), (dict(n_heads_q=0), SHAPE),
    (dict(seq_len_q=101), SHAPE),                     # causal needs Sq <= Sk
    (dict(table_rows=99), SHAPE),                     # default positions leave the table
    (dict(scale=float("nan")), SHAPE), (dict(scale=float("inf")), SHAPE),
    (dict(scale=1e-40), SHAPE), (dict(scale=-1e-45), SHAPE),   # |scale| log2 e not normal
    (dict(scale=1e39), SHAPE), (dict(scale=-1e300), SHAPE),    # ... or past float32
    (dict(batch=-1), SHAPE), (dict(q_pos_batch_stride=-1), SHAPE),
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(v=None), NULL), (dict(cos=None), NULL),
    (dict(q=A16 * 1024 + 2), ALIGN), (dict(o=A16 * 4096 + 8), ALIGN),
    (dict(sin=A16 * 9000 + 4), ALIGN),
    (dict(q_pos=A16 * 10000 + 2, k_pos=A16 * 10000), ALIGN),
    (dict(o=A16 * 1024), ALIAS),                      # O onto Q
    (dict(o=A16 * 1024 + 2 * 8 * 100 * 128 * 2 - 32), ALIAS),   # O runs into K
    (dict(cos=A16 * 4096 + 64), ALIAS),               # table inside O
    (dict(q_pos=A16 * 4096, k_pos=A16 * 10000), ALIAS),
    (dict(k_rotated=2), SHAPE),
    # one head's K/V rows, and a table, must each stay under 4 GiB (32-bit
    # offsets in the kernel)
    (dict(seq_len_k=1 << 24, causal=0, rotate=0), SHAPE),
    (dict(table_rows=1 << 24), SHAPE),
])
def test_attention_validation_errors(change, expected):
    assert call_attn(attn_desc(**change)) == expected


def call_k_once(d, ws):
    return rp.lib().rope_attention_fwd_k_once(ctypes.byref(d) if d is not None else None, ws,
                                              None)


WS = A16 * 20000  # a workspace address clear of every operand of attn_desc()


@pytest.mark.parametrize("change,ws,expected", [
    (dict(), None, NULL),                               # rotation needs the workspace
    (dict(), WS + 8, ALIGN),
    (dict(k_rotated=1), WS, SHAPE),                     # the call rotates K itself
    (dict(), A16 * 1024, ALIAS),                        # onto Q
    (dict(), A16 * 1024 + 2 * 8 * 100 * 128 * 2 + 64, ALIAS),   # onto K
    (dict(), A16 * 4096 + 16, ALIAS),                   # onto O
    (dict(), A16 * 8192 - 16, ALIAS),                   # runs into cos
    (dict(q_pos=WS + 4096, k_pos=A16 * 30000), WS, ALIAS),       # over an index row
    (dict(dtype=1), WS, DTYPE),                         # the attention's own checks first
    (dict(scale=float("nan")), WS, SHAPE),
])
def test_attention_k_once_validation_errors(change, ws, expected):
    assert call_k_once(attn_desc(**change), ws) == expected


def test_attention_k_once_empty_and_null():
    assert call_k_once(None, WS) == NULL
    assert call_k_once(attn_desc(seq_len_q=0, q=None, k=None, v=None, o=None), None) == OK


def test_attention_empty_and_null():
    assert call_attn(None) == NULL
    # no queries: nothing to do, even with NULL data pointers
    assert call_attn(attn_desc(seq_len_q=0, q=None, k=None, v=None, o=None)) == OK
    assert call_attn(attn_desc(batch=0, q=None, o=None)) == OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks behaviour with no GPU present")
@pytest.mark.parametrize("change", [
    dict(),
    dict(causal=0, seq_len_q=130),                       # non-causal, Sq > Sk
    dict(seq_len_k=0, k=None, v=None, seq_len_q=0),      # (empty: OK, checked above)
    dict(seq_len_k=0, k=None, v=None, causal=0),         # no keys: K and V may be NULL
    dict(rotate=0, cos=None, sin=None, table_rows=0),    # plain attention needs no table
    dict(rotary_dim=0, cos=None, sin=None),
    dict(pairing=1, rotary_dim=8, head_dim=64),
    dict(q_pos=A16 * 10000, k_pos=A16 * 10100, q_pos_batch_stride=100, k_pos_batch_stride=100,
         table_rows=4),                                  # index positions: any table size
    dict(cos=A16 * 1024, sin=A16 * 1024 + 64),           # tables may share memory with inputs
    dict(scale=-0.125), dict(scale=1e-30),               # any sign; small but normal
])
def test_attention_accepts_valid_descriptors(change):
    rc = call_attn(attn_desc(**change))
    assert rc in ((OK,) if change.get("seq_len_q") == 0 else (HIP,))


def test_attention_desc_layout_matches_the_c_compiler(tmp_path):
    src = tmp_path / "attn_layout.c"
    src.write_text('''#include <stddef.h>
#include <stdio.h>
#include "librope.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(rope_attn_desc_t), offsetof(rope_attn_desc_t, q),
         offsetof(rope_attn_desc_t, table_rows), offsetof(rope_attn_desc_t, q_pos),
         offsetof(rope_attn_desc_t, k_pos_batch_stride), offsetof(rope_attn_desc_t, scale));
  return 0;
}
''')
    exe = tmp_path / "attn_layout"
    subprocess.run(["gcc", "-std=c11", f"-I{os.path.join(ROOT, 'include')}", "-o", str(exe),
                    str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    D = rp.RopeAttnDesc
    assert got == [ctypes.sizeof(D), D.q.offset, D.table_rows.offset, D.q_pos.offset,
                   D.k_pos_batch_stride.offset, D.scale.offset]


def test_binding_marshals_attention():
    q = torch.zeros(2, 8, 50, 64, dtype=torch.bfloat16)
    k = torch.zeros(2, 2, 70, 64, dtype=torch.bfloat16)
    c = torch.zeros(70, 16)
    o = torch.empty_like(q)
    d = rp.make_attn_desc(q, k, k, c, c, o, causal=True)
    assert (d.batch, d.n_heads_q, d.n_heads_k, d.seq_len_q, d.seq_len_k, d.head_dim,
            d.rotary_dim, d.table_rows, d.causal, d.rotate) == (2, 8, 2, 50, 70, 64, 32, 70, 1, 1)
    kp = torch.arange(140, dtype=torch.int32)
    qp = torch.arange(50, dtype=torch.int32)
    d = rp.make_attn_desc(q, k, k, c, c, o, q_pos=qp, k_pos=kp)
    assert d.q_pos_batch_stride == 0 and d.k_pos_batch_stride == 70
    with pytest.raises(ValueError):
        rp.make_attn_desc(q, k, k, c, c, o, k_pos=kp[:69])
    with pytest.raises(ValueError):
        rp.make_attn_desc(q, k, k[:, :1].contiguous(), c, c, o)
    with pytest.raises(ValueError):
        rp.make_attn_desc(q, k, k, c, c, o[:, :, :10])


def test_attention_sizes_whose_byte_counts_overflow():
    # each size within the 32-bit index limit, their product past int64
    big = 1 << 30
    assert call_attn(attn_desc(batch=big, n_heads_q=big, n_heads_k=big, seq_len_q=big,
                               seq_len_k=big, causal=0)) == SHAPE
    assert call_attn(attn_desc(table_rows=(1 << 62))) == SHAPE
    # an index batch stride whose extent overflows
    assert call_attn(attn_desc(q_pos=A16 * 10000, k_pos=A16 * 10100,
                               q_pos_batch_stride=(1 << 62), k_pos_batch_stride=100)) == SHAPE


@pytest.mark.parametrize("change", [
    dict(q_in=rp.RopeView(A16, 1 << 62, 64, 512)),           # batch stride past int64
    dict(table_row_stride=1 << 61),                           # table extent past int64
    dict(pos=A16 * 1000, pos_batch_stride=1 << 62),           # index extent past int64
])
def test_apply_extents_that_overflow_are_rejected(change):
    assert call_apply(apply_desc(**change)) == SHAPE


# ----------------------------------------- the binding guards host pointers
def _cpu_operands():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    c = torch.zeros(8, 32)
    return q, k, c


def test_binding_rejects_host_tensors_before_any_library_call(monkeypatch):
    """librope cannot tell a host pointer from a device pointer without
    touching the GPU; every binding call must refuse host tensors itself,
    before it reaches the C library (replaced here by one that fails the
    test if called)."""
    def no_call():
        raise AssertionError("the C library was reached with host tensors")
    monkeypatch.setattr(rp, "lib", no_call)
    q, k, c = _cpu_operands()
    pos = torch.zeros(8, dtype=torch.int32)
    calls = [
        lambda: rp.rope_fwd_qk(q, k, c, c),
        lambda: rp.rope_bwd_qk(q, k, c, c),
        lambda: rp.rope_fwd_q(q, c, c),
        lambda: rp.rope_bwd_q(q, c, c, pos=pos),
        lambda: rp.rope_apply(q, k, c, c),
        lambda: rp.rope_apply(q, k, None, None, theta=1e4),
        lambda: rp.rope_apply_xpos(q, k, c, c, c, c),
        lambda: rp.prepare(q, k, c, c),
        lambda: rp.prepare_apply(q, k, c, c),
        lambda: rp.prepare_apply_xpos(q, k, c, c, c, c),
        lambda: rp.rope_attention(q, k, k, c, c),
        lambda: rp.prepare_attention(q, k, k, c, c, torch.empty_like(q)),
        lambda: rp.rope_attention_noalloc(q, k, k, c, c, torch.empty_like(q)),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="on the GPU"):
            call()


def test_attention_descriptor_checks_its_tables():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    o = torch.empty_like(q)
    c = torch.zeros(8, 32)
    d = rp.make_attn_desc(q, k, k, c, c, o)
    assert d.rotary_dim == 64 and d.table_rows == 8
    d = rp.make_attn_desc(q, k, k, c[:, :16].contiguous(), c[:, :16].contiguous(), o,
                          rotary_dim=32)
    assert d.rotary_dim == 32
    bad = [
        dict(cos=c.to(torch.bfloat16), sin=c.to(torch.bfloat16)),        # not float32
        dict(cos=torch.zeros(8, 64)[:, ::2], sin=torch.zeros(8, 64)[:, ::2]),  # column slice
        dict(cos=c, sin=c, rotary_dim=32),                                 # R/2 != columns
        dict(cos=c, sin=torch.zeros(8, 16)),                               # sin unlike cos
        dict(cos=c, sin=None),
    ]
    for b in bad:
        kw = dict(b)
        cos, sin = kw.pop("cos"), kw.pop("sin")
        with pytest.raises(ValueError):
            rp.make_attn_desc(q, k, k, cos, sin, o, **kw)


def test_describe_validates_without_a_device():
    L = rp.lib()
    buf = ctypes.create_string_buffer(256)
    assert L.rope_describe(A16, A16 * 3, ctypes.byref(good_desc()), 1, None, 256) == NULL
    assert L.rope_describe(A16, A16 * 3, ctypes.byref(good_desc()), 1, buf, 0) == NULL
    bad = good_desc()
    bad.rotary_dim = 3
    assert L.rope_describe(A16, A16 * 3, ctypes.byref(bad), 1, buf, 256) == SHAPE
    assert buf.value == b""


def test_no_alloc_attention_rejects_k_beyond_its_array():
    """rope_attention_fwd_k_once_noalloc stages rope(K) in a 64 MiB device
    array: a larger K is ROPE_ERR_SHAPE, found on the host before any HIP
    call; a K that fits passes validation (and then needs a device)."""
    L = rp.lib()
    far = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, cos=5 << 40, sin=6 << 40)
    # K = 2 * 2 * 65537 * 128 bf16 values: 2 KiB more than 64 MiB
    big = attn_desc(seq_len_q=65537, seq_len_k=65537, table_rows=65537, **far)
    assert L.rope_attention_fwd_k_once_noalloc(ctypes.byref(big), None) == SHAPE
    fits = attn_desc(seq_len_q=65536, seq_len_k=65536, table_rows=65536, **far)
    assert L.rope_attention_fwd_k_once_noalloc(ctypes.byref(fits), None) == HIP
    assert L.rope_attention_fwd_k_once_noalloc(None, None) == NULL
    assert L.rope_attention_fwd_k_once_noalloc(ctypes.byref(attn_desc(k_rotated=1)),
                                                None) == SHAPE

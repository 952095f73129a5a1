"""GPU checks against values the method fixes exactly, not against tolerances.

  - Position 0 is the identity ("Rotary Embedding Kernel", Overview: the
    angle of position 0 is 0, so cos = 1 and sin = 0 exactly): every row at
    position 0 comes back bit for bit, for every dtype, pairing and layout, with
    tables and with angles computed from theta.
  - Unit vectors: a pair (1, 0) becomes (cos, sin) and (0, 1) becomes
    (-sin, cos). In float32 the kernel's arithmetic is exact here, so the
    outputs must equal, bit for bit, the oracle's own float32 table (cos and
    sin of the binary64 angle, rounded once), and for the backward the same
    with sin negated.
  - An index is a gather: rotating with an index tensor equals rotating the
    same rows with the table rows the index names copied into a contiguous
    table and no index (positions s = 0, 1, ...), bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import rotary_position_embedding_fwd_amd as rp
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).numpy()


POS0_CASES = {
    "f32_bhsd_split": W.TINY_F32,
    "bf16_bhsd_split": W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=300, table_rows=300),
    "f16_bshd_interleaved": W.BSHD_INTERLEAVED.scaled(batch=2, seq_len=333, table_rows=333),
    "bf16_partial": W.PARTIAL_INDEXED.scaled(pos_kind="none", table_rows=1026),
}


@pytest.mark.parametrize("angles", ["tables", "theta"])
@pytest.mark.parametrize("name", list(POS0_CASES))
def test_position_zero_is_the_identity(name, angles):
    w = POS0_CASES[name]
    say(f"[gpu] position 0 identity {name} {angles}")
    t = W.tensors(w)
    zeros = torch.zeros(w.seq_len, dtype=torch.int32, device=DEV)
    for direction in (1, -1):
        q, k = t["q"].to(DEV), t["k"].to(DEV)
        if angles == "tables":
            cos, sin = (x.to(DEV) for x in rp.rope_build_table(w.table_rows, w.rotary_dim,
                                                               w.theta))
            rp.rope_apply(q, k, cos, sin, layout=w.layout, pairing=w.pairing,
                          rotary_dim=w.rotary_dim, direction=direction, pos=zeros,
                          pos_batch_stride=0)
        else:
            rp.rope_apply(q, k, None, None, layout=w.layout, pairing=w.pairing,
                          rotary_dim=w.rotary_dim, direction=direction, pos=zeros,
                          pos_batch_stride=0, theta=w.theta, max_positions=w.table_rows)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(q), _bits(t["q"])), (name, direction)
        assert np.array_equal(_bits(k), _bits(t["k"])), (name, direction)


@pytest.mark.parametrize("name", list(POS0_CASES))
def test_first_token_rows_unchanged(name):
    """Without an index, token 0 sits at position 0: its rows are unchanged
    while the rest of the call rotates."""
    w = POS0_CASES[name]
    t = W.tensors(w)
    cos, sin = (x.to(DEV) for x in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
    q, k = t["q"].to(DEV), t["k"].to(DEV)
    rp.rope_fwd_qk(q, k, cos, sin, layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim)
    torch.cuda.synchronize()
    for g, x in ((q, t["q"]), (k, t["k"])):
        g0 = g[:, :, 0] if w.layout == "bhsd" else g[:, 0]
        x0 = x[:, :, 0] if w.layout == "bhsd" else x[:, 0]
        assert np.array_equal(_bits(g0), _bits(x0))
        g1 = g[:, :, 1] if w.layout == "bhsd" else g[:, 1]
        x1 = x[:, :, 1] if w.layout == "bhsd" else x[:, 1]
        assert not np.array_equal(_bits(g1), _bits(x1))


@pytest.mark.parametrize("pairing", ["split_half", "interleaved"])
@pytest.mark.parametrize("theta,R,rows", [(10000.0, 64, 128), (500000.0, 128, 4096)])
def test_unit_vectors_give_the_table_f32(pairing, theta, R, rows):
    """fp32 rows holding (1, 0) in every pair of one token and (0, 1) in the
    next: the outputs are the oracle's fp32 cos/sin values bit for bit."""
    say(f"[gpu] unit vectors fp32 {pairing} theta={theta} R={R} rows={rows}")
    half = R // 2
    S, H, D = rows, 3, R + 6
    x = torch.zeros(1, H, S, D, dtype=torch.float32)
    if pairing == "split_half":
        j1, j2 = np.arange(half), np.arange(half) + half
    else:
        j1, j2 = 2 * np.arange(half), 2 * np.arange(half) + 1
    x[:, :, 0::2, j1] = 1.0   # even tokens: (x1, x2) = (1, 0)
    x[:, :, 1::2, j2] = 1.0   # odd tokens:  (x1, x2) = (0, 1)
    x[..., R:] = 3.25
    c32, s32 = orc.table(theta, R, rows)
    cos, sin = (a.to(DEV) for a in rp.rope_build_table(rows, R, theta))
    for direction in (1, -1):
        q = x.clone().to(DEV)
        rp.rope_fwd_q(q, cos, sin, layout="bhsd", pairing=pairing, rotary_dim=R) \
            if direction == 1 else rp.rope_bwd_q(q, cos, sin, layout="bhsd", pairing=pairing,
                                                 rotary_dim=R)
        torch.cuda.synchronize()
        y = q.cpu().numpy()
        sg = np.float32(direction)
        zero = np.float32(0.0)
        even, odd = y[:, :, 0::2], y[:, :, 1::2]
        for h in range(H):
            # (1, 0) -> (c, sigma s); each output is a sum of an exact product
            # and an exact zero, so a zero comes out +0 (IEEE: -0 + +0 = +0)
            assert np.array_equal(even[0, h][:, j1].view(np.int32),
                                  (c32[0::2] + zero).view(np.int32))
            assert np.array_equal(even[0, h][:, j2].view(np.int32),
                                  (sg * s32[0::2] + zero).view(np.int32))
            # (0, 1) -> (-sigma s, c)
            assert np.array_equal(odd[0, h][:, j1].view(np.int32),
                                  (-sg * s32[1::2] + zero).view(np.int32))
            assert np.array_equal(odd[0, h][:, j2].view(np.int32),
                                  (c32[1::2] + zero).view(np.int32))
        assert np.all(y[..., R:] == 3.25)


def _gather_tables(cos, sin, rows_idx):
    return cos[rows_idx.long()].contiguous(), sin[rows_idx.long()].contiguous()


def test_index_is_a_gather_partial_rotary():
    """The partial-rotary workload's index (two skipped tokens, then
    start + 0, 1, ...): its rotated tokens equal the same rows rotated with
    the gathered table rows and no index; the skipped rows are unchanged."""
    w = W.PARTIAL_INDEXED
    t = W.tensors(w)
    pos = W.positions(w)
    cos, sin = (x.to(DEV) for x in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
    q, k = t["q"].to(DEV), t["k"].to(DEV)
    rp.rope_fwd_qk(q, k, cos, sin, layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim,
                   pos=pos.to(DEV), pos_batch_stride=0)
    m = w.n_masked
    gc, gs = _gather_tables(cos, sin, pos[m:].to(DEV))
    q2, k2 = t["q"].to(DEV), t["k"].to(DEV)
    # the rotated tokens as [B,H,S-m,D] views (no index: positions 0 .. S-m-1)
    rp.rope_apply(q2[:, :, m:], k2[:, :, m:], gc, gs, layout="bhsd", pairing=w.pairing,
                  rotary_dim=w.rotary_dim)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(q), _bits(q2)) and np.array_equal(_bits(k), _bits(k2))
    assert np.array_equal(_bits(q[:, :, :m]), _bits(t["q"][:, :, :m]))


def test_index_is_a_gather_decode():
    """Decode: one position per sequence. Q [256, 32, 1, 128] is, in memory,
    [1, 256, 32, 128] with the sequences as tokens; rotating that view with
    the gathered table rows and no index equals the indexed decode call."""
    w = W.DECODE
    t = W.tensors(w)
    pos = W.positions(w)
    cos, sin = (x.to(DEV) for x in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
    q, k = t["q"].to(DEV), t["k"].to(DEV)
    rp.rope_fwd_qk(q, k, cos, sin, layout="bhsd", pairing=w.pairing, rotary_dim=w.rotary_dim,
                   pos=pos.to(DEV), pos_batch_stride=1)
    gc, gs = _gather_tables(cos, sin, pos.to(DEV))
    q2 = t["q"].to(DEV).view(1, w.batch, w.n_heads_q, w.head_dim)
    k2 = t["k"].to(DEV).view(1, w.batch, w.n_heads_k, w.head_dim)
    rp.rope_fwd_qk(q2, k2, gc, gs, layout="bshd", pairing=w.pairing, rotary_dim=w.rotary_dim)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(q), _bits(q2.view(q.shape)))
    assert np.array_equal(_bits(k), _bits(k2.view(k.shape)))
    # and the oracle agrees with both
    for g, x in ((q, t["q"]), (k, t["k"])):
        P.assert_parity(P.storage(g.cpu()), P.oracle_rope(w, x, 1, pos), P.storage(x),
                        w.dtype, w.layout, w.rotary_dim)

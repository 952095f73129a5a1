"""GPU parity at the full sizes of the large workloads, on every element.

The Llama GQA prefill ([4, 32+8, 4096, 128] bf16), BSHD interleaved
([8, 2048, 16+16, 64] fp16) and long-context ([1, 32+8, 131072, 128] bf16)
calls run through the C ABI in the launch configuration bench.py times
(automatic launch shape, in place), forward on seeded Q/K and backward on
seeded dQ/dK. Every output element is compared with the CPU oracle at the
tolerances of tests/_parity.py (float32 math inside, 16-bit outputs within
one unit of the oracle's single rounding; untouched dims bit-exact).

The oracle is plain scalar C; to finish in seconds it is called on one
(batch, head) slice at a time ([B,H,S,D]) or one batch at a time
([B,S,H,D]) from a pool of threads (ctypes releases the interpreter lock).
Slicing changes nothing it computes: each slice keeps its own positions
(s = 0 .. S-1 of the full sequence) and the full table.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as orc
import rotary_position_embedding_fwd_amd as rp
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
WORKERS = max(1, min(16, os.cpu_count() or 1))


def say(msg):
    print(msg, flush=True)


def _slices(w):
    """Index tuples that cut a tensor of workload w into oracle-sized slices."""
    if w.layout == "bhsd":
        return lambda H: [(slice(b, b + 1), slice(h, h + 1))
                          for b in range(w.batch) for h in range(H)]
    return lambda H: [(slice(b, b + 1),) for b in range(w.batch)]


def _compare_sliced(w, got, inp, direction, what):
    """Oracle on each slice of `inp`, compared with the same slice of `got`."""
    heads = inp.shape[1] if w.layout == "bhsd" else inp.shape[2]
    g_st, x_st = P.storage(got), P.storage(inp)

    def one(ix):
        xs = np.ascontiguousarray(x_st[ix])
        gs = np.ascontiguousarray(g_st[ix])
        ref = orc.rope(xs, w.dtype, layout=w.layout, pairing=w.pairing, direction=direction,
                       rotary_dim=w.rotary_dim, theta=w.theta, table_rows=w.table_rows)
        return P.assert_parity(gs, ref, xs, w.dtype, w.layout, w.rotary_dim, None,
                               f"{what} slice {ix}")

    with ThreadPoolExecutor(WORKERS) as ex:
        stats = list(ex.map(one, _slices(w)(heads)))
    key = "max_abs" if w.dtype == "f32" else "max_ord"
    return max(s[key] for s in stats), sum(s.get("n_off_by_one", 0) for s in stats)


@pytest.mark.parametrize("direction", [1, -1])
@pytest.mark.parametrize("name", ["llama_gqa_prefill_bf16", "bshd_interleaved_fp16",
                                  "long_context_bf16"])
def test_full_size_every_element(name, direction):
    w = W.BY_NAME[name]
    names = ("q", "k") if direction == 1 else ("dq", "dk")
    say(f"[gpu] full size every element: {name} dir={direction} "
        f"q{tuple(w.q_shape)} k{tuple(w.k_shape)} {w.dtype}")
    t = W.tensors(w, names)
    cos, sin = (x.to(DEV) for x in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
    qd, kd = t[names[0]].to(DEV), t[names[1]].to(DEV)
    fn = rp.rope_fwd_qk if direction == 1 else rp.rope_bwd_qk
    fn(qd, kd, cos, sin, layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim)
    torch.cuda.synchronize()
    gq, gk = qd.cpu(), kd.cpu()
    del qd, kd
    for g, x, tag in ((gq, t[names[0]], "q"), (gk, t[names[1]], "k")):
        mx, n1 = _compare_sliced(w, g, x, direction, f"{name} {tag} dir={direction}")
        say(f"[gpu]   {tag}: max distance {mx}, elements one unit off: {n1} of {x.numel()}")


def test_head_lanes_long_form_with_a_ragged_head_group():
    """Heads 16 MiB apart take the long-sequence head-lanes form (4 tokens x
    20 heads per workgroup); 20 + 5 heads leave a ragged second group."""
    w = W.LONG_CONTEXT.scaled(seq_len=65536, table_rows=65536, n_heads_q=20, n_heads_k=5)
    say(f"[gpu] head lanes, long form: q{tuple(w.q_shape)} k{tuple(w.k_shape)}")
    t = W.tensors(w)
    cos, sin = (x.to(DEV) for x in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
    qd, kd = t["q"].to(DEV), t["k"].to(DEV)
    rp.rope_fwd_qk(qd, kd, cos, sin, layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim)
    torch.cuda.synchronize()
    for g, x, tag in ((qd.cpu(), t["q"], "q"), (kd.cpu(), t["k"], "k")):
        mx, n1 = _compare_sliced(w, g, x, 1, f"long form {tag}")
        say(f"[gpu]   {tag}: max distance {mx}, one unit off: {n1}")


@pytest.mark.parametrize("direction", [1, -1])
def test_flat_pair_full_size_every_element(direction):
    """The BSHD workload's shape with split-half pairs ([8, 2048, 16+16, 64]
    fp16): the flat pair-lanes kernel at full size, every element, both
    directions; rope_describe confirms the kernel."""
    w = W.BSHD_INTERLEAVED.scaled(pairing=W.SPLIT_HALF)
    names = ("q", "k") if direction == 1 else ("dq", "dk")
    say(f"[gpu] flat pair full size every element: dir={direction} q{tuple(w.q_shape)}")
    t = W.tensors(w, names)
    cos, sin = (x.to(DEV) for x in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
    qd, kd = t[names[0]].to(DEV), t[names[1]].to(DEV)
    kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim)
    assert rp.rope_describe(qd, kd, cos, sin, **kw).startswith("rope_flat_pair_kernel")
    fn = rp.rope_fwd_qk if direction == 1 else rp.rope_bwd_qk
    fn(qd, kd, cos, sin, **kw)
    torch.cuda.synchronize()
    for g, x, tag in ((qd.cpu(), t[names[0]], "q"), (kd.cpu(), t[names[1]], "k")):
        mx, n1 = _compare_sliced(w, g, x, direction, f"flat pair {tag} dir={direction}")
        say(f"[gpu]   {tag}: max distance {mx}, one unit off: {n1} of {x.numel()}")

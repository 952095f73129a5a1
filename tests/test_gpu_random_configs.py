"""GPU parity on seeded random configurations.

Each case draws one problem from its own fixed seed: storage dtype, layout
([B,H,S,D], [B,S,H,D], or Q/K views into one packed [B, S, (Hq + 2 Hk) D]
buffer), pairing, head and rotary dims, head counts, batch and a ragged
sequence length, positions (none, or an index row, shared or per sequence,
holding skipped and out-of-table entries), the cos/sin source (tables or
angles from theta), in place or out of place, and the direction.

The call runs three ways: AUTO (whatever kernel the planner picks for that
shape: head lanes, flat, flat pair lanes, pair lanes, token or rows) and the
two forced grid shapes. AUTO is compared with the oracle on every element
(tests/_parity.py's bar), and the three results bit for bit with each other:
every kernel rotates each pair with the same float32 steps, so the bits must
agree whichever shape runs. Views' neighbours (the V part of a packed buffer)
stay bit-exact, and out-of-place calls leave their inputs untouched.
"""
import os

import numpy as np
import pytest
import torch

import oracle as orc
import rotary_position_embedding_fwd_amd as rp
import workloads as W
from tests import _parity as P
from tests._random_configs import draw as _draw, workload

DEV = "cuda"
# LIBROPE_RANDOM_SCALE=n runs n times as many cases (a longer sweep on demand)
N_CASES = 160 * int(os.environ.get("LIBROPE_RANDOM_SCALE", "1"))
ELEMENT_BUDGET = 3 << 20  # Q + K elements per case, so the oracle takes well under a second


def draw(case: int) -> dict:
    return _draw(9100 + case, ELEMENT_BUDGET)


def say(msg):
    print(msg, flush=True)


def inputs(c):
    """CPU tensors: (buffer, q, k, the V part or None), q and k views of the
    buffer in packed layout."""
    B, S, Hq, Hk, D = c["batch"], c["seq_len"], c["n_heads_q"], c["n_heads_k"], c["head_dim"]
    if c["layout"] == "packed":
        qkv = W.normal((B, S, (Hq + 2 * Hk) * D), c["dtype"], c["seed"])
        q = qkv[..., :Hq * D].view(B, S, Hq, D)
        k = qkv[..., Hq * D:(Hq + Hk) * D].view(B, S, Hk, D)
        return qkv, q, k, qkv[..., (Hq + Hk) * D:]
    shape = (lambda h: (B, h, S, D)) if c["layout"] == "bhsd" else (lambda h: (B, S, h, D))
    q = W.normal(shape(Hq), c["dtype"], c["seed"])
    k = W.normal(shape(Hk), c["dtype"], c["seed"] + 50)
    return None, q, k, None


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def run(c, launch: str):
    """One call on fresh device copies; returns CPU results (q, k, V part,
    q input, k input after the call)."""
    buf, q, k, vpart = inputs(c)
    if buf is not None:
        g = buf.to(DEV)
        B, S, Hq, Hk, D = c["batch"], c["seq_len"], c["n_heads_q"], c["n_heads_k"], c["head_dim"]
        gq = g[..., :Hq * D].view(B, S, Hq, D)
        gk = g[..., Hq * D:(Hq + Hk) * D].view(B, S, Hk, D)
    else:
        gq, gk = q.to(DEV), k.to(DEV)
    layout = "bhsd" if c["layout"] == "bhsd" else "bshd"
    kw = dict(layout=layout, pairing=c["pairing"], rotary_dim=c["rotary_dim"],
              direction=c["direction"], launch=launch)
    if c["pos"] is not None:
        kw["pos"] = torch.from_numpy(c["pos"]).to(DEV)
        kw["pos_batch_stride"] = c["pos_batch_stride"]
    if c["angles"] == "theta":
        cos = sin = None
        kw.update(theta=c["theta"], max_positions=c["table_rows"])
    else:
        cos, sin = rp.rope_build_table(c["table_rows"], c["rotary_dim"], c["theta"])
        cos, sin = cos.to(DEV), sin.to(DEV)
    oq = ok = None
    if c["out_of_place"]:
        oq = torch.full(gq.shape, 3.0, dtype=gq.dtype, device=DEV)
        ok = torch.full(gk.shape, 3.0, dtype=gk.dtype, device=DEV)
        kw.update(q_out=oq, k_out=ok)
    rq, rk = rp.rope_apply(gq, gk, cos, sin, **kw)
    torch.cuda.synchronize()
    vp = None if buf is None else g[..., (c["n_heads_q"] + c["n_heads_k"]) * c["head_dim"]:].cpu()
    return rq.cpu(), rk.cpu(), vp, gq.cpu(), gk.cpu()


def oracle(c, x: torch.Tensor) -> np.ndarray:
    w = workload(c)
    layout = "bhsd" if c["layout"] == "bhsd" else "bshd"
    return orc.rope(P.storage(x.contiguous()), c["dtype"], layout=layout, pairing=c["pairing"],
                    direction=c["direction"], rotary_dim=c["rotary_dim"], theta=c["theta"],
                    pos=c["pos"], pos_batch_stride=(c["pos_batch_stride"] or 0),
                    table_rows=w.table_rows)


def masked(c, heads_axis_first: bool) -> np.ndarray:
    w = workload(c).scaled(layout="bhsd" if heads_axis_first else "bshd")
    pos = None if c["pos"] is None else torch.from_numpy(c["pos"])
    return P.masked_tokens(w, pos, pos_batch_stride=c["pos_batch_stride"])


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(case):
    c = draw(case)
    say(f"[gpu] random case {case}: " + ", ".join(
        f"{k}={v}" for k, v in c.items() if k not in ("pos",)) +
        ("" if c["pos"] is None else f", pos[{len(c['pos'])}]"))
    outs = {}
    for launch in ("auto", "rows", "token"):
        outs[launch] = run(c, launch)
    _, q, k, vpart = inputs(c)
    if c["layout"] != "packed" and c["angles"] == "table" and not c["out_of_place"]:
        cos, sin = rp.rope_build_table(c["table_rows"], c["rotary_dim"], c["theta"])
        kw = dict(layout=c["layout"], pairing=c["pairing"], rotary_dim=c["rotary_dim"])
        if c["pos"] is not None:
            kw.update(pos=torch.from_numpy(c["pos"]).to(DEV),
                      pos_batch_stride=c["pos_batch_stride"])
        say("[gpu]   auto: " + rp.rope_describe(q.to(DEV), k.to(DEV), cos.to(DEV), sin.to(DEV),
                                                **kw))
    a = outs["auto"]
    for launch in ("rows", "token"):
        o = outs[launch]
        for i, what in ((0, "q"), (1, "k")):
            assert torch.equal(bits(a[i]), bits(o[i])), f"auto vs {launch}: {what} differs"
    first = c["layout"] == "bhsd"
    for got, x, what in ((a[0], q, "q"), (a[1], k, "k")):
        P.assert_parity(P.storage(got.contiguous()), oracle(c, x), P.storage(x.contiguous()),
                        c["dtype"], "bhsd" if first else "bshd", c["rotary_dim"],
                        masked(c, first), f"case {case} {what}")
    if vpart is not None:
        assert torch.equal(bits(a[2]), bits(vpart)), "V part of the packed buffer changed"
    if c["out_of_place"]:
        assert torch.equal(bits(a[3]), bits(q)), "out-of-place call changed q"
        assert torch.equal(bits(a[4]), bits(k)), "out-of-place call changed k"


def test_draws_cover_the_space():
    """The seeded draws reach every layout, dtype, pairing, angle source and
    both position kinds (a check of the generator, no GPU work)."""
    cs = [draw(i) for i in range(N_CASES)]
    for key, values in (("layout", {"bhsd", "bshd", "packed"}), ("dtype", {"f32", "f16", "bf16"}),
                        ("pairing", {W.SPLIT_HALF, W.INTERLEAVED}),
                        ("angles", {"table", "theta"}), ("direction", {1, -1}),
                        ("out_of_place", {True, False})):
        assert {c[key] for c in cs} == values, key
    assert any(c["pos"] is not None for c in cs) and any(c["pos"] is None for c in cs)
    assert any(c["rotary_dim"] < c["head_dim"] for c in cs)
    assert any(c["seq_len"] == 1 for c in cs)


@pytest.mark.gpu
def test_draws_reach_every_kernel():
    """AUTO's choice over the draws (contiguous in-place table calls, through
    rope_describe, which enqueues nothing) includes every kernel family."""
    seen = set()
    for i in range(N_CASES):
        c = draw(i)
        if c["layout"] == "packed" or c["angles"] != "table" or c["out_of_place"]:
            continue
        _, q, k, _ = inputs(c)
        cos, sin = rp.rope_build_table(c["table_rows"], c["rotary_dim"], c["theta"])
        kw = dict(layout=c["layout"], pairing=c["pairing"], rotary_dim=c["rotary_dim"])
        if c["pos"] is not None:
            kw.update(pos=torch.from_numpy(c["pos"]).to(DEV),
                      pos_batch_stride=c["pos_batch_stride"])
        d = rp.rope_describe(q.to(DEV), k.to(DEV), cos.to(DEV), sin.to(DEV), **kw)
        seen.add(d.split()[0].split("<")[0])
    say(f"[gpu] kernels AUTO chose over the draws: {sorted(seen)}")
    for name in ("rope_head_lanes_kernel", "rope_flat_kernel", "rope_flat_pair_kernel",
                 "rope_pair_lanes_kernel", "rope_token_kernel", "rope_rows_kernel"):
        assert name in seen, name

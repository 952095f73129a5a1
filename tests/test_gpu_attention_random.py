"""GPU parity of attention over rotated Q and K on seeded random configurations.

Each case draws from its own seed: batch, K/V heads and the GQA ratio, head
dim 64 or 128, pairing and rotary dim (a multiple of 32 for split-half pairs,
of 8 for interleaved ones, 0 = no rotation), causal or not, the query and
key lengths (ragged; Sq <= Sk when causal), positions (none, one shared
index row with two skipped tokens, or per-sequence indices holding skipped
and out-of-table entries), the softmax scale (default, or drawn with either
sign), and the form: the fused call or K rotated once into a workspace.
The output is compared with the oracle on every element under the bound of
tests/_attn.py. The grid sizes the draws produce also reach the forms for
small grids at head dim 64 (two or four wave groups).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_fwd_amd as rp
import workloads as W
from tests import _attn as A

DEV = "cuda"
# LIBROPE_RANDOM_SCALE=n runs n times as many cases (a longer sweep on demand)
N_CASES = 40 * int(os.environ.get("LIBROPE_RANDOM_SCALE", "1"))
WORK_BUDGET = 1.5e8  # B * Hq * Sq * Sk * D per case, so the oracle and bound stay quick


def say(msg):
    print(msg, flush=True)


def draw(case: int) -> dict:
    r = np.random.RandomState(9500 + case)
    c = {"batch": int(r.choice([1, 2, 3]))}
    hk = int(r.choice([1, 2, 3]))
    c["n_heads_k"] = hk
    c["n_heads_q"] = hk * int(r.choice([1, 2, 3, 4, 6, 8, 16]))
    c["head_dim"] = D = int(r.choice([64, 128]))
    c["pairing"] = str(r.choice([W.SPLIT_HALF, W.INTERLEAVED]))
    step = 32 if c["pairing"] == W.SPLIT_HALF else 8
    c["rotary_dim"] = D if r.rand() < 0.5 else step * int(r.randint(0, D // step + 1))
    c["causal"] = bool(r.rand() < 0.6)
    sk = int(r.randint(1, 600))
    sq = int(r.randint(1, sk + 1)) if c["causal"] else int(r.randint(1, 600))
    # keep the oracle's work bounded
    while c["batch"] * c["n_heads_q"] * sq * sk * D > WORK_BUDGET and sk > 1:
        sk = max(1, sk // 2)
        sq = min(sq, sk) if c["causal"] else max(1, sq // 2)
    c["seq_len_q"], c["seq_len_k"] = sq, sk
    kind = str(r.choice(["none", "none", "shared_cls", "per_sequence"]))
    if kind == "shared_cls" and sq != sk:
        kind = "none"
    c["positions"] = kind
    c["table_rows"] = max(sq, sk) + int(r.randint(0, 40))
    c["scale"] = 0.0 if r.rand() < 0.7 else float(r.choice([-1, 1]) * r.uniform(0.02, 0.5))
    c["form"] = str(r.choice(["fused", "k_once"]))
    c["seed"] = 9700 + case
    return c


def positions(c):
    B, sq, sk, rows = c["batch"], c["seq_len_q"], c["seq_len_k"], c["table_rows"]
    if c["positions"] == "none":
        return None, None
    if c["positions"] == "shared_cls":
        p = torch.cat([torch.full((2,), -1, dtype=torch.int32),
                       torch.arange(max(sq - 2, 0), dtype=torch.int32)])[:sq]
        return p, p
    qp = W.random_positions(B * sq, rows + 1, c["seed"] + 1, low=-1)
    kp = W.random_positions(B * sk, rows + 1, c["seed"] + 2, low=-1)
    return qp, kp


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_attention(case):
    c = draw(case)
    say(f"[gpu] attention random case {case}: " + ", ".join(f"{k}={v}" for k, v in c.items()))
    B, Hq, Hk, D = c["batch"], c["n_heads_q"], c["n_heads_k"], c["head_dim"]
    sq, sk, R = c["seq_len_q"], c["seq_len_k"], c["rotary_dim"]
    q = W.normal((B, Hq, sq, D), "bf16", c["seed"])
    k = W.normal((B, Hk, sk, D), "bf16", c["seed"] + 10)
    v = W.normal((B, Hk, sk, D), "bf16", c["seed"] + 20)
    qp, kp = positions(c)
    rotate = R > 0
    kw = dict(pairing=c["pairing"], rotary_dim=R, causal=c["causal"], rotate=rotate,
              q_pos=None if qp is None else qp.to(DEV), k_pos=None if kp is None else kp.to(DEV),
              scale=c["scale"])
    if rotate:
        cos, sin = (t.to(DEV) for t in rp.rope_build_table(c["table_rows"], R, 10000.0))
        ocs = oracle.table(10000.0, R, c["table_rows"])
    else:
        cos = sin = None
        ocs = (None, None)
    kd = k.to(DEV)
    ws = torch.full_like(kd, float("nan")) if c["form"] == "k_once" and rotate else None
    o = rp.rope_attention(q.to(DEV), kd, v.to(DEV), cos, sin, k_workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu().view(torch.int16), k.view(torch.int16)), "K changed"
    ref, tol = A.reference(q, k, v, *ocs, pairing=c["pairing"], rotary_dim=R,
                           causal=c["causal"], q_pos=qp, k_pos=kp, rotate=rotate,
                           scale=c["scale"] or None)
    worst = A.check(o.cpu(), ref, tol, f"random case {case}")
    say(f"[gpu]   worst error / bound = {worst:.3f}")


def test_attention_draws_cover_the_space():
    cs = [draw(i) for i in range(N_CASES)]
    for key, values in (("head_dim", {64, 128}), ("pairing", {W.SPLIT_HALF, W.INTERLEAVED}),
                        ("causal", {True, False}), ("form", {"fused", "k_once"}),
                        ("positions", {"none", "shared_cls", "per_sequence"})):
        assert {c[key] for c in cs} == values, key
    assert any(c["rotary_dim"] == 0 for c in cs)
    assert any(0 < c["rotary_dim"] < c["head_dim"] for c in cs)
    assert any(c["scale"] < 0 for c in cs) and any(c["scale"] > 0 for c in cs)
    assert any(c["n_heads_q"] > c["n_heads_k"] for c in cs)

"""GPU parity of the fused attention (rope_attention_fwd) against the oracle.

Every call goes through the ctypes binding to librope.so. The expected values
come from oracle.rope_attention and the per-element bound from tests/_attn.py
(derived from the kernel's bf16/float32 arithmetic). Sizes:
  - oracle-sized cases compare every element: several query and key tiles
    with ragged tails, both pairings, partial rotary dims, GQA and MQA,
    causal and not, index positions with skipped tokens;
  - the full-size Llama prefill runs in the launch configuration bench.py
    times and is compared on sampled query blocks, which the oracle computes
    exactly as sub-problems (a block of query rows against the keys they
    see, with their positions given explicitly);
  - fusing the rotation into the kernel changes nothing: the fused output
    equals, bit for bit, the stand-alone rotation followed by the same
    kernel with rotation off.
"""
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_fwd_amd as rp
import workloads as W
from tests import _attn as A

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def tables(rows, R, theta=10000.0):
    """(library tables on the GPU, the oracle's host copies for the bound)."""
    c, s = rp.rope_build_table(rows, R, theta)
    oc, os_ = oracle.table(theta, R, rows)
    return (c.to(DEV), s.to(DEV)), (oc, os_)


def run(q, k, v, gt, **kw):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for name in ("q_pos", "k_pos"):
        if kw.get(name) is not None:
            kw[name] = kw[name].to(DEV)
    o = rp.rope_attention(qd, kd, vd, gt[0] if gt else None, gt[1] if gt else None, **kw)
    torch.cuda.synchronize()
    return o.cpu()


def inputs(B, Hq, Hk, Sq, Sk, D, seed):
    return (W.normal((B, Hq, Sq, D), "bf16", seed), W.normal((B, Hk, Sk, D), "bf16", seed + 1),
            W.normal((B, Hk, Sk, D), "bf16", seed + 2))


def positions(kind, B, S, rows, seed):
    if kind == "none":
        return None
    if kind == "cls":          # two unrotated tokens, then 0, 1, ...
        return torch.cat([torch.full((2,), -1, dtype=torch.int32),
                          torch.arange(S - 2, dtype=torch.int32)])
    if kind == "random":       # per batch, including -1 and rows (both pass through)
        return W.random_positions(B * S, rows + 1, seed, low=-1)
    raise ValueError(kind)


# name: B Hq Hk Sq Sk D R pairing causal positions
CASES = {
    "d128_split_causal_ragged": (1, 4, 1, 130, 130, 128, 128, "split_half", True, "none"),
    "d128_split_gqa_noncausal": (2, 8, 2, 77, 200, 128, 128, "split_half", False, "none"),
    "d128_split_partial96": (1, 2, 1, 150, 150, 128, 96, "split_half", True, "none"),
    "d128_split_partial32": (2, 2, 2, 65, 65, 128, 32, "split_half", False, "random"),
    "d128_interleaved": (1, 4, 2, 129, 129, 128, 128, "interleaved", True, "none"),
    "d128_interleaved_partial8": (1, 2, 1, 70, 130, 128, 8, "interleaved", False, "random"),
    "d64_split_cls": (1, 4, 4, 258, 258, 64, 32, "split_half", True, "cls"),
    "d64_split_full": (2, 2, 1, 100, 100, 64, 64, "split_half", True, "random"),
    "d64_interleaved": (1, 3, 1, 64, 193, 64, 64, "interleaved", True, "none"),
    "d64_interleaved_partial24": (1, 2, 2, 33, 33, 64, 24, "interleaved", False, "none"),
    "decode_like_sq1": (3, 8, 2, 1, 300, 128, 128, "split_half", True, "none"),
    "short_sq3": (1, 4, 1, 3, 129, 64, 64, "split_half", True, "none"),
    "no_rotation": (1, 2, 1, 96, 96, 128, 0, "split_half", True, "none"),
    # 8 query heads per workgroup (32 rows each) and 16 per K/V head
    "gqa_8_heads_per_workgroup": (1, 16, 2, 70, 140, 128, 128, "split_half", True, "none"),
    "gqa_16_to_1": (2, 16, 1, 40, 97, 64, 64, "interleaved", False, "random"),
    # GQA 3:1 (one head per workgroup), more queries than keys, not causal
    "gqa_3_to_1_sq_gt_sk": (1, 6, 2, 300, 100, 128, 64, "split_half", False, "none"),
    "batch_8_short": (8, 4, 2, 33, 65, 64, 32, "split_half", True, "random"),
    # head dim 64 with grids of at least 256 workgroups: one wave group (the
    # cases above at head dim 64 take four groups, the next one two)
    "d64_two_wave_groups": (1, 24, 24, 1024, 1024, 64, 64, "split_half", True, "none"),
    "d64_wide_grid_split_half": (4, 32, 8, 520, 520, 64, 64, "split_half", True, "none"),
    "d64_wide_grid_interleaved": (2, 64, 8, 520, 520, 64, 64, "interleaved", False, "random"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_every_element_matches_oracle(name):
    B, Hq, Hk, Sq, Sk, D, R, pairing, causal, pk = CASES[name]
    say(f"[gpu] attention {name}: B{B} Hq{Hq} Hk{Hk} Sq{Sq} Sk{Sk} D{D} R{R} {pairing} "
        f"causal={causal} pos={pk}")
    q, k, v = inputs(B, Hq, Hk, Sq, Sk, D, 8000 + Sq + Sk)
    rows = max(Sq, Sk)
    qp = positions(pk, B, Sq, rows, 8100 + Sq)
    kp = positions(pk, B, Sk, rows, 8200 + Sk) if pk != "cls" else qp
    if R:
        gt, ot = tables(rows, R)
    else:
        gt, ot = None, (None, None)
    got = run(q, k, v, gt, pairing=pairing, rotary_dim=R, causal=causal, q_pos=qp, k_pos=kp,
              rotate=R > 0)
    ref, tol = A.reference(q, k, v, *ot, pairing=pairing, rotary_dim=R, causal=causal,
                           q_pos=qp, k_pos=kp, rotate=R > 0)
    worst = A.check(got, ref, tol, name)
    say(f"[gpu]   worst error / bound = {worst:.3f}")


def test_cls_skip_full_size():
    w = W.ATTN_CLS_SKIP
    t = W.attn_tensors(w)
    pos = W.attn_positions(w)
    say(f"[gpu] attention {w.name} full size q{w.q_shape}")
    gt, ot = tables(w.table_rows, w.rotary_dim, w.theta)
    got = run(t["q"], t["k"], t["v"], gt, pairing=w.pairing, rotary_dim=w.rotary_dim,
              causal=w.causal, q_pos=pos, k_pos=pos)
    ref, tol = A.reference(t["q"], t["k"], t["v"], *ot, pairing=w.pairing,
                           rotary_dim=w.rotary_dim, theta=w.theta, causal=w.causal, q_pos=pos,
                           k_pos=pos)
    say(f"[gpu]   worst error / bound = {A.check(got, ref, tol, w.name):.3f}")


def test_llama_prefill_full_size_sampled():
    w = W.ATTN_LLAMA_PREFILL
    t = W.attn_tensors(w)
    say(f"[gpu] attention {w.name} full size q{w.q_shape} kv{w.kv_shape}")
    gt, ot = tables(w.table_rows, w.rotary_dim, w.theta)
    got = run(t["q"], t["k"], t["v"], gt, pairing=w.pairing, rotary_dim=w.rotary_dim,
              causal=w.causal)
    Sq, Sk, n = w.seq_len_q, w.seq_len_k, 32
    group = w.n_heads_q // w.n_heads_k
    worst = 0.0
    for b, h, r0 in ((0, 0, 0), (0, 31, Sq - n), (1, 9, 1000), (2, 17, 2048 + 7),
                     (3, 30, 4001), (3, 4, 64)):
        hk = h // group
        m = r0 + n + (Sk - Sq) if w.causal else Sk
        qb = t["q"][b:b + 1, h:h + 1, r0:r0 + n]
        kb = t["k"][b:b + 1, hk:hk + 1, :m]
        vb = t["v"][b:b + 1, hk:hk + 1, :m]
        qp = torch.arange(r0, r0 + n, dtype=torch.int32) + (Sk - Sq)
        kp = torch.arange(m, dtype=torch.int32)
        ref, tol = A.reference(qb, kb, vb, *ot, pairing=w.pairing, rotary_dim=w.rotary_dim,
                               theta=w.theta, causal=w.causal, q_pos=qp, k_pos=kp)
        worst = max(worst, A.check(got[b:b + 1, h:h + 1, r0:r0 + n], ref, tol,
                                   f"{w.name} b{b} h{h} rows {r0}..{r0 + n - 1}"))
    say(f"[gpu]   worst error / bound over the samples = {worst:.3f}")
    # every output row is finite and each row is a convex combination of V rows
    assert torch.isfinite(got.float()).all()
    vmax = t["v"].float().abs().amax(dim=2, keepdim=True)        # [B, Hk, 1, D]
    vmax = vmax.repeat_interleave(group, dim=1)
    assert (got.float().abs() <= vmax * (1 + 2.0 ** -7) + 1e-6).all()


# name: B Hq Hk Sq Sk D R pairing causal positions
FUSED_CASES = {
    "split_gqa_causal": (2, 8, 2, 200, 200, 128, 128, "split_half", True, "none"),
    "split_partial_positions": (2, 4, 4, 130, 130, 64, 32, "split_half", False, "random"),
    "interleaved_sq_lt_sk": (1, 4, 1, 100, 230, 128, 64, "interleaved", True, "none"),
}


@pytest.mark.parametrize("name", list(FUSED_CASES))
def test_fused_equals_rotation_then_attention(name):
    B, Hq, Hk, Sq, Sk, D, R, pairing, causal, pk = FUSED_CASES[name]
    say(f"[gpu] attention fused vs unfused {name}")
    q, k, v = inputs(B, Hq, Hk, Sq, Sk, D, 8500 + Sq)
    rows = max(Sq, Sk) + 8
    gt, _ = tables(rows, R)
    qp = positions(pk, B, Sq, rows, 8600)
    kp = positions(pk, B, Sk, rows, 8700)
    kw = dict(pairing=pairing, rotary_dim=R, causal=causal)
    fused = run(q, k, v, gt, q_pos=qp, k_pos=kp, **kw)
    # stand-alone rotation of Q and K (query i at i + Sk - Sq without an index)
    qd, kd = q.to(DEV), k.to(DEV)
    qpos = (torch.arange(Sq, dtype=torch.int32) + (Sk - Sq)) if qp is None else qp
    kpos = torch.arange(Sk, dtype=torch.int32) if kp is None else kp
    rp.rope_fwd_q(qd, gt[0], gt[1], pairing=pairing, rotary_dim=R, pos=qpos.to(DEV),
                  pos_batch_stride=Sq if qpos.numel() >= B * Sq else 0)
    rp.rope_fwd_q(kd, gt[0], gt[1], pairing=pairing, rotary_dim=R, pos=kpos.to(DEV),
                  pos_batch_stride=Sk if kpos.numel() >= B * Sk else 0)
    unfused = run(qd, kd, v, None, rotate=False, **kw)
    assert torch.equal(fused.view(torch.int16), unfused.view(torch.int16))


K_ONCE_CASES = dict(FUSED_CASES, **{
    "cls_positions_d64": (1, 4, 4, 258, 258, 64, 32, "split_half", True, "cls"),
    "gqa_16_to_1_interleaved": (2, 16, 1, 40, 97, 64, 64, "interleaved", False, "random"),
})


@pytest.mark.parametrize("name", list(K_ONCE_CASES))
def test_k_once_equals_fused(name):
    # rope(K) written once into a workspace, then the attention rotating only
    # Q: the same bits as the fused call; and the workspace holds rope_fwd_q's K
    B, Hq, Hk, Sq, Sk, D, R, pairing, causal, pk = K_ONCE_CASES[name]
    say(f"[gpu] attention K once vs fused {name}")
    q, k, v = inputs(B, Hq, Hk, Sq, Sk, D, 8900 + Sq)
    rows = max(Sq, Sk) + 8
    gt, _ = tables(rows, R)
    qp = positions(pk, B, Sq, rows, 8910)
    kp = positions(pk, B, Sk, rows, 8920) if pk != "cls" else qp
    kw = dict(pairing=pairing, rotary_dim=R, causal=causal, q_pos=qp, k_pos=kp)
    fused = run(q, k, v, gt, **kw)
    kd = k.to(DEV)
    ws = torch.full_like(kd, float("nan"))
    once = run(q, kd, v, gt, k_workspace=ws, **kw)
    assert torch.equal(fused.view(torch.int16), once.view(torch.int16))
    assert torch.equal(kd.cpu(), k)  # K itself is left as it was
    kpos = torch.arange(Sk, dtype=torch.int32) if kp is None else kp
    kr = kd.clone()
    rp.rope_fwd_q(kr, gt[0], gt[1], pairing=pairing, rotary_dim=R, pos=kpos.to(DEV),
                  pos_batch_stride=Sk if kpos.numel() >= B * Sk else 0)
    assert torch.equal(ws.view(torch.int16), kr.view(torch.int16))


def test_k_rotated_descriptor_with_rope_fwd_q():
    # a caller that already holds rope(K) (here from rope_fwd_q) sets
    # k_rotated: the same bits as the fused call
    B, Hq, Hk, Sq, Sk, D, R = 1, 8, 2, 150, 150, 128, 128
    q, k, v = inputs(B, Hq, Hk, Sq, Sk, D, 8960)
    gt, _ = tables(Sk, R)
    fused = run(q, k, v, gt, rotary_dim=R, causal=True)
    kr = k.to(DEV)
    rp.rope_fwd_q(kr, gt[0], gt[1], rotary_dim=R)
    got = run(q, kr, v, gt, rotary_dim=R, causal=True, k_rotated=True)
    assert torch.equal(fused.view(torch.int16), got.view(torch.int16))


def test_k_once_full_size_equals_fused():
    w = W.ATTN_LLAMA_PREFILL
    t = {key: x.to(DEV) for key, x in W.attn_tensors(w).items()}
    say(f"[gpu] attention K once vs fused, {w.name} full size")
    gt, _ = tables(w.table_rows, w.rotary_dim, w.theta)
    kw = dict(pairing=w.pairing, rotary_dim=w.rotary_dim, causal=w.causal)
    fused = rp.rope_attention(t["q"], t["k"], t["v"], gt[0], gt[1], **kw)
    once = rp.rope_attention(t["q"], t["k"], t["v"], gt[0], gt[1],
                             k_workspace=torch.empty_like(t["k"]), **kw)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), once.view(torch.int16))


def test_no_keys_gives_zeros_and_empty_queries_do_nothing():
    q = W.normal((1, 2, 40, 128), "bf16", 8800).to(DEV)
    k = torch.empty((1, 1, 0, 128), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    c, s = tables(8, 128)[0]
    o = torch.full_like(q, 7.0)
    rp.rope_attention(q, k, v, c, s, o=o, causal=False)
    torch.cuda.synchronize()
    assert (o == 0).all()
    qe = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    ke = W.normal((1, 1, 5, 128), "bf16", 8801).to(DEV)
    oe = rp.rope_attention(qe, ke, ke.clone(), c, s)
    torch.cuda.synchronize()
    assert oe.numel() == 0


def test_explicit_scale_matches_oracle():
    B, Hq, Hk, Sq, Sk, D, R = 1, 2, 1, 70, 70, 64, 64
    q, k, v = inputs(B, Hq, Hk, Sq, Sk, D, 8900)
    gt, ot = tables(Sk, R)
    got = run(q, k, v, gt, rotary_dim=R, causal=True, scale=0.3)
    ref, tol = A.reference(q, k, v, *ot, rotary_dim=R, causal=True, scale=0.3)
    A.check(got, ref, tol, "explicit scale")


@pytest.mark.parametrize("scale", [-0.3, 2.0, -2.0, 1e-3])
def test_any_scale_matches_oracle(scale):
    # negative: the softmax of -|scale| S (the kernel takes -Q); |scale| 2:
    # the row max jumps by more than 8 in the base-2 exponent between many
    # 32-key steps, so the output is rescaled often, and weights far below
    # the max underflow to 0; 1e-3: nearly uniform weights, the reference max
    # never moves after the first step
    B, Hq, Hk, Sq, Sk, D, R = 1, 4, 2, 150, 300, 128, 128
    say(f"scale {scale}")
    q, k, v = inputs(B, Hq, Hk, Sq, Sk, D, 8950)
    gt, ot = tables(Sk, R)
    got = run(q, k, v, gt, rotary_dim=R, causal=True, scale=scale)
    ref, tol = A.reference(q, k, v, *ot, rotary_dim=R, causal=True, scale=scale)
    A.check(got, ref, tol, f"scale {scale}")

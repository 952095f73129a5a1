"""The error bound of tests/_attn.py, checked on the CPU.

Two directions:
  - a numerical model of the kernel's arithmetic (float32 scores, online
    softmax over 32-key steps in base 2 whose reference max moves only when
    a step's max passes it by more than 8, weights rounded to bf16 before
    they multiply V, float32 accumulation, bf16 output), written here in
    numpy from that description, stays inside the bound, both as one walk
    over the keys and as 2 or 4 walks that take turns on the 64-key tiles,
    merged at the end (the form for small grids at head dim 64);
  - mistakes planted in the oracle (a key dropped, the causal diagonal moved
    by one, the wrong pairing, positions off by one, K left unrotated, the
    wrong K/V head for a query head) land outside it.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import _attn as A


def _inputs(B, Hq, Hk, Sq, Sk, D, seed):
    q = W.normal((B, Hq, Sq, D), "bf16", seed)
    k = W.normal((B, Hk, Sk, D), "bf16", seed + 1)
    v = W.normal((B, Hk, Sk, D), "bf16", seed + 2)
    return q, k, v


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _kernel_model(q, k, v, cos, sin, *, pairing, R, theta, causal, q_pos=None, k_pos=None,
                  scale=None, groups=1):
    """The kernel's arithmetic in numpy float32 (see the module docstring).

    groups: the form for small grids at head dim 64, where G = 2 or 4 groups
    of waves take turns on the 64-key tiles (group g: tiles g, g + G, ...)
    with their own running states, merged at the end by rescaling every
    state to the largest reference max and adding them in group order."""
    qs, ks, vs = (oracle.torch_to_storage(t) for t in (q, k, v))
    B, Hq, Sq, D = qs.shape
    Hk, Sk = ks.shape[1], ks.shape[2]
    qp = A._positions(q_pos, B, Sq, Sk - Sq).astype(np.int32)
    kp = A._positions(k_pos, B, Sk, 0).astype(np.int32)
    qr = A.bf16_values(oracle.rope(qs, "bf16", pairing=pairing, rotary_dim=R, theta=theta,
                                   pos=qp, pos_batch_stride=Sq, table_rows=cos.shape[0]))
    kr = A.bf16_values(oracle.rope(ks, "bf16", pairing=pairing, rotary_dim=R, theta=theta,
                                   pos=kp, pos_batch_stride=Sk, table_rows=cos.shape[0]))
    vv = A.bf16_values(vs).astype(np.float32)
    c = np.float32((1.0 / np.sqrt(D) if scale is None else scale) * 1.4426950408889634)
    out = np.zeros((B, Hq, Sq, D), np.float64)
    g = Hq // Hk
    for b in range(B):
        for h in range(Hq):
            Q = qr[b, h].astype(np.float32)
            K = kr[b, h // g].astype(np.float32)
            V = vv[b, h // g]
            states = []
            for g0 in range(groups):
                steps = [k0 for t0 in range(64 * g0, Sk, 64 * groups)
                         for k0 in (t0, t0 + 32) if k0 < Sk]
                states.append(_walk(Q, K, V, c, steps, Sk, causal))
            m, l, acc = states[0]
            if groups > 1:
                mm = m.copy()
                for mg, _, _ in states[1:]:
                    mm = np.maximum(mm, mg)
                with np.errstate(invalid="ignore"):
                    f = [np.where(np.isneginf(mm), 0, np.exp2(mg - mm)).astype(np.float32)
                         for mg, _, _ in states]
                l = (l * f[0]).astype(np.float32)
                acc = (acc * f[0][:, None]).astype(np.float32)
                for (_, lg, accg), fg in zip(states[1:], f[1:]):
                    l = (l + lg * fg).astype(np.float32)
                    acc = (acc + accg * fg[:, None]).astype(np.float32)
            inv = np.where(l > 0, 1 / l, 0).astype(np.float32)
            out[b, h] = _bf16(acc * inv[:, None])
    return out


def _walk(Q, K, V, c, steps, Sk, causal):
    """One running softmax state over the 32-key steps starting at `steps`."""
    Sq, D = Q.shape
    m = np.full(Sq, -np.inf, np.float32)
    l = np.zeros(Sq, np.float32)
    acc = np.zeros((Sq, D), np.float32)
    for k0 in steps:
        kk = np.arange(k0, min(k0 + 32, Sk))
        x = (Q @ K[kk].T) * c
        if causal:
            x = np.where(kk[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq), x, -np.inf)
        m_t = x.max(axis=1)
        # (-inf - -inf gives NaN in the branches np.where discards)
        with np.errstate(invalid="ignore"):
            move = m_t - m > 8
            m_new = np.where(move, m_t, m).astype(np.float32)
            alpha = np.where(move, np.exp2(m - m_new), np.float32(1)).astype(np.float32)
            p = np.where(np.isneginf(x), np.float32(0), np.exp2(x - m_new[:, None]))
        p = p.astype(np.float32)
        l = l * alpha + p.sum(axis=1, dtype=np.float32)
        acc = acc * alpha[:, None] + _bf16(p) @ V[kk]
        m = m_new
    return m, l, acc


CASES = [
    # B Hq Hk Sq Sk D R pairing causal
    (1, 2, 1, 130, 130, 64, 64, "split_half", True),
    (2, 4, 2, 77, 200, 128, 128, "split_half", False),
    (1, 2, 2, 129, 129, 64, 32, "interleaved", True),
    (1, 1, 1, 1, 257, 128, 96, "split_half", True),
]


@pytest.mark.parametrize("groups", [1, 2, 4], ids=["one_group", "two_groups", "four_groups"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_kernel_model_inside_bound(orc, case, groups):
    B, Hq, Hk, Sq, Sk, D, R, pairing, causal = case
    q, k, v = _inputs(B, Hq, Hk, Sq, Sk, D, 7100 + Sq)
    cos, sin = oracle.table(10000.0, R, max(Sq, Sk))
    ref, tol = A.reference(q, k, v, cos, sin, pairing=pairing, rotary_dim=R, causal=causal)
    got = _kernel_model(q, k, v, cos, sin, pairing=pairing, R=R, theta=10000.0, causal=causal,
                        groups=groups)
    err = np.abs(got - ref)
    assert (err <= tol).all(), float((err / tol).max())
    # the bound is not vacuous: well under the size of the outputs
    assert np.median(tol) < 0.02 * np.median(np.abs(A.bf16_values(
        oracle.torch_to_storage(v)))) + 0.01


@pytest.mark.parametrize("groups", [1, 2, 4], ids=["one_group", "two_groups", "four_groups"])
@pytest.mark.parametrize("scale", [-0.3, 2.0, -2.0])
def test_kernel_model_inside_bound_any_scale(orc, scale, groups):
    # large |scale|: the row max jumps by more than 8 in the base-2 exponent
    # between many 32-key steps, so the model rescales often; negative: the
    # softmax of -|scale| S
    B, Hq, Hk, Sq, Sk, D, R = 1, 2, 1, 100, 300, 64, 64
    q, k, v = _inputs(B, Hq, Hk, Sq, Sk, D, 7200)
    cos, sin = oracle.table(10000.0, R, Sk)
    ref, tol = A.reference(q, k, v, cos, sin, rotary_dim=R, causal=True, scale=scale)
    got = _kernel_model(q, k, v, cos, sin, pairing="split_half", R=R, theta=10000.0,
                        causal=True, scale=scale, groups=groups)
    err = np.abs(got - ref)
    assert (err <= tol).all(), float((err / tol).max())


def _mutant_violates(ref, tol, mut, min_frac=0.01):
    bad = np.abs(mut - ref) > tol
    return bad.mean() >= min_frac


def test_planted_mistakes_fall_outside(orc):
    B, Hq, Hk, Sq, Sk, D, R = 1, 4, 2, 130, 130, 64, 64
    q, k, v = _inputs(B, Hq, Hk, Sq, Sk, D, 7300)
    cos, sin = oracle.table(10000.0, R, Sk)
    qs, ks, vs = (oracle.torch_to_storage(t) for t in (q, k, v))
    qp = np.arange(Sq, dtype=np.int32)
    kp = np.arange(Sk, dtype=np.int32)
    ref, tol = A.reference(q, k, v, cos, sin, causal=True)
    ref_nc, tol_nc = A.reference(q, k, v, cos, sin, causal=False)
    base = dict(pairing="split_half", rotary_dim=R, theta=10000.0, table_rows=Sk, scale=None)

    def orc_att(qa, ka, va, qpos, kpos, causal=True, **over):
        kw = dict(base, **over)
        return oracle.rope_attention(qa, ka, va, "bf16", qpos=qpos, qpos_batch_stride=0,
                                     kpos=kpos, kpos_batch_stride=0, causal=causal, **kw)

    # the same call reproduces the expected values exactly
    assert np.array_equal(orc_att(qs, ks, vs, qp, kp), ref)
    mutants = {
        # the last key of every query row dropped (non-causal)
        "dropped key": (orc_att(qs, ks[:, :, :-1].copy(), vs[:, :, :-1].copy(), qp, kp[:-1],
                                causal=False), ref_nc, tol_nc),
        # the causal diagonal moved by one: each query loses its own key (rows
        # 1.. against keys 0..Sk-2 keep the shape causal attention accepts)
        "causal off by one": (orc_att(qs[:, :, 1:].copy(), ks[:, :, :-1].copy(),
                                      vs[:, :, :-1].copy(), qp[1:], kp[:-1]),
                              ref[:, :, 1:], tol[:, :, 1:]),
        "wrong pairing": (orc_att(qs, ks, vs, qp, kp, pairing="interleaved"), ref, tol),
        "query positions off by one": (orc_att(qs, ks, vs, qp + 1, kp), ref, tol),
        "keys not rotated": (orc_att(qs, ks, vs, qp, np.full(Sk, -1, np.int32)), ref, tol),
        "wrong kv head": (orc_att(qs, ks[:, ::-1].copy(), vs[:, ::-1].copy(), qp, kp), ref, tol),
    }
    for name, (mut, r, t) in mutants.items():
        assert _mutant_violates(r, t, mut), name


def test_unrounded_weights_are_distinguishable(orc):
    # the bound is tight enough that a kernel which skipped the bf16 rounding
    # of its weights would still pass, but one that rounded them twice (to
    # 4 bits) would not
    B, Hq, Hk, Sq, Sk, D, R = 1, 1, 1, 64, 200, 64, 64
    q, k, v = _inputs(B, Hq, Hk, Sq, Sk, D, 7400)
    cos, sin = oracle.table(10000.0, R, Sk)
    ref, tol = A.reference(q, k, v, cos, sin)
    qs, ks, vs = (oracle.torch_to_storage(t) for t in (q, k, v))
    qr = A.bf16_values(oracle.rope(qs, "bf16", rotary_dim=R, pos=np.arange(Sq, dtype=np.int32)
                                   + (Sk - Sq), table_rows=Sk))[0, 0]
    kr = A.bf16_values(oracle.rope(ks, "bf16", rotary_dim=R, table_rows=Sk))[0, 0]
    vv = A.bf16_values(vs)[0, 0]
    s = qr @ kr.T / np.sqrt(D)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    l = w.sum(axis=1, keepdims=True)
    exact = (w @ vv) / l
    assert (np.abs(exact - ref[0, 0]) <= tol[0, 0]).all()
    coarse = w / w.max(axis=1, keepdims=True)
    e = np.floor(np.log2(np.maximum(coarse, 1e-300)))
    coarse = np.round(coarse / 2.0 ** (e - 3)) * 2.0 ** (e - 3) * w.max(axis=1, keepdims=True)
    assert _mutant_violates(ref[0, 0], tol[0, 0], (coarse @ vv) / l)

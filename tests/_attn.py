"""Oracle reference and error bound for attention over rotated Q and K.

The expected output comes from oracle.rope_attention (binary64 attention over
Q and K rotated and rounded to bf16 exactly as the stand-alone rotation
stores them). The tolerance is an error bound of the matrix-core kernel's
arithmetic, element by element, built from oracle results only:

  1. Softmax weights rounded to bf16 before they multiply V: each weight
     moves by at most u = 2^-8 of itself, so the output moves by at most
     u * sum_j w_j |v_j| = u * A, where A is the oracle's attention with |V|.
  2. Errors in the scores: float32 accumulation of the D products
     (gamma = (D + 16) * 2^-24 of sum |q_d k_d|), the float32 scale product and
     exp2 (a few 2^-23 in the base-2 exponent), and rotated elements whose
     exact value lies within float32 rounding of a bf16 midpoint (the kernel
     may round those the other way: one bf16 ulp). If every score of row i
     moves by at most eps_i, every weight moves by a factor within
     exp(+-2 eps_i), so the output moves by at most (exp(2 eps_i) - 1) * A.
  3. float32 running sums over Sk keys (weights, output accumulators and the
     rescales between key steps): 2 (Sk + 128) 2^-24 * A; and the rescale
     factor exp2((m_old - m_new) * |scale| log2 e), applied at most once per
     32-key step (the kernel moves its reference max only when the new max
     passes it by more than 8 in the base-2 exponent, so the weights stay
     below 2^8; a bf16 weight's relative rounding does not depend on its
     size), each off by its argument's rounding and exp2's error, which adds
     (ceil(Sk / 32) + 2) * ln2 * (2^-23 |x|max + 2^-22) to eps_i. The two
     extra factors cover the form for small grids at head dim 64, where G =
     2 or 4 groups of waves take turns on the 64-key tiles, each walking at
     most 2 ceil(ceil(Sk / 64) / G) <= ceil(Sk / 64) + 1 steps of 32 keys,
     and the groups' states then merge with one more rescale each; the
     merge's products and sums are at most seven more float32 roundings,
     inside the running-sum term's 128 spare keys.
  4. The final rounding of O to bf16: u * |O|.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

import oracle

U16 = 2.0 ** -8           # unit roundoff of bf16 (8 significant bits)
ULP16_REL = 2.0 ** -7     # one bf16 ulp, relative to the value, at most
F32_BAND = 2.0 ** -20     # relative distance to a bf16 midpoint that the
                          # kernel's float32 rotation may cross (8 float32 ulps)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 storage bits -> float64 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _positions(pos, batch: int, seq: int, default_offset: int):
    """[batch, seq] int64 positions: an index row (shared or per batch), or
    s + default_offset."""
    if pos is None:
        return np.broadcast_to(np.arange(seq, dtype=np.int64) + default_offset, (batch, seq))
    p = np.asarray(pos, dtype=np.int64).reshape(-1)
    if p.size >= batch * seq:
        return p[:batch * seq].reshape(batch, seq)
    return np.broadcast_to(p[:seq], (batch, seq))


def _near_midpoint(y: np.ndarray, mag: np.ndarray) -> np.ndarray:
    """Elements whose exact value y lies so close to a bf16 rounding boundary
    that a float32 evaluation may round to the other neighbour."""
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.exp2(e - 7)
    frac = a / ulp
    dist = np.abs(frac - np.floor(frac) - 0.5) * ulp
    return (a > 0) & (dist <= F32_BAND * a + 2.0 ** -40 * mag)


def _rotation_slack(x: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray,
                    pairing: str, R: int) -> np.ndarray:
    """Per element of x [B,H,S,D] (float64 values of bf16 inputs): how far the
    kernel's rotated bf16 value may sit from the oracle's (0 or one ulp)."""
    out = np.zeros_like(x)
    if R == 0:
        return out
    half = R // 2
    rows = cos.shape[0]
    ok = (pos >= 0) & (pos < rows)                          # [B, S]
    pc = np.where(ok, pos, 0)
    c = cos.astype(np.float64)[pc][:, None]                 # [B, 1, S, half]
    s = sin.astype(np.float64)[pc][:, None]
    if pairing == "split_half":
        i1, i2 = np.arange(half), np.arange(half) + half
    else:
        i1, i2 = np.arange(0, R, 2), np.arange(1, R, 2)
    x1, x2 = x[..., i1], x[..., i2]
    mag = np.abs(x1) + np.abs(x2)
    for idx, y in ((i1, x1 * c - x2 * s), (i2, x2 * c + x1 * s)):
        amb = _near_midpoint(y, mag) & ok[:, None, :, None]
        out[..., idx] = np.where(amb, ULP16_REL * np.abs(y), 0.0)
    return out


def reference(q, k, v, cos: Optional[np.ndarray], sin: Optional[np.ndarray], *,
              pairing: str = "split_half", rotary_dim: Optional[int] = None,
              theta: float = 10000.0, q_pos=None, k_pos=None, causal: bool = False,
              scale: Optional[float] = None, rotate: bool = True):
    """(expected, tolerance), both float64 [B,Hq,Sq,D], for bf16 CPU tensors
    q [B,Hq,Sq,D], k and v [B,Hk,Sk,D] and the fp32 tables the kernel is given
    (from oracle.table). q_pos / k_pos: int32 index rows (shared or per
    batch) or None."""
    qs, ks, vs = (oracle.torch_to_storage(t) for t in (q, k, v))
    B, Hq, Sq, D = qs.shape
    Hk, Sk = ks.shape[1], ks.shape[2]
    R = 0 if not rotate else (D if rotary_dim is None else rotary_dim)
    rows = 0 if cos is None else cos.shape[0]
    sc = 1.0 / np.sqrt(D) if not scale else scale
    asc = abs(sc)
    qp = _positions(q_pos, B, Sq, Sk - Sq)
    kp = _positions(k_pos, B, Sk, 0)
    qp32 = np.ascontiguousarray(qp, dtype=np.int32)
    kp32 = np.ascontiguousarray(kp, dtype=np.int32)
    kw = dict(pairing=pairing, rotary_dim=R, theta=theta, qpos=qp32, qpos_batch_stride=Sq,
              kpos=kp32, kpos_batch_stride=Sk, table_rows=max(rows, 1), causal=causal,
              scale=sc)
    ref = oracle.rope_attention(qs, ks, vs, "bf16", **kw)
    a_abs = oracle.rope_attention(qs, ks, vs & np.uint16(0x7FFF), "bf16", **kw)

    # rotated Q and K as the oracle rounds them, and the kernel's possible slack
    if R:
        qr = bf16_values(oracle.rope(qs, "bf16", pairing=pairing, rotary_dim=R, theta=theta,
                                     pos=qp32, pos_batch_stride=Sq, table_rows=rows))
        kr = bf16_values(oracle.rope(ks, "bf16", pairing=pairing, rotary_dim=R, theta=theta,
                                     pos=kp32, pos_batch_stride=Sk, table_rows=rows))
        dq = _rotation_slack(bf16_values(qs), qp, cos, sin, pairing, R)
        dk = _rotation_slack(bf16_values(ks), kp, cos, sin, pairing, R)
    else:
        qr, kr = bf16_values(qs), bf16_values(ks)
        dq, dk = np.zeros_like(qr), np.zeros_like(kr)

    gamma = (D + 16) * 2.0 ** -24
    log2e = 1.4426950408889634
    eps = np.zeros((B, Hq, Sq))
    visible = np.ones((Sq, Sk), bool)
    if causal:
        visible = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq)
    group = Hq // Hk
    for b in range(B):
        for h in range(Hq):
            Q, dQ = qr[b, h], dq[b, h]
            K, dK = kr[b, h // group], dk[b, h // group]
            aq, ak = np.abs(Q), np.abs(K)
            e = dQ @ (ak + dK).T + aq @ dK.T + gamma * (aq @ ak.T)
            s = np.abs(Q @ K.T) * asc * log2e
            e = asc * e + np.log(2.0) * (2.0 ** -22 * s + 2.0 ** -21)
            e = np.where(visible, e, 0.0)
            if Sk:
                xmax = np.where(visible, s, 0.0).max(axis=1)
                rescale = (-(-Sk // 32) + 2) * np.log(2.0) * (2.0 ** -23 * xmax + 2.0 ** -22)
                eps[b, h] = e.max(axis=1) + rescale
    grow = np.exp(2.0 * eps)[..., None]
    pre = a_abs * grow * (U16 + 2.0 * (Sk + 128) * 2.0 ** -24) + (grow - 1.0) * a_abs
    tol = pre + U16 * (np.abs(ref) + pre)
    return ref, tol


def check(got, ref: np.ndarray, tol: np.ndarray, what: str = ""):
    """Assert |got - ref| <= tol element-wise; got: a bf16 torch tensor."""
    import torch
    g = got.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite outputs"
    err = np.abs(g - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside the bound; worst at "
                             f"{tuple(int(x) for x in i)}: got {g[i]!r}, expected {ref[i]!r}, "
                             f"bound {tol[i]!r}")
    return float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0

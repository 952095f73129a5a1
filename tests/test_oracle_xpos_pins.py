"""Pins of the XPOS oracle (oracle_rope_xpos, oracle_rope_xpos_exact,
oracle_xpos_table), all on the CPU and independent of it.

The pages name XPOS (rotary-embedding-torch docs, Key Parameters: use_xpos)
without its formula; the oracle follows the xPos paper's scales (Sun et al.,
"A Length-Extrapolatable Transformer"): pair i of a query at n is scaled by
zeta_i^((n-c)/B), of a key at m by zeta_i^(-(m-c)/B), with
zeta_i = (i/(R/2) + gamma)/(1 + gamma).

  - zeta and the factor tables against mpmath at 60 digits, each entry
    rounded once to float32 (skipping entries within binary64 error of a
    float32 rounding boundary); closed forms zeta_0 = gamma/(1+gamma), the
    factor 1 at p = c, zeta_i and 1/zeta_i one scale base away;
  - table-mode outputs against exact rational arithmetic on Fractions,
    rounded to the storage format by tests/_exact.py;
  - in exact mode, a query and a key at the same position keep their plain
    dot product (the factors cancel and the rotation is orthogonal), moving
    both positions by the same amount leaves every pairwise product
    unchanged (only n - m matters), and for one pair the product is plain
    RoPE's times zeta_0^((n-m)/B);
  - with every position at c the result is plain RoPE, bit for bit.
test_oracle_mutants.py plants mistakes in the XPOS code and checks that
these pins catch them.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle
import workloads as W
from tests import _exact as X

DT = {"f32": 0, "f16": 1, "bf16": 2}


def _zeta_mp(gamma, R, i):
    g = mpmath.mpf(gamma)
    return (mpmath.mpf(i) / (mpmath.mpf(R) / 2) + g) / (1 + g)


@pytest.mark.parametrize("gamma,R", [(0.4, 128), (0.4, 32), (1.5, 64)])
def test_zeta_closed_forms(orc, gamma, R):
    assert oracle.xpos_zeta(gamma, R, 0) == gamma / (1 + gamma)
    with mpmath.workdps(60):
        for i in range(R // 2):
            z = oracle.xpos_zeta(gamma, R, i)
            assert abs(mpmath.mpf(z) - _zeta_mp(gamma, R, i)) <= mpmath.mpf(2) ** -52 * z
    # zeta grows with i and stays in (0, 1)
    zs = [oracle.xpos_zeta(gamma, R, i) for i in range(R // 2)]
    assert all(0 < a < b < 1 for a, b in zip(zs, zs[1:]))


@pytest.mark.parametrize("B,gamma,center", [(512.0, 0.4, 0.0), (64.0, 0.4, 100.0),
                                            (128.0, 0.9, 37.0)])
def test_factor_tables_against_mpmath(orc, B, gamma, center):
    R, rows = 32, 300
    zq, zk = oracle.xpos_table(R, rows, scale_base=B, gamma=gamma, center=center)
    checked = 0
    with mpmath.workdps(60):
        for p in list(range(0, rows, 7)) + [int(center)]:
            e = (mpmath.mpf(p) - mpmath.mpf(center)) / mpmath.mpf(B)
            for i in range(R // 2):
                z = _zeta_mp(gamma, R, i)
                for got, ex in ((zq[p, i], z ** e), (zk[p, i], z ** -e)):
                    if X.near_f32_midpoint(ex):
                        continue
                    assert float(got) == X.rn24_mp(ex), (p, i)
                    checked += 1
    assert checked > 1000
    c = int(center)
    assert (zq[c] == 1).all() and (zk[c] == 1).all()
    # one scale base away: zeta_i and its reciprocal, rounded once
    if c + int(B) < rows:
        for i in range(R // 2):
            z = oracle.xpos_zeta(gamma, R, i)
            assert zq[c + int(B), i] == np.float32(z) or abs(
                float(zq[c + int(B), i]) - z) <= 2 ** -24 * z
            assert abs(float(zk[c + int(B), i]) - 1 / z) <= 2 ** -23 / z


def _near_mid(y: Fraction, fmt: str) -> bool:
    prec, emin, _ = X.FORMATS[fmt]
    if y == 0:
        return False
    a = abs(y)
    e = max(X._floor_log2(a), emin)
    q = Fraction(2) ** (e - prec + 1)
    frac = a / q - int(a / q)
    return abs(frac - Fraction(1, 2)) * q <= a * Fraction(2) ** -50


@pytest.mark.parametrize("dtype,pairing,is_key,direction", [
    ("bf16", "split_half", False, 1), ("f16", "interleaved", True, -1),
    ("f32", "split_half", True, 1), ("bf16", "interleaved", False, -1)])
def test_table_mode_against_exact_rationals(orc, dtype, pairing, is_key, direction):
    B_, H, S, D, R = 1, 2, 9, 24, 16
    scale_base, gamma, center, rows = 4.0, 0.4, 3.0, 12
    x = W.normal((B_, H, S, D), dtype, 9100 + DT[dtype])
    xs = oracle.torch_to_storage(x)
    pos = np.array([0, 5, -1, 11, 3, 12, 7, 2, 9], np.int32)
    got = oracle.rope_xpos(xs, dtype, is_key=is_key, pairing=pairing, direction=direction,
                           rotary_dim=R, pos=pos, table_rows=rows, scale_base=scale_base,
                           gamma=gamma, center=center)
    cos, sin = oracle.table(10000.0, R, rows)
    zq, zk = oracle.xpos_table(R, rows, scale_base=scale_base, gamma=gamma, center=center)
    z = zk if is_key else zq
    fmt = dtype
    bits = xs.view(np.uint32) if dtype == "f32" else xs
    gbits = got.view(np.uint32) if dtype == "f32" else got
    for h in range(H):
        for s in range(S):
            p = int(pos[s])
            if p < 0 or p >= rows:
                assert np.array_equal(gbits[0, h, s], bits[0, h, s])
                continue
            for i in range(R // 2):
                j1, j2 = (i, i + R // 2) if pairing == "split_half" else (2 * i, 2 * i + 1)
                x1 = X.value_of(int(bits[0, h, s, j1]), fmt)
                x2 = X.value_of(int(bits[0, h, s, j2]), fmt)
                c, sn = Fraction(float(cos[p, i])), direction * Fraction(float(sin[p, i]))
                f = Fraction(float(z[p, i]))
                for j, y in ((j1, (x1 * c - x2 * sn) * f), (j2, (x1 * sn + x2 * c) * f)):
                    if _near_mid(y, fmt):
                        continue
                    assert int(gbits[0, h, s, j]) == X.bits_of(X.round_ne(y, fmt), fmt), \
                        (h, s, j)
            assert np.array_equal(gbits[0, h, s, R:], bits[0, h, s, R:])


def test_same_position_keeps_the_dot_product(orc):
    rng = np.random.default_rng(5)
    S, D = 40, 64
    q = rng.standard_normal((1, 1, S, D))
    k = rng.standard_normal((1, 1, S, D))
    kw = dict(rotary_dim=D, scale_base=16.0, center=7.0, table_rows=S)
    qx = oracle.rope_xpos_exact(q, is_key=False, **kw)
    kx = oracle.rope_xpos_exact(k, is_key=True, **kw)
    plain = (q * k).sum(-1)
    assert np.allclose((qx * kx).sum(-1), plain, rtol=1e-12, atol=1e-12)
    # while each row on its own is scaled away from its input
    assert not np.allclose(np.abs(qx).sum(-1), np.abs(q).sum(-1), rtol=1e-3)


def test_only_relative_positions_matter(orc):
    rng = np.random.default_rng(6)
    D, n = 32, 12
    q = rng.standard_normal((1, 1, n, D))
    k = rng.standard_normal((1, 1, n, D))
    base = rng.integers(0, 50, n).astype(np.int32)
    kw = dict(rotary_dim=D, scale_base=8.0, gamma=0.4, table_rows=400)

    def scores(shift):
        p = base + shift
        qx = oracle.rope_xpos_exact(q, is_key=False, pos=p, **kw)[0, 0]
        kx = oracle.rope_xpos_exact(k, is_key=True, pos=p[::-1].copy(), **kw)[0, 0]
        return qx @ kx.T

    s0 = scores(0)
    for shift in (1, 37, 250):
        assert np.allclose(scores(shift), s0, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("n,m", [(40, 0), (3, 90), (17, 17)])
def test_one_pair_decays_by_zeta_to_the_distance(orc, n, m):
    # R = 2: one pair, whose product with XPOS is plain RoPE's times
    # zeta_0^((n - m)/B), zeta_0 = gamma / (1 + gamma)
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 1, 2))
    k = rng.standard_normal((1, 1, 1, 2))
    kw = dict(rotary_dim=2, table_rows=100)
    qx = oracle.rope_xpos_exact(q, is_key=False, pos=np.array([n], np.int32), scale_base=8.0,
                                center=5.0, **kw)
    kx = oracle.rope_xpos_exact(k, is_key=True, pos=np.array([m], np.int32), scale_base=8.0,
                                center=5.0, **kw)
    qp = oracle.rope_exact(q, pos=np.array([n], np.int32), **kw)
    kp = oracle.rope_exact(k, pos=np.array([m], np.int32), **kw)
    ratio = (qx * kx).sum() / (qp * kp).sum()
    assert abs(ratio - (0.4 / 1.4) ** ((n - m) / 8.0)) <= 1e-12 * ratio


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_factor_one_is_plain_rope(orc, dtype):
    x = oracle.torch_to_storage(W.normal((2, 3, 10, 64), dtype, 9300))
    pos = np.full(20, 77, np.int32)
    a = oracle.rope_xpos(x, dtype, is_key=True, pos=pos, pos_batch_stride=10, table_rows=100,
                         center=77.0)
    b = oracle.rope(x, dtype, pos=pos, pos_batch_stride=10, table_rows=100)
    assert np.array_equal(a, b)

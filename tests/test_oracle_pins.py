"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself or retypes its formula: each
checks a closed form, a property of rotations, a brute-force consequence, a
special case that reduces to a library routine (numpy / mpmath), or exact
rational arithmetic. Together they are chosen so that a dropped term, a wrong
sign, a wrong pair index, a swapped cos/sin, a wrong frequency exponent or a
wrong position fails at least one of them (tests/test_oracle_mutants.py plants
such mistakes and checks that they are caught).
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import workloads as W
from tests import _exact as X

DTYPES = ("f32", "f16", "bf16")
PAIRINGS = ("split_half", "interleaved")


def _rand_storage(shape, dtype, seed):
    from oracle import torch_to_storage
    return torch_to_storage(W.normal(shape, dtype, seed))


def _as_f64(arr, dtype, orc):
    if dtype == "f32":
        return arr.astype(np.float64)
    if dtype == "bf16":
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.view(np.float16).astype(np.float64)


def _pair_dims(pairing, R, i):
    return (i, i + R // 2) if pairing == "split_half" else (2 * i, 2 * i + 1)


# --------------------------------------------------------------- P1 identity

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("pairing", PAIRINGS)
def test_position_zero_is_identity_bitexact(orc, dtype, pairing):
    """Angle 0 gives cos 1, sin 0: the row is returned bit for bit."""
    x = _rand_storage((2, 3, 5, 32), dtype, 11)
    y = orc.rope(x, dtype, pairing=pairing, pos=np.zeros(5, np.int32), table_rows=8)
    assert np.array_equal(y, x)
    y = orc.rope(x, dtype, pairing=pairing)  # p = s: row s = 0 untouched
    assert np.array_equal(y[:, :, 0], x[:, :, 0])
    assert not np.array_equal(y[:, :, 1], x[:, :, 1])


# ------------------------------------------------- P2 unit vectors / tables

def test_freq_closed_forms(orc):
    """freq_0 = 1 for any base; the last frequency of R=64, theta=1e4 is
    10^(-4*62/64) = 10^-3.875; R=2 has only freq_0."""
    for theta in (10000.0, 500000.0, 2.5):
        assert orc.freq(theta, 64, 0) == 1.0
    assert orc.freq(10000.0, 64, 31) == pytest.approx(10 ** -3.875, rel=2e-16)
    assert orc.freq(10000.0, 64, 31) == pytest.approx(1.333521432163324e-4, rel=1e-15)
    assert orc.freq(10000.0, 4, 1) == pytest.approx(0.01, rel=1e-16)
    assert orc.freq(500000.0, 128, 32) == pytest.approx(500000.0 ** -0.5, rel=1e-16)


def test_freq_matches_high_precision_power(orc):
    rng = np.random.default_rng(3)
    for _ in range(300):
        R = int(rng.choice([2, 8, 32, 64, 96, 128, 256]))
        theta = float(rng.choice([10000.0, 500000.0, 1e6, 12.5]))
        i = int(rng.integers(0, R // 2))
        expo = -(2.0 * i) / R  # the binary64 exponent of the definition
        with mpmath.workdps(50):
            ref = mpmath.power(mpmath.mpf(theta), mpmath.mpf(expo))
        got = orc.freq(theta, R, i)
        assert abs(got - float(ref)) <= abs(float(ref)) * 2.0 ** -52


def test_table_column0_known_values(orc):
    """Column 0 has freq 1, so row p holds RN32(cos p), RN32(sin p)."""
    c, s = orc.table(10000.0, 64, 4)
    assert c[0, 0] == np.float32(1.0) and s[0, 0] == np.float32(0.0)
    assert c[1, 0] == np.float32(0.5403023058681398)  # cos 1
    assert s[1, 0] == np.float32(0.8414709848078965)  # sin 1
    assert c[2, 0] == np.float32(-0.4161468365471424)  # cos 2
    assert s[3, 0] == np.float32(0.1411200080598672)  # sin 3
    rows = 4096
    c, s = orc.table(500000.0, 128, rows)
    p = np.arange(rows, dtype=np.float64)
    assert np.array_equal(c[:, 0], np.cos(p).astype(np.float32))
    assert np.array_equal(s[:, 0], np.sin(p).astype(np.float32))
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)


def test_table_matches_mpmath(orc):
    """Entries equal cos/sin of the binary64 angle rounded once to float32,
    computed in 60-digit arithmetic; any difference must be a float32 midpoint
    case that binary64 cannot resolve."""
    rng = np.random.default_rng(5)
    for theta, R, rows in ((10000.0, 128, 4096), (500000.0, 128, 131072),
                           (10000.0, 32, 9216)):
        c, s = orc.table(theta, R, rows)
        for _ in range(400):
            p = int(rng.integers(0, rows))
            i = int(rng.integers(0, R // 2))
            angle = float(p) * orc.freq(theta, R, i)  # the binary64 angle
            with mpmath.workdps(60):
                a = mpmath.mpf(angle)
                mc, ms = mpmath.cos(a), mpmath.sin(a)
            for got, ref in ((c[p, i], mc), (s[p, i], ms)):
                if float(got) != X.rn24_mp(ref):
                    assert X.near_f32_midpoint(ref), (theta, R, p, i, got, ref)


@pytest.mark.parametrize("pairing", PAIRINGS)
def test_unit_vectors_give_cos_and_sin(orc, pairing):
    """(1,0) -> (c, s) and (0,1) -> (-s, c) for every pair: fixes the rotation
    direction, which pair dims belong together, and that cos/sin are not
    swapped; backward gives (c, -s) and (s, c)."""
    R, D, rows, theta = 16, 24, 50, 10000.0
    c, s = orc.table(theta, R, rows)
    p = 37
    for i in range(R // 2):
        j1, j2 = _pair_dims(pairing, R, i)
        for direction in (1, -1):
            e1 = np.zeros((1, 1, 1, D), np.float32)
            e1[..., j1] = 1.0
            e2 = np.zeros((1, 1, 1, D), np.float32)
            e2[..., j2] = 1.0
            pos = np.array([p], np.int32)
            y1 = orc.rope(e1, "f32", pairing=pairing, direction=direction, rotary_dim=R,
                          pos=pos, table_rows=rows, theta=theta)[0, 0, 0]
            y2 = orc.rope(e2, "f32", pairing=pairing, direction=direction, rotary_dim=R,
                          pos=pos, table_rows=rows, theta=theta)[0, 0, 0]
            sg = np.float32(direction)
            assert y1[j1] == c[p, i] and y1[j2] == sg * s[p, i]
            assert y2[j1] == -sg * s[p, i] and y2[j2] == c[p, i]
            others = [j for j in range(D) if j not in (j1, j2)]
            assert np.all(y1[others] == 0) and np.all(y2[others] == 0)


# ------------------------------------------------- P3-P5 rotation properties

@pytest.mark.parametrize("pairing", PAIRINGS)
def test_pair_norms_preserved(orc, pairing):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 3, 40, 32))
    y = orc.rope_exact(x, pairing=pairing, theta=500000.0)
    R = 32
    for i in range(R // 2):
        j1, j2 = _pair_dims(pairing, R, i)
        n0 = x[..., j1] ** 2 + x[..., j2] ** 2
        n1 = y[..., j1] ** 2 + y[..., j2] ** 2
        np.testing.assert_allclose(n1, n0, rtol=1e-12)


@pytest.mark.parametrize("pairing", PAIRINGS)
@pytest.mark.parametrize("layout", ("bhsd", "bshd"))
def test_backward_inverts_forward(orc, pairing, layout):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 33, 3, 48) if layout == "bshd" else (2, 3, 33, 48))
    kw = dict(pairing=pairing, layout=layout, rotary_dim=32, theta=10000.0)
    y = orc.rope_exact(orc.rope_exact(x, direction=1, **kw), direction=-1, **kw)
    np.testing.assert_allclose(y, x, rtol=0, atol=1e-12)
    # table mode in fp32: each rotation errs by ~1 float32 ulp
    x32 = x.astype(np.float32)
    y32 = orc.rope(orc.rope(x32, "f32", direction=1, **kw), "f32", direction=-1, **kw)
    assert np.max(np.abs(y32 - x32)) <= 4e-6 * max(1.0, np.max(np.abs(x32)))


def test_backward_is_the_adjoint(orc):
    """<fwd(x), g> = <x, bwd(g)>: backward is the transpose of forward."""
    rng = np.random.default_rng(9)
    for pairing in PAIRINGS:
        x = rng.standard_normal((2, 4, 17, 32))
        g = rng.standard_normal((2, 4, 17, 32))
        kw = dict(pairing=pairing, rotary_dim=24, theta=10000.0)
        lhs = np.sum(orc.rope_exact(x, direction=1, **kw) * g)
        rhs = np.sum(x * orc.rope_exact(g, direction=-1, **kw))
        assert lhs == pytest.approx(rhs, rel=1e-12)


def test_positions_compose(orc):
    """Rotating by position m then by n equals rotating by m + n."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1, 2, 12, 16))
    m = rng.integers(0, 500, 12).astype(np.int32)
    n = rng.integers(0, 500, 12).astype(np.int32)
    kw = dict(theta=10000.0, table_rows=2000)
    y = orc.rope_exact(orc.rope_exact(x, pos=m, **kw), pos=n, **kw)
    z = orc.rope_exact(x, pos=(m + n).astype(np.int32), **kw)
    np.testing.assert_allclose(y, z, rtol=0, atol=1e-9)


def test_linear_in_the_input(orc):
    rng = np.random.default_rng(12)
    x, z = rng.standard_normal((2, 1, 2, 9, 16))
    a, b = 0.75, -2.5
    kw = dict(theta=10000.0, pairing="interleaved")
    lhs = orc.rope_exact(a * x + b * z, **kw)
    rhs = a * orc.rope_exact(x, **kw) + b * orc.rope_exact(z, **kw)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


# ------------------------------------- P6 relative position, brute force

@pytest.mark.parametrize("pairing", PAIRINGS)
def test_dot_product_depends_only_on_offset(orc, pairing):
    """<rope(q, m), rope(k, n)> equals
       sum_i (q1 k1 + q2 k2) cos((n-m) f_i) + (q2 k1 - q1 k2) sin((n-m) f_i)
    for all m, n in [0, 32) -- the relative-position property that motivates
    rotating both queries and keys."""
    R, N, theta = 16, 32, 100.0
    rng = np.random.default_rng(13)
    q = rng.standard_normal(R)
    k = rng.standard_normal(R)
    Q = np.broadcast_to(q, (1, 1, N, R)).copy()
    K = np.broadcast_to(k, (1, 1, N, R)).copy()
    rq = orc.rope_exact(Q, pairing=pairing, theta=theta)[0, 0]
    rk = orc.rope_exact(K, pairing=pairing, theta=theta)[0, 0]
    dots = rq @ rk.T  # [m, n]
    f = theta ** (-(2.0 * np.arange(R // 2)) / R)
    j1, j2 = zip(*[_pair_dims(pairing, R, i) for i in range(R // 2)])
    q1, q2, k1, k2 = q[list(j1)], q[list(j2)], k[list(j1)], k[list(j2)]
    for m in range(N):
        for n in range(N):
            d = (n - m) * f
            ref = np.sum((q1 * k1 + q2 * k2) * np.cos(d) + (q2 * k1 - q1 * k2) * np.sin(d))
            assert dots[m, n] == pytest.approx(ref, abs=1e-12 * R)


# --------------------------------------------------- P7 pairing permutation

@pytest.mark.parametrize("dtype", DTYPES)
def test_interleaved_is_permuted_split_half(orc, dtype):
    """With P mapping dim i -> 2i and i + R/2 -> 2i + 1 (dims >= R fixed),
    interleaved(P x) == P split_half(x), bit for bit."""
    R, D = 32, 40
    x = _rand_storage((2, 3, 21, D), dtype, 14)
    perm = np.arange(D)
    for i in range(R // 2):
        perm[2 * i] = i
        perm[2 * i + 1] = i + R // 2
    kw = dict(rotary_dim=R, theta=10000.0)
    a = orc.rope(x[..., perm], dtype, pairing="interleaved", **kw)
    b = orc.rope(x, dtype, pairing="split_half", **kw)[..., perm]
    assert np.array_equal(a, b)


# ------------------------------------------------------ P8 index semantics

@pytest.mark.parametrize("dtype", DTYPES)
def test_index_path_equals_gather(orc, dtype):
    """Token s with index p gets exactly what a token sitting at position p
    gets without indices; an index arange(S) is the same as no index."""
    B, H, S, D, rows = 2, 2, 9, 16, 64
    x = _rand_storage((B, H, S, D), dtype, 15)
    pos = W.random_positions(S, rows, 16).numpy()
    y = orc.rope(x, dtype, pos=pos, table_rows=rows)
    for s in range(S):
        p = int(pos[s])
        z = np.zeros((B, H, p + 1, D), x.dtype)
        z[:, :, p] = x[:, :, s]
        ref = orc.rope(z, dtype, table_rows=rows)[:, :, p]
        assert np.array_equal(y[:, :, s], ref)
    same = orc.rope(x, dtype, pos=np.arange(S, dtype=np.int32), table_rows=rows)
    assert np.array_equal(same, orc.rope(x, dtype, table_rows=rows))


def test_index_batch_stride(orc):
    """pos[b * stride + s]: a [B, S] index equals one call per sequence."""
    B, H, S, D, rows = 3, 2, 5, 16, 100
    x = _rand_storage((B, H, S, D), "bf16", 17)
    pos = W.random_positions(B * S, rows, 18).numpy()
    y = orc.rope(x, "bf16", pos=pos, pos_batch_stride=S, table_rows=rows)
    for b in range(B):
        ref = orc.rope(x[b:b + 1], "bf16", pos=pos[b * S:(b + 1) * S], table_rows=rows)
        assert np.array_equal(y[b:b + 1], ref)
    # stride 0: every sequence shares one index row
    y0 = orc.rope(x, "bf16", pos=pos[:S], pos_batch_stride=0, table_rows=rows)
    for b in range(B):
        ref = orc.rope(x[b:b + 1], "bf16", pos=pos[:S], table_rows=rows)
        assert np.array_equal(y0[b:b + 1], ref)


def test_layouts_are_transposes(orc):
    """[B,S,H,D] results are the [B,H,S,D] results transposed."""
    x = _rand_storage((2, 3, 11, 32), "f16", 19)
    a = orc.rope(x, "f16", layout="bhsd", pairing="interleaved")
    b = orc.rope(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), "f16", layout="bshd",
                 pairing="interleaved")
    assert np.array_equal(a, b.transpose(0, 2, 1, 3))


# ------------------------------------------------------ P9 pass-through

@pytest.mark.parametrize("dtype", DTYPES)
def test_pass_through_lanes_bitexact(orc, dtype):
    """Dims >= R and tokens with index < 0 or >= table_rows keep their bits,
    even when they hold NaN or Inf."""
    B, H, S, D, R, rows = 2, 3, 7, 64, 32, 50
    x = _rand_storage((B, H, S, D), dtype, 20)
    specials = {"f32": np.array([np.nan, np.inf, -np.inf, -0.0], np.float32).view(np.uint32),
                "f16": np.array([0x7e01, 0x7c00, 0xfc00, 0x8000], np.uint16),
                "bf16": np.array([0x7fc1, 0x7f80, 0xff80, 0x8000], np.uint16)}[dtype]
    xs = x.view(np.uint32) if dtype == "f32" else x
    xs[..., R:R + 4] = specials
    xs[:, :, 1, :4] = specials  # a masked token
    pos = np.array([3, -1, 49, 50, 1 << 30, -7, 0], np.int32)
    y = orc.rope(x, dtype, rotary_dim=R, pos=pos, table_rows=rows)
    v = (lambda a: a.view(np.uint32)) if dtype == "f32" else (lambda a: a)
    assert np.array_equal(v(y)[..., R:], v(x)[..., R:])
    for s in (1, 3, 4, 5):  # masked: negative or beyond the table
        assert np.array_equal(v(y)[:, :, s], v(x)[:, :, s])
    assert np.array_equal(v(y)[:, :, 6], v(x)[:, :, 6])  # position 0
    assert not np.array_equal(v(y)[:, :, 0, :R], v(x)[:, :, 0, :R])


# ---------------------------------------------- conversions and rounding

def test_rounding_matches_exact_rationals(orc):
    """binary64 -> f16 / bf16 bits equals exact rational round-to-nearest-even,
    over normal, subnormal, midpoint and overflow cases."""
    rng = np.random.default_rng(21)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-30, 20, 3000)))
    vals += list(rng.standard_normal(500) * 2.0 ** -130)  # bf16 subnormals
    vals += [65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -25, 2.0 ** -24 * 1.5,
             3.0 * 2.0 ** -26, -(2.0 ** -25) * 1.0000001, 1.0 + 2.0 ** -11,
             1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3.4e38, 3.39e38,
             2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -133, 0.0, -0.0]
    for v in vals:
        for fmt in ("f16", "bf16"):
            ref = X.round_ne(Fraction(v), fmt)
            if ref == 0.0 and np.signbit(v):
                ref = -0.0
            assert orc.to_bits(float(v), fmt) == X.bits_of(ref, fmt), (v, fmt)
    # numpy's double -> half conversion is a second, correctly rounded reference
    arr = np.array(vals[:3000])
    ref16 = arr.astype(np.float16).view(np.uint16)
    assert all(orc.to_bits(float(v), "f16") == int(r) for v, r in zip(arr, ref16))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("pairing", PAIRINGS)
def test_outputs_are_exact_rotation_rounded_once(orc, dtype, pairing):
    """Each output equals RNE_dtype(x1*c32 -+ x2*s32) computed in exact
    rational arithmetic from the float32 table entries, for both directions.
    Inputs are scaled so fp16 subnormals and overflow both occur."""
    R, D, rows, theta = 32, 32, 300, 10000.0
    x = _rand_storage((1, 2, 24, D), "f32", 22) * np.float32(1.0)
    scale = np.float32(1e-6) if dtype == "f16" else np.float32(1.0)
    x[0, 0] *= scale
    if dtype == "f16":
        # finite inputs near the top of the range, so some outputs overflow
        x[0, 1, :4] = np.clip(x[0, 1, :4] * np.float32(40000.0), -65000.0, 65000.0)
    import torch
    xs = {"f32": x, "f16": x.astype(np.float16).view(np.uint16),
          "bf16": torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
          .view(np.uint16)}[dtype]
    pos = W.random_positions(24, rows, 23).numpy()
    c, s = orc.table(theta, R, rows)
    xv = _as_f64(xs, dtype, orc)
    for direction in (1, -1):
        y = orc.rope(xs, dtype, pairing=pairing, direction=direction, rotary_dim=R,
                     pos=pos, table_rows=rows, theta=theta)
        ybits = y.view(np.uint32) if dtype == "f32" else y
        for h in range(2):
            for t in range(24):
                p = int(pos[t])
                for i in range(R // 2):
                    j1, j2 = _pair_dims(pairing, R, i)
                    x1, x2 = Fraction(xv[0, h, t, j1]), Fraction(xv[0, h, t, j2])
                    cc, ss = Fraction(float(c[p, i])), Fraction(float(s[p, i])) * direction
                    e1 = X.round_ne(x1 * cc - x2 * ss, dtype)
                    e2 = X.round_ne(x1 * ss + x2 * cc, dtype)
                    for got, ref, exact in ((ybits[0, h, t, j1], e1, x1 * cc - x2 * ss),
                                            (ybits[0, h, t, j2], e2, x1 * ss + x2 * cc)):
                        if ref == 0.0 and exact < 0:
                            ref = -0.0
                        assert int(got) == X.bits_of(ref, dtype), (h, t, i, direction)


# --------------------------------------- the pages' own examples, as inputs

def test_cls_register_tokens_skipped_with_partial_rotary(orc):
    """rotary-embedding-torch docs, flash_attn_with_rotary example: q of shape
    (1, 8, 1024 + 2, 64), rotary dim 32, the 2 leading tokens not rotated; the
    other 1024 tokens sit at positions 0..1023."""
    S, D, R = 1026, 64, 32
    x = _rand_storage((1, 8, S, D), "bf16", 24)
    pos = np.concatenate([[-1, -1], np.arange(1024)]).astype(np.int32)
    y = orc.rope(x, "bf16", rotary_dim=R, pos=pos, table_rows=1024)
    assert np.array_equal(y[:, :, :2], x[:, :, :2])
    assert np.array_equal(y[..., R:], x[..., R:])
    assert np.array_equal(y[:, :, 2], x[:, :, 2])  # position 0
    # the rotated part equals the plain (index-free) call on tokens 2..1025
    ref = orc.rope(np.ascontiguousarray(x[:, :, 2:]), "bf16", rotary_dim=R,
                   table_rows=1024)
    assert np.array_equal(y[:, :, 2:], ref)


def test_prefix_offset_positions(orc):
    """Unsloth page, Custom Position IDs for Prefix-Tuning: positions
    arange(seq_len) + prefix_len rotate token s like token s + prefix_len of
    a longer sequence."""
    S, prefix = 40, 13
    x = _rand_storage((1, 4, S, 64), "f16", 25)
    y = orc.rope(x, "f16", pos=np.arange(S, dtype=np.int32) + prefix,
                 table_rows=S + prefix)
    big = np.zeros((1, 4, S + prefix, 64), np.uint16)
    big[:, :, prefix:] = x
    ref = orc.rope(big, "f16")[:, :, prefix:]
    assert np.array_equal(y, ref)


def test_rejects_bad_arguments(orc):
    x = np.zeros((1, 1, 4, 8), np.float32)
    with pytest.raises(orc.OracleError):
        orc.rope(x, "f32", rotary_dim=10)  # R > D
    with pytest.raises(orc.OracleError):
        orc.rope(x, "f32", rotary_dim=3)  # odd R
    with pytest.raises(orc.OracleError):
        orc.rope(x, "f32", table_rows=2)  # S > table rows without an index


# ---------------------------------------------------------------- interpolate_factor
# rotary-embedding-torch docs, Key Parameters: `interpolate_factor` scales the
# sequence positions (default 1.0). Read as a divisor: angle = (p / s) * freq_i.

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_interpolate_factor_one_is_no_scaling(orc, dtype):
    w = W.TINY_F32.scaled(dtype=dtype)
    x = W.tensors(w)["q"]
    from tests import _parity as P
    xs = P.storage(x)
    assert np.array_equal(orc.rope(xs, dtype, theta=w.theta),
                          orc.rope(xs, dtype, theta=w.theta, interpolate_factor=1.0))


@pytest.mark.parametrize("s,scale", [(2.0, 2), (4.0, 4), (0.5, None)])
def test_interpolate_factor_divides_positions(orc, s, scale):
    """With factor s, position p rotates as position p / s does with factor 1,
    bit for bit when p / s is exact: s = 2 at 2q equals 1 at q, and s = 1/2
    at q equals 1 at 2q."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((1, 3, 17, 32)).astype(np.float32)
    q = rng.integers(0, 3000, 17).astype(np.int32)
    kw = dict(theta=10000.0, table_rows=20000)
    if scale is not None:
        got = orc.rope(x, "f32", pos=(q * scale).astype(np.int32), interpolate_factor=s, **kw)
        ref = orc.rope(x, "f32", pos=q, **kw)
    else:
        got = orc.rope(x, "f32", pos=q, interpolate_factor=s, **kw)
        ref = orc.rope(x, "f32", pos=(2 * q).astype(np.int32), **kw)
    assert np.array_equal(got, ref)


def test_interpolated_table_matches_mpmath(orc):
    """A non-dyadic factor: entries equal cos/sin of (p / 3) * freq_i in
    binary64, evaluated in 60-digit arithmetic and rounded once to float32."""
    rng = np.random.default_rng(43)
    theta, R, rows, s = 10000.0, 64, 5000, 3.0
    c, sn = orc.table(theta, R, rows, interpolate_factor=s)
    c1, _ = orc.table(theta, R, rows)
    assert not np.array_equal(c, c1)
    for _ in range(300):
        p = int(rng.integers(0, rows))
        i = int(rng.integers(0, R // 2))
        angle = (float(p) / s) * orc.freq(theta, R, i)  # the binary64 angle
        with mpmath.workdps(60):
            a = mpmath.mpf(angle)
            mc, ms = mpmath.cos(a), mpmath.sin(a)
        for got, ref in ((c[p, i], mc), (sn[p, i], ms)):
            if float(got) != X.rn24_mp(ref):
                assert X.near_f32_midpoint(ref), (p, i, got, ref)


def test_exact_mode_interpolation_composes(orc):
    """Exact mode with factor s at positions m equals factor 1 at the real
    positions m / s (checked through composition: s = 4, positions 4q)."""
    rng = np.random.default_rng(45)
    x = rng.standard_normal((1, 2, 9, 16))
    q = rng.integers(0, 800, 9).astype(np.int32)
    kw = dict(theta=10000.0, table_rows=5000)
    y = orc.rope_exact(x, pos=(4 * q).astype(np.int32), interpolate_factor=4.0, **kw)
    z = orc.rope_exact(x, pos=q, **kw)
    np.testing.assert_allclose(y, z, rtol=0, atol=1e-12)


def test_rejects_bad_interpolate_factor(orc):
    x = np.zeros((1, 1, 4, 8), np.float32)
    for s in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(orc.OracleError):
            orc.rope(x, "f32", interpolate_factor=s)

"""Pins of the oracle's RoPE attention (rotary-embedding-torch docs,
flash_attn_with_rotary): the closed forms and invariants that softmax
attention over rotated Q and K must satisfy, chosen so that a plausible
slip (a dropped scale, a causal off-by-one, a wrong GQA head map, K left
unrotated, V swapped for K) fails at least one."""
import numpy as np
import pytest

DT = "f32"


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def test_single_key_returns_its_value(orc):
    """softmax over one key is 1: the output is that key's V row, exactly."""
    rng = np.random.default_rng(101)
    q, k, v = _rand(rng, 2, 3, 5, 16), _rand(rng, 2, 3, 1, 16), _rand(rng, 2, 3, 1, 16)
    o = orc.rope_attention(q, k, v, DT, table_rows=8)
    assert np.array_equal(o, np.broadcast_to(v.astype(np.float64), o.shape))


def test_identical_keys_average_the_values(orc):
    """Equal keys at the same position score equally: the output is the mean
    of V (rotation cannot break the tie)."""
    rng = np.random.default_rng(102)
    q, v = _rand(rng, 1, 2, 4, 16), _rand(rng, 1, 2, 7, 16)
    k = np.broadcast_to(_rand(rng, 1, 2, 1, 16), (1, 2, 7, 16)).copy()
    kpos = np.zeros(7, np.int32)
    o = orc.rope_attention(q, k, v, DT, kpos=kpos, table_rows=8)
    np.testing.assert_allclose(o, np.broadcast_to(v.astype(np.float64).mean(2, keepdims=True), o.shape),
                               rtol=0, atol=1e-12)


def test_zero_scale_causal_is_the_prefix_mean(orc):
    rng = np.random.default_rng(103)
    q, k, v = _rand(rng, 1, 1, 6, 8), _rand(rng, 1, 1, 6, 8), _rand(rng, 1, 1, 6, 8)
    o = orc.rope_attention(q, k, v, DT, causal=True, scale=0.0)
    ref = np.cumsum(v.astype(np.float64), 2) / np.arange(1, 7)[None, None, :, None]
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("sq,sk", [(9, 9), (3, 9)])
def test_causal_equals_visible_prefix(orc, sq, sk):
    """Query i sees keys 0 .. i + Sk - Sq: it equals non-causal attention over
    exactly that prefix, with the same query position, bit for bit."""
    rng = np.random.default_rng(104)
    q, k, v = _rand(rng, 1, 2, sq, 16), _rand(rng, 1, 2, sk, 16), _rand(rng, 1, 2, sk, 16)
    o = orc.rope_attention(q, k, v, DT, causal=True, table_rows=sk)
    for i in range(sq):
        last = i + sk - sq
        oi = orc.rope_attention(q[:, :, i:i + 1], k[:, :, :last + 1], v[:, :, :last + 1], DT,
                                qpos=np.array([last], np.int32), table_rows=sk)
        assert np.array_equal(o[:, :, i:i + 1], oi), i


def test_gqa_equals_repeated_kv_heads(orc):
    """Query head h reads K/V head h / (Hq / Hk)."""
    rng = np.random.default_rng(105)
    q, k, v = _rand(rng, 2, 4, 5, 16), _rand(rng, 2, 2, 5, 16), _rand(rng, 2, 2, 5, 16)
    o = orc.rope_attention(q, k, v, DT, causal=True)
    rep = [0, 0, 1, 1]
    o_rep = orc.rope_attention(q, k[:, rep], v[:, rep], DT, causal=True)
    assert np.array_equal(o, o_rep)


def test_key_permutation_invariance(orc):
    """Non-causal attention is a sum over keys: permuting the keys together
    with their positions and values leaves the output unchanged."""
    rng = np.random.default_rng(106)
    q, k, v = _rand(rng, 1, 2, 4, 16), _rand(rng, 1, 2, 10, 16), _rand(rng, 1, 2, 10, 16)
    perm = rng.permutation(10)
    o = orc.rope_attention(q, k, v, DT, kpos=np.arange(10, dtype=np.int32), table_rows=16)
    op = orc.rope_attention(q, k[:, :, perm], v[:, :, perm], DT,
                            kpos=perm.astype(np.int32), table_rows=16)
    np.testing.assert_allclose(o, op, rtol=0, atol=1e-12)


@pytest.mark.parametrize("pairing", ["split_half", "interleaved"])
def test_scores_depend_on_relative_position(orc, pairing):
    """RoPE makes q(m).k(n) a function of m - n: shifting every query and key
    position by the same amount leaves the attention output unchanged (up to
    the float32 rounding of the tables and of the rotated Q and K). This
    fixes that both Q and K are rotated, and in the same sense."""
    rng = np.random.default_rng(107)
    q, k, v = _rand(rng, 1, 2, 6, 32), _rand(rng, 1, 2, 9, 32), _rand(rng, 1, 2, 9, 32)
    qp, kp = rng.integers(0, 50, 6).astype(np.int32), rng.integers(0, 50, 9).astype(np.int32)
    kw = dict(pairing=pairing, table_rows=2000)
    o = orc.rope_attention(q, k, v, DT, qpos=qp, kpos=kp, **kw)
    o2 = orc.rope_attention(q, k, v, DT, qpos=qp + 1234, kpos=kp + 1234, **kw)
    np.testing.assert_allclose(o, o2, rtol=0, atol=2e-4)
    # and the positions do matter: a shift of the keys alone changes it
    o3 = orc.rope_attention(q, k, v, DT, qpos=qp, kpos=kp + 7, **kw)
    assert np.abs(o - o3).max() > 1e-2


def test_rejects_bad_arguments(orc):
    z = np.zeros((1, 3, 4, 8), np.float32)
    with pytest.raises(orc.OracleError):
        orc.rope_attention(z, z[:, :2], z[:, :2], DT)  # Hq not a multiple of Hk
    with pytest.raises(orc.OracleError):
        orc.rope_attention(z, z[:, :, :2], z[:, :, :2], DT, causal=True)  # Sq > Sk

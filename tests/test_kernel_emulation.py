"""librope's kernels run on the host, under AddressSanitizer, against the oracle.

tests/emu/rope_emu.hip plans each call exactly as the library does and runs
every workgroup and lane of the planned grid on host buffers of exact size.
This checks, on the CPU and before any GPU run, that the index arithmetic
of both grid shapes stays in bounds for every access width, pairing, layout
and ragged size below, touches each element once, and computes what the
oracle computes (same tolerances as the GPU parity tests).
"""
import os
import fcntl
import struct
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import rotary_position_embedding_fwd_amd as rp
import workloads as W
from tests import _exact as X
from tests import _parity as P
from tests._random_configs import draw as draw_config, workload as config_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EMU_SRC = os.path.join(ROOT, "tests", "emu", "rope_emu.hip")
EMU_BIN = os.path.join(ROOT, "tests", "emu", "_build", "rope_emu")
CSRC = os.path.join(ROOT, "rotary_position_embedding_fwd_amd", "csrc")
DEPS = [EMU_SRC, os.path.join(CSRC, "rope_kernels.hpp"), os.path.join(CSRC, "rope_plan.hpp"),
        os.path.join(ROOT, "include", "librope.h")]

CODES = {"dtype": {"f32": 0, "f16": 1, "bf16": 2}, "layout": {"bhsd": 0, "bshd": 1},
         "pairing": {"split_half": 0, "interleaved": 1},
         "launch": {"auto": 0, "rows": 1, "token": 2}}


def _emu_stale():
    return (not os.path.exists(EMU_BIN) or
            os.path.getmtime(EMU_BIN) < max(os.path.getmtime(p) for p in DEPS))


@pytest.fixture(scope="module")
def emu():
    # several pytest-xdist workers may get here at once: build under a lock,
    # into a private file that is renamed into place when complete
    os.makedirs(os.path.dirname(EMU_BIN), exist_ok=True)
    with open(EMU_BIN + ".lock", "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        if _emu_stale():
            tmp = f"{EMU_BIN}.{os.getpid()}"
            cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-host-only", "-O1",
                   "-g", "-std=c++17", "-ffp-contract=off", "-Xarch_host", "-fsanitize=address",
                   "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
                   "-o", tmp, EMU_SRC]
            subprocess.run(cmd, check=True, capture_output=True)
            os.replace(tmp, EMU_BIN)
    return EMU_BIN


def run_emu(emu, w, q, k, cos, sin, pos, direction=1, launch="auto", with_k=True,
            q_offset=0, k_offset=0, cus=256, pos_batch_stride=None, overrides=None):
    with tempfile.TemporaryDirectory() as job:
        desc = dict(batch=w.batch, n_heads_q=w.n_heads_q, n_heads_k=w.n_heads_k,
                    seq_len=w.seq_len, head_dim=w.head_dim, rotary_dim=w.rotary_dim,
                    dtype=CODES["dtype"][w.dtype], layout=CODES["layout"][w.layout],
                    pairing=CODES["pairing"][w.pairing], launch=CODES["launch"][launch],
                    table_rows=cos.shape[0],
                    pos_batch_stride=(w.pos_batch_stride if pos_batch_stride is None
                                      else pos_batch_stride),
                    with_k=int(with_k), direction=direction, cus=cus, q_offset=q_offset,
                    k_offset=k_offset, pos_count=0 if pos is None else pos.numel())
        desc.update(overrides or {})
        with open(os.path.join(job, "desc.txt"), "w") as f:
            for key, v in desc.items():
                f.write(f"{key} {int(v)}\n")
        P.storage(q).tofile(os.path.join(job, "q.bin"))
        if with_k:
            P.storage(k).tofile(os.path.join(job, "k.bin"))
        cos.numpy().tofile(os.path.join(job, "cos.bin"))
        sin.numpy().tofile(os.path.join(job, "sin.bin"))
        if pos is not None:
            pos.numpy().astype(np.int32).tofile(os.path.join(job, "pos.bin"))
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
        r = subprocess.run([emu, job], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stdout + r.stderr[-4000:]
        plan = dict(line.split() for line in r.stdout.strip().splitlines())
        plan = {key: int(v) for key, v in plan.items()}
        if plan["status"] != 0:
            return plan, None, None
        st = P.storage(q)
        qo = np.fromfile(os.path.join(job, "q_out.bin"), dtype=st.dtype).reshape(st.shape)
        ko = None
        if with_k:
            sk = P.storage(k)
            ko = np.fromfile(os.path.join(job, "k_out.bin"), dtype=sk.dtype).reshape(sk.shape)
        return plan, qo, ko


def _inputs(w, seed_shift=0):
    t = W.tensors(w, ("q", "k"))
    pos = W.positions(w)
    cos, sin = rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta)
    return t["q"], t["k"], pos, cos, sin


def check(emu, w, direction=1, launch="auto", with_k=True, q_offset=0, k_offset=0, cus=256,
          pos=None, use_workload_pos=True, expect=None, overrides=None):
    q, k, wpos, cos, sin = _inputs(w)
    if use_workload_pos:
        pos = wpos
    plan, qo, ko = run_emu(emu, w, q, k, cos, sin, pos, direction, launch, with_k, q_offset,
                           k_offset, cus, overrides=overrides)
    assert plan["status"] == 0, plan
    for key, v in (expect or {}).items():
        assert plan[key] == v, (key, plan)
    masked = P.masked_tokens(w, pos)
    P.assert_parity(qo, P.oracle_rope(w, q, direction, pos), P.storage(q), w.dtype, w.layout,
                    w.rotary_dim, masked, "q")
    if with_k:
        P.assert_parity(ko, P.oracle_rope(w, k, direction, pos), P.storage(k), w.dtype,
                        w.layout, w.rotary_dim, masked, "k")
    return plan


SMALL = {
    "tiny_fp32": W.TINY_F32,
    "llama_ragged": W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=77, table_rows=80),
    "bshd_interleaved_ragged": W.BSHD_INTERLEAVED.scaled(batch=3, seq_len=45, table_rows=45),
    "partial_indexed": W.PARTIAL_INDEXED.scaled(seq_len=130, pos_start_max=9000),
    "decode": W.DECODE.scaled(batch=19),
    "long_theta": W.LONG_CONTEXT.scaled(seq_len=64, table_rows=131072),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("direction", [1, -1])
def test_emulated_workloads_match_oracle(emu, name, direction):
    check(emu, SMALL[name], direction)


@pytest.mark.parametrize("name", ["llama_ragged", "bshd_interleaved_ragged", "partial_indexed",
                                  "decode", "tiny_fp32"])
@pytest.mark.parametrize("launch", ["rows", "token"])
def test_both_grid_shapes(emu, name, launch):
    check(emu, SMALL[name], 1, launch, expect={"token": int(launch == "token")})


def test_auto_shape_selection(emu):
    """Decode, views whose heads of a token are adjacent ([B,S,H,D]), and
    [B,H,S,D] prefill too small to fill the chip with the rows shape even at
    one head per lane, take the token shape; otherwise rows."""
    assert check(emu, SMALL["decode"])["token"] == 1
    assert check(emu, SMALL["decode"], cus=1)["token"] == 1
    assert check(emu, SMALL["llama_ragged"])["token"] == 1  # 154 tokens on 256 CUs
    plan = check(emu, SMALL["llama_ragged"], cus=1)  # same tokens, a 1-CU device
    assert plan["token"] == 0 and plan["group_slow"] == 1 and plan["head_lanes"] == 1
    plan = check(emu, SMALL["llama_ragged"], launch="rows", cus=1)
    assert plan["token"] == 0 and plan["group_slow"] == 1 and plan["heads_per_group"] == 4
    # the same tokens as [B,S,H,D]: token shape on any device
    assert check(emu, SMALL["llama_ragged"].scaled(layout="bshd"), cus=1)["token"] == 1
    assert check(emu, SMALL["bshd_interleaved_ragged"], cus=1)["token"] == 1
    # one Q head: [B,S,1,D] is [B,1,S,D]; rows on a device it fills
    plan = check(emu, SMALL["llama_ragged"].scaled(layout="bshd", n_heads_q=1, n_heads_k=1),
                 cus=1)
    assert plan["token"] == 0


@pytest.mark.parametrize("cus", [1, 7, 256, 1000])
def test_grid_heuristic_any_cu_count(emu, cus):
    """Head grouping depends on the CU count; every choice must cover all work."""
    check(emu, SMALL["llama_ragged"], 1, cus=cus)


@pytest.mark.parametrize("name", ["llama_ragged", "bshd_interleaved_ragged", "partial_indexed"])
@pytest.mark.parametrize("group_slow", [0, 1])
@pytest.mark.parametrize("heads_per_group", [1, 3, 8, 100])
def test_head_groups_in_either_order(emu, name, group_slow, heads_per_group):
    """Every head-group size and both workgroup orders cover all rows once."""
    plan = check(emu, SMALL[name], 1, "rows",
                 overrides=dict(heads_per_group=heads_per_group, group_slow=group_slow))
    assert plan["group_slow"] == group_slow


def test_q_only(emu):
    check(emu, SMALL["llama_ragged"], 1, with_k=False)
    check(emu, SMALL["decode"], -1, with_k=False)


@pytest.mark.parametrize("q_off,k_off,vec", [(1, 0, 1), (2, 0, 2), (4, 4, 4), (0, 6, 2),
                                             (8, 8, 8)])
def test_misaligned_bases_use_narrower_accesses(emu, q_off, k_off, vec):
    w = SMALL["llama_ragged"].scaled(seq_len=9, table_rows=9)
    check(emu, w, 1, q_offset=q_off, k_offset=k_off, expect={"vec": vec})


@pytest.mark.parametrize("spec,vec,aligned", [
    (dict(head_dim=24, rotary_dim=24), 4, 1),            # R/2 = 12
    (dict(head_dim=48, rotary_dim=48), 8, 1),            # lanes = 3 (not a power of 2)
    (dict(head_dim=66, rotary_dim=64), 2, 1),            # D only 2-divisible
    (dict(head_dim=130, rotary_dim=2), 1, 1),            # one pair per row
    (dict(head_dim=256, rotary_dim=128), 8, 1),          # partial rotary, wide head
    (dict(head_dim=256, rotary_dim=256), 8, 1),          # 16 lanes per row
])
def test_head_and_rotary_dims(emu, spec, vec, aligned):
    w = SMALL["llama_ragged"].scaled(seq_len=11, table_rows=11, **spec)
    check(emu, w, 1, expect={"vec": vec, "aligned": aligned})
    check(emu, w, -1, launch="token")


@pytest.mark.parametrize("spec,vec,aligned", [
    (dict(head_dim=31, rotary_dim=30), 2, 0),  # odd D: rows not pair-aligned
    (dict(head_dim=62, rotary_dim=62), 2, 1),
    (dict(head_dim=40, rotary_dim=24), 8, 1),
])
def test_interleaved_dims(emu, spec, vec, aligned):
    w = SMALL["bshd_interleaved_ragged"].scaled(seq_len=13, table_rows=13, **spec)
    check(emu, w, 1, expect={"vec": vec, "aligned": aligned})
    check(emu, w.scaled(layout="bhsd"), -1, launch="token")


def test_single_pass_token_shape_only_when_the_grid_covers_everything(emu):
    assert check(emu, SMALL["decode"])["single"] == 1
    plan = check(emu, SMALL["decode"], cus=1)  # one workgroup per token on any device
    assert plan["single"] == 1 and plan["grid"] == 19 and plan["tokens_per_block"] == 1
    w = SMALL["decode"].scaled(batch=100)
    plan = check(emu, w, cus=1, overrides=dict(token_grid=7))  # 7 workgroups loop over 100
    assert plan["token"] == 1 and plan["single"] == 0 and plan["grid"] == 7


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("token_grid", [0, 3])
@pytest.mark.parametrize("direction", [1, -1])
def test_small_tokens_share_a_workgroup(emu, layout, token_grid, direction):
    """3 heads x 4 lanes = 12 lanes per token: 21 consecutive tokens per
    workgroup (252 of 256 lanes), one pass or a grid-stride loop, with a
    ragged last group of tokens (400 = 19 * 21 + 1)."""
    w = SMALL["llama_ragged"].scaled(n_heads_q=2, n_heads_k=1, head_dim=64, rotary_dim=64,
                                     seq_len=200, table_rows=200, layout=layout)
    plan = check(emu, w, direction, launch="token", cus=1,
                 overrides=dict(token_grid=token_grid))
    assert plan["tokens_per_block"] == 21 and plan["block"] == 256
    assert plan["grid"] == (3 if token_grid else 20)
    assert plan["single"] == (0 if token_grid else 1)


@pytest.mark.parametrize("direction", [1, -1])
def test_interleaved_lanes_take_two_items(emu, direction):
    """Interleaved pairs: each token-shape lane takes items i and i + L. 32
    heads x 8 chunks = 256 items on 128 lanes; then 15 items per token (odd)
    packed 8 tokens to a workgroup: 120 items on 60 lanes, and a ragged last
    workgroup of tokens."""
    w = SMALL["bshd_interleaved_ragged"]
    plan = check(emu, w, direction, launch="token")
    assert plan["block"] == 128 and plan["single"] == 1 and plan["tokens_per_block"] == 1
    w = w.scaled(n_heads_q=3, n_heads_k=2, head_dim=40, rotary_dim=24)
    plan = check(emu, w, direction, launch="token", cus=1)
    assert plan["lanes"] == 3 and plan["tokens_per_block"] == 8 and plan["block"] == 64
    assert plan["single"] == 1 and plan["grid"] == 17  # ceil(135 / 8)
    check(emu, w, direction, launch="token", cus=1, overrides=dict(token_grid=5))


def test_token_packing_keeps_the_chip_filled(emu):
    """Tokens per workgroup shrink so the grid keeps 16 workgroups per CU
    (the token shape, forced: AUTO gives this dense view the flat shape)."""
    w = SMALL["llama_ragged"].scaled(n_heads_q=2, n_heads_k=1, head_dim=64, rotary_dim=64,
                                     layout="bshd")
    assert check(emu, w, launch="token", cus=1)["tokens_per_block"] == 9  # 154 // 16
    assert check(emu, w, launch="token", cus=256)["tokens_per_block"] == 1
    assert check(emu, w)["flat"] == 1


def test_many_heads_loop_in_token_shape(emu):
    """(Hq + Hk) * lanes above 1024 lanes: the token shape loops within a workgroup."""
    w = SMALL["decode"].scaled(n_heads_q=96, n_heads_k=8, head_dim=256, rotary_dim=256,
                               batch=3)
    plan = check(emu, w, 1, launch="token")
    assert plan["block"] == 1024 and plan["single"] == 0


def test_mqa_single_kv_head(emu):
    check(emu, SMALL["llama_ragged"].scaled(n_heads_k=1), 1)


def test_out_of_table_indices_pass_through(emu):
    w = SMALL["partial_indexed"].scaled(seq_len=20, table_rows=50)
    pos = torch.tensor([-5, 0, 49, 50, 1 << 30, -(1 << 30), 7, 3, 2, 1, 0, 48, 51, 9, 8, 7,
                        6, 5, 4, 3], dtype=torch.int32)
    check(emu, w, 1, pos=pos, use_workload_pos=False)
    check(emu, w, -1, launch="token", pos=pos, use_workload_pos=False)


def test_per_sequence_positions_in_prefill(emu):
    w = SMALL["llama_ragged"].scaled(seq_len=10, table_rows=1000, pos_kind="none")
    pos = W.random_positions(w.batch * w.seq_len, 1000, 77)
    q, k, _, cos, sin = _inputs(w)
    plan, qo, ko = run_emu(emu, w, q, k, cos, sin, pos, 1, "auto", True,
                           pos_batch_stride=w.seq_len)
    for x, o in ((q, qo), (k, ko)):
        ref = P.oracle_rope(w, x, 1, pos, pos_batch_stride=w.seq_len)
        P.assert_parity(o, ref, P.storage(x), w.dtype, w.layout, w.rotary_dim,
                        P.masked_tokens(w, pos, pos_batch_stride=w.seq_len))


@pytest.mark.parametrize("change", [dict(batch=0), dict(seq_len=0), dict(rotary_dim=0)])
def test_empty_work(emu, change):
    w = SMALL["llama_ragged"].scaled(**change)
    if w.rotary_dim == 0:
        w = w.scaled(table_rows=w.seq_len)
    q, k, pos, cos, sin = _inputs(w)
    plan, qo, ko = run_emu(emu, w, q, k, cos, sin, pos)
    assert plan["status"] == 0 and plan["empty"] == 1
    assert np.array_equal(qo, P.storage(q))


# ------------------------------------------------ the general form (rope_apply)

def _strided(buf, spec, shape):
    """View [B,H,S,D] of 1-d storage `buf` at (offset, sb, sh, ss)."""
    off, sb, sh, ss = spec
    return torch.as_strided(buf, shape, (sb, sh, ss, 1), off)


def _f64_bits(x: float) -> int:
    return struct.unpack("<q", struct.pack("<d", float(x)))[0]


def run_emu_apply(emu, w, in_buf, q_in, k_in, cos, sin, *, out_buf=None, q_out=None,
                  k_out=None, pos=None, direction=1, launch="auto", t_row=0, t_col=1,
                  cus=256, pos_batch_stride=None, theta=None, interpolate_factor=1.0,
                  table_rows=None, overrides=None):
    """Run rope_apply's plan in the emulator. Views are (offset, sb, sh, ss)
    element specs into in_buf / out_buf (1-d torch storage). With `theta`,
    angles are computed from theta (cos/sin may then be None)."""
    with tempfile.TemporaryDirectory() as job:
        desc = dict(apply=1, batch=w.batch, seq_len=w.seq_len, head_dim=w.head_dim,
                    rotary_dim=w.rotary_dim, n_heads_q=w.n_heads_q,
                    n_heads_k=0 if k_in is None else w.n_heads_k,
                    dtype=CODES["dtype"][w.dtype], pairing=CODES["pairing"][w.pairing],
                    launch=CODES["launch"][launch], direction=direction,
                    in_elems=in_buf.numel(), out_elems=0 if out_buf is None else out_buf.numel(),
                    table_elems=0 if cos is None else cos.numel(),
                    table_rows=(cos.shape[0] if table_rows is None else table_rows),
                    t_row=t_row, t_col=t_col,
                    pos_count=0 if pos is None else pos.numel(),
                    pos_batch_stride=(w.pos_batch_stride if pos_batch_stride is None
                                      else pos_batch_stride), cus=cus,
                    angles=0 if theta is None else 1,
                    theta_bits=_f64_bits(0.0 if theta is None else theta),
                    interp_bits=_f64_bits(interpolate_factor))
        desc.update(overrides or {})
        for name, spec in (("q_in", q_in), ("k_in", k_in), ("q_out", q_out), ("k_out", k_out)):
            if spec is None:
                desc[name + "_off"] = -1
            else:
                for key, v in zip(("off", "sb", "sh", "ss"), spec):
                    desc[f"{name}_{key}"] = v
        with open(os.path.join(job, "desc.txt"), "w") as f:
            for key, v in desc.items():
                f.write(f"{key} {int(v)}\n")
        P.storage(in_buf).tofile(os.path.join(job, "in.bin"))
        if out_buf is not None:
            P.storage(out_buf).tofile(os.path.join(job, "out.bin"))
        if cos is not None:
            cos.contiguous().numpy().tofile(os.path.join(job, "cos.bin"))
            sin.contiguous().numpy().tofile(os.path.join(job, "sin.bin"))
        if pos is not None:
            pos.numpy().astype(np.int32).tofile(os.path.join(job, "pos.bin"))
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
        r = subprocess.run([emu, job], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stdout + r.stderr[-4000:]
        plan = {key: int(v) for key, v in
                (line.split() for line in r.stdout.strip().splitlines())}
        if plan["status"] != 0:
            return plan, None, None
        dt = W.TORCH_DTYPES[w.dtype]

        def back(path, like):
            st = P.storage(like)
            arr = np.fromfile(path, dtype=st.dtype)
            t = torch.from_numpy(arr.copy())
            return t if dt == torch.float32 else t.view(dt)
        in_after = back(os.path.join(job, "in_after.bin"), in_buf)
        out_after = None if out_buf is None else back(os.path.join(job, "out_after.bin"), out_buf)
        return plan, in_after, out_after


def _half_tables(w):
    return rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta)


def _oracle_view(w, x, direction, pos, heads, pos_batch_stride=None):
    wv = w.scaled(layout="bhsd", n_heads_q=heads)
    return P.oracle_rope(wv, x.contiguous(), direction, pos, pos_batch_stride=pos_batch_stride)


def _assert_view(w, got, x, direction, pos, heads, pos_batch_stride=None):
    ref = _oracle_view(w, x, direction, pos, heads, pos_batch_stride)
    masked = P.masked_tokens(w, pos, pos_batch_stride=pos_batch_stride)
    P.assert_parity(P.storage(got.contiguous()), ref, P.storage(x.contiguous()), w.dtype,
                    "bhsd", w.rotary_dim, masked)


PACKED = W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=37, n_heads_q=8, n_heads_k=2,
                                    table_rows=40)


def _packed(w, seed=5):
    """[B, S, (Hq + 2 Hk) * D] packed QKV storage and the Q, K view specs."""
    B, S, D, Hq, Hk = w.batch, w.seq_len, w.head_dim, w.n_heads_q, w.n_heads_k
    Wd = (Hq + 2 * Hk) * D
    buf = W.normal((B * S * Wd,), w.dtype, seed)
    q = (0, S * Wd, D, Wd)
    k = (Hq * D, S * Wd, D, Wd)
    v_region = (B, S, Wd)
    return buf, q, k, v_region


@pytest.mark.parametrize("launch", ["auto", "rows", "token"])
@pytest.mark.parametrize("direction", [1, -1])
def test_packed_qkv_in_place(emu, launch, direction):
    w = PACKED
    buf, qs, ks, _ = _packed(w)
    cos, sin = _half_tables(w)
    plan, after, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, launch=launch,
                                   direction=direction)
    assert plan["status"] == 0 and plan["oop"] == 0
    qshape = (w.batch, w.n_heads_q, w.seq_len, w.head_dim)
    kshape = (w.batch, w.n_heads_k, w.seq_len, w.head_dim)
    _assert_view(w, _strided(after, qs, qshape), _strided(buf, qs, qshape), direction, None,
                 w.n_heads_q)
    _assert_view(w, _strided(after, ks, kshape), _strided(buf, ks, kshape), direction, None,
                 w.n_heads_k)
    # the V part of every token is untouched, bit for bit
    B, S, D, Hq, Hk = w.batch, w.seq_len, w.head_dim, w.n_heads_q, w.n_heads_k
    v0 = buf.view(B, S, -1)[..., (Hq + Hk) * D:]
    v1 = after.view(B, S, -1)[..., (Hq + Hk) * D:]
    assert np.array_equal(P.storage(v0.contiguous()), P.storage(v1.contiguous()))


@pytest.mark.parametrize("launch", ["rows", "token"])
def test_packed_qkv_out_of_place_partial_rotary_with_skipped_tokens(emu, launch):
    w = PACKED.scaled(rotary_dim=64, table_rows=100)
    buf, qs, ks, _ = _packed(w, seed=6)
    cos, sin = _half_tables(w)
    B, S, D, Hq, Hk = w.batch, w.seq_len, w.head_dim, w.n_heads_q, w.n_heads_k
    out = torch.zeros(B * (Hq + Hk) * S * D, dtype=W.TORCH_DTYPES[w.dtype])
    qo = (0, Hq * S * D, S * D, D)
    ko = (B * Hq * S * D, Hk * S * D, S * D, D)
    pos = W.random_positions(S, 130, 9, low=-20)  # some negative, some past the table
    plan, after, out_after = run_emu_apply(emu, w, buf, qs, ks, cos, sin, out_buf=out,
                                           q_out=qo, k_out=ko, pos=pos, launch=launch,
                                           pos_batch_stride=0)
    assert plan["oop"] == 1
    assert np.array_equal(P.storage(after), P.storage(buf))  # inputs untouched
    qshape, kshape = (B, Hq, S, D), (B, Hk, S, D)
    _assert_view(w, _strided(out_after, qo, qshape), _strided(buf, qs, qshape), 1, pos, Hq,
                 pos_batch_stride=0)
    _assert_view(w, _strided(out_after, ko, kshape), _strided(buf, ks, kshape), 1, pos, Hk,
                 pos_batch_stride=0)


@pytest.mark.parametrize("table_layout", ["duplicated", "interleaved", "padded"])
@pytest.mark.parametrize("pairing", ["split_half", "interleaved"])
def test_table_layouts(emu, table_layout, pairing):
    w = PACKED.scaled(pairing=pairing)
    buf, qs, ks, _ = _packed(w, seed=7)
    c, s = _half_tables(w)
    if table_layout == "duplicated":
        cos, sin, t_row, t_col = torch.cat([c, c], 1), torch.cat([s, s], 1), w.rotary_dim, 1
    elif table_layout == "interleaved":
        cos, sin = c.repeat_interleave(2, 1), s.repeat_interleave(2, 1)
        t_row, t_col = w.rotary_dim, 2
    else:  # rows padded to R/2 + 4 floats
        pad = torch.full((c.shape[0], 4), float("nan"))
        cos, sin = torch.cat([c, pad], 1), torch.cat([s, pad], 1)
        t_row, t_col = w.rotary_dim // 2 + 4, 1
    plan, after, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, t_row=t_row, t_col=t_col)
    assert plan["t_vec"] == (1 if t_col == 1 else 0)
    qshape = (w.batch, w.n_heads_q, w.seq_len, w.head_dim)
    _assert_view(w, _strided(after, qs, qshape), _strided(buf, qs, qshape), 1, None,
                 w.n_heads_q)


def test_padded_rows_and_broadcast_input_out_of_place(emu):
    """[B,H,S,D] rows padded to D + 8 elements, rotated in place; and one
    sequence broadcast (batch stride 0) into a [B,H,S,D] output."""
    w = PACKED.scaled(n_heads_k=0, seq_len=21, table_rows=21)
    B, H, S, D = w.batch, w.n_heads_q, w.seq_len, w.head_dim
    cos, sin = _half_tables(w)
    rs = D + 8
    buf = W.normal((B * H * S * rs,), w.dtype, 11)
    spec = (0, H * S * rs, S * rs, rs)
    plan, after, _ = run_emu_apply(emu, w, buf, spec, None, cos, sin)
    shape = (B, H, S, D)
    _assert_view(w, _strided(after, spec, shape), _strided(buf, spec, shape), 1, None, H)
    pads = torch.as_strided(after, (B * H * S, 8), (rs, 1), D)
    pads0 = torch.as_strided(buf, (B * H * S, 8), (rs, 1), D)
    assert np.array_equal(P.storage(pads.contiguous()), P.storage(pads0.contiguous()))
    # broadcast: every batch reads the same sequence
    one = W.normal((H * S * D,), w.dtype, 12)
    out = torch.zeros(B * H * S * D, dtype=W.TORCH_DTYPES[w.dtype])
    ispec, ospec = (0, 0, S * D, D), (0, H * S * D, S * D, D)
    plan, after, out_after = run_emu_apply(emu, w, one, ispec, None, cos, sin, out_buf=out,
                                           q_out=ospec, direction=-1)
    assert plan["status"] == 0 and plan["oop"] == 1
    _assert_view(w, _strided(out_after, ospec, shape), _strided(one, ispec, shape), -1, None, H)


def test_odd_head_dim_interleaved_out_of_place(emu):
    w = W.BSHD_INTERLEAVED.scaled(batch=2, seq_len=9, n_heads_q=3, n_heads_k=2, head_dim=31,
                                  rotary_dim=30, table_rows=9, layout="bhsd")
    B, S, D = w.batch, w.seq_len, w.head_dim
    cos, sin = _half_tables(w)
    buf = W.normal((B * 5 * S * D,), w.dtype, 13)
    qs, ks = (0, 3 * S * D, S * D, D), (B * 3 * S * D, 2 * S * D, S * D, D)
    out = torch.zeros_like(buf)
    plan, _, out_after = run_emu_apply(emu, w, buf, qs, ks, cos, sin, out_buf=out, q_out=qs,
                                       k_out=ks)
    assert plan["aligned"] == 0 and plan["oop"] == 1
    _assert_view(w, _strided(out_after, qs, (B, 3, S, D)), _strided(buf, qs, (B, 3, S, D)), 1,
                 None, 3)
    _assert_view(w, _strided(out_after, ks, (B, 2, S, D)), _strided(buf, ks, (B, 2, S, D)), 1,
                 None, 2)


@pytest.mark.parametrize("case,expected", [
    ("outputs_overlap", -6), ("k_inside_q_heads", -6), ("output_not_injective", -6),
    ("direction_zero", -4), ("col_stride_three", -4), ("negative_stride", -2),
    ("table_row_stride_too_small", -2), ("q_shifted_into_k", -6), ("packed_ok", 0)])
def test_apply_validation(emu, case, expected):
    w = PACKED
    buf, qs, ks, _ = _packed(w)
    cos, sin = _half_tables(w)
    kw = {}
    if case == "outputs_overlap":
        # outputs live in a second buffer; with identical offsets the validator
        # cannot tell the buffers apart only if the pointers coincide, so place
        # Q's output exactly over K's input by writing into the input buffer
        plan, _, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, out_buf=None, q_out=None)
        assert plan["status"] == 0
        d_out = torch.zeros_like(buf)
        plan, _, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, out_buf=d_out, q_out=qs,
                                   k_out=qs)
        assert plan["status"] == expected  # both outputs on the same elements
        assert plan["status"] == expected
        return
    if case == "k_inside_q_heads":
        ks = (w.head_dim * 3, *ks[1:])
    if case == "output_not_injective":
        qs = (0, qs[1], 0, qs[3])
    if case == "direction_zero":
        kw["direction"] = 0
    if case == "col_stride_three":
        kw["t_col"] = 3
    if case == "negative_stride":
        qs = (qs[0] + qs[1], -qs[1], qs[2], qs[3])
    if case == "table_row_stride_too_small":
        kw["t_row"] = w.rotary_dim // 2 - 1
    if case == "q_shifted_into_k":  # Q's last head now shares elements with K's first
        buf = torch.cat([buf, buf[:1]])
        qs = (1, *qs[1:])
    plan, _, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, **kw)
    assert plan["status"] == expected


# ------------------------------------------------- angles computed from theta

def _qk_views(w, layout):
    """Q and K of workload w stored back to back in one buffer, as (offset,
    sb, sh, ss) view specs in the given layout; returns buf, specs, tensors."""
    t = W.tensors(w)
    q, k = t["q"], t["k"]  # in w.layout
    B, S, D, Hq, Hk = w.batch, w.seq_len, w.head_dim, w.n_heads_q, w.n_heads_k
    buf = torch.cat([q.reshape(-1), k.reshape(-1)])
    if layout == "bhsd":
        qs, ks = (0, Hq * S * D, S * D, D), (q.numel(), Hk * S * D, S * D, D)
    else:
        qs, ks = (0, S * Hq * D, D, Hq * D), (q.numel(), S * Hk * D, D, Hk * D)
    return buf, qs, ks, q, k


def _theta_case(emu, w, *, launch="auto", direction=1, interp=1.0, pos=None,
                pos_batch_stride=None, max_positions=None, cus=256, overrides=None):
    """Run w with angles computed from theta and compare with the oracle
    (table mode with the same theta and interpolate_factor) and with the
    table path of the emulated library on the same inputs."""
    buf, qs, ks, q, k = _qk_views(w, w.layout)
    rows = max_positions if max_positions is not None else w.table_rows
    pbs = w.pos_batch_stride if pos_batch_stride is None else pos_batch_stride
    plan, after, _ = run_emu_apply(emu, w, buf, qs, ks, None, None, pos=pos, direction=direction,
                                   launch=launch, cus=cus, pos_batch_stride=pbs,
                                   theta=w.theta, interpolate_factor=interp, table_rows=rows,
                                   overrides=overrides)
    assert plan["status"] == 0 and plan["angles"] == 1, plan
    qa, ka = after[:q.numel()].view(q.shape), after[q.numel():].view(k.shape)
    masked = P.masked_tokens(w, pos, table_rows=rows, pos_batch_stride=pbs)
    for got, x in ((qa, q), (ka, k)):
        ref = P.oracle_rope(w.scaled(n_heads_q=x.shape[1] if w.layout == "bhsd" else x.shape[2]),
                            x, direction, pos, pos_batch_stride=pbs, table_rows=rows,
                            interpolate_factor=interp)
        P.assert_parity(P.storage(got), ref, P.storage(x), w.dtype, w.layout, w.rotary_dim,
                        masked)
    # the table path on the same call: cos/sin agree to the last bit except
    # where a value lies within ~1e-15 of a float32 rounding boundary
    cos, sin = rp.rope_build_table(rows, w.rotary_dim, w.theta, interp)
    _, after_t, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, pos=pos, direction=direction,
                                  launch=launch, cus=cus, pos_batch_stride=pbs,
                                  overrides=overrides)
    same = np.mean(P.storage(after) == P.storage(after_t))
    assert same >= 0.999, same
    return plan


@pytest.mark.parametrize("launch", ["rows", "token"])
@pytest.mark.parametrize("direction", [1, -1])
def test_theta_matches_oracle_both_shapes(emu, launch, direction):
    plan = _theta_case(emu, SMALL["llama_ragged"], launch=launch, direction=direction)
    assert plan["token"] == (launch == "token")
    # single-pass token shape: the token's R/2 (cos, sin) pairs in shared memory
    assert plan["lds_bytes"] == (SMALL["llama_ragged"].rotary_dim // 2 * 8 if launch == "token"
                                 else 0)


@pytest.mark.parametrize("interp", [1.0, 3.0, 0.5])
def test_theta_interpolate_factor(emu, interp):
    w = SMALL["llama_ragged"]
    _theta_case(emu, w, interp=interp, launch="rows")
    _theta_case(emu, w, interp=interp, launch="token", direction=-1)


def test_theta_interleaved_two_items_per_lane(emu):
    plan = _theta_case(emu, SMALL["bshd_interleaved_ragged"], launch="token")
    assert plan["block"] == 128 and plan["single"] == 1


def test_theta_packed_tokens_and_loop(emu):
    w = SMALL["llama_ragged"].scaled(n_heads_q=2, n_heads_k=1, head_dim=64, rotary_dim=64,
                                     seq_len=200, table_rows=200, layout="bshd")
    plan = _theta_case(emu, w, launch="token", cus=1, interp=2.0)
    # 12 items per token: 21 tokens per workgroup (400 // 16 = 25 allows it)
    assert plan["tokens_per_block"] == 21 and plan["single"] == 1
    assert plan["lds_bytes"] == 21 * 32 * 8  # [token][frequency] (cos, sin) pairs
    plan = _theta_case(emu, w, launch="token", cus=1, overrides=dict(token_grid=3))
    assert plan["single"] == 0 and plan["lds_bytes"] == 0


@pytest.mark.parametrize("direction", [1, -1])
def test_theta_decode_large_positions(emu, direction):
    """Decode: one token per workgroup, positions up to 32767 with theta = 5e5."""
    w = SMALL["decode"]
    pos = W.positions(w)
    plan = _theta_case(emu, w, direction=direction, pos=pos)
    assert plan["token"] == 1 and plan["tokens_per_block"] == 1


def test_theta_long_positions(emu):
    """Positions near 131071 (angles ~1.3e5 rad at the lowest frequency)."""
    w = SMALL["long_theta"]
    pos = torch.arange(131071 - 63, 131072, dtype=torch.int32)
    _theta_case(emu, w, pos=pos, pos_batch_stride=0, max_positions=131072, launch="rows")
    _theta_case(emu, w, pos=pos, pos_batch_stride=0, max_positions=131072, launch="token")


def test_theta_skipped_tokens_partial_rotary(emu):
    w = SMALL["partial_indexed"]
    pos = W.positions(w)
    for launch in ("rows", "token"):
        _theta_case(emu, w, pos=pos, launch=launch)


def _theta_status(emu, **kw):
    w = SMALL["llama_ragged"].scaled(seq_len=4, table_rows=4)
    buf, qs, ks, q, k = _qk_views(w, w.layout)
    args = dict(theta=w.theta, interpolate_factor=1.0, table_rows=4)
    overrides = {}
    for key, v in kw.items():
        if key in ("theta", "interpolate_factor", "table_rows"):
            args[key] = v
        else:
            overrides[key] = v
    plan, _, _ = run_emu_apply(emu, w, buf, qs, ks, None, None, overrides=overrides, **args)
    return plan["status"]


def test_theta_validation(emu):
    SHAPE, LAYOUT = -2, -4
    assert _theta_status(emu) == 0  # no tables needed
    for bad in (0.0, -10.0, float("inf"), float("nan")):
        assert _theta_status(emu, theta=bad) == SHAPE
        assert _theta_status(emu, interpolate_factor=bad) == SHAPE
    assert _theta_status(emu, angles=2) == LAYOUT
    # the largest angle, (table_rows - 1) / interpolate_factor, must stay <= 2^40
    assert _theta_status(emu, table_rows=2 ** 31 - 1, interpolate_factor=1e-3) == SHAPE
    assert _theta_status(emu, table_rows=2 ** 31 - 1, interpolate_factor=1.0) == 0


def _kernel_sincos(emu, angles):
    with tempfile.TemporaryDirectory() as job:
        with open(os.path.join(job, "desc.txt"), "w") as f:
            f.write(f"sincos 1\ncount {len(angles)}\n")
        np.asarray(angles, np.float64).tofile(os.path.join(job, "angles.bin"))
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
        r = subprocess.run([emu, job], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stderr[-2000:]
        return np.fromfile(os.path.join(job, "sincos.bin"), np.float32).reshape(-1, 2)


def test_kernel_sincos_is_correctly_rounded(emu):
    """The kernels' cos/sin (Cody-Waite reduction by pi/2, Taylor series in
    binary64, one rounding) against 60-digit mpmath rounded once to float32:
    equal except for values within ~1e-15 of a float32 rounding boundary. The
    angles cover the kernels' range: RoPE angles p * theta^(-2i/R) up to 1.3e5,
    angles within 1e-9 of multiples of pi/2 (where the reduction cancels),
    negative angles, tiny angles and the 2^40 limit."""
    import mpmath
    rng = np.random.default_rng(77)
    ang = [0.0, -0.0, 1e-20, 1e-8, -1e-8, 0.5, 1.0, 2.0 ** 40, -(2.0 ** 40)]
    ang += list(rng.uniform(-10, 10, 2000))
    ang += list(rng.uniform(0, 131072, 3000))
    ang += list(np.exp(rng.uniform(np.log(1e-6), np.log(2.0 ** 40), 3000)))
    with mpmath.workdps(60):
        halfpi = mpmath.pi / 2
        for k in rng.integers(1, 2 ** 30, 1000):
            near = float(halfpi * int(k))  # nearest binary64 to k pi/2
            ang += [near, np.nextafter(near, np.inf), np.nextafter(near, -np.inf)]
        theta, R = 500000.0, 128
        for p in (1, 7, 4095, 32767, 131071):
            for i in range(R // 2):
                ang.append(float(p) * (theta ** (-(2.0 * i) / R)))
    ang = np.asarray(ang, np.float64)
    got = _kernel_sincos(emu, ang)
    bad = 0
    with mpmath.workdps(60):
        for x, (gc, gs) in zip(ang, got):
            a = mpmath.mpf(float(x))
            for g, ref in ((gc, mpmath.cos(a)), (gs, mpmath.sin(a))):
                r = X.rn24_mp(ref)
                if float(g) != r:
                    bad += 1
                    # only a value within 1e-15 (absolute) of the midpoint
                    # between the two float32 neighbours may round the other way
                    mid = (mpmath.mpf(r) + mpmath.mpf(float(g))) / 2
                    assert abs(float(g) - r) <= abs(np.spacing(np.float32(r))) * 1.01, (x, g, r)
                    assert abs(ref - mid) <= mpmath.mpf("1e-15"), (x, g, ref)
    assert bad <= 2, bad


# -------------------------------------------- rows shape, one chunk per lane
# Split-half, in place, 16-byte chunks, L = (R/2)/V chunks per half a power
# of two <= 16: each lane holds one chunk and takes its pair partner's chunk
# from lane ^ L. The emulator runs the wave's phases in lockstep. The results
# must equal the pair-per-lane form of the same plan bit for bit (and the
# oracle, through check()).
PAIR_CASES = {
    # name: workload, expected L
    "bf16_R128_L8": (W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=77, table_rows=80), 8),
    "bf16_R64_L4": (W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=50, head_dim=64, rotary_dim=64,
                                                table_rows=50, n_heads_q=6, n_heads_k=2), 4),
    "f32_R64_L8": (W.TINY_F32.scaled(seq_len=70, table_rows=70), 8),
    "f16_R32_L2": (W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=33, head_dim=64, rotary_dim=32,
                                               dtype="f16", table_rows=33, n_heads_q=4,
                                               n_heads_k=4), 2),
    "bf16_R256_L16": (W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=40, head_dim=256,
                                                  rotary_dim=256, table_rows=40, n_heads_q=5,
                                                  n_heads_k=1), 16),
    "bf16_R16_L1": (W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=45, head_dim=64, rotary_dim=16,
                                                table_rows=45, n_heads_q=3, n_heads_k=3), 1),
    "indexed_partial": (W.PARTIAL_INDEXED.scaled(seq_len=130, pos_start_max=9000), 2),
}


@pytest.mark.parametrize("name", list(PAIR_CASES))
@pytest.mark.parametrize("direction", [1, -1])
def test_one_chunk_per_lane_equals_chunk_pairs(emu, name, direction):
    w, L = PAIR_CASES[name]
    plan = check(emu, w, direction, launch="rows",
                 expect=dict(pair=1, lanes=2 * L))
    q, k, wpos, cos, sin = _inputs(w)
    _, q1, k1 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "rows")
    plan0, q0, k0 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "rows",
                            overrides=dict(no_pair=1))
    assert plan0["pair"] == 0 and plan0["lanes"] == L, plan0
    assert np.array_equal(q1, q0) and np.array_equal(k1, k0)
    assert plan["grid"] >= plan0["grid"]


@pytest.mark.parametrize("group_slow", [0, 1])
@pytest.mark.parametrize("heads_per_group", [1, 3, 40])
def test_one_chunk_per_lane_any_head_groups(emu, group_slow, heads_per_group):
    w = W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=37, table_rows=40)
    check(emu, w, launch="rows", expect=dict(pair=1),
          overrides=dict(heads_per_group=heads_per_group, group_slow=group_slow))


def test_one_chunk_per_lane_only_where_it_applies(emu):
    w = W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=40, table_rows=40)
    assert check(emu, w, launch="rows")["pair"] == 1
    # interleaved pairs, 8-byte chunks (misaligned base), or L = 3 (R = 48)
    assert check(emu, w.scaled(pairing=W.INTERLEAVED), launch="rows")["pair"] == 0
    assert check(emu, w, launch="rows", q_offset=4)["pair"] == 0
    assert check(emu, w.scaled(rotary_dim=48, head_dim=64), launch="rows")["pair"] == 0
    # the token shape never uses it
    assert check(emu, w, launch="token")["pair"] == 0


def plan_of(emu, w, launch="auto", cus=256):
    """The library's plan for rope_fwd_qk on workload w at full size (nothing runs)."""
    with tempfile.TemporaryDirectory() as job:
        desc = dict(plan_only=1, batch=w.batch, n_heads_q=w.n_heads_q, n_heads_k=w.n_heads_k,
                    seq_len=w.seq_len, head_dim=w.head_dim, rotary_dim=w.rotary_dim,
                    dtype=CODES["dtype"][w.dtype], layout=CODES["layout"][w.layout],
                    pairing=CODES["pairing"][w.pairing], launch=CODES["launch"][launch],
                    table_rows=w.table_rows, cus=cus)
        with open(os.path.join(job, "desc.txt"), "w") as f:
            for key, v in desc.items():
                f.write(f"{key} {int(v)}\n")
        r = subprocess.run([emu, job], capture_output=True, text=True, timeout=60)
        assert r.returncode == 0, r.stderr[-2000:]
        return {k: int(v) for k, v in (line.split() for line in r.stdout.strip().splitlines())}


def test_full_size_plans(emu):
    # Llama prefill (heads 1 MiB apart): head lanes, 8 tokens x 8 heads per
    # workgroup; long context (heads 32 MiB apart): 4 tokens x 20 heads
    p = plan_of(emu, W.LLAMA_GQA_PREFILL)
    assert (p["token"], p["head_lanes"], p["tokens_per_block"], p["heads_per_group"],
            p["block"], p["grid"]) == (0, 1, 8, 8, 512, 2048 * 5), p
    p = plan_of(emu, W.LONG_CONTEXT)
    assert (p["token"], p["head_lanes"], p["tokens_per_block"], p["heads_per_group"],
            p["block"], p["grid"]) == (0, 1, 4, 20, 640, 32768 * 2), p
    # an explicit rows launch keeps the rows kernels: one chunk per lane in
    # 4-head groups at Llama prefill, chunk pairs in 8-head groups at long
    # context (its cos/sin table is re-read per group)
    p = plan_of(emu, W.LLAMA_GQA_PREFILL, launch="rows")
    assert (p["token"], p["heads_per_group"], p["pair"], p["lanes"]) == (0, 4, 1, 16), p
    p = plan_of(emu, W.LONG_CONTEXT, launch="rows")
    assert (p["token"], p["heads_per_group"], p["pair"], p["lanes"]) == (0, 8, 0, 8), p
    # heads 4 and 8 MiB apart: the rows kernels
    for S in (16384, 32768):
        p = plan_of(emu, W.LONG_CONTEXT.scaled(batch=131072 // S, seq_len=S, table_rows=S))
        assert (p["token"], p["head_lanes"]) == (0, 0), p
    assert plan_of(emu, W.DECODE)["token"] == 1
    p = plan_of(emu, W.BSHD_INTERLEAVED)
    assert (p["token"], p["flat"], p["block"], p["grid"]) == (1, 1, 64, 8 * 2048 * 32 * 8 // 64), p


def test_theta_angles_keep_chunk_pairs(emu):
    # both lanes of a pair would evaluate the same sin/cos: the plan keeps a
    # chunk pair per lane when angles come from theta
    w = W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=40, table_rows=40)
    plan = _theta_case(emu, w, launch="rows")
    assert plan["pair"] == 0 and plan["lanes"] == 8, plan


# -------------------------------------------------------- head-lanes shape
# [B,H,S,D] split-half calls in 16-byte chunks, in place, with tables: one
# chunk of one (token, head) per lane, tokens_per_block x lanes x
# heads_per_group lanes per workgroup. Each case must equal the oracle and,
# bit for bit, the rows kernels of the same call (launch="rows").
HEAD_LANES_CASES = {
    # name: workload, expected (tokens_per_block, heads_per_group)
    "llama_ragged": (W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=77, table_rows=80), (8, 8)),
    "heads_not_a_multiple": (W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=21, table_rows=21,
                                                        n_heads_q=9, n_heads_k=3), (8, 8)),
    "indexed_skips": (W.PARTIAL_INDEXED.scaled(seq_len=130, pos_start_max=9000, head_dim=128,
                                              rotary_dim=128), (8, 8)),
    "f16_R256": (W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=19, head_dim=256, rotary_dim=256,
                                            dtype="f16", table_rows=19, n_heads_q=6,
                                            n_heads_k=2), (4, 8)),
    "f32_R128": (W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=23, dtype="f32", table_rows=23,
                                            n_heads_q=8, n_heads_k=1), (4, 8)),
}


@pytest.mark.parametrize("name", list(HEAD_LANES_CASES))
@pytest.mark.parametrize("direction", [1, -1])
def test_head_lanes_match_oracle_and_rows(emu, name, direction):
    w, (tpb, hpg) = HEAD_LANES_CASES[name]
    plan = check(emu, w, direction, cus=1,
                 expect=dict(token=0, head_lanes=1, tokens_per_block=tpb, heads_per_group=hpg))
    q, k, wpos, cos, sin = _inputs(w)
    _, q1, k1 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "auto", cus=1)
    plan0, q0, k0 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "rows", cus=1)
    assert plan0["head_lanes"] == 0
    assert np.array_equal(q1, q0) and np.array_equal(k1, k0)
    assert plan["block"] == plan["lanes"] * tpb * hpg


@pytest.mark.parametrize("tshift,heads", [(2, 20), (0, 1), (5, 3), (1, 40)])
def test_head_lanes_any_token_and_head_counts(emu, tshift, heads):
    """The long-sequence form (4 tokens x 20 heads) and other counts cover
    every row once, with ragged token tiles and head groups."""
    w = W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=37, table_rows=40, n_heads_q=16,
                                   n_heads_k=8)
    check(emu, w, -1, cus=1, expect=dict(head_lanes=1, heads_per_group=heads,
                                         tokens_per_block=1 << tshift),
          overrides=dict(hl_tshift=tshift, heads_per_group=heads))


def test_head_lanes_only_where_they_apply(emu):
    w = W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=40, table_rows=40)
    assert check(emu, w, cus=1)["head_lanes"] == 1
    # explicit rows or token launch, interleaved pairs, 8-byte chunks, fewer
    # than 8 heads, angles from theta: not this shape
    assert check(emu, w, launch="rows", cus=1)["head_lanes"] == 0
    assert check(emu, w, launch="token", cus=1)["head_lanes"] == 0
    assert check(emu, w.scaled(pairing=W.INTERLEAVED), cus=1)["head_lanes"] == 0
    assert check(emu, w, q_offset=4, cus=1)["head_lanes"] == 0
    assert check(emu, w.scaled(n_heads_q=5, n_heads_k=2), cus=1)["head_lanes"] == 0
    assert _theta_case(emu, w, cus=1)["head_lanes"] == 0
    # rotated spans under 256 bytes keep the pair-lanes rows kernel (four
    # sequences, so the table's re-reads allow 4-head groups)
    plan = check(emu, w.scaled(batch=4, rotary_dim=64), cus=1)
    assert plan["head_lanes"] == 0 and plan["pair"] == 1
    plan = check(emu, W.PARTIAL_INDEXED.scaled(batch=4, seq_len=130, pos_start_max=9000), cus=1)
    assert plan["head_lanes"] == 0


# -------------------------------------------------------------- flat shape
FLAT_CASES = {
    "bshd_interleaved_ragged": W.BSHD_INTERLEAVED.scaled(batch=3, seq_len=45, table_rows=45),
    "q_heads_differ": W.BSHD_INTERLEAVED.scaled(batch=2, seq_len=13, table_rows=13,
                                                n_heads_q=12, n_heads_k=4),
    "partial_rotary_bf16": W.BSHD_INTERLEAVED.scaled(batch=2, seq_len=17, table_rows=17,
                                                     dtype="bf16", rotary_dim=48),
    "f32_odd_lanes": W.BSHD_INTERLEAVED.scaled(batch=1, seq_len=29, table_rows=29,
                                               dtype="f32", head_dim=24, rotary_dim=24),
    "skipped_tokens": W.PARTIAL_INDEXED.scaled(seq_len=70, pos_start_max=9000, layout="bshd",
                                               pairing="interleaved"),
}


@pytest.mark.parametrize("name", list(FLAT_CASES))
@pytest.mark.parametrize("direction", [1, -1])
def test_flat_matches_oracle_and_token_kernel(emu, name, direction):
    w = FLAT_CASES[name]
    plan = check(emu, w, direction, expect=dict(token=1, flat=1, block=64))
    q, k, wpos, cos, sin = _inputs(w)
    _, q1, k1 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "auto")
    plan0, q0, k0 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "token")
    assert plan0["flat"] == 0
    assert np.array_equal(q1, q0) and np.array_equal(k1, k0)
    assert plan["grid"] * 64 >= (w.n_heads_q + w.n_heads_k) * w.batch * w.seq_len


def test_flat_q_only_and_misaligned(emu):
    w = FLAT_CASES["bshd_interleaved_ragged"]
    assert check(emu, w, with_k=False)["flat"] == 1
    # 4-byte aligned base: 2-element chunks, still flat
    assert check(emu, w, q_offset=2, expect=dict(vec=2))["flat"] == 1


def test_flat_only_where_it_applies(emu):
    w = FLAT_CASES["bshd_interleaved_ragged"]
    assert check(emu, w.scaled(seq_len=1, table_rows=1))["flat"] == 0
    # rotated spans past 256 bytes: the token kernel
    assert check(emu, w.scaled(dtype="bf16", head_dim=256, rotary_dim=256))["flat"] == 0
    assert check(emu, w.scaled(layout="bhsd"))["flat"] == 0
    assert check(emu, w, launch="token")["flat"] == 0


# ------------------------------------------- flat shape, split-half pairs
# One 16-byte chunk per lane, the partner half's chunk from the partner lane
# (rope_flat_pair_kernel), emulated with the wave's load, exchange and store
# phases in lockstep. L = R / (2V) from 1 to 4 (rotated spans up to 128 bytes).
FLAT_PAIR_CASES = {
    "bshd_split_d64_fp16": W.BSHD_INTERLEAVED.scaled(batch=3, seq_len=45, table_rows=45,
                                                     pairing=W.SPLIT_HALF),       # L = 4
    "partial_r64_of_128_bf16": W.LLAMA_GQA_PREFILL.scaled(batch=2, seq_len=21, table_rows=21,
                                                          layout="bshd", rotary_dim=64),  # L = 4
    "partial_r16_of_64": W.BSHD_INTERLEAVED.scaled(batch=2, seq_len=19, table_rows=19,
                                                   pairing=W.SPLIT_HALF, dtype="bf16",
                                                   rotary_dim=16),                # L = 1
    "partial_r32_f32": W.BSHD_INTERLEAVED.scaled(batch=1, seq_len=23, table_rows=23,
                                                 pairing=W.SPLIT_HALF, dtype="f32",
                                                 rotary_dim=32),                  # L = 4
    "q_heads_differ": W.BSHD_INTERLEAVED.scaled(batch=2, seq_len=13, table_rows=13,
                                                pairing=W.SPLIT_HALF, n_heads_q=12,
                                                n_heads_k=4),
    "skipped_tokens": W.PARTIAL_INDEXED.scaled(seq_len=70, pos_start_max=9000, layout="bshd"),
}


@pytest.mark.parametrize("name", list(FLAT_PAIR_CASES))
@pytest.mark.parametrize("direction", [1, -1])
def test_flat_pair_matches_oracle_and_token_kernel(emu, name, direction):
    """Every element against the oracle, and bit for bit against the token
    kernel's chunk-pair form of the same call."""
    w = FLAT_PAIR_CASES[name]
    plan = check(emu, w, direction, expect=dict(token=1, flat=1, block=64))
    half = w.rotary_dim // 2
    vec = 16 // {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    assert plan["lanes"] == 2 * (half // vec), plan
    q, k, wpos, cos, sin = _inputs(w)
    _, q1, k1 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "auto")
    plan0, q0, k0 = run_emu(emu, w, q, k, cos, sin, wpos, direction, "token")
    assert plan0["flat"] == 0
    assert np.array_equal(q1, q0) and np.array_equal(k1, k0)


def test_flat_pair_q_only(emu):
    w = FLAT_PAIR_CASES["bshd_split_d64_fp16"]
    assert check(emu, w, with_k=False)["flat"] == 1


def test_flat_pair_only_where_it_applies(emu):
    w = FLAT_PAIR_CASES["bshd_split_d64_fp16"]
    # 4-byte aligned base: 2-element chunks, no partner exchange of 16 bytes
    assert check(emu, w, q_offset=2, expect=dict(vec=2))["flat"] == 0
    # 128-byte halves and wider (R = 128 and 256 in 16-bit): the token kernel
    wide = W.LLAMA_GQA_PREFILL.scaled(batch=1, seq_len=9, table_rows=9, layout="bshd")
    assert check(emu, wide)["flat"] == 0
    assert check(emu, wide.scaled(n_heads_q=3, n_heads_k=1, head_dim=256,
                                  rotary_dim=256))["flat"] == 0
    assert check(emu, w.scaled(layout="bhsd"))["flat"] == 0
    assert check(emu, w, launch="token")["flat"] == 0


@pytest.mark.parametrize("spec", [dict(head_dim=64, rotary_dim=64),
                                  dict(head_dim=64, rotary_dim=32, table_rows=100),
                                  dict(pairing="interleaved"),
                                  dict(pairing="interleaved", head_dim=64, rotary_dim=48,
                                       table_rows=100)])
def test_packed_qkv_flat_pair(emu, spec):
    """Q and K as views into packed QKV storage: AUTO runs a flat kernel
    (split-half spans up to 128 bytes: pair lanes; interleaved spans up to
    256 bytes), the items numbered token by token over Q's then K's heads;
    the result equals the token kernel's bit for bit, the oracle's on every
    element, and V's part of each token is untouched."""
    w = PACKED.scaled(**spec)
    buf, qs, ks, _ = _packed(w, seed=8)
    cos, sin = _half_tables(w)
    pos = (W.random_positions(w.seq_len, 130, 11, low=-20) if spec.get("table_rows")
           else None)
    kw = dict(pos=pos, pos_batch_stride=0) if pos is not None else {}
    plan, after, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, launch="auto", **kw)
    assert plan["status"] == 0 and plan["flat"] == 1 and plan["oop"] == 0, plan
    plan0, after0, _ = run_emu_apply(emu, w, buf, qs, ks, cos, sin, launch="token", **kw)
    assert plan0["flat"] == 0
    assert np.array_equal(P.storage(after), P.storage(after0))
    qshape = (w.batch, w.n_heads_q, w.seq_len, w.head_dim)
    kshape = (w.batch, w.n_heads_k, w.seq_len, w.head_dim)
    extra = dict(pos_batch_stride=0) if pos is not None else {}
    _assert_view(w, _strided(after, qs, qshape), _strided(buf, qs, qshape), 1, pos,
                 w.n_heads_q, **extra)
    _assert_view(w, _strided(after, ks, kshape), _strided(buf, ks, kshape), 1, pos,
                 w.n_heads_k, **extra)
    B, S, D, Hq, Hk = w.batch, w.seq_len, w.head_dim, w.n_heads_q, w.n_heads_k
    v0 = buf.view(B, S, -1)[..., (Hq + Hk) * D:]
    v1 = after.view(B, S, -1)[..., (Hq + Hk) * D:]
    assert np.array_equal(P.storage(v0.contiguous()), P.storage(v1.contiguous()))


RANDOM_EMU_CASES = 80
RANDOM_EMU_CUS = (1, 4, 256)


@pytest.mark.parametrize("case", range(RANDOM_EMU_CASES))
def test_random_configurations_emulated(emu, case):
    """Seeded random configurations (tests/_random_configs.py, restricted to
    contiguous tensors, cos/sin tables and in-place calls): AUTO's kernel
    against the oracle on every element, and bit for bit against both forced
    grid shapes. The device size cycles through 1, 4 and 256 compute units,
    so that small calls also take the shapes that AUTO keeps for calls that
    fill the device."""
    c = draw_config(20000 + case, 150_000, views=False)
    cus = RANDOM_EMU_CUS[case % len(RANDOM_EMU_CUS)]
    w = config_workload(c)
    q = W.normal(w.q_shape, w.dtype, c["seed"])
    k = W.normal(w.k_shape, w.dtype, c["seed"] + 50)
    cos, sin = rp.rope_build_table(c["table_rows"], w.rotary_dim, w.theta)
    pos = None if c["pos"] is None else torch.from_numpy(c["pos"])
    pbs = c["pos_batch_stride"] or 0
    outs = []
    for launch in ("auto", "rows", "token"):
        plan, qo, ko = run_emu(emu, w, q, k, cos, sin, pos, c["direction"], launch,
                               cus=cus, pos_batch_stride=pbs)
        assert plan["status"] == 0, (launch, plan)
        outs.append((qo, ko))
    for qo, ko in outs[1:]:
        assert np.array_equal(qo, outs[0][0]) and np.array_equal(ko, outs[0][1])
    masked = P.masked_tokens(w, pos, pos_batch_stride=pbs)
    for got, x, what in ((outs[0][0], q, "q"), (outs[0][1], k, "k")):
        P.assert_parity(got, P.oracle_rope(w, x, c["direction"], pos, pos_batch_stride=pbs),
                        P.storage(x), w.dtype, w.layout, w.rotary_dim, masked,
                        f"random case {case} {what}")


def test_random_configurations_reach_every_kernel(emu):
    """AUTO's plans over the emulated draws (those without an index) include
    every kernel: head lanes, flat, flat pair lanes, pair lanes, token, rows."""
    seen = set()
    for case in range(RANDOM_EMU_CASES):
        c = draw_config(20000 + case, 150_000, views=False)
        if c["pos"] is not None:
            continue
        p = plan_of(emu, config_workload(c), cus=RANDOM_EMU_CUS[case % len(RANDOM_EMU_CUS)])
        seen.add("flat_pair" if p["flat"] and c["pairing"] == W.SPLIT_HALF else
                 "flat" if p["flat"] else "head_lanes" if p["head_lanes"] else
                 "token" if p["token"] else "pair_lanes" if p["pair"] else "rows")
    assert seen == {"flat_pair", "flat", "head_lanes", "token", "pair_lanes", "rows"}, seen

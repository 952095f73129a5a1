"""RoPE with XPOS scaling (rope_apply_xpos): host emulation and GPU parity.

The oracle (oracle_rope_xpos) and its pins are in test_oracle_xpos_pins.py.
Here: the library's host table builder equals the oracle's tables bit for
bit; the kernel body runs on the CPU under AddressSanitizer over every lane
of the planned grid (tests/emu/xpos_emu.hip) and through the C ABI on the
GPU, each against the oracle; and the C ABI's argument checks.

Kernel tolerance: 16-bit outputs within 1 unit of the monotone order (as
rope_apply); float32 outputs within 2 float32 ulps (the kernel rounds the
rotation and the product with the factor to float32, the oracle rounds the
binary64 value once).
"""
import fcntl
import os
import subprocess
import tempfile
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_fwd_amd as rp
import workloads as W
from tests import _parity as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EMU_SRC = os.path.join(ROOT, "tests", "emu", "xpos_emu.hip")
EMU_BIN = os.path.join(ROOT, "tests", "emu", "_build", "xpos_emu")
CSRC = os.path.join(ROOT, "rotary_position_embedding_fwd_amd", "csrc")
DEPS = [EMU_SRC, os.path.join(CSRC, "rope_xpos.hpp"), os.path.join(CSRC, "rope_kernels.hpp"),
        os.path.join(CSRC, "rope_plan.hpp"), os.path.join(ROOT, "include", "librope.h")]
DT = {"f32": 0, "f16": 1, "bf16": 2}
PAIR = {"split_half": 0, "interleaved": 1}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


# ------------------------------------------------------ table builder

def test_library_table_builder_matches_oracle(orc):
    for R, rows, B, g, c in [(128, 4096, 512.0, 0.4, 2048.0), (64, 100, 32.0, 0.4, 0.0)]:
        zq, zk = rp.rope_build_xpos_table(rows, R, B, g, c)
        oq, ok = oracle.xpos_table(R, rows, scale_base=B, gamma=g, center=c)
        assert np.array_equal(zq.numpy(), oq) and np.array_equal(zk.numpy(), ok)


# ------------------------------------------------------- host emulation

@pytest.fixture(scope="module")
def emu():
    os.makedirs(os.path.dirname(EMU_BIN), exist_ok=True)
    with open(EMU_BIN + ".lock", "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        if (not os.path.exists(EMU_BIN) or
                os.path.getmtime(EMU_BIN) < max(os.path.getmtime(p) for p in DEPS)):
            tmp = f"{EMU_BIN}.{os.getpid()}"
            cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-host-only", "-O1",
                   "-g", "-std=c++17", "-ffp-contract=off", "-Xarch_host", "-fsanitize=address",
                   "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
                   "-o", tmp, EMU_SRC]
            subprocess.run(cmd, check=True, capture_output=True)
            os.replace(tmp, EMU_BIN)
    return EMU_BIN


# B S Hq Hk D R dtype pairing layout oop pos_kind direction scale_base center
# and the chunk width the plan picks (0: element shape)
CASES = [
    (1, 37, 3, 1, 64, 64, "bf16", "split_half", "bhsd", False, "none", 1, 512.0, 0.0, 8),
    (2, 19, 4, 2, 128, 96, "f16", "split_half", "bshd", True, "none", -1, 16.0, 9.0, 8),
    (1, 50, 2, 2, 64, 32, "f32", "interleaved", "bhsd", True, "skip", 1, 8.0, 25.0, 4),
    (2, 7, 5, 0, 72, 40, "bf16", "interleaved", "bshd", False, "skip", 1, 4.0, 0.0, 8),
    (1, 30, 2, 1, 65, 64, "f32", "split_half", "bhsd", True, "none", -1, 32.0, 15.0, 1),
    (3, 1, 8, 2, 128, 128, "bf16", "split_half", "bhsd", False, "decode", 1, 512.0, 1000.0, 8),
    (1, 300, 1, 1, 256, 256, "f16", "split_half", "bshd", True, "none", 1, 64.0, 150.0, 8),
    (1, 11, 2, 1, 66, 36, "bf16", "interleaved", "bhsd", True, "skip", -1, 16.0, 3.0, 2),
    (1, 5, 2, 2, 33, 20, "f16", "interleaved", "bshd", False, "none", 1, 8.0, 2.0, 0),
    (2, 9, 3, 1, 34, 32, "bf16", "split_half", "bhsd", True, "none", 1, 64.0, 4.0, 2),
    (1, 13, 2, 2, 68, 64, "f16", "split_half", "bhsd", False, "skip", 1, 32.0, 6.0, 4),
    (1, 200, 3, 0, 12, 12, "f32", "interleaved", "bshd", True, "skip", 1, 2.0, 50.0, 4),
    # enough lanes for 8 heads per lane: one group spans Q and K, the last is
    # ragged; and the token-slow order of views with adjacent heads
    (1, 16384, 5, 5, 64, 64, "bf16", "split_half", "bhsd", False, "none", 1, 512.0, 8192.0, 8),
    (1, 9000, 5, 2, 64, 48, "f16", "interleaved", "bshd", True, "skip", -1, 512.0, 100.0, 8),
    # split-half in place with 16-byte chunks: 4 (f32), 16 and 1 chunks per
    # half, skipped tokens, backward
    (2, 40, 4, 2, 32, 32, "f32", "split_half", "bhsd", False, "skip", -1, 16.0, 10.0, 4),
    (1, 20, 2, 1, 256, 256, "bf16", "split_half", "bhsd", False, "none", 1, 64.0, 5.0, 8),
    (1, 30, 3, 3, 64, 16, "bf16", "split_half", "bhsd", False, "skip", 1, 8.0, 3.0, 8),
]


# The lanes shape (one chunk of one (token, head) per lane, in place,
# 16-byte chunks): the fields above, then the expected form (1 head-major,
# 2 token-major) and heads per workgroup group (head-major).
LANES_CASES = [
    (2, 300, 6, 2, 128, 128, "bf16", "split_half", "bhsd", False, "skip", 1, 512.0, 100.0, 8,
     1, 8),
    (1, 100, 9, 3, 128, 128, "bf16", "split_half", "bhsd", False, "none", -1, 64.0, 50.0, 8,
     1, 8),
    (1, 60, 6, 2, 64, 64, "f32", "split_half", "bhsd", False, "none", 1, 32.0, 20.0, 4, 1, 8),
    (2, 50, 8, 2, 128, 128, "bf16", "split_half", "bshd", False, "none", 1, 512.0, 25.0, 8,
     2, 1),
    (1, 40, 4, 4, 64, 64, "f16", "interleaved", "bshd", False, "skip", -1, 16.0, 10.0, 8, 2, 1),
    (3, 1, 5, 3, 64, 64, "bf16", "interleaved", "bhsd", False, "decode", 1, 8.0, 3.0, 8, 1, 8),
    # heads 16 MiB apart: the long-sequence workgroups (chunks x 2 tokens x 8 heads)
    (1, 32768, 6, 2, 128, 128, "f32", "split_half", "bhsd", False, "none", 1, 512.0, 16384.0,
     4, 1, 8),
]


def case_id(c):
    return "-".join(str(x) for x in c[:12])


def _positions(kind, B, S, rows, seed):
    if kind == "none":
        return None, 0
    g = np.random.default_rng(seed)
    if kind == "skip":  # a shared row with skipped and out-of-table entries
        p = g.integers(0, rows, S).astype(np.int32)
        p[::5] = -1
        p[3::7] = rows + 2
        return p, 0
    if kind == "decode":  # one position per batch row
        return g.integers(0, rows, B).astype(np.int32), 1
    raise ValueError(kind)


def _case_data(c, seed=9500):
    B, S, Hq, Hk, D, R, dtype, pairing, layout, oop, pkind, direction, sb, center = c[:14]
    shape_q = (B, Hq, S, D) if layout == "bhsd" else (B, S, Hq, D)
    shape_k = (B, Hk, S, D) if layout == "bhsd" else (B, S, Hk, D)
    q = W.normal(shape_q, dtype, seed)
    k = W.normal(shape_k, dtype, seed + 1) if Hk else None
    rows = max(S, 64) + 3
    pos, pbs = _positions(pkind, B, S, rows, seed + 2)
    cos, sin = oracle.table(10000.0, R, rows)
    zq, zk = oracle.xpos_table(R, rows, scale_base=sb, gamma=0.4, center=center)
    return q, k, pos, pbs, rows, cos, sin, zq, zk


def _expected(c, q, k, pos, pbs, rows):
    B, S, Hq, Hk, D, R, dtype, pairing, layout, oop, pkind, direction, sb, center = c[:14]
    kw = dict(layout=layout, pairing=pairing, direction=direction, rotary_dim=R, pos=pos,
              pos_batch_stride=pbs, table_rows=rows, scale_base=sb, gamma=0.4, center=center)
    eq = oracle.rope_xpos(oracle.torch_to_storage(q), dtype, is_key=False, **kw)
    ek = None if k is None else oracle.rope_xpos(oracle.torch_to_storage(k), dtype,
                                                 is_key=True, **kw)
    return eq, ek


def _strides(shape, layout):
    B, A, C, D = shape
    if layout == "bhsd":   # [B,H,S,D]: (sb, sh, ss)
        return A * C * D, C * D, D
    return A * C * D, D, C * D  # [B,S,H,D]: sb, sh = D, ss = H*D


def _ord32(bits):
    b = bits.astype(np.int64)
    mag = b & 0x7FFFFFFF
    return np.where(b & 0x80000000, -mag, mag)


def check(got, ref, dtype, what):
    if dtype == "f32":
        d = np.abs(_ord32(got.view(np.uint32)) - _ord32(ref.view(np.uint32)))
        assert int(d.max()) <= 2, f"{what}: {int(d.max())} float32 ulps apart"
    else:
        d = np.abs(P.ord16(got) - P.ord16(ref))
        assert int(d.max()) <= P.ORD_TOL, f"{what}: {int(d.max())} units apart"


def run_emu(emu, c, q, k, pos, pbs, rows, cos, sin, zq, zk):
    B, S, Hq, Hk, D, R, dtype, pairing, layout, oop, pkind, direction, sb, center = c[:14]
    qs = oracle.torch_to_storage(q)
    ks = None if k is None else oracle.torch_to_storage(k)
    with tempfile.TemporaryDirectory() as job:
        qsb, qsh, qss = _strides(q.shape, layout)
        desc = dict(B=B, S=S, D=D, R=R, Hq=Hq, Hk=Hk, dtype=DT[dtype], pairing=PAIR[pairing],
                    direction=direction, oop=int(oop), qn=qs.size, kn=0 if ks is None else ks.size,
                    tn=cos.size, pn=0 if pos is None else pos.size, table_rows=rows,
                    t_row=R // 2, t_col=1, pos_bs=pbs, qsb=qsb, qsh=qsh, qss=qss)
        if ks is not None:
            desc.update(zip(("ksb", "ksh", "kss"), _strides(k.shape, layout)))
        with open(os.path.join(job, "desc.txt"), "w") as f:
            for key, v in desc.items():
                f.write(f"{key} {int(v)}\n")
        qs.tofile(os.path.join(job, "q.bin"))
        if ks is not None:
            ks.tofile(os.path.join(job, "k.bin"))
        for name, arr in (("cos", cos), ("sin", sin), ("zq", zq), ("zk", zk)):
            arr.tofile(os.path.join(job, f"{name}.bin"))
        if pos is not None:
            pos.tofile(os.path.join(job, "pos.bin"))
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
        r = subprocess.run([emu, job], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stdout + r.stderr[-4000:]
        out = dict(line.split() for line in r.stdout.strip().splitlines())
        status = int(out["status"])
        if status:
            return status, None, None
        run_emu.last_vec = int(out["vec"])
        run_emu.last_group = int(out["heads_per_group"])
        run_emu.last_lanes = int(out["lanes"])
        go = np.fromfile(os.path.join(job, "q_out.bin"), dtype=qs.dtype).reshape(qs.shape)
        gk = None if ks is None else np.fromfile(os.path.join(job, "k_out.bin"),
                                                 dtype=ks.dtype).reshape(ks.shape)
        return 0, go, gk


@pytest.mark.parametrize("c", LANES_CASES, ids=case_id)
def test_emulated_lanes_shape_matches_oracle(orc, emu, c):
    q, k, pos, pbs, rows, cos, sin, zq, zk = _case_data(c)
    status, gq, gk = run_emu(emu, c, q, k, pos, pbs, rows, cos, sin, zq, zk)
    assert status == 0
    assert (run_emu.last_vec, run_emu.last_lanes) == (c[14], c[15])
    if c[15] == 1:
        assert run_emu.last_group == c[16]
    eq, ek = _expected(c, q, k, pos, pbs, rows)
    check(gq, eq, c[6], "q")
    if ek is not None:
        check(gk, ek, c[6], "k")


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_emulated_kernel_matches_oracle(orc, emu, c):
    q, k, pos, pbs, rows, cos, sin, zq, zk = _case_data(c)
    status, gq, gk = run_emu(emu, c, q, k, pos, pbs, rows, cos, sin, zq, zk)
    assert status == 0
    assert run_emu.last_vec == c[14]  # the shape this case is meant to cover
    if c[1] * c[4] >= 9000 * 64:
        # 8 heads per lane; views with adjacent heads run one head per lane
        assert run_emu.last_group == (1 if c[8] == "bshd" else 8)
    eq, ek = _expected(c, q, k, pos, pbs, rows)
    dtype = c[6]
    check(gq, eq, dtype, "q")
    if ek is not None:
        check(gk, ek, dtype, "k")
    # pass-through lanes are bit-exact (dims >= R; skipped tokens)
    R = c[5]
    for g, e in ((gq, eq), (gk, ek)):
        if g is None:
            continue
        gb = g.view(np.uint32) if dtype == "f32" else g
        eb = e.view(np.uint32) if dtype == "f32" else e
        assert np.array_equal(gb[..., R:], eb[..., R:])


# ------------------------------------------------------------ the C ABI

def _abi_desc(**over):
    """A valid rope_apply descriptor for a [1, 2, 8, 64] bf16 Q/K pair at fake
    16-byte aligned addresses (nothing is dereferenced on the error paths)."""
    A = 1 << 40
    d = rp.RopeApplyDesc()
    d.batch, d.seq_len, d.head_dim, d.rotary_dim = 1, 8, 64, 64
    d.n_heads_q, d.n_heads_k = 2, 1
    d.dtype, d.pairing, d.launch, d.direction = 2, 0, 0, 1
    d.q_in = rp.RopeView(A, 2 * 8 * 64, 8 * 64, 64)
    d.k_in = rp.RopeView(A + 65536, 8 * 64, 8 * 64, 64)
    d.cos, d.sin = A + 2 * 65536, A + 3 * 65536
    d.table_rows = 8
    d.table_col_stride = 1
    d.angles = 0
    for key, v in over.items():
        setattr(d, key, v)
    return d


def _call(d, zq=(1 << 40) + 4 * 65536, zk=(1 << 40) + 5 * 65536):
    import ctypes
    return rp.lib().rope_apply_xpos(ctypes.byref(d), zq, zk, None)


def test_abi_validation():
    OK, NULL, SHAPE, LAYOUT, ALIGN, ALIAS = 0, -1, -2, -4, -5, -6
    assert _call(_abi_desc(angles=1, theta=10000.0, interpolate_factor=1.0)) == LAYOUT
    assert _call(_abi_desc(launch=1)) == LAYOUT
    assert _call(_abi_desc(), zq=None) == NULL
    assert _call(_abi_desc(), zk=None) == NULL
    assert _call(_abi_desc(), zq=(1 << 40) + 4 * 65536 + 2) == ALIGN
    # no K heads: no key table needed (the next check to fail is Q's table)
    assert _call(_abi_desc(n_heads_k=0), zq=(1 << 40) + 4 * 65536 + 2, zk=None) == ALIGN
    assert _call(_abi_desc(), zk=(1 << 40) + 64) == ALIAS    # inside Q, written in place
    assert _call(_abi_desc(rotary_dim=63)) == SHAPE
    assert _call(_abi_desc(seq_len=0), zq=None, zk=None) == OK   # empty: nothing to do
    import ctypes
    assert rp.lib().rope_apply_xpos(None, None, None, None) == NULL


def test_abi_table_builder_errors():
    import ctypes
    L = rp.lib()
    buf = (ctypes.c_float * 64)()
    SHAPE, NULL = -2, -1
    for args in [(4, 17, 512.0, 0.4, 0.0), (4, 16, 0.0, 0.4, 0.0), (4, 16, 512.0, -1.0, 0.0),
                 (4, 16, float("inf"), 0.4, 0.0), (4, 16, 512.0, 0.4, float("nan")),
                 (-1, 16, 512.0, 0.4, 0.0)]:
        assert L.rope_build_xpos_table(buf, buf, *args) == SHAPE, args
    assert L.rope_build_xpos_table(None, buf, 4, 16, 512.0, 0.4, 0.0) == NULL
    assert L.rope_build_xpos_table(None, None, 0, 16, 512.0, 0.4, 0.0) == 0


# ------------------------------------------------------------ on the GPU

def _gpu_call(c, q, k, pos, pbs, rows, cos, sin, zq, zk, stream=None):
    B, S, Hq, Hk, D, R, dtype, pairing, layout, oop, pkind, direction, sb, center = c[:14]
    dev = "cuda"
    qd = q.to(dev)
    kd = None if k is None else k.to(dev)
    kw = dict(layout=layout, pairing=pairing, rotary_dim=R, direction=direction)
    if pos is not None:
        kw["pos"] = torch.from_numpy(pos).to(dev)
        kw["pos_batch_stride"] = pbs
    if oop:
        kw["q_out"] = torch.empty_like(qd)
        if kd is not None:
            kw["k_out"] = torch.empty_like(kd)
    t = [torch.from_numpy(a).to(dev) for a in (cos, sin, zq, zk)]
    oq, ok = rp.rope_apply_xpos(qd, kd, t[0], t[1], t[2], t[3], **kw)
    torch.cuda.synchronize()
    return (oracle.torch_to_storage(oq.cpu()),
            None if ok is None else oracle.torch_to_storage(ok.cpu()))


@pytest.mark.gpu
@pytest.mark.parametrize("c", CASES + LANES_CASES, ids=case_id)
def test_gpu_matches_oracle(orc, c):
    print(f"xpos case {case_id(c)}", flush=True)
    q, k, pos, pbs, rows, cos, sin, zq, zk = _case_data(c)
    gq, gk = _gpu_call(c, q, k, pos, pbs, rows, cos, sin, zq, zk)
    eq, ek = _expected(c, q, k, pos, pbs, rows)
    check(gq, eq, c[6], "q")
    if ek is not None:
        check(gk, ek, c[6], "k")


@pytest.mark.gpu
@pytest.mark.parametrize("direction", [1, -1])
def test_gpu_full_llama_size(orc, direction):
    # the Llama GQA prefill shape in place, every element against the oracle
    w = W.LLAMA_GQA_PREFILL
    c = (w.batch, w.seq_len, w.n_heads_q, w.n_heads_k, w.head_dim, w.rotary_dim, w.dtype,
         w.pairing, w.layout, False, "none", direction, 512.0, w.seq_len / 2, 8)
    print(f"xpos full size, direction {direction}", flush=True)
    t = W.tensors(w, ("q", "k"))
    rows = w.table_rows
    cos, sin = oracle.table(w.theta, w.rotary_dim, rows)
    zq, zk = oracle.xpos_table(w.rotary_dim, rows, scale_base=512.0, gamma=0.4,
                               center=w.seq_len / 2)
    gq, gk = _gpu_call(c, t["q"], t["k"], None, 0, rows, cos, sin, zq, zk)
    eq, ek = _expected(c, t["q"], t["k"], None, 0, rows)
    check(gq, eq, w.dtype, "q")
    check(gk, ek, w.dtype, "k")


# ------------------------------------------------ seeded random configurations

def random_case(seed: int, budget: int) -> tuple:
    """One case in the tuple form above (its first 14 fields), drawn from
    `seed`: sizes, dtype, pairing, layout, in/out of place, positions,
    direction and the XPOS parameters; Q + K hold at most about `budget`
    elements."""
    r = np.random.RandomState(seed)
    dtype = str(r.choice(["f32", "f16", "bf16"]))
    pairing = str(r.choice(["split_half", "interleaved"]))
    layout = str(r.choice(["bhsd", "bshd"]))
    D = int(r.choice([8, 16, 32, 40, 64, 66, 72, 96, 128, 256]))
    R = D - D % 2 if r.rand() < 0.6 else 2 * int(r.randint(1, D // 2 + 1))
    Hq = int(r.choice([1, 2, 3, 5, 8, 12, 16, 32]))
    Hk = int(r.randint(0, Hq + 1))
    B = int(r.choice([1, 2, 3]))
    S = int(r.choice([1, 2, 9, 64, 100, 300, 700]))
    S = max(1, min(S, budget // max(1, B * (Hq + Hk) * D)))
    pkind = str(r.choice(["none", "none", "skip"])) if S > 1 else str(r.choice(["none",
                                                                                 "decode"]))
    oop = bool(r.rand() < 0.3)
    direction = int(r.choice([1, -1]))
    sb = float(r.choice([2.0, 16.0, 512.0]))
    center = float(r.randint(0, S + 1))
    return (B, S, Hq, Hk, D, R, dtype, pairing, layout, oop, pkind, direction, sb, center)


def _check_random(c, gq, gk):
    q, k, pos, pbs, rows, cos, sin, zq, zk = _case_data(c, seed=9600)
    eq, ek = _expected(c, q, k, pos, pbs, rows)
    check(gq, eq, c[6], "q")
    if ek is not None:
        check(gk, ek, c[6], "k")


@pytest.mark.parametrize("case", range(40))
def test_emulated_random_cases(orc, emu, case):
    c = random_case(31000 + case, 120_000)
    q, k, pos, pbs, rows, cos, sin, zq, zk = _case_data(c, seed=9600)
    status, gq, gk = run_emu(emu, c, q, k, pos, pbs, rows, cos, sin, zq, zk)
    assert status == 0, c
    _check_random(c, gq, gk)


# LIBROPE_RANDOM_SCALE=n runs n times as many GPU cases (a longer sweep on demand)
GPU_RANDOM_CASES = 60 * int(os.environ.get("LIBROPE_RANDOM_SCALE", "1"))


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(GPU_RANDOM_CASES))
def test_gpu_random_cases(orc, case):
    c = random_case(32000 + case, 2_000_000)
    print(f"xpos random case {case}: {c}", flush=True)
    q, k, pos, pbs, rows, cos, sin, zq, zk = _case_data(c, seed=9600)
    gq, gk = _gpu_call(c, q, k, pos, pbs, rows, cos, sin, zq, zk)
    _check_random(c, gq, gk)

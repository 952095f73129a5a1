"""Every address of the fused attention kernel, checked on the host.

tests/emu/attn_bounds.hip plans each call exactly as the library does and
walks every workgroup, lane and key tile of the planned grid through the
kernel's own index functions: each Q/K/V/O, cos/sin and position access must
fall inside its buffer. The double-buffered tile pipeline is simulated phase
by phase: staging writes land in their tile's buffer, no LDS cell is written
by two lanes in one phase, no cell is both read and written in one phase,
and every cell read for tile kt holds tile kt. Small grids at head dim 64
take 2 or 4 wave groups (the groups take turns on the key tiles with their
own buffers and merge their softmax states through LDS at the end): the
walk follows each group and checks the merge's LDS slots.
The walk runs under AddressSanitizer, so the position reads are real reads
of index arrays of exact size.
"""
import fcntl
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "emu", "attn_bounds.hip")
BIN = os.path.join(ROOT, "tests", "emu", "_build", "attn_bounds")
CSRC = os.path.join(ROOT, "rotary_position_embedding_fwd_amd", "csrc")
DEPS = [SRC, os.path.join(CSRC, "rope_attention.hpp"), os.path.join(CSRC, "rope_attn_plan.hpp"),
        os.path.join(CSRC, "rope_kernels.hpp"), os.path.join(ROOT, "include", "librope.h")]

SPLIT, INTER = 0, 1

# B Hq Hk Sq Sk D R pairing causal table_rows qpos kpos [k_rotated]
CASES = [
    (1, 2, 1, 130, 130, 128, 128, SPLIT, 0, 200, 0, 0),     # ragged tiles
    (2, 4, 2, 77, 200, 64, 64, SPLIT, 1, 256, 0, 0),        # causal, Sq < Sk
    (1, 2, 2, 129, 129, 128, 64, INTER, 1, 130, 1, 1),      # interleaved, index positions
    (1, 1, 1, 1, 1, 64, 32, SPLIT, 0, 1, 0, 0),             # one query, one key
    (2, 8, 2, 257, 300, 128, 96, SPLIT, 1, 300, 1, 0),      # GQA 4:1, R = 3/4 D
    (1, 3, 1, 64, 65, 64, 8, INTER, 0, 65, 0, 1),           # MQA, the smallest R
    (1, 2, 1, 300, 64, 128, 0, SPLIT, 0, 0, 0, 0),          # no rotation, Sq > Sk
    (1, 2, 1, 3, 500, 128, 128, INTER, 1, 512, 1, 1),       # decode-like Sq
    (1, 8, 8, 1026, 1026, 64, 32, SPLIT, 1, 1024, 1, 1),    # skipped CLS/register tokens
    (1, 2, 1, 64, 64, 128, 32, SPLIT, 0, 64, 0, 0),         # H16 = 1
    (1, 2, 1, 64, 64, 128, 96, SPLIT, 0, 64, 0, 0),         # H16 = 3
    (1, 2, 1, 64, 64, 64, 64, INTER, 1, 64, 0, 0),
    (2, 16, 2, 100, 300, 128, 128, SPLIT, 1, 300, 0, 1),    # 8 heads per workgroup
    (1, 6, 3, 70, 70, 64, 64, SPLIT, 0, 70, 0, 0),          # GQA 2:1
    (1, 12, 1, 40, 520, 128, 64, INTER, 1, 520, 1, 0),      # MQA 12:1 (4 heads per group)
    (1, 16, 2, 70, 140, 128, 128, SPLIT, 1, 140, 0, 0),     # GQA 8:1 (8 heads per group)
    (2, 16, 1, 40, 97, 64, 64, INTER, 0, 97, 1, 1),         # GQA 16:1
    (1, 6, 2, 300, 100, 128, 64, SPLIT, 0, 300, 0, 0),      # GQA 3:1, Sq > Sk
    (8, 4, 2, 33, 65, 64, 32, SPLIT, 1, 65, 1, 1),          # batch 8
    # K arrives rotated (rope_attention_fwd_k_once): the copy-only K staging
    # with Q still rotated in the kernel
    (2, 32, 8, 300, 300, 128, 128, SPLIT, 1, 300, 0, 0, 1),
    (1, 2, 2, 129, 129, 128, 64, INTER, 1, 130, 1, 1, 1),
    (2, 8, 2, 257, 300, 128, 96, SPLIT, 1, 300, 1, 0, 1),
    (1, 8, 8, 1026, 1026, 64, 32, SPLIT, 1, 1024, 1, 1, 1),
    # head dim 64 with a grid of at least 256 workgroups: one wave group
    (4, 32, 8, 520, 520, 64, 64, SPLIT, 1, 520, 0, 0),
    (4, 32, 8, 520, 520, 64, 64, INTER, 0, 520, 1, 1, 1),
    # four groups with 8 query heads per K/V head (2 per workgroup), a tile
    # count that is not a multiple of 4
    (1, 16, 2, 200, 200, 64, 64, SPLIT, 1, 200, 0, 0),
    (1, 16, 2, 200, 200, 64, 32, SPLIT, 0, 200, 1, 1, 1),
    # two groups (128 workgroups unsplit)
    (1, 32, 32, 1024, 1024, 64, 64, SPLIT, 1, 1024, 0, 0),
    (1, 32, 32, 300, 1024, 64, 64, INTER, 0, 1024, 1, 1, 1),
]

# (case, expected wave groups)
GROUP_CHOICE = [
    ((1, 8, 8, 1026, 1026, 64, 32, SPLIT, 1, 1024, 1, 1), 4),   # 40 workgroups unsplit
    ((4, 32, 8, 520, 520, 64, 64, SPLIT, 1, 520, 0, 0), 1),     # 288
    ((1, 2, 1, 130, 130, 128, 128, SPLIT, 0, 200, 0, 0), 1),    # head dim 128: never
    ((1, 16, 2, 200, 200, 64, 64, SPLIT, 1, 200, 0, 0), 4),     # 14, 8 heads -> 2 per group
    ((1, 16, 16, 1024, 1024, 64, 64, SPLIT, 1, 1024, 0, 0), 4),  # 64: 256 with 4 groups
    # 128 workgroups unsplit: 256 with two groups still fit the chip once
    ((1, 32, 32, 1024, 1024, 64, 64, SPLIT, 1, 1024, 0, 0), 2),
    # 192 workgroups unsplit: 384 with two groups would put two on some CUs
    ((1, 48, 48, 1024, 1024, 64, 64, SPLIT, 1, 1024, 0, 0), 1),
]


@pytest.fixture(scope="module")
def harness():
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    with open(BIN + ".lock", "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        if (not os.path.exists(BIN) or
                os.path.getmtime(BIN) < max(os.path.getmtime(p) for p in DEPS)):
            tmp = f"{BIN}.{os.getpid()}"
            cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-host-only", "-O1",
                   "-g", "-std=c++17", "-Xarch_host", "-fsanitize=address",
                   "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
                   "-o", tmp, SRC]
            subprocess.run(cmd, check=True, capture_output=True)
            os.replace(tmp, BIN)
    return BIN


def walk(harness, case):
    r = subprocess.run([harness] + [str(x) for x in case], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = dict(line.split() for line in r.stdout.strip().splitlines())
    return {k: int(v) for k, v in out.items()}, r.stderr


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_every_access_in_bounds(harness, case):
    out, err = walk(harness, case)
    assert out["plan"] == 0
    assert out["accesses"] > 0
    assert out["violations"] == 0, err[-2000:]


def test_rejected_shapes_plan_nothing(harness):
    # head_dim 96 is not built; split-half R must be a multiple of 32
    for case in [(1, 2, 1, 64, 64, 96, 64, SPLIT, 0, 64, 0, 0),
                 (1, 2, 1, 64, 64, 128, 48, SPLIT, 0, 64, 0, 0),
                 (1, 3, 2, 64, 64, 128, 64, SPLIT, 0, 64, 0, 0),
                 (1, 2, 1, 65, 64, 128, 64, SPLIT, 1, 64, 0, 0)]:
        out, _ = walk(harness, case)
        assert out["plan"] < 0
        assert out["accesses"] == 0


@pytest.mark.parametrize("case,groups", GROUP_CHOICE, ids=lambda c: "x".join(map(str, c))
                         if isinstance(c, tuple) else str(c))
def test_wave_group_choice(harness, case, groups):
    out, _ = walk(harness, case)
    assert out["plan"] == 0
    assert out["groups"] == groups

"""Seeded random configurations of the rotation, for the parity sweeps
(tests/test_gpu_random_configs.py on the GPU, tests/test_kernel_emulation.py
on the kernel emulator). Draws only shapes, dtypes, modes and integer
positions; the values come from workloads.normal."""
import numpy as np

import workloads as W


def draw(seed: int, budget: int, views: bool = True) -> dict:
    """One configuration, a pure function of `seed`; Q + K hold at most about
    `budget` elements. views False: contiguous [B,H,S,D] or [B,S,H,D] tensors,
    cos/sin tables, in place (what the kernel emulator takes)."""
    r = np.random.RandomState(seed)
    c = {}
    # a third of the cases come from the shapes the fast kernels take
    # (16-bit, head dim 64 or 128, at least 8 heads, a few hundred tokens)
    common = r.rand() < 1 / 3
    c["dtype"] = str(r.choice(["f16", "bf16"] if common else ["f32", "f16", "bf16"]))
    c["layout"] = str(r.choice(["bhsd", "bshd", "packed"] if views else ["bhsd", "bshd"]))
    c["pairing"] = str(r.choice([W.SPLIT_HALF, W.INTERLEAVED]))
    D = int(r.choice([64, 128] if common else [8, 16, 24, 32, 40, 64, 72, 96, 128, 256]))
    c["head_dim"] = D
    c["rotary_dim"] = D if common or r.rand() < 0.6 else 2 * int(r.randint(1, D // 2 + 1))
    Hq = int(r.choice([8, 16, 32] if common else [1, 2, 3, 4, 5, 8, 12, 16, 32, 40]))
    c["n_heads_q"] = Hq
    c["n_heads_k"] = Hq if r.rand() < 0.3 else int(r.randint(1, Hq + 1))
    c["batch"] = int(r.choice([1, 2, 3, 4]))
    S = int(r.choice([129, 257, 700] if common else [1, 2, 7, 64, 100, 129, 257, 513, 700,
                                                      1000]))
    per_token = c["batch"] * (Hq + c["n_heads_k"]) * D
    c["seq_len"] = max(1, min(S, budget // per_token))
    S = c["seq_len"]
    c["theta"] = float(r.choice([10000.0, 500000.0]))
    c["angles"] = "theta" if r.rand() < (0.05 if common else 0.2) and views else "table"
    c["direction"] = int(r.choice([1, -1]))
    c["out_of_place"] = bool(r.rand() < (0.05 if common else 0.25)) and views
    if r.rand() < (0.1 if common else 0.35):
        # an index row: skipped (-1, -2) and out-of-table entries among the rest
        c["table_rows"] = int(r.randint(1, 2 * S + 10))
        c["pos_batch_stride"] = int(r.choice([0, S]))
        n = S if c["pos_batch_stride"] == 0 else c["batch"] * S
        c["pos"] = r.randint(-2, c["table_rows"] + 3, size=n).astype(np.int32)
    else:
        c["table_rows"] = S + int(r.randint(0, 100))
        c["pos_batch_stride"] = None
        c["pos"] = None
    c["seed"] = seed + 200
    return c


def workload(c) -> W.Workload:
    return W.Workload(f"random_{c['seed']}", 0, c["batch"], c["n_heads_q"], c["n_heads_k"],
                      c["seq_len"], c["head_dim"], c["rotary_dim"], c["dtype"],
                      W.BHSD if c["layout"] == "bhsd" else W.BSHD, c["pairing"], c["theta"],
                      c["table_rows"])

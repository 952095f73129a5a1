"""Host-side logic of bench.py, on the CPU: algorithmic bytes, counter summary,
and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("w,expected", [
    # 2 * e * R * tokens * (Hq + Hk) + 4 * R * distinct positions + 4 * index entries
    (W.TINY_F32, 2 * 4 * 64 * 128 * 16 + 4 * 64 * 128),
    (W.LLAMA_GQA_PREFILL, 2 * 2 * 128 * 16384 * 40 + 4 * 128 * 4096),
    (W.BSHD_INTERLEAVED, 2 * 2 * 64 * 16384 * 32 + 4 * 64 * 2048),
    (W.LONG_CONTEXT, 2 * 2 * 128 * 131072 * 40 + 4 * 128 * 131072),
    # two masked tokens; 1024 distinct positions shared by both sequences; 1026 indices
    (W.PARTIAL_INDEXED, 2 * 2 * 32 * (2 * 1024) * 24 + 4 * 32 * 1024 + 4 * 1026),
])
def test_algorithmic_bytes(w, expected):
    assert bench.algorithmic_bytes(w, W.positions(w)) == expected


def test_algorithmic_bytes_decode_counts_distinct_rows():
    pos = W.positions(W.DECODE)
    distinct = len(set(pos.tolist()))
    assert bench.algorithmic_bytes(W.DECODE, pos) == (2 * 2 * 128 * 256 * 40 + 4 * 128 * distinct
                                                     + 4 * 256)


BENCH_LINE = {
    "warmup": 2, "steps": 3,
    "config": {"workload": "llama_gqa_prefill_bf16", "algorithmic_bytes_per_call": 1000},
    "roofline": {"launch": "rope_head_lanes_kernel dtype=bf16 vec=8 grid=10 block=512",
                 "avg_launch_us": 1.0},
    "configs": [{"workload": "long_context_bf16", "warmup": 1, "steps": 2,
                 "algorithmic_bytes_per_call": 5000, "us_per_launch": 2.0,
                 "kernel": "rope_head_lanes_kernel dtype=bf16 vec=8 grid=20 block=640"}],
}


def test_pmc_summary_scales_by_the_copy(tmp_path):
    header = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,"
              "Kernel_Id,Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,"
              "Accum_VGPR_Count,SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,"
              "End_Timestamp\n")
    kern = "void rope::rope_head_lanes_kernel<__bf16, 8, 0, true, false>(rope::Args)"

    def write(d, counter, rows):
        os.makedirs(d / "host", exist_ok=True)
        with open(d / "host" / "x_counter_collection.csv", "w") as f:
            f.write(header)
            for i, (name, grid, wg, v) in enumerate(rows):
                f.write(f'{i},{i},"Agent 1",1,1,1,{grid},1,"{name}",{wg},0,0,8,0,8,'
                        f'"{counter}",{v},0,1\n')

    fd, wd = tmp_path / "f", tmp_path / "w"
    # two launches of the Llama grid (10 x 512), one of the long-context grid (20 x 640)
    cp = "__amd_rocclr_copyBuffer"
    # a device clone (the bench's own) before the launches, then the three
    # calibration copies of 1 GiB at the end
    write(fd, "FETCH_SIZE", [(cp, 1, 1, 1000.0), (kern, 5120, 512, 100.0),
                             (kern, 5120, 512, 102.0), (kern, 12800, 640, 700.0),
                             ("void at::native::vectorized_elementwise_kernel", 1, 1, 1.0)] +
          [(cp, 1, 1, 524288.0)] * 3)
    write(wd, "WRITE_SIZE", [(cp, 1, 1, 2000.0), (kern, 5120, 512, 200.0),
                             (kern, 5120, 512, 200.0), (kern, 12800, 640, 900.0)] +
          [(cp, 1, 1, 1048576.0)] * 3)
    bj = tmp_path / "b.json"
    bj.write_text("noise\n" + json.dumps(BENCH_LINE) + "\n")
    out = tmp_path / "t.json"
    bench.summarize_pmc(str(fd), str(wd), str(bj), out=str(out))
    t = json.load(open(out))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    llama = t["workloads"]["llama_gqa_prefill_bf16"]
    assert llama["bytes_per_launch"] == round(101.0 * 1024 * 2 + 200.0 * 1024)
    assert llama["dispatches"] == [2, 2]
    assert t["workloads"]["long_context_bf16"]["bytes_per_launch"] == round(
        700.0 * 1024 * 2 + 900.0 * 1024)
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


def test_trace_summary_drops_warmup_and_matches_grids(tmp_path):
    """Only the timed launches of each workload's kernel (matched by name and
    grid, in dispatch order, after its warmup) enter the summary."""
    d = tmp_path / "trace" / "host"
    os.makedirs(d)
    kern = "void rope::rope_head_lanes_kernel<__bf16, 8, 0, true, false>(rope::Args)"
    rows = []
    # Llama: a settle phase and 2 warmup steps (slow), then 3 timed steps (6 launches)
    rows += [(kern, 512, 5120, 9000)] * 11 + [(kern, 512, 5120, 1000)] * 6
    rows += [("stream_rmw_kernel", 64, 100, 5)]
    # long context: 1 warmup step then 2 timed steps
    rows += [(kern, 640, 12800, 9000)] * 2 + [(kern, 640, 12800, 2000)] * 4
    with open(d / "x_kernel_trace.csv", "w") as f:
        f.write("Kind,Dispatch_Id,Kernel_Name,Workgroup_Size_X,Grid_Size_X,Start_Timestamp,"
                "End_Timestamp\n")
        t = 0
        for i, (name, wg, grid, dur) in enumerate(rows):
            f.write(f'KERNEL_DISPATCH,{i + 1},"{name}",{wg},{grid},{t},{t + dur}\n')
            t += dur + 10
    bj = tmp_path / "b.json"
    bj.write_text(json.dumps(BENCH_LINE) + "\n")
    import io
    import contextlib
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        bench.summarize_trace(str(tmp_path / "trace"), str(bj))
    res = json.loads(buf.getvalue())
    a, b = res["workloads"]
    assert (a["launches"], a["mean_us"], a["max_us"], a["settle_and_warmup_dropped"]) == (
        6, 1.0, 1.0, 11)
    assert (b["launches"], b["mean_us"], b["settle_and_warmup_dropped"]) == (4, 2.0, 2)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_attention_flops_count_visible_pairs():
    # causal with Sq == Sk: query i sees i + 1 keys, S (S + 1) / 2 pairs per head
    w = W.ATTN_LLAMA_PREFILL
    S = w.seq_len_q
    assert bench.attention_flops(w) == 4 * w.head_dim * (S * (S + 1) // 2) * w.batch * w.n_heads_q
    # non-causal: every pair; causal with Sq < Sk: the last Sq rows of the square
    assert bench.attention_flops(w.scaled(causal=False)) == 4 * 128 * S * S * 4 * 32
    v = w.scaled(seq_len_q=3, seq_len_k=10, batch=1, n_heads_q=1)
    assert bench.attention_flops(v) == 4 * 128 * (8 + 9 + 10)

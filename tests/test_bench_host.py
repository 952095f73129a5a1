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


def test_pmc_summary_scales_by_the_copy(tmp_path, monkeypatch):
    header = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,"
              "Kernel_Id,Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,"
              "Accum_VGPR_Count,SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,"
              "End_Timestamp\n")
    kern = "_ZN4rope22rope_pair_lanes_kernelIDF16bLi8ELi4EEEvNS_4ArgsE"

    def write(d, counter, rows):
        os.makedirs(d / "host", exist_ok=True)
        with open(d / "host" / "x_counter_collection.csv", "w") as f:
            f.write(header)
            for i, (name, v) in enumerate(rows):
                f.write(f'{i},{i},"Agent 1",1,1,1,1,1,"{name}",256,0,0,8,0,8,"{counter}",{v},0,1\n')

    fd, wd = tmp_path / "f", tmp_path / "w"
    write(fd, "FETCH_SIZE", [(kern, 100.0), (kern, 102.0), ("__amd_rocclr_copyBuffer", 524288.0),
                             ("void at::native::vectorized_elementwise_kernel", 1.0)])
    write(wd, "WRITE_SIZE", [(kern, 200.0), (kern, 200.0),
                             ("__amd_rocclr_copyBuffer", 1048576.0)])
    out = tmp_path / "t.json"
    bench.summarize_pmc(str(fd), str(wd), out=str(out))
    t = json.load(open(out))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["bytes_per_launch"] == round(101.0 * 1024 * 2 + 200.0 * 1024)
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


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

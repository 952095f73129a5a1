#!/usr/bin/env python3
"""Benchmark of librope's fused Q+K RoPE on one MI355X.

One step = the whole hot path once over one batch of the Llama-style GQA
prefill workload (bf16, Q [4, 32, 4096, 128], K [4, 8, 4096, 128], split-half
pairs, fp32 cos/sin tables [4096, 64], theta 10000): the forward rotation of
Q and K in place, then the backward rotation of the incoming gradients dQ,
dK in place. Inputs are resident in HBM before timing starts. Each step uses
the next of several buffer sets, whose total exceeds the 256 MB Infinity
Cache, so a step does not find its operands in cache from an earlier step.

Printed: one JSON line. `value` is achieved GB/s over the algorithmic bytes
(read + write of the rotated part of every Q/K row once, each cos/sin row
once, the indices once). It carries a `roofline` object for the dominant
kernel (its launch duration measured with HIP events on the launch stream),
`configs` with the same measurement on the other two large prefill
workloads (BSHD interleaved fp16 and long context), the in-place stream
ceiling at each workload's size, a `cpu_baseline` (the CPU oracle timed on
the host, one thread and all host threads) and the decode-shape µs/call.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --summarize-trace TRACE_DIR BENCH_JSON   (rocprofv3 kernel trace
        of a bench run -> per-kernel durations of the timed launches only)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused QK RoPE fwd+bwd achieved HBM GB/s (% of peak); µs/call at decode shape"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "rotary_position_embedding_fwd_amd", "csrc", f)
                  for f in ("rope_kernels.hpp", "rope_plan.hpp", "librope.hip")]
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_prefill_workloads.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, pos, tables: bool = True) -> int:
    """Bytes the method must move for one call on workload w.

    read + write of the first R dims of every rotated Q and K row, each
    distinct cos/sin row once (2 tables x R/2 x 4 B; none when the angles are
    computed from theta), each index once.
    """
    import numpy as np
    e = 4 if w.dtype == "f32" else 2
    R = w.rotary_dim
    rows_h = w.n_heads_q + w.n_heads_k
    if pos is None:
        n_tok = w.batch * w.seq_len
        distinct = w.seq_len
        idx_bytes = 0
    else:
        p = pos.numpy().astype(np.int64)
        bs = w.pos_batch_stride
        idx = (np.arange(w.batch)[:, None] * bs + np.arange(w.seq_len)[None, :]).ravel()
        pv = p[idx]
        valid = (pv >= 0) & (pv < w.table_rows)
        n_tok = int(valid.sum())
        distinct = int(np.unique(pv[valid]).size)
        idx_bytes = 4 * int(np.unique(idx).size)
    rotated = e * R * n_tok * rows_h
    return 2 * rotated + (4 * R * distinct if tables else 0) + idx_bytes


def device_inputs(w, sets: int, which=("q", "k", "dq", "dk"), grads_from_qk: bool = False):
    """Seeded host tensors and `sets` device copies. grads_from_qk: draw only
    q and k on the host and give each set dq, dk as device copies of them
    (the values do not change the timing; drawing them costs seconds of host
    time on the long-context shape)."""
    import workloads as W
    draw = ("q", "k") if grads_from_qk else which
    t = W.tensors(w, draw)
    out = []
    for i in range(sets):
        d = {k: v.to("cuda") for k, v in t.items()}
        if grads_from_qk:
            d["dq"], d["dk"] = d["q"].clone(), d["k"].clone()
        out.append(d)
    return t, out


SETTLE_MS = 100.0


def settle(step, ms: float = SETTLE_MS):
    """Run `step` untimed until `ms` of wall time have passed: the GPU's
    clocks rise to their sustained level only after tens of milliseconds of
    load (measured on MI355X: timed windows straight after idle vary by up to
    20 % for a 23 µs kernel, and are steady after 50 ms of work)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1000.0 < ms:
        for _ in range(8):
            step(i)
            i += 1
        torch.cuda.synchronize()


def time_prefill(w, steps: int, warmup: int, sets: int, grads_from_qk: bool = False):
    """Time `steps` steps back to back between two HIP events on the launch
    stream. Forward and backward are the same kernel (the sign of sin is an
    argument), so the region divided by 2 * steps is that kernel's average
    launch duration, inter-launch gaps included."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    pos = W.positions(w)
    cos, sin = rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta)
    cos, sin = cos.cuda(), sin.cuda()
    host, bufs = device_inputs(w, sets, grads_from_qk=grads_from_qk)
    stream = torch.cuda.current_stream()
    kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim,
              pos=None if pos is None else pos.cuda(), stream=stream)
    fwd = [rp.prepare(b["q"], b["k"], cos, sin, **kw) for b in bufs]
    bwd = [rp.prepare(b["dq"], b["dk"], cos, sin, **kw) for b in bufs]
    kw.pop("stream")
    kernel = rp.rope_describe(bufs[0]["q"], bufs[0]["k"], cos, sin, **kw)

    def step(i):
        fwd[i % sets].rope_fwd_qk()
        bwd[i % sets].rope_bwd_qk()

    settle(step)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        step(warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    del fwd, bwd, bufs
    torch.cuda.empty_cache()
    return dict(total_ms=total_ms, wall_s=wall, pos=pos, host=host, kernel=kernel)


def _kernel_fields(desc: str) -> dict:
    """rope_describe's line split into the kernel name and its key=value fields."""
    parts = desc.split()
    out = {"name": parts[0]}
    for p in parts[1:]:
        if "=" in p:
            k, v = p.split("=", 1)
            out[k] = int(v) if v.lstrip("-").isdigit() else v
    return out


# The other large prefill workloads, measured like the headline step:
# (workload, steps, warmup, buffer sets). Sets are sized so one cycle of
# them exceeds the 256 MB Infinity Cache.
EXTRA_CONFIGS = (("BSHD_INTERLEAVED", 200, 40, 4), ("LONG_CONTEXT", 20, 10, 2))


def time_config(w, steps: int, warmup: int, sets: int, ceiling: bool = True):
    """One workload's fwd+bwd steps in place, as the headline step; beside it
    the in-place stream ceiling over a buffer of the same Q+K size."""
    r = time_prefill(w, steps, warmup, sets, grads_from_qk=True)
    per_call = algorithmic_bytes(w, r["pos"])
    avg_us = r["total_ms"] * 1000.0 / (2 * steps)
    gbs = per_call / (avg_us * 1e-6) / 1e9
    out = {"workload": w.name, "q_shape": list(w.q_shape), "k_shape": list(w.k_shape),
           "storage_dtype": w.dtype, "layout": w.layout, "pairing": w.pairing,
           "rotary_dim": w.rotary_dim, "table": [w.table_rows, w.rotary_dim // 2],
           "theta": w.theta, "step": "rope_fwd_qk(Q,K) + rope_bwd_qk(dQ,dK), in place",
           "steps": steps, "warmup": warmup, "buffer_sets": sets,
           "algorithmic_bytes_per_call": per_call,
           "us_per_launch": round(avg_us, 3), "GBps": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "kernel": r["kernel"], "traffic": stored_traffic(w.name)}
    if ceiling:
        e = 4 if w.dtype == "f32" else 2
        qk = e * w.head_dim * w.batch * w.seq_len * (w.n_heads_q + w.n_heads_k)
        c = stream_ceiling(qk, reps=max(10, steps), sets=max(2, -(-600_000_000 // qk)))
        c["frac_achieved_of_ceiling"] = round(gbs / c["GBps"], 4)
        out["measured_stream_ceiling"] = c
    return out


def time_decode(calls: int = 2000, warmup: int = 50, theta: bool = False):
    """Decode-shape forward calls: back to back from Python, one at a time
    between events, and replayed from a captured HIP graph. theta: angles
    computed from theta through rope_apply instead of read from tables."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    w = W.DECODE
    pos = W.positions(w).cuda()
    cos, sin = rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta)
    cos, sin = cos.cuda(), sin.cuda()
    t = W.tensors(w)
    q, k = t["q"].cuda(), t["k"].cuda()
    stream = torch.cuda.current_stream()
    def make(st):
        if theta:
            c = rp.prepare_apply(q, k, None, None, layout=w.layout, pairing=w.pairing,
                                 rotary_dim=w.rotary_dim, pos=pos, theta=w.theta,
                                 max_positions=w.table_rows, stream=st)
            return c.rope_apply
        return rp.prepare(q, k, cos, sin, layout=w.layout, pairing=w.pairing,
                          rotary_dim=w.rotary_dim, pos=pos, stream=st).rope_fwd_qk
    call = make(stream)
    settle(lambda i: call())
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(calls):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    per_call_us = a.elapsed_time(b) * 1000.0 / calls
    # one launch at a time, events around each
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(200)]
    for e0, e1 in evs:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    kern = sorted(e0.elapsed_time(e1) * 1000.0 for e0, e1 in evs)
    # the same calls replayed from a captured HIP graph: no host launch cost
    per_graph, replays = 100, 20
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.graph(g, stream=side):
        gcall = make(side)
        for _ in range(per_graph):
            gcall()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    graph_us = a.elapsed_time(b) * 1000.0 / (per_graph * replays)
    nbytes = algorithmic_bytes(w, pos.cpu(), tables=not theta)
    desc = ("theta mode (rope_apply)" if theta else
            rp.rope_describe(q, k, cos, sin, layout=w.layout, pairing=w.pairing,
                             rotary_dim=w.rotary_dim, pos=pos))
    return {"workload": w.name, "angles": "theta" if theta else "tables",
            "us_per_call_graph_replay": round(graph_us, 3),
            "empty_kernel_us_per_call_graph_replay": empty_kernel_floor(),
            "us_per_call_back_to_back": round(per_call_us, 3),
            "us_event_pair_median": round(kern[len(kern) // 2], 3),
            "algorithmic_bytes": nbytes, "calls": calls, "warmup": warmup,
            "graph_calls": per_graph * replays, "kernel": desc,
            "note": "graph replay: 100 captured calls per graph replayed 20 times (no host "
                    "launch cost); empty kernel: a one-workgroup kernel replayed the same "
                    "way (the launch floor); back to back: Python ctypes launches, bound by "
                    "the host call rate; event pair: one call between two HIP events, event "
                    "overhead included (not a kernel duration: the kernel-only duration "
                    "comes from the rocprofv3 trace)"}


def _graph_us_per_call(make, per_graph: int = 100, replays: int = 20) -> float:
    """µs per call of make(stream)() replayed from a captured HIP graph of
    `per_graph` calls (no host launch cost), after a settle phase."""
    import torch
    stream = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.graph(g, stream=side):
        call = make(side)
        for _ in range(per_graph):
            call()
    torch.cuda.synchronize()
    settle(lambda i: g.replay())
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1000.0 / (per_graph * replays)


def time_decode_sweep(batches=(1, 4, 16, 64, 128, 256, 512, 1024, 2048)):
    """The decode call (one token per sequence, Q [n, 32, 1, 128], K [n, 8,
    1, 128], bf16, a position per sequence) at several sequence counts n,
    each replayed from a captured graph, beside the empty-kernel floor. A
    least-squares line through (bytes, µs) splits the per-call time into a
    fixed part and a part that grows with the bytes moved."""
    import numpy as np
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    base = W.DECODE
    cos, sin = rp.rope_build_table(base.table_rows, base.rotary_dim, base.theta)
    cos, sin = cos.cuda(), sin.cuda()
    floor = empty_kernel_floor()
    rows = []
    for n in batches:
        w = base.scaled(batch=n)
        pos = W.positions(w).cuda()
        t = W.tensors(w, ("q", "k"))
        q, k = t["q"].cuda(), t["k"].cuda()

        def make(st):
            return rp.prepare(q, k, cos, sin, layout=w.layout, pairing=w.pairing,
                              rotary_dim=w.rotary_dim, pos=pos, stream=st).rope_fwd_qk
        us = _graph_us_per_call(make)
        nbytes = algorithmic_bytes(w, pos.cpu())
        desc = rp.rope_describe(q, k, cos, sin, layout=w.layout, pairing=w.pairing,
                                rotary_dim=w.rotary_dim, pos=pos)
        rows.append({"sequences": n, "algorithmic_bytes": nbytes,
                     "us_per_call_graph_replay": round(us, 3),
                     "us_above_empty_kernel": round(us - floor, 3),
                     "kernel": _kernel_fields(desc)})
        del q, k, t
    # the line through the counts up to the decode shape's 256 sequences
    # (beyond it the operands no longer stay in the L2 caches between calls)
    fit_rows = [r for r in rows if r["sequences"] <= base.batch]
    x = np.array([r["algorithmic_bytes"] for r in fit_rows], dtype=np.float64)
    y = np.array([r["us_per_call_graph_replay"] for r in fit_rows], dtype=np.float64)
    slope, icpt = np.polyfit(x, y, 1)
    return {"workload": "decode_bf16 sweep over sequence count", "rows": rows,
            "empty_kernel_us_per_call_graph_replay": floor,
            "fit": {"fixed_us": round(float(icpt), 3),
                    "fixed_us_above_empty_kernel": round(float(icpt) - floor, 3),
                    "GBps_of_the_growing_part": round(1e-3 / float(slope), 1)},
            "note": "every row: 100 captured calls replayed 20 times on the same buffers; "
                    "fit: least squares of µs per call against algorithmic bytes over the "
                    "rows up to %d sequences" % base.batch}


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "rotary_position_embedding_fwd_amd", "libstream_probe.so")
    lib = ctypes.CDLL(path)
    lib.stream_rmw_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint,
                                     ctypes.c_void_p]
    lib.stream_rmw_probe.restype = ctypes.c_int
    lib.mfma_rate_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.mfma_rate_probe.restype = ctypes.c_int
    return lib


def mfma_ceiling(blocks: int = 1024, iters: int = 4000, reps: int = 5):
    """TFLOP/s that chains of v_mfma_f32_32x32x16_bf16 on register operands
    sustain over the whole GPU (libstream_probe.so): the attainable rate of
    the bf16 matrix cores, beside their published peak."""
    import torch
    lib = _probe_lib()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    settle(lambda i: lib.mfma_rate_probe(out.data_ptr(), blocks, iters, stream.cuda_stream))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        assert lib.mfma_rate_probe(out.data_ptr(), blocks, iters, stream.cuda_stream) == 0
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / reps
    flops = blocks * 4 * iters * 16 * 32768
    return {"kernel": "mfma_rate_kernel (4 chains of v_mfma_f32_32x32x16_bf16 per wave)",
            "flops_per_launch": flops, "avg_launch_us": round(us, 2),
            "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1)}


def stream_ceiling(nbytes: int = 160 << 20, reps: int = 40, sets: int = 4):
    """GB/s of a plain in-place read+write stream (libstream_probe.so) over
    `nbytes` per launch, cycling through `sets` buffers whose total exceeds
    the 256 MB Infinity Cache, launched back to back like the RoPE calls: the
    attainable HBM rate of an operation that reads and writes every byte
    once, at that size."""
    import torch
    lib = _probe_lib()
    nbytes = (nbytes // 16) * 16
    bufs = [torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(sets)]
    stream = torch.cuda.current_stream()
    for i in range(3):
        assert lib.stream_rmw_probe(bufs[i % sets].data_ptr(), nbytes, 0,
                                    stream.cuda_stream) == 0
    settle(lambda i: lib.stream_rmw_probe(bufs[i % sets].data_ptr(), nbytes, 0,
                                          stream.cuda_stream))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        lib.stream_rmw_probe(bufs[i % sets].data_ptr(), nbytes, 0, stream.cuda_stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / reps
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "stream_rmw_kernel (16 B non-temporal load + store per lane)",
            "bytes_per_launch": 2 * nbytes, "buffer_sets": sets, "avg_launch_us": round(us, 2),
            "GBps": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}


def empty_kernel_floor(calls: int = 100, replays: int = 20):
    """µs per call of a one-workgroup kernel on 1 KiB, replayed from a captured
    HIP graph: the launch floor under the decode measurement."""
    import torch
    lib = _probe_lib()
    buf = torch.zeros(256, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(calls):
            lib.stream_rmw_probe(buf.data_ptr(), 1024, 0, side.cuda_stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1000.0 / (calls * replays), 3)


def time_workload(w, launches=("auto", "rows", "token"), target_s: float = 0.15):
    """µs per call and GB/s of rope_fwd_qk and rope_bwd_qk on workload w,
    back to back on one stream, cycling through enough buffer sets to exceed
    the 256 MB Infinity Cache when the workload allows."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    pos = W.positions(w)
    cos, sin = rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta)
    cos, sin = cos.cuda(), sin.cuda()
    e = 4 if w.dtype == "f32" else 2
    qk_bytes = e * w.head_dim * w.batch * w.seq_len * (w.n_heads_q + w.n_heads_k)
    sets = max(1, min(8, -(-600_000_000 // max(qk_bytes, 1))))
    host, bufs = device_inputs(w, sets)
    stream = torch.cuda.current_stream()
    nbytes = algorithmic_bytes(w, pos)
    results = []
    for launch in launches:
        kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim, launch=launch,
                  pos=None if pos is None else pos.cuda(), stream=stream)
        fwd = [rp.prepare(b["q"], b["k"], cos, sin, **kw) for b in bufs]
        bwd = [rp.prepare(b["dq"], b["dk"], cos, sin, **kw) for b in bufs]
        out = {"workload": w.name, "launch": launch, "buffer_sets": sets,
               "algorithmic_bytes_per_call": nbytes}
        _time_calls(out, fwd, bwd, sets, nbytes, target_s, stream)
        if launch == "auto" and nbytes < (64 << 20):
            # small calls are bound by the launch: their µs per call replayed
            # from a captured graph (one buffer set), beside the empty kernel's
            b0 = bufs[0]
            gkw = dict(kw, stream=None)

            def make(st, b0=b0, gkw=gkw):
                return rp.prepare(b0["q"], b0["k"], cos, sin, **dict(gkw, stream=st)).rope_fwd_qk
            out["fwd_us_per_call_graph_replay"] = round(_graph_us_per_call(make), 3)
            out["empty_kernel_us_per_call_graph_replay"] = empty_kernel_floor()
        results.append(out)
    del bufs
    torch.cuda.empty_cache()
    return results


def _time_calls(out, fwd, bwd, sets, nbytes, target_s, stream, method=None):
    import torch
    fm = method or "rope_fwd_qk"
    bm = method or "rope_bwd_qk"
    for name, calls in (("fwd", [getattr(c, fm) for c in fwd]),
                        ("bwd", [getattr(c, bm) for c in bwd])):
        settle(lambda i: calls[i % sets]())
        for i in range(10):
            calls[i % sets]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(5):
            calls[i % sets]()
        torch.cuda.synchronize()
        est = max((time.perf_counter() - t0) / 5, 1e-6)
        reps = int(min(5000, max(20, target_s / est)))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            calls[i % sets]()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1000.0 / reps
        out[f"{name}_us_per_call"] = round(us, 3)
        out[f"{name}_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        out[f"{name}_pct_of_hbm_peak"] = round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)
        out[f"{name}_reps"] = reps


def time_theta(target_s: float = 0.15):
    """Angles computed from theta (no cos/sin tables): rope_apply on the Llama
    prefill workload ([B,H,S,D], rows shape) and on its packed-QKV form (token
    shape), forward and backward in place; and decode calls replayed from a
    captured HIP graph."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    results = []
    stream = torch.cuda.current_stream()
    w = W.LLAMA_GQA_PREFILL
    nbytes = algorithmic_bytes(w, None, tables=False)
    _, sets = device_inputs(w, 3, ("q", "k"))
    kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim, theta=w.theta,
              max_positions=w.table_rows, stream=stream)
    fwd = [rp.prepare_apply(x["q"], x["k"], None, None, **kw) for x in sets]
    bwd = [rp.prepare_apply(x["q"], x["k"], None, None, direction=-1, **kw) for x in sets]
    out = {"workload": w.name, "launch": "theta_angles", "buffer_sets": len(sets),
           "algorithmic_bytes_per_call": nbytes}
    _time_calls(out, fwd, bwd, len(sets), nbytes, target_s, stream, method="rope_apply")
    results.append(out)
    del sets, fwd, bwd
    B, S, Hq, Hk, D = w.batch, w.seq_len, w.n_heads_q, w.n_heads_k, w.head_dim
    host = W.normal((B, S, (Hq + 2 * Hk) * D), w.dtype, w.seed("q"))
    bufs = [host.cuda() for _ in range(3)]
    views = [(g[..., :Hq * D].view(B, S, Hq, D), g[..., Hq * D:(Hq + Hk) * D].view(B, S, Hk, D))
             for g in bufs]
    kw["layout"] = "bshd"
    fwd = [rp.prepare_apply(q, k, None, None, **kw) for q, k in views]
    bwd = [rp.prepare_apply(q, k, None, None, direction=-1, **kw) for q, k in views]
    out = {"workload": w.name, "launch": "theta_angles_packed_qkv_in_place", "buffer_sets": 3,
           "algorithmic_bytes_per_call": nbytes}
    _time_calls(out, fwd, bwd, 3, nbytes, target_s, stream, method="rope_apply")
    results.append(out)
    del bufs, views, fwd, bwd
    torch.cuda.empty_cache()
    results.append(time_decode(theta=True))
    return results


def time_xpos(target_s: float = 0.15):
    """RoPE with XPOS factors (rope_apply_xpos) on the Llama prefill workload,
    forward and backward in place, [B,H,S,D] and packed QKV; beside it the
    same rotation without factors (rope_apply), on the same buffers."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    results = []
    stream = torch.cuda.current_stream()
    w = W.LLAMA_GQA_PREFILL
    # the factor tables add two more [S, R/2] float32 rows per position
    nbytes = algorithmic_bytes(w, None) + 4 * w.rotary_dim * w.seq_len
    cos, sin = (t.cuda() for t in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
    zq, zk = (t.cuda() for t in rp.rope_build_xpos_table(w.table_rows, w.rotary_dim, 512.0, 0.4,
                                                          w.seq_len / 2))
    _, sets = device_inputs(w, 3, ("q", "k"))
    B, S, Hq, Hk, D = w.batch, w.seq_len, w.n_heads_q, w.n_heads_k, w.head_dim
    host = W.normal((B, S, (Hq + 2 * Hk) * D), w.dtype, w.seed("q"))
    bufs = [host.cuda() for _ in range(3)]
    packed = [(g[..., :Hq * D].view(B, S, Hq, D), g[..., Hq * D:(Hq + Hk) * D].view(B, S, Hk, D))
              for g in bufs]
    for layout, views in (("bhsd", [(x["q"], x["k"]) for x in sets]), ("bshd", packed)):
        kw = dict(layout=layout, pairing=w.pairing, rotary_dim=w.rotary_dim, stream=stream)
        fwd = [rp.prepare_apply_xpos(q, k, cos, sin, zq, zk, **kw) for q, k in views]
        bwd = [rp.prepare_apply_xpos(q, k, cos, sin, zq, zk, direction=-1, **kw)
               for q, k in views]
        out = {"workload": w.name, "call": "rope_apply_xpos",
               "views": "[B,H,S,D]" if layout == "bhsd" else "packed QKV [B,S,H,D]",
               "xpos": {"scale_base": 512.0, "gamma": 0.4, "center": w.seq_len / 2},
               "buffer_sets": 3, "algorithmic_bytes_per_call": nbytes,
               "kernel": "rope_xpos_lanes_kernel (one 16-byte chunk of one (token, head) per lane)"}
        _time_calls(out, fwd, bwd, 3, nbytes, target_s, stream, method="rope_apply_xpos")
        results.append(out)
        plain_bytes = algorithmic_bytes(w, None)
        fwd = [rp.prepare_apply(q, k, cos, sin, **kw) for q, k in views]
        bwd = [rp.prepare_apply(q, k, cos, sin, direction=-1, **kw) for q, k in views]
        out = {"workload": w.name, "call": "rope_apply (no XPOS, for comparison)",
               "views": "[B,H,S,D]" if layout == "bhsd" else "packed QKV [B,S,H,D]",
               "buffer_sets": 3, "algorithmic_bytes_per_call": plain_bytes}
        _time_calls(out, fwd, bwd, 3, plain_bytes, target_s, stream, method="rope_apply")
        results.append(out)
        del fwd, bwd
    return results


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, published


def attention_flops(w) -> int:
    """Algorithmic flops of one attention call: 2 D for each visible (query,
    key) pair in S = Q K^T and 2 D more in O = P V, for every (batch, head)."""
    Sq, Sk = w.seq_len_q, w.seq_len_k
    if w.causal:
        # query i sees keys 0 .. i + Sk - Sq
        pairs = sum(min(Sk, i + Sk - Sq + 1) for i in range(Sq))
    else:
        pairs = Sq * Sk
    return 4 * w.head_dim * pairs * w.batch * w.n_heads_q


def _time_event(fn, stream, target_s: float):
    """Average µs per call of fn() on `stream`, between HIP events."""
    import torch
    settle(lambda i: fn())
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    est = max(time.perf_counter() - t0, 1e-6)
    reps = int(min(2000, max(10, target_s / est)))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1000.0 / reps, reps


def time_attention(target_s: float = 0.5):
    """Attention over rotated Q and K: the fused call (rope_attention_fwd,
    rotation inside the kernel) against the unfused sequence (rope_apply
    writing rotated copies of Q and K, then the same attention kernel with
    rotation off) and the K-once call (rope_attention_fwd_k_once: rope(K)
    into a workspace, Q rotated in the kernel), on the causal Llama GQA
    prefill shape and on the CLS-skipping partial-rotary example. One JSON
    object per workload."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    stream = torch.cuda.current_stream()
    ceiling = mfma_ceiling()
    results = []
    for w in W.ATTN_ALL:
        t = {k: v.cuda() for k, v in W.attn_tensors(w).items()}
        pos = W.attn_positions(w)
        pos = None if pos is None else pos.cuda()
        c, s = (x.cuda() for x in rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta))
        o = torch.empty_like(t["q"])
        kw = dict(pairing=w.pairing, rotary_dim=w.rotary_dim, causal=w.causal, q_pos=pos,
                  k_pos=pos, stream=stream)
        fused = rp.prepare_attention(t["q"], t["k"], t["v"], c, s, o, **kw)
        qr, kr = torch.empty_like(t["q"]), torch.empty_like(t["k"])
        rot = rp.prepare_apply(t["q"], t["k"], c, s, q_out=qr, k_out=kr, pairing=w.pairing,
                               rotary_dim=w.rotary_dim, pos=pos, stream=stream)
        plain = rp.prepare_attention(qr, kr, t["v"], c, s, o, rotate=False, **kw)
        # K rotated once into a workspace, only Q rotated in the kernel
        k_once = rp.prepare_attention(t["q"], t["k"], t["v"], c, s, o, k_workspace=kr, **kw)
        flops = attention_flops(w)
        fused_us, reps = _time_event(fused.rope_attention_fwd, stream, target_s)
        k_once_us, _ = _time_event(k_once.rope_attention_fwd, stream, target_s)
        plain_us, _ = _time_event(plain.rope_attention_fwd, stream, target_s)
        rot_us, _ = _time_event(rot.rope_apply, stream, target_s / 4)

        def unfused():
            rot.rope_apply()
            plain.rope_attention_fwd()
        unfused_us, _ = _time_event(unfused, stream, target_s)
        tf = flops / (fused_us * 1e-6) / 1e12
        results.append({
            "workload": w.name, "q_shape": list(w.q_shape), "kv_shape": list(w.kv_shape),
            "rotary_dim": w.rotary_dim, "pairing": w.pairing, "causal": w.causal,
            "positions": w.pos_kind, "algorithmic_flops_per_call": flops,
            "fused_us_per_call": round(fused_us, 2),
            "fused_TFLOPs": round(tf, 1),
            "fused_frac_of_mfma_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "attention_without_rotation_us": round(plain_us, 2),
            "rotation_out_of_place_us": round(rot_us, 2),
            "unfused_us_per_call": round(unfused_us, 2),
            "fused_saves_us": round(unfused_us - fused_us, 2),
            "k_once_us_per_call": round(k_once_us, 2),
            "k_once_TFLOPs": round(flops / (k_once_us * 1e-6) / 1e12, 1),
            "k_once_frac_of_mfma_bf16_peak": round(
                flops / (k_once_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "attention_without_rotation_TFLOPs": round(flops / (plain_us * 1e-6) / 1e12, 1),
            "attention_without_rotation_frac_of_mfma_bf16_peak": round(
                flops / (plain_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "measured_mfma_bf16_ceiling": ceiling,
            "fused_frac_of_measured_mfma_ceiling": round(tf / ceiling["TFLOPs"], 4),
            "k_once_frac_of_measured_mfma_ceiling": round(
                flops / (k_once_us * 1e-6) / 1e12 / ceiling["TFLOPs"], 4),
            "reps": reps,
            "kernel": "rope_attention_kernel (v_mfma_f32_32x32x16_bf16)",
        })
        del t, o, qr, kr, fused, rot, plain, k_once
        torch.cuda.empty_cache()
    return results


def time_general_form(w, target_s: float = 0.15):
    """rope_apply on workload w's shapes laid out as one packed QKV buffer
    [B, S, (Hq + 2 Hk) * D] (Q and K rotated in place where they sit), and
    out of place from the packed buffer into separate [B, S, H, D] outputs.
    GB/s over the same algorithmic bytes as the contiguous call (R = D here,
    so out of place moves the same bytes)."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    B, S, Hq, Hk, D = w.batch, w.seq_len, w.n_heads_q, w.n_heads_k, w.head_dim
    cos, sin = rp.rope_build_table(w.table_rows, w.rotary_dim, w.theta)
    cos, sin = cos.cuda(), sin.cuda()
    dt = W.TORCH_DTYPES[w.dtype]
    e = 4 if w.dtype == "f32" else 2
    qkv_bytes = B * S * (Hq + 2 * Hk) * D * e
    sets = max(1, min(4, -(-600_000_000 // qkv_bytes)))
    host = W.normal((B, S, (Hq + 2 * Hk) * D), w.dtype, w.seed("q"))
    bufs = [host.cuda() for _ in range(sets)]
    outs = [(torch.empty(B, S, Hq, D, dtype=dt, device="cuda"),
             torch.empty(B, S, Hk, D, dtype=dt, device="cuda")) for _ in range(sets)]
    stream = torch.cuda.current_stream()
    nbytes = algorithmic_bytes(w, None)
    kw = dict(layout="bshd", pairing=w.pairing, rotary_dim=w.rotary_dim, stream=stream)

    def views(g):
        return (g[..., :Hq * D].view(B, S, Hq, D),
                g[..., Hq * D:(Hq + Hk) * D].view(B, S, Hk, D))
    results = []
    for mode in ("packed_qkv_in_place", "packed_qkv_out_of_place"):
        calls = []
        for i, g in enumerate(bufs):
            q, k = views(g)
            extra = {} if mode.endswith("in_place") else dict(q_out=outs[i][0], k_out=outs[i][1])
            f = rp.prepare_apply(q, k, cos, sin, **kw, **extra)
            b = rp.prepare_apply(q, k, cos, sin, direction=-1, **kw, **extra)
            calls.append((f, b))
        out = {"workload": w.name, "launch": mode, "buffer_sets": sets,
               "algorithmic_bytes_per_call": nbytes}
        _time_calls(out, [c[0] for c in calls], [c[1] for c in calls], sets, nbytes, target_s,
                    stream, method="rope_apply")
        results.append(out)
    del bufs, outs
    torch.cuda.empty_cache()
    return results


# [B, S, Hq, Hk, D, dtype] shapes for the token-major launch-shape comparison
LAYOUT_MATRIX_SHAPES = {
    "[4, 4096, 32+8, 128] bf16": (4, 4096, 32, 8, 128, "bf16"),
    "[8, 2048, 16+16, 64] fp16": (8, 2048, 16, 16, 64, "f16"),
    "[4, 4096, 32+32, 64] bf16": (4, 4096, 32, 32, 64, "bf16"),
    "[2, 4096, 16+4, 256] bf16": (2, 4096, 16, 4, 256, "bf16"),
}


def time_layout_matrix(reps: int = 400):
    """rows vs token launch on token-major views ([B,S,H,D] tensors and Q/K
    views into a packed QKV buffer), both pairings, and the automatic
    choice beside them (which may be a shape only it launches): forward
    rope_apply in place, reps calls over 3 buffer sets between two HIP
    events."""
    import torch
    import rotary_position_embedding_fwd_amd as rp
    import workloads as W
    stream = torch.cuda.current_stream()
    for name, (B, S, Hq, Hk, D, dt) in LAYOUT_MATRIX_SHAPES.items():
        cos, sin = rp.rope_build_table(S, D, 10000.0)
        cos, sin = cos.cuda(), sin.cuda()
        nbytes = 2 * (2 if dt != "f32" else 4) * B * S * (Hq + Hk) * D + 8 * S * (D // 2)
        for view in ("bshd", "packed"):
            sets = []
            for i in range(3):
                if view == "bshd":
                    sets.append((W.normal((B, S, Hq, D), dt, 9000 + i).cuda(),
                                 W.normal((B, S, Hk, D), dt, 9100 + i).cuda()))
                else:
                    g = W.normal((B, S, (Hq + 2 * Hk) * D), dt, 9200 + i).cuda()
                    sets.append((g[..., :Hq * D].view(B, S, Hq, D),
                                 g[..., Hq * D:(Hq + Hk) * D].view(B, S, Hk, D), g))
            for pairing in ("split_half", "interleaved"):
                res = {"shape": name, "view": view, "pairing": pairing}
                for launch in ("rows", "token", "auto"):
                    calls = [rp.prepare_apply(x[0], x[1], cos, sin, layout="bshd",
                                              pairing=pairing, launch=launch,
                                              stream=stream).rope_apply for x in sets]
                    for c in calls:
                        c()
                    torch.cuda.synchronize()
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for i in range(reps):
                        calls[i % len(calls)]()
                    b.record(stream)
                    torch.cuda.synchronize()
                    us = a.elapsed_time(b) * 1000.0 / reps
                    res[f"{launch}_us"] = round(us, 2)
                    res[f"{launch}_GBps"] = round(nbytes / us / 1e3, 1)
                yield res
            del sets
            torch.cuda.empty_cache()


def _oracle_call_slices(w, x, direction, pos):
    """The oracle's calls for one tensor of workload w, one per (batch, head)
    slice ([B,H,S,D]) or per batch ([B,S,H,D]); each slice keeps its own
    positions, so the slices together compute exactly the whole call."""
    import oracle
    kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim, theta=w.theta,
              table_rows=w.table_rows)
    pv = None if pos is None else pos.numpy()
    calls = []
    if w.layout == "bhsd":
        for b in range(x.shape[0]):
            pb = None if pv is None else pv[b * w.pos_batch_stride:b * w.pos_batch_stride +
                                              w.seq_len]
            for h in range(x.shape[1]):
                calls.append((x[b:b + 1, h:h + 1], dict(kw, pos=pb, direction=direction)))
    else:
        for b in range(x.shape[0]):
            pb = None if pv is None else pv[b * w.pos_batch_stride:b * w.pos_batch_stride +
                                              w.seq_len]
            calls.append((x[b:b + 1], dict(kw, pos=pb, direction=direction)))
    return [(lambda a=a, k=k: oracle.rope(a, w.dtype, **k)) for a, k in calls]


def cpu_baseline(w, host, pos, steps: int = 2, all_steps: int = 4):
    """The CPU oracle, as it stands: `steps` full steps (fwd of Q, K + bwd of
    dQ, dK) of w on one thread (about 10 s on the Llama prefill workload),
    then `all_steps` steps with the same calls cut into (batch, head) slices
    run on every host thread; and the oracle's table build for w."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    orc = oracle
    orc.load()
    arrs = {k: orc.torch_to_storage(v) for k, v in host.items()}
    kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim, theta=w.theta,
              pos=None if pos is None else pos.numpy(), pos_batch_stride=w.pos_batch_stride,
              table_rows=w.table_rows)
    t0 = time.perf_counter()
    for _ in range(steps):
        orc.rope(arrs["q"], w.dtype, direction=1, **kw)
        orc.rope(arrs["k"], w.dtype, direction=1, **kw)
        orc.rope(arrs["dq"], w.dtype, direction=-1, **kw)
        orc.rope(arrs["dk"], w.dtype, direction=-1, **kw)
    dt1 = time.perf_counter() - t0
    threads = max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                  else (os.cpu_count() or 1))
    jobs = []
    for name, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        jobs += _oracle_call_slices(w, arrs[name], direction, pos)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        for _ in range(all_steps):
            list(ex.map(lambda f: f(), jobs))
    dtn = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.table(w.theta, w.rotary_dim, w.table_rows)
    dtab = time.perf_counter() - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    step_bytes = 2 * algorithmic_bytes(w, pos)
    return {"value": round(all_steps * step_bytes / dtn / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle", "seconds": round(dtn, 3),
            "sample": f"{all_steps} full steps (fwd of Q,K + bwd of dQ,dK) of {w.name}, the "
                      f"scalar binary64 oracle on (batch, head) slices over {threads} host "
                      f"threads",
            "single_thread": {"value": round(steps * step_bytes / dt1 / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "seconds": round(dt1, 3),
                              "sample": f"{steps} full steps of {w.name}, one thread"},
            "table_build_s": round(dtab, 4),
            "table_build": f"the oracle's float32 cos/sin table [{w.table_rows}, "
                           f"{w.rotary_dim // 2}] from theta {w.theta}",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model}


def stored_traffic(workload: str):
    """HBM traffic per launch of `workload`'s kernel from the committed
    rocprofv3 counter summary, or None when there is none or the kernel
    sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("workloads", {}).get(workload, {}).get("bytes_per_launch")


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3):
    """A plain device copy of known size, for scaling the FETCH/WRITE counters."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def _bench_entries(b):
    """(workload, kernel description, algorithmic bytes per call) of each timed
    workload of a bench JSON line."""
    out = [(b["config"]["workload"], b["roofline"]["launch"],
            b["config"]["algorithmic_bytes_per_call"])]
    for c in b.get("configs", []):
        out.append((c["workload"], c["kernel"], c["algorithmic_bytes_per_call"]))
    return out


def summarize_counters(pmc_dir: str, out: str):
    """Mean of every counter of a rocprofv3 --pmc run per kernel launch shape
    (kernel name, grid, workgroup size), with the dispatch count, into a small
    JSON file (the raw per-dispatch files run to tens of MB)."""
    import csv
    acc = {}
    for p in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0),
                       int(r.get("Workgroup_Size", 0) or 0))
                e = acc.setdefault(key, {"vgpr": r.get("VGPR_Count"),
                                         "agpr": r.get("Accum_VGPR_Count"),
                                         "lds": r.get("LDS_Block_Size"), "counters": {}})
                s = e["counters"].setdefault(r["Counter_Name"], [0.0, 0])
                s[0] += float(r["Counter_Value"])
                s[1] += 1
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    d = e.setdefault("ns", {})
                    d[r.get("Dispatch_Id")] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    res = []
    for (name, grid, block), e in sorted(acc.items(), key=lambda kv: kv[0]):
        n = max(c[1] for c in e["counters"].values())
        ns = list(e.get("ns", {}).values())
        res.append({"kernel": name, "grid": grid, "block": block, "dispatches": n,
                    "vgpr": e["vgpr"], "agpr": e["agpr"], "lds": e["lds"],
                    "mean_ns": sum(ns) / len(ns) if ns else None,
                    "mean": {k: c[0] / c[1] for k, c in sorted(e["counters"].items())}})
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(f"{len(res)} launch shapes -> {out}")


def summarize_pmc(fetch_dir: str, write_dir: str, bench_json: str, out: str = TRAFFIC_FILE):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
    `bench.py --copy-calibration` into per-launch HBM traffic of each timed
    workload's kernel (matched by name and grid size), each counter scaled by
    its reading for the 1 GiB device copy."""
    import csv

    def read(d, counter):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        rows.append((int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"],
                                     int(r.get("Grid_Size", 0) or 0),
                                     int(r.get("Workgroup_Size", 0) or 0),
                                     float(r["Counter_Value"])))
        rows.sort()
        return [r[1:] for r in rows]

    def calibration(rows, reps=3):
        # the bench's own device-to-device clones run the same copy kernel;
        # the calibration copies are the last `reps` of them
        vals = [v for n, g, wg, v in rows if "copyBuffer" in n][-reps:]
        return sum(vals) / len(vals) if len(vals) == reps else None

    def pick(rows, name, grid=None, block=None):
        vals = [v for n, g, wg, v in rows
                if name in n and (grid is None or g == grid) and (block is None or wg == block)]
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    with open(bench_json) as f:
        b = json.loads([ln for ln in f if ln.startswith("{")][-1])
    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    copy_bytes = 1 << 30
    f_c = calibration(fetch)  # the runtime's device-to-device copy
    w_c = calibration(write)
    res = {"copy_bytes": copy_bytes, "copy_fetch_kib": f_c, "copy_write_kib": w_c,
           "workloads": {}}
    if f_c and w_c:
        res["fetch_scale"] = copy_bytes / (f_c * 1024)
        res["write_scale"] = copy_bytes / (w_c * 1024)
    for workload, launch, alg in _bench_entries(b):
        k = _kernel_fields(launch)
        items = k.get("grid", 0) * k.get("block", 0)
        f_k, nf = pick(fetch, k["name"], items, k.get("block"))
        w_k, nw = pick(write, k["name"], items, k.get("block"))
        e = {"kernel": k["name"], "grid": k.get("grid"), "block": k.get("block"),
             "fetch_kib_per_launch": f_k, "write_kib_per_launch": w_k,
             "dispatches": [nf, nw], "algorithmic_bytes_per_launch": alg}
        if None not in (f_k, w_k) and "fetch_scale" in res:
            e["bytes_per_launch"] = round(f_k * 1024 * res["fetch_scale"] +
                                          w_k * 1024 * res["write_scale"])
            e["traffic_over_algorithmic"] = round(e["bytes_per_launch"] / alg, 4)
        res["workloads"][workload] = e
    res["kernel_source_hash"] = kernel_source_hash()
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def _trace_rows(trace_dir: str):
    """Kernel dispatches of a rocprofv3 --kernel-trace run, in dispatch order:
    (name, workgroup size, grid size in work-items, duration ns)."""
    import csv
    rows = []
    for p in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                rows.append((int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"],
                             int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 0)) or 0),
                             int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0),
                             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    return [r[1:] for r in rows]


def _stats_us(ns):
    import statistics
    us = [x / 1000.0 for x in ns]
    return {"launches": len(us), "mean_us": round(statistics.fmean(us), 3),
            "median_us": round(statistics.median(us), 3), "min_us": round(min(us), 3),
            "max_us": round(max(us), 3)}


def summarize_kernels(trace_dir: str, out: str):
    """Per-kernel durations of every dispatch in a rocprofv3 kernel trace,
    grouped by kernel name and grid, into a small JSON file."""
    groups = {}
    for name, wg, grid, ns in _trace_rows(trace_dir):
        groups.setdefault((name, grid, wg), []).append(ns)
    res = [dict(kernel=k[0], grid=k[1], block=k[2], **_stats_us(v))
           for k, v in sorted(groups.items())]
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(f"{len(res)} launch shapes -> {out}")


def summarize_trace(trace_dir: str, bench_json: str):
    """Per-kernel durations of the launches bench.py timed, from a rocprofv3
    kernel trace of that bench run: for each timed workload, the dispatches
    of its kernel with its grid, in order, minus the warmup launches, then
    exactly the timed ones. Prints one JSON object (mean, median, min, max
    µs per launch, and GB/s over the algorithmic bytes)."""
    with open(bench_json) as f:
        line = [ln for ln in f if ln.startswith("{")][-1]
    b = json.loads(line)
    rows = _trace_rows(trace_dir)
    entries = [dict(workload=b["config"]["workload"], launch=b["roofline"]["launch"],
                    warmup=b["warmup"], steps=b["steps"],
                    bytes=b["config"]["algorithmic_bytes_per_call"],
                    bench_us=b["roofline"]["avg_launch_us"])]
    for c in b.get("configs", []):
        entries.append(dict(workload=c["workload"], launch=c["kernel"], warmup=c["warmup"],
                            steps=c["steps"], bytes=c["algorithmic_bytes_per_call"],
                            bench_us=c["us_per_launch"]))
    out = {"trace_dir": trace_dir, "workloads": []}
    used = set()
    for e in entries:
        k = _kernel_fields(e["launch"])
        items = k.get("grid", 0) * k.get("block", 0)
        idx = [i for i, (name, wg, grid, _) in enumerate(rows)
               if i not in used and k["name"] in name and wg == k.get("block") and
               grid == items]
        # the settle phase and the warmup come first; the timed launches are
        # the last 2 * steps dispatches of this kernel and grid
        take = 2 * e["steps"]
        timed = idx[-take:] if len(idx) >= take else []
        used.update(idx)
        res = {"workload": e["workload"], "kernel": k["name"], "grid": k.get("grid"),
               "block": k.get("block"), "dispatches_found": len(idx),
               "settle_and_warmup_dropped": max(0, len(idx) - take),
               "bench_event_avg_launch_us": e["bench_us"]}
        if timed:
            st = _stats_us([rows[i][3] for i in timed])
            st["GBps_at_mean"] = round(e["bytes"] / (st["mean_us"] * 1e-6) / 1e9, 1)
            st["frac_at_mean"] = round(st["GBps_at_mean"] / HBM_PEAK_GBS, 4)
            res.update(st)
        out["workloads"].append(res)
    if "decode" in b and b["decode"].get("kernel"):
        k = _kernel_fields(b["decode"]["kernel"])
        items = k.get("grid", 0) * k.get("block", 0)
        idx = [i for i, (name, wg, grid, _) in enumerate(rows)
               if i not in used and k["name"] in name and wg == k.get("block") and
               grid == items]
        if idx:
            res = {"workload": b["decode"]["workload"], "kernel": k["name"],
                   "grid": k.get("grid"), "block": k.get("block"),
                   "note": "every decode dispatch (warmup, eager, event-pair and graph "
                           "replays)"}
            res.update(_stats_us([rows[i][3] for i in idx]))
            out["decode"] = res
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=3,
                    help="buffer sets cycled through (3 x 320 MiB > the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the BSHD interleaved and long-context configs")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for counter scaling)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_JSON"))
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "OUT_JSON"),
                    help="mean of each counter of a --pmc run per kernel launch shape")
    ap.add_argument("--summarize-kernels", nargs=2, metavar=("TRACE_DIR", "OUT_JSON"),
                    help="durations of every kernel of a --kernel-trace run per launch shape")
    ap.add_argument("--workloads", action="store_true",
                    help="time every workload (both grid shapes); one JSON line each")
    ap.add_argument("--general-form", action="store_true",
                    help="time only rope_apply on the Llama prefill shape as packed QKV, "
                         "in place and out of place")
    ap.add_argument("--theta", action="store_true",
                    help="time the path with cos/sin computed from theta (no tables)")
    ap.add_argument("--layout-matrix", action="store_true",
                    help="rows vs token launch on token-major views, by shape and pairing")
    ap.add_argument("--xpos", action="store_true",
                    help="RoPE with XPOS factors (rope_apply_xpos) against plain rope_apply")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="decode calls at several sequence counts against the launch floor")
    ap.add_argument("--attention", action="store_true",
                    help="time attention with RoPE fused on the loaded Q/K blocks, against "
                         "rotation followed by attention")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_kernels:
        summarize_kernels(*args.summarize_kernels)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the RoPE path has no cross-GPU step, "
              "and librope runs on a single MI355X per process. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import rotary_position_embedding_fwd_amd as rp
    rp.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.theta:
        for res in time_theta():
            print(json.dumps(res), flush=True)
        return
    if args.xpos:
        for res in time_xpos():
            print(json.dumps(res), flush=True)
        return
    if args.decode_sweep:
        print(json.dumps(time_decode_sweep()), flush=True)
        return
    if args.attention:
        for res in time_attention():
            print(json.dumps(res), flush=True)
        return
    if args.layout_matrix:
        for res in time_layout_matrix():
            print(json.dumps(res), flush=True)
        return
    if args.general_form:
        for res in time_general_form(W.LLAMA_GQA_PREFILL):
            print(json.dumps(res), flush=True)
        return
    if args.workloads:
        for wl in W.ALL:
            for res in time_workload(wl):
                print(json.dumps(res), flush=True)
        for res in time_general_form(W.LLAMA_GQA_PREFILL):
            print(json.dumps(res), flush=True)
        return

    w = W.LLAMA_GQA_PREFILL
    r = time_prefill(w, args.steps, args.warmup, args.sets)
    per_call = algorithmic_bytes(w, r["pos"])
    step_bytes = 2 * per_call
    total_s = r["total_ms"] / 1000.0
    gbs = args.steps * step_bytes / total_s / 1e9
    launches = 2 * args.steps
    avg_launch_us = r["total_ms"] * 1000.0 / launches
    achieved = per_call / (avg_launch_us * 1e-6) / 1e9
    traffic = stored_traffic(w.name)
    kernel = _kernel_fields(r["kernel"])
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["total_ms"] / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "q_shape": list(w.q_shape), "k_shape": list(w.k_shape),
                   "storage_dtype": w.dtype, "layout": w.layout, "pairing": w.pairing,
                   "rotary_dim": w.rotary_dim, "table": [w.table_rows, w.rotary_dim // 2],
                   "theta": w.theta, "step": "rope_fwd_qk(Q,K) + rope_bwd_qk(dQ,dK), in place",
                   "buffer_sets": args.sets,
                   "algorithmic_bytes_per_call": per_call},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": kernel["name"] + " (fwd and bwd launches)",
                     "launch": r["kernel"],
                     "algorithmic_bytes_per_launch": per_call,
                     "avg_launch_us": round(avg_launch_us, 3),
                     "launches_timed": launches},
        "wall_s_timed": round(r["wall_s"], 4),
    }
    if not args.no_ceiling:
        e = 2
        qk = e * w.head_dim * w.batch * w.seq_len * (w.n_heads_q + w.n_heads_k)
        ceil = stream_ceiling(qk, reps=2 * args.steps, sets=max(2, -(-600_000_000 // qk)))
        ceil["frac_achieved_of_ceiling"] = round(achieved / ceil["GBps"], 4)
        out["roofline"]["measured_stream_ceiling"] = ceil
    if not args.no_configs:
        out["configs"] = [time_config(getattr(W, name), st, wu, sets,
                                      ceiling=not args.no_ceiling)
                          for name, st, wu, sets in EXTRA_CONFIGS]
    if not args.no_decode:
        out["decode"] = time_decode()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, r["host"], r["pos"])
    if args.copy_calibration:
        copy_calibration()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

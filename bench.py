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
a `cpu_baseline` (the CPU oracle timed on the host) and the decode-shape
µs/call.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
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
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_rope_pair_lanes_kernel_bf16_llama_gqa_prefill.json")


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


def device_inputs(w, sets: int, which=("q", "k", "dq", "dk")):
    import torch
    import workloads as W
    t = W.tensors(w, which)
    out = []
    for i in range(sets):
        out.append({k: v.to("cuda") for k, v in t.items()})
    return t, out


def time_prefill(w, steps: int, warmup: int, sets: int):
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
    host, bufs = device_inputs(w, sets)
    stream = torch.cuda.current_stream()
    kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim,
              pos=None if pos is None else pos.cuda(), stream=stream)
    fwd = [rp.prepare(b["q"], b["k"], cos, sin, **kw) for b in bufs]
    bwd = [rp.prepare(b["dq"], b["dk"], cos, sin, **kw) for b in bufs]

    def step(i):
        fwd[i % sets].rope_fwd_qk()
        bwd[i % sets].rope_bwd_qk()

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

    return dict(total_ms=total_ms, wall_s=wall, pos=pos, host=host)


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
    return {"workload": w.name, "angles": "theta" if theta else "tables",
            "us_per_call_graph_replay": round(graph_us, 3),
            "us_per_call_back_to_back": round(per_call_us, 3),
            "us_kernel_event_median": round(kern[len(kern) // 2], 3),
            "algorithmic_bytes": nbytes, "calls": calls,
            "note": "graph replay: 100 captured calls per graph; back to back: Python "
                    "ctypes launches, bound by the host call rate"}


def stream_ceiling(nbytes: int = 3 << 29, reps: int = 20):
    """GB/s of a plain in-place read+write stream (libstream_probe.so) over a
    buffer larger than the 256 MB Infinity Cache: the attainable HBM rate of
    an operation that reads and writes every byte once."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "rotary_position_embedding_fwd_amd", "libstream_probe.so")
    lib = ctypes.CDLL(path)
    lib.stream_rmw_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint,
                                     ctypes.c_void_p]
    lib.stream_rmw_probe.restype = ctypes.c_int
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        assert lib.stream_rmw_probe(buf.data_ptr(), nbytes, 0, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        lib.stream_rmw_probe(buf.data_ptr(), nbytes, 0, stream.cuda_stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / reps
    del buf
    return {"kernel": "stream_rmw_kernel (16 B non-temporal load + store per lane)",
            "bytes_per_launch": 2 * nbytes, "avg_launch_us": round(us, 2),
            "GBps": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}


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
               "kernel": "rope_xpos_kernel (16-byte chunks, 8 heads per lane)"}
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
    views into a packed QKV buffer), both pairings: forward rope_apply in
    place, reps calls over 3 buffer sets between two HIP events."""
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
                for launch in ("rows", "token"):
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


def cpu_baseline(w, host, pos, steps: int = 2):
    """The CPU oracle, as it stands, on `steps` full steps (fwd + bwd) of w,
    1 thread: about 10 s of CPU work on the Llama prefill workload."""
    import oracle
    orc = oracle
    orc.load()
    nbytes = steps * 2 * algorithmic_bytes(w, pos)
    kw = dict(layout=w.layout, pairing=w.pairing, rotary_dim=w.rotary_dim, theta=w.theta,
              pos=None if pos is None else pos.numpy(), pos_batch_stride=w.pos_batch_stride,
              table_rows=w.table_rows)
    arrs = {k: orc.torch_to_storage(v) for k, v in host.items()}
    t0 = time.perf_counter()
    for _ in range(steps):
        orc.rope(arrs["q"], w.dtype, direction=1, **kw)
        orc.rope(arrs["k"], w.dtype, direction=1, **kw)
        orc.rope(arrs["dq"], w.dtype, direction=-1, **kw)
        orc.rope(arrs["dk"], w.dtype, direction=-1, **kw)
    dt = time.perf_counter() - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{steps} full steps (fwd of Q,K + bwd of dQ,dK) of {w.name}, "
                      f"single-threaded scalar binary64 oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model}


def stored_traffic():
    """HBM traffic per launch from the committed rocprofv3 counter summary, or
    None when the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3):
    """A plain device copy of known size, for scaling the FETCH/WRITE counters."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def summarize_pmc(fetch_dir: str, write_dir: str, out: str = TRAFFIC_FILE):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
    `bench.py --copy-calibration` into per-launch traffic of the forward
    prefill kernel, scaled by the counters of the 1 GiB copy."""
    import csv
    import workloads as W

    def read(d, counter):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return rows

    def pick(rows, pred):
        vals = [v for n, v in rows if pred(n)]
        return sum(vals) / len(vals) if vals else None

    # the kernel the bench's step runs (the one-chunk-per-lane rows kernel)
    is_fwd = lambda n: "rope_pair_lanes_kernel" in n and "bf16" in n.replace("DF16b", "bf16")  # noqa
    is_copy = lambda n: "copyBuffer" in n  # the runtime's device-to-device copy  # noqa
    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    f_k, w_k = pick(fetch, is_fwd), pick(write, is_fwd)
    f_c, w_c = pick(fetch, is_copy), pick(write, is_copy)
    copy_bytes = 1 << 30
    res = {"kernel": "rope_pair_lanes_kernel<__bf16, 8, 4> (forward and backward launches)",
           "workload": W.LLAMA_GQA_PREFILL.name,
           "fetch_kib_per_launch": f_k, "write_kib_per_launch": w_k,
           "copy_fetch_kib": f_c, "copy_write_kib": w_c}
    if None not in (f_k, w_k, f_c, w_c):
        rf, rw = copy_bytes / (f_c * 1024), copy_bytes / (w_c * 1024)
        res.update({"fetch_scale": rf, "write_scale": rw,
                    "bytes_per_launch": round(f_k * 1024 * rf + w_k * 1024 * rw),
                    "algorithmic_bytes_per_launch":
                        algorithmic_bytes(W.LLAMA_GQA_PREFILL, None)})
    res["kernel_source_hash"] = kernel_source_hash()
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for counter scaling)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
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
    ap.add_argument("--attention", action="store_true",
                    help="time attention with RoPE fused on the loaded Q/K blocks, against "
                         "rotation followed by attention")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the RoPE path has no cross-GPU step, "
              "and this build runs on a single MI355X. Use --gpus 1.", file=sys.stderr)
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
    traffic = stored_traffic()
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
                     "kernel": "rope_pair_lanes_kernel<__bf16, 8, 4> (fwd and bwd launches)",
                     "algorithmic_bytes_per_launch": per_call,
                     "avg_launch_us": round(avg_launch_us, 3),
                     "launches_timed": launches},
        "wall_s_timed": round(r["wall_s"], 4),
    }
    if not args.no_ceiling:
        ceil = stream_ceiling()
        ceil["frac_achieved_of_ceiling"] = round(achieved / ceil["GBps"], 4)
        out["roofline"]["measured_stream_ceiling"] = ceil
    if not args.no_decode:
        out["decode"] = time_decode()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, r["host"], r["pos"])
    if args.copy_calibration:
        copy_calibration()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs for rotary position embedding, shared by both sides.

This module only draws numbers: query/key (and incoming-gradient) values and
integer position indices, with fixed seeds and the shapes of the workloads
below. It holds none of the method's arithmetic: no frequencies, no angles,
no cos/sin and no rotation. The GPU library builds its cos/sin tables itself
and the CPU oracle computes its own, so the two sides meet only here.

Workload shapes follow the pages' statement of the problem:
  - Q [batch, n_heads, seq_len, head_dim] and K [batch, n_heads_K, seq_len,
    head_dim] ("How Unsloth Optimizes RoPE Embedding Computations in Triton
    Kernels", Usage Examples / Manual Triton Kernel Invocation), with GQA
    n_heads_K <= n_heads;
  - the [batch, seq, heads, dim] layout (rotary-embedding-torch docs, Key
    Parameters, seq_before_head_dim);
  - split-half or interleaved pairs ("Rotary Embedding Kernel", Paired
    Element Layout);
  - a rotary dim smaller than the head dim (rotary-embedding-torch docs,
    RotaryEmbedding(dim=32) on head dim 64) and per-token int32 positions with
    the first two (CLS/register) tokens left unrotated (same docs,
    flash_attn_with_rotary example; Unsloth page, Custom Position IDs).

Values are N(0, 1) float32 from a seeded CPU torch.Generator, then rounded to
nearest-even into the storage dtype. Seeds are 1000 * workload.index + a
per-tensor offset (q 0, k 1, dq 2, dk 3, positions 4).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

BHSD = "bhsd"
BSHD = "bshd"
SPLIT_HALF = "split_half"
INTERLEAVED = "interleaved"

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

SEED_OFFSETS = {"q": 0, "k": 1, "dq": 2, "dk": 3, "pos": 4, "v": 5, "kpos": 6}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic RoPE problem: shapes, storage dtype, table and positions.

    pos_kind:
      "none"        no index tensor; token s sits at position s.
      "cls_offset"  one shared int32 index row of length seq_len: the first
                    `n_masked` entries are -1 (left unrotated), the rest are
                    start + 0, 1, ... with a seeded start in [0, pos_start_max).
      "uniform"     one int32 position per sequence (seq_len must be 1),
                    uniform in [0, table_rows).
    """

    name: str
    index: int
    batch: int
    n_heads_q: int
    n_heads_k: int
    seq_len: int
    head_dim: int
    rotary_dim: int
    dtype: str
    layout: str
    pairing: str
    theta: float
    table_rows: int
    pos_kind: str = "none"
    n_masked: int = 0
    pos_start_max: int = 0

    def shape(self, n_heads: int) -> tuple:
        if self.layout == BHSD:
            return (self.batch, n_heads, self.seq_len, self.head_dim)
        return (self.batch, self.seq_len, n_heads, self.head_dim)

    @property
    def q_shape(self) -> tuple:
        return self.shape(self.n_heads_q)

    @property
    def k_shape(self) -> tuple:
        return self.shape(self.n_heads_k)

    @property
    def pos_batch_stride(self) -> int:
        return 1 if self.pos_kind == "uniform" else 0

    def seed(self, what: str) -> int:
        return 1000 * self.index + SEED_OFFSETS[what]

    def scaled(self, **changes) -> "Workload":
        """A copy with some sizes changed (for oracle-sized parity cases)."""
        return dataclasses.replace(self, **changes)


# The five problems (six shapes) that the library is measured and checked on.
TINY_F32 = Workload("tiny_fp32_split", 1, 1, 8, 8, 128, 64, 64, "f32", BHSD,
                    SPLIT_HALF, 10000.0, 128)
LLAMA_GQA_PREFILL = Workload("llama_gqa_prefill_bf16", 2, 4, 32, 8, 4096, 128, 128,
                             "bf16", BHSD, SPLIT_HALF, 10000.0, 4096)
BSHD_INTERLEAVED = Workload("bshd_interleaved_fp16", 3, 8, 16, 16, 2048, 64, 64, "f16",
                            BSHD, INTERLEAVED, 10000.0, 2048)
PARTIAL_INDEXED = Workload("partial_rotary_indexed_bf16", 4, 2, 12, 12, 1026, 64, 32,
                           "bf16", BHSD, SPLIT_HALF, 10000.0, 9216,
                           pos_kind="cls_offset", n_masked=2, pos_start_max=8192)
DECODE = Workload("decode_bf16", 5, 256, 32, 8, 1, 128, 128, "bf16", BHSD, SPLIT_HALF,
                  500000.0, 32768, pos_kind="uniform")
LONG_CONTEXT = Workload("long_context_bf16", 6, 1, 32, 8, 131072, 128, 128, "bf16",
                        BHSD, SPLIT_HALF, 500000.0, 131072)

ALL = (TINY_F32, LLAMA_GQA_PREFILL, BSHD_INTERLEAVED, PARTIAL_INDEXED, DECODE,
       LONG_CONTEXT)
BY_NAME = {w.name: w for w in ALL}


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """One synthetic problem for attention over rotated Q and K: Q
    [batch, n_heads_q, seq_len_q, head_dim], K and V [batch, n_heads_k,
    seq_len_k, head_dim] (rotary-embedding-torch docs, flash_attn_with_rotary,
    Input Tensor Shapes), bf16 storage.

    pos_kind "none": key j at position j, query i at i + seq_len_k - seq_len_q;
    "cls_offset": one shared index row for queries and keys (seq_len_q ==
    seq_len_k), the first `n_masked` tokens at -1 (not rotated), the rest
    start + 0, 1, ... with a seeded start in [0, pos_start_max] (the docs'
    example skips two CLS/register tokens and rotates the rest from 0).
    """

    name: str
    index: int
    batch: int
    n_heads_q: int
    n_heads_k: int
    seq_len_q: int
    seq_len_k: int
    head_dim: int
    rotary_dim: int
    pairing: str
    theta: float
    table_rows: int
    causal: bool
    pos_kind: str = "none"
    n_masked: int = 0
    pos_start_max: int = 0
    dtype: str = "bf16"

    @property
    def q_shape(self) -> tuple:
        return (self.batch, self.n_heads_q, self.seq_len_q, self.head_dim)

    @property
    def kv_shape(self) -> tuple:
        return (self.batch, self.n_heads_k, self.seq_len_k, self.head_dim)

    def seed(self, what: str) -> int:
        return 1000 * self.index + SEED_OFFSETS[what]

    def scaled(self, **changes) -> "AttnWorkload":
        return dataclasses.replace(self, **changes)


# Causal GQA prefill attention at the Llama shape of the RoPE workloads above.
ATTN_LLAMA_PREFILL = AttnWorkload("attn_llama_gqa_prefill_bf16", 7, 4, 32, 8, 4096, 4096,
                                  128, 128, SPLIT_HALF, 10000.0, 4096, True)
# The docs' example: 1024 rotated tokens after two unrotated ones, R = 32 of
# head dim 64, causal.
ATTN_CLS_SKIP = AttnWorkload("attn_cls_skip_partial_bf16", 8, 1, 8, 8, 1026, 1026, 64, 32,
                             SPLIT_HALF, 10000.0, 1024, True, pos_kind="cls_offset",
                             n_masked=2, pos_start_max=0)

ATTN_ALL = (ATTN_LLAMA_PREFILL, ATTN_CLS_SKIP)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal(shape, dtype: str, seed: int) -> torch.Tensor:
    """N(0,1) float32 draws, rounded to nearest-even into `dtype` (CPU)."""
    x = torch.randn(shape, dtype=torch.float32, generator=_gen(seed))
    return x if dtype == "f32" else x.to(TORCH_DTYPES[dtype])


def tensors(w: Workload, which=("q", "k")) -> dict:
    """Seeded CPU tensors for the named operands of workload `w`."""
    out = {}
    for name in which:
        heads = w.n_heads_q if name in ("q", "dq") else w.n_heads_k
        out[name] = normal(w.shape(heads), w.dtype, w.seed(name))
    return out


def positions(w: Workload) -> Optional[torch.Tensor]:
    """The int32 index tensor of workload `w` on the CPU, or None."""
    if w.pos_kind == "none":
        return None
    g = _gen(w.seed("pos"))
    if w.pos_kind == "cls_offset":
        start = int(torch.randint(0, w.pos_start_max, (1,), generator=g))
        n = w.seq_len - w.n_masked
        body = torch.arange(n, dtype=torch.int32) + start
        head = torch.full((w.n_masked,), -1, dtype=torch.int32)
        return torch.cat([head, body])
    if w.pos_kind == "uniform":
        if w.seq_len != 1:
            raise ValueError("uniform positions are drawn per sequence (seq_len 1)")
        return torch.randint(0, w.table_rows, (w.batch,), generator=g, dtype=torch.int32)
    raise ValueError(f"unknown pos_kind {w.pos_kind!r}")


def random_positions(n: int, high: int, seed: int, low: int = 0) -> torch.Tensor:
    """Uniform int32 positions in [low, high) for edge-case tests."""
    return torch.randint(low, high, (n,), generator=_gen(seed), dtype=torch.int32)


def attn_tensors(w: AttnWorkload) -> dict:
    """Seeded CPU q, k, v of attention workload `w`."""
    return {"q": normal(w.q_shape, w.dtype, w.seed("q")),
            "k": normal(w.kv_shape, w.dtype, w.seed("k")),
            "v": normal(w.kv_shape, w.dtype, w.seed("v"))}


def attn_positions(w: AttnWorkload) -> Optional[torch.Tensor]:
    """The shared int32 index row of attention workload `w`, or None."""
    if w.pos_kind == "none":
        return None
    if w.pos_kind == "cls_offset":
        if w.seq_len_q != w.seq_len_k:
            raise ValueError("a shared index row needs seq_len_q == seq_len_k")
        g = _gen(w.seed("pos"))
        start = int(torch.randint(0, w.pos_start_max + 1, (1,), generator=g))
        n = w.seq_len_k - w.n_masked
        body = torch.arange(n, dtype=torch.int32) + start
        head = torch.full((w.n_masked,), -1, dtype=torch.int32)
        return torch.cat([head, body])
    raise ValueError(f"unknown pos_kind {w.pos_kind!r}")

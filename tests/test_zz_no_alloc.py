"""The allocation-free K-once attention (rope_attention_fwd_k_once_noalloc)
against the K-once call with a caller workspace (rope_attention_fwd_k_once),
through the C ABI: the same kernels, so the outputs must agree bit for bit.
Two calls in a row on one device share the library's staging array; the
second, smaller one must not see anything of the first."""
import numpy as np
import pytest
import torch

import rotary_position_embedding_fwd_amd as rp
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(B, Hq, Hk, S, D, R, seed, causal=True, pos=None, pairing="split_half"):
    q = W.normal((B, Hq, S, D), "bf16", seed).to(DEV)
    k = W.normal((B, Hk, S, D), "bf16", seed + 1).to(DEV)
    v = W.normal((B, Hk, S, D), "bf16", seed + 2).to(DEV)
    rows = S if pos is None else int(pos.max()) + 1
    c, s = (x.to(DEV) for x in rp.rope_build_table(rows, R, 10000.0))
    kw = dict(pairing=pairing, rotary_dim=R, causal=causal)
    if pos is not None:
        kw.update(q_pos=pos.to(DEV), k_pos=pos.to(DEV))
    return q, k, v, c, s, kw


def test_no_alloc_k_once_equals_workspace_call_twice():
    cases = [
        # a large call first (GQA 4:1, causal), then a smaller one (partial
        # rotary, head dim 64, positions with two skipped tokens)
        (2, 16, 4, 1024, 128, 128, 7100, True, None, "split_half"),
        (1, 8, 8, 300, 64, 32, 7200, True,
         torch.cat([torch.tensor([-1, -1], dtype=torch.int32),
                    torch.arange(298, dtype=torch.int32)]), "split_half"),
    ]
    for B, Hq, Hk, S, D, R, seed, causal, pos, pairing in cases:
        print(f"[gpu] no-alloc K once: q[{B},{Hq},{S},{D}] k heads {Hk} R={R}", flush=True)
        q, k, v, c, s, kw = _case(B, Hq, Hk, S, D, R, seed, causal, pos, pairing)
        ws = torch.empty_like(k)
        o_ws = torch.empty_like(q)
        rp.rope_attention(q, k, v, c, s, o=o_ws, k_workspace=ws, **kw)
        o_na = torch.full_like(q, 7.0)
        rp.rope_attention_noalloc(q, k, v, c, s, o_na, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
        # and the fused call (no workspace at all) gives the same bits
        o_f = torch.empty_like(q)
        rp.rope_attention(q, k, v, c, s, o=o_f, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_f.view(torch.int16), o_na.view(torch.int16))

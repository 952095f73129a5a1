// rope_plan.hpp -- host-side planning for librope: argument validation, the
// access width, and the grid shape. No GPU calls happen here, so the same
// plan drives the real launch (librope.hip) and the host emulation of the
// kernels used to check index arithmetic and bounds on the CPU.
#pragma once

#include <stdint.h>

#include "librope.h"
#include "rope_kernels.hpp"

namespace rope {

struct Plan {
  Args a;
  bool token;      // grid shape: token (one token per workgroup) or rows
  int vec;         // access width V (elements)
  bool aligned;    // V-element accesses are V-element aligned
  int dtype;       // rope_dtype_t
  int pairing;     // rope_pairing_t
  int64_t grid;    // workgroups
  int block;       // lanes per workgroup
  bool empty;      // nothing to do
  bool single;     // token shape: one workgroup per token, one lane per item
};

inline int64_t elem_bytes(int32_t dtype) { return dtype == ROPE_F32 ? 4 : 2; }

inline bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

inline bool is_empty(const rope_desc_t* d, int64_t hk) {
  return d->batch == 0 || d->seq_len == 0 || d->rotary_dim == 0 || d->n_heads_q + hk == 0;
}

// Checks that need no GPU and never dereference a device pointer.
inline rope_status_t validate(const void* q, const void* k, const rope_desc_t* d, bool with_k) {
  if (!d) return ROPE_ERR_NULL;
  if (d->dtype < ROPE_F32 || d->dtype > ROPE_BF16) return ROPE_ERR_DTYPE;
  if (d->layout != ROPE_BHSD && d->layout != ROPE_BSHD) return ROPE_ERR_LAYOUT;
  if (d->pairing != ROPE_SPLIT_HALF && d->pairing != ROPE_INTERLEAVED) return ROPE_ERR_LAYOUT;
  if (d->launch < ROPE_LAUNCH_AUTO || d->launch > ROPE_LAUNCH_TOKEN) return ROPE_ERR_LAYOUT;
  const int64_t hk = with_k ? d->n_heads_k : 0;
  if (d->batch < 0 || d->n_heads_q < 0 || d->seq_len < 0 || d->head_dim < 0 ||
      d->rotary_dim < 0 || d->table_rows < 0 || hk < 0)
    return ROPE_ERR_SHAPE;
  if ((d->rotary_dim & 1) || d->rotary_dim > d->head_dim) return ROPE_ERR_SHAPE;
  if (with_k && hk > d->n_heads_q) return ROPE_ERR_SHAPE;
  // heads and dims index with 32-bit integers inside the kernels
  if (d->n_heads_q + hk > ((int64_t)1 << 30) || d->rotary_dim > ((int64_t)1 << 30))
    return ROPE_ERR_SHAPE;
  if (is_empty(d, hk)) return ROPE_OK;
  if (!d->pos && d->seq_len > d->table_rows) return ROPE_ERR_SHAPE;
  if (d->pos && d->pos_batch_stride < 0) return ROPE_ERR_SHAPE;
  if ((d->n_heads_q > 0 && !q) || (hk > 0 && !k) || !d->cos || !d->sin) return ROPE_ERR_NULL;
  const int64_t e = elem_bytes(d->dtype);
  if ((reinterpret_cast<uintptr_t>(q) % e) || (hk > 0 && reinterpret_cast<uintptr_t>(k) % e))
    return ROPE_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(d->cos) % 16) || (reinterpret_cast<uintptr_t>(d->sin) % 16) ||
      (reinterpret_cast<uintptr_t>(d->pos) % 4))
    return ROPE_ERR_ALIGN;
  const int64_t row = d->batch * d->seq_len * d->head_dim * e;
  if (with_k && ranges_overlap(q, row * d->n_heads_q, k, row * hk)) return ROPE_ERR_ALIAS;
  return ROPE_OK;
}

// Largest access width V (elements, a power of two, at most 16 bytes) that
// keeps every chunk access V-aligned: V must divide the head dim, the span
// that chunks tile (R/2 for split-half, R for interleaved) and the element
// offset of each base pointer.
inline int pick_vec(const rope_desc_t* d, const void* q, const void* k, int64_t hk) {
  const int64_t e = elem_bytes(d->dtype);
  const int64_t span = d->pairing == ROPE_SPLIT_HALF ? d->rotary_dim / 2 : d->rotary_dim;
  const uintptr_t qa = reinterpret_cast<uintptr_t>(q) / e;
  const uintptr_t ka = hk > 0 ? reinterpret_cast<uintptr_t>(k) / e : 0;
  int v = (int)(16 / e);
  while (v > 1 && (d->head_dim % v || span % v || qa % v || ka % v)) v >>= 1;
  return v;
}

inline void set_strides(const rope_desc_t* d, int64_t heads, int64_t* sb, int64_t* sh,
                        int64_t* ss) {
  const int64_t S = d->seq_len, D = d->head_dim;
  if (d->layout == ROPE_BHSD) {  // [B, H, S, D]
    *sb = heads * S * D;
    *sh = S * D;
    *ss = D;
  } else {  // [B, S, H, D]
    *sb = S * heads * D;
    *ss = heads * D;
    *sh = D;
  }
}

// Validate and plan one call. `cus` is the device's compute-unit count.
inline rope_status_t make_plan(void* q, void* k, const rope_desc_t* d, bool with_k,
                               float sin_sign, int cus, Plan* pl) {
  const rope_status_t vs = validate(q, k, d, with_k);
  if (vs != ROPE_OK) return vs;
  *pl = Plan{};
  const int64_t hk = with_k ? d->n_heads_k : 0;
  pl->empty = is_empty(d, hk);
  if (pl->empty) return ROPE_OK;

  Args& a = pl->a;
  a.q = static_cast<char*>(q);
  a.k = static_cast<char*>(k);
  set_strides(d, d->n_heads_q, &a.q_sb, &a.q_sh, &a.q_ss);
  set_strides(d, hk, &a.k_sb, &a.k_sh, &a.k_ss);
  a.cos = d->cos;
  a.sin = d->sin;
  a.pos = d->pos;
  a.pos_bs = d->pos_batch_stride;
  a.table_rows = d->table_rows;
  a.batch = d->batch;
  a.seq_len = d->seq_len;
  a.n_tokens = d->batch * d->seq_len;
  a.half = (int32_t)(d->rotary_dim / 2);
  a.n_heads_q = (int32_t)d->n_heads_q;
  a.n_heads_k = (int32_t)hk;
  a.sin_sign = sin_sign;

  pl->dtype = d->dtype;
  pl->pairing = d->pairing;
  int v = pick_vec(d, q, k, hk);
  pl->aligned = true;
  if (d->pairing == ROPE_INTERLEAVED && v < 2) {
    // interleaved pairs that are not 2-element aligned: element-wise pairs
    v = 2;
    pl->aligned = false;
  }
  pl->vec = v;
  const int64_t span = d->pairing == ROPE_SPLIT_HALF ? d->rotary_dim / 2 : d->rotary_dim;
  a.lanes = (int32_t)(span / v);
  a.lanes_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((int64_t)1 << sh == a.lanes) a.lanes_shift = sh;
  const int h_total = a.n_heads_q + a.n_heads_k;

  // Rows shape: 256 (token, chunk) items per workgroup, each lane walking a
  // group of heads. Its waves per head group:
  a.n_items = a.n_tokens * a.lanes;
  const int64_t tiles = (a.n_items + kRowsBlock - 1) / kRowsBlock;
  const int64_t waves_per_group = tiles * (kRowsBlock / 64);
  const int64_t target_waves = (int64_t)cus * 8;

  pl->token = d->launch == ROPE_LAUNCH_TOKEN;
  if (d->launch == ROPE_LAUNCH_AUTO) {
    // decode, or too few tokens for the rows shape to fill the chip even
    // with one head per lane: one token per workgroup instead
    pl->token = d->seq_len == 1 || waves_per_group * h_total < target_waves;
  }

  if (pl->token) {
    const int64_t per_token = (int64_t)h_total * a.lanes;
    const int64_t want = ((per_token + 63) / 64) * 64;
    pl->block = (int)(want < 1024 ? want : 1024);
    const int64_t max_grid = (int64_t)cus * 64;
    pl->grid = a.n_tokens < max_grid ? a.n_tokens : max_grid;
    pl->single = pl->grid == a.n_tokens && pl->block >= per_token;
  } else {
    // Head groups, walked in group-slow order (all tiles of group 0, then of
    // group 1, ...): on MI355X this streams HBM best when a lane walks 4 heads
    // (one unrolled batch). Each group reads the cos/sin rows of its tokens
    // again, so groups grow in steps of 4 heads until those re-reads stay
    // under 15% of the call's Q/K traffic (long sequences have big tables);
    // they shrink below 4 heads only when there are too few waves.
    const int64_t e = elem_bytes(d->dtype);
    const int64_t rows_touched = d->pos ? (d->table_rows < a.n_tokens ? d->table_rows : a.n_tokens)
                                        : d->seq_len;
    const double table_pass = 4.0 * (double)d->rotary_dim * (double)rows_touched;
    const double qk_bytes = 2.0 * (double)e * (double)d->rotary_dim * (double)a.n_tokens * h_total;
    int g = 4;
    while (g < h_total && (double)((h_total + g - 1) / g) * table_pass > 0.15 * qk_bytes) g += 4;
    if (g > h_total) g = h_total;
    int64_t groups = (h_total + g - 1) / g;
    if (waves_per_group * groups < target_waves) {
      groups = (target_waves + waves_per_group - 1) / waves_per_group;
      if (groups > h_total) groups = h_total;
      g = (int)((h_total + groups - 1) / groups);
    }
    a.heads_per_group = g;
    a.n_groups = (int32_t)((h_total + g - 1) / g);
    a.n_tiles = tiles;
    a.group_slow = 1;
    const int64_t n_wg = tiles * a.n_groups;
    if (n_wg > 0x7fffffff) return ROPE_ERR_SHAPE;
    pl->grid = n_wg;
    pl->block = kRowsBlock;
  }
  return ROPE_OK;
}

// Call f.template run<T, V, PAIR, ALIGNED>() for the plan's kernel variant.
// The variants instantiated here are all the plans above can produce.
template <class F>
auto dispatch(const Plan& pl, F& f) -> decltype(f.template run<float, 1, kSplitHalf, true>()) {
  const bool split = pl.pairing == ROPE_SPLIT_HALF;
  switch (pl.dtype) {
    case ROPE_F32:
      if (split) {
        if (pl.vec == 4) return f.template run<float, 4, kSplitHalf, true>();
        if (pl.vec == 2) return f.template run<float, 2, kSplitHalf, true>();
        return f.template run<float, 1, kSplitHalf, true>();
      }
      if (!pl.aligned) return f.template run<float, 2, kInterleaved, false>();
      if (pl.vec == 4) return f.template run<float, 4, kInterleaved, true>();
      return f.template run<float, 2, kInterleaved, true>();
    case ROPE_F16:
      if (split) {
        if (pl.vec == 8) return f.template run<_Float16, 8, kSplitHalf, true>();
        if (pl.vec == 4) return f.template run<_Float16, 4, kSplitHalf, true>();
        if (pl.vec == 2) return f.template run<_Float16, 2, kSplitHalf, true>();
        return f.template run<_Float16, 1, kSplitHalf, true>();
      }
      if (!pl.aligned) return f.template run<_Float16, 2, kInterleaved, false>();
      if (pl.vec == 8) return f.template run<_Float16, 8, kInterleaved, true>();
      if (pl.vec == 4) return f.template run<_Float16, 4, kInterleaved, true>();
      return f.template run<_Float16, 2, kInterleaved, true>();
    default:
      if (split) {
        if (pl.vec == 8) return f.template run<__bf16, 8, kSplitHalf, true>();
        if (pl.vec == 4) return f.template run<__bf16, 4, kSplitHalf, true>();
        if (pl.vec == 2) return f.template run<__bf16, 2, kSplitHalf, true>();
        return f.template run<__bf16, 1, kSplitHalf, true>();
      }
      if (!pl.aligned) return f.template run<__bf16, 2, kInterleaved, false>();
      if (pl.vec == 8) return f.template run<__bf16, 8, kInterleaved, true>();
      if (pl.vec == 4) return f.template run<__bf16, 4, kInterleaved, true>();
      return f.template run<__bf16, 2, kInterleaved, true>();
  }
}

}  // namespace rope

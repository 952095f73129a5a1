// rope_attn_plan.hpp -- host-side checks and launch plan of the fused
// attention (rope_attention.hpp). Never touches device memory.
#pragma once

#include <stdint.h>

#include <cfloat>
#include <cmath>

#include "librope.h"
#include "rope_attention.hpp"

namespace rope {
namespace attn {

struct AttnPlan {
  AttnArgs a;
  bool empty;
  int64_t grid;
  int head_dim;
  int pairing;
  int h16;  // split-half: (R/2)/16; 0 otherwise
  int64_t lds;
};

inline bool ranges_meet(const void* p, int64_t bytes, const void* q, int64_t qbytes) {
  if (!p || !q || bytes <= 0 || qbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + (uintptr_t)bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + (uintptr_t)qbytes;
  return a0 < b1 && b0 < a1;
}

inline rope_status_t make_attn_plan(const rope_attn_desc_t* d, AttnPlan* pl) {
  if (!d || !pl) return ROPE_ERR_NULL;
  *pl = AttnPlan{};
  if (d->dtype != ROPE_BF16) return ROPE_ERR_DTYPE;
  if (d->pairing != ROPE_SPLIT_HALF && d->pairing != ROPE_INTERLEAVED) return ROPE_ERR_LAYOUT;
  const int64_t B = d->batch, Hq = d->n_heads_q, Hk = d->n_heads_k, Sq = d->seq_len_q,
                Sk = d->seq_len_k, D = d->head_dim, R = d->rotary_dim;
  if (B < 0 || Sq < 0 || Sk < 0 || Hq < 1 || Hk < 1 || Hq % Hk) return ROPE_ERR_SHAPE;
  if (D != 64 && D != 128) return ROPE_ERR_SHAPE;
  if (R < 0 || R > D || (R & 1)) return ROPE_ERR_SHAPE;
  if (d->pairing == ROPE_SPLIT_HALF ? (R % 32) : (R % 8)) return ROPE_ERR_SHAPE;
  if (d->causal && Sq > Sk) return ROPE_ERR_SHAPE;
  if (!std::isfinite(d->scale) || d->table_rows < 0) return ROPE_ERR_SHAPE;
  if (d->k_rotated != 0 && d->k_rotated != 1) return ROPE_ERR_SHAPE;
  // the kernel works with |scale| * log2(e) as a normal float32 (a negative
  // scale enters as a sign flip of Q)
  const double scale = d->scale != 0.0 ? d->scale : 1.0 / std::sqrt((double)D);
  const float scale_log2e = (float)(std::fabs(scale) * 1.4426950408889634);  // log2(e)
  if (!(scale_log2e >= FLT_MIN && scale_log2e <= FLT_MAX)) return ROPE_ERR_SHAPE;
  if (d->q_pos_batch_stride < 0 || d->k_pos_batch_stride < 0) return ROPE_ERR_SHAPE;
  // 32-bit index arithmetic inside the kernel
  const int64_t lim = (int64_t)1 << 30;
  if (B > lim || Hq > lim || Sq > lim || Sk > lim) return ROPE_ERR_SHAPE;
  // the kernel reads one head's K and V rows and the tables through 32-bit
  // byte offsets from a per-workgroup base: each must stay under 4 GiB
  const int64_t lim32 = ((int64_t)1 << 32) - 16;
  if (Sk * D * 2 > lim32 || (R > 0 && d->table_rows > lim32 / (R * 2))) return ROPE_ERR_SHAPE;
  // byte counts of Q/O and K/V (and the table) must not overflow
  int64_t qbytes = 0, kvbytes = 0, tbytes = 0;
  if (__builtin_mul_overflow(B * Hq, Sq, &qbytes) || __builtin_mul_overflow(qbytes, D * 2, &qbytes) ||
      __builtin_mul_overflow(B * Hk, Sk, &kvbytes) ||
      __builtin_mul_overflow(kvbytes, D * 2, &kvbytes) ||
      __builtin_mul_overflow(d->table_rows, R * 2, &tbytes))
    return ROPE_ERR_SHAPE;
  pl->empty = B == 0 || Sq == 0;
  if (pl->empty) return ROPE_OK;
  const bool rotate = d->rotate && R > 0;
  if (rotate && ((!d->q_pos || !d->k_pos) && Sk > d->table_rows)) return ROPE_ERR_SHAPE;
  if (!d->q || !d->o || (Sk > 0 && (!d->k || !d->v))) return ROPE_ERR_NULL;
  if (rotate && (!d->cos || !d->sin)) return ROPE_ERR_NULL;
  auto mis = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) % m) != 0; };
  if (mis(d->q, 16) || mis(d->k, 16) || mis(d->v, 16) || mis(d->o, 16)) return ROPE_ERR_ALIGN;
  if (rotate && (mis(d->cos, 16) || mis(d->sin, 16))) return ROPE_ERR_ALIGN;
  if (mis(d->q_pos, 4) || mis(d->k_pos, 4)) return ROPE_ERR_ALIGN;
  if (ranges_meet(d->o, qbytes, d->q, qbytes) || ranges_meet(d->o, qbytes, d->k, kvbytes) ||
      ranges_meet(d->o, qbytes, d->v, kvbytes))
    return ROPE_ERR_ALIAS;
  if (rotate && (ranges_meet(d->o, qbytes, d->cos, tbytes) ||
                 ranges_meet(d->o, qbytes, d->sin, tbytes)))
    return ROPE_ERR_ALIAS;
  // the index arrays' extents: ((B - 1) * stride + S) int32 entries
  auto index_bytes = [&](int64_t stride, int64_t S, int64_t* out) {
    int64_t n = 0;
    return !__builtin_mul_overflow(B - 1, stride, &n) && !__builtin_add_overflow(n, S, &n) &&
           !__builtin_mul_overflow(n, (int64_t)4, out);
  };
  int64_t qpb = 0, kpb = 0;
  if ((d->q_pos && !index_bytes(d->q_pos_batch_stride, Sq, &qpb)) ||
      (d->k_pos && !index_bytes(d->k_pos_batch_stride, Sk, &kpb)))
    return ROPE_ERR_SHAPE;
  if (d->q_pos && ranges_meet(d->o, qbytes, d->q_pos, qpb)) return ROPE_ERR_ALIAS;
  if (d->k_pos && ranges_meet(d->o, qbytes, d->k_pos, kpb)) return ROPE_ERR_ALIAS;

  AttnArgs& a = pl->a;
  a.q = static_cast<const __bf16*>(d->q);
  a.k = static_cast<const __bf16*>(d->k);
  a.v = static_cast<const __bf16*>(d->v);
  a.o = static_cast<__bf16*>(d->o);
  a.cos = d->cos;
  a.sin = d->sin;
  a.q_pos = d->q_pos;
  a.k_pos = d->k_pos;
  a.q_pos_bs = d->q_pos_batch_stride;
  a.k_pos_bs = d->k_pos_batch_stride;
  a.table_rows = d->table_rows;
  a.batch = (int32_t)B;
  a.n_heads_q = (int32_t)Hq;
  a.n_heads_k = (int32_t)Hk;
  a.seq_q = (int32_t)Sq;
  a.seq_k = (int32_t)Sk;
  a.half = rotate ? (int32_t)(R / 2) : 0;
  a.rotate = rotate ? 1 : 0;
  a.rotate_k = (rotate && !d->k_rotated) ? 1 : 0;
  a.causal = d->causal ? 1 : 0;
  // query heads per workgroup: the largest power of two (at most the 8
  // waves) dividing the group of query heads that share a K/V head, so one
  // staged K/V tile serves all 256 rows of the workgroup
  const int64_t group = Hq / Hk;
  int32_t hw = 1;
  while (hw < kWaves && group % (2 * hw) == 0) hw *= 2;
  // Small grids at head dim 64: G = 2 or 4 groups of waves share each
  // workgroup's rows (256 / G of them) and take turns on its key tiles,
  // which divides the chain of dependent tiles a workgroup walks by G and
  // multiplies the workgroups by G. It pays while the grid still fits the
  // 256 compute units once (on MI355X, causal, 1024 tokens, two groups:
  // 16 heads 24.1 us vs 32.6, 32 heads 24.7 vs 33.2, but 48 heads 38.1 vs
  // 33.4 and 64 heads 46.2 vs 33.6).
  const int64_t grid_full = (Sq + kRows / hw - 1) / (kRows / hw) * (Hq / hw) * B;
  int32_t groups = 1;
  if (D == 64)
    while (groups < 4 && 2 * groups * grid_full <= 256) groups *= 2;
  a.groups = groups;
  while (hw > kWaves / groups) hw /= 2;  // a group's waves cover its heads
  const int32_t rows_wg = kRows / groups;
  a.hw = hw;
  a.rows = rows_wg / hw;
  a.head_groups = (int32_t)(Hq / hw);
  a.q_tiles = (int32_t)((Sq + a.rows - 1) / a.rows);
  a.scale_log2e = scale_log2e;
  a.negate_q = scale < 0.0;
  pl->grid = (int64_t)a.q_tiles * a.head_groups * B;
  if (pl->grid > 0x7fffffff) return ROPE_ERR_SHAPE;
  pl->head_dim = (int)D;
  pl->pairing = d->pairing;
  pl->h16 = (rotate && d->pairing == ROPE_SPLIT_HALF) ? (int)(R / 32) : 0;
  pl->lds = D == 64 ? lds_bytes_groups<64>(groups) : lds_bytes_groups<128>(groups);
  return ROPE_OK;
}

}  // namespace attn
}  // namespace rope

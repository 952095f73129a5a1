// rope_xpos.hpp -- RoPE with XPOS scaling, on the general form of rope_apply
// (strided views, in place or out of place, cos/sin tables).
//
// XPOS (rotary-embedding-torch docs, Key Parameters: `use_xpos`, length
// extrapolation) multiplies each rotated pair i of a query row at position p
// by zeta_i^e and each rotated pair of a key row by zeta_i^-e, e = (p - c)/B,
// so that a query at n and a key at m meet with the factor zeta_i^((n-m)/B).
// The pages name the option only; the scales here are those of the xPos
// paper (Sun et al., "A Length-Extrapolatable Transformer", ACL 2023):
// zeta_i = (2i/R + gamma) / (1 + gamma), gamma = 0.4, scale base B = 512.
// The caller passes them as two float32 tables laid out like cos and sin
// (rope_build_xpos_table). A factor is the same for both elements of a pair,
// so it commutes with the pair's rotation: the backward (sin negated) uses
// the same tables.
//
// One workgroup per token; its lanes walk (head, slot) items, slot k < R/2
// being pair k of the row (split-half: dims k and k + R/2; interleaved: 2k
// and 2k + 1) and, out of place, slots past R/2 copying two of the dims >= R.
// Within a head row consecutive lanes take consecutive slots, so each half of
// a split-half row (and an interleaved row) is read and written coalesced.
// The body is a plain function of (token, lane) so that the host can run it
// over every lane of a grid and check every access.
#pragma once

#include <stdint.h>

#include <cfloat>
#include <cmath>

#include "librope.h"
#include "rope_kernels.hpp"
#include "rope_plan.hpp"

namespace rope {
namespace xpos {

constexpr int kBlock = 256;  // lanes per workgroup (one token)

struct XArgs {
  View q_in, k_in, q_out, k_out;  // outputs equal the inputs in place
  const float* cos;               // frequency i of position p at [p*t_row + i*t_col]
  const float* sin;
  const float* zq;                // XPOS factors of query rows, laid out like cos
  const float* zk;                // ... of key rows
  const int32_t* pos;             // nullptr: p = s
  int64_t t_row, pos_bs, table_rows, seq_len, n_tokens;
  int32_t t_col;
  int32_t half;                   // R / 2
  int32_t head_dim;
  int32_t n_heads_q, n_heads_k;
  int32_t slots;                  // items per head row: R/2, or ceil(D/2) out of place
  int32_t interleaved;
  int32_t oop;                    // some output differs from its input
  float sin_sign;                 // +1 forward, -1 backward
};

// All items of one token that lane t of its workgroup owns.
template <typename T>
ROPE_HD void xpos_token(const XArgs& a, int64_t token, int t) {
  const int64_t b = token / a.seq_len, s = token - b * a.seq_len;
  const int64_t p = a.pos ? (int64_t)a.pos[b * a.pos_bs + s] : s;
  const bool rot = p >= 0 && p < a.table_rows;
  const int per_token = (a.n_heads_q + a.n_heads_k) * a.slots;
  for (int idx = t; idx < per_token; idx += kBlock) {
    const int head = idx / a.slots, k = idx - head * a.slots;
    const bool is_k = head >= a.n_heads_q;
    const int h = is_k ? head - a.n_heads_q : head;
    const View& vi = is_k ? a.k_in : a.q_in;
    const View& vo = is_k ? a.k_out : a.q_out;
    const T* in = reinterpret_cast<const T*>(vi.base) + b * vi.sb + h * vi.sh + s * vi.ss;
    T* out = reinterpret_cast<T*>(vo.base) + b * vo.sb + h * vo.sh + s * vo.ss;
    if (k < a.half) {
      const int j1 = a.interleaved ? 2 * k : k;
      const int j2 = a.interleaved ? 2 * k + 1 : k + a.half;
      if (!rot) {  // a skipped token: untouched in place, copied out of place
        if (a.oop) {
          out[j1] = in[j1];
          out[j2] = in[j2];
        }
        continue;
      }
      const int64_t ti = p * a.t_row + (int64_t)k * a.t_col;
      const float c = a.cos[ti], sn = a.sin_sign * a.sin[ti];
      const float z = is_k ? a.zk[ti] : a.zq[ti];
      float y1, y2;
      rotate_pair(to_f32(in[j1]), to_f32(in[j2]), c, sn, y1, y2);
      out[j1] = from_f32<T>(y1 * z);
      out[j2] = from_f32<T>(y2 * z);
    } else {  // out of place only: two of the dims >= R
      const int j = 2 * k;
      out[j] = in[j];
      if (j + 1 < a.head_dim) out[j + 1] = in[j + 1];
    }
  }
}

struct XPlan {
  XArgs a;
  bool empty;
  int dtype;
};

// Validate a rope_apply_xpos call and plan it. Never touches device memory.
inline rope_status_t make_xpos_plan(const rope_apply_desc_t* d, const float* zq, const float* zk,
                                    XPlan* pl) {
  if (!pl) return ROPE_ERR_NULL;
  *pl = XPlan{};
  const rope_status_t vs = validate_apply(d);
  if (vs != ROPE_OK) return vs;
  if (d->angles != ROPE_ANGLES_TABLE) return ROPE_ERR_LAYOUT;
  if (d->launch != ROPE_LAUNCH_AUTO) return ROPE_ERR_LAYOUT;
  pl->empty = apply_is_empty(d);
  if (pl->empty) return ROPE_OK;
  if ((d->n_heads_q > 0 && !zq) || (d->n_heads_k > 0 && !zk)) return ROPE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(zq) % 4) || (reinterpret_cast<uintptr_t>(zk) % 4))
    return ROPE_ERR_ALIGN;
  // 32-bit lane indices inside a token
  const int64_t slots_in = d->rotary_dim / 2;
  const int64_t slots_oop = (d->head_dim + 1) / 2;
  if ((d->n_heads_q + d->n_heads_k) * slots_oop > ((int64_t)1 << 30)) return ROPE_ERR_SHAPE;
  if (d->batch * d->seq_len > 0x7fffffff) return ROPE_ERR_SHAPE;  // one workgroup per token

  XArgs& a = pl->a;
  a.q_in = to_view(d->q_in);
  a.k_in = to_view(d->k_in);
  a.q_out = d->q_out.data ? to_view(d->q_out) : a.q_in;
  a.k_out = d->k_out.data ? to_view(d->k_out) : a.k_in;
  auto same = [](const View& x, const View& y) {
    return x.base == y.base && x.sb == y.sb && x.sh == y.sh && x.ss == y.ss;
  };
  const bool oop = !same(a.q_in, a.q_out) || (d->n_heads_k > 0 && !same(a.k_in, a.k_out));
  a.cos = d->cos;
  a.sin = d->sin;
  a.zq = zq;
  a.zk = zk;
  a.pos = d->pos;
  a.half = (int32_t)(d->rotary_dim / 2);
  a.t_row = d->table_row_stride ? d->table_row_stride : a.half;
  a.t_col = (int32_t)d->table_col_stride;
  a.pos_bs = d->pos_batch_stride;
  a.table_rows = d->table_rows;
  a.seq_len = d->seq_len;
  a.n_tokens = d->batch * d->seq_len;
  a.head_dim = (int32_t)d->head_dim;
  a.n_heads_q = (int32_t)d->n_heads_q;
  a.n_heads_k = (int32_t)d->n_heads_k;
  a.slots = (int32_t)(oop ? slots_oop : slots_in);
  a.interleaved = d->pairing == ROPE_INTERLEAVED ? 1 : 0;
  a.oop = oop ? 1 : 0;
  a.sin_sign = (float)d->direction;
  pl->dtype = d->dtype;

  // The factor tables span what cos and sin span, and no written view may
  // meet them (they are read for the whole launch).
  int64_t tbytes = 0;
  if (d->table_rows > 0 &&
      (__builtin_mul_overflow(d->table_rows - 1, a.t_row, &tbytes) ||
       __builtin_add_overflow(tbytes, (int64_t)(a.half - 1) * a.t_col + 1, &tbytes) ||
       __builtin_mul_overflow(tbytes, (int64_t)4, &tbytes)))
    return ROPE_ERR_SHAPE;
  const int64_t e = elem_bytes(d->dtype);
  const ViewX qo = view_x(d->q_out.data ? d->q_out : d->q_in, d->batch, d->n_heads_q,
                          d->seq_len, d->head_dim);
  const ViewX ko = view_x(d->k_out.data ? d->k_out : d->k_in, d->batch, d->n_heads_k,
                          d->seq_len, d->head_dim);
  auto meets_written = [&](const void* base) {
    if (!base || tbytes <= 0) return false;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base), hi = lo + (uintptr_t)tbytes;
    for (const ViewX* w : {&qo, &ko}) {
      if (view_empty(*w)) continue;
      const uintptr_t w0 = w->p, w1 = w->p + (uintptr_t)(view_span(*w) * e);
      if (lo < w1 && w0 < hi) return true;
    }
    return false;
  };
  if ((d->n_heads_q > 0 && meets_written(zq)) || (d->n_heads_k > 0 && meets_written(zk)))
    return ROPE_ERR_ALIAS;
  return ROPE_OK;
}

// zeta_i^((p - center) / scale_base) for query rows and its inverse power for
// key rows, zeta_i = (2i/R + gamma) / (1 + gamma): binary64, each entry
// rounded once to float32. Row p, column i of [table_rows, R/2].
inline rope_status_t build_xpos_table(float* zq, float* zk, int64_t table_rows,
                                      int64_t rotary_dim, double scale_base, double gamma,
                                      double center) {
  if (table_rows < 0 || rotary_dim < 0 || (rotary_dim & 1) || !(scale_base > 0.0) ||
      !std::isfinite(scale_base) || !(gamma > 0.0) || !std::isfinite(gamma) ||
      !std::isfinite(center))
    return ROPE_ERR_SHAPE;
  const int64_t half = rotary_dim / 2;
  if (table_rows == 0 || half == 0) return ROPE_OK;
  if (!zq || !zk) return ROPE_ERR_NULL;
  for (int64_t i = 0; i < half; ++i) {
    const double zeta = (2.0 * (double)i / (double)rotary_dim + gamma) / (1.0 + gamma);
    for (int64_t p = 0; p < table_rows; ++p) {
      const double ex = ((double)p - center) / scale_base;
      zq[p * half + i] = (float)std::pow(zeta, ex);
      zk[p * half + i] = (float)std::pow(zeta, -ex);
    }
  }
  return ROPE_OK;
}

}  // namespace xpos
}  // namespace rope

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
// Chunked shape (xpos_block): a lane owns one chunk of one token and walks
// it over a group of heads, loading the chunk's cos, sin and factors once and
// issuing several heads' loads before their stores. A
// chunk is V contiguous elements moved as one access, V the widest that
// every view's alignment allows (as for rope_apply): split-half chunk c
// covers pairs cV .. cV+V-1 (dims cV.. and R/2+cV..), interleaved chunk c the
// V/2 pairs of dims cV .. cV+V-1; out of place, further chunks copy the dims
// >= R. Consecutive lanes take consecutive chunks of a row, then the next
// token, so rows stream coalesced.
// Element shape (xpos_token), for interleaved views that are not even
// 2-element aligned: one workgroup per token, lanes over (head, pair) items.
// Both bodies are plain functions of (workgroup, lane) so that the host can
// run them over every lane of a grid and check every access.
#pragma once

#include <stdint.h>

#include <cfloat>
#include <cmath>

#include "librope.h"
#include "rope_kernels.hpp"
#include "rope_plan.hpp"

namespace rope {
namespace xpos {

constexpr int kBlock = 256;  // lanes per workgroup

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
  // chunked shape
  int32_t chunks;                 // pair chunks per head row
  int32_t row_items;              // chunks per head row, copies included
  int32_t heads_per_group;        // rows one lane walks
  int32_t n_groups;               // ceil((Hq + Hk) / heads_per_group)
  int32_t token_major;            // 1: lanes run token-slow (views with adjacent heads)
  int32_t t_vec;                  // 1: a chunk's table entries load as float4s
  int64_t n_items;                // lanes: head groups x tokens x row_items
  // lanes shape
  int32_t chunks_shift;           // log2(chunks)
  int32_t tokens_per_block;       // head-major: tokens of a workgroup
  int32_t tokens_shift;           // log2(tokens_per_block)
  int32_t pad0;
  int64_t n_tiles;                // head-major: token tiles per head group
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

// Factor, cos and sin of NP consecutive pairs from pair `first` of row p.
template <int NP>
ROPE_HD void load_tables(const XArgs& a, int64_t p, int first, bool key, float* c, float* sn,
                         float* z) {
  const float* zt = key ? a.zk : a.zq;
  const int64_t base = p * a.t_row + (int64_t)first * a.t_col;
  if constexpr (NP % 4 == 0) {
    if (a.t_vec) {
#pragma unroll
      for (int j = 0; j < NP; j += 4) {
        const float4 cv = *reinterpret_cast<const float4*>(a.cos + base + j);
        const float4 sv = *reinterpret_cast<const float4*>(a.sin + base + j);
        const float4 zv = *reinterpret_cast<const float4*>(zt + base + j);
        c[j] = cv.x; c[j + 1] = cv.y; c[j + 2] = cv.z; c[j + 3] = cv.w;
        sn[j] = sv.x; sn[j + 1] = sv.y; sn[j + 2] = sv.z; sn[j + 3] = sv.w;
        z[j] = zv.x; z[j + 1] = zv.y; z[j + 2] = zv.z; z[j + 3] = zv.w;
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int64_t ti = base + (int64_t)j * a.t_col;
    c[j] = a.cos[ti];
    sn[j] = a.sin[ti];
    z[j] = zt[ti];
  }
}

// The item of lane t of workgroup `blk` (chunked shape): one chunk of one
// token, walked over a group of G heads (Q heads first, then K heads), so
// the chunk's cos, sin and factors are loaded once for G rows. Items run
// chunk fastest, then token, then head group.
template <typename T, int V, int PAIR, int U>
ROPE_HD void xpos_block(const XArgs& a, int64_t blk, int t) {
  constexpr int NP = PAIR == kSplitHalf ? V : V / 2;  // pairs per chunk
  static_assert(NP >= 1, "an interleaved chunk holds at least one pair");
  const int64_t item = blk * kBlock + t;
  if (item >= a.n_items) return;
  int64_t g, token;
  int c;
  if (a.token_major) {  // token, head group, chunk: a token's rows are adjacent
    const int64_t per_token = (int64_t)a.n_groups * a.row_items;
    token = item / per_token;
    const int64_t rest = item - token * per_token;
    g = rest / a.row_items;
    c = (int)(rest - g * a.row_items);
  } else {  // head group, token, chunk
    const int64_t per_group = a.n_tokens * a.row_items;
    g = item / per_group;
    const int64_t rest = item - g * per_group;
    token = rest / a.row_items;
    c = (int)(rest - token * a.row_items);
  }
  const int64_t b = token / a.seq_len, s = token - b * a.seq_len;
  const int h_total = a.n_heads_q + a.n_heads_k;
  const int h0 = (int)g * a.heads_per_group;
  const int h1 = imin(h_total, h0 + a.heads_per_group);
  auto row = [&](int head, bool out) {
    const bool is_k = head >= a.n_heads_q;
    const int h = is_k ? head - a.n_heads_q : head;
    const View& v = out ? (is_k ? a.k_out : a.q_out) : (is_k ? a.k_in : a.q_in);
    return reinterpret_cast<T*>(v.base) + b * v.sb + h * v.sh + s * v.ss;
  };
  if (c >= a.chunks) {  // out of place only: dims >= R, V at a time
    const int j0 = 2 * a.half + (c - a.chunks) * V;
    for (int head = h0; head < h1; ++head) {
      const T* in = row(head, false);
      T* out = row(head, true);
      if (j0 + V <= a.head_dim) {
        Chunk<T, V, true> x;
        x.load(in + j0);
        x.store(out + j0);
      } else {
        for (int j = j0; j < a.head_dim; ++j) out[j] = in[j];
      }
    }
    return;
  }
  const int64_t p = a.pos ? (int64_t)a.pos[b * a.pos_bs + s] : s;
  const bool rot = p >= 0 && p < a.table_rows;
  if (!rot && !a.oop) return;  // a skipped token: untouched in place
  const int first = PAIR == kSplitHalf ? c * V : c * NP;  // first pair of the chunk
  float cs[NP], sn[NP], zq[NP], zk[NP];
  if (rot) {
    if (h0 < a.n_heads_q) load_tables<NP>(a, p, first, false, cs, sn, zq);
    if (h1 > a.n_heads_q) load_tables<NP>(a, p, first, true, cs, sn, zk);
#pragma unroll
    for (int j = 0; j < NP; ++j) sn[j] *= a.sin_sign;
  }
  // U heads at a time: all their loads are issued before the first store
  constexpr int kU = U;
  for (int hb = h0; hb < h1; hb += kU) {
    if constexpr (PAIR == kSplitHalf) {
      Chunk<T, V, true> x1[kU], x2[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (hb + u < h1) {
          const T* in = row(hb + u, false);
          x1[u].load(in + c * V);
          x2[u].load(in + a.half + c * V);
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (hb + u < h1) {
          const float* z = hb + u >= a.n_heads_q ? zk : zq;
          if (rot) {
#pragma unroll
            for (int j = 0; j < NP; ++j) {
              float y1, y2;
              rotate_pair(to_f32(x1[u].v[j]), to_f32(x2[u].v[j]), cs[j], sn[j], y1, y2);
              x1[u].v[j] = from_f32<T>(y1 * z[j]);
              x2[u].v[j] = from_f32<T>(y2 * z[j]);
            }
          }
          T* out = row(hb + u, true);
          x1[u].store(out + c * V);
          x2[u].store(out + a.half + c * V);
        }
      }
    } else {
      Chunk<T, V, true> x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (hb + u < h1) x[u].load(row(hb + u, false) + c * V);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (hb + u < h1) {
          const float* z = hb + u >= a.n_heads_q ? zk : zq;
          if (rot) {
#pragma unroll
            for (int j = 0; j < NP; ++j) {
              float y1, y2;
              rotate_pair(to_f32(x[u].v[2 * j]), to_f32(x[u].v[2 * j + 1]), cs[j], sn[j], y1,
                          y2);
              x[u].v[2 * j] = from_f32<T>(y1 * z[j]);
              x[u].v[2 * j + 1] = from_f32<T>(y2 * z[j]);
            }
          }
          x[u].store(row(hb + u, true) + c * V);
        }
      }
    }
  }
}

// ------------------------------------------------------------ lanes shape
// One chunk of one (token, head) per lane and nothing looped: in place,
// 16-byte chunks, [rows, R/2]-style tables (every table read a float4).
//   head-major views (TOKEN false): the workgroups of rope_head_lanes_kernel,
//     tokens_per_block tokens x chunks x heads_per_group heads, lanes chunk
//     fastest, then token, then head; workgroups over the token tiles of head
//     group 0 first. The heads of a group ask for the same cos/sin rows.
//   token-major views (TOKEN true): one token per workgroup, lanes over
//     (head, chunk), so a workgroup walks the token's adjacent rows.
// A lane issues its row loads and its cos, sin and factor loads back to back;
// whether the call has an index tensor (IDX) is a compile-time choice, so no
// branch joins the two cases after the loads. A skipped token (IDX) asks for
// table row 0 like the others and is not written.
template <typename T, int V, int PAIR, bool IDX, bool TOKEN>
ROPE_HD void xpos_lanes(const XArgs& a, int64_t blk, int t) {
  constexpr int NP = PAIR == kSplitHalf ? V : V / 2;  // pairs per chunk
  static_assert(NP % 4 == 0, "table entries move as float4s");
  const int c = t & (a.chunks - 1);
  const int rest = t >> a.chunks_shift;
  const int h_total = a.n_heads_q + a.n_heads_k;
  int64_t n;
  int head;
  if constexpr (TOKEN) {
    n = blk;
    head = rest;
    if (head >= h_total) return;
  } else {
    const int tl = rest & (a.tokens_per_block - 1);
    const int hl = rest >> a.tokens_shift;
    const int64_t group = blk / a.n_tiles;
    const int64_t tile = blk - group * a.n_tiles;
    n = (tile << a.tokens_shift) + tl;
    head = (int)group * a.heads_per_group + hl;
    if (n >= a.n_tokens || hl >= a.heads_per_group || head >= h_total) return;
  }
  const int64_t b = n / a.seq_len, s = n - b * a.seq_len;
  const bool is_k = head >= a.n_heads_q;
  const int h = is_k ? head - a.n_heads_q : head;
  const View& v = is_k ? a.k_in : a.q_in;
  T* row = reinterpret_cast<T*>(v.base) + b * v.sb + h * v.sh + s * v.ss;
  Chunk<T, V, true> x1, x2;  // split-half: both halves; interleaved: x1 only
  if constexpr (PAIR == kSplitHalf) {
    x1.load(row + c * V);
    x2.load(row + a.half + c * V);
  } else {
    x1.load(row + c * V);
  }
  int64_t p = s;  // without an index the host has checked seq_len <= table_rows
  if constexpr (IDX) {
    if (a.table_rows == 0) return;  // uniform: every token is skipped
    p = a.pos[b * a.pos_bs + s];
    if (p >= a.table_rows) p = -1;
  }
  const int64_t base = (p < 0 ? 0 : p) * a.t_row + (int64_t)c * NP;
  const float* zt = is_k ? a.zk : a.zq;
  float cs[NP], sn[NP], z[NP];
#pragma unroll
  for (int j = 0; j < NP; j += 4) {
    const float4 cv = *reinterpret_cast<const float4*>(a.cos + base + j);
    const float4 sv = *reinterpret_cast<const float4*>(a.sin + base + j);
    const float4 zv = *reinterpret_cast<const float4*>(zt + base + j);
    cs[j] = cv.x; cs[j + 1] = cv.y; cs[j + 2] = cv.z; cs[j + 3] = cv.w;
    sn[j] = sv.x; sn[j + 1] = sv.y; sn[j + 2] = sv.z; sn[j + 3] = sv.w;
    z[j] = zv.x; z[j + 1] = zv.y; z[j + 2] = zv.z; z[j + 3] = zv.w;
  }
  if constexpr (IDX) {
    if (p < 0) return;  // a skipped token: untouched in place
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    float y1, y2;
    if constexpr (PAIR == kSplitHalf) {
      rotate_pair(to_f32(x1.v[j]), to_f32(x2.v[j]), cs[j], a.sin_sign * sn[j], y1, y2);
      x1.v[j] = from_f32<T>(y1 * z[j]);
      x2.v[j] = from_f32<T>(y2 * z[j]);
    } else {
      rotate_pair(to_f32(x1.v[2 * j]), to_f32(x1.v[2 * j + 1]), cs[j], a.sin_sign * sn[j], y1,
                  y2);
      x1.v[2 * j] = from_f32<T>(y1 * z[j]);
      x1.v[2 * j + 1] = from_f32<T>(y2 * z[j]);
    }
  }
  if constexpr (PAIR == kSplitHalf) {
    x1.store(row + c * V);
    x2.store(row + a.half + c * V);
  } else {
    x1.store(row + c * V);
  }
}

struct XPlan {
  XArgs a;
  bool empty;
  int dtype;
  int vec;         // chunk width V; 0: element shape
  int64_t grid;    // workgroups
  int lanes;       // 0: chunked or element shape; 1: lanes, head-major; 2: lanes, token-major
  int block;       // lanes per workgroup (lanes shape; the others use kBlock)
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

  // chunked shape unless interleaved pairs are not 2-element aligned
  const int v = pick_vec(d);
  const bool chunked = !(a.interleaved && v < 2);
  if (chunked) {
    pl->vec = v;
    a.chunks = (int32_t)((a.interleaved ? d->rotary_dim : d->rotary_dim / 2) / v);
    const int64_t copies = oop ? (d->head_dim - d->rotary_dim + v - 1) / v : 0;
    a.row_items = (int32_t)(a.chunks + copies);
    // 8 heads per lane, fewer when that would leave the chip short of lanes
    // (measured on MI355X, Llama prefill [B,H,S,D]: 62.1 us with 8, 64.4 us
    // with 4, 73.5 us with 2). Views whose heads of a token are adjacent in
    // memory ([B,S,H,D], packed QKV) run one head per lane, token-slow, so a
    // wave's lanes sweep each token's rows in memory order (Llama shape as
    // packed QKV: 72 us that way, 88 us with 4 heads per lane).
    const int64_t h_total = d->n_heads_q + d->n_heads_k;
    a.token_major = (d->n_heads_q > 1 && d->q_in.stride_h < d->q_in.stride_s) ? 1 : 0;
    int64_t g = a.token_major ? 1 : (h_total < 8 ? h_total : 8);
    while (g > 1 && ((h_total + g - 1) / g) * a.n_tokens * a.row_items < 256 * 256) g /= 2;
    a.heads_per_group = (int32_t)g;
    a.n_groups = (int32_t)((h_total + g - 1) / g);
    int64_t items = 0;
    if (__builtin_mul_overflow((int64_t)a.n_groups, a.n_tokens * a.row_items, &items))
      return ROPE_ERR_SHAPE;
    a.n_items = items;
    const int np = a.interleaved ? v / 2 : v;
    a.t_vec = (np % 4 == 0 && a.t_col == 1 && a.t_row % 4 == 0 &&
               reinterpret_cast<uintptr_t>(zq) % 16 == 0 &&
               reinterpret_cast<uintptr_t>(zk) % 16 == 0) ? 1 : 0;
    pl->grid = (a.n_items + kBlock - 1) / kBlock;
    if (pl->grid > 0x7fffffff) return ROPE_ERR_SHAPE;
    // The lanes shape (xpos_lanes) where it applies: in place, 16-byte
    // chunks, a power-of-two number of chunks per row, table entries as
    // float4s. Head-major views take the rope_head_lanes_kernel rule on the
    // distance between heads (measured there; in between the rule leaves
    // them to the chunked shape); token-major views one token per workgroup.
    int cshift = -1;
    for (int sh = 0; sh < 11; ++sh)
      if ((1 << sh) == a.chunks) cshift = sh;
    const int64_t head_gap = d->q_in.stride_h * elem_bytes(d->dtype);
    if (!oop && a.t_vec && (int64_t)v * elem_bytes(d->dtype) == 16 && cshift >= 0) {
      a.chunks_shift = cshift;
      if (a.token_major) {
        const int64_t lanes = ((h_total << cshift) + 63) / 64 * 64;
        if (lanes <= 1024) {
          pl->lanes = 2;
          pl->block = (int)lanes;
          pl->grid = a.n_tokens;
        }
      } else if (h_total >= 8 && (head_gap <= ((int64_t)2 << 20) ||
                                  head_gap >= ((int64_t)16 << 20))) {
        const int span = head_gap <= ((int64_t)2 << 20) ? 64 : 32;
        const int hpg = (int)(h_total < (span == 64 ? 8 : 20) ? h_total : (span == 64 ? 8 : 20));
        if (a.chunks <= span) {
          int tshift = 0;
          while ((a.chunks << (tshift + 1)) <= span) ++tshift;
          a.tokens_per_block = 1 << tshift;
          a.tokens_shift = tshift;
          a.heads_per_group = hpg;
          a.n_groups = (int32_t)((h_total + hpg - 1) / hpg);
          a.n_tiles = (a.n_tokens + a.tokens_per_block - 1) / a.tokens_per_block;
          const int64_t n_wg = a.n_tiles * a.n_groups;
          if (n_wg <= 0x7fffffff) {
            pl->lanes = 1;
            pl->block = (a.chunks << tshift) * hpg;
            pl->grid = n_wg;
          }
        }
      }
    }
  } else {
    pl->vec = 0;
    pl->grid = a.n_tokens;
  }

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

// Calls f.template chunked<T, V, PAIR, U>() or f.template element<T>() for
// the plan's shape (F: the GPU launcher, or the host emulation). U: heads
// whose loads go out together, 4 when a lane walks several heads (one head
// per lane keeps the register count, and occupancy, of a single head:
// measured on MI355X, packed QKV Llama, 79 us with U = 4 against 72 us).
// False for a combination no plan produces.
template <typename T, int V, int PAIR, class F>
void dispatch_u(const XPlan& pl, F& f) {
  if (pl.a.heads_per_group > 1) f.template chunked<T, V, PAIR, 4>();
  else f.template chunked<T, V, PAIR, 1>();
}

template <typename T, int VMAX, class F>
bool dispatch_vec(const XPlan& pl, F& f) {
  const bool inter = pl.a.interleaved != 0;
  switch (pl.vec) {
    case 1:
      if (inter) return false;
      dispatch_u<T, 1, kSplitHalf>(pl, f);
      return true;
    case 2:
      if (inter) dispatch_u<T, 2, kInterleaved>(pl, f);
      else dispatch_u<T, 2, kSplitHalf>(pl, f);
      return true;
    case 4:
      if (inter) dispatch_u<T, 4, kInterleaved>(pl, f);
      else dispatch_u<T, 4, kSplitHalf>(pl, f);
      return true;
    case 8:
      if constexpr (VMAX >= 8) {
        if (inter) dispatch_u<T, 8, kInterleaved>(pl, f);
        else dispatch_u<T, 8, kSplitHalf>(pl, f);
        return true;
      }
      return false;
  }
  return false;
}

// The lanes shape: split-half V = 16 / sizeof(T), or interleaved with V / 2 a
// multiple of 4 (8 16-bit elements).
template <typename T, class F>
bool dispatch_lanes(const XPlan& pl, F& f) {
  constexpr int V = 16 / (int)sizeof(T);
  const bool idx = pl.a.pos != nullptr, tok = pl.lanes == 2;
  if (!pl.a.interleaved) {
    if (idx) tok ? f.template lanes<T, V, kSplitHalf, true, true>()
                 : f.template lanes<T, V, kSplitHalf, true, false>();
    else tok ? f.template lanes<T, V, kSplitHalf, false, true>()
             : f.template lanes<T, V, kSplitHalf, false, false>();
    return true;
  }
  if constexpr (V == 8) {
    if (idx) tok ? f.template lanes<T, V, kInterleaved, true, true>()
                 : f.template lanes<T, V, kInterleaved, true, false>();
    else tok ? f.template lanes<T, V, kInterleaved, false, true>()
             : f.template lanes<T, V, kInterleaved, false, false>();
    return true;
  }
  return false;
}

template <class F>
bool dispatch(const XPlan& pl, F& f) {
  if (pl.lanes) {
    switch (pl.dtype) {
      case ROPE_F32: return dispatch_lanes<float>(pl, f);
      case ROPE_F16: return dispatch_lanes<_Float16>(pl, f);
      case ROPE_BF16: return dispatch_lanes<__bf16>(pl, f);
    }
    return false;
  }
  if (pl.vec == 0) {
    switch (pl.dtype) {
      case ROPE_F32: f.template element<float>(); return true;
      case ROPE_F16: f.template element<_Float16>(); return true;
      case ROPE_BF16: f.template element<__bf16>(); return true;
    }
    return false;
  }
  switch (pl.dtype) {
    case ROPE_F32: return dispatch_vec<float, 4>(pl, f);
    case ROPE_F16: return dispatch_vec<_Float16, 8>(pl, f);
    case ROPE_BF16: return dispatch_vec<__bf16, 8>(pl, f);
  }
  return false;
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

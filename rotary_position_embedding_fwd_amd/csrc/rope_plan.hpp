// rope_plan.hpp -- host-side planning for librope: argument validation, the
// access width, and the grid shape. No GPU calls happen here, so the same
// plan drives the real launch (librope.hip) and the host emulation of the
// kernels used to check index arithmetic and bounds on the CPU.
//
// Every call is first put in the general form of rope_apply (strided input
// and output views, table strides, direction); the contiguous entry points
// only fill that form from their layout.
#pragma once

#include <stdint.h>

#include <cmath>

#include "librope.h"
#include "rope_kernels.hpp"

namespace rope {

struct Plan {
  Args a;
  bool token;      // grid shape: token (a few tokens per workgroup) or rows
  int vec;         // access width V (elements)
  bool aligned;    // V-element accesses are V-element aligned
  int dtype;       // rope_dtype_t
  int pairing;     // rope_pairing_t
  int64_t grid;    // workgroups
  int block;       // lanes per workgroup
  bool empty;      // nothing to do
  bool single;     // token shape: the grid covers every token, no loops
  bool oop;        // some output differs from its input
  bool pair;       // rows shape, one chunk per lane (rope_pair_lanes_kernel)
  bool head_lanes; // rows shape, one (token, head) chunk per lane (rope_head_lanes_kernel)
  bool flat;       // token shape, items over the whole call (rope_flat_kernel)
  int64_t lds_bytes;  // dynamic shared memory per workgroup

  // token shape: which rope_token_kernel instantiation runs the plan
  int token_mode() const {
    if (!single) return kTokenLoop;
    return a.tokens_per_block == 1 ? kTokenOne : kTokenPacked;
  }
};

// Angles computed from theta: the largest rotary dim (the token kernel keeps a
// token's R/2 cos/sin pairs in shared memory) and the largest angle, in
// radians, for which the kernels' argument reduction keeps |r| <= pi/4 + 1e-4.
constexpr int64_t kMaxThetaRotaryDim = 8192;
constexpr double kMaxThetaAngle = 1099511627776.0;  // 2^40

// Token shape: (head, chunk) items a workgroup aims for when tokens are small.
constexpr int64_t kTokenItems = 256;

inline int64_t elem_bytes(int32_t dtype) { return dtype == ROPE_F32 ? 4 : 2; }

inline bool apply_is_empty(const rope_apply_desc_t* d) {
  return d->batch == 0 || d->seq_len == 0 || d->rotary_dim == 0 ||
         d->n_heads_q + d->n_heads_k == 0;
}

// ------------------------------------------------------------------ views
// A view with its extents [B, H, S, D], for the overlap and width checks.
struct ViewX {
  uintptr_t p;
  int64_t sb, sh, ss;
  int64_t B, H, S, D;
};

inline ViewX view_x(const rope_view_t& v, int64_t B, int64_t H, int64_t S, int64_t D) {
  return ViewX{reinterpret_cast<uintptr_t>(v.data), v.stride_b, v.stride_h, v.stride_s,
               B, H, S, D};
}

inline bool view_empty(const ViewX& v) { return !v.B || !v.H || !v.S || !v.D; }

// Elements from the first to one past the last addressed element.
inline int64_t view_span(const ViewX& v) {
  if (view_empty(v)) return 0;
  return (v.B - 1) * v.sb + (v.H - 1) * v.sh + (v.S - 1) * v.ss + v.D;
}

// view_span in bytes, false when it does not fit in int64 (absurd strides or
// sizes would otherwise wrap the overlap checks below)
inline bool view_bytes(const ViewX& v, int64_t e, int64_t* out) {
  *out = 0;
  if (view_empty(v)) return true;
  int64_t t = 0, n = v.D;
  const int64_t ext[3] = {v.B, v.H, v.S}, st[3] = {v.sb, v.sh, v.ss};
  for (int i = 0; i < 3; ++i)
    if (__builtin_mul_overflow(ext[i] - 1, st[i], &t) || __builtin_add_overflow(n, t, &n))
      return false;
  return !__builtin_mul_overflow(n, e, out);
}

// Sufficient condition for no two (b, h, s, j) to share an element: ordered
// by stride, every dim of extent > 1 steps over everything the smaller ones
// cover. All the usual layouts ([B,H,S,D], [B,S,H,D], views into packed QKV)
// satisfy it.
inline bool view_injective(const ViewX& v) {
  if (view_empty(v)) return true;
  int64_t st[3] = {v.sb, v.sh, v.ss}, ex[3] = {v.B, v.H, v.S};
  for (int i = 0; i < 3; ++i)  // sort the three dims by stride
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i]) {
        const int64_t t0 = st[i], t1 = ex[i];
        st[i] = st[j], ex[i] = ex[j];
        st[j] = t0, ex[j] = t1;
      }
  int64_t covered = v.D;
  for (int i = 0; i < 3; ++i) {
    if (ex[i] <= 1) continue;
    if (st[i] < covered) return false;
    covered += (ex[i] - 1) * st[i];
  }
  return true;
}

inline bool same_view(const ViewX& a, const ViewX& b) {
  return a.p == b.p && a.sb == b.sb && a.sh == b.sh && a.ss == b.ss && a.B == b.B &&
         a.H == b.H && a.S == b.S && a.D == b.D;
}

// Token period of a view: the stride between consecutive tokens' cells, or 0
// when its tokens do not tile memory with one period.
inline int64_t token_period(const ViewX& v) {
  if (v.S > 1) {
    if (v.B > 1 && (v.ss <= 0 || v.sb % v.ss != 0)) return 0;
    return v.ss;
  }
  return v.B > 1 ? v.sb : 0;
}

// True when the two views cannot address a common element. Byte ranges that
// do not meet are disjoint; so are views that interleave token by token
// (packed QKV): same token period P, each view's heads inside a cell of P
// elements, and the second view's cell span falling entirely beside the
// first's.
inline bool views_disjoint(const ViewX& a, const ViewX& b, int64_t e) {
  if (view_empty(a) || view_empty(b)) return true;
  const uintptr_t a0 = a.p, a1 = a.p + (uintptr_t)(view_span(a) * e);
  const uintptr_t b0 = b.p, b1 = b.p + (uintptr_t)(view_span(b) * e);
  if (a1 <= b0 || b1 <= a0) return true;
  const int64_t P = token_period(a);
  if (P <= 0 || P != token_period(b)) return false;
  const int64_t ext_a = (a.H - 1) * a.sh + a.D, ext_b = (b.H - 1) * b.sh + b.D;
  if (ext_a > P || ext_b > P) return false;
  const int64_t delta_bytes = (int64_t)(b.p - a.p);  // two's complement wrap is fine
  if (delta_bytes % e) return false;
  int64_t r = (delta_bytes / e) % P;
  if (r < 0) r += P;
  return r >= ext_a && r + ext_b <= P;
}

// ------------------------------------------------------------ validation
// Checks that need no GPU and never dereference a device pointer.
inline rope_status_t validate_apply(const rope_apply_desc_t* d) {
  if (!d) return ROPE_ERR_NULL;
  if (d->dtype < ROPE_F32 || d->dtype > ROPE_BF16) return ROPE_ERR_DTYPE;
  if (d->pairing != ROPE_SPLIT_HALF && d->pairing != ROPE_INTERLEAVED) return ROPE_ERR_LAYOUT;
  if (d->launch < ROPE_LAUNCH_AUTO || d->launch > ROPE_LAUNCH_TOKEN) return ROPE_ERR_LAYOUT;
  if (d->direction != 1 && d->direction != -1) return ROPE_ERR_LAYOUT;
  if (d->angles != ROPE_ANGLES_TABLE && d->angles != ROPE_ANGLES_THETA) return ROPE_ERR_LAYOUT;
  const bool tables = d->angles == ROPE_ANGLES_TABLE;
  if (tables && d->table_col_stride != 1 && d->table_col_stride != 2) return ROPE_ERR_LAYOUT;
  const int64_t hk = d->n_heads_k;
  if (d->batch < 0 || d->n_heads_q < 0 || d->seq_len < 0 || d->head_dim < 0 ||
      d->rotary_dim < 0 || d->table_rows < 0 || hk < 0)
    return ROPE_ERR_SHAPE;
  if ((d->rotary_dim & 1) || d->rotary_dim > d->head_dim) return ROPE_ERR_SHAPE;
  if (hk > d->n_heads_q) return ROPE_ERR_SHAPE;
  // heads and dims index with 32-bit integers inside the kernels
  if (d->n_heads_q + hk > ((int64_t)1 << 30) || d->head_dim > ((int64_t)1 << 30))
    return ROPE_ERR_SHAPE;
  if (!tables) {
    if (!(d->theta > 0.0) || !std::isfinite(d->theta) || !(d->interpolate_factor > 0.0) ||
        !std::isfinite(d->interpolate_factor) || d->rotary_dim > kMaxThetaRotaryDim)
      return ROPE_ERR_SHAPE;
    // The largest angle must stay inside the range where the kernels' sin/cos
    // argument reduction is accurate.
    const double max_freq = d->theta >= 1.0 ? 1.0 : 1.0 / d->theta;
    const double max_pos = d->table_rows > 0 ? (double)(d->table_rows - 1) : 0.0;
    if (max_pos / d->interpolate_factor * max_freq > kMaxThetaAngle) return ROPE_ERR_SHAPE;
  }
  if (apply_is_empty(d)) return ROPE_OK;
  if (!d->pos && d->seq_len > d->table_rows) return ROPE_ERR_SHAPE;
  if (d->pos && d->pos_batch_stride < 0) return ROPE_ERR_SHAPE;
  const rope_view_t* views[4] = {&d->q_in, &d->k_in, &d->q_out, &d->k_out};
  for (const rope_view_t* v : views)
    if (v->stride_b < 0 || v->stride_h < 0 || v->stride_s < 0) return ROPE_ERR_SHAPE;
  const int64_t half = d->rotary_dim / 2;
  const int64_t t_row = d->table_row_stride ? d->table_row_stride : half;
  if (tables && (t_row < 0 || t_row < (half - 1) * d->table_col_stride + 1))
    return ROPE_ERR_SHAPE;
  if ((d->n_heads_q > 0 && !d->q_in.data) || (hk > 0 && !d->k_in.data) ||
      (tables && (!d->cos || !d->sin)))
    return ROPE_ERR_NULL;
  const int64_t e = elem_bytes(d->dtype);
  for (const rope_view_t* v : views)
    if (reinterpret_cast<uintptr_t>(v->data) % e) return ROPE_ERR_ALIGN;
  if ((tables && ((reinterpret_cast<uintptr_t>(d->cos) % 16) ||
                  (reinterpret_cast<uintptr_t>(d->sin) % 16))) ||
      (reinterpret_cast<uintptr_t>(d->pos) % 4))
    return ROPE_ERR_ALIGN;

  // Written views (an output, or the input itself in place) must not address
  // one element twice, must not overlap each other, and must not overlap any
  // input other than their own identical input.
  const int64_t B = d->batch, S = d->seq_len, D = d->head_dim;
  const ViewX qi = view_x(d->q_in, B, d->n_heads_q, S, D);
  const ViewX ki = view_x(d->k_in, B, hk, S, D);
  const ViewX qo = d->q_out.data ? view_x(d->q_out, B, d->n_heads_q, S, D) : qi;
  const ViewX ko = d->k_out.data ? view_x(d->k_out, B, hk, S, D) : ki;
  // every extent below fits in int64
  int64_t span = 0, tokens = 0;
  for (const ViewX* x : {&qi, &ki, &qo, &ko})
    if (!view_bytes(*x, e, &span)) return ROPE_ERR_SHAPE;
  if (__builtin_mul_overflow(B, S, &tokens)) return ROPE_ERR_SHAPE;
  int64_t pos_bytes = 0, table_bytes = 0;
  if (d->pos && (__builtin_mul_overflow(B - 1, d->pos_batch_stride, &pos_bytes) ||
                 __builtin_add_overflow(pos_bytes, S, &pos_bytes) ||
                 __builtin_mul_overflow(pos_bytes, (int64_t)4, &pos_bytes)))
    return ROPE_ERR_SHAPE;
  if (tables && d->table_rows > 0 &&
      (__builtin_mul_overflow(d->table_rows - 1, t_row, &table_bytes) ||
       __builtin_add_overflow(table_bytes, (half - 1) * d->table_col_stride + 1, &table_bytes) ||
       __builtin_mul_overflow(table_bytes, (int64_t)4, &table_bytes)))
    return ROPE_ERR_SHAPE;
  if (!view_injective(qo) || !view_injective(ko)) return ROPE_ERR_ALIAS;
  if (!views_disjoint(qo, ko, e)) return ROPE_ERR_ALIAS;
  if (!same_view(qo, qi) && !views_disjoint(qo, qi, e)) return ROPE_ERR_ALIAS;
  if (!same_view(ko, ki) && !views_disjoint(ko, ki, e)) return ROPE_ERR_ALIAS;
  if (!views_disjoint(qo, ki, e) || !views_disjoint(ko, qi, e)) return ROPE_ERR_ALIAS;

  // The index array and the tables are read-only for the whole launch (the
  // kernels may read the index through the scalar cache): no written view
  // may meet their byte ranges.
  auto meets_written = [&](const void* base, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base), hi = lo + (uintptr_t)bytes;
    for (const ViewX* w : {&qo, &ko}) {
      if (view_empty(*w) || bytes <= 0) continue;
      const uintptr_t w0 = w->p, w1 = w->p + (uintptr_t)(view_span(*w) * e);
      if (lo < w1 && w0 < hi) return true;
    }
    return false;
  };
  if (d->pos && meets_written(d->pos, pos_bytes)) return ROPE_ERR_ALIAS;
  if (tables && d->table_rows > 0 &&
      (meets_written(d->cos, table_bytes) || meets_written(d->sin, table_bytes)))
    return ROPE_ERR_ALIAS;
  return ROPE_OK;
}

// The contiguous entry points in the general form: strides from the layout,
// outputs in place, a [table_rows, R/2] table.
inline rope_status_t desc_to_apply(const void* q, const void* k, const rope_desc_t* d,
                                   bool with_k, int direction, rope_apply_desc_t* out) {
  if (!d) return ROPE_ERR_NULL;
  if (d->dtype < ROPE_F32 || d->dtype > ROPE_BF16) return ROPE_ERR_DTYPE;
  if (d->layout != ROPE_BHSD && d->layout != ROPE_BSHD) return ROPE_ERR_LAYOUT;
  rope_apply_desc_t a{};
  a.batch = d->batch;
  a.seq_len = d->seq_len;
  a.head_dim = d->head_dim;
  a.rotary_dim = d->rotary_dim;
  a.n_heads_q = d->n_heads_q;
  a.n_heads_k = with_k ? d->n_heads_k : 0;
  a.dtype = d->dtype;
  a.pairing = d->pairing;
  a.launch = d->launch;
  a.direction = direction;
  const int64_t S = d->seq_len, D = d->head_dim;
  const int64_t heads[2] = {d->n_heads_q, a.n_heads_k};
  rope_view_t* views[2] = {&a.q_in, &a.k_in};
  const void* data[2] = {q, with_k ? k : nullptr};
  for (int i = 0; i < 2; ++i) {
    rope_view_t& v = *views[i];
    v.data = const_cast<void*>(data[i]);
    if (d->layout == ROPE_BHSD) {  // [B, H, S, D]
      v.stride_b = heads[i] * S * D;
      v.stride_h = S * D;
      v.stride_s = D;
    } else {  // [B, S, H, D]
      v.stride_b = S * heads[i] * D;
      v.stride_s = heads[i] * D;
      v.stride_h = D;
    }
  }
  a.cos = d->cos;
  a.sin = d->sin;
  a.table_rows = d->table_rows;
  a.table_row_stride = 0;
  a.table_col_stride = 1;
  a.pos = d->pos;
  a.pos_batch_stride = d->pos_batch_stride;
  *out = a;
  return ROPE_OK;
}

inline rope_status_t validate(const void* q, const void* k, const rope_desc_t* d, bool with_k) {
  rope_apply_desc_t a;
  const rope_status_t st = desc_to_apply(q, k, d, with_k, 1, &a);
  return st != ROPE_OK ? st : validate_apply(&a);
}

// ------------------------------------------------------------------ plan
// Largest access width V (elements, a power of two, at most 16 bytes) that
// keeps every chunk access V-aligned: V must divide the span that chunks
// tile (R/2 for split-half, R for interleaved), the element offset of every
// view and every stride of a dim with more than one index.
inline int pick_vec(const rope_apply_desc_t* d) {
  const int64_t e = elem_bytes(d->dtype);
  const int64_t span = d->pairing == ROPE_SPLIT_HALF ? d->rotary_dim / 2 : d->rotary_dim;
  const int64_t heads[4] = {d->n_heads_q, d->n_heads_k, d->n_heads_q, d->n_heads_k};
  const rope_view_t* views[4] = {&d->q_in, &d->k_in, &d->q_out, &d->k_out};
  int v = (int)(16 / e);
  auto fits = [&](int w) {
    if (span % w) return false;
    for (int i = 0; i < 4; ++i) {
      const rope_view_t& x = *views[i];
      if (!x.data || heads[i] == 0) continue;
      if ((reinterpret_cast<uintptr_t>(x.data) / e) % w) return false;
      if ((d->batch > 1 && x.stride_b % w) || (heads[i] > 1 && x.stride_h % w) ||
          (d->seq_len > 1 && x.stride_s % w))
        return false;
    }
    return true;
  };
  while (v > 1 && !fits(v)) v >>= 1;
  return v;
}

inline View to_view(const rope_view_t& v) {
  return View{static_cast<char*>(v.data), v.stride_b, v.stride_h, v.stride_s};
}

// Q and K views whose heads of a token are adjacent (a token's rows form one
// contiguous stretch), whatever the token and batch strides: [B,S,H,D]
// tensors and Q/K views into a packed QKV buffer.
inline bool heads_adjacent(const rope_apply_desc_t* d) {
  const rope_view_t* views[2] = {&d->q_in, &d->k_in};
  const int64_t heads[2] = {d->n_heads_q, d->n_heads_k};
  for (int i = 0; i < 2; ++i)
    if (heads[i] > 1 && views[i]->stride_h != d->head_dim) return false;
  return true;
}

// Validate and plan one call. `cus` is the device's compute-unit count.
inline rope_status_t make_plan_apply(const rope_apply_desc_t* d, int cus, Plan* pl) {
  const rope_status_t vs = validate_apply(d);
  if (vs != ROPE_OK) return vs;
  *pl = Plan{};
  pl->empty = apply_is_empty(d);
  if (pl->empty) return ROPE_OK;

  Args& a = pl->a;
  a.q_in = to_view(d->q_in);
  a.k_in = to_view(d->k_in);
  a.q_out = d->q_out.data ? to_view(d->q_out) : a.q_in;
  a.k_out = d->k_out.data ? to_view(d->k_out) : a.k_in;
  auto same = [](const View& x, const View& y) {
    return x.base == y.base && x.sb == y.sb && x.sh == y.sh && x.ss == y.ss;
  };
  pl->oop = !same(a.q_in, a.q_out) || (d->n_heads_k > 0 && !same(a.k_in, a.k_out));
  a.cos = d->cos;
  a.sin = d->sin;
  a.half = (int32_t)(d->rotary_dim / 2);
  a.t_row = d->table_row_stride ? d->table_row_stride : a.half;
  a.t_col = (int32_t)d->table_col_stride;
  a.pos = d->pos;
  a.pos_bs = d->pos_batch_stride;
  a.table_rows = d->table_rows;
  a.batch = d->batch;
  a.seq_len = d->seq_len;
  a.n_tokens = d->batch * d->seq_len;
  a.head_dim = (int32_t)d->head_dim;
  a.n_heads_q = (int32_t)d->n_heads_q;
  a.n_heads_k = (int32_t)d->n_heads_k;
  a.sin_sign = (float)d->direction;
  a.angles = d->angles == ROPE_ANGLES_THETA ? 1 : 0;
  if (a.angles) {
    a.l2_step = -2.0 * std::log2(d->theta) / (double)d->rotary_dim;
    a.interp = d->interpolate_factor;
  }

  pl->dtype = d->dtype;
  pl->pairing = d->pairing;
  int v = pick_vec(d);
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
  // cos/sin of a chunk in vector loads: contiguous frequencies, and a row
  // stride that keeps each chunk's slice aligned to the load width
  const int np = d->pairing == ROPE_SPLIT_HALF ? v : v / 2;
  const int tw = np < 4 ? np : 4;
  a.t_vec = (a.t_col == 1 && a.t_row % tw == 0) ? 1 : 0;
  const int h_total = a.n_heads_q + a.n_heads_k;

  // Rows shape: 256 (token, chunk) items per workgroup, each lane walking a
  // group of heads. Its waves per head group:
  a.n_items = a.n_tokens * a.lanes;
  int64_t tiles = (a.n_items + kRowsBlock - 1) / kRowsBlock;
  const int64_t waves_per_group = tiles * (kRowsBlock / 64);
  const int64_t target_waves = (int64_t)cus * 8;

  // Token shape lanes per token; the kernel indexes them with 32-bit ints.
  const int64_t per_token = (int64_t)h_total * a.lanes;
  const bool token_fits = per_token <= ((int64_t)1 << 30);

  // Views whose heads of a token are adjacent in memory ([B,S,H,D], packed
  // QKV) are walked in memory order by the token shape and strided by the
  // rows shape, whose lanes step from token to token. (Measured on MI355X,
  // [4,4096,32+8,128] bf16 in place: 53-55 us as tokens, 59-85 us for every
  // rows grid tried; [4,32+8,4096,128] is the other way round, 56 vs 65 us.)
  const bool token_major = d->n_heads_q > 1 && d->q_in.stride_h < d->q_in.stride_s;
  pl->token = d->launch == ROPE_LAUNCH_TOKEN;
  if (d->launch == ROPE_LAUNCH_TOKEN && !token_fits) return ROPE_ERR_SHAPE;
  if (d->launch == ROPE_LAUNCH_AUTO) {
    // decode, token-major views, or too few tokens for the rows shape to
    // fill the chip even with one head per lane
    pl->token = token_fits && (d->seq_len == 1 || token_major ||
                               waves_per_group * h_total < target_waves);
  }

  if (pl->token) {
    // Several consecutive tokens per workgroup when a token has few items (up
    // to kTokenItems items), as long as the grid keeps 16 workgroups per CU:
    // small calls are latency-bound and gain from more, smaller workgroups.
    int64_t tpb = 1;
    if (per_token < kTokenItems) {
      tpb = kTokenItems / per_token;
      const int64_t fill = a.n_tokens / ((int64_t)cus * 16);
      if (tpb > fill) tpb = fill > 1 ? fill : 1;
    }
    a.tokens_per_block = (int32_t)tpb;
    const int64_t ipl = token_items_per_lane(d->pairing == ROPE_INTERLEAVED ? kInterleaved
                                                                            : kSplitHalf);
    const int64_t lanes_needed = (tpb * per_token + ipl - 1) / ipl;
    const int64_t want = ((lanes_needed + 63) / 64) * 64;
    pl->block = (int)(want < 1024 ? want : 1024);
    // one workgroup per token group: measured faster than a grid-stride loop
    // over a chip-sized grid at every prefill shape tried
    const int64_t blocks = (a.n_tokens + tpb - 1) / tpb;
    const int64_t max_grid = (int64_t)1 << 30;
    pl->grid = blocks < max_grid ? blocks : max_grid;
    pl->single = pl->grid == blocks && pl->block >= lanes_needed;
    if (a.angles && pl->single) pl->lds_bytes = theta_shared_bytes(tpb, a.half);
    // Flat shape for token-major calls of many tokens whose heads of a token
    // are adjacent: items numbered over the whole call token by token (each
    // token's Q heads, then its K heads), so the grid walks the rows in
    // memory order. Measured on MI355X in place, forward, on dense [B,S,H,D]
    // tensors, fwd µs (flat / token kernel):
    //   interleaved pairs: [8,2048,16+16,64] fp16 22.9 / 23.8,
    //     [4,4096,32+32,64] bf16 42.3 / 43.3, [4,4096,32+8,128] bf16
    //     52.6 / 56.5, but [2,4096,16+4,256] bf16 37.3 / 30.6: so rotated
    //     spans up to 256 bytes;
    //   split-half pairs, one 16-byte chunk per lane with the partner
    //     exchange (rope_flat_pair_kernel): [8,2048,16+16,64] fp16
    //     24.7 / 28.2 and [4,4096,32+32,64] bf16 46.7 / 54.2, where a chunk
    //     pair per lane covers half of every 128-byte line per access; with
    //     128-byte halves the token kernel's full-line accesses win
    //     ([4,4096,32+8,128] 57.4 / 52.2, [2,4096,16+4,256] 35.4 / 27.4):
    //     so spans up to 128 bytes (L = R / (2V) <= 4). The items are then
    //     both halves' chunks, twice as many.
    // Views whose heads of a token are adjacent, tokens adjacent or not (Q/K
    // in a packed QKV buffer): with the items numbered token by token, packed
    // [4,4096,32+8,128] bf16 interleaved 54.6 / 57.3 us, [8,2048,16+16,64]
    // fp16 split-half 25.2 / 27.3, [4,4096,32+32,64] bf16 split-half
    // 47.2 / 50.6.
    const int64_t span_bytes = (int64_t)d->rotary_dim * elem_bytes(d->dtype);
    const bool flat_pair = d->pairing == ROPE_SPLIT_HALF &&
                           (int64_t)v * elem_bytes(d->dtype) == 16 && a.lanes_shift >= 0 &&
                           span_bytes <= 128;
    const bool flat_inter = d->pairing == ROPE_INTERLEAVED && span_bytes <= 256;
    const int64_t flat_items = a.n_tokens * per_token * (flat_pair ? 2 : 1);
    if (d->launch == ROPE_LAUNCH_AUTO && d->seq_len > 1 && !pl->oop && !a.angles && a.t_vec &&
        (flat_inter || flat_pair) && heads_adjacent(d) &&
        pl->aligned &&
        flat_items / kFlatBlock < ((int64_t)1 << 30)) {
      pl->flat = true;
      pl->single = false;
      if (flat_pair) {
        a.lanes *= 2;
        a.lanes_shift += 1;
      }
      a.tokens_per_block = 1;
      a.n_items = flat_items;
      pl->block = kFlatBlock;
      pl->grid = (flat_items + kFlatBlock - 1) / kFlatBlock;
    }
  } else {
    // Head groups, walked in group-slow order (all tiles of group 0, then of
    // group 1, ...): on MI355X this streams HBM best when a lane walks 4 heads
    // (one unrolled batch). Each group reads the cos/sin rows of its tokens
    // again, so groups grow in steps of 4 heads until those re-reads stay
    // under 15% of the call's Q/K traffic (long sequences have big tables);
    // they shrink below 4 heads only when there are too few waves.
    const int64_t e = elem_bytes(d->dtype);
    const int64_t rows_touched =
        d->pos ? (d->table_rows < a.n_tokens ? d->table_rows : a.n_tokens) : d->seq_len;
    const double table_pass = 4.0 * (double)d->rotary_dim * (double)rows_touched;
    const double qk_bytes =
        2.0 * (double)e * (double)d->rotary_dim * (double)a.n_tokens * h_total;
    int g = 4;
    while (g < h_total && (double)((h_total + g - 1) / g) * table_pass > 0.15 * qk_bytes) g += 4;
    if (g > h_total) g = h_total;
    int64_t groups = (h_total + g - 1) / g;
    if (waves_per_group * groups < target_waves) {
      groups = (target_waves + waves_per_group - 1) / waves_per_group;
      if (groups > h_total) groups = h_total;
      g = (int)((h_total + groups - 1) / groups);
    }
    // One chunk per lane (rope_pair_lanes_kernel) where it applies:
    // split-half, in place, 16-byte chunks, L = R / (2V) a power of two
    // <= kPairLanesMax, cos/sin read from tables, and a lane walking at
    // most 4 heads (one unrolled batch). Measured on MI355X, in place:
    // Llama [4,32+8,4096,128] bf16, 4-head groups, 54.9 us against 56.4 us
    // with a chunk pair per lane; long context [1,32+8,131072,128], 8-head
    // groups, 600 us against 472 us; angles from theta, where both lanes of
    // a pair would evaluate the same sin/cos, 73.3 us against 58.3 us.
    // Lanes then count both halves' chunks: twice the items.
    // Head lanes (rope_head_lanes_kernel): split-half pairs in 16-byte
    // chunks, in place, cos/sin from [rows, R/2]-style tables, at least 8
    // heads. Each lane rotates one chunk of one (token, head) and nothing is
    // looped; the workgroup's token and head counts come from the distance
    // between consecutive heads' rows, measured on MI355X with bf16
    // [B, 32+8, S, 128] calls of 2.7 GB (fwd/bwd in place, cold):
    //   heads <= 2 MiB apart (S <= 4096): 64 lanes of consecutive tokens per
    //     head, 8 heads per workgroup. Llama [4,32+8,4096,128]: 53.0-54.3 us
    //     against 54.8-55.6 us for the one-chunk-per-lane rows kernel.
    //   heads >= 16 MiB apart (S >= 65536): 32 lanes per head, 20 heads.
    //     [1,32+8,131072,128]: 430 us against 470-479 us; [2,..,65536,..]:
    //     449 us against 587-591 us.
    //   in between (S = 16384, 32768) the rows kernels measured as fast or
    //     faster (467-471 us against 475-505 us), so they stay.
    const int64_t head_gap = d->q_in.stride_h * elem_bytes(d->dtype);
    int hl_span = 0, hl_heads = 0;
    if (head_gap <= ((int64_t)2 << 20)) {
      hl_span = 64;
      hl_heads = 8;
    } else if (head_gap >= ((int64_t)16 << 20)) {
      hl_span = 32;
      hl_heads = 20;
    }
    // Rotated spans under 256 bytes (halves under one 128-byte line) keep
    // the pair-lanes rows kernel: there a chunk pair per lane makes each
    // access of a wave cover half lines. Measured (fwd, head lanes / pair
    // lanes): [4,32+8,4096,64] bf16 35.5 / 31.8 us, [4,32+32,4096,64] bf16
    // 55.5 / 49.4, [8,16+16,2048,64] fp16 32.2 / 28.9, R = 64 of 128 bf16
    // 34.0 / 32.2, R = 32 of 64 bf16 18.7 / 17.0.
    const bool hl_wide = (int64_t)d->rotary_dim * elem_bytes(d->dtype) >= 256;
    pl->head_lanes = d->launch == ROPE_LAUNCH_AUTO && hl_span > 0 && hl_wide &&
                     d->pairing == ROPE_SPLIT_HALF && !pl->oop && pl->aligned && !a.angles &&
                     a.t_vec && (int64_t)v * elem_bytes(d->dtype) == 16 && a.lanes_shift >= 0 &&
                     a.lanes <= hl_span && h_total >= 8;
    if (pl->head_lanes) {
      int tshift = 0;
      while ((a.lanes << (tshift + 1)) <= hl_span) ++tshift;
      const int hpg = hl_heads < h_total ? hl_heads : h_total;
      a.tokens_per_block = 1 << tshift;
      a.tokens_shift = tshift;
      a.heads_per_group = hpg;
      a.n_groups = (h_total + hpg - 1) / hpg;
      a.n_tiles = (a.n_tokens + a.tokens_per_block - 1) / a.tokens_per_block;
      a.group_slow = 1;
      const int64_t n_wg = a.n_tiles * a.n_groups;
      if (n_wg > 0x7fffffff) return ROPE_ERR_SHAPE;
      pl->grid = n_wg;
      pl->block = (a.lanes << tshift) * hpg;
      return ROPE_OK;
    }
    pl->pair = d->pairing == ROPE_SPLIT_HALF && !pl->oop && pl->aligned && !a.angles &&
               (int64_t)v * elem_bytes(d->dtype) == 16 && a.lanes_shift >= 0 &&
               a.lanes <= kPairLanesMax && g <= 4;
    if (pl->pair) {
      a.lanes *= 2;
      a.lanes_shift += 1;
      a.n_items = a.n_tokens * a.lanes;
      tiles = (a.n_items + kRowsBlock - 1) / kRowsBlock;
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

inline rope_status_t make_plan(void* q, void* k, const rope_desc_t* d, bool with_k,
                               float sin_sign, int cus, Plan* pl) {
  rope_apply_desc_t a;
  const rope_status_t st = desc_to_apply(q, k, d, with_k, sin_sign < 0 ? -1 : 1, &a);
  return st != ROPE_OK ? st : make_plan_apply(&a, cus, pl);
}

// Call f.template run<T, V, PAIR, ALIGNED>() for the plan's kernel variant
// (the functor picks grid shape and in/out-of-place from the plan). The
// variants instantiated here are all the plans above can produce.
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

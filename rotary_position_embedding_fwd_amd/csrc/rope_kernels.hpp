// rope_kernels.hpp -- gfx950 device code for fused rotary position embedding.
//
// The operation is an elementwise map that moves ~4 bytes per rotated pair
// (16-bit) and does ~10 float ops on it, so it is bound by HBM bandwidth
// ("Rotary Embedding Kernel", Overview: memory-bound, measured in GB/s). The
// kernels therefore aim at three things only: whole-row 128-bit loads and
// stores, cos/sin read once per token and reused for several Q and K heads of
// that token (the reuse that head grouping buys in How Unsloth Optimizes RoPE
// Embedding Computations in Triton Kernels, Triton Kernel Architecture for
// RoPE), and an HBM access order that streams well on MI355X.
//
// Work unit. A token row of R rotated dims is cut into `lanes` chunks of V
// contiguous elements per access:
//   split-half  : chunk c covers dims [cV, cV+V) and [R/2+cV, R/2+cV+V): V pairs
//   interleaved : chunk c covers dims [cV, cV+V): V/2 adjacent pairs
// ("Rotary Embedding Kernel", Paired Element Layout). A lane owns one chunk of
// one token and holds that chunk's cos/sin in registers.
//
// Tensors are strided views [batch, head, seq, dim] with a contiguous dim
// axis, read from an input view and written to an output view; in place the
// output is the input. Out of place (OOP), the lanes also copy the dims >= R
// and the rows of skipped tokens, so the output is complete.
//
// Two grid shapes share the same per-chunk device functions:
//   rope_rows_kernel  : lanes over (token, chunk); each lane walks a group of
//                       heads (Q heads first, then K heads). For prefill.
//   rope_token_kernel : a few consecutive tokens per workgroup, lanes over
//                       (token, head, chunk). For decode (seq_len 1), views
//                       whose heads of a token are adjacent ([B,S,H,D], packed
//                       QKV) and calls too small for the rows shape.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Kernel bodies are plain functions of (block, thread) so the same code can
// also be run on the host, one workgroup and lane at a time, to check index
// arithmetic and bounds before anything reaches a GPU.
#define ROPE_HD __host__ __device__ __forceinline__

namespace rope {

enum Pairing : int { kSplitHalf = 0, kInterleaved = 1 };

ROPE_HD int imin(int x, int y) { return x < y ? x : y; }
ROPE_HD int imax(int x, int y) { return x > y ? x : y; }

// A strided 4-d view: element (b, h, s, j) at base + b*sb + h*sh + s*ss + j.
struct View {
  char* base;
  int64_t sb, sh, ss;  // element strides
};

// Everything a launch needs, passed by value as the kernel argument. Fields
// are ordered so that an in-place token-shape call (decode) reads only the
// first three 64-byte lines of the argument block, which the scalar cache
// fetches in few round trips; fields of the rows kernel and of out-of-place
// calls come last.
struct Args {
  // line 0: input views
  View q_in, k_in;           // K view unused when n_heads_k == 0
  // line 1: pointers and 64-bit sizes
  const float* cos;          // frequency i of position p at [p*t_row + i*t_col]
  const float* sin;
  const int32_t* pos;        // nullptr: p = s
  int64_t t_row;             // table row stride (floats)
  int64_t pos_bs;            // index batch stride
  int64_t table_rows;
  int64_t seq_len;
  int64_t n_tokens;          // batch * seq_len
  // line 2: 32-bit fields
  int32_t half;              // R / 2
  int32_t n_heads_q;
  int32_t n_heads_k;
  int32_t lanes;             // chunks per token row
  int32_t lanes_shift;       // log2(lanes) when lanes is a power of two, else -1
  float sin_sign;            // +1 forward, -1 backward
  int32_t t_col;             // table column stride (1 or 2)
  int32_t t_vec;             // 1: a chunk's cos/sin are contiguous and aligned
  int32_t angles;            // 0: cos/sin tables; 1: computed from theta
  int32_t tokens_per_block;  // token kernel: consecutive tokens per workgroup
  int32_t head_dim;          // D (out-of-place copies)
  int32_t heads_per_group;   // rows kernel: heads walked by one lane
  int32_t n_groups;          // rows kernel: head groups
  int32_t group_slow;        // rows kernel: workgroup ids run over tiles first
  // the rest
  int64_t n_tiles;           // rows kernel: 256-item tiles
  int64_t n_items;           // rows kernel: n_tokens * lanes
  int64_t batch;
  View q_out, k_out;         // equal to the inputs in place
  double l2_step;            // angles from theta: -2 log2(theta) / R
  double interp;             // angles from theta: positions are divided by it
  int32_t tokens_shift;      // head-lanes shape: log2(tokens_per_block)
  int32_t pad0;
};

// ------------------------------------------------------------ storage I/O
// A chunk of N elements of T is moved as one access of N * sizeof(T) bytes
// when the address allows it (ALIGNED), else element by element.

ROPE_HD float to_f32(float x) { return x; }
ROPE_HD float to_f32(_Float16 x) { return static_cast<float>(x); }
ROPE_HD float to_f32(__bf16 x) { return static_cast<float>(x); }

// float -> storage type, round to nearest-even (plain IEEE conversions; the
// f16 conversion is v_cvt_f16_f32 under the default round-to-nearest mode,
// the bf16 one is gfx950's round-to-nearest-even convert).
template <typename T> ROPE_HD T from_f32(float x) {
  return static_cast<T>(x);
}

// Q/K rows are touched exactly once per call, so their loads and stores are
// non-temporal: they stream past the caches instead of evicting the cos/sin
// rows that every head of a token re-reads. (Measured on MI355X: streaming
// hints on both the loads and the stores are worth ~15% of kernel time; on
// only one side, ~5%.) On the host the plain accesses are used.
template <typename V>
ROPE_HD V stream_load(const V* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
template <typename V>
ROPE_HD void stream_store(const V& v, V* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

template <typename T, int N, bool ALIGNED> struct Chunk {
  typedef T vec_t __attribute__((ext_vector_type(N)));
  T v[N];

  ROPE_HD void load(const T* p) {
    if constexpr (ALIGNED) {
      const vec_t x = stream_load(reinterpret_cast<const vec_t*>(p));
#pragma unroll
      for (int j = 0; j < N; ++j) v[j] = x[j];
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) v[j] = stream_load(p + j);
    }
  }
  ROPE_HD void store(T* p) const {
    if constexpr (ALIGNED) {
      vec_t x;
#pragma unroll
      for (int j = 0; j < N; ++j) x[j] = v[j];
      stream_store(x, reinterpret_cast<vec_t*>(p));
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) stream_store(v[j], p + j);
    }
  }
};

// Scalar chunks need no vector type.
template <typename T, bool ALIGNED> struct Chunk<T, 1, ALIGNED> {
  T v[1];
  ROPE_HD void load(const T* p) { v[0] = stream_load(p); }
  ROPE_HD void store(T* p) const { stream_store(v[0], p); }
};

// ------------------------------------------------------------ the rotation
// One pair, float32, each output rounded once more than the exact value:
// the product x2*s is split into its rounded value and its exact error
// (TwoProduct by FMA; Ogita, Rump and Oishi, "Accurate sum and dot product",
// SIAM J. Sci. Comput. 26(6), 2005), the other product is absorbed exactly by
// an FMA, and the error term is added back. Even under heavy cancellation the
// float32 result stays within about one float32 ulp of the exact value, so
// the 16-bit rounding that follows lands on the nearest or an adjacent value.
// sn already carries the direction: +sin forward, -sin backward.
ROPE_HD void rotate_pair(float x1, float x2, float c, float sn, float& y1, float& y2) {
  const float p1 = x2 * sn;
  const float e1 = __builtin_fmaf(x2, sn, -p1);  // x2*sn - p1, exact
  y1 = __builtin_fmaf(x1, c, -p1) - e1;          // x1*c - x2*sn
  const float p2 = x1 * sn;
  const float e2 = __builtin_fmaf(x1, sn, -p2);  // x1*sn - p2, exact
  y2 = __builtin_fmaf(x2, c, p2) + e2;           // x1*sn + x2*c
}

// Pairs per chunk.
template <int V, int PAIR> struct ChunkGeom {
  static constexpr int kPairs = PAIR == kSplitHalf ? V : V / 2;
};

// ------------------------------------------------- angles from theta
// cos and sin of the binary64 angle x, each rounded once to float32.
// Argument reduction after W. J. Cody and W. Waite (Software Manual for the
// Elementary Functions, 1980): x = k (pi/2) + r with k the integer nearest to
// x (2/pi) and pi/2 carried as two binary64 parts (hi + lo = pi/2 to within
// 1.5e-33), so that r is within ~1e-16 of its exact value for |x| < 2^40
// (the planner keeps angles below that). Then the Taylor series of sin and
// cos about 0 on |r| <= pi/4 (+ a sliver), through the r^15 and r^16 terms:
// the first terms dropped are below 5e-17. Everything before the final
// rounding is binary64, so the float32 results are the correctly rounded
// cos(x) and sin(x) except within ~1e-16 of a rounding boundary. The quadrant
// k mod 4 then swaps and negates the pair.
ROPE_HD void sincos_f32(double x, float* c_out, float* s_out) {
  constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;  // 2/pi
  constexpr double kPio2Hi = 0x1.921fb54442d18p+0;     // pi/2 rounded to binary64
  constexpr double kPio2Lo = 0x1.1a62633145c07p-54;    // pi/2 - kPio2Hi, rounded
  const double k = __builtin_rint(x * kTwoOverPi);
  double r = __builtin_fma(-k, kPio2Hi, x);
  r = __builtin_fma(-k, kPio2Lo, r);
  const double r2 = r * r;
  // sin r = r + r^3 (-1/3! + r^2/5! - r^4/7! + ... - r^12/15!)
  double ps = -1.0 / 1307674368000.0;
  ps = __builtin_fma(ps, r2, 1.0 / 6227020800.0);
  ps = __builtin_fma(ps, r2, -1.0 / 39916800.0);
  ps = __builtin_fma(ps, r2, 1.0 / 362880.0);
  ps = __builtin_fma(ps, r2, -1.0 / 5040.0);
  ps = __builtin_fma(ps, r2, 1.0 / 120.0);
  ps = __builtin_fma(ps, r2, -1.0 / 6.0);
  const double sr = __builtin_fma(r * r2, ps, r);
  // cos r = 1 + r^2 (-1/2! + r^2/4! - r^4/6! + ... + r^14/16!)
  double pc = 1.0 / 20922789888000.0;
  pc = __builtin_fma(pc, r2, -1.0 / 87178291200.0);
  pc = __builtin_fma(pc, r2, 1.0 / 479001600.0);
  pc = __builtin_fma(pc, r2, -1.0 / 3628800.0);
  pc = __builtin_fma(pc, r2, 1.0 / 40320.0);
  pc = __builtin_fma(pc, r2, -1.0 / 720.0);
  pc = __builtin_fma(pc, r2, 1.0 / 24.0);
  pc = __builtin_fma(pc, r2, -0.5);
  const double cr = __builtin_fma(r2, pc, 1.0);
  // x = k pi/2 + r: quadrant 1 gives (-sin r, cos r), 2 (-cos r, -sin r),
  // 3 (sin r, -cos r)
  const int q = (int)((int64_t)k & 3);
  const double cv = (q & 1) ? sr : cr;
  const double sv = (q & 1) ? cr : sr;
  *c_out = (float)((q == 1 || q == 2) ? -cv : cv);
  *s_out = (float)((q & 2) ? -sv : sv);
}

// The angle of frequency i at position p: (p / interpolate_factor) * theta^(-2i/R),
// the power formed as exp2(i * (-2 log2(theta) / R)), all in binary64. The
// frequency does not depend on p, so callers can form it before the position
// arrives; a factor of 1 skips the division (whose result would be p).
ROPE_HD double theta_freq(const Args& a, int i) { return exp2((double)i * a.l2_step); }
ROPE_HD double theta_pos(const Args& a, int64_t p) {
  return a.interp == 1.0 ? (double)p : (double)p / a.interp;
}
ROPE_HD double theta_angle(const Args& a, int64_t p, int i) {
  return theta_pos(a, p) * theta_freq(a, i);
}

// Where a chunk's cos/sin come from.
enum TrigSource : int {
  kTrigVec = 0,     // [rows, R/2]-style table, NP contiguous floats per chunk
  kTrigScalar = 1,  // any other table layout, one value at a time
  kTrigTheta = 2,   // computed from theta by this lane
};

// cos/sin of one chunk: frequencies first .. first+NP-1 at position p. With a
// [rows, R/2] (or halves-duplicated [rows, R]) table these are NP contiguous
// floats, aligned to min(16, 4*NP) bytes (the tables are 16-byte aligned and
// the plan checks that the row stride keeps them so), and move in vector
// loads (kTrigVec); a repeat-interleaved table is read one value at a time.
// The source is chosen once at the top of each kernel, so each copy of the
// body is straight-line code whose loads the compiler can wait for one by one.
template <int V, int PAIR> struct Trig {
  static constexpr int NP = ChunkGeom<V, PAIR>::kPairs;
  static constexpr int W = NP < 4 ? NP : 4;  // floats per vector load
  typedef float vec_t __attribute__((ext_vector_type(W)));
  float c[NP], s[NP];
  float sign;  // +1 forward, -1 backward; applied in the rotation, so that no
               // arithmetic waits on the loads here

  template <int SRC>
  ROPE_HD void load(const Args& a, int64_t p, int first) {
    sign = a.sin_sign;
    if constexpr (SRC == kTrigTheta) {
#pragma unroll
      for (int j = 0; j < NP; ++j) sincos_f32(theta_angle(a, p, first + j), &c[j], &s[j]);
      return;
    } else {
      const float* cr = a.cos + p * a.t_row;
      const float* sr = a.sin + p * a.t_row;
      if constexpr (SRC == kTrigVec) {
#pragma unroll
        for (int j = 0; j < NP; j += W) {
          const vec_t cv = *reinterpret_cast<const vec_t*>(cr + first + j);
          const vec_t sv = *reinterpret_cast<const vec_t*>(sr + first + j);
#pragma unroll
          for (int w = 0; w < W; ++w) {
            c[j + w] = cv[w];
            s[j + w] = sv[w];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          c[j] = cr[(int64_t)(first + j) * a.t_col];
          s[j] = sr[(int64_t)(first + j) * a.t_col];
        }
      }
    }
  }

  // From the workgroup's shared cos/sin: (cos, sin) pairs of one token's
  // frequencies, starting at float index 2 * first.
  ROPE_HD void from_shared(const Args& a, const float* lds, int first) {
    sign = a.sin_sign;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      c[j] = lds[2 * (first + j)];
      s[j] = lds[2 * (first + j) + 1];
    }
  }
};

// One chunk of a row: load from the input row, rotate, store to the output row.
//   c : chunk index; half = R/2
template <typename T, int V, int PAIR, bool ALIGNED> struct RowChunk {
  static constexpr int NP = ChunkGeom<V, PAIR>::kPairs;
  Chunk<T, V, ALIGNED> a;  // split: first half; interleaved: the chunk
  Chunk<T, V, ALIGNED> b;  // split: second half; interleaved: unused

  ROPE_HD void load(const T* row, int c, int half) {
    if constexpr (PAIR == kSplitHalf) {
      a.load(row + c * V);
      b.load(row + half + c * V);
    } else {
      a.load(row + c * V);
    }
  }

  ROPE_HD void rotate(const Trig<V, PAIR>& t) {
    if constexpr (PAIR == kSplitHalf) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        float y1, y2;
        rotate_pair(to_f32(a.v[j]), to_f32(b.v[j]), t.c[j], t.sign * t.s[j], y1, y2);
        a.v[j] = from_f32<T>(y1);
        b.v[j] = from_f32<T>(y2);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        float y1, y2;
        rotate_pair(to_f32(a.v[2 * j]), to_f32(a.v[2 * j + 1]), t.c[j], t.sign * t.s[j], y1,
                    y2);
        a.v[2 * j] = from_f32<T>(y1);
        a.v[2 * j + 1] = from_f32<T>(y2);
      }
    }
  }

  ROPE_HD void store(T* row, int c, int half) const {
    if constexpr (PAIR == kSplitHalf) {
      a.store(row + c * V);
      b.store(row + half + c * V);
    } else {
      a.store(row + c * V);
    }
  }
};

// Out of place only: copy dims [from, to) of a row, lane c of `lanes` taking
// V-element chunks c, c+lanes, ... and lane 0 the elements past the last
// whole chunk (only when V does not divide the span).
template <typename T, int V, bool ALIGNED>
ROPE_HD void copy_span(const T* in, T* out, int from, int to, int c, int lanes) {
  const int n = (to - from) / V;
  for (int k = c; k < n; k += lanes) {
    Chunk<T, V, ALIGNED> x;
    x.load(in + from + k * V);
    x.store(out + from + k * V);
  }
  if (c == 0)
    for (int j = from + n * V; j < to; ++j) stream_store(stream_load(in + j), out + j);
}

template <typename T>
ROPE_HD T* view_row(const View& v, int64_t h, int64_t b, int64_t s) {
  return reinterpret_cast<T*>(v.base) + (b * v.sb + h * v.sh + s * v.ss);
}

// Position of token (b, s), or -1 when the token passes through. The index
// array does not change during a launch (no written view overlaps it), so on
// the device it is read through the constant address space: where (b, s) is
// the same for the whole wave, that is one scalar load, whose wait does not
// hold up the row loads already in flight.
ROPE_HD int64_t token_pos(const Args& a, int64_t b, int64_t s) {
  if (!a.pos) return s < a.table_rows ? s : -1;
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const const_i32* idx = reinterpret_cast<const const_i32*>(reinterpret_cast<uintptr_t>(a.pos));
  const int64_t p = idx[b * a.pos_bs + s];
#else
  const int64_t p = a.pos[b * a.pos_bs + s];
#endif
  return (p < 0 || p >= a.table_rows) ? -1 : p;
}

// ------------------------------------------------------ rows (prefill) shape
// Rotate one lane's chunk in heads [h_lo, h_hi) of one tensor, whose rows for
// this token start at `in` / `out` and are `sh_in` / `sh_out` elements apart.
// U heads are loaded before any is rotated so U row loads are in flight.
template <typename T, int V, int PAIR, bool ALIGNED, int U, bool OOP>
ROPE_HD void rotate_heads(const Args& a, const T* in, int64_t sh_in, T* out, int64_t sh_out,
                          int h_lo, int h_hi, int c, const Trig<V, PAIR>& t) {
  for (int h0 = h_lo; h0 < h_hi; h0 += U) {
    RowChunk<T, V, PAIR, ALIGNED> r[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (h0 + u < h_hi) r[u].load(in + (int64_t)(h0 + u) * sh_in, c, a.half);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (h0 + u < h_hi) {
        r[u].rotate(t);
        r[u].store(out + (int64_t)(h0 + u) * sh_out, c, a.half);
      }
    }
    if constexpr (OOP) {
      for (int u = 0; u < U && h0 + u < h_hi; ++u)
        copy_span<T, V, ALIGNED>(in + (int64_t)(h0 + u) * sh_in,
                                 out + (int64_t)(h0 + u) * sh_out, 2 * a.half, a.head_dim,
                                 c, a.lanes);
    }
  }
}

// Out of place, a skipped token's rows are copied whole.
template <typename T, int V, bool ALIGNED>
ROPE_HD void copy_heads(const Args& a, const T* in, int64_t sh_in, T* out, int64_t sh_out,
                        int h_lo, int h_hi, int c) {
  for (int h = h_lo; h < h_hi; ++h)
    copy_span<T, V, ALIGNED>(in + (int64_t)h * sh_in, out + (int64_t)h * sh_out, 0,
                             a.head_dim, c, a.lanes);
}

// Tokens are numbered in memory order (n = b * seq_len + s), so in the [B,H,S,D]
// layout the 4 waves of a workgroup cover 32 consecutive rows (8 KiB at
// D=128, bf16) of each head they visit. Workgroup ids run over (tile, head
// group), in either order (group_slow: all tiles of group 0 first), and are
// left in the hardware's round-robin order over the XCDs: renumbering them so
// that each XCD owns one contiguous range of tiles was measured ~10% slower.
constexpr int kRowsBlock = 256;

template <typename T, int V, int PAIR, bool ALIGNED, int U, bool OOP, int SRC>
ROPE_HD void rows_body(const Args& a, int64_t block, int thread) {
  int64_t tile;
  int group;
  if (a.group_slow) {  // all tiles of head group 0, then of group 1, ...
    group = (int)(block / a.n_tiles);
    tile = block - (int64_t)group * a.n_tiles;
  } else {  // all head groups of tile 0, then of tile 1, ...
    tile = block / a.n_groups;
    group = (int)(block - tile * a.n_groups);
  }
  const int64_t item = tile * kRowsBlock + thread;
  if (item >= a.n_items) return;
  const int64_t n = item / a.lanes;
  const int c = (int)(item - n * a.lanes);
  const int64_t b = n / a.seq_len;
  const int64_t s = n - b * a.seq_len;

  const int h_begin = group * a.heads_per_group;
  const int h_end = imin(h_begin + a.heads_per_group, a.n_heads_q + a.n_heads_k);
  const int q_lo = h_begin, q_hi = imin(h_end, a.n_heads_q);
  const int k_lo = imax(h_begin - a.n_heads_q, 0), k_hi = h_end - a.n_heads_q;
  const T* qi = view_row<T>(a.q_in, 0, b, s);
  const T* ki = view_row<T>(a.k_in, 0, b, s);
  // in place the output views are the input views
  T* qo = OOP ? view_row<T>(a.q_out, 0, b, s) : const_cast<T*>(qi);
  T* ko = OOP ? view_row<T>(a.k_out, 0, b, s) : const_cast<T*>(ki);

  const int64_t p = token_pos(a, b, s);
  if (p < 0) {  // skipped token: in place nothing is read or written
    if constexpr (OOP) {
      if (q_lo < q_hi)
        copy_heads<T, V, ALIGNED>(a, qi, a.q_in.sh, qo, a.q_out.sh, q_lo, q_hi, c);
      if (k_lo < k_hi)
        copy_heads<T, V, ALIGNED>(a, ki, a.k_in.sh, ko, a.k_out.sh, k_lo, k_hi, c);
    }
    return;
  }

  Trig<V, PAIR> t;
  t.template load<SRC>(a, p, c * ChunkGeom<V, PAIR>::kPairs);
  if (q_lo < q_hi)
    rotate_heads<T, V, PAIR, ALIGNED, U, OOP>(a, qi, a.q_in.sh, qo, a.q_out.sh, q_lo, q_hi, c,
                                              t);
  if (k_lo < k_hi)
    rotate_heads<T, V, PAIR, ALIGNED, U, OOP>(a, ki, a.k_in.sh, ko, a.k_out.sh, k_lo, k_hi, c,
                                              t);
}

// The kernel entry, also run on the host by the emulator.
template <typename T, int V, int PAIR, bool ALIGNED, int U, bool OOP>
ROPE_HD void rows_entry(const Args& a, int64_t block, int thread) {
  if (a.angles)
    rows_body<T, V, PAIR, ALIGNED, U, OOP, kTrigTheta>(a, block, thread);
  else if (a.t_vec)
    rows_body<T, V, PAIR, ALIGNED, U, OOP, kTrigVec>(a, block, thread);
  else
    rows_body<T, V, PAIR, ALIGNED, U, OOP, kTrigScalar>(a, block, thread);
}

template <typename T, int V, int PAIR, bool ALIGNED, int U, bool OOP>
__global__ void __launch_bounds__(kRowsBlock) rope_rows_kernel(Args a) {
  rows_entry<T, V, PAIR, ALIGNED, U, OOP>(a, blockIdx.x, threadIdx.x);
}

// -------------------------------------- rows shape, one chunk per lane
// Split-half pairs, in place, 16-byte aligned chunks, and L = R / (2 V) a
// power of two no larger than kPairLanesMax. The 2L lanes of a token hold
// its 2L chunks, lane c2 the chunk c2 % L of half c2 / L, so each row access
// of a wave covers the whole rotated span of 64 / (2L) tokens. A lane takes
// the chunk of its pair partner (lane c2 ^ L: the same chunk of the other
// half) from that lane's registers and writes only its own chunk:
//   lower half  y = x1 c - x2 s  = own c + other (-s)
//   upper half  y = x2 c + x1 s  = own c + other (+s)
// in the steps of rotate_pair, which it reproduces bit for bit (negating s
// is exact and commutes with every rounding there).
constexpr int kPairLanesMax = 16;

ROPE_HD float rotate_own(float own, float other, float c, float s_eff) {
  const float p = other * s_eff;
  const float e = __builtin_fmaf(other, s_eff, -p);  // other*s_eff - p, exact
  return __builtin_fmaf(own, c, p) + e;
}

template <typename T, int V, int U, int SRC> struct PairLaneWork {
  using C = Chunk<T, V, true>;
  Trig<V, kSplitHalf> t;
  T* row[2];         // Q and K rows of this token at head 0, at this lane's chunk
  int64_t sh[2];     // head strides
  int lo[2], hi[2];  // head ranges of this workgroup's group, per tensor
  bool upper;        // this lane holds the second half's chunk
  C own[U], other[U];

  // false: this lane has nothing to do (past the last token, or a skipped
  // token; the partner lane then has nothing to do either)
  ROPE_HD bool begin(const Args& a, int64_t block, int thread) {
    int64_t tile;
    int group;
    if (a.group_slow) {
      group = (int)(block / a.n_tiles);
      tile = block - (int64_t)group * a.n_tiles;
    } else {
      tile = block / a.n_groups;
      group = (int)(block - tile * a.n_groups);
    }
    const int64_t item = tile * kRowsBlock + thread;
    if (item >= a.n_items) return false;
    const int64_t n = item >> a.lanes_shift;
    const int c2 = (int)(item & (a.lanes - 1));
    const int L = a.lanes >> 1;
    upper = (c2 & L) != 0;
    const int c = c2 & (L - 1);
    const int64_t b = n / a.seq_len;
    const int64_t s = n - b * a.seq_len;
    const int64_t p = token_pos(a, b, s);
    if (p < 0) return false;
    const int h_begin = group * a.heads_per_group;
    const int h_end = imin(h_begin + a.heads_per_group, a.n_heads_q + a.n_heads_k);
    lo[0] = h_begin;
    hi[0] = imin(h_end, a.n_heads_q);
    lo[1] = imax(h_begin - a.n_heads_q, 0);
    hi[1] = h_end - a.n_heads_q;
    const int off = (upper ? a.half : 0) + c * V;
    row[0] = view_row<T>(a.q_in, 0, b, s) + off;
    row[1] = view_row<T>(a.k_in, 0, b, s) + off;
    sh[0] = a.q_in.sh;
    sh[1] = a.k_in.sh;
    t.template load<SRC>(a, p, c * V);
    return true;
  }
  ROPE_HD void load(int x, int h0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (h0 + u < hi[x]) own[u].load(row[x] + (int64_t)(h0 + u) * sh[x]);
  }
  // rotate the own chunks with the partner chunks in other[], store
  ROPE_HD void finish(int x, int h0) {
    const float sg = upper ? t.sign : -t.sign;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (h0 + u < hi[x]) {
#pragma unroll
        for (int j = 0; j < V; ++j)
          own[u].v[j] = from_f32<T>(
              rotate_own(to_f32(own[u].v[j]), to_f32(other[u].v[j]), t.c[j], sg * t.s[j]));
        own[u].store(row[x] + (int64_t)(h0 + u) * sh[x]);
      }
    }
  }
};

#if defined(__HIP_DEVICE_COMPILE__)
// The 32-bit word w of lane (this lane ^ L), L a power of two <= 16: a DPP
// row rotation by 8 for L = 8 (within each row of 16 lanes, rotating by 8 is
// xor 8), the LDS crossbar's swizzle (xor within 32 lanes) otherwise.
__device__ __forceinline__ uint32_t partner_word(uint32_t w, int L) {
  const int x = (int)w;
  switch (L) {
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x128, 0xf, 0xf, false);
    case 1: return (uint32_t)__builtin_amdgcn_ds_swizzle(x, (1 << 10) | 0x1f);
    case 2: return (uint32_t)__builtin_amdgcn_ds_swizzle(x, (2 << 10) | 0x1f);
    case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle(x, (4 << 10) | 0x1f);
    default: return (uint32_t)__builtin_amdgcn_ds_swizzle(x, (16 << 10) | 0x1f);
  }
}

template <typename T, int V>
__device__ __forceinline__ void partner_chunk(const Chunk<T, V, true>& own,
                                              Chunk<T, V, true>& other, int L) {
  static_assert(V * sizeof(T) == 16, "pair lanes move 16-byte chunks");
  uint32_t w[4];
  __builtin_memcpy(w, own.v, 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = partner_word(w[i], L);
  __builtin_memcpy(other.v, w, 16);
}

template <typename T, int V, int U, int SRC>
__device__ __forceinline__ void pair_lanes_body(const Args& a) {
  PairLaneWork<T, V, U, SRC> w;
  if (!w.begin(a, blockIdx.x, threadIdx.x)) return;
  const int L = a.lanes >> 1;
#pragma unroll
  for (int x = 0; x < 2; ++x)
    for (int h0 = w.lo[x]; h0 < w.hi[x]; h0 += U) {
      w.load(x, h0);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (h0 + u < w.hi[x]) partner_chunk<T, V>(w.own[u], w.other[u], L);
      w.finish(x, h0);
    }
}
#endif

template <typename T, int V, int U>
__global__ void __launch_bounds__(kRowsBlock) rope_pair_lanes_kernel(Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (a.angles)
    pair_lanes_body<T, V, U, kTrigTheta>(a);
  else if (a.t_vec)
    pair_lanes_body<T, V, U, kTrigVec>(a);
  else
    pair_lanes_body<T, V, U, kTrigScalar>(a);
#endif
}

// One lane's chunk c of the row of token (b, s) at `in`, rotated into `out`.
// The row load and the cos/sin loads are issued back to back. IDX (whether
// the call has an index tensor) is a compile-time choice, made by the host
// per launch: where the two cases shared one body, the compiler joined them
// after the loads and made the cos/sin loads wait for the row load.
//   IDX false: positions are the sequence indices, all inside the table (the
//     host rejects seq_len > table_rows without an index), so nothing is
//     skipped and nothing branches.
//   IDX true: a skipped token (position out of the table) asks for row 0 of
//     the table like the others and only its store is dropped (out of place
//     its row is copied); with no table rows at all every token is skipped
//     and no table read is issued.
template <typename T, int V, int PAIR, bool ALIGNED, bool OOP, int SRC, bool IDX>
ROPE_HD void rotate_one_chunk(const Args& a, const T* in, T* out, int64_t b, int64_t s, int c) {
  RowChunk<T, V, PAIR, ALIGNED> r;
  r.load(in, c, a.half);
  Trig<V, PAIR> t;
  if constexpr (!IDX) {
    t.template load<SRC>(a, s, c * ChunkGeom<V, PAIR>::kPairs);
  } else {
    const int64_t p = token_pos(a, b, s);
    if (SRC != kTrigTheta && a.table_rows == 0) {  // uniform: nothing to rotate
      if constexpr (OOP) copy_span<T, V, ALIGNED>(in, out, 0, a.head_dim, c, a.lanes);
      return;
    }
    t.template load<SRC>(a, p < 0 ? 0 : p, c * ChunkGeom<V, PAIR>::kPairs);
    if (p < 0) {  // skipped token: in place nothing is written
      if constexpr (OOP) copy_span<T, V, ALIGNED>(in, out, 0, a.head_dim, c, a.lanes);
      return;
    }
  }
  r.rotate(t);
  r.store(out, c, a.half);
  if constexpr (OOP) copy_span<T, V, ALIGNED>(in, out, 2 * a.half, a.head_dim, c, a.lanes);
}

// ------------------------------------------------------- head-lanes shape
// One chunk of one (token, head) per lane and nothing looped: a workgroup
// holds tokens_per_block consecutive tokens x `lanes` chunks x heads_per_group
// heads of one head group, lanes numbered chunk fastest, then token, then
// head. A wave therefore covers whole rotated spans of consecutive tokens of
// one head (or of two), every lane issues its row loads and its cos/sin loads
// at once, and the heads of the group ask for the same cos/sin rows, which
// the first wave brings into the compute unit's cache for the others.
// Workgroup ids run over all token tiles of head group 0, then group 1, ...
// Chosen for [B,H,S,D] views whose rows are split-half pairs in 16-byte
// chunks; the planner fixes the workgroup's token and head counts from the
// distance between heads.
template <typename T, int V, int PAIR, bool ALIGNED, bool OOP, int SRC, bool IDX>
ROPE_HD void head_lanes_body(const Args& a, int64_t block, int thread) {
  const int c = thread & (a.lanes - 1);
  const int rest = thread >> a.lanes_shift;
  const int tl = rest & (a.tokens_per_block - 1);
  const int hl = rest >> a.tokens_shift;
  const int64_t group = block / a.n_tiles;
  const int64_t tile = block - group * a.n_tiles;
  const int64_t n = (tile << a.tokens_shift) + tl;
  const int h = (int)group * a.heads_per_group + hl;
  if (n >= a.n_tokens || hl >= a.heads_per_group || h >= a.n_heads_q + a.n_heads_k) return;
  const int64_t b = n / a.seq_len;
  const int64_t s = n - b * a.seq_len;
  const bool is_q = h < a.n_heads_q;
  const int hh = is_q ? h : h - a.n_heads_q;
  const T* in = view_row<T>(is_q ? a.q_in : a.k_in, hh, b, s);
  T* out = OOP ? view_row<T>(is_q ? a.q_out : a.k_out, hh, b, s) : const_cast<T*>(in);
  rotate_one_chunk<T, V, PAIR, ALIGNED, OOP, SRC, IDX>(a, in, out, b, s, c);
}

// Every (source, index) form, chosen at run time: for the host emulation.
template <typename T, int V, int PAIR, bool ALIGNED, bool OOP>
ROPE_HD void head_lanes_entry(const Args& a, int64_t block, int thread) {
  if (a.angles)
    head_lanes_body<T, V, PAIR, ALIGNED, OOP, kTrigTheta, true>(a, block, thread);
  else if (!a.t_vec)
    head_lanes_body<T, V, PAIR, ALIGNED, OOP, kTrigScalar, true>(a, block, thread);
  else if (a.pos)
    head_lanes_body<T, V, PAIR, ALIGNED, OOP, kTrigVec, true>(a, block, thread);
  else
    head_lanes_body<T, V, PAIR, ALIGNED, OOP, kTrigVec, false>(a, block, thread);
}

// The planner gives this shape [rows, R/2]-style tables only (kTrigVec).
template <typename T, int V, int PAIR, bool ALIGNED, bool OOP, bool IDX>
__global__ void __launch_bounds__(1024) rope_head_lanes_kernel(Args a) {
  head_lanes_body<T, V, PAIR, ALIGNED, OOP, kTrigVec, IDX>(a, blockIdx.x, threadIdx.x);
}

// ------------------------------------------------------------- flat shape
// One (token, head, chunk) item per lane, items numbered over the whole call
// token by token, each token's Q heads then its K heads, chunk fastest. For
// views whose heads of a token are adjacent ([B,S,H,D] tensors, Q and K in a
// packed QKV buffer) consecutive lanes and consecutive workgroups then walk
// the rows in memory order, token after token, like a plain stream (in a
// packed buffer skipping only each token's V). Small workgroups (kFlatBlock
// lanes) measured best on MI355X. (Numbering all of Q before all of K was
// measured too: the same on [B,S,H,D] tensors, but on packed QKV the K pass
// then touches 2 of every 12 KiB: 57.3 us against 54.6 us at [4, 4096,
// 32+8, 128] bf16 with interleaved pairs, where the token kernel takes 57.3.)
constexpr int kFlatBlock = 64;

template <typename T, int V, int PAIR, bool ALIGNED, bool OOP, int SRC, bool IDX>
ROPE_HD void flat_body(const Args& a, int64_t block, int thread) {
  const int64_t g = block * kFlatBlock + thread;
  if (g >= a.n_items) return;
  const int heads_all = a.n_heads_q + a.n_heads_k;
  int64_t row;
  int c;
  if (a.lanes_shift >= 0) {
    row = g >> a.lanes_shift;
    c = (int)(g & (a.lanes - 1));
  } else {
    row = g / a.lanes;
    c = (int)(g - row * a.lanes);
  }
  const int64_t n = row / heads_all;
  const int hh = (int)(row - n * heads_all);
  const bool is_q = hh < a.n_heads_q;
  const int h = is_q ? hh : hh - a.n_heads_q;
  const int64_t b = n / a.seq_len;
  const int64_t s = n - b * a.seq_len;
  const T* in = view_row<T>(is_q ? a.q_in : a.k_in, h, b, s);
  T* out = OOP ? view_row<T>(is_q ? a.q_out : a.k_out, h, b, s) : const_cast<T*>(in);
  rotate_one_chunk<T, V, PAIR, ALIGNED, OOP, SRC, IDX>(a, in, out, b, s, c);
}

template <typename T, int V, int PAIR, bool ALIGNED, bool OOP>
ROPE_HD void flat_entry(const Args& a, int64_t block, int thread) {
  if (a.angles)
    flat_body<T, V, PAIR, ALIGNED, OOP, kTrigTheta, true>(a, block, thread);
  else if (!a.t_vec)
    flat_body<T, V, PAIR, ALIGNED, OOP, kTrigScalar, true>(a, block, thread);
  else if (a.pos)
    flat_body<T, V, PAIR, ALIGNED, OOP, kTrigVec, true>(a, block, thread);
  else
    flat_body<T, V, PAIR, ALIGNED, OOP, kTrigVec, false>(a, block, thread);
}

template <typename T, int V, int PAIR, bool ALIGNED, bool OOP, bool IDX>
__global__ void __launch_bounds__(kFlatBlock) rope_flat_kernel(Args a) {
  flat_body<T, V, PAIR, ALIGNED, OOP, kTrigVec, IDX>(a, blockIdx.x, threadIdx.x);
}

// Flat shape with split-half pairs: one 16-byte chunk per lane. The 2L
// chunks of a row's rotated span (L = R / (2 V), a power of two <= 16) sit on
// 2L consecutive lanes, lane c2 holding chunk c2 % L of half c2 / L, so every
// row access of a wave covers whole consecutive spans, as a plain stream's
// would; with a chunk pair per lane instead, each access of a wave covers one
// half of every span (64 bytes of each 128-byte line at R = 64, 16-bit). The
// pair partner's chunk (lane c2 ^ L, the same chunk of the other half) comes
// from that lane's registers, and each lane writes only its own chunk, in the
// steps of the pair-lanes rows kernel (rotate_own), which give rotate_pair's
// bits. Rows start at multiples of 2L in the item numbering and 2L divides
// the 64-lane workgroup, so both lanes of a pair are in one wave and share
// every skip decision. begin() loads; the caller exchanges; finish() rotates
// and stores.
template <typename T, int V, int SRC, bool IDX> struct FlatPairWork {
  using C = Chunk<T, V, true>;
  Trig<V, kSplitHalf> t;
  T* row;
  bool upper, store;
  C own, other;

  // false: no item (past the end of the call)
  ROPE_HD bool begin(const Args& a, int64_t block, int thread) {
    const int64_t g = block * kFlatBlock + thread;
    if (g >= a.n_items) return false;
    const int heads_all = a.n_heads_q + a.n_heads_k;
    const int64_t r = g >> a.lanes_shift;
    const int c2 = (int)(g & (a.lanes - 1));
    const int L = a.lanes >> 1;
    upper = (c2 & L) != 0;
    const int c = c2 & (L - 1);
    const int64_t n = r / heads_all;
    const int hh = (int)(r - n * heads_all);
    const bool is_q = hh < a.n_heads_q;
    const int h = is_q ? hh : hh - a.n_heads_q;
    const int64_t b = n / a.seq_len;
    const int64_t s = n - b * a.seq_len;
    row = const_cast<T*>(view_row<T>(is_q ? a.q_in : a.k_in, h, b, s)) + (upper ? a.half : 0) +
          c * V;
    own.load(row);
    if constexpr (!IDX) {
      store = true;
      t.template load<SRC>(a, s, c * V);
    } else {
      const int64_t p = token_pos(a, b, s);
      store = p >= 0;
      // with no table rows every token is skipped and no table read is issued
      if (SRC == kTrigTheta || a.table_rows > 0) t.template load<SRC>(a, p < 0 ? 0 : p, c * V);
    }
    return true;
  }
  ROPE_HD void finish() {
    if (!store) return;  // a skipped token: nothing is written
    const float sg = upper ? t.sign : -t.sign;
#pragma unroll
    for (int j = 0; j < V; ++j)
      own.v[j] = from_f32<T>(rotate_own(to_f32(own.v[j]), to_f32(other.v[j]), t.c[j], sg * t.s[j]));
    own.store(row);
  }
};

template <typename T, int V, bool IDX>
__global__ void __launch_bounds__(kFlatBlock) rope_flat_pair_kernel(Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  FlatPairWork<T, V, kTrigVec, IDX> w;
  if (!w.begin(a, blockIdx.x, threadIdx.x)) return;
  partner_chunk<T, V>(w.own, w.other, a.lanes >> 1);
  w.finish();
#endif
}

// ------------------------------------------------------------- token shape
// Lanes cover (head, chunk) items of a token. Each lane's head rows are
// requested before the position, so the row loads overlap the dependent
// index -> cos/sin chain.
ROPE_HD void split_item(const Args& a, int it, int* h, int* c) {
  if (a.lanes_shift >= 0) {
    *h = it >> a.lanes_shift;
    *c = it & ((1 << a.lanes_shift) - 1);
  } else {
    *h = it / a.lanes;
    *c = it - *h * a.lanes;
  }
}

// Items per lane in the single-pass token kernel: enough that a lane keeps two
// 16-byte row accesses in flight. A split-half chunk is already two accesses
// (one per half); an interleaved chunk is one, so its lanes take two items.
// (Measured on MI355X with interleaved pairs, [B,S,H,D] bf16: 67.7 -> 54.5 us
// at [4,4096,32+8,128], 34.4 -> 28.7 us at [2,4096,16+4,256]; a second
// split-half item per lane was 3-6 % slower.)
constexpr int token_items_per_lane(int pairing) { return pairing == kInterleaved ? 2 : 1; }

// K items of the token shape, run together, as one lane's state: begin()
// issues all row loads; positions() reads the tokens' positions; then either
// finish<SRC>() loads or computes the cos/sin and rotates and stores, or, for
// angles computed once per workgroup into shared memory, finish_shared()
// reads them there. Item k is (head, chunk) item it[k] of token n[k] (local
// token tl[k] of the workgroup) and is stored only if live[k]; a lane whose
// item 0 is not live has nothing to do. A dead item k > 0 loads item 0's row
// and cos/sin instead of branching around its loads, so every load of the
// lane is issued in one straight run. SAME: every item is of token n[0] (one
// token per workgroup), so the token's position is read once.
template <typename T, int V, int PAIR, bool ALIGNED, bool OOP, int K, bool SAME>
struct TokenWork {
  static constexpr int NP = ChunkGeom<V, PAIR>::kPairs;
  const T* in[K];
  T* out[K];
  int c[K], tl[K];
  int64_t b[K], s[K], p[K];
  bool live[K];
  RowChunk<T, V, PAIR, ALIGNED> r[K];

  ROPE_HD bool begin(const Args& a, const int64_t* n_in, const int* it_in, const int* tl_in,
                     const bool* live_in) {
    if (!live_in[0]) return false;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      live[k] = live_in[k];
      const bool own = k == 0 || live[k];
      const int64_t n = own ? n_in[k] : n_in[0];
      const int it = own ? it_in[k] : it_in[0];
      tl[k] = own ? tl_in[k] : tl_in[0];
      if (SAME && k > 0) {
        b[k] = b[0];
        s[k] = s[0];
      } else {
        b[k] = a.seq_len == 1 ? n : n / a.seq_len;  // decode: no division
        s[k] = n - b[k] * a.seq_len;
      }
      int h;
      split_item(a, it, &h, &c[k]);
      const bool is_q = h < a.n_heads_q;
      const int hh = is_q ? h : h - a.n_heads_q;
      in[k] = view_row<T>(is_q ? a.q_in : a.k_in, hh, b[k], s[k]);
      // in place the output view is the input view
      out[k] = OOP ? view_row<T>(is_q ? a.q_out : a.k_out, hh, b[k], s[k]) : const_cast<T*>(in[k]);
      r[k].load(in[k], c[k], a.half);
    }
    return true;
  }

  ROPE_HD void positions(const Args& a) {
#pragma unroll
    for (int k = 0; k < K; ++k) p[k] = (SAME && k > 0) ? p[0] : token_pos(a, b[k], s[k]);
  }

  ROPE_HD void store(const Args& a, const Trig<V, PAIR>* t) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k > 0 && !live[k]) continue;
      if (p[k] < 0) {  // skipped token: in place nothing is written
        if constexpr (OOP) copy_span<T, V, ALIGNED>(in[k], out[k], 0, a.head_dim, c[k], a.lanes);
        continue;
      }
      r[k].rotate(t[k]);
      r[k].store(out[k], c[k], a.half);
      if constexpr (OOP)
        copy_span<T, V, ALIGNED>(in[k], out[k], 2 * a.half, a.head_dim, c[k], a.lanes);
    }
  }

  template <int SRC>
  ROPE_HD void finish(const Args& a) {
    positions(a);
    Trig<V, PAIR> t[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (p[k] >= 0) t[k].template load<SRC>(a, p[k], c[k] * NP);
    store(a, t);
  }

  // lds: the workgroup's (cos, sin) pairs, [token][frequency] (see theta_fill)
  ROPE_HD void finish_shared(const Args& a, const float* lds) {
    Trig<V, PAIR> t[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (p[k] >= 0) t[k].from_shared(a, lds, tl[k] * a.half + c[k] * NP);
    store(a, t);
  }
};

// A workgroup owns tokens_per_block consecutive tokens at a time; its items
// are numbered (token, head, chunk) with the chunk fastest, so that when the
// heads of a token are adjacent in memory the workgroup walks one contiguous
// stretch. Three instantiations, chosen by the planner:
//   kTokenOne    : one token per workgroup, the grid covers every token, and
//                  each lane holds at most token_items_per_lane(PAIR) items,
//                  i and i + L for L lanes. The token index is uniform across
//                  the wave, so the index load is a scalar load. Decode and
//                  token-major prefill; kept apart so that its code is short.
//   kTokenPacked : the same with tokens_per_block > 1 tokens per workgroup.
//   kTokenLoop   : workgroups loop over tokens, one item per lane at a time.
enum TokenMode : int { kTokenLoop = 0, kTokenPacked = 1, kTokenOne = 2 };

// The items of lane `thread` in the single-pass modes (kTokenOne,
// kTokenPacked): L lanes, lane t holding items t and t + L of the
// workgroup's tokens_per_block * (Hq + Hk) * lanes items.
template <int MODE, int K>
ROPE_HD int single_pass_items(const Args& a, int64_t block, int thread, int64_t* n, int* it,
                              int* tl, bool* live) {
  const int per_token = (a.n_heads_q + a.n_heads_k) * a.lanes;
  const int tpb = MODE == kTokenOne ? 1 : a.tokens_per_block;
  const int items = tpb * per_token;
  const int L = (items + K - 1) / K;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int i = thread + k * L;
    if constexpr (MODE == kTokenOne) {
      n[k] = block;
      it[k] = i;
      tl[k] = 0;
      live[k] = thread < L && i < items;
    } else {
      tl[k] = i / per_token;
      n[k] = block * tpb + tl[k];
      it[k] = i - tl[k] * per_token;
      live[k] = thread < L && i < items && n[k] < a.n_tokens;
    }
  }
  return L;
}

template <typename T, int V, int PAIR, bool ALIGNED, int MODE, bool OOP, int SRC>
ROPE_HD void token_body(const Args& a, int64_t block, int64_t grid, int thread,
                        int block_dim) {
  constexpr int K = token_items_per_lane(PAIR);
  if constexpr (MODE == kTokenOne || MODE == kTokenPacked) {
    int64_t n[K];
    int it[K], tl[K];
    bool live[K];
    single_pass_items<MODE, K>(a, block, thread, n, it, tl, live);
    TokenWork<T, V, PAIR, ALIGNED, OOP, K, MODE == kTokenOne> w;
    if (w.begin(a, n, it, tl, live)) w.template finish<SRC>(a);
  } else {
    const int per_token = (a.n_heads_q + a.n_heads_k) * a.lanes;
    const int tpb = a.tokens_per_block;
    const int per_block = tpb * per_token;
    for (int64_t n0 = block * tpb; n0 < a.n_tokens; n0 += grid * tpb)
      for (int i = thread; i < per_block; i += block_dim) {
        const int tl = tpb == 1 ? 0 : i / per_token;
        const int64_t n = n0 + tl;
        const int it = i - tl * per_token;
        const bool live = n < a.n_tokens;
        TokenWork<T, V, PAIR, ALIGNED, OOP, 1, true> w;
        if (w.begin(a, &n, &it, &tl, &live)) w.template finish<SRC>(a);
      }
  }
}

// The kernel entry for cos/sin read from tables, or computed per lane (the
// loop mode), also run on the host by the emulator.
template <typename T, int V, int PAIR, bool ALIGNED, int MODE, bool OOP>
ROPE_HD void token_entry(const Args& a, int64_t block, int64_t grid, int thread,
                         int block_dim) {
  if (a.angles)
    token_body<T, V, PAIR, ALIGNED, MODE, OOP, kTrigTheta>(a, block, grid, thread, block_dim);
  else if (a.t_vec)
    token_body<T, V, PAIR, ALIGNED, MODE, OOP, kTrigVec>(a, block, grid, thread, block_dim);
  else
    token_body<T, V, PAIR, ALIGNED, MODE, OOP, kTrigScalar>(a, block, grid, thread, block_dim);
}

// Angles computed from theta in the single-pass modes: the workgroup's
// tokens_per_block * R/2 (cos, sin) pairs are computed once, one pair per
// lane and pass, into shared memory laid out [token][frequency][cos, sin],
// instead of by every head's lane. Skipped tokens' pairs are left unset; no
// item reads them.
template <int MODE>
ROPE_HD void theta_fill(const Args& a, int64_t block, int thread, int block_dim, float* lds) {
  const int tpb = MODE == kTokenOne ? 1 : a.tokens_per_block;
  const int values = tpb * a.half;
  if constexpr (MODE == kTokenOne) {
    // One token: its position is read once (uniform: a scalar load). Each
    // lane forms its frequency before the position arrives, and computes the
    // pair even for a skipped token (as position 0) so that no branch sits
    // between the position and the arithmetic; only the store is skipped.
    const int64_t b = a.seq_len == 1 ? block : block / a.seq_len;
    const int64_t p = token_pos(a, b, block - b * a.seq_len);
    for (int v = thread; v < values; v += block_dim) {
      const double f = theta_freq(a, v);
      float c, sn;
      sincos_f32(theta_pos(a, p < 0 ? 0 : p) * f, &c, &sn);
      if (p >= 0) {
        lds[2 * v] = c;
        lds[2 * v + 1] = sn;
      }
    }
  } else {
    for (int v = thread; v < values; v += block_dim) {
      const int tl = v / a.half;
      const int i = v - tl * a.half;
      const int64_t n = block * tpb + tl;
      if (n >= a.n_tokens) continue;
      const double f = theta_freq(a, i);
      const int64_t b = a.seq_len == 1 ? n : n / a.seq_len;
      const int64_t p = token_pos(a, b, n - b * a.seq_len);
      float c, sn;
      sincos_f32(theta_pos(a, p < 0 ? 0 : p) * f, &c, &sn);
      if (p >= 0) {
        lds[2 * v] = c;
        lds[2 * v + 1] = sn;
      }
    }
  }
}

// Shared memory of the single-pass modes with angles from theta, in bytes.
ROPE_HD int64_t theta_shared_bytes(int64_t tokens_per_block, int64_t half) {
  return tokens_per_block * half * 2 * (int64_t)sizeof(float);
}

// The angles-from-theta path of the single-pass modes (device only: it holds
// a workgroup barrier). Every lane reaches the barrier: lanes without items
// still compute shared cos/sin.
template <typename T, int V, int PAIR, bool ALIGNED, int MODE, bool OOP>
__device__ __forceinline__ void token_theta_single(const Args& a) {
  extern __shared__ float lds[];
  constexpr int K = token_items_per_lane(PAIR);
  int64_t n[K];
  int it[K], tl[K];
  bool live[K];
  single_pass_items<MODE, K>(a, blockIdx.x, threadIdx.x, n, it, tl, live);
  TokenWork<T, V, PAIR, ALIGNED, OOP, K, MODE == kTokenOne> w;
  const bool has = w.begin(a, n, it, tl, live);  // row loads in flight
  if (has) w.positions(a);
  theta_fill<MODE>(a, blockIdx.x, threadIdx.x, blockDim.x, lds);
  __syncthreads();
  if (has) w.finish_shared(a, lds);
}

// SRC: a TrigSource fixed at compile time, or kSrcRuntime to choose from the
// arguments. The one-token mode (decode) gets one instantiation per source, so
// that each loads its arguments once, up front: a runtime branch on the
// source made the compiler fetch the table path's arguments only after the
// branch, a second round trip on the decode latency path (~0.1 us measured).
constexpr int kSrcRuntime = -1;

template <typename T, int V, int PAIR, bool ALIGNED, int MODE, bool OOP, int SRC>
__global__ void __launch_bounds__(1024) rope_token_kernel(Args a) {
  constexpr bool single = MODE == kTokenOne || MODE == kTokenPacked;
  // Ask for one field of each of the argument block's first three 64-byte
  // lines before anything else, so that the scalar cache fetches all three in
  // one round trip; left to itself the compiler fetches them one after
  // another as they are first used, each a round trip on the decode latency
  // path (measured: 2.42 -> 2.34 us per graph-replayed decode call).
  asm volatile("" ::"s"(a.q_in.base), "s"(a.cos), "s"(a.half));
  if constexpr (SRC == kTrigTheta && single) {
    token_theta_single<T, V, PAIR, ALIGNED, MODE, OOP>(a);
  } else if constexpr (SRC != kSrcRuntime) {
    token_body<T, V, PAIR, ALIGNED, MODE, OOP, SRC>(a, blockIdx.x, gridDim.x, threadIdx.x,
                                                    blockDim.x);
  } else {
    if (single && a.angles)
      token_theta_single<T, V, PAIR, ALIGNED, MODE, OOP>(a);
    else
      token_entry<T, V, PAIR, ALIGNED, MODE, OOP>(a, blockIdx.x, gridDim.x, threadIdx.x,
                                                  blockDim.x);
  }
}

}  // namespace rope

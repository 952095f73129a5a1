// rope_kernels.hpp -- gfx950 device code for fused rotary position embedding.
//
// The operation is an elementwise map that moves ~4 bytes per rotated pair
// (16-bit) and does ~10 float ops on it, so it is bound by HBM bandwidth
// ("Rotary Embedding Kernel", Overview: memory-bound, judged in GB/s). The
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

// Everything a launch needs, passed by value as the kernel argument.
struct Args {
  View q_in, k_in;           // K views unused when n_heads_k == 0
  View q_out, k_out;         // equal to the inputs in place
  const float* cos;          // frequency i of position p at [p*t_row + i*t_col]
  const float* sin;
  int64_t t_row;             // table row stride (floats)
  int32_t t_col;             // table column stride (1 or 2)
  int32_t t_vec;             // 1: a chunk's cos/sin are contiguous and aligned
  const int32_t* pos;        // nullptr: p = s
  int64_t pos_bs;            // index batch stride
  int64_t table_rows;
  int64_t batch;
  int64_t seq_len;
  int64_t n_tokens;          // batch * seq_len
  int64_t n_items;           // n_tokens * lanes (rows kernel)
  int32_t head_dim;          // D (out-of-place copies)
  int32_t half;              // R / 2
  int32_t n_heads_q;
  int32_t n_heads_k;
  int32_t lanes;             // chunks per token row
  int32_t lanes_shift;       // log2(lanes) when lanes is a power of two, else -1
  int32_t heads_per_group;   // rows kernel: heads walked by one lane
  int32_t n_groups;          // rows kernel: head groups
  int32_t group_slow;        // rows kernel: workgroup ids run over tiles first
  int64_t n_tiles;           // rows kernel: 256-item tiles
  int32_t tokens_per_block;  // token kernel: consecutive tokens per workgroup
  float sin_sign;            // +1 forward, -1 backward
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

// cos/sin of one chunk: frequencies first .. first+NP-1 of row p. With a
// [rows, R/2] (or halves-duplicated [rows, R]) table these are NP contiguous
// floats, aligned to min(16, 4*NP) bytes (the tables are 16-byte aligned and
// the plan checks that the row stride keeps them so), and move in vector
// loads (TVEC); a repeat-interleaved table is read one value at a time. TVEC
// is chosen once at the top of each kernel, so each copy of the body is
// straight-line code whose loads the compiler can wait for one by one.
template <int V, int PAIR> struct Trig {
  static constexpr int NP = ChunkGeom<V, PAIR>::kPairs;
  static constexpr int W = NP < 4 ? NP : 4;  // floats per vector load
  typedef float vec_t __attribute__((ext_vector_type(W)));
  float c[NP], s[NP];
  float sign;  // +1 forward, -1 backward; applied in the rotation, so that no
               // arithmetic waits on the loads here

  template <bool TVEC>
  ROPE_HD void load(const Args& a, int64_t p, int first) {
    sign = a.sin_sign;
    const float* cr = a.cos + p * a.t_row;
    const float* sr = a.sin + p * a.t_row;
    if constexpr (TVEC) {
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

template <typename T, int V, int PAIR, bool ALIGNED, int U, bool OOP, bool TVEC>
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
  t.template load<TVEC>(a, p, c * ChunkGeom<V, PAIR>::kPairs);
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
  if (a.t_vec)
    rows_body<T, V, PAIR, ALIGNED, U, OOP, true>(a, block, thread);
  else
    rows_body<T, V, PAIR, ALIGNED, U, OOP, false>(a, block, thread);
}

template <typename T, int V, int PAIR, bool ALIGNED, int U, bool OOP>
__global__ void __launch_bounds__(kRowsBlock) rope_rows_kernel(Args a) {
  rows_entry<T, V, PAIR, ALIGNED, U, OOP>(a, blockIdx.x, threadIdx.x);
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

// K items of the token shape, run together: all row loads, then the
// positions and cos/sin, then rotate and store. Item k is (head, chunk) item
// it[k] of token n[k] and is stored only if live[k]; a lane whose item 0 is
// not live has nothing to do. A dead item k > 0 loads item 0's row and
// cos/sin instead of branching around its loads, so every load of the lane is
// issued in one straight run. SAME: every item is of token n[0] (one token per
// workgroup), so the token's position is read once.
template <typename T, int V, int PAIR, bool ALIGNED, bool OOP, bool TVEC, int K, bool SAME>
ROPE_HD void token_items(const Args& a, const int64_t* n_in, const int* it_in,
                         const bool* live) {
  if (!live[0]) return;
  int64_t n[K];
  int it[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    n[k] = (k == 0 || live[k]) ? n_in[k] : n_in[0];
    it[k] = (k == 0 || live[k]) ? it_in[k] : it_in[0];
  }
  const T* in[K];
  T* out[K];
  int c[K];
  int64_t b[K], s[K], p[K];
  RowChunk<T, V, PAIR, ALIGNED> r[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (SAME && k > 0) {
      b[k] = b[0];
      s[k] = s[0];
    } else {
      b[k] = a.seq_len == 1 ? n[k] : n[k] / a.seq_len;  // decode: no division
      s[k] = n[k] - b[k] * a.seq_len;
    }
    int h;
    split_item(a, it[k], &h, &c[k]);
    const bool is_q = h < a.n_heads_q;
    const int hh = is_q ? h : h - a.n_heads_q;
    in[k] = view_row<T>(is_q ? a.q_in : a.k_in, hh, b[k], s[k]);
    // in place the output view is the input view
    out[k] = OOP ? view_row<T>(is_q ? a.q_out : a.k_out, hh, b[k], s[k]) : const_cast<T*>(in[k]);
    r[k].load(in[k], c[k], a.half);
  }
  Trig<V, PAIR> t[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    p[k] = (SAME && k > 0) ? p[0] : token_pos(a, b[k], s[k]);
    if (p[k] >= 0) t[k].template load<TVEC>(a, p[k], c[k] * ChunkGeom<V, PAIR>::kPairs);
  }
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

template <typename T, int V, int PAIR, bool ALIGNED, int MODE, bool OOP, bool TVEC>
ROPE_HD void token_body(const Args& a, int64_t block, int64_t grid, int thread,
                        int block_dim) {
  const int per_token = (a.n_heads_q + a.n_heads_k) * a.lanes;
  const int tpb = a.tokens_per_block;
  constexpr int K = token_items_per_lane(PAIR);
  if constexpr (MODE == kTokenOne) {
    const int L = (per_token + K - 1) / K;
    if (thread >= L) return;  // the block is rounded up to whole waves
    int64_t n[K];
    int it[K];
    bool live[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      n[k] = block;
      it[k] = thread + k * L;
      live[k] = it[k] < per_token;
    }
    token_items<T, V, PAIR, ALIGNED, OOP, TVEC, K, true>(a, n, it, live);
  } else if constexpr (MODE == kTokenPacked) {
    const int items = tpb * per_token;
    const int L = (items + K - 1) / K;
    if (thread >= L) return;
    int64_t n[K];
    int it[K];
    bool live[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = thread + k * L;
      const int tl = i / per_token;
      n[k] = block * tpb + tl;
      it[k] = i - tl * per_token;
      live[k] = i < items && n[k] < a.n_tokens;
    }
    token_items<T, V, PAIR, ALIGNED, OOP, TVEC, K, false>(a, n, it, live);
  } else {
    const int per_block = tpb * per_token;
    for (int64_t n0 = block * tpb; n0 < a.n_tokens; n0 += grid * tpb)
      for (int i = thread; i < per_block; i += block_dim) {
        const int tl = tpb == 1 ? 0 : i / per_token;
        const int64_t n = n0 + tl;
        const int it = i - tl * per_token;
        const bool live = n < a.n_tokens;
        token_items<T, V, PAIR, ALIGNED, OOP, TVEC, 1, true>(a, &n, &it, &live);
      }
  }
}

// The kernel entry, also run on the host by the emulator.
template <typename T, int V, int PAIR, bool ALIGNED, int MODE, bool OOP>
ROPE_HD void token_entry(const Args& a, int64_t block, int64_t grid, int thread,
                         int block_dim) {
  if (a.t_vec)
    token_body<T, V, PAIR, ALIGNED, MODE, OOP, true>(a, block, grid, thread, block_dim);
  else
    token_body<T, V, PAIR, ALIGNED, MODE, OOP, false>(a, block, grid, thread, block_dim);
}

template <typename T, int V, int PAIR, bool ALIGNED, int MODE, bool OOP>
__global__ void __launch_bounds__(1024) rope_token_kernel(Args a) {
  token_entry<T, V, PAIR, ALIGNED, MODE, OOP>(a, blockIdx.x, gridDim.x, threadIdx.x,
                                              blockDim.x);
}

}  // namespace rope

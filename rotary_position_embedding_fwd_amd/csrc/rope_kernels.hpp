// rope_kernels.hpp -- gfx950 device code for fused rotary position embedding.
//
// The operation is an elementwise map that moves ~4 bytes per rotated pair
// (16-bit) and does ~10 float ops on it, so it is bound by HBM bandwidth
// ("Rotary Embedding Kernel", Overview: memory-bound, judged in GB/s). The
// kernels therefore aim at three things only: whole-row 128-bit loads and
// stores, cos/sin read once per token and reused for every Q and K head of
// that token (the reuse that head grouping buys in How Unsloth Optimizes RoPE
// Embedding Computations in Triton Kernels, Triton Kernel Architecture for
// RoPE), and enough loads in flight per CU to cover HBM latency.
//
// Work unit. A token row of R rotated dims is cut into `lanes` chunks of V
// contiguous elements per access:
//   split-half  : chunk c covers dims [cV, cV+V) and [R/2+cV, R/2+cV+V): V pairs
//   interleaved : chunk c covers dims [cV, cV+V): V/2 adjacent pairs
// ("Rotary Embedding Kernel", Paired Element Layout). A lane owns one chunk of
// one token and holds that chunk's cos/sin in registers.
//
// Two grid shapes share the same per-chunk device function:
//   rope_rows_kernel  : lanes over (token, chunk); each lane walks a group of
//                       heads (Q heads first, then K heads). For prefill.
//   rope_token_kernel : one token per workgroup iteration, lanes over (head,
//                       chunk). For decode (seq_len 1), where there are too
//                       few tokens to fill the chip with the first shape.
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

// Everything a launch needs, passed by value as the kernel argument.
struct Args {
  char* q;  // Q base (bytes)
  char* k;  // K base (bytes); unused when n_heads_k == 0
  int64_t q_sb, q_sh, q_ss;  // Q element strides: batch, head, sequence
  int64_t k_sb, k_sh, k_ss;  // K element strides
  const float* cos;          // [table_rows, half]
  const float* sin;
  const int32_t* pos;        // nullptr: p = s
  int64_t pos_bs;            // index batch stride
  int64_t table_rows;
  int64_t batch;
  int64_t seq_len;
  int64_t n_tokens;          // batch * seq_len
  int64_t n_items;           // n_tokens * lanes (rows kernel)
  int32_t half;              // R / 2: cos/sin row length
  int32_t n_heads_q;
  int32_t n_heads_k;
  int32_t lanes;             // chunks per token row
  int32_t lanes_shift;       // log2(lanes) when lanes is a power of two, else -1
  int32_t heads_per_group;   // rows kernel: heads walked by one lane
  int32_t n_groups;          // rows kernel: head groups
  int32_t group_slow;        // rows kernel: workgroup ids run over tiles first
  int64_t n_tiles;           // rows kernel: 256-item tiles
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
ROPE_HD void rotate_pair(float x1, float x2, float c, float sn,
                                            float& y1, float& y2) {
  const float p1 = x2 * sn;
  const float e1 = __builtin_fmaf(x2, sn, -p1);  // x2*sn - p1, exact
  y1 = __builtin_fmaf(x1, c, -p1) - e1;          // x1*c - x2*sn
  const float p2 = x1 * sn;
  const float e2 = __builtin_fmaf(x1, sn, -p2);  // x1*sn - p2, exact
  y2 = __builtin_fmaf(x2, c, p2) + e2;           // x1*sn + x2*c
}

// Pairs per chunk and the chunk's column in the cos/sin row.
template <int V, int PAIR> struct ChunkGeom {
  static constexpr int kPairs = PAIR == kSplitHalf ? V : V / 2;
};

// cos/sin of one chunk: kPairs consecutive floats of row p. The row length
// (R/2) is a multiple of kPairs and the tables are 16-byte aligned, so the
// slice is aligned to min(16, 4 * kPairs) bytes and moves in vector loads.
template <int V, int PAIR> struct Trig {
  static constexpr int NP = ChunkGeom<V, PAIR>::kPairs;
  static constexpr int W = NP < 4 ? NP : 4;  // floats per load
  typedef float vec_t __attribute__((ext_vector_type(W)));
  float c[NP], s[NP];

  ROPE_HD void load(const float* cos_row, const float* sin_row, int col,
                                       float sign) {
#pragma unroll
    for (int j = 0; j < NP; j += W) {
      const vec_t cv = *reinterpret_cast<const vec_t*>(cos_row + col + j);
      const vec_t sv = *reinterpret_cast<const vec_t*>(sin_row + col + j);
#pragma unroll
      for (int w = 0; w < W; ++w) {
        c[j + w] = cv[w];
        s[j + w] = sign * sv[w];
      }
    }
  }
};

// Rotate one chunk of a row in place.
//   row : first element of the head row
//   c   : chunk index
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
        rotate_pair(to_f32(a.v[j]), to_f32(b.v[j]), t.c[j], t.s[j], y1, y2);
        a.v[j] = from_f32<T>(y1);
        b.v[j] = from_f32<T>(y2);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        float y1, y2;
        rotate_pair(to_f32(a.v[2 * j]), to_f32(a.v[2 * j + 1]), t.c[j], t.s[j], y1, y2);
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

// Row start of head h (Q heads first, then K heads) for token (b, s).
template <typename T>
ROPE_HD T* head_row(const Args& a, int h, int64_t b, int64_t s) {
  if (h < a.n_heads_q)
    return reinterpret_cast<T*>(a.q) + (b * a.q_sb + (int64_t)h * a.q_sh + s * a.q_ss);
  return reinterpret_cast<T*>(a.k) +
         (b * a.k_sb + (int64_t)(h - a.n_heads_q) * a.k_sh + s * a.k_ss);
}

// Position of token (b, s), or -1 when the token passes through.
ROPE_HD int64_t token_pos(const Args& a, int64_t b, int64_t s) {
  const int64_t p = a.pos ? (int64_t)a.pos[b * a.pos_bs + s] : s;
  return (p < 0 || p >= a.table_rows) ? -1 : p;
}

// ------------------------------------------------------ rows (prefill) shape
// Rotate one lane's chunk in heads [h_lo, h_hi) of one tensor whose rows for
// this token start at `base` and are `stride` elements apart. U heads are
// loaded before any is rotated so that U row loads are in flight at once.
template <typename T, int V, int PAIR, bool ALIGNED, int U>
ROPE_HD void rotate_heads(T* base, int64_t stride, int h_lo, int h_hi,
                                             int c, int half, const Trig<V, PAIR>& t) {
  for (int h0 = h_lo; h0 < h_hi; h0 += U) {
    RowChunk<T, V, PAIR, ALIGNED> r[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (h0 + u < h_hi) r[u].load(base + (int64_t)(h0 + u) * stride, c, half);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (h0 + u < h_hi) {
        r[u].rotate(t);
        r[u].store(base + (int64_t)(h0 + u) * stride, c, half);
      }
    }
  }
}

// Tokens are numbered in memory order (n = b * seq_len + s), so in the [B,H,S,D]
// layout the 4 waves of a workgroup cover 32 consecutive rows (8 KiB at
// D=128, bf16) of each head they visit. Workgroup ids run over (tile, head
// group) with the group fastest, and are left in the hardware's round-robin
// order over the XCDs: renumbering them so that each XCD owns one contiguous
// range of tiles was measured ~10% slower.
constexpr int kRowsBlock = 256;

template <typename T, int V, int PAIR, bool ALIGNED, int U>
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

  const int64_t p = token_pos(a, b, s);
  if (p < 0) return;  // masked token: nothing is read or written

  Trig<V, PAIR> t;
  t.load(a.cos + p * a.half, a.sin + p * a.half, c * ChunkGeom<V, PAIR>::kPairs, a.sin_sign);

  const int h_begin = group * a.heads_per_group;
  const int h_end = imin(h_begin + a.heads_per_group, a.n_heads_q + a.n_heads_k);
  if (h_begin < a.n_heads_q) {
    T* qb = reinterpret_cast<T*>(a.q) + (b * a.q_sb + s * a.q_ss);
    rotate_heads<T, V, PAIR, ALIGNED, U>(qb, a.q_sh, h_begin, imin(h_end, a.n_heads_q), c,
                                         a.half, t);
  }
  if (h_end > a.n_heads_q) {
    T* kb = reinterpret_cast<T*>(a.k) + (b * a.k_sb + s * a.k_ss);
    rotate_heads<T, V, PAIR, ALIGNED, U>(kb, a.k_sh, imax(h_begin - a.n_heads_q, 0),
                                         h_end - a.n_heads_q, c, a.half, t);
  }
}

template <typename T, int V, int PAIR, bool ALIGNED, int U>
__global__ void __launch_bounds__(kRowsBlock) rope_rows_kernel(Args a) {
  rows_body<T, V, PAIR, ALIGNED, U>(a, blockIdx.x, threadIdx.x);
}

// ------------------------------------------------------ token (decode) shape
// One token per workgroup iteration; lanes cover (head, chunk) pairs of that
// token. The head rows are requested before the position, so the row loads
// overlap the dependent index -> cos/sin chain.
ROPE_HD void split_item(const Args& a, int it, int* h, int* c) {
  if (a.lanes_shift >= 0) {
    *h = it >> a.lanes_shift;
    *c = it & ((1 << a.lanes_shift) - 1);
  } else {
    *h = it / a.lanes;
    *c = it - *h * a.lanes;
  }
}

template <typename T, int V, int PAIR, bool ALIGNED>
ROPE_HD void token_item(const Args& a, int64_t n, int it) {
  const int64_t b = n / a.seq_len;
  const int64_t s = n - b * a.seq_len;
  int h, c;
  split_item(a, it, &h, &c);
  T* row = head_row<T>(a, h, b, s);
  RowChunk<T, V, PAIR, ALIGNED> r;
  r.load(row, c, a.half);
  const int64_t p = token_pos(a, b, s);
  if (p < 0) return;
  Trig<V, PAIR> t;
  t.load(a.cos + p * a.half, a.sin + p * a.half, c * ChunkGeom<V, PAIR>::kPairs, a.sin_sign);
  r.rotate(t);
  r.store(row, c, a.half);
}

// SINGLE: the grid has one workgroup per token and each workgroup one lane
// per (head, chunk), so no loop is needed (the decode case).
template <typename T, int V, int PAIR, bool ALIGNED, bool SINGLE>
ROPE_HD void token_body(const Args& a, int64_t block, int64_t grid, int thread,
                        int block_dim) {
  const int per_token = (a.n_heads_q + a.n_heads_k) * a.lanes;
  if constexpr (SINGLE) {
    if (thread < per_token) token_item<T, V, PAIR, ALIGNED>(a, block, thread);
  } else {
    for (int64_t n = block; n < a.n_tokens; n += grid)
      for (int it = thread; it < per_token; it += block_dim)
        token_item<T, V, PAIR, ALIGNED>(a, n, it);
  }
}

template <typename T, int V, int PAIR, bool ALIGNED, bool SINGLE>
__global__ void __launch_bounds__(1024) rope_token_kernel(Args a) {
  token_body<T, V, PAIR, ALIGNED, SINGLE>(a, blockIdx.x, gridDim.x, threadIdx.x, blockDim.x);
}

}  // namespace rope

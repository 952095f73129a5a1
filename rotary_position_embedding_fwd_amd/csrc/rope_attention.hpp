// rope_attention.hpp -- attention with RoPE applied to the loaded Q and K
// blocks, for gfx950 matrix cores (rotary-embedding-torch docs,
// flash_attn_with_rotary: the rotation happens on the Q and K blocks inside
// the attention kernel, so no rotated Q or K is written to memory; GQA; causal
// masking; per-token positions with skipped tokens).
//
// O = softmax(scale * rope(Q) rope(K)^T [+ causal mask]) V, per (batch, query
// head), with K/V head h / (Hq / Hk). rope() is the same pair rotation, in the
// same float32 arithmetic, as the stand-alone kernels (rope_kernels.hpp), and
// the rotated values are rounded to bf16 as the stand-alone pass would store
// them, so the fused result equals rope_fwd_qk followed by attention.
//
// Shape of the computation (one workgroup = 8 waves = 256 query rows: 32
// rows per wave, from hw query heads that share one K/V head, 256 / hw rows
// of each; the two lanes l and l + 32 of a wave share one query row):
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16. Each lane's accumulators hold
//                 its query's scores against 32 of a 64-key tile, so the
//                 softmax statistics are per lane plus one exchange with the
//                 partner lane (lane ^ 32, v_permlane32_swap).
//   O^T += V^T P^T  with the same instruction; the score registers are the
//                 P^T operand directly, under a fixed permutation of the keys
//                 inside each 16-key step that V^T's reads follow.
// Q is loaded and rotated once into the registers of the B operand of S^T.
// Each 64-key tile of K is rotated once per workgroup, for all its 256 rows,
// while it is staged into LDS ([key][dim], rows padded by 16 bytes); V is
// staged transposed ([dim][key], padded, keys in v_slot order) so that the A
// operand of O^T is one 16-byte LDS read per lane and step. Tiles are
// double-buffered: the next tile is fetched while the current one is worked
// on and staged into the other buffer after its products, with one barrier
// per tile. Small grids at head dim 64 use G = 2 or 4 wave groups instead:
// 256 / G rows per workgroup, held by every group, each group taking every
// G-th key tile into its own double buffer, the groups' softmax states
// merged at the end (the rotated K is then staged per group's tiles).
// The softmax runs in base 2 with the scale folded into log2(e), one online
// step per 32-key half of a tile; the halves are software-pipelined so that
// one half's softmax sits beside the other half's matrix instructions. Each
// row's reference max moves only when a step's max passes it by more than 8
// in the base-2 exponent, which keeps the weights below 2^8 and the output
// rescales rare. A negative scale is taken as |scale| with Q negated.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (checked on the device by a
// probe): A (32x16): lane l, slot i holds A[l%32][(l/32)*8 + i]; B (16x32):
// B[(l/32)*8 + i][l%32]; C/D (32x32 float): accumulator j of lane l holds
// C[8*(j/4) + 4*(l/32) + j%4][l%32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rope_kernels.hpp"

namespace rope {
namespace attn {

constexpr int kWaves = 8;
constexpr int kBlock = 64 * kWaves;         // lanes per workgroup
constexpr int kRows = 32 * kWaves;          // query rows per workgroup (one wave group)
constexpr int kKeys = 64;                   // keys per tile
constexpr int kKPad = 8;                    // K tile row padding (bf16)
constexpr int kVPad = 8;                    // V^T tile row padding (bf16)
constexpr int kXcds = 8;                    // accelerator dies, one L2 each

struct AttnArgs {
  const __bf16* q;    // [B, Hq, Sq, D]
  const __bf16* k;    // [B, Hk, Sk, D]
  const __bf16* v;    // [B, Hk, Sk, D]
  __bf16* o;          // [B, Hq, Sq, D]
  const float* cos;   // [table_rows, R/2]
  const float* sin;
  const int32_t* q_pos;  // nullptr: query row i at i + Sk - Sq
  const int32_t* k_pos;  // nullptr: key row j at j
  int64_t q_pos_bs, k_pos_bs;
  int64_t table_rows;
  int32_t batch, n_heads_q, n_heads_k, seq_q, seq_k;
  int32_t half;          // R / 2
  int32_t rotate;        // 0: no rotation (plain attention, for the unfused path)
  int32_t rotate_k;      // 0: K arrives rotated (or no rotation): stage it as it is
  int32_t causal;
  int32_t groups;        // wave groups taking turns on the key tiles: 1, 2 or 4
  int32_t hw;            // query heads per workgroup (a power of 2 dividing Hq / Hk)
  int32_t rows;          // query rows of each head per workgroup: kRows / hw
  int32_t head_groups;   // Hq / hw
  int32_t q_tiles;       // ceil(Sq / rows)
  int32_t negate_q;      // 1: the scale is negative; the scores are taken with -Q
  float scale_log2e;     // |softmax scale| * log2(e), a normal float
};

// ------------------------------------------------------------- addresses
// Everything that forms an address is a plain function of the indices, so
// the host can enumerate the whole grid and check every access against the
// buffers before the kernel first runs on a device.

template <int D> ROPE_HD int64_t row_of(const AttnArgs& a, int b, int h, int heads, int seq,
                                        int s) {
  return (((int64_t)b * heads + h) * seq + s) * D;
}

// K tile staging items, in three classes; item n of lane t in a class is
// class item t + n * NT (NT staging lanes), and class item it covers key it / per_key,
// chunk it % per_key:
//   - split-half pair items (R/16 = 2 H16 per key): chunk j rotates the
//     pairs of dims 8j .. 8j + 7 with R/2 + 8j .. R/2 + 8j + 7;
//   - split-half copy items ((D - R)/8 per key): chunk j copies dims
//     R + 8j .. R + 8j + 7;
//   - interleaved items (D/8 per key): chunk j holds dims 8j .. 8j + 7,
//     rotated (4 pairs) when 8j < R.
// The counts are fixed by the instantiation (R = 32 H16 for split-half).
template <int D, int PAIR, int H16, int NT = kBlock> struct KPlan {
  static constexpr int kPair = PAIR == kSplitHalf ? 2 * H16 : 0;
  static constexpr int kCopy = PAIR == kSplitHalf ? D / 8 - 4 * H16 : 0;
  static constexpr int kInter = PAIR == kSplitHalf ? 0 : D / 8;
  // NT: the lanes that stage a tile (the workgroup, or one wave group)
  static constexpr int lanes(int per_key) { return (kKeys * per_key + NT - 1) / NT; }
  static constexpr int kPairN = lanes(kPair), kCopyN = lanes(kCopy), kInterN = lanes(kInter);
};

// LDS layout, in bf16 elements: two buffers, each a K tile
// [kKeys][D + kKPad] followed by a V^T tile [D][kKeys + kVPad] (keys in
// v_slot order).
template <int D> constexpr int k_lds_elems() { return kKeys * (D + kKPad); }
template <int D> constexpr int v_lds_elems() { return D * (kKeys + kVPad); }
template <int D> constexpr int buf_elems() { return k_lds_elems<D>() + v_lds_elems<D>(); }
// G wave groups: a double buffer per group
template <int D> constexpr int lds_bytes_groups(int g) { return 2 * 2 * g * buf_elems<D>(); }
template <int D> ROPE_HD int k_lds(int buf, int key, int dim) {
  return buf * buf_elems<D>() + key * (D + kKPad) + dim;
}
// V^T slot of key `key` (0 .. kKeys-1) of a tile: inside each 16-key group
// the second and third quads trade places, so the 8 keys one lane feeds a
// product step (keys 4 hs .. 4 hs + 3 and 8 + 4 hs .. 11 + 4 hs of the
// group) sit in the 8 consecutive slots 8 hs .. 8 hs + 7: one 16-byte read.
ROPE_HD int v_slot(int key) {
  const int q = (key >> 2) & 3;
  const int qs = q == 1 ? 2 : (q == 2 ? 1 : q);
  return (key & ~15) | (qs << 2) | (key & 3);
}
template <int D> ROPE_HD int v_lds(int buf, int dim, int slot) {
  return buf * buf_elems<D>() + k_lds_elems<D>() + dim * (kKeys + kVPad) + slot;
}

// Workgroup -> (batch, head group, query tile). Workgroups are handed to
// the dies round-robin (workgroup w to die w % 8), so the work list is cut
// into 8 contiguous ranges and die x walks range x: the query tiles of one
// head group, and the groups of one K/V head, run on one die and share its
// L2. Within a group the tiles go from the last (most keys when causal) to
// the first, so the short ones fill the tail of the launch.
struct Work {
  int b, hg, q_tile;
};
ROPE_HD Work work_of(const AttnArgs& a, int64_t blk) {
  const int64_t n = (int64_t)a.q_tiles * a.head_groups * a.batch;
  const int64_t full = n / kXcds, rem = n % kXcds;
  const int64_t x = blk % kXcds, local = blk / kXcds;
  const int64_t w = x * full + (x < rem ? x : rem) + local;
  Work r;
  r.q_tile = a.q_tiles - 1 - (int)(w % a.q_tiles);
  r.hg = (int)((w / a.q_tiles) % a.head_groups);
  r.b = (int)(w / ((int64_t)a.q_tiles * a.head_groups));
  return r;
}

// Wave w of a workgroup: query head hg * hw + w / (kWaves / hw), rows
// q_tile * rows + (w % (kWaves / hw)) * 32 .. + 31. With G wave groups
// (w / (kWaves / G)), the groups hold the same rows and take turns on the
// key tiles; the role is that of wave w % (kWaves / G) among kWaves / G.
struct WaveRole {
  int h, row0;
};
// (groups = a.groups, passed as the kernel's compile-time count)
ROPE_HD WaveRole wave_role(const AttnArgs& a, const Work& wk, int wave, int groups) {
  const int waves = kWaves / groups;
  const int w = wave % waves;
  const int per_head = waves / a.hw;
  return WaveRole{wk.hg * a.hw + w / per_head, wk.q_tile * a.rows + (w % per_head) * 32};
}

// V tile staging: item it holds 4 consecutive keys (4 k4 .. 4 k4 + 3) of 8
// dims (8 c .. 8 c + 7); consecutive lanes take consecutive key quads, so the
// transposed tile is written 8 bytes (4 keys of one dim) at a time.
template <int D> constexpr int v_items() { return (kKeys / 4) * (D / 8); }
struct VItem {
  int k4, c;
};
ROPE_HD VItem v_item(int it) { return VItem{it % (kKeys / 4), it / (kKeys / 4)}; }

// Position of query row i / key row j (or -1: not rotated).
ROPE_HD int64_t query_pos(const AttnArgs& a, int b, int i) {
  int64_t p = a.q_pos ? (int64_t)a.q_pos[(int64_t)b * a.q_pos_bs + i]
                      : (int64_t)i + (a.seq_k - a.seq_q);
  return (p < 0 || p >= a.table_rows) ? -1 : p;
}
ROPE_HD int64_t key_pos(const AttnArgs& a, int b, int j) {
  int64_t p = a.k_pos ? (int64_t)a.k_pos[(int64_t)b * a.k_pos_bs + j] : (int64_t)j;
  return (p < 0 || p >= a.table_rows) ? -1 : p;
}

// Key tiles a workgroup visits: all of them, or (causal) up to the last key
// visible to its last query row.
ROPE_HD int key_tiles(const AttnArgs& a, int q_tile) {
  int last_key = a.seq_k - 1;
  if (a.causal) {
    const int q_last = imin(a.seq_q - 1, q_tile * a.rows + a.rows - 1);
    last_key = imin(last_key, q_last + (a.seq_k - a.seq_q));
  }
  return last_key < 0 ? 0 : last_key / kKeys + 1;
}

// --------------------------------------------------------------- helpers
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Rotate two 8-element chunks (x1 = first halves of 8 pairs, x2 = second
// halves) with NP = 8 frequencies, or one chunk of 4 interleaved pairs.
ROPE_HD void rotate_split8(bf16x8& x1, bf16x8& x2, const float* c, const float* s) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float y1, y2;
    rotate_pair(to_f32(x1[j]), to_f32(x2[j]), c[j], s[j], y1, y2);
    x1[j] = from_f32<__bf16>(y1);
    x2[j] = from_f32<__bf16>(y2);
  }
}
ROPE_HD void rotate_inter8(bf16x8& x, const float* c, const float* s) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float y1, y2;
    rotate_pair(to_f32(x[2 * j]), to_f32(x[2 * j + 1]), c[j], s[j], y1, y2);
    x[2 * j] = from_f32<__bf16>(y1);
    x[2 * j + 1] = from_f32<__bf16>(y2);
  }
}

// n (4 or 8) table entries from `first` (a multiple of 4) of row p: 16-byte
// loads (tables are 16-byte aligned and R/2 is a multiple of 4).
ROPE_HD void load_cs(const AttnArgs& a, int64_t p, int first, int n, float* c, float* s) {
  const uint32_t off = ((uint32_t)p * (uint32_t)a.half + (uint32_t)first) * 4u;
  const float4* cr = reinterpret_cast<const float4*>(reinterpret_cast<const char*>(a.cos) + off);
  const float4* sr = reinterpret_cast<const float4*>(reinterpret_cast<const char*>(a.sin) + off);
  for (int j = 0; j < n / 4; ++j) {
    const float4 cv = cr[j], sv = sr[j];
    c[4 * j] = cv.x;
    c[4 * j + 1] = cv.y;
    c[4 * j + 2] = cv.z;
    c[4 * j + 3] = cv.w;
    s[4 * j] = sv.x;
    s[4 * j + 1] = sv.y;
    s[4 * j + 2] = sv.z;
    s[4 * j + 3] = sv.w;
  }
}

#if defined(__HIP_DEVICE_COMPILE__)
// Combine x with the partner lane l ^ 32 (the other half of the row): gfx950's
// v_permlane32_swap exchanges the two 32-lane halves of a register in the
// vector ALU. Swapping x with itself leaves (lower half's value, upper half's
// value) in the two results of every lane, so max and sum come out the same,
// bit for bit, in both lanes of a row.
__device__ __forceinline__ float wave_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
#endif

// ------------------------------------------------------- tile staging
template <int D, int NT = kBlock> constexpr int v_items_max() {
  return (v_items<D>() + NT - 1) / NT;
}
constexpr int at_least_1(int n) { return n > 0 ? n : 1; }
// Whether staging item it (lane t + n * NT, t < NT, n below the per-lane
// count) exists: always when the NT lanes share the items evenly, which the
// compiler then knows without a per-lane test.
ROPE_HD bool fits(int it, int items, int nt) { return items % nt == 0 || it < items; }

// Raw rows of one tile (and the cos/sin of its rotated items) held in
// registers between fetch and staging.
template <int D, int PAIR, int H16, int NT = kBlock> struct KStage {
  using P = KPlan<D, PAIR, H16, NT>;
  bf16x8 px1[at_least_1(P::kPairN)], px2[at_least_1(P::kPairN)];
  float pc[at_least_1(P::kPairN)][8], ps[at_least_1(P::kPairN)][8];
  bool prot[at_least_1(P::kPairN)];
  bf16x8 cx[at_least_1(P::kCopyN)];
  bf16x8 ix[at_least_1(P::kInterN)];
  float ic[at_least_1(P::kInterN)][4], is[at_least_1(P::kInterN)][4];
  bool irot[at_least_1(P::kInterN)];
};
template <int D, int NT = kBlock> struct VStage {
  u32x4 x[v_items_max<D, NT>()][4];  // 4 key rows x 8 dims, as bf16 pairs
};

#if defined(__HIP_DEVICE_COMPILE__)
// CHECK false: the tile lies wholly inside Sk, key j sits at position j and
// every position has a table row (no index, Sk <= table_rows), so no key is
// tested and every key is rotated: the fetch has no branches.
template <int D, int PAIR, int H16, int NT = kBlock, bool CHECK = true>
__device__ __forceinline__ void fetch_k(const AttnArgs& a, int b, const __bf16* kbase, int k0,
                                        int t, KStage<D, PAIR, H16, NT>& ks) {
  using P = KPlan<D, PAIR, H16, NT>;
  const int R = 2 * a.half;      // interleaved: the rotated dims
  constexpr int kR = 32 * H16;   // split-half: the rotated dims, fixed by the instantiation
  const bf16x8 z = {};
  if constexpr (P::kPair > 0) {
#pragma unroll
    for (int n = 0; n < P::kPairN; ++n) {
      const int it = t + n * NT;
      ks.px1[n] = z;
      ks.px2[n] = z;
      ks.prot[n] = false;
      if (fits(it, kKeys * P::kPair, NT)) {
        const int key = k0 + it / P::kPair, j = it % P::kPair;
        if (!CHECK || key < a.seq_k) {
          const char* kb = reinterpret_cast<const char*>(kbase);
          const uint32_t o1 = ((uint32_t)key * D + 8u * j) * 2u;
          ks.px1[n] = *reinterpret_cast<const bf16x8*>(kb + o1);
          ks.px2[n] = *reinterpret_cast<const bf16x8*>(kb + o1 + 32u * H16);
          if constexpr (CHECK) {
            const int64_t p = a.rotate_k ? key_pos(a, b, key) : -1;
            if (p >= 0) {
              load_cs(a, p, 8 * j, 8, ks.pc[n], ks.ps[n]);
              ks.prot[n] = true;
            }
          } else {
            load_cs(a, key, 8 * j, 8, ks.pc[n], ks.ps[n]);
          }
        }
      }
    }
  }
  if constexpr (P::kCopy > 0) {
#pragma unroll
    for (int n = 0; n < P::kCopyN; ++n) {
      const int it = t + n * NT;
      ks.cx[n] = z;
      if (fits(it, kKeys * P::kCopy, NT)) {
        const int key = k0 + it / P::kCopy, j = it % P::kCopy;
        if (!CHECK || key < a.seq_k)
          ks.cx[n] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kbase) +
                                                      ((uint32_t)key * D + kR + 8u * j) * 2u);
      }
    }
  }
  if constexpr (P::kInter > 0) {
#pragma unroll
    for (int n = 0; n < P::kInterN; ++n) {
      const int it = t + n * NT;
      ks.ix[n] = z;
      ks.irot[n] = false;
      if (fits(it, kKeys * P::kInter, NT)) {
        const int key = k0 + it / P::kInter, j = it % P::kInter;
        if (!CHECK || key < a.seq_k) {
          ks.ix[n] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kbase) +
                                                      ((uint32_t)key * D + 8u * j) * 2u);
          if (8 * j < R) {
            if constexpr (CHECK) {
              const int64_t p = a.rotate_k ? key_pos(a, b, key) : -1;
              if (p >= 0) {
                load_cs(a, p, 4 * j, 4, ks.ic[n], ks.is[n]);
                ks.irot[n] = true;
              }
            } else {
              load_cs(a, key, 4 * j, 4, ks.ic[n], ks.is[n]);
            }
          }
        }
      }
    }
  }
}

// Rotate the fetched K items with the cos/sin fetched beside them and write
// them to the K tile of buffer `buf`. CHECK false (the fetch's form): every
// item is rotated, with no branches.
template <int D, int PAIR, int H16, int NT = kBlock, bool CHECK = true>
__device__ __forceinline__ void stage_k(const AttnArgs& a, int t, KStage<D, PAIR, H16, NT>& ks,
                                        __bf16* lds, int buf) {
  using P = KPlan<D, PAIR, H16, NT>;
  constexpr int kR = 32 * H16;   // split-half: the rotated dims, fixed by the instantiation
  if constexpr (P::kPair > 0) {
#pragma unroll
    for (int n = 0; n < P::kPairN; ++n) {
      const int it = t + n * NT;
      if (fits(it, kKeys * P::kPair, NT)) {
        const int kk = it / P::kPair, j = it % P::kPair;
        if (!CHECK || ks.prot[n]) rotate_split8(ks.px1[n], ks.px2[n], ks.pc[n], ks.ps[n]);
        *reinterpret_cast<bf16x8*>(&lds[k_lds<D>(buf, kk, 8 * j)]) = ks.px1[n];
        *reinterpret_cast<bf16x8*>(&lds[k_lds<D>(buf, kk, 16 * H16 + 8 * j)]) = ks.px2[n];
      }
    }
  }
  if constexpr (P::kCopy > 0) {
#pragma unroll
    for (int n = 0; n < P::kCopyN; ++n) {
      const int it = t + n * NT;
      if (fits(it, kKeys * P::kCopy, NT)) {
        const int kk = it / P::kCopy, j = it % P::kCopy;
        *reinterpret_cast<bf16x8*>(&lds[k_lds<D>(buf, kk, kR + 8 * j)]) = ks.cx[n];
      }
    }
  }
  if constexpr (P::kInter > 0) {
#pragma unroll
    for (int n = 0; n < P::kInterN; ++n) {
      const int it = t + n * NT;
      if (fits(it, kKeys * P::kInter, NT)) {
        const int kk = it / P::kInter, j = it % P::kInter;
        // (unchecked: every key is rotated, and exactly the chunks inside R)
        if (CHECK ? ks.irot[n] : 8 * j < 2 * a.half) rotate_inter8(ks.ix[n], ks.ic[n], ks.is[n]);
        *reinterpret_cast<bf16x8*>(&lds[k_lds<D>(buf, kk, 8 * j)]) = ks.ix[n];
      }
    }
  }
}

template <int D, int NT = kBlock, bool CHECK = true>
__device__ __forceinline__ void fetch_v(const AttnArgs& a, const __bf16* vbase, int k0, int t,
                                        VStage<D, NT>& vs) {
#pragma unroll
  for (int n = 0; n < v_items_max<D, NT>(); ++n) {
    const int it = t + n * NT;
    if (fits(it, v_items<D>(), NT)) {
      const VItem vi = v_item(it);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * vi.k4 + r;
        u32x4 z = {};
        vs.x[n][r] = !CHECK || key < a.seq_k
                         ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(vbase) +
                                                           ((uint32_t)key * D + vi.c * 8u) * 2u)
                         : z;
      }
    }
  }
}

// V tile, transposed: 4 keys x 8 dims per item, 8-byte LDS writes. Word w
// of a row holds dims 2w (low half) and 2w + 1 (high half); a byte permute
// pairs the same half of two rows.
template <int D, int NT = kBlock>
__device__ __forceinline__ void stage_v(int t, const VStage<D, NT>& vs, __bf16* lds, int buf) {
  constexpr uint32_t kLow = 0x05040100u, kHigh = 0x07060302u;
#pragma unroll
  for (int n = 0; n < v_items_max<D, NT>(); ++n) {
    const int it = t + n * NT;
    if (fits(it, v_items<D>(), NT)) {
      const VItem vi = v_item(it);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 even = {__builtin_amdgcn_perm(vs.x[n][1][w], vs.x[n][0][w], kLow),
                            __builtin_amdgcn_perm(vs.x[n][3][w], vs.x[n][2][w], kLow)};
        const u32x2 odd = {__builtin_amdgcn_perm(vs.x[n][1][w], vs.x[n][0][w], kHigh),
                           __builtin_amdgcn_perm(vs.x[n][3][w], vs.x[n][2][w], kHigh)};
        const int slot = v_slot(4 * vi.k4);  // the quad stays contiguous
        *reinterpret_cast<u32x2*>(&lds[v_lds<D>(buf, vi.c * 8 + 2 * w, slot)]) = even;
        *reinterpret_cast<u32x2*>(&lds[v_lds<D>(buf, vi.c * 8 + 2 * w + 1, slot)]) = odd;
      }
    }
  }
}
#endif

// ---------------------------------------------------------------- kernel
template <bool B> struct Bool {
  static constexpr bool value = B;
};

// H16: split-half pairs, (R/2)/16 (the register distance between the two
// chunks of a pair; a compile-time constant so the registers stay registers);
// 0 for interleaved pairs.
template <int D, int PAIR, int H16, bool KR, int G>
__global__ void __launch_bounds__(kBlock, 2) rope_attention_kernel(AttnArgs a) {
  static_assert(G == 1 || G == 2 || G == 4, "1, 2 or 4 wave groups");
#if defined(__HIP_DEVICE_COMPILE__)
  // K staging: rotated while staged (KR, the fused form), or copied as it
  // arrives (K already rotated; the copy-only plan keeps no cos/sin
  // registers for it)
  constexpr int KP = KR ? PAIR : kSplitHalf;
  constexpr int KH = KR ? H16 : 0;
  // G wave groups (small grids; 1 otherwise): the groups hold the same
  // 256 / G rows and take turns on the key tiles (group g: tiles g, g + G,
  // ...), each staging its own tiles into its own double buffer (NT lanes
  // stage a tile); their softmax states merge at the end. The chain of
  // tiles a workgroup walks is divided by G.
  constexpr int NT = kBlock / G;
  constexpr int kStride = G;  // tiles between a group's steps
  extern __shared__ __bf16 lds[];
  const Work wk = work_of(a, blockIdx.x);
  const int q_tile = wk.q_tile, b = wk.b;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const WaveRole role = wave_role(a, wk, wave, G);
  const int h = role.h;
  // the same for every wave (readfirstlane: the compiler keeps it scalar)
  const int hk = __builtin_amdgcn_readfirstlane(h / (a.n_heads_q / a.n_heads_k));
  const int hs = lane >> 5;  // which half of the wave: k slots 0-7 or 8-15
  const int qi = role.row0 + (lane & 31);  // this lane's query row
  constexpr int kSteps = D / 16;  // k-steps of S^T over the head dim
  const int R = 2 * a.half;
  const int grp = G == 1 ? 0 : wave / (kWaves / G);  // wave group
  const int ts = t - grp * NT;          // lane among the group's stagers
  // LDS buffer of a group's step: parity of the step, then the group
  auto buf_of = [&](int step) { return G * (step & 1) + grp; };

  const int n_tiles = key_tiles(a, q_tile);
  const __bf16* kbase = a.k + row_of<D>(a, b, hk, a.n_heads_k, a.seq_k, 0);
  const __bf16* vbase = a.v + row_of<D>(a, b, hk, a.n_heads_k, a.seq_k, 0);

  // ---- Q: this lane's half of its query row, rotated, as B operands.
  bf16x8 qreg[kSteps];
  {
    const bool q_ok = qi < a.seq_q;
    const __bf16* qrow = a.q + row_of<D>(a, b, h, a.n_heads_q, a.seq_q, q_ok ? qi : 0);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      bf16x8 z = {};
      qreg[s] = q_ok ? *reinterpret_cast<const bf16x8*>(qrow + s * 16 + hs * 8) : z;
    }
    const int64_t p = (q_ok && a.rotate) ? query_pos(a, b, qi) : -1;
    if (p >= 0) {
      float c[8], sn[8];
      if constexpr (PAIR == kSplitHalf) {
        // chunk s (dims s*16 + hs*8 .. +7, all < R/2 = 16*H16) pairs with
        // chunk s + H16 of this lane (dims + R/2)
#pragma unroll
        for (int s = 0; s < H16; ++s) {
          load_cs(a, p, s * 16 + hs * 8, 8, c, sn);
          rotate_split8(qreg[s], qreg[s + H16], c, sn);
        }
      } else {
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const int d = s * 16 + hs * 8;  // 4 interleaved pairs, freqs d/2 ..
          if (d < R) {
            load_cs(a, p, d / 2, 4, c, sn);
            rotate_inter8(qreg[s], c, sn);
          }
        }
      }
    }
  }

  // A negative scale: -Q with |scale|. Negating bf16 is exact and so is
  // negating every product and partial sum, so the scores are exactly -S.
  if (a.negate_q) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qreg[s]) ^ 0x80008000u);
  }

  // ---- running softmax state and O^T accumulators (D/32 tiles of 32 dims)
  float m_run = -__builtin_inff(), l_run = 0.0f;
  floatx16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (floatx16){};

  const int causal_shift = a.seq_k - a.seq_q;
  // every key is rotated at its own index (checked once: uniform)
  const bool plain_keys = !KR || (a.k_pos == nullptr && a.seq_k <= a.table_rows);
  // this wave's query rows, for the masking decisions (uniform per wave)
  const int wq_first = role.row0;
  const int wq_last = imin(wq_first + 31, a.seq_q - 1);

  // Tile kt sits in LDS buffer kt & 1 while its products run. The raw K and
  // V rows (and key positions) of tile kt + 1 are fetched into registers
  // while tile kt is worked on, and staged into the other buffer after its
  // products: that buffer's last readers (tile kt - 1) all passed the
  // previous barrier, and its next readers wait for this iteration's
  // barrier. The fetched registers never cross an iteration.
  if (grp < n_tiles) {  // tile grp (tile 0 with one group)
    KStage<D, KP, KH, NT> ks0;
    VStage<D, NT> vs0;
    fetch_k<D, KP, KH, NT>(a, b, kbase, grp * kKeys, ts, ks0);
    fetch_v<D, NT>(a, vbase, grp * kKeys, ts, vs0);
    stage_k<D, KP, KH, NT>(a, ts, ks0, lds, buf_of(0));
    stage_v<D, NT>(ts, vs0, lds, buf_of(0));
  }
  __syncthreads();
  // a wave whose rows all lie past Sq computes nothing (it still stages)
  const bool live = wq_first < a.seq_q;
  const float c = a.scale_log2e;
  // every wave runs the same number of steps (the barriers are shared)
  const int n_steps = (n_tiles + G - 1) / G;
  struct Step {
    int kt, k0;
    bool more, work, edge, fast;
  };
  auto step_of = [&](int step) {
    Step r;
    r.kt = step * kStride + grp;  // this group's tile
    r.k0 = r.kt * kKeys;
    r.more = r.kt + kStride < n_tiles;
    // a tile wholly after this wave's causal diagonal adds nothing: its
    // scores are all masked, so the running max, sum and output stay as
    // they are (the wave still stages the next tile and meets the barriers)
    r.work = live && r.kt < n_tiles && (!a.causal || r.k0 <= wq_last + causal_shift);
    // masks only where the tile reaches past Sk or this wave's diagonal
    r.edge = r.k0 + kKeys > a.seq_k ||
             (a.causal && r.k0 + kKeys - 1 > wq_first + causal_shift);
    // The common step: this wave has keys to take, none masked, the next
    // tile lies wholly inside Sk and (when K is rotated here) its keys sit
    // at positions 0 .. Sk - 1 of the table. Each condition, once false,
    // stays false for the later steps, so the common steps come first.
    r.fast = r.work && !r.edge && r.more && r.k0 + (kStride + 1) * kKeys <= a.seq_k && plain_keys;
    return r;
  };
  // One step over a tile. FAST: the common step, with no branches (but the
  // rare output rescale), so the compiler can place the vector work of the
  // softmax, the fetch and the rotation between the matrix instructions. It
  // runs in a loop of its own, so neither loop holds the other's registers.
  auto run_step = [&](int step, auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const Step sp = step_of(step);
    const int k0 = sp.k0;
    const bool more = sp.more, work = sp.work, edge = sp.edge;
    const int buf = buf_of(step);

    // S^T = K Q^T for one 32-key half of the tile: the half's K fragments are
    // read from LDS, then its chain of products. Lane slot j holds key
    // half*32 + 8*(j/4) + 4*hs + j%4 of its query row.
    auto scores = [&](int half) {
      bf16x8 kf[kSteps];
#pragma unroll
      for (int st = 0; st < kSteps; ++st)
        kf[st] = *reinterpret_cast<const bf16x8*>(
            &lds[k_lds<D>(buf, half * 32 + (lane & 31), st * 16 + hs * 8)]);
      // keep every read of the half ahead of its first product (left to
      // itself the compiler interleaves them, one LDS round trip per product)
      __builtin_amdgcn_sched_barrier(0);
      floatx16 sh = {};
#pragma unroll
      for (int st = 0; st < kSteps; ++st)
        sh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qreg[st], sh, 0, 0, 0);
      return sh;
    };
    auto mask = [&](floatx16& sh, int half) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + half * 32 + 8 * (j / 4) + 4 * hs + (j % 4);
        const bool vis = key < a.seq_k && (!a.causal || key <= qi + causal_shift);
        if (!vis) sh[j] = -__builtin_inff();
      }
    };
    // Online softmax over one 32-key half, in base 2 on the raw scores: each
    // weight is exp2(s * c - m * c), one fused multiply-add, with m the
    // row's reference max. m moves to the half's max only when that passes
    // it by more than 8 in the base-2 exponent, so weights stay below 2^8
    // and the output is rarely rescaled. Returns the rescale factor; the
    // weights come back as bf16, two 16-key k-steps.
    auto softmax = [&](floatx16& sh, bf16x8* pb) {
      float m_t = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 16; ++j) m_t = fmaxf(m_t, sh[j]);
      m_t = wave_max32(m_t);
      // false when both are -inf (a row with no visible key so far)
      const bool move = (m_t - m_run) * c > 8.0f;
      const float m_new = move ? m_t : m_run;
      const float alpha = move ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
      // a row with no visible key so far (m_new = -inf) keeps weights 0
      const float mc = m_new == -__builtin_inff() ? 0.0f : m_new * c;
      float l_t = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[j], c, -mc));
        sh[j] = pj;
        l_t += pj;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[u][i] = from_f32<__bf16>(sh[8 * u + i]);
      l_t = wave_sum32(l_t);
      l_run = l_run * alpha + l_t;
      m_run = m_new;
      return alpha;
    };
    // rescale the output only when some lane's reference max moved
    auto rescale = [&](float alpha) {
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[i][j] *= alpha;
      }
    };
    // O^T += V^T P^T over one half: k-step u covers keys half*32 + 16u ..
    // +15, the lane's weights pb[u] (slots 8u .. 8u+7 of its scores, keys
    // 16u + 8*(i/4) + 4*hs + i%4), against V^T slots half*32 + 16u + 8hs ..
    // +7, which hold the same keys in that order. Each step's V^T fragments
    // are read before its products.
    auto output = [&](int half, const bf16x8* pb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int slot = half * 32 + 16 * u + 8 * hs;
        u32x4 va[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int dim = dt * 32 + (lane & 31);
          va[dt] = *reinterpret_cast<const u32x4*>(&lds[v_lds<D>(buf, dim, slot)]);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, va[dt]), pb[u], acc[dt], 0, 0, 0);
      }
    };

    // The two halves are software-pipelined: the second half's score
    // products run beside the first half's softmax, and the first half's
    // output products beside the second half's softmax. The next tile's
    // fetch is issued between the two, after the score products, and its
    // rotation runs beside the second half's output products.
    floatx16 s0, s1;
    bf16x8 p0[2], p1[2];
    KStage<D, KP, KH, NT> ks;
    VStage<D, NT> vs;
    const int k_next = k0 + kStride * kKeys;
    if constexpr (FAST) {
      s0 = scores(0);
      s1 = scores(1);
      rescale(softmax(s0, p0));
      fetch_k<D, KP, KH, NT, false>(a, b, kbase, k_next, ts, ks);
      fetch_v<D, NT, false>(a, vbase, k_next, ts, vs);
      output(0, p0);
      rescale(softmax(s1, p1));
      output(1, p1);
      stage_k<D, KP, KH, NT, false>(a, ts, ks, lds, buf_of(step + 1));
      // ask the scheduler for the next tile's rotation between the second
      // half's output products: per 16-key step, its V^T reads, then each
      // product followed by a share of the rotation's vector instructions
      // (a scheduling hint; the instructions and their results are the same)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x100, D / 32, 0);  // LDS reads
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);   // VALU
        }
      }
      stage_v<D, NT>(ts, vs, lds, buf_of(step + 1));
    } else {
      if (work) {
        s0 = scores(0);
        if (edge) mask(s0, 0);
        s1 = scores(1);
        rescale(softmax(s0, p0));
        if (edge) mask(s1, 1);
      }
      if (more) {
        fetch_k<D, KP, KH, NT>(a, b, kbase, k_next, ts, ks);
        fetch_v<D, NT>(a, vbase, k_next, ts, vs);
      }
      if (work) {
        output(0, p0);
        rescale(softmax(s1, p1));
        output(1, p1);
      }
      if (more) {
        stage_k<D, KP, KH, NT>(a, ts, ks, lds, buf_of(step + 1));
        stage_v<D, NT>(ts, vs, lds, buf_of(step + 1));
      }
    }
    __syncthreads();
  };
  int n_fast = 0;
  while (n_fast < n_steps && step_of(n_fast).fast) ++n_fast;
  for (int step = 0; step < n_fast; ++step) run_step(step, Bool<true>{});
  for (int step = n_fast; step < n_steps; ++step) run_step(step, Bool<false>{});

  if constexpr (G > 1) {
    // Merge: groups 1 .. G-1 leave their running max, sum and output in LDS
    // (every tile read ended at the last barrier); group 0 takes them for
    // the same rows (the same lane of waves w + kWaves/G, ...), rescales
    // every state to the largest reference max and writes O. Per lane: m, l,
    // then the D/32 x 16 accumulators.
    constexpr int kState = 2 + 16 * (D / 32);
    constexpr int kWg = kWaves / G;  // waves per group
    float* const base = reinterpret_cast<float*>(lds);
    auto slot = [&](int g) { return base + (((g - 1) * kWg + wave % kWg) * 64 + lane) * kState; };
    if (grp > 0) {
      float* st = slot(grp);
      st[0] = m_run;
      st[1] = l_run;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) st[2 + 16 * i + j] = acc[i][j];
    }
    __syncthreads();
    if (grp > 0) return;
    float m = m_run;
#pragma unroll
    for (int g = 1; g < G; ++g) m = fmaxf(m, slot(g)[0]);
    // a row with no visible key in any group keeps zeros
    const bool none = m == -__builtin_inff();
    const float a0 = none ? 0.0f : __builtin_amdgcn_exp2f((m_run - m) * c);
    l_run = l_run * a0;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[i][j] = acc[i][j] * a0;
#pragma unroll
    for (int g = 1; g < G; ++g) {
      const float* st = slot(g);
      const float ag = none ? 0.0f : __builtin_amdgcn_exp2f((st[0] - m) * c);
      l_run = l_run + st[1] * ag;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = acc[i][j] + st[2 + 16 * i + j] * ag;
    }
  }

  // ---- O = acc / l: lane holds dims dt*32 + 8*(j/4) + 4*hs + j%4 of its row
  if (qi < a.seq_q) {
    __bf16* orow = a.o + row_of<D>(a, b, h, a.n_heads_q, a.seq_q, qi);
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = from_f32<__bf16>(acc[dt][4 * g + i] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * g + 4 * hs) = out;
      }
  }
#endif
}

}  // namespace attn
}  // namespace rope

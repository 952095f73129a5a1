// attn_bounds.hip -- test harness: checks, on the host, every global and LDS
// access of the fused attention kernel against its buffers.
//
// The kernel (rope_attention.hpp) runs on matrix cores and cannot execute on
// the host, so this walks its loops instead: every workgroup, lane and key
// tile of the planned grid, forming each address with the kernel's own index
// functions (row_of, k_lds, v_lds, query_pos, key_pos, key_tiles, KItems) and
// counting any that falls outside the exact extent of its buffer.
//
// usage: attn_bounds B Hq Hk Sq Sk D R pairing causal table_rows qpos kpos
//   (qpos / kpos: 0 = no index, 1 = an index of Sq / Sk entries per batch)
// prints "plan <status>" then "violations <n>" and "accesses <n>".
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "librope.h"
#include "rope_attn_plan.hpp"

using namespace rope;
using namespace rope::attn;

namespace {

struct Checker {
  long long violations = 0, accesses = 0;
  // LDS cells written / read by the first key tile of the first workgroup
  // (the staging pattern is the same for every tile and workgroup)
  std::vector<int> written, read;
  bool track = false;
  void wrote(int first, int count) {
    if (track)
      for (int i = first; i < first + count; ++i)
        if (i >= 0 && i < (int)written.size()) ++written[i];
  }
  void reads(int first, int count) {
    if (track)
      for (int i = first; i < first + count; ++i)
        if (i >= 0 && i < (int)read.size()) ++read[i];
  }
  void check(long long first, long long count, long long extent, const char* what) {
    ++accesses;
    if (first < 0 || first + count > extent) {
      if (violations < 10) fprintf(stderr, "out of bounds: %s [%lld, %lld) of %lld\n", what,
                                   first, first + count, extent);
      ++violations;
    }
  }
};

template <int D, int PAIR>
void walk(const AttnPlan& pl, int64_t q_elems, int64_t kv_elems, int64_t table_elems,
          int64_t qpos_elems, int64_t kpos_elems, Checker& ck) {
  const AttnArgs& a = pl.a;
  const int lds_elems = lds_bytes<D>() / 2;
  const int R = 2 * a.half;
  const int per_key = KItems<D, PAIR>::per_key(a);
  const int rchunks = R / 8;
  ck.written.assign(lds_elems, 0);
  ck.read.assign(lds_elems, 0);
  // positions through the kernel's own functions, with the index reads checked
  auto qpos = [&](int b, int i) {
    if (a.q_pos) ck.check((int64_t)b * a.q_pos_bs + i, 1, qpos_elems, "q_pos");
    return query_pos(a, b, i);
  };
  auto kpos = [&](int b, int j) {
    if (a.k_pos) ck.check((int64_t)b * a.k_pos_bs + j, 1, kpos_elems, "k_pos");
    return key_pos(a, b, j);
  };
  // the workgroup -> work map is a bijection onto (batch, head, query tile)
  std::vector<char> seen((size_t)pl.grid, 0);
  for (int64_t blk = 0; blk < pl.grid; ++blk) {
    const Work wk = work_of(a, blk);
    const bool inside = wk.b >= 0 && wk.b < a.batch && wk.h >= 0 && wk.h < a.n_heads_q &&
                        wk.q_tile >= 0 && wk.q_tile < a.q_tiles;
    ck.check(inside ? 0 : -1, 1, 1, "work item outside the problem");
    if (inside) {
      const int64_t id = ((int64_t)wk.b * a.n_heads_q + wk.h) * a.q_tiles + wk.q_tile;
      ck.check(seen[id]++ ? -1 : 0, 1, 1, "work item given twice");
    }
  }
  for (int64_t blk = 0; blk < pl.grid; ++blk) {
    const Work wk = work_of(a, blk);
    const int q_tile = wk.q_tile, h = wk.h, b = wk.b;
    const int hk = h / (a.n_heads_q / a.n_heads_k);
    const int n_tiles = key_tiles(a, q_tile);
    const int64_t kbase = row_of<D>(a, b, hk, a.n_heads_k, a.seq_k, 0);
    for (int t = 0; t < kBlock; ++t) {
      const int lane = t & 63, wave = t >> 6, hs = lane >> 5;
      const int qi = q_tile * kQueries + wave * 32 + (lane & 31);
      const bool q_ok = qi < a.seq_q;
      const int64_t qrow = row_of<D>(a, b, h, a.n_heads_q, a.seq_q, q_ok ? qi : 0);
      for (int s = 0; s < D / 16; ++s)
        if (q_ok) ck.check(qrow + s * 16 + hs * 8, 8, q_elems, "q load");
      const int64_t p = (q_ok && a.rotate) ? qpos(b, qi) : -1;
      if (p >= 0) {
        if (PAIR == kSplitHalf) {
          for (int s = 0; s < a.half / 16; ++s) {
            ck.check(p * a.half + s * 16 + hs * 8, 8, table_elems, "q cos/sin");
            if (s + a.half / 16 >= D / 16) ck.check(0, 1, 0, "q pair register");
          }
        } else {
          for (int s = 0; s < D / 16; ++s)
            if (s * 16 + hs * 8 < R) ck.check(p * a.half + (s * 16 + hs * 8) / 2, 4, table_elems,
                                              "q cos/sin");
        }
      }
      for (int kt = 0; kt < n_tiles; ++kt) {
        const int k0 = kt * kKeys;
        ck.track = blk == 0 && kt == 0;
        for (int it = t; it < kKeys * per_key; it += kBlock) {
          const int kk = it / per_key, item = it - kk * per_key;
          const int key = k0 + kk;
          const bool ok = key < a.seq_k;
          const int64_t krow = kbase + (int64_t)(ok ? key : 0) * D;
          const int64_t kp = (ok && a.rotate) ? kpos(b, key) : -1;
          if (PAIR == kSplitHalf) {
            const int npair = rchunks / 2;
            if (item < npair) {
              const int d1 = item * 8, d2 = a.half + item * 8;
              if (ok) {
                ck.check(krow + d1, 8, kv_elems, "k load");
                ck.check(krow + d2, 8, kv_elems, "k load");
              }
              if (kp >= 0) ck.check(kp * a.half + d1, 8, table_elems, "k cos/sin");
              ck.check(k_lds<D>(kk, d1), 8, k_lds_elems<D>(), "k lds");
              ck.check(k_lds<D>(kk, d2), 8, k_lds_elems<D>(), "k lds");
              ck.wrote(k_lds<D>(kk, d1), 8);
              ck.wrote(k_lds<D>(kk, d2), 8);
            } else {
              const int d = R + (item - npair) * 8;
              if (ok) ck.check(krow + d, 8, kv_elems, "k load");
              ck.check(k_lds<D>(kk, d), 8, k_lds_elems<D>(), "k lds");
              ck.wrote(k_lds<D>(kk, d), 8);
            }
          } else {
            const int d = item * 8;
            if (ok) ck.check(krow + d, 8, kv_elems, "k load");
            if (item < rchunks && kp >= 0)
              ck.check(kp * a.half + d / 2, 4, table_elems, "k cos/sin");
            ck.check(k_lds<D>(kk, d), 8, k_lds_elems<D>(), "k lds");
            ck.wrote(k_lds<D>(kk, d), 8);
          }
        }
        for (int it = t; it < v_items<D>(); it += kBlock) {
          const VItem vi = v_item(it);
          for (int r = 0; r < 4; ++r) {
            const int key = k0 + 4 * vi.k4 + r;
            if (key < a.seq_k)
              ck.check(kbase + (int64_t)key * D + vi.c * 8, 8, kv_elems, "v load");
          }
          for (int i = 0; i < 8; ++i) {
            const int off = v_lds<D>(vi.c * 8 + i, 4 * vi.k4);
            ck.check(off, 4, lds_elems, "v lds");
            ck.check(off % 4 == 0 ? 0 : -1, 1, 1, "v lds write not 8-byte aligned");
            ck.wrote(off, 4);
            if (off < k_lds_elems<D>()) ck.check(0, 1, 0, "v lds inside the k tile");
          }
        }
        for (int half = 0; half < 2; ++half)
          for (int st = 0; st < D / 16; ++st)
          {
            const int off = k_lds<D>(half * 32 + (lane & 31), st * 16 + hs * 8);
            ck.check(off, 8, k_lds_elems<D>(), "k lds read");
            ck.reads(off, 8);
          }
        for (int half = 0; half < 2; ++half)
          for (int u = 0; u < 2; ++u) {
            const int kb = half * 32 + 16 * u + 4 * hs;
            for (int dt = 0; dt < D / 32; ++dt) {
              const int dim = dt * 32 + (lane & 31);
              ck.check(v_lds<D>(dim, kb), 4, lds_elems, "v lds read");
              ck.check(v_lds<D>(dim, kb + 8), 4, lds_elems, "v lds read");
              ck.reads(v_lds<D>(dim, kb), 4);
              ck.reads(v_lds<D>(dim, kb + 8), 4);
              if (kb + 8 + 4 > kKeys) ck.check(0, 1, 0, "v key beyond the tile");
            }
          }
      }
      if (q_ok) {
        const int64_t orow = row_of<D>(a, b, h, a.n_heads_q, a.seq_q, qi);
        for (int dt = 0; dt < D / 32; ++dt)
          for (int g = 0; g < 4; ++g) ck.check(orow + dt * 32 + 8 * g + 4 * hs, 4, q_elems, "o store");
      }
    }
  }
  // every cell is written at most once per tile, and every cell read was written
  ck.track = false;
  for (int i = 0; i < lds_elems; ++i) {
    ck.check(ck.written[i] > 1 ? -1 : 0, 1, 1, "lds cell written twice");
    if (ck.read[i] > 0) ck.check(ck.written[i] == 1 ? 0 : -1, 1, 1, "lds cell read, never written");
  }
}

// the first entries hold the positions at the edges of the table: the last
// row, one past it (passes through) and -1 (passes through)
void edge_positions(std::vector<int32_t>& p, int64_t rows) {
  const int32_t e[3] = {(int32_t)rows - 1, (int32_t)rows, -1};
  for (size_t i = 0; i < 3 && i < p.size(); ++i) p[i] = e[i];
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 13) {
    fprintf(stderr, "usage: attn_bounds B Hq Hk Sq Sk D R pairing causal table_rows qpos kpos\n");
    return 2;
  }
  long long v[12];
  for (int i = 0; i < 12; ++i) v[i] = atoll(argv[i + 1]);
  rope_attn_desc_t d{};
  d.batch = v[0];
  d.n_heads_q = v[1];
  d.n_heads_k = v[2];
  d.seq_len_q = v[3];
  d.seq_len_k = v[4];
  d.head_dim = v[5];
  d.rotary_dim = v[6];
  d.pairing = (int32_t)v[7];
  d.causal = (int32_t)v[8];
  d.table_rows = v[9];
  d.dtype = ROPE_BF16;
  d.rotate = 1;
  // fake, 16-byte aligned, disjoint addresses: the walk never dereferences them
  const uintptr_t base = (uintptr_t)1 << 40;
  const int64_t q_elems = d.batch * d.n_heads_q * d.seq_len_q * d.head_dim;
  const int64_t kv_elems = d.batch * d.n_heads_k * d.seq_len_k * d.head_dim;
  const int64_t table_elems = d.table_rows * (d.rotary_dim / 2);
  d.q = (const void*)base;
  d.k = (const void*)(base + ((uintptr_t)1 << 36));
  d.v = (const void*)(base + ((uintptr_t)2 << 36));
  d.o = (void*)(base + ((uintptr_t)3 << 36));
  d.cos = (const float*)(base + ((uintptr_t)4 << 36));
  d.sin = (const float*)(base + ((uintptr_t)5 << 36));
  // index arrays are read through the kernel's position functions: real ones
  std::vector<int32_t> qp, kp;
  if (v[10]) {
    qp.resize((size_t)(d.batch * d.seq_len_q) + 1);
    for (size_t i = 0; i < qp.size(); ++i) qp[i] = (int32_t)((i * 7) % (d.table_rows + 3)) - 1;
    edge_positions(qp, d.table_rows);
    d.q_pos = qp.data();
    d.q_pos_batch_stride = d.seq_len_q;
  }
  if (v[11]) {
    kp.resize((size_t)(d.batch * d.seq_len_k) + 1);
    for (size_t i = 0; i < kp.size(); ++i) kp[i] = (int32_t)((i * 5) % (d.table_rows + 3)) - 1;
    edge_positions(kp, d.table_rows);
    d.k_pos = kp.data();
    d.k_pos_batch_stride = d.seq_len_k;
  }
  AttnPlan pl;
  const rope_status_t st = make_attn_plan(&d, &pl);
  printf("plan %d\n", (int)st);
  if (st != ROPE_OK || pl.empty) {
    printf("violations 0\naccesses 0\n");
    return 0;
  }
  Checker ck;
  const int64_t qpos_elems = d.batch * d.seq_len_q, kpos_elems = d.batch * d.seq_len_k;
  if (pl.head_dim == 64) {
    if (pl.pairing == ROPE_SPLIT_HALF)
      walk<64, kSplitHalf>(pl, q_elems, kv_elems, table_elems, qpos_elems, kpos_elems, ck);
    else
      walk<64, kInterleaved>(pl, q_elems, kv_elems, table_elems, qpos_elems, kpos_elems, ck);
  } else {
    if (pl.pairing == ROPE_SPLIT_HALF)
      walk<128, kSplitHalf>(pl, q_elems, kv_elems, table_elems, qpos_elems, kpos_elems, ck);
    else
      walk<128, kInterleaved>(pl, q_elems, kv_elems, table_elems, qpos_elems, kpos_elems, ck);
  }
  printf("violations %lld\naccesses %lld\n", ck.violations, ck.accesses);
  return 0;
}

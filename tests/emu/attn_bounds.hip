// attn_bounds.hip -- test harness: checks, on the host, every global and LDS
// access of the fused attention kernel against its buffers.
//
// The kernel (rope_attention.hpp) runs on matrix cores and cannot execute on
// the host, so this walks its loops instead: every workgroup, lane and key
// tile of the planned grid, forming each address with the kernel's own index
// functions (work_of, wave_role, row_of, k_lds, v_lds, v_slot, query_pos,
// key_pos, key_tiles, KPlan) and counting any that falls outside the exact extent of
// its buffer. The tile pipeline is simulated phase by phase, a phase being
// the work between two barriers (stage the first tile; then per step, the
// reads of the step's buffer and the staging of the next tile into the
// other one; with G wave groups, each group does so on its own tiles and
// buffers): each staging write must land in its tile's buffer, no LDS cell
// may be written by two lanes or both read and written in one phase, and
// every cell read for tile kt must hold tile kt. With G > 1, the final merge
// (the other groups' softmax states through LDS) is checked the same way.
//
// usage: attn_bounds B Hq Hk Sq Sk D R pairing causal table_rows qpos kpos [k_rotated]
//   (qpos / kpos: 0 = no index, 1 = an index of Sq / Sk entries per batch;
//   k_rotated: 1 = K arrives rotated and is staged by the copy-only plan)
// prints "plan <status>" then "violations <n>" and "accesses <n>".
#include <algorithm>
#include <type_traits>
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
  void check(long long first, long long count, long long extent, const char* what) {
    ++accesses;
    if (first < 0 || first + count > extent) {
      if (violations < 10) fprintf(stderr, "out of bounds: %s [%lld, %lld) of %lld\n", what,
                                   first, first + count, extent);
      ++violations;
    }
  }
  void fail(bool bad, const char* what) { check(bad ? -1 : 0, 1, 1, what); }
};

// LDS cell ownership of one workgroup: the tile whose staging last wrote
// each cell, and the lane that wrote it in the current staging phase.
struct LdsModel {
  std::vector<int> tile, writer, wrote_in, read_in;
  explicit LdsModel(int n) : tile(n, -1), writer(n, -1), wrote_in(n, -1), read_in(n, -1) {}
};

template <int D, int PAIR, int H16, bool KR, int G>
void walk(const AttnPlan& pl, int64_t q_elems, int64_t kv_elems, int64_t table_elems,
          int64_t qpos_elems, int64_t kpos_elems, Checker& ck) {
  const AttnArgs& a = pl.a;
  // the kernel's choice of staging lanes and tile stride, and its LDS
  constexpr int NT = kBlock / G;
  constexpr int kStride = G;
  constexpr int kGroups = G;
  constexpr bool SPLIT = G > 1;
  ck.fail(G != a.groups, "instantiation matches the wave groups");
  ck.fail(SPLIT && D != 64, "wave groups only at head dim 64");
  ck.fail(pl.lds != lds_bytes_groups<D>(G), "plan's LDS size");
  ck.fail(pl.lds > 160 * 1024, "the workgroup's LDS fits a compute unit");
  // the kernel forms K/V and cos/sin addresses as 32-bit byte offsets from
  // a head's (or the table's) base: every offset it can form must fit
  ck.fail((int64_t)a.seq_k * D * 2 > ((int64_t)1 << 32) - 16, "K/V head rows under 4 GiB");
  ck.fail(a.rotate && a.table_rows * a.half * 4 > ((int64_t)1 << 32) - 16,
          "cos/sin table under 4 GiB");
  const int lds_elems = (int)(pl.lds / 2);
  const int R = 2 * a.half;
  // K staging: the kernel's plan for this instantiation (rotated while
  // staged, or the copy-only plan when K arrives rotated)
  using P = KPlan<D, KR ? PAIR : kSplitHalf, KR ? H16 : 0, NT>;
  constexpr int kRK = KR ? 32 * H16 : 0;  // split-half: dims the pair items cover
  ck.fail(KR != (a.rotate_k != 0) && a.rotate, "instantiation matches rotate_k");
  // the instantiation's item classes cover each key's D dims exactly once
  ck.fail(PAIR == kSplitHalf && R != 32 * H16, "split-half R is 32 H16");
  ck.fail(16 * P::kPair + 8 * P::kCopy + 8 * P::kInter != D, "items cover the head dim");
  auto qpos = [&](int b, int i) {
    if (a.q_pos) ck.check((int64_t)b * a.q_pos_bs + i, 1, qpos_elems, "q_pos");
    return query_pos(a, b, i);
  };
  auto kpos = [&](int b, int j) {
    if (a.k_pos) ck.check((int64_t)b * a.k_pos_bs + j, 1, kpos_elems, "k_pos");
    return key_pos(a, b, j);
  };
  // the workgroup -> work map is a bijection onto (batch, head group, query tile)
  std::vector<char> seen((size_t)pl.grid, 0);
  for (int64_t blk = 0; blk < pl.grid; ++blk) {
    const Work wk = work_of(a, blk);
    const bool inside = wk.b >= 0 && wk.b < a.batch && wk.hg >= 0 && wk.hg < a.head_groups &&
                        wk.q_tile >= 0 && wk.q_tile < a.q_tiles;
    ck.fail(!inside, "work item outside the problem");
    if (inside) {
      const int64_t id = ((int64_t)wk.b * a.head_groups + wk.hg) * a.q_tiles + wk.q_tile;
      ck.fail(seen[id]++ != 0, "work item given twice");
    }
  }
  // every (batch, head, row) is some wave's row exactly once
  ck.fail((int64_t)a.head_groups * a.hw != a.n_heads_q, "head groups cover the heads");
  ck.fail(a.rows * a.hw != kRows / kGroups || (int64_t)a.q_tiles * a.rows < a.seq_q,
          "rows cover Sq");
  ck.fail((a.n_heads_q / a.n_heads_k) % a.hw != 0, "a workgroup spans two K/V heads");
  // every (batch, query head, row < Sq) belongs to exactly one lane's query
  // (with G groups: to one lane of group 0, whose twins in the other groups
  // hold the same row)
  std::vector<char> owned((size_t)a.batch * a.n_heads_q * a.seq_q, 0);
  for (int64_t blk = 0; blk < pl.grid; ++blk) {
    const Work wk = work_of(a, blk);
    for (int wave = 0; wave < kWaves / kGroups; ++wave) {
      const WaveRole role = wave_role(a, wk, wave, G);
      for (int g = 1; g < G; ++g) {
        const WaveRole twin = wave_role(a, wk, wave + g * (kWaves / G), G);
        ck.fail(twin.h != role.h || twin.row0 != role.row0, "group twins share rows");
      }
      for (int r = 0; r < 32; ++r) {  // lanes r and r + 32 share row row0 + r
        const int qi = role.row0 + r;
        if (qi < a.seq_q && role.h >= 0 && role.h < a.n_heads_q)
          ck.fail(owned[((size_t)wk.b * a.n_heads_q + role.h) * a.seq_q + qi]++ != 0,
                  "query row owned twice");
      }
    }
  }
  for (char c : owned) ck.fail(c != 1, "query row owned by no lane");
  for (int64_t blk = 0; blk < pl.grid; ++blk) {
    const Work wk = work_of(a, blk);
    const int b = wk.b;
    const int n_tiles = key_tiles(a, wk.q_tile);
    const int hk0 = wave_role(a, wk, 0, G).h / (a.n_heads_q / a.n_heads_k);
    const int64_t kbase = row_of<D>(a, b, hk0, a.n_heads_k, a.seq_k, 0);
    // Q loads and rotation, O stores
    for (int t = 0; t < kBlock; ++t) {
      const int lane = t & 63, wave = t >> 6, hs = lane >> 5;
      const WaveRole role = wave_role(a, wk, wave, G);
      ck.fail(role.h < 0 || role.h >= a.n_heads_q, "wave head");
      ck.fail(role.h / (a.n_heads_q / a.n_heads_k) != hk0, "waves of one workgroup share K/V");
      const int qi = role.row0 + (lane & 31);
      const bool q_ok = qi < a.seq_q;
      if (!q_ok) continue;
      const int64_t qrow = row_of<D>(a, b, role.h, a.n_heads_q, a.seq_q, qi);
      for (int s = 0; s < D / 16; ++s) ck.check(qrow + s * 16 + hs * 8, 8, q_elems, "q load");
      const int64_t p = a.rotate ? qpos(b, qi) : -1;
      if (p >= 0) {
        if (PAIR == kSplitHalf) {
          for (int s = 0; s < a.half / 16; ++s) {
            ck.check(p * a.half + s * 16 + hs * 8, 8, table_elems, "q cos/sin");
            ck.fail(s + a.half / 16 >= D / 16, "q pair register");
          }
        } else {
          for (int s = 0; s < D / 16; ++s)
            if (s * 16 + hs * 8 < R)
              ck.check(p * a.half + (s * 16 + hs * 8) / 2, 4, table_elems, "q cos/sin");
        }
      }
      // only group 0 writes O
      if (wave < kWaves / kGroups)
        for (int dt = 0; dt < D / 32; ++dt)
          for (int g = 0; g < 4; ++g)
            ck.check(qrow + dt * 32 + 8 * g + 4 * hs, 4, q_elems, "o store");
    }
    // the tile pipeline, phase by phase: group g stages tile g into buffer
    // buf_of(g, 0); then in step s, group g reads tile s * kStride + g from
    // buf_of(g, s) and stages tile s * kStride + g + kStride into
    // buf_of(g, s + 1)
    auto buf_of = [&](int g, int step) { return G * (step & 1) + g; };
    LdsModel m(lds_elems);
    int phase = 0;
    auto stage = [&](int tile, int buf, int grp) {
      const int k0 = tile * kKeys;
      auto wrote = [&](int off, int n, int t, const char* what) {
        ck.check(off, n, lds_elems, what);
        const int lo = buf * buf_elems<D>(), hi = lo + buf_elems<D>();
        ck.fail(off < lo || off + n > hi, "staging outside its buffer");
        for (int i = off; i < off + n && i >= 0 && i < lds_elems; ++i) {
          ck.fail(m.wrote_in[i] == phase && m.writer[i] != t, "lds cell written by two lanes");
          ck.fail(m.read_in[i] == phase, "lds cell read and written in one phase");
          m.writer[i] = t;
          m.wrote_in[i] = phase;
          m.tile[i] = tile;
        }
      };
      for (int ts = 0; ts < NT; ++ts) {
        const int t = grp * NT + ts;
        // split-half pair items: rotate dims 8j.. with R/2 + 8j..
        for (int it = ts; it < kKeys * P::kPair; it += NT) {
          const int kk = it / P::kPair, j = it % P::kPair;
          const int key = k0 + kk;
          if (key < a.seq_k) {
            const int64_t krow = kbase + (int64_t)key * D;
            ck.check(krow + 8 * j, 8, kv_elems, "k load");
            ck.check(krow + kRK / 2 + 8 * j, 8, kv_elems, "k load");
            const int64_t kp = kpos(b, key);
            if (kp >= 0) ck.check(kp * a.half + 8 * j, 8, table_elems, "k cos/sin");
          }
          wrote(k_lds<D>(buf, kk, 8 * j), 8, t, "k lds");
          wrote(k_lds<D>(buf, kk, kRK / 2 + 8 * j), 8, t, "k lds");
        }
        // split-half copy items: dims R + 8j..
        for (int it = ts; it < kKeys * P::kCopy; it += NT) {
          const int kk = it / P::kCopy, j = it % P::kCopy;
          const int key = k0 + kk;
          if (key < a.seq_k) ck.check(kbase + (int64_t)key * D + kRK + 8 * j, 8, kv_elems, "k load");
          wrote(k_lds<D>(buf, kk, kRK + 8 * j), 8, t, "k lds");
        }
        // interleaved items: dims 8j.., rotated when 8j < R
        for (int it = ts; it < kKeys * P::kInter; it += NT) {
          const int kk = it / P::kInter, j = it % P::kInter;
          const int key = k0 + kk;
          if (key < a.seq_k) {
            ck.check(kbase + (int64_t)key * D + 8 * j, 8, kv_elems, "k load");
            const int64_t kp = (8 * j < R && a.rotate_k) ? kpos(b, key) : -1;
            if (kp >= 0) ck.check(kp * a.half + 4 * j, 4, table_elems, "k cos/sin");
          }
          wrote(k_lds<D>(buf, kk, 8 * j), 8, t, "k lds");
        }
        // the lanes' item counts stay within the registers the kernel keeps
        ck.fail((ts + P::kPairN * NT) < kKeys * P::kPair, "pair items per lane");
        ck.fail((ts + P::kCopyN * NT) < kKeys * P::kCopy, "copy items per lane");
        ck.fail((ts + P::kInterN * NT) < kKeys * P::kInter, "interleaved items per lane");
        ck.fail((ts + v_items_max<D, NT>() * NT) < v_items<D>(), "v items per lane");
        for (int it = ts; it < v_items<D>(); it += NT) {
          const VItem vi = v_item(it);
          for (int r = 0; r < 4; ++r) {
            const int key = k0 + 4 * vi.k4 + r;
            if (key < a.seq_k) ck.check(kbase + (int64_t)key * D + vi.c * 8, 8, kv_elems, "v load");
          }
          for (int i = 0; i < 8; ++i) {
            const int off = v_lds<D>(buf, vi.c * 8 + i, v_slot(4 * vi.k4));
            ck.fail(off % 4 != 0, "v lds write not 8-byte aligned");
            ck.fail(off < buf * buf_elems<D>() + k_lds_elems<D>(), "v lds inside the k tile");
            wrote(off, 4, t, "v lds");
          }
        }
      }
    };
    auto read = [&](int off, int n, int tile, const char* what) {
      ck.check(off, n, lds_elems, what);
      for (int i = off; i < off + n && i >= 0 && i < lds_elems; ++i) {
        ck.fail(m.tile[i] != tile, "lds read of a cell not staged for this tile");
        ck.fail(m.wrote_in[i] == phase, "lds cell read and written in one phase");
        m.read_in[i] = phase;
      }
    };
    for (int g = 0; g < kGroups; ++g)
      if (g < n_tiles) stage(g, buf_of(g, 0), g);
    const int n_steps = (n_tiles + kStride - 1) / kStride;
    for (int step = 0; step < n_steps; ++step) {
      ++phase;  // the barrier before the step
      for (int t = 0; t < kBlock; ++t) {
        const int lane = t & 63, wave = t >> 6, hs = lane >> 5, grp = wave / (kWaves / kGroups);
        const int kt = step * kStride + grp, k0 = kt * kKeys, buf = buf_of(grp, step);
        if (kt >= n_tiles) continue;
        const WaveRole role = wave_role(a, wk, wave, G);
        const int wq_last = imin(role.row0 + 31, a.seq_q - 1);
        if (role.row0 >= a.seq_q) continue;
        if (a.causal && k0 > wq_last + (a.seq_k - a.seq_q)) continue;
        for (int half = 0; half < 2; ++half)
          for (int st = 0; st < D / 16; ++st)
            read(k_lds<D>(buf, half * 32 + (lane & 31), st * 16 + hs * 8), 8, kt, "k lds read");
        for (int half = 0; half < 2; ++half)
          for (int u = 0; u < 2; ++u) {
            const int slot = half * 32 + 16 * u + 8 * hs;
            // the 8 slots hold the keys this lane's P^T slots stand for
            const int kb = half * 32 + 16 * u + 4 * hs;
            for (int i = 0; i < 8; ++i)
              ck.fail(v_slot(i < 4 ? kb + i : kb + 8 + (i - 4)) != slot + i, "v slot order");
            for (int dt = 0; dt < D / 32; ++dt) {
              const int dim = dt * 32 + (lane & 31);
              const int off = v_lds<D>(buf, dim, slot);
              ck.fail(off % 8 != 0, "v lds read not 16-byte aligned");
              read(off, 8, kt, "v lds read");
            }
          }
      }
      for (int g = 0; g < kGroups; ++g) {
        const int kt = step * kStride + g;
        if (kt + kStride < n_tiles) stage(kt + kStride, buf_of(g, step + 1), g);
      }
    }
    if (SPLIT) {
      // merge: after the last barrier, each lane of groups 1 .. G-1 writes
      // its state (m, l, D/32 x 16 accumulators) to float slot
      // ((g - 1) * kWg + wave % kWg) * 64 + lane, times kState; after one
      // more barrier its twin in group 0 reads every group's slot
      constexpr int kState = 2 + 16 * (D / 32);
      constexpr int kWg = kWaves / G;
      const int cells = (int)(pl.lds / 4);
      std::vector<int> who(cells, -1);
      auto slot = [&](int g, int wave, int lane) {
        return (((g - 1) * kWg + wave % kWg) * 64 + lane) * kState;
      };
      for (int t = NT; t < kBlock; ++t) {
        const int off = slot((t >> 6) / kWg, t >> 6, t & 63);
        ck.check(off, kState, cells, "merge state write");
        for (int i = off; i < off + kState && i >= 0 && i < cells; ++i) {
          ck.fail(who[i] != -1, "merge cell written by two lanes");
          who[i] = t;
        }
      }
      for (int t = 0; t < NT; ++t)
        for (int g = 1; g < G; ++g) {
          const int off = slot(g, t >> 6, t & 63);
          ck.check(off, kState, cells, "merge state read");
          for (int i = off; i < off + kState && i >= 0 && i < cells; ++i)
            ck.fail(who[i] != t + g * NT, "merge reads its twin's state");
        }
    }
  }
}

}  // namespace

namespace {

// the first entries hold the positions at the edges of the table: the last
// row, one past it (passes through) and -1 (passes through)
void edge_positions(std::vector<int32_t>& p, int64_t rows) {
  const int32_t e[3] = {(int32_t)rows - 1, (int32_t)rows, -1};
  for (size_t i = 0; i < 3 && i < p.size(); ++i) p[i] = e[i];
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 13 && argc != 14) {
    fprintf(stderr,
            "usage: attn_bounds B Hq Hk Sq Sk D R pairing causal table_rows qpos kpos "
            "[k_rotated]\n");
    return 2;
  }
  long long v[13] = {};
  for (int i = 0; i < argc - 1; ++i) v[i] = atoll(argv[i + 1]);
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
  d.k_rotated = (int32_t)v[12];
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
  printf("plan %d\ngroups %d\n", (int)st, (int)pl.a.groups);
  if (st != ROPE_OK || pl.empty) {
    printf("violations 0\naccesses 0\n");
    return 0;
  }
  Checker ck;
  const int64_t qpos_elems = d.batch * d.seq_len_q, kpos_elems = d.batch * d.seq_len_k;
  const int64_t a1 = qpos_elems, a2 = kpos_elems;
  auto run = [&](auto d_tag, auto pair_tag, auto h_tag) {
    constexpr int DD = decltype(d_tag)::value, PP = decltype(pair_tag)::value,
                  HH = decltype(h_tag)::value;
    // the launcher's choice: K rotated in the kernel unless it arrives rotated
    // (a plan without rotation uses the rotating instantiation, H16 = 0)
    // (the instantiations with wave groups exist at head dim 64)
    const bool kr = pl.a.rotate_k || (PP == kSplitHalf && HH == 0);
    auto go = [&](auto g_tag) {
      constexpr int GG = decltype(g_tag)::value;
      if (kr) walk<DD, PP, HH, true, GG>(pl, q_elems, kv_elems, table_elems, a1, a2, ck);
      else walk<DD, PP, HH, false, GG>(pl, q_elems, kv_elems, table_elems, a1, a2, ck);
    };
    if constexpr (DD == 64) {
      if (pl.a.groups == 2) return go(std::integral_constant<int, 2>{});
      if (pl.a.groups == 4) return go(std::integral_constant<int, 4>{});
    }
    ck.fail(pl.a.groups != 1, "wave groups the launcher has no kernel for");
    go(std::integral_constant<int, 1>{});
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  using SP = std::integral_constant<int, kSplitHalf>;
  using IN = std::integral_constant<int, kInterleaved>;
  if (pl.pairing == ROPE_INTERLEAVED) {
    if (pl.head_dim == 64) run(D64{}, IN{}, I0{}); else run(D128{}, IN{}, I0{});
  } else if (pl.head_dim == 64) {
    switch (pl.h16) {
      case 0: run(D64{}, SP{}, I0{}); break;
      case 1: run(D64{}, SP{}, I1{}); break;
      case 2: run(D64{}, SP{}, I2{}); break;
      default: ck.fail(true, "h16 beyond head dim 64");
    }
  } else {
    switch (pl.h16) {
      case 0: run(D128{}, SP{}, I0{}); break;
      case 1: run(D128{}, SP{}, I1{}); break;
      case 2: run(D128{}, SP{}, I2{}); break;
      case 3: run(D128{}, SP{}, I3{}); break;
      case 4: run(D128{}, SP{}, I4{}); break;
      default: ck.fail(true, "h16 beyond head dim 128");
    }
  }
  printf("violations %lld\naccesses %lld\n", ck.violations, ck.accesses);
  return 0;
}

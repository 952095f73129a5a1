// rope_emu.hip -- test harness: runs librope's kernel bodies on the host.
//
// Built for the host only (no device code is executed) and with
// AddressSanitizer, it plans a call exactly as librope does, then runs every
// workgroup and every lane of the planned grid one after another on host
// buffers allocated to their exact sizes, so any out-of-bounds access of the
// kernel index arithmetic is reported by the sanitizer. The Python tests
// compare its outputs with the CPU oracle.
//
// usage: rope_emu JOB_DIR
//   JOB_DIR/desc.txt : "key value" lines (see read_job)
//   JOB_DIR/{q,k,cos,sin,pos}.bin : raw inputs (pos/k only when used)
// writes JOB_DIR/{q_out,k_out}.bin and prints the plan on stdout.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "librope.h"
#include "rope_kernels.hpp"
#include "rope_plan.hpp"

namespace {

std::map<std::string, long long> read_job(const std::string& dir) {
  std::map<std::string, long long> kv;
  FILE* f = fopen((dir + "/desc.txt").c_str(), "r");
  if (!f) {
    perror("desc.txt");
    exit(2);
  }
  char key[64];
  long long val;
  while (fscanf(f, "%63s %lld", key, &val) == 2) kv[key] = val;
  fclose(f);
  return kv;
}

// Exactly `bytes` long (the sanitizer guards both ends), 16-byte aligned.
void* exact_alloc(size_t bytes) {
  void* p = nullptr;
  if (posix_memalign(&p, 16, bytes ? bytes : 1)) exit(3);
  return p;
}

void* read_file(const std::string& path, size_t bytes, size_t offset_bytes) {
  char* base = static_cast<char*>(exact_alloc(offset_bytes + bytes));
  FILE* f = fopen(path.c_str(), "rb");
  if (!f) {
    perror(path.c_str());
    exit(2);
  }
  if (bytes && fread(base + offset_bytes, 1, bytes, f) != bytes) {
    fprintf(stderr, "short read %s\n", path.c_str());
    exit(2);
  }
  fclose(f);
  return base + offset_bytes;
}

void write_file(const std::string& path, const void* p, size_t bytes) {
  FILE* f = fopen(path.c_str(), "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) exit(4);
  fclose(f);
}

struct HostRunner {
  const rope::Plan& pl;

  // Token kernel, single-pass modes, angles from theta: the kernel's three
  // phases around its barrier, each run for every lane of the workgroup
  // before the next. Shared memory is an exact-size buffer of NaNs, so a
  // read of an entry no lane wrote shows up in the outputs.
  template <typename T, int V, int PAIR, bool AL, bool OOP, int MODE>
  void theta_block(int64_t blk) {
    constexpr int K = rope::token_items_per_lane(PAIR);
    using Work = rope::TokenWork<T, V, PAIR, AL, OOP, K, MODE == rope::kTokenOne>;
    std::vector<Work> ws(pl.block);
    std::vector<char> has(pl.block);
    std::vector<float> lds((size_t)pl.lds_bytes / sizeof(float), std::nanf(""));
    for (int t = 0; t < pl.block; ++t) {
      int64_t n[K];
      int it[K], tl[K];
      bool live[K];
      rope::single_pass_items<MODE, K>(pl.a, blk, t, n, it, tl, live);
      has[t] = ws[t].begin(pl.a, n, it, tl, live);
      if (has[t]) ws[t].positions(pl.a);
    }
    for (int t = 0; t < pl.block; ++t) rope::theta_fill<MODE>(pl.a, blk, t, pl.block, lds.data());
    for (int t = 0; t < pl.block; ++t)
      if (has[t]) ws[t].finish_shared(pl.a, lds.data());
  }

  // Rows shape, one chunk per lane: the kernel's phases (load, partner
  // exchange, rotate and store) run for every lane of the workgroup before
  // the next, as the wave runs them in lockstep; each lane takes its
  // partner's loaded chunk from that lane's registers.
  template <typename T, int V, int SRC>
  void pair_block(int64_t blk) {
    using Work = rope::PairLaneWork<T, V, 4, SRC>;
    std::vector<Work> ws(pl.block);
    std::vector<char> live(pl.block);
    int first = -1;
    for (int t = 0; t < pl.block; ++t) {
      live[t] = ws[t].begin(pl.a, blk, t);
      if (live[t] && first < 0) first = t;
    }
    if (first < 0) return;
    const int L = pl.a.lanes >> 1;
    for (int t = 0; t < pl.block; ++t) {
      if (!live[t]) continue;
      // a live lane's partner is live, in the same wave, with the same heads
      const int q = t ^ L;
      if (q >= pl.block || !live[q] || (q >> 6) != (t >> 6) || ws[q].upper == ws[t].upper) {
        fprintf(stderr, "pair lanes: lane %d has no partner\n", t);
        exit(5);
      }
      for (int x = 0; x < 2; ++x)
        if (ws[t].lo[x] != ws[first].lo[x] || ws[t].hi[x] != ws[first].hi[x]) {
          fprintf(stderr, "pair lanes: head ranges differ within a workgroup\n");
          exit(5);
        }
    }
    for (int x = 0; x < 2; ++x)
      for (int h0 = ws[first].lo[x]; h0 < ws[first].hi[x]; h0 += 4) {
        for (int t = 0; t < pl.block; ++t)
          if (live[t]) ws[t].load(x, h0);
        for (int t = 0; t < pl.block; ++t)
          if (live[t])
            for (int u = 0; u < 4; ++u) ws[t].other[u] = ws[t ^ L].own[u];
        for (int t = 0; t < pl.block; ++t)
          if (live[t]) ws[t].finish(x, h0);
      }
  }

  // Flat shape with split-half pairs: the kernel's phases (load, partner
  // exchange, rotate and store) run for every lane of the workgroup (one
  // wave) before the next, each lane taking its partner's loaded chunk from
  // that lane's registers.
  template <typename T, int V, bool IDX>
  void flat_pair_block(int64_t blk) {
    using Work = rope::FlatPairWork<T, V, rope::kTrigVec, IDX>;
    std::vector<Work> ws(pl.block);
    std::vector<char> live(pl.block);
    for (int t = 0; t < pl.block; ++t) live[t] = ws[t].begin(pl.a, blk, t);
    const int L = pl.a.lanes >> 1;
    for (int t = 0; t < pl.block; ++t) {
      if (!live[t]) continue;
      // a live lane's partner is live, in the same wave, holds the other
      // half and makes the same skip decision
      const int q = t ^ L;
      if (q >= pl.block || !live[q] || (q >> 6) != (t >> 6) || ws[q].upper == ws[t].upper ||
          ws[q].store != ws[t].store) {
        fprintf(stderr, "flat pair lanes: lane %d has no partner\n", t);
        exit(5);
      }
    }
    for (int t = 0; t < pl.block; ++t)
      if (live[t]) ws[t].other = ws[t ^ L].own;
    for (int t = 0; t < pl.block; ++t)
      if (live[t]) ws[t].finish();
  }

  template <typename T, int V, int PAIR, bool AL, bool OOP>
  void go() {
    if constexpr (PAIR == rope::kSplitHalf && AL && !OOP && V * sizeof(T) == 16) {
      if (pl.flat) {
        for (int64_t blk = 0; blk < pl.grid; ++blk) {
          if (pl.a.pos)
            flat_pair_block<T, V, true>(blk);
          else
            flat_pair_block<T, V, false>(blk);
        }
        return;
      }
    }
    if constexpr (PAIR == rope::kSplitHalf && AL && !OOP && V * sizeof(T) == 16) {
      if (!pl.token && pl.pair) {
        for (int64_t blk = 0; blk < pl.grid; ++blk) {
          if (pl.a.angles)
            pair_block<T, V, rope::kTrigTheta>(blk);
          else if (pl.a.t_vec)
            pair_block<T, V, rope::kTrigVec>(blk);
          else
            pair_block<T, V, rope::kTrigScalar>(blk);
        }
        return;
      }
    }
    if (pl.head_lanes || pl.flat) {
      for (int64_t blk = 0; blk < pl.grid; ++blk)
        for (int t = 0; t < pl.block; ++t) {
          if (pl.head_lanes)
            rope::head_lanes_entry<T, V, PAIR, AL, OOP>(pl.a, blk, t);
          else
            rope::flat_entry<T, V, PAIR, AL, OOP>(pl.a, blk, t);
        }
      return;
    }
    if (pl.token && pl.a.angles && pl.token_mode() != rope::kTokenLoop) {
      for (int64_t blk = 0; blk < pl.grid; ++blk) {
        if (pl.token_mode() == rope::kTokenOne)
          theta_block<T, V, PAIR, AL, OOP, rope::kTokenOne>(blk);
        else
          theta_block<T, V, PAIR, AL, OOP, rope::kTokenPacked>(blk);
      }
      return;
    }
    for (int64_t blk = 0; blk < pl.grid; ++blk)
      for (int t = 0; t < pl.block; ++t) {
        if (pl.token && pl.token_mode() == rope::kTokenOne)
          rope::token_entry<T, V, PAIR, AL, rope::kTokenOne, OOP>(pl.a, blk, pl.grid, t,
                                                                   pl.block);
        else if (pl.token && pl.token_mode() == rope::kTokenPacked)
          rope::token_entry<T, V, PAIR, AL, rope::kTokenPacked, OOP>(pl.a, blk, pl.grid, t,
                                                                      pl.block);
        else if (pl.token)
          rope::token_entry<T, V, PAIR, AL, rope::kTokenLoop, OOP>(pl.a, blk, pl.grid, t,
                                                                    pl.block);
        else
          rope::rows_entry<T, V, PAIR, AL, 4, OOP>(pl.a, blk, t);
      }
  }

  template <typename T, int V, int PAIR, bool AL>
  int run() {
    if (pl.oop)
      go<T, V, PAIR, AL, true>();
    else
      go<T, V, PAIR, AL, false>();
    return 0;
  }
};

void print_plan(const rope::Plan& pl) {
  printf("empty %d\ntoken %d\nvec %d\naligned %d\ngrid %lld\nblock %d\nlanes %d\n"
         "heads_per_group %d\nn_groups %d\ngroup_slow %d\nsingle %d\noop %d\nt_vec %d\n"
         "tokens_per_block %d\nangles %d\nlds_bytes %lld\npair %d\nhead_lanes %d\nflat %d\n",
         (int)pl.empty, (int)pl.token, pl.vec, (int)pl.aligned, (long long)pl.grid, pl.block,
         pl.a.lanes, pl.a.heads_per_group, pl.a.n_groups, pl.a.group_slow, (int)pl.single,
         (int)pl.oop, pl.a.t_vec, pl.a.tokens_per_block, pl.a.angles,
         (long long)pl.lds_bytes, (int)pl.pair, (int)pl.head_lanes, (int)pl.flat);
}

// test-only overrides of the rows-kernel grid (one chunk or a chunk pair per
// lane, head-group size and order)
void apply_overrides(rope::Plan& pl, std::map<std::string, long long>& kv) {
  if (!pl.empty && !pl.token && pl.pair && kv["no_pair"] > 0) {
    // the pair-per-lane form of the same plan: half the lanes per token
    pl.pair = false;
    pl.a.lanes /= 2;
    pl.a.lanes_shift -= 1;
    pl.a.n_items = pl.a.n_tokens * pl.a.lanes;
    pl.a.n_tiles = (pl.a.n_items + rope::kRowsBlock - 1) / rope::kRowsBlock;
    pl.grid = pl.a.n_tiles * pl.a.n_groups;
  }
  if (!pl.empty && pl.head_lanes && (kv["heads_per_group"] > 0 || kv.count("hl_tshift"))) {
    // the head-lanes grid with other token and head counts per workgroup
    const int h_total = pl.a.n_heads_q + pl.a.n_heads_k;
    if (kv.count("hl_tshift")) {
      pl.a.tokens_shift = (int32_t)kv["hl_tshift"];
      pl.a.tokens_per_block = 1 << pl.a.tokens_shift;
      pl.a.n_tiles = (pl.a.n_tokens + pl.a.tokens_per_block - 1) / pl.a.tokens_per_block;
    }
    if (kv["heads_per_group"] > 0) pl.a.heads_per_group = (int32_t)kv["heads_per_group"];
    pl.a.n_groups = (h_total + pl.a.heads_per_group - 1) / pl.a.heads_per_group;
    pl.block = (pl.a.lanes << pl.a.tokens_shift) * pl.a.heads_per_group;
    pl.grid = pl.a.n_tiles * pl.a.n_groups;
    return;
  }
  if (!pl.empty && !pl.token && kv["heads_per_group"] > 0) {
    const int h_total = pl.a.n_heads_q + pl.a.n_heads_k;
    pl.a.heads_per_group = (int32_t)kv["heads_per_group"];
    pl.a.n_groups = (h_total + pl.a.heads_per_group - 1) / pl.a.heads_per_group;
    pl.grid = pl.a.n_tiles * pl.a.n_groups;
  }
  if (!pl.empty && !pl.token && kv.count("group_slow")) pl.a.group_slow = (int32_t)kv["group_slow"];
  // token shape: a smaller grid than planned runs the grid-stride loop
  if (!pl.empty && pl.token && kv["token_grid"] > 0 && kv["token_grid"] < pl.grid) {
    pl.grid = kv["token_grid"];
    pl.single = false;
    pl.lds_bytes = 0;  // the loop mode computes angles per lane
  }
}

rope_view_t read_view(std::map<std::string, long long>& kv, const std::string& name, char* base,
                      size_t e) {
  rope_view_t v{};
  if (kv[name + "_off"] < 0) return v;  // absent (in place)
  v.data = base + (size_t)kv[name + "_off"] * e;
  v.stride_b = kv[name + "_sb"];
  v.stride_h = kv[name + "_sh"];
  v.stride_s = kv[name + "_ss"];
  return v;
}

// General form: JOB_DIR/in.bin (in_elems) holds the Q and K input views,
// JOB_DIR/out.bin (out_elems, may be 0) the output views; cos/sin.bin hold
// table_elems floats. Writes in_after.bin and out_after.bin.
int apply_mode(const std::string& dir, std::map<std::string, long long>& kv) {
  rope_apply_desc_t d{};
  d.batch = kv["batch"];
  d.seq_len = kv["seq_len"];
  d.head_dim = kv["head_dim"];
  d.rotary_dim = kv["rotary_dim"];
  d.n_heads_q = kv["n_heads_q"];
  d.n_heads_k = kv["n_heads_k"];
  d.dtype = (int32_t)kv["dtype"];
  d.pairing = (int32_t)kv["pairing"];
  d.launch = (int32_t)kv["launch"];
  d.direction = (int32_t)kv["direction"];
  const size_t e = d.dtype == ROPE_F32 ? 4 : 2;
  const size_t in_bytes = (size_t)kv["in_elems"] * e, out_bytes = (size_t)kv["out_elems"] * e;
  char* in = static_cast<char*>(read_file(dir + "/in.bin", in_bytes, 0));
  char* out = out_bytes ? static_cast<char*>(read_file(dir + "/out.bin", out_bytes, 0)) : nullptr;
  d.q_in = read_view(kv, "q_in", in, e);
  d.k_in = read_view(kv, "k_in", in, e);
  d.q_out = read_view(kv, "q_out", out, e);
  d.k_out = read_view(kv, "k_out", out, e);
  const size_t tb = (size_t)kv["table_elems"] * 4;
  if (tb) {
    d.cos = static_cast<const float*>(read_file(dir + "/cos.bin", tb, 0));
    d.sin = static_cast<const float*>(read_file(dir + "/sin.bin", tb, 0));
  }
  d.angles = (int32_t)kv["angles"];
  // binary64 arguments travel as their bit patterns
  const long long theta_bits = kv["theta_bits"], interp_bits = kv["interp_bits"];
  memcpy(&d.theta, &theta_bits, sizeof(double));
  memcpy(&d.interpolate_factor, &interp_bits, sizeof(double));
  d.table_rows = kv["table_rows"];
  d.table_row_stride = kv["t_row"];
  d.table_col_stride = kv["t_col"];
  if (kv["pos_count"] > 0)
    d.pos = static_cast<const int32_t*>(
        read_file(dir + "/pos.bin", (size_t)kv["pos_count"] * 4, 0));
  d.pos_batch_stride = kv["pos_batch_stride"];
  rope::Plan pl;
  const int cus = kv.count("cus") ? (int)kv["cus"] : 256;
  const rope_status_t st = rope::make_plan_apply(&d, cus, &pl);
  printf("status %d\n", (int)st);
  if (st != ROPE_OK) return 0;
  apply_overrides(pl, kv);
  print_plan(pl);
  if (!pl.empty) {
    HostRunner runner{pl};
    rope::dispatch(pl, runner);
  }
  write_file(dir + "/in_after.bin", in, in_bytes);
  if (out_bytes) write_file(dir + "/out_after.bin", out, out_bytes);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: rope_emu JOB_DIR\n");
    return 2;
  }
  const std::string dir = argv[1];
  auto kv = read_job(dir);
  if (kv["apply"]) return apply_mode(dir, kv);
  if (kv["plan_only"]) {
    // the plan of a rope_fwd_qk call at any size, for 16-byte aligned Q and
    // K (fake addresses: nothing runs, nothing is dereferenced)
    rope_desc_t d{};
    d.batch = kv["batch"];
    d.n_heads_q = kv["n_heads_q"];
    d.n_heads_k = kv["n_heads_k"];
    d.seq_len = kv["seq_len"];
    d.head_dim = kv["head_dim"];
    d.rotary_dim = kv["rotary_dim"];
    d.dtype = (int32_t)kv["dtype"];
    d.layout = (int32_t)kv["layout"];
    d.pairing = (int32_t)kv["pairing"];
    d.launch = (int32_t)kv["launch"];
    d.table_rows = kv["table_rows"];
    d.cos = reinterpret_cast<const float*>((uintptr_t)1 << 44);
    d.sin = reinterpret_cast<const float*>((uintptr_t)2 << 44);
    void* q = reinterpret_cast<void*>((uintptr_t)3 << 44);
    void* k = reinterpret_cast<void*>((uintptr_t)4 << 44);
    rope::Plan pl;
    const int cus = kv.count("cus") ? (int)kv["cus"] : 256;
    const rope_status_t st = rope::make_plan(q, k, &d, true, 1.0f, cus, &pl);
    printf("status %d\n", (int)st);
    if (st == ROPE_OK) print_plan(pl);
    return 0;
  }
  if (kv["sincos"]) {
    // the kernels' cos/sin of binary64 angles: angles.bin (count doubles) ->
    // sincos.bin (count (cos, sin) float pairs)
    const size_t count = (size_t)kv["count"];
    const double* x = static_cast<const double*>(read_file(dir + "/angles.bin", count * 8, 0));
    std::vector<float> out(2 * count);
    for (size_t i = 0; i < count; ++i) rope::sincos_f32(x[i], &out[2 * i], &out[2 * i + 1]);
    write_file(dir + "/sincos.bin", out.data(), out.size() * sizeof(float));
    printf("status 0\n");
    return 0;
  }
  rope_desc_t d{};
  d.batch = kv["batch"];
  d.n_heads_q = kv["n_heads_q"];
  d.n_heads_k = kv["n_heads_k"];
  d.seq_len = kv["seq_len"];
  d.head_dim = kv["head_dim"];
  d.rotary_dim = kv["rotary_dim"];
  d.dtype = (int32_t)kv["dtype"];
  d.layout = (int32_t)kv["layout"];
  d.pairing = (int32_t)kv["pairing"];
  d.launch = (int32_t)kv["launch"];
  d.table_rows = kv["table_rows"];
  d.pos_batch_stride = kv["pos_batch_stride"];
  const bool with_k = kv["with_k"] != 0;
  const float sign = kv["direction"] < 0 ? -1.0f : 1.0f;
  const int cus = kv.count("cus") ? (int)kv["cus"] : 256;
  const size_t e = d.dtype == ROPE_F32 ? 4 : 2;
  const size_t row = (size_t)(d.batch * d.seq_len * d.head_dim);
  const size_t qb = row * d.n_heads_q * e, kb = with_k ? row * d.n_heads_k * e : 0;
  const size_t tb = (size_t)(d.table_rows * (d.rotary_dim / 2)) * 4;

  void* q = read_file(dir + "/q.bin", qb, (size_t)kv["q_offset"] * e);
  void* k = with_k ? read_file(dir + "/k.bin", kb, (size_t)kv["k_offset"] * e) : nullptr;
  d.cos = static_cast<const float*>(read_file(dir + "/cos.bin", tb, 0));
  d.sin = static_cast<const float*>(read_file(dir + "/sin.bin", tb, 0));
  if (kv["pos_count"] > 0)
    d.pos = static_cast<const int32_t*>(
        read_file(dir + "/pos.bin", (size_t)kv["pos_count"] * 4, 0));

  rope::Plan pl;
  const rope_status_t st = rope::make_plan(q, k, &d, with_k, sign, cus, &pl);
  printf("status %d\n", (int)st);
  if (st != ROPE_OK) return 0;
  apply_overrides(pl, kv);
  print_plan(pl);
  if (!pl.empty) {
    HostRunner runner{pl};
    rope::dispatch(pl, runner);
  }
  write_file(dir + "/q_out.bin", q, qb);
  if (with_k) write_file(dir + "/k_out.bin", k, kb);
  return 0;
}

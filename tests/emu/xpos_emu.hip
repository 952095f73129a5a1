// xpos_emu.hip -- test harness: runs the XPOS kernel body on the host.
//
// Built for the host only, with AddressSanitizer. It plans a rope_apply_xpos
// call exactly as librope does, then runs every lane of every workgroup of
// the planned grid on host buffers allocated to their exact sizes, so an
// out-of-bounds access of the index arithmetic is reported by the sanitizer.
// Output buffers of out-of-place calls start as a NaN pattern, so an element
// that no lane writes shows up in the comparison with the oracle.
//
// usage: xpos_emu JOB_DIR
//   JOB_DIR/desc.txt : "key value" lines
//   JOB_DIR/{q,k,cos,sin,zq,zk,pos}.bin : raw inputs (k/pos only when used)
// writes JOB_DIR/{q_out,k_out}.bin and prints "status N".
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>

#include "librope.h"
#include "rope_xpos.hpp"

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

void* exact_alloc(size_t bytes) {
  void* p = nullptr;
  if (posix_memalign(&p, 16, bytes ? bytes : 1)) exit(3);
  return p;
}

void* read_file(const std::string& path, size_t bytes) {
  void* p = exact_alloc(bytes);
  if (!bytes) return p;
  FILE* f = fopen(path.c_str(), "rb");
  if (!f || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot read %s\n", path.c_str());
    exit(2);
  }
  fclose(f);
  return p;
}

void write_file(const std::string& path, const void* p, size_t bytes) {
  FILE* f = fopen(path.c_str(), "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) exit(4);
  fclose(f);
}

// Every lane of every workgroup of the planned grid, one after another.
struct HostRunner {
  const rope::xpos::XPlan& pl;
  template <typename T, int V, int PAIR, int U>
  void chunked() {
    for (int64_t blk = 0; blk < pl.grid; ++blk)
      for (int t = 0; t < rope::xpos::kBlock; ++t)
        rope::xpos::xpos_block<T, V, PAIR, U>(pl.a, blk, t);
  }
  template <typename T, int V, int PAIR, bool IDX, bool TOKEN>
  void lanes() {
    for (int64_t blk = 0; blk < pl.grid; ++blk)
      for (int t = 0; t < pl.block; ++t)
        rope::xpos::xpos_lanes<T, V, PAIR, IDX, TOKEN>(pl.a, blk, t);
  }
  template <typename T>
  void element() {
    for (int64_t blk = 0; blk < pl.grid; ++blk)
      for (int t = 0; t < rope::xpos::kBlock; ++t) rope::xpos::xpos_token<T>(pl.a, blk, t);
  }
};

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: xpos_emu JOB_DIR\n");
    return 2;
  }
  const std::string dir = argv[1];
  auto kv = read_job(dir);
  const int dtype = (int)kv["dtype"];
  const size_t e = dtype == ROPE_F32 ? 4 : 2;
  const size_t qn = (size_t)kv["qn"], kn = (size_t)kv["kn"], tn = (size_t)kv["tn"],
               pn = (size_t)kv["pn"];
  const bool oop = kv["oop"] != 0;
  void* q = read_file(dir + "/q.bin", qn * e);
  void* k = kn ? read_file(dir + "/k.bin", kn * e) : nullptr;
  const float* cs = static_cast<const float*>(read_file(dir + "/cos.bin", tn * 4));
  const float* sn = static_cast<const float*>(read_file(dir + "/sin.bin", tn * 4));
  const float* zq = static_cast<const float*>(read_file(dir + "/zq.bin", tn * 4));
  const float* zk = static_cast<const float*>(read_file(dir + "/zk.bin", tn * 4));
  const int32_t* pos = pn ? static_cast<const int32_t*>(read_file(dir + "/pos.bin", pn * 4))
                          : nullptr;
  void* qo = nullptr;
  void* ko = nullptr;
  if (oop) {
    qo = exact_alloc(qn * e);
    memset(qo, 0xff, qn * e);  // NaN in every dtype
    if (kn) {
      ko = exact_alloc(kn * e);
      memset(ko, 0xff, kn * e);
    }
  }

  rope_apply_desc_t d{};
  d.batch = kv["B"];
  d.seq_len = kv["S"];
  d.head_dim = kv["D"];
  d.rotary_dim = kv["R"];
  d.n_heads_q = kv["Hq"];
  d.n_heads_k = kv["Hk"];
  d.dtype = dtype;
  d.pairing = (int32_t)kv["pairing"];
  d.launch = ROPE_LAUNCH_AUTO;
  d.direction = (int32_t)kv["direction"];
  d.q_in = rope_view_t{q, kv["qsb"], kv["qsh"], kv["qss"]};
  if (kn) d.k_in = rope_view_t{k, kv["ksb"], kv["ksh"], kv["kss"]};
  if (oop) {
    d.q_out = rope_view_t{qo, kv["qsb"], kv["qsh"], kv["qss"]};
    if (kn) d.k_out = rope_view_t{ko, kv["ksb"], kv["ksh"], kv["kss"]};
  }
  d.cos = cs;
  d.sin = sn;
  d.table_rows = kv["table_rows"];
  d.table_row_stride = kv["t_row"];
  d.table_col_stride = kv["t_col"];
  d.pos = pos;
  d.pos_batch_stride = kv["pos_bs"];
  d.angles = ROPE_ANGLES_TABLE;

  rope::xpos::XPlan pl;
  const rope_status_t st = rope::xpos::make_xpos_plan(&d, zq, kn ? zk : nullptr, &pl);
  printf("status %d\n", (int)st);
  if (st != ROPE_OK) return 0;
  printf("vec %d\ngrid %lld\nheads_per_group %d\nlanes %d\nblock %d\n", pl.vec,
         (long long)pl.grid, (int)pl.a.heads_per_group, pl.lanes, pl.block);
  if (!pl.empty) {
    HostRunner run{pl};
    if (!rope::xpos::dispatch(pl, run)) {
      fprintf(stderr, "no kernel for this plan\n");
      return 5;
    }
  }
  write_file(dir + "/q_out.bin", oop ? qo : q, qn * e);
  if (kn) write_file(dir + "/k_out.bin", oop ? ko : k, kn * e);
  return 0;
}

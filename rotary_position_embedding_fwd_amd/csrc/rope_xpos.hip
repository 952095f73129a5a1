// rope_xpos.hip -- the C ABI of RoPE with XPOS scaling (rope_xpos.hpp).
#include <hip/hip_runtime.h>

#include "librope.h"
#include "rope_xpos.hpp"

namespace {

template <typename T, int V, int PAIR, int U>
__global__ void __launch_bounds__(rope::xpos::kBlock)
    rope_xpos_kernel(rope::xpos::XArgs a) {
  rope::xpos::xpos_block<T, V, PAIR, U>(a, blockIdx.x, (int)threadIdx.x);
}

template <typename T, int V, int PAIR, bool IDX, bool TOKEN>
__global__ void __launch_bounds__(1024) rope_xpos_lanes_kernel(rope::xpos::XArgs a) {
  rope::xpos::xpos_lanes<T, V, PAIR, IDX, TOKEN>(a, blockIdx.x, (int)threadIdx.x);
}

template <typename T>
__global__ void __launch_bounds__(rope::xpos::kBlock)
    rope_xpos_element_kernel(rope::xpos::XArgs a) {
  rope::xpos::xpos_token<T>(a, blockIdx.x, (int)threadIdx.x);
}

struct Launcher {
  const rope::xpos::XPlan& pl;
  hipStream_t st;
  template <typename T, int V, int PAIR, int U>
  void chunked() {
    hipLaunchKernelGGL((rope_xpos_kernel<T, V, PAIR, U>), dim3((unsigned)pl.grid),
                       dim3(rope::xpos::kBlock), 0, st, pl.a);
  }
  template <typename T, int V, int PAIR, bool IDX, bool TOKEN>
  void lanes() {
    hipLaunchKernelGGL((rope_xpos_lanes_kernel<T, V, PAIR, IDX, TOKEN>),
                       dim3((unsigned)pl.grid), dim3(pl.block), 0, st, pl.a);
  }
  template <typename T>
  void element() {
    hipLaunchKernelGGL(rope_xpos_element_kernel<T>, dim3((unsigned)pl.grid),
                       dim3(rope::xpos::kBlock), 0, st, pl.a);
  }
};

}  // namespace

extern "C" {

rope_status_t rope_apply_xpos(const rope_apply_desc_t* d, const float* xpos_q,
                              const float* xpos_k, void* stream) {
  rope::xpos::XPlan pl;
  const rope_status_t st = rope::xpos::make_xpos_plan(d, xpos_q, xpos_k, &pl);
  if (st != ROPE_OK || pl.empty) return st;
  Launcher launch{pl, static_cast<hipStream_t>(stream)};
  if (!rope::xpos::dispatch(pl, launch)) return ROPE_ERR_HIP;  // no plan produces this
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status_t rope_build_xpos_table(float* xpos_q, float* xpos_k, int64_t table_rows,
                                    int64_t rotary_dim, double scale_base, double gamma,
                                    double center) {
  return rope::xpos::build_xpos_table(xpos_q, xpos_k, table_rows, rotary_dim, scale_base, gamma,
                                      center);
}

}  // extern "C"

// rope_xpos.hip -- the C ABI of RoPE with XPOS scaling (rope_xpos.hpp).
#include <hip/hip_runtime.h>

#include "librope.h"
#include "rope_xpos.hpp"

namespace {

template <typename T>
__global__ void __launch_bounds__(rope::xpos::kBlock)
    rope_xpos_kernel(rope::xpos::XArgs a) {
  rope::xpos::xpos_token<T>(a, blockIdx.x, (int)threadIdx.x);
}

template <typename T>
hipError_t launch_xpos(const rope::xpos::XPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL(rope_xpos_kernel<T>, dim3((unsigned)pl.a.n_tokens),
                     dim3(rope::xpos::kBlock), 0, st, pl.a);
  return hipGetLastError();
}

}  // namespace

extern "C" {

rope_status_t rope_apply_xpos(const rope_apply_desc_t* d, const float* xpos_q,
                              const float* xpos_k, void* stream) {
  rope::xpos::XPlan pl;
  const rope_status_t st = rope::xpos::make_xpos_plan(d, xpos_q, xpos_k, &pl);
  if (st != ROPE_OK || pl.empty) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorInvalidValue;
  switch (pl.dtype) {
    case ROPE_F32: e = launch_xpos<float>(pl, s); break;
    case ROPE_F16: e = launch_xpos<_Float16>(pl, s); break;
    case ROPE_BF16: e = launch_xpos<__bf16>(pl, s); break;
  }
  return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status_t rope_build_xpos_table(float* xpos_q, float* xpos_k, int64_t table_rows,
                                    int64_t rotary_dim, double scale_base, double gamma,
                                    double center) {
  return rope::xpos::build_xpos_table(xpos_q, xpos_k, table_rows, rotary_dim, scale_base, gamma,
                                      center);
}

}  // extern "C"

// librope.hip -- host side of the librope C ABI (declared in include/librope.h).
//
// Each entry point validates its descriptor without touching the GPU, picks
// the access width and grid shape, and enqueues one kernel on the caller's
// stream. Nothing here allocates device memory or waits for the GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "librope.h"
#include "rope_kernels.hpp"
#include "rope_plan.hpp"

namespace {

constexpr int kVersion = 10400;  // 1.4.0: flat pair-lanes kernel for split-half token-major calls
constexpr int kMaxDevices = 64;

// Compute units per device, read once per device.
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Enqueues the planned kernel variant on a stream.
struct GpuLauncher {
  const rope::Plan& pl;
  hipStream_t st;

  template <typename T, int V, int PAIR, bool AL, bool OOP>
  void launch() {
    const dim3 grid((unsigned)pl.grid), block((unsigned)pl.block);
    const int mode = pl.token ? pl.token_mode() : -1;
    const unsigned lds = (unsigned)pl.lds_bytes;
    constexpr int RT = rope::kSrcRuntime;
    if (launch_only_auto<T, V, PAIR, AL, OOP>(grid, block)) return;
    if (mode == rope::kTokenOne && pl.a.angles)
      hipLaunchKernelGGL(
          (rope::rope_token_kernel<T, V, PAIR, AL, rope::kTokenOne, OOP, rope::kTrigTheta>), grid,
          block, lds, st, pl.a);
    else if (mode == rope::kTokenOne && pl.a.t_vec)
      hipLaunchKernelGGL(
          (rope::rope_token_kernel<T, V, PAIR, AL, rope::kTokenOne, OOP, rope::kTrigVec>), grid,
          block, 0, st, pl.a);
    else if (mode == rope::kTokenOne)
      hipLaunchKernelGGL(
          (rope::rope_token_kernel<T, V, PAIR, AL, rope::kTokenOne, OOP, rope::kTrigScalar>),
          grid, block, 0, st, pl.a);
    else if (mode == rope::kTokenPacked)
      hipLaunchKernelGGL((rope::rope_token_kernel<T, V, PAIR, AL, rope::kTokenPacked, OOP, RT>),
                         grid, block, lds, st, pl.a);
    else if (mode == rope::kTokenLoop)
      hipLaunchKernelGGL((rope::rope_token_kernel<T, V, PAIR, AL, rope::kTokenLoop, OOP, RT>),
                         grid, block, 0, st, pl.a);
    else if (!launch_pair<T, V, PAIR, AL, OOP>(grid, block))
      hipLaunchKernelGGL((rope::rope_rows_kernel<T, V, PAIR, AL, 4, OOP>), grid, block, 0, st,
                         pl.a);
  }

  // the forms only the automatic launch picks, instantiated for the calls the
  // planner gives them (in place; head lanes and flat pair lanes: split-half
  // 16-byte chunks; flat: interleaved pairs)
  template <typename T, int V, int PAIR, bool AL, bool OOP>
  bool launch_only_auto(dim3 grid, dim3 block) {
    const bool idx = pl.a.pos != nullptr;
    if constexpr (!OOP && AL && PAIR == rope::kSplitHalf && V * sizeof(T) == 16) {
      if (pl.head_lanes) {
        if (idx)
          hipLaunchKernelGGL((rope::rope_head_lanes_kernel<T, V, PAIR, AL, OOP, true>), grid,
                             block, 0, st, pl.a);
        else
          hipLaunchKernelGGL((rope::rope_head_lanes_kernel<T, V, PAIR, AL, OOP, false>), grid,
                             block, 0, st, pl.a);
        return true;
      }
      if (pl.flat) {
        if (idx)
          hipLaunchKernelGGL((rope::rope_flat_pair_kernel<T, V, true>), grid, block, 0, st, pl.a);
        else
          hipLaunchKernelGGL((rope::rope_flat_pair_kernel<T, V, false>), grid, block, 0, st,
                             pl.a);
        return true;
      }
    }
    if constexpr (!OOP && AL && PAIR == rope::kInterleaved) {
      if (pl.flat) {
        if (idx)
          hipLaunchKernelGGL((rope::rope_flat_kernel<T, V, PAIR, AL, OOP, true>), grid, block,
                             0, st, pl.a);
        else
          hipLaunchKernelGGL((rope::rope_flat_kernel<T, V, PAIR, AL, OOP, false>), grid, block,
                             0, st, pl.a);
        return true;
      }
    }
    return false;
  }

  // the one-chunk-per-lane rows kernel, for the plans that chose it
  template <typename T, int V, int PAIR, bool AL, bool OOP>
  bool launch_pair(dim3 grid, dim3 block) {
    if constexpr (PAIR == rope::kSplitHalf && AL && !OOP && V * sizeof(T) == 16) {
      if (pl.pair) {
        hipLaunchKernelGGL((rope::rope_pair_lanes_kernel<T, V, 4>), grid, block, 0, st, pl.a);
        return true;
      }
    }
    return false;
  }

  template <typename T, int V, int PAIR, bool AL>
  hipError_t run() {
    if (pl.oop)
      launch<T, V, PAIR, AL, true>();
    else
      launch<T, V, PAIR, AL, false>();
    return hipGetLastError();
  }
};

rope_status_t run_apply(const rope_apply_desc_t* d, void* stream) {
  // validation first: it needs no device and touches no device memory
  const rope_status_t vs = rope::validate_apply(d);
  if (vs != ROPE_OK) return vs;
  if (rope::apply_is_empty(d)) return ROPE_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ROPE_ERR_HIP;
  rope::Plan pl;
  const rope_status_t ps = rope::make_plan_apply(d, cu_count(dev), &pl);
  if (ps != ROPE_OK || pl.empty) return ps;
  GpuLauncher launcher{pl, static_cast<hipStream_t>(stream)};
  return rope::dispatch(pl, launcher) == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

// The kernel a plan launches, as it is named in traces, and its grid.
void describe_plan(const rope::Plan& pl, char* buf, int64_t len) {
  const char* kernel = "none (empty call)";
  if (!pl.empty) {
    if (pl.flat && pl.pairing == ROPE_SPLIT_HALF)
      kernel = "rope_flat_pair_kernel";
    else if (pl.flat)
      kernel = "rope_flat_kernel";
    else if (pl.head_lanes)
      kernel = "rope_head_lanes_kernel";
    else if (pl.token)
      kernel = "rope_token_kernel";
    else if (pl.pair)
      kernel = "rope_pair_lanes_kernel";
    else
      kernel = "rope_rows_kernel";
  }
  static const char* kDtypes[] = {"f32", "f16", "bf16"};
  const char* dt = pl.dtype >= 0 && pl.dtype <= 2 ? kDtypes[pl.dtype] : "?";
  snprintf(buf, (size_t)len,
           "%s dtype=%s vec=%d pairing=%s grid=%lld block=%d lanes_per_token=%d "
           "tokens_per_workgroup=%d heads_per_group=%d%s",
           kernel, dt, pl.vec, pl.pairing == ROPE_INTERLEAVED ? "interleaved" : "split_half",
           (long long)pl.grid, pl.block, pl.a.lanes, pl.a.tokens_per_block,
           pl.a.heads_per_group, pl.oop ? " out_of_place" : "");
}

rope_status_t run(void* q, void* k, const rope_desc_t* d, void* stream, bool with_k,
                  int direction) {
  rope_apply_desc_t a;
  const rope_status_t st = rope::desc_to_apply(q, k, d, with_k, direction, &a);
  return st != ROPE_OK ? st : run_apply(&a, stream);
}

}  // namespace


extern "C" {

rope_status_t rope_fwd_qk(void* q, void* k, const rope_desc_t* d, void* stream) {
  return run(q, k, d, stream, true, 1);
}

rope_status_t rope_bwd_qk(void* dq, void* dk, const rope_desc_t* d, void* stream) {
  return run(dq, dk, d, stream, true, -1);
}

rope_status_t rope_fwd_q(void* q, const rope_desc_t* d, void* stream) {
  return run(q, nullptr, d, stream, false, 1);
}

rope_status_t rope_bwd_q(void* dq, const rope_desc_t* d, void* stream) {
  return run(dq, nullptr, d, stream, false, -1);
}

rope_status_t rope_apply(const rope_apply_desc_t* d, void* stream) { return run_apply(d, stream); }

rope_status_t rope_describe(const void* q, const void* k, const rope_desc_t* d, int with_k,
                            char* buf, int64_t len) {
  if (!buf || len < 1) return ROPE_ERR_NULL;
  buf[0] = 0;
  rope_apply_desc_t a;
  const rope_status_t st = rope::desc_to_apply(q, k, d, with_k != 0, 1, &a);
  if (st != ROPE_OK) return st;
  const rope_status_t vs = rope::validate_apply(&a);
  if (vs != ROPE_OK) return vs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ROPE_ERR_HIP;
  rope::Plan pl;
  const rope_status_t ps = rope::make_plan_apply(&a, cu_count(dev), &pl);
  if (ps != ROPE_OK) return ps;
  describe_plan(pl, buf, len);
  return ROPE_OK;
}

rope_status_t rope_build_table(float* cos_out, float* sin_out, int64_t table_rows,
                               int64_t rotary_dim, double theta, double interpolate_factor) {
  if (table_rows < 0 || rotary_dim < 0 || (rotary_dim & 1) || !(theta > 0.0) ||
      !std::isfinite(theta) || !(interpolate_factor > 0.0) || !std::isfinite(interpolate_factor))
    return ROPE_ERR_SHAPE;
  const int64_t half = rotary_dim / 2;
  if (table_rows == 0 || half == 0) return ROPE_OK;
  if (!cos_out || !sin_out) return ROPE_ERR_NULL;
  for (int64_t i = 0; i < half; ++i) {
    // theta^(-2i/R), exponent and power in binary64
    const double inv_freq = std::pow(theta, -(2.0 * (double)i) / (double)rotary_dim);
    for (int64_t p = 0; p < table_rows; ++p) {
      const double angle = ((double)p / interpolate_factor) * inv_freq;
      cos_out[p * half + i] = (float)std::cos(angle);
      sin_out[p * half + i] = (float)std::sin(angle);
    }
  }
  return ROPE_OK;
}

const char* rope_status_string(rope_status_t s) {
  switch (s) {
    case ROPE_OK: return "ok";
    case ROPE_ERR_NULL: return "a required pointer is NULL";
    case ROPE_ERR_SHAPE: return "invalid or inconsistent sizes, or a number out of range";
    case ROPE_ERR_DTYPE: return "unknown dtype";
    case ROPE_ERR_LAYOUT: return "unknown layout, pairing, launch shape or angle source";
    case ROPE_ERR_ALIGN: return "misaligned pointer";
    case ROPE_ERR_ALIAS: return "written data overlaps other operands";
    case ROPE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int rope_version(void) { return kVersion; }

}  // extern "C"

// stream_probe.hip -- the bandwidth a plain in-place read-modify-write stream
// reaches on this GPU, measured beside the RoPE kernels by the benchmark.
//
// Each lane moves one 16-byte chunk: a non-temporal load and a non-temporal
// store of the same address, 64-lane workgroups in memory order. This is the
// fastest pattern for an in-place 1:1 read/write stream found on MI355X, so
// it stands for the attainable HBM ceiling of an operation that, like RoPE,
// reads and writes every byte once. It is a measurement aid only; nothing in
// librope calls it.
//
// mfma_rate_probe: the rate the bf16 matrix cores sustain on this GPU, for
// the same purpose beside the attention kernel. Every wave runs chains of
// v_mfma_f32_32x32x16_bf16 on register operands (four independent
// accumulators; no memory traffic but one store per lane at the end).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int probe_u4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(64) stream_rmw_kernel(probe_u4* x, int64_t n, unsigned mask) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(x + i) ^ mask, x + i);
}

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_rate_kernel(float* out, int iters, float seed) {
  const int t = threadIdx.x;
  probe_bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(t + i));
    b[i] = (__bf16)(seed * (float)(i - t));
  }
  probe_f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(int64_t)blockIdx.x * 256 + t] = s;
}

extern "C" {

// x: device buffer of `bytes` bytes (a multiple of 16, 16-byte aligned).
// Rewrites every 16-byte chunk with itself XOR `mask` (mask 0: unchanged
// contents). Enqueued on `stream`; returns 0, or -1 for bad arguments, -7
// for a HIP launch error.
int stream_rmw_probe(void* x, int64_t bytes, unsigned mask, void* stream) {
  if (!x || bytes < 0 || (bytes % 16) || (reinterpret_cast<uintptr_t>(x) % 16)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  const int64_t grid = (n + 63) / 64;
  if (grid > 0x7fffffff) return -1;
  hipLaunchKernelGGL(stream_rmw_kernel, dim3((unsigned)grid), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<probe_u4*>(x), n, mask);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// out: device buffer of blocks * 256 floats. Runs `blocks` workgroups of 4
// waves, each wave 16 * iters MFMAs of 32 x 32 x 16 (32768 flops each).
// Returns 0, -1 for bad arguments, -7 for a HIP launch error.
int mfma_rate_probe(void* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<float*>(out), iters, 1e-3f);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"

// stream_probe.hip -- the bandwidth a plain in-place read-modify-write stream
// reaches on this GPU, measured beside the RoPE kernels by the benchmark.
//
// Each lane moves one 16-byte chunk: a non-temporal load and a non-temporal
// store of the same address, 64-lane workgroups in memory order. This is the
// fastest pattern for an in-place 1:1 read/write stream found on MI355X, so
// it stands for the attainable HBM ceiling of an operation that, like RoPE,
// reads and writes every byte once. It is a measurement aid only; nothing in
// librope calls it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int probe_u4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(64) stream_rmw_kernel(probe_u4* x, int64_t n, unsigned mask) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(x + i) ^ mask, x + i);
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

}  // extern "C"

// rope_attention.hip -- host side of the attention entry points: the fused
// call (rope_attention_fwd) and the one that rotates K once first
// (rope_attention_fwd_k_once). Validation and the launch plan are in
// rope_attn_plan.hpp, the kernel in rope_attention.hpp.
//
// Why rotate K once: the fused kernel rotates each K tile in every workgroup
// that reads it; on long sequences many workgroups read each tile (64 per
// tile on a 4096-token causal prefill with 256-row workgroups), and those
// rotations cost more than writing rope(K) once and reading it back. Given a
// K-sized buffer from the caller, rope_attention_fwd_k_once runs rope_apply
// (rope(K) into the buffer, rounded to bf16 exactly as the fused kernel
// rounds it) and then the attention kernel that rotates only Q, both on the
// caller's stream. The library allocates nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "librope.h"
#include "rope_attn_plan.hpp"

namespace {

// KR: the K tiles are rotated while staged (the fused form); otherwise K
// arrives rotated and is staged by the copy-only plan, with no cos/sin
// registers for it.
template <int D, int PAIR, int H16, bool KR, int G>
hipError_t launch_attention_one(const rope::attn::AttnPlan& pl, hipStream_t st) {
  auto kernel = rope::attn::rope_attention_kernel<D, PAIR, H16, KR, G>;
  // the double-buffered tiles take more than the default 64 KiB of dynamic
  // LDS at head dim 128 (and with several wave groups): raise the kernel's
  // limit once (per process; the attribute belongs to the kernel, not to a
  // device)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      rope::attn::lds_bytes_groups<D>(G));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kernel, dim3((unsigned)pl.grid), dim3(rope::attn::kBlock), (unsigned)pl.lds,
                     st, pl.a);
  return hipGetLastError();
}

// several wave groups exist at head dim 64 only (the plan chooses them there)
template <int D, int PAIR, int H16, bool KR>
hipError_t launch_attention(const rope::attn::AttnPlan& pl, hipStream_t st) {
  if constexpr (D == 64) {
    if (pl.a.groups == 2) return launch_attention_one<D, PAIR, H16, KR, 2>(pl, st);
    if (pl.a.groups == 4) return launch_attention_one<D, PAIR, H16, KR, 4>(pl, st);
  }
  if (pl.a.groups != 1) return hipErrorInvalidValue;  // unreachable: see the plan
  return launch_attention_one<D, PAIR, H16, KR, 1>(pl, st);
}

template <int D, int PAIR, int H16>
hipError_t launch_attention_kr(const rope::attn::AttnPlan& pl, hipStream_t st) {
  if (pl.a.rotate_k) return launch_attention<D, PAIR, H16, true>(pl, st);
  return launch_attention<D, PAIR, H16, false>(pl, st);
}

template <int D>
hipError_t launch_attention_d(const rope::attn::AttnPlan& pl, hipStream_t st) {
  using rope::kInterleaved;
  using rope::kSplitHalf;
  if (pl.pairing == ROPE_INTERLEAVED) return launch_attention_kr<D, kInterleaved, 0>(pl, st);
  switch (pl.h16) {
    case 0: return launch_attention<D, kSplitHalf, 0, true>(pl, st);  // no rotation at all
    case 1: return launch_attention_kr<D, kSplitHalf, 1>(pl, st);
    case 2: return launch_attention_kr<D, kSplitHalf, 2>(pl, st);
  }
  if constexpr (D == 128) {
    switch (pl.h16) {
      case 3: return launch_attention_kr<D, kSplitHalf, 3>(pl, st);
      case 4: return launch_attention_kr<D, kSplitHalf, 4>(pl, st);
    }
  }
  return hipErrorInvalidValue;  // unreachable: the plan bounds h16 by D / 32
}

// ------------------------------------------- allocation-free K-once call
// rope_attention_fwd_k_once_noalloc stages rope(K) in this file-scope device
// array instead of a caller buffer. Each device that loads the library holds
// its own copy (kNoAllocKBytes) until the process ends. Host code never uses
// the array's name as an address: the address of each device's copy is looked
// up once per device with hipGetSymbolAddress and kept below.
constexpr int64_t kNoAllocKBytes = (int64_t)64 << 20;  // rope(K) of up to 32 Mi bf16 values
static __device__ __align__(256) unsigned char scratch[kNoAllocKBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];

// The address of `scratch` on device `dev`, which must be the current device;
// nullptr if the runtime cannot give it. Two threads that race here both store
// the same address.
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" rope_status_t rope_attention_fwd(const rope_attn_desc_t* d, void* stream) {
  rope::attn::AttnPlan pl;
  const rope_status_t st = rope::attn::make_attn_plan(d, &pl);
  if (st != ROPE_OK || pl.empty) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ROPE_ERR_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = pl.head_dim == 64 ? launch_attention_d<64>(pl, s)
                                         : launch_attention_d<128>(pl, s);
  return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

extern "C" rope_status_t rope_attention_fwd_k_once(const rope_attn_desc_t* d, void* k_workspace,
                                                   void* stream) {
  if (!d) return ROPE_ERR_NULL;
  if (d->k_rotated) return ROPE_ERR_SHAPE;  // this call rotates K itself
  rope::attn::AttnPlan pl;
  const rope_status_t st = rope::attn::make_attn_plan(d, &pl);
  if (st != ROPE_OK || pl.empty) return st;
  const bool rotate = d->rotate && d->rotary_dim > 0;
  if (!rotate || d->seq_len_k == 0) return rope_attention_fwd(d, stream);  // no K to rotate

  if (!k_workspace) return ROPE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(k_workspace) % 16) return ROPE_ERR_ALIGN;
  // extents (the plan has checked that they fit in int64)
  const int64_t B = d->batch, Hq = d->n_heads_q, Hk = d->n_heads_k, Sq = d->seq_len_q,
                Sk = d->seq_len_k, D = d->head_dim;
  const int64_t qbytes = B * Hq * Sq * D * 2, kvbytes = B * Hk * Sk * D * 2;
  const int64_t tbytes = d->table_rows * d->rotary_dim * 2;
  auto index_bytes = [&](const int32_t* p, int64_t stride, int64_t S) -> int64_t {
    return p ? ((B - 1) * stride + S) * 4 : 0;
  };
  using rope::attn::ranges_meet;
  // the workspace is written first and read by the attention: it may meet
  // no operand of either call
  if (ranges_meet(k_workspace, kvbytes, d->q, qbytes) ||
      ranges_meet(k_workspace, kvbytes, d->k, kvbytes) ||
      ranges_meet(k_workspace, kvbytes, d->v, kvbytes) ||
      ranges_meet(k_workspace, kvbytes, d->o, qbytes) ||
      ranges_meet(k_workspace, kvbytes, d->cos, tbytes) ||
      ranges_meet(k_workspace, kvbytes, d->sin, tbytes) ||
      ranges_meet(k_workspace, kvbytes, d->q_pos,
                  index_bytes(d->q_pos, d->q_pos_batch_stride, Sq)) ||
      ranges_meet(k_workspace, kvbytes, d->k_pos,
                  index_bytes(d->k_pos, d->k_pos_batch_stride, Sk)))
    return ROPE_ERR_ALIAS;

  // rope(K) into the workspace: K as the query-only input of rope_apply, key
  // j at position k_pos[j] (or j), out-of-table keys copied unrotated
  rope_apply_desc_t ad{};
  ad.batch = B;
  ad.seq_len = Sk;
  ad.head_dim = D;
  ad.rotary_dim = d->rotary_dim;
  ad.n_heads_q = Hk;
  ad.n_heads_k = 0;
  ad.dtype = ROPE_BF16;
  ad.pairing = d->pairing;
  ad.launch = ROPE_LAUNCH_AUTO;
  ad.direction = 1;
  ad.q_in = rope_view_t{const_cast<void*>(d->k), Hk * Sk * D, Sk * D, D};
  ad.q_out = rope_view_t{k_workspace, Hk * Sk * D, Sk * D, D};
  ad.cos = d->cos;
  ad.sin = d->sin;
  ad.table_rows = d->table_rows;
  ad.table_row_stride = 0;
  ad.table_col_stride = 1;
  ad.pos = d->k_pos;
  ad.pos_batch_stride = d->k_pos_batch_stride;
  ad.angles = ROPE_ANGLES_TABLE;
  const rope_status_t rs = rope_apply(&ad, stream);
  if (rs != ROPE_OK) return rs;

  rope_attn_desc_t da = *d;
  da.k = k_workspace;
  da.k_rotated = 1;
  return rope_attention_fwd(&da, stream);
}

extern "C" rope_status_t rope_attention_fwd_k_once_noalloc(const rope_attn_desc_t* d,
                                                           void* stream) {
  if (!d) return ROPE_ERR_NULL;
  if (d->k_rotated) return ROPE_ERR_SHAPE;  // this call rotates K itself
  rope::attn::AttnPlan pl;
  const rope_status_t st = rope::attn::make_attn_plan(d, &pl);
  if (st != ROPE_OK || pl.empty) return st;
  const bool rotate = d->rotate && d->rotary_dim > 0;
  if (!rotate || d->seq_len_k == 0) return rope_attention_fwd(d, stream);  // no K to rotate
  // the plan has checked that the extents fit in int64
  const int64_t kbytes = d->batch * d->n_heads_k * d->seq_len_k * d->head_dim * 2;
  if (kbytes > kNoAllocKBytes) return ROPE_ERR_SHAPE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ROPE_ERR_HIP;
  void* ws = device_scratch(dev);
  if (!ws) return ROPE_ERR_HIP;
  return rope_attention_fwd_k_once(d, ws, stream);
}

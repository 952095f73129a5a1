/*
 * librope.h -- fused rotary position embedding (RoPE) for AMD MI355X (gfx950).
 *
 * C ABI. Every entry point validates its arguments on the host, then enqueues
 * GPU work on the caller's HIP stream and returns; nothing here waits for the
 * GPU, allocates device memory or falls back to another implementation.
 *
 * What is computed. For each token (b, s) at position p and each pair
 * (x1, x2) of the first R dims of every head row,
 *
 *     forward : (x1, x2) <- (x1*cos[p,i] - x2*sin[p,i], x1*sin[p,i] + x2*cos[p,i])
 *     backward: (x1, x2) <- (x1*cos[p,i] + x2*sin[p,i], -x1*sin[p,i] + x2*cos[p,i])
 *
 * ("Rotary Embedding Kernel", Overview: the pair rotation, applied per
 * position along the sequence. How Unsloth Optimizes RoPE Embedding
 * Computations in Triton Kernels, Frequently Asked Questions: the backward
 * pass is the forward kernel under a flag; for a rotation that is the
 * transpose, i.e. sin negated.) Arithmetic is float32 for every storage
 * dtype; each result is rounded once to the storage dtype, nearest-even.
 *
 * Pairs ("Rotary Embedding Kernel", Paired Element Layout):
 *     ROPE_SPLIT_HALF  : (x[i], x[i + R/2]),  i < R/2
 *     ROPE_INTERLEAVED : (x[2i], x[2i + 1]),  i < R/2
 * Dims R .. D-1 are never read or written (rotary-embedding-torch docs, Key
 * Parameters: `dim` is the width of the rotated part).
 *
 * Positions (How Unsloth Optimizes RoPE ..., Support for Custom Position IDs
 * and Custom Position IDs for Prefix-Tuning; rotary-embedding-torch docs,
 * flash_attn_with_rotary, skipping CLS/register tokens):
 *     pos == NULL : p = s
 *     pos != NULL : p = pos[b * pos_batch_stride + s]
 * A token whose p is < 0 or >= table_rows is left untouched (every dim keeps
 * its bits); that is how leading CLS/register tokens are skipped.
 *
 * Layouts:
 *     ROPE_BHSD : Q [batch, n_heads_q, seq_len, head_dim], K [batch, n_heads_k, ...]
 *                 (Unsloth page, Usage Examples)
 *     ROPE_BSHD : Q [batch, seq_len, n_heads_q, head_dim] (rotary-embedding-torch
 *                 docs, seq_before_head_dim)
 * Both dense and contiguous. GQA: 0 <= n_heads_k <= n_heads_q (Unsloth page,
 * Manual Triton Kernel Invocation, separate n_heads_K); 0 rotates Q only.
 *
 * Tables (How Unsloth Optimizes RoPE ..., Usage Examples: precomputed cos and
 * sin; "Rotary Embedding Kernel", Common Pitfalls: [seq_len, D/2], broadcast
 * over batch and heads): cos and sin are float32, row-major
 * [table_rows, R/2]; row p holds the values of position p. rope_build_table
 * fills them for the standard frequencies.
 *
 * Ownership and lifetime. Every pointer in a call is caller-owned. q, k, cos,
 * sin and pos are device memory on the current HIP device and must stay valid
 * until the enqueued work completes. q and k are modified in place and must
 * not overlap each other, nor the cos, sin and pos arrays, which must not
 * change while the work runs. The library keeps no mutable global state beyond a
 * per-device cache of the compute-unit count, filled once; calls are
 * reentrant and may be issued from several threads on different streams.
 *
 * Errors. A negative rope_status_t means nothing was enqueued (validation
 * errors), or that the launch itself failed (ROPE_ERR_HIP, reported by
 * hipGetLastError right after the launch). Index values are device data and
 * are not inspected on the host: an out-of-range index is not an error, the
 * token simply passes through.
 */
#ifndef LIBROPE_H
#define LIBROPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rope_status {
  ROPE_OK = 0,
  ROPE_ERR_NULL = -1,   /* a required pointer is NULL */
  ROPE_ERR_SHAPE = -2,  /* a size is negative or inconsistent */
  ROPE_ERR_DTYPE = -3,  /* unknown dtype code */
  ROPE_ERR_LAYOUT = -4, /* unknown layout, pairing or launch-shape code */
  ROPE_ERR_ALIGN = -5,  /* q/k data not aligned to its element size, cos or sin
                           not 16-byte aligned, or pos not 4-byte aligned */
  ROPE_ERR_ALIAS = -6,  /* written data overlaps other operands (see the calls) */
  ROPE_ERR_HIP = -7     /* the HIP runtime reported an error */
} rope_status_t;

typedef enum rope_dtype { ROPE_F32 = 0, ROPE_F16 = 1, ROPE_BF16 = 2 } rope_dtype_t;
typedef enum rope_layout { ROPE_BHSD = 0, ROPE_BSHD = 1 } rope_layout_t;
typedef enum rope_pairing { ROPE_SPLIT_HALF = 0, ROPE_INTERLEAVED = 1 } rope_pairing_t;

/* Which grid shape to launch. AUTO walks memory in order: the token shape
 * when a token's heads are adjacent ([B,S,H,D], packed QKV) and at decode
 * (seq_len 1), the rows shape for [B,H,S,D] unless there are too few tokens
 * to fill the device; within each, AUTO may also pick a form that only it
 * launches (one (token, head) chunk per lane for [B,H,S,D] split-half calls,
 * items over the whole call, token by token, for token-major interleaved
 * calls with rotated spans up to 256 bytes and split-half calls with spans
 * up to 128 bytes, where a token's heads are adjacent). Every
 * shape runs the same per-pair arithmetic and gives bit-identical results;
 * ROWS and TOKEN force the named shape's general kernels (for comparisons). */
typedef enum rope_launch {
  ROPE_LAUNCH_AUTO = 0,
  ROPE_LAUNCH_ROWS = 1,  /* lanes over (token, chunk), loop over heads */
  ROPE_LAUNCH_TOKEN = 2  /* a few tokens per workgroup, lanes over (token, head, chunk) */
} rope_launch_t;

/* Where rope_apply takes cos and sin from. */
typedef enum rope_angles {
  ROPE_ANGLES_TABLE = 0, /* the caller's cos/sin tables */
  ROPE_ANGLES_THETA = 1  /* computed in the kernel from theta and interpolate_factor */
} rope_angles_t;

typedef struct rope_desc {
  int64_t batch;       /* B >= 0 */
  int64_t n_heads_q;   /* Hq >= 0 */
  int64_t n_heads_k;   /* Hk, 0 <= Hk <= Hq for the _qk calls; ignored by the _q calls */
  int64_t seq_len;     /* S >= 0 */
  int64_t head_dim;    /* D >= 0 */
  int64_t rotary_dim;  /* R, even, 0 <= R <= D */
  int32_t dtype;       /* rope_dtype_t: storage type of q and k */
  int32_t layout;      /* rope_layout_t */
  int32_t pairing;     /* rope_pairing_t */
  int32_t launch;      /* rope_launch_t; 0 = automatic */
  const float *cos;    /* device, float32 [table_rows, R/2], 16-byte aligned */
  const float *sin;    /* device, float32 [table_rows, R/2], 16-byte aligned */
  int64_t table_rows;  /* rows of cos and sin (the largest position + 1) */
  const int32_t *pos;  /* device int32 indices, or NULL for p = s */
  int64_t pos_batch_stride; /* index of token (b, s) is pos[b * stride + s]; 0 shares one row */
} rope_desc_t;

/* Forward RoPE on Q and K in one launch, in place (How Unsloth Optimizes
 * RoPE ..., Triton Kernel Architecture for RoPE: one kernel rotates the query
 * and key heads of a token together, so each cos/sin row is read once for
 * both; Manual Triton Kernel Invocation: Q, K, cos, sin, optional int32
 * positions and the number of K heads are its arguments).
 * q: device, d->dtype elements in d->layout, shape with n_heads_q heads.
 * k: device, same with n_heads_k heads; must not overlap q.
 * ROPE_ERR_ALIAS when q and k overlap, or either overlaps cos, sin or the
 * index entries the call reads.
 * stream: a hipStream_t, or NULL for the null stream.
 * Returns ROPE_OK, a validation error (nothing enqueued) or ROPE_ERR_HIP.
 * Empty work (batch, seq_len, all heads or rotary_dim zero) returns ROPE_OK
 * and enqueues nothing. */
rope_status_t rope_fwd_qk(void *q, void *k, const rope_desc_t *d, void *stream);

/* Backward of rope_fwd_qk: rotates incoming gradients dq, dk in place by the
 * opposite angle (How Unsloth Optimizes RoPE ..., Frequently Asked Questions:
 * the backward pass runs the same kernel with its backward flag set). Same
 * arguments and errors as rope_fwd_qk. */
rope_status_t rope_bwd_qk(void *dq, void *dk, const rope_desc_t *d, void *stream);

/* Forward RoPE on Q only (How Unsloth Optimizes RoPE ..., Triton Kernel
 * Architecture for RoPE: the query-only kernel). d->n_heads_k is ignored. */
rope_status_t rope_fwd_q(void *q, const rope_desc_t *d, void *stream);

/* Backward of rope_fwd_q. */
rope_status_t rope_bwd_q(void *dq, const rope_desc_t *d, void *stream);

/* ------------------------------------------------------------------------
 * General form: strided views, out-of-place, other table layouts.
 *
 * The usual call site rotates Q and K where a fused projection left them,
 * e.g. as views into one packed QKV buffer, without first copying them to
 * contiguous tensors (How Unsloth Optimizes RoPE ..., Manual Triton Kernel
 * Invocation: the kernel takes explicit strides for the batch, head and
 * sequence dims). rope_apply takes every tensor as a strided view and can
 * write its result to separate outputs.
 */

/* A view of a 4-d tensor indexed [batch, head, seq, dim]. The dim axis is
 * contiguous (stride 1); the other three strides are in elements, >= 0.
 * Element (b, h, s, j) is at data + (b*stride_b + h*stride_h + s*stride_s + j)
 * elements. */
typedef struct rope_view {
  void *data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_s;
} rope_view_t;

typedef struct rope_apply_desc {
  int64_t batch;        /* B >= 0 */
  int64_t seq_len;      /* S >= 0 */
  int64_t head_dim;     /* D >= 0 */
  int64_t rotary_dim;   /* R, even, 0 <= R <= D */
  int64_t n_heads_q;    /* Hq >= 0 */
  int64_t n_heads_k;    /* 0 <= Hk <= Hq; 0 rotates Q only */
  int32_t dtype;        /* rope_dtype_t */
  int32_t pairing;      /* rope_pairing_t */
  int32_t launch;       /* rope_launch_t */
  int32_t direction;    /* +1 forward, -1 backward (sin negated) */
  rope_view_t q_in;     /* device */
  rope_view_t k_in;     /* device; ignored when n_heads_k == 0 */
  rope_view_t q_out;    /* data NULL: write back into q_in (in place) */
  rope_view_t k_out;    /* data NULL: write back into k_in (in place) */
  const float *cos;     /* device, 16-byte aligned */
  const float *sin;     /* device, 16-byte aligned */
  int64_t table_rows;   /* rows of cos and sin */
  /* Frequency i of position p is read at cos[p*table_row_stride + i*table_col_stride]:
   *   [rows, R/2]                       row stride R/2 (or 0), col stride 1
   *   [rows, R] halves duplicated       row stride R,          col stride 1
   *     (cos(cat(f, f)), the split-half convention of many model codes)
   *   [rows, R] each value repeated     row stride R,          col stride 2
   *     (repeat_interleave, the interleaved convention)           */
  int64_t table_row_stride;  /* floats; 0 means R/2 */
  int64_t table_col_stride;  /* 1 or 2 */
  const int32_t *pos;        /* device int32 indices or NULL (p = s) */
  int64_t pos_batch_stride;
  /* angles == ROPE_ANGLES_THETA: no tables. cos, sin and the table strides
   * are ignored (cos and sin may be NULL); table_rows only bounds the
   * positions (an index >= table_rows passes through, as with tables).
   * Frequency i of position p is cos/sin of (p / interpolate_factor) *
   * theta^(-2i/R) (rotary-embedding-torch docs, Key Parameters: `theta` is
   * the frequency base, `interpolate_factor` scales the positions, here as a
   * divisor), computed in binary64 and rounded once to float32 per value:
   * the values rope_build_table would store, except where an exact value
   * lies within ~1e-15 relative of a float32 rounding boundary. */
  double theta;              /* > 0, finite */
  double interpolate_factor; /* > 0, finite; 1 = positions as given */
  int32_t angles;            /* rope_angles_t */
  int32_t reserved;          /* set to 0 */
} rope_apply_desc_t;

/* Rotate Q (and K) as described by `d`, in place or out of place, on `stream`.
 * Same arithmetic, pairing and index rules as rope_fwd_qk. Out of place, the
 * outputs receive every element: rotated dims and, bit for bit, dims >= R
 * and the rows of tokens whose index is out of range. Outputs must not
 * overlap each other or any input, except that an output may be exactly its
 * own input (same pointer and strides), which is the in-place case. Two
 * views overlap when they could address a common element; Q and K views
 * that interleave token by token (packed QKV) without sharing elements are
 * accepted. No written view may meet the byte range of cos, sin or the index
 * entries the call reads. Any of these is ROPE_ERR_ALIAS.
 * Errors: as rope_fwd_qk; ROPE_ERR_SHAPE also for negative strides, a table
 * stride that cannot hold R/2 frequencies, or (ROPE_ANGLES_THETA) a theta
 * or interpolate_factor that is not finite and > 0, or R > 8192;
 * ROPE_ERR_LAYOUT for a direction other than +-1, a table column stride
 * other than 1 or 2, or an unknown `angles`;
 * ROPE_ERR_ALIGN when a view's data is not aligned to its element size, cos
 * or sin is not 16-byte aligned, or pos is not 4-byte aligned. */
rope_status_t rope_apply(const rope_apply_desc_t *d, void *stream);

/* ------------------------------------------------------ XPOS scaling
 * rope_apply with XPOS scaling (rotary-embedding-torch docs, Key Parameters:
 * `use_xpos`, Extrapolatable Positional Encoding for length extrapolation).
 * After the rotation, both elements of pair i of a query row at position p
 * are multiplied by xpos_q[p*row + i*col] and those of a key row by
 * xpos_k[...], with row/col the table strides of cos and sin; for the xPos
 * paper's scales these hold zeta_i^e and zeta_i^-e (rope_build_xpos_table),
 * so a query at n and a key at m meet with the factor zeta_i^((n-m)/B). The
 * pages name XPOS without its formula; the one used is the xPos paper's
 * (Sun et al., "A Length-Extrapolatable Transformer", ACL 2023).
 *   - y = RN32(RN32(rotation) * factor), then rounded to the dtype; the
 *     rotation is rope_apply's. A factor does not change within a pair, so
 *     it commutes with the rotation: direction = -1 (the backward) uses the
 *     same tables.
 *   - d as for rope_apply, with angles = ROPE_ANGLES_TABLE and launch =
 *     ROPE_LAUNCH_AUTO (ROPE_ERR_LAYOUT otherwise). xpos_q / xpos_k: device
 *     float32, 4-byte aligned, laid out like cos and sin; NULL only when
 *     there are no Q (resp. K) heads. A skipped token (index out of the
 *     table) is not scaled either.
 * Errors as rope_apply, and ROPE_ERR_NULL / ROPE_ERR_ALIGN / ROPE_ERR_ALIAS
 * for the factor tables (a written view may not overlap them). */
rope_status_t rope_apply_xpos(const rope_apply_desc_t *d, const float *xpos_q,
                              const float *xpos_k, void *stream);

/* Fill host float32 tables xpos_q / xpos_k, each [table_rows, R/2] row-major:
 * row p, column i holds zeta_i^e and zeta_i^-e with
 * zeta_i = (2i/R + gamma) / (1 + gamma) and e = (p - center) / scale_base,
 * formed in binary64 and rounded once to float32 (the xPos paper uses
 * gamma = 0.4, scale_base = 512; center 0 gives its exponent p / B, and a
 * center near the middle of the positions keeps both tables in range for
 * long sequences). Host memory, caller-owned. ROPE_ERR_SHAPE for a negative
 * size, an odd rotary_dim, or a scale_base or gamma that is not finite and
 * > 0, or a center that is not finite; ROPE_ERR_NULL for NULL outputs with
 * non-empty work. */
rope_status_t rope_build_xpos_table(float *xpos_q, float *xpos_k, int64_t table_rows,
                                    int64_t rotary_dim, double scale_base, double gamma,
                                    double center);

/* ---------------------------------------------- attention with RoPE fused
 * Attention whose Q and K are rotated inside the kernel, on the blocks it
 * loads, so no rotated Q or K is written to memory (rotary-embedding-torch
 * docs, flash_attn_with_rotary; GQA repeats the K/V heads; is_causal):
 *   O[b,h] = softmax(scale * rope(Q[b,h]) rope(K[b,h'])^T  [causal mask]) V[b,h']
 * with h' = h / (Hq / Hk). rope() is the rotation of rope_fwd_qk (same
 * table, pairing, positions and float32 arithmetic), its results rounded to
 * bf16 as that call would store them: the output equals rope_fwd_qk on Q and
 * K followed by the same attention with `rotate` = 0.
 *   - Q [B, Hq, Sq, D], K and V [B, Hk, Sk, D], O [B, Hq, Sq, D]: dense,
 *     contiguous, bf16, 16-byte aligned. O must not overlap any input.
 *   - positions: q_pos / k_pos as in rope_desc_t (per batch stride), or NULL:
 *     key j at j, query i at i + Sk - Sq; out-of-table indices pass through.
 *   - causal: key j is visible to query i when j <= i + Sk - Sq (needs
 *     Sq <= Sk). A query with no visible key (Sk = 0) gets zeros; K and V
 *     may then be NULL.
 *   - scale: 0 means 1 / sqrt(head_dim). Any sign; |scale| * log2(e) must
 *     be a normal float32, and the scaled scores must stay finite in float32.
 * Matrix-core kernel: the products run as bf16 with float32 accumulation and
 * the softmax weights are rounded to bf16 before they multiply V.
 * Limits: head_dim 64 or 128; split-half pairs need R % 32 == 0 and
 * interleaved pairs R % 8 == 0 (R = 0: no rotation); one head's K (and V)
 * rows, Sk * D * 2 bytes, and a cos/sin table, table_rows * R/2 * 4 bytes,
 * each under 4 GiB (the kernel addresses inside them with 32-bit offsets). */
typedef struct rope_attn_desc {
  int64_t batch;
  int64_t n_heads_q;    /* Hq >= 1 */
  int64_t n_heads_k;    /* Hk >= 1, Hq % Hk == 0 */
  int64_t seq_len_q;    /* Sq >= 0 */
  int64_t seq_len_k;    /* Sk >= 0 */
  int64_t head_dim;     /* D: 64 or 128 */
  int64_t rotary_dim;   /* R, even, <= D (see the limits above) */
  int32_t dtype;        /* ROPE_BF16 */
  int32_t pairing;      /* rope_pairing_t */
  int32_t causal;       /* 0 or 1 */
  int32_t rotate;       /* 1: rotate Q and K; 0: plain attention */
  const void *q;
  const void *k;
  const void *v;
  void *o;
  const float *cos;     /* [table_rows, R/2], 16-byte aligned; unused if rotate == 0 */
  const float *sin;
  int64_t table_rows;
  const int32_t *q_pos;
  int64_t q_pos_batch_stride;
  const int32_t *k_pos;
  int64_t k_pos_batch_stride;
  double scale;
  int32_t k_rotated;    /* 1: K already holds rope(K) (e.g. from rope_fwd_qk); only Q
                           is rotated in the kernel. 0: both (the fused form) */
  int32_t reserved;     /* set to 0 */
} rope_attn_desc_t;

/* Enqueue the fused attention on `stream`. Errors as rope_apply:
 * ROPE_ERR_DTYPE for a dtype other than bf16, ROPE_ERR_SHAPE for sizes
 * outside the limits above (or Hq % Hk != 0, or causal with Sq > Sk, or a
 * scale that is not finite or whose |scale| * log2(e) is not a normal float32,
 * or positions without an index reaching table_rows),
 * ROPE_ERR_LAYOUT for an unknown pairing, ROPE_ERR_ALIGN, ROPE_ERR_ALIAS when
 * O overlaps an input. */
rope_status_t rope_attention_fwd(const rope_attn_desc_t *d, void *stream);

/* The same attention with K rotated once instead of once per workgroup:
 * rope_apply writes rope(K) into the caller's `k_workspace` (device,
 * 16-byte aligned, B*Hk*Sk*D bf16 elements, laid out like K), then
 * rope_attention_fwd runs on it with k_rotated = 1, both on `stream`. The
 * result equals rope_attention_fwd's bit for bit. On long sequences, where
 * many workgroups read each K tile, this is the faster form. For callers
 * that can spare a K-sized buffer; the library still allocates nothing.
 * Errors as rope_attention_fwd (d->k_rotated must be 0), and ROPE_ERR_NULL /
 * ROPE_ERR_ALIGN / ROPE_ERR_ALIAS for a missing or misaligned workspace or
 * one that overlaps any operand. With no rotation (rotate = 0 or R = 0) the
 * workspace is not touched. */
rope_status_t rope_attention_fwd_k_once(const rope_attn_desc_t *d, void *k_workspace,
                                        void *stream);

/* rope_attention_fwd_k_once without a caller workspace, for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): rope(K) is staged in a device array the
 * library holds, 64 MiB per device (K of up to 32 Mi bf16 values, e.g.
 * [4, 8, 8192, 128]), set aside when the library's code is loaded on a device
 * and kept until the process ends. This call allocates nothing.
 * Same descriptor, result (bit for bit) and errors as
 * rope_attention_fwd_k_once, plus ROPE_ERR_SHAPE when B * Hk * Sk * D bf16
 * values exceed 64 MiB, and ROPE_ERR_HIP when the array's address cannot be
 * obtained. Every call on one device uses the same array: calls that overlap
 * on one device (different streams, or different host threads, with no
 * ordering between them) race and give wrong results; calls ordered on one
 * stream do not. The array keeps the last call's rope(K); each call writes
 * all of the part it reads before reading it. */
rope_status_t rope_attention_fwd_k_once_noalloc(const rope_attn_desc_t *d, void *stream);

/* Fill host float32 tables cos_out/sin_out, each [table_rows, R/2] row-major,
 * with cos and sin of (p / interpolate_factor) * theta^(-2i/R) for row p and
 * column i: the exponent -2i/R, the scaled position and the angle are formed
 * in binary64 and each entry is rounded once to float32 (rotary-embedding-torch
 * docs, Key Parameters: `theta` is the base of the frequencies, default
 * 10000; `interpolate_factor` scales the positions, default 1; "Rotary
 * Embedding Kernel": cos/sin are precomputed). Host memory, caller-owned;
 * runs on the calling thread.
 * Returns ROPE_ERR_NULL for NULL outputs with non-empty work and
 * ROPE_ERR_SHAPE for a negative size, an odd rotary_dim, or a theta or
 * interpolate_factor that is not finite and > 0. */
rope_status_t rope_build_table(float *cos_out, float *sin_out, int64_t table_rows,
                               int64_t rotary_dim, double theta, double interpolate_factor);

/* Which kernel and grid rope_fwd_qk (with_k != 0) or rope_fwd_q (with_k ==
 * 0) would launch for these arguments on the current device, as one line of
 * text ("rope_head_lanes_kernel dtype=bf16 vec=8 ... grid=10240 block=512
 * ..."; the kernel name is the one traces show). For benchmarks and
 * diagnostics: nothing is enqueued, q and k are not dereferenced, and the
 * backward calls launch the same kernel. buf: host memory of len bytes,
 * always NUL-terminated. Errors as rope_fwd_qk (validation), ROPE_ERR_NULL
 * for a NULL or empty buf, ROPE_ERR_HIP when there is no current device. */
rope_status_t rope_describe(const void *q, const void *k, const rope_desc_t *d, int with_k,
                            char *buf, int64_t len);

/* A static, human-readable name for a status code ("unknown status" for
 * codes this library never returns). */
const char *rope_status_string(rope_status_t s);

/* Library version, major * 10000 + minor * 100 + patch. */
int rope_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBROPE_H */

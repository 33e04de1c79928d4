/*
 * ttt_attn.h - C ABI of the TTT sparse tree attention library (MI355X / gfx950).
 *
 * The operation is softmax attention under the mask of the SpecForge paper review,
 * "§3 Technical architecture -> Compute optimisation -> Sparse Tree Attention ->
 * BlockMask construction algorithm" (restated in "§4 Core formulas -> BlockMask
 * construction"), used when an EAGLE-3 draft model is trained with training-time
 * test (TTT):
 *
 *   M_causal = (q_i >= kv_i) and (kv_i < T)
 *   M_suffix = (kv_i >= Q_LEN) and (kv_i mod Q_LEN < T) and ((kv_i - q_i) mod Q_LEN == 0)
 *   M        = M_causal or M_suffix
 *
 * Query row i (0 <= i < Q_LEN) of TTT step k sees keys 0..min(i, T-1) of block 0 and,
 * when i < T, key t*Q_LEN + i of every later block t = 1..k.  Padded rows (i >= T) see
 * keys 0..T-1.  A row with no visible key (T == 0) gets o = 0 and lse = -inf.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layouts   contiguous, row-major:
 *              q, o, dout, dq      [B, Hq,  Q_LEN, d]
 *              k, v, dk, dv        [B, Hkv, (k+1)*Q_LEN, d]   (block t = rows [t*Q_LEN, (t+1)*Q_LEN))
 *              lse                 [B, Hq,  Q_LEN]  fp32, natural log
 *              seq_T               [B] int32, device memory, one valid length per sequence
 *            Query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups).
 *  Pointers  All tensors and the workspace are device memory owned by the caller; base
 *            addresses must be 16-byte aligned.  The library never allocates, frees or
 *            synchronises and keeps no state between calls (except the optional timing
 *            records below).  Concurrent calls need distinct workspaces.
 *  Outputs   write-only and fully overwritten: o, lse, dq, dk, dv.  dk/dv rows that no
 *            query sees are written 0.  Gradients are not accumulated across calls.
 *  seq_T     read on the device only; values outside [0, Q_LEN] are clamped into it.
 *  Streams   all work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *            The return value reports argument validation and launch status only.
 *  Errors    0 on success, else one of the negative TTT_E_* codes; nothing is launched
 *            when validation fails.  No exception crosses the ABI.
 */
#ifndef TTT_ATTN_H
#define TTT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ttt_attn_dtype {
  TTT_DTYPE_F32 = 0,  /* fp32 tensors, fp32 arithmetic (VALU)                       */
  TTT_DTYPE_BF16 = 1  /* bf16 tensors, bf16 MFMA with fp32 accumulation; lse in fp32 */
};

/*
 * Path selection (ttt_attn_params.flags; bf16 only, the fp32 path ignores them).  All paths
 * give the same result up to rounding.  0 = default:
 *   - forward: the diagonal keys of blocks 1..k are merged inside the causal kernel, which
 *     writes the final o and lse (no fp32 intermediate state);
 *   - backward: the dK/dV kernel stores dS of block 0 (bf16, in the workspace) and the dQ
 *     kernel computes dQ = scale * dS K from it, one matrix product per tile.
 * TTT_FLAG_SEPARATE_SUFFIX: the forward's causal kernel writes an fp32 state (o_c, lse_c)
 *   that the standalone bandwidth-bound suffix kernel merges (the fp32 path always does so).
 * TTT_FLAG_RECOMPUTE_DQ: no stored dS (a much smaller backward workspace); the dQ kernel
 *   recomputes S and dP, three products per tile.  dk/dv are bitwise the same either way.
 * TTT_FLAG_DENSE_DIAGONAL (a measurement variant, not for production): the diagonal keys go
 *   through the matrix cores as masked tiles, the way a block-sparse mask (FlexAttention's
 *   BlockMask) would evaluate them.  Forward: two masked 64-key tiles per block t per 128-query
 *   tile instead of the per-row merge.  Backward (k > 0): extra workgroups of the dK/dV kernel,
 *   one per 128-key tile of each block t, take the 128 queries of that tile as masked tiles,
 *   and the dQ kernel recomputes S and dP over the causal tiles and two masked tiles per
 *   block t, writing the final dq (no suffix kernel, no stored dS).  Cannot be combined with
 *   TTT_FLAG_SEPARATE_SUFFIX; the whole-TTT backward ignores it.
 * TTT_FLAG_FUSED_SUFFIX_BWD (backward, k > 0): the dK/dV workgroup of each 128-key tile of
 *   block 0 also computes the suffix key rows t*Q_LEN + i (t = 1..k) of the same rows i: their
 *   dK/dV, and the fp32 dQ term of each head, which the stored-dS dQ kernel adds before it
 *   writes the final dq (no suffix kernel).  Not with TTT_FLAG_RECOMPUTE_DQ or
 *   TTT_FLAG_DENSE_DIAGONAL; the whole-TTT backward ignores it.
 * Otherwise, in the backward the suffix kernel adds the diagonal keys' terms for k > 0.  The
 * workspace sizes below depend on the flags.
 */
enum ttt_attn_flags {
  TTT_FLAG_SEPARATE_SUFFIX = 1,
  TTT_FLAG_RECOMPUTE_DQ = 2,
  TTT_FLAG_DENSE_DIAGONAL = 4,
  TTT_FLAG_FUSED_SUFFIX_BWD = 8
};

enum ttt_attn_status {
  TTT_OK = 0,
  TTT_E_NULL = -1,        /* a required pointer is NULL                              */
  TTT_E_SHAPE = -2,       /* non-positive size, Hq % Hkv != 0, ttt_step < 0, scale <= 0, overflow */
  TTT_E_UNSUPPORTED = -3, /* head_dim/dtype/q_len combination not built (see below)  */
  TTT_E_ALIGN = -4,       /* a pointer is not 16-byte aligned                        */
  TTT_E_WORKSPACE = -5,   /* workspace smaller than *_workspace_size()               */
  TTT_E_HIP = -6,         /* a kernel launch failed (hipGetLastError)                */
  TTT_E_SCRATCH = -7      /* ttt_attn_bwd_noalloc: the call needs more than TTT_NOALLOC_SCRATCH_BYTES */
};

/*
 * Problem description.  Supported combinations:
 *   dtype F32 : head_dim in {64, 128}, any q_len >= 1 (vector-ALU kernels).
 *   dtype BF16: head_dim in {64, 128}, any q_len >= 1.  head_dim 128 with q_len a multiple of
 *               128 runs on the matrix-core kernels (the fast path).  head_dim 64 with q_len a
 *               multiple of 128 runs on the same kernels through head_dim-128 copies of the
 *               rows whose upper half is zero (exact: the zero half adds nothing to any sum),
 *               which the workspace (ttt_attn_bwd_noalloc: its scratch array) holds; the flags
 *               below apply to both.  The whole-TTT calls take these two; other bf16 shapes
 *               run on the vector-ALU kernels (bf16 storage, fp32 arithmetic).
 * scale multiplies q.k before masking (1/sqrt(head_dim) in the usual setting); it must be
 * finite and positive (the streaming softmax tracks the row maximum of the raw q.k).
 */
typedef struct ttt_attn_params {
  int32_t batch;     /* B                                  */
  int32_t heads_q;   /* Hq                                 */
  int32_t heads_kv;  /* Hkv, divides Hq                    */
  int32_t q_len;     /* Q_LEN                              */
  int32_t head_dim;  /* d                                  */
  int32_t ttt_step;  /* k >= 0; the KV length is (k+1)*Q_LEN */
  float scale;
  int32_t dtype;     /* enum ttt_attn_dtype                */
  int32_t flags;     /* enum ttt_attn_flags; unknown bits -> TTT_E_UNSUPPORTED */
} ttt_attn_params;

/* Bytes of device workspace the call needs (0 when the params are invalid). */
size_t ttt_attn_fwd_workspace_size(const ttt_attn_params* p);
size_t ttt_attn_bwd_workspace_size(const ttt_attn_params* p);

/*
 * The default bf16 backward workspace holds the dS of block 0: B * Hq * n(n+1)/2 blocks of
 * 2 KB, n = Q_LEN / 32 (1.08 GB at B 2, Hq 32, Q_LEN 4096); TTT_FLAG_RECOMPUTE_DQ avoids it.
 * It also holds the dK/dV kernel's work-queue counters, another reason why calls in flight
 * at the same time need distinct workspaces.  At bf16 head_dim 64 on the matrix-core kernels
 * it starts with head_dim-128 copies of q, k, v, o (backward: also dout, dq, dk, dv).
 */

/*
 * Forward: o = softmax_M(scale * q k^T) v and lse = log sum_{j in M} exp(scale * q.k_j).
 * Streaming softmax (the review's §3 "Sparse Tree Attention": computed flash-style so the
 * logits are never stored): the causal block 0 runs as tiled MFMA with fully masked
 * tiles skipped; the diagonal suffix keys of blocks 1..k are gathered per query and
 * merged into the same softmax state.
 */
int ttt_attn_fwd(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                 const int32_t* seq_T, void* o, float* lse, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * Backward: gradients of sum(dout * o) for the o/lse produced by ttt_attn_fwd on the same
 * inputs.  The review's §3 "Sparse Tree Attention" computes the attention flash-style so the
 * logits are never stored; so P is recomputed here from lse (nothing else is saved by the
 * forward), and the softmax Jacobian, the identity the review's §4 "In-place backward" writes
 * out for the loss, gives dS = P * (dP - rowsum(dout * o)) with dP = dout v^T; then
 * dq = scale * dS k, dk = scale * dS^T q, dv = P^T dout.  dk/dv of every KV row are produced by
 * exactly one workgroup summing the query heads of its GQA group in a fixed order (bitwise
 * deterministic).  dq rows are likewise owned by one workgroup each.
 * Arguments: p, q, k, v, seq_T as for ttt_attn_fwd; o and lse the forward's outputs; dout
 * the gradient of o (layout of q); dq (layout of q), dk and dv (layout of k) are written;
 * workspace of at least ttt_attn_bwd_workspace_size(p) bytes.  Errors as for ttt_attn_fwd.
 */
int ttt_attn_bwd(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                 const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Whole TTT sweep (bf16 only): the K = p->ttt_step + 1 steps of one TTT unroll over a single
 * KV cache, without per-step copies of the cache.  Layouts (contiguous):
 *   q, o, dout, dq   [K, B, Hq, Q_LEN, d]     step-major: step k's tensors of the per-step API
 *   lse              [K, B, Hq, Q_LEN]
 *   k, v, dk, dv     [B, Hkv, K*Q_LEN, d]     the cache: block t = rows [t*Q_LEN, (t+1)*Q_LEN)
 * Step k attends rows [0, (k+1)*Q_LEN) of the cache under the mask above (block 0 causal,
 * blocks 1..k diagonal).  The forward writes o and lse of every step.  The backward writes dq
 * of every step and the total gradient of the cache, dk/dv = sum over the steps k of step
 * k's dK/dV (block t receives the diagonal gradients of every step k >= t, block 0 the causal
 * gradient of all of them); every sum is kept in fp32 inside the kernels (block 0's in one
 * dK/dV launch over the queries of all steps, blocks 1..k in one suffix launch over all steps)
 * and rounded to bf16 once.  The backward's workspace holds D, lse * log2(e), the fp32 block-0
 * dQ of steps 1..k and (stored-dS path) the dS blocks of every step: 8.5 GB at B 2, Hq 32,
 * Q_LEN 4096, K 7, against 0.95 GB with TTT_FLAG_RECOMPUTE_DQ (which then recomputes S and dP
 * in the dQ kernel, about 6% more time for that workload).
 * Launches run in order on `stream`; flags select the paths as for the per-step calls.
 * Same error codes; fp32 data returns TTT_E_UNSUPPORTED.
 */
size_t ttt_attn_fwd_sweep_workspace_size(const ttt_attn_params* p);
size_t ttt_attn_bwd_sweep_workspace_size(const ttt_attn_params* p);
int ttt_attn_fwd_sweep(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_T, void* o, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);
int ttt_attn_bwd_sweep(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * No-allocation backward, for callers that cannot allocate device memory or take a workspace
 * argument (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as ttt_attn_bwd without the workspace: the
 * backward's scratch (D, lse * log2(e), split dK/dV partials, the fp32 dQ accumulator, and at
 * bf16 head_dim 64 the zero-padded head_dim-128 copies of the rows) lives in
 * a device array of TTT_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the dQ kernel recomputes S and dP (TTT_FLAG_RECOMPUTE_DQ is implied:
 * the stored-dS path needs a logits-sized buffer), so dq, dk and dv are bitwise those of
 * ttt_attn_bwd with that flag.  The call allocates nothing, apart from hipEvents when the
 * timing API below is enabled.  Calls whose scratch need exceeds the maximum return
 * TTT_E_SCRATCH before anything is launched (the five workloads of this library, up to
 * B 8 x Hq 32 x Q_LEN 2048 and B 2 x Hq 32 x Q_LEN 4096, fit).  The array belongs to the
 * current HIP device, which must be the device of `stream` and of the tensors; the first call
 * on a device looks up the array's address (hipGetSymbolAddress) and is best made before any
 * graph capture, later calls only enqueue kernels.  Every call on
 * one GPU shares that GPU's array, so calls that may overlap on one GPU (several streams or
 * threads) race and must be ordered by the caller.
 */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)320 << 20)
int ttt_attn_bwd_noalloc(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                         const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, void* stream);

/* Static text for a status code. */
const char* ttt_attn_status_string(int status);

/*
 * ABI version (major * 100 + minor).  1.04 runs bf16 head_dim 64 with q_len a multiple of 128
 * on the matrix-core kernels (larger workspaces for those shapes); 1.03 added
 * ttt_attn_bwd_noalloc (with TTT_E_SCRATCH),
 * TTT_FLAG_FUSED_SUFFIX_BWD and ttt_attn_timing_flush, and made the timing calls thread-safe;
 * 1.02 changed the whole-TTT backward's workspace size.
 */
int ttt_attn_version(void);

/*
 * Optional per-kernel timing, for measurement.  When enabled, every kernel launch of
 * ttt_attn_fwd/bwd is bracketed by hipEvents on the launch stream; ttt_attn_timing_read
 * synchronises those events and returns, per kernel name, the number of launches and the
 * summed milliseconds since the last reset.  Off by default.  Thread-safe: launches from
 * several threads may be timed at once, and a read or reset counts the launches that have
 * returned from their library call by then (one still inside its call is counted by the next
 * read).  While enabled, each timed launch takes a pair of hipEvents from a pool that grows as
 * needed and lasts until the process ends.
 */
typedef struct ttt_attn_kernel_time {
  char name[48];
  int32_t launches;
  double total_ms;
} ttt_attn_kernel_time;

int ttt_attn_timing_enable(int on);                       /* returns previous setting      */
int ttt_attn_timing_read(ttt_attn_kernel_time* out, int max_entries); /* entries written, <0 on error */
void ttt_attn_timing_reset(void);
/*
 * Cold-cache timing: while timing is enabled and a buffer is set, every timed launch is
 * preceded (outside its events) by a kernel that overwrites `bytes` of `buf` with plain
 * stores, so each kernel starts with caches that hold none of its data (give more than the
 * 256 MB last-level cache).  buf is caller-owned device memory, 16-byte aligned, bytes a
 * non-zero multiple of 16 (else TTT_E_ALIGN); NULL turns it off.  The buffer is shared by every
 * thread's timed launches: launches on different streams then overwrite it concurrently.
 */
int ttt_attn_timing_flush(void* buf, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* TTT_ATTN_H */

// Internal launchers: one per kernel family, all asynchronous on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.cuh"

namespace ttt {

// Per-launch timing hook (implemented by the host library).  While timing is enabled it holds
// its own pair of events from the start of the launch to the end of the scope.
struct LaunchTimer {
  LaunchTimer(const char* name, hipStream_t st);
  ~LaunchTimer();
  const char* name_;
  hipStream_t st_;
  hipEvent_t start_, stop_;
  bool on_;
};

// Forward.
// final_out: o (bf16) and lse are final; for k > 0 the kernel merges the suffix keys itself
// (per-lane gather, or with dense_diagonal as masked matrix-core tiles).  Otherwise it writes
// the fp32 causal state (o_c, lse_c) for the suffix kernel.
hipError_t launch_fwd_causal_mfma(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                                  const int32_t* seq_T, void* o, float* lse, bool final_out,
                                  bool dense_diagonal, hipStream_t st);
template <typename T>
hipError_t launch_fwd_causal_valu(const Shape& s, const T* q, const T* k, const T* v,
                                  const int32_t* seq_T, void* o, float* lse, bool final_out,
                                  hipStream_t st);
template <typename T>
hipError_t launch_fwd_suffix(const Shape& s, const T* q, const T* k, const T* v,
                             const int32_t* seq_T, const float* oc, const float* lsec, T* o,
                             float* lse, hipStream_t st);


// Backward.
// D = rowsum(dout * o); with lse2 set also lse2 = lse * log2(e); with sched set also zeroes
// the dK/dV kernel's queue counters (sched[32 i], i < 8).
template <typename T>
hipError_t launch_bwd_rowdot(const Shape& s, const T* o, const T* dout, float* Dd,
                             const float* lse, float* lse2, unsigned* sched, hipStream_t st);
// lse2 = lse * log2(e) (from launch_bwd_rowdot); sched: the 8 queue counters (sched[32 i]),
// zero on entry (launch_bwd_rowdot sets them just before on the same stream).
// With dq_suf set (and k > 0) each workgroup also takes the suffix key rows t*Q_LEN + i of
// its key tile's rows i: their dK/dV, and the fp32 dQ term of every head written to dq_suf.
hipError_t launch_bwd_dkdv_mfma(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                                const bf16* dout, const float* lse2, const float* Dd,
                                const int32_t* seq_T, bf16* dk, bf16* dv, float* part,
                                int nsplit, bf16* ds_out, bool dense_diagonal, float* dq_suf,
                                unsigned* sched, hipStream_t st);
hipError_t launch_bwd_dkdv_reduce(const Shape& s, const float* part, int nsplit, bf16* dk,
                                  bf16* dv, hipStream_t st);
hipError_t launch_bwd_dq_mfma(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                              const bf16* dout, const float* lse, const float* Dd,
                              const int32_t* seq_T, void* dq, bool final_out,
                              bool dense_diagonal, hipStream_t st);
// final_out with dq_add: adds the fp32 term dq_add before the bf16 write.
hipError_t launch_bwd_dq_ds(const Shape& s, const bf16* k, const bf16* ds, const int32_t* seq_T,
                            void* dq, bool final_out, const float* dq_add, hipStream_t st);
template <typename T>
hipError_t launch_bwd_dkdv_valu(const Shape& s, const T* q, const T* k, const T* v,
                                const T* dout, const float* lse, const float* Dd,
                                const int32_t* seq_T, T* dk, T* dv, hipStream_t st);
template <typename T>
hipError_t launch_bwd_dq_valu(const Shape& s, const T* q, const T* k, const T* v, const T* dout,
                              const float* lse, const float* Dd, const int32_t* seq_T, void* dq,
                              bool final_out, hipStream_t st);
template <typename T>
hipError_t launch_bwd_suffix(const Shape& s, const T* q, const T* k, const T* v, const T* dout,
                             const float* lse, const float* Dd, const int32_t* seq_T,
                             const float* dq_acc, T* dq, T* dk, T* dv, hipStream_t st);
// Whole TTT (s.step = K - 1, s.KV = K * L): the diagonal keys of blocks 1..K-1 for the queries
// of steps 1..K-1 (stacked step after step); dq_acc holds the fp32 block-0 dQ of steps
// 1..K-1 and is overwritten; writes dq of steps 1..K-1 and dk/dv of blocks 1..K-1.
hipError_t launch_bwd_suffix_sweep(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                                   const bf16* dout, const float* lse, const float* Dd,
                                   const int32_t* seq_T, float* dq_acc, bf16* dq, bf16* dk,
                                   bf16* dv, hipStream_t st);

// bf16 rows of 64 elements into rows of 128 whose upper half is zero (pad), and the first 64
// elements of each 128-element row back (unpad); rows = number of rows.
hipError_t launch_pad64(const void* src, void* dst, size_t rows, hipStream_t st);
hipError_t launch_unpad64(const void* src, void* dst, size_t rows, hipStream_t st);

// Cache flush for measurement: overwrites `bytes` (a multiple of 16) of buf.
hipError_t launch_flush_fill(void* buf, size_t bytes, hipStream_t st);

// In-place masked softmax-loss gradient.
template <typename T>
hipError_t launch_loss_grad(int64_t rows, int V, T* z, const T* p, const float* g, float* loss,
                            hipStream_t st);

}  // namespace ttt

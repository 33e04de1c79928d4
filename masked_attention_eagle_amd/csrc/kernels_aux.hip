// Backward row term D_i = rowsum(dO_i * O_i) (bandwidth-bound), and the head_dim-64 row copies.
#include "launch.h"

namespace ttt {

// ----------------------------------------------------------------------------------------
// D_i = sum_d dO_i * O_i, the row term of the softmax Jacobian (dS = P * (dP - D)).
// 16 lanes per row.  With lse2 set it also writes lse_i * log2(e), the base-2 row offset of
// P = exp2(S * scale * log2(e) - lse * log2(e)), so that the matrix-core dK/dV kernel, whose
// lanes each meet 16 rows per tile, subtracts it without a multiply per element.  With sched
// set, workgroup 0 also sets the matrix-core dK/dV kernel's 8 queue counters (one per
// 128-byte line, sched[32 i]) to zero: that kernel runs next on the same stream.
// ----------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ o,
                                                     const T* __restrict__ dout,
                                                     float* __restrict__ Dd,
                                                     const float* __restrict__ lse,
                                                     float* __restrict__ lse2,
                                                     unsigned* __restrict__ sched, size_t nrows) {
  constexpr int E = D / 16;
  if (sched && blockIdx.x == 0 && threadIdx.x < 8) sched[32 * threadIdx.x] = 0u;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (row >= nrows) return;
  float a[E], c[E];
  load_vec<T, E>(o + row * D + sub * E, a);
  load_vec<T, E>(dout + row * D + sub * E, c);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc += a[e] * c[e];
  acc = sum16(acc);
  if (sub == 0) {
    Dd[row] = acc;
    if (lse2) lse2[row] = lse[row] * kLog2e;
  }
}

template <typename T>
hipError_t launch_bwd_rowdot(const Shape& s, const T* o, const T* dout, float* Dd,
                             const float* lse, float* lse2, unsigned* sched, hipStream_t st) {
  const size_t nrows = (size_t)s.B * s.Hq * s.L * s.nst;
  const dim3 grid((unsigned)((nrows + 15) / 16));
  LaunchTimer timer("bwd_rowdot", st);
  if (s.D == 64)
    rowdot_kernel<T, 64><<<grid, 256, 0, st>>>(o, dout, Dd, lse, lse2, sched, nrows);
  else
    rowdot_kernel<T, 128><<<grid, 256, 0, st>>>(o, dout, Dd, lse, lse2, sched, nrows);
  return hipGetLastError();
}
template hipError_t launch_bwd_rowdot<float>(const Shape&, const float*, const float*, float*,
                                             const float*, float*, unsigned*, hipStream_t);
template hipError_t launch_bwd_rowdot<bf16>(const Shape&, const bf16*, const bf16*, float*,
                                            const float*, float*, unsigned*, hipStream_t);

// bf16 rows of 64 elements (128 bytes) to rows of 128 whose upper half is zero, and back: the
// head_dim-64 problem on the matrix-core kernels, which tile a 128-element head.  One 16-byte
// chunk per thread and step; every index stays below rows * 16 (padded) or rows * 8.
__global__ __launch_bounds__(256) void pad64_kernel(const bf16x8* __restrict__ src,
                                                    bf16x8* __restrict__ dst, size_t rows) {
  const size_t n = rows * 16, stride = (size_t)gridDim.x * 256;
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (bf16)0.f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const size_t r = i >> 4;
    const int c = (int)(i & 15);
    dst[i] = c < 8 ? src[r * 8 + c] : z;
  }
}

__global__ __launch_bounds__(256) void unpad64_kernel(const bf16x8* __restrict__ src,
                                                      bf16x8* __restrict__ dst, size_t rows) {
  const size_t n = rows * 8, stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    dst[i] = src[(i >> 3) * 16 + (i & 7)];
}

hipError_t launch_pad64(const void* src, void* dst, size_t rows, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const size_t blocks = (rows * 16 + 255) / 256;
  LaunchTimer timer("pad64", st);
  pad64_kernel<<<dim3((unsigned)(blocks < 16384 ? blocks : 16384)), 256, 0, st>>>(
      reinterpret_cast<const bf16x8*>(src), reinterpret_cast<bf16x8*>(dst), rows);
  return hipGetLastError();
}

hipError_t launch_unpad64(const void* src, void* dst, size_t rows, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const size_t blocks = (rows * 8 + 255) / 256;
  LaunchTimer timer("unpad64", st);
  unpad64_kernel<<<dim3((unsigned)(blocks < 16384 ? blocks : 16384)), 256, 0, st>>>(
      reinterpret_cast<const bf16x8*>(src), reinterpret_cast<bf16x8*>(dst), rows);
  return hipGetLastError();
}

// Writes `bytes` (a multiple of 16) of buf with plain stores: run before a timed launch, it
// replaces what the caches (L2 and the memory-side last-level cache) hold.
__global__ __launch_bounds__(256) void flush_fill_kernel(f32x4* __restrict__ buf, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) buf[i] = z;
}

hipError_t launch_flush_fill(void* buf, size_t bytes, hipStream_t st) {
  flush_fill_kernel<<<dim3(2048), 256, 0, st>>>(reinterpret_cast<f32x4*>(buf), bytes / 16);
  return hipGetLastError();
}

}  // namespace ttt

// Small bandwidth-bound helpers: operand layout transforms and the backward row dot.
#include "launch.h"

namespace ttt {

// ----------------------------------------------------------------------------------------
// [rows][128] -> [128][rows] for the operands that the matrix cores consume along the token
// axis (V^T in the forward, Q^T, dO^T and K^T in the backward).  Positions inside each group
// of 16 tokens are stored with bits 2 and 3 swapped (swap23), the order in which a 32x32
// accumulator hands its probabilities to the next product, so that every lane reads its 8
// operands with one 16-byte LDS load.
// ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_swz_kernel(const bf16* __restrict__ src,
                                                            bf16* __restrict__ dst, int rows,
                                                            size_t src_slab_stride) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][128 + 8];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * 64;
  const bf16* sp = src + (size_t)blockIdx.y * src_slab_stride + (size_t)r0 * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;
    *reinterpret_cast<bf16x8*>(&tile[row][col]) =
        *reinterpret_cast<const bf16x8*>(sp + (size_t)row * 128 + col);
  }
  __syncthreads();
  bf16* dp = dst + (size_t)blockIdx.y * 128 * rows + r0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, d = c >> 3, p0 = (c & 7) * 8;
    bf16x8 w;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) w[jj] = tile[(p0 & ~15) + swap23((p0 & 15) + jj)][d];
    *reinterpret_cast<bf16x8*>(dp + (size_t)d * rows + p0) = w;
  }
}

hipError_t launch_transpose_swz(const bf16* src, bf16* dst, int rows, size_t src_slab_stride,
                                int nslabs, hipStream_t st) {
  const dim3 grid(rows / 64, nslabs);
  LaunchTimer timer("transpose_swz", st);
  transpose_swz_kernel<<<grid, 256, 0, st>>>(src, dst, rows, src_slab_stride);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// D_i = sum_d dO_i * O_i, the row term of the softmax Jacobian (dS = P * (dP - D)).
// 16 lanes per row.
// ----------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ o,
                                                     const T* __restrict__ dout,
                                                     float* __restrict__ Dd, size_t nrows) {
  constexpr int E = D / 16;
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
  if (sub == 0) Dd[row] = acc;
}

template <typename T>
hipError_t launch_bwd_rowdot(const Shape& s, const T* o, const T* dout, float* Dd, hipStream_t st) {
  const size_t nrows = (size_t)s.B * s.Hq * s.L;
  const dim3 grid((unsigned)((nrows + 15) / 16));
  LaunchTimer timer("bwd_rowdot", st);
  if (s.D == 64)
    rowdot_kernel<T, 64><<<grid, 256, 0, st>>>(o, dout, Dd, nrows);
  else
    rowdot_kernel<T, 128><<<grid, 256, 0, st>>>(o, dout, Dd, nrows);
  return hipGetLastError();
}
template hipError_t launch_bwd_rowdot<float>(const Shape&, const float*, const float*, float*,
                                             hipStream_t);
template hipError_t launch_bwd_rowdot<bf16>(const Shape&, const bf16*, const bf16*, float*,
                                            hipStream_t);

}  // namespace ttt

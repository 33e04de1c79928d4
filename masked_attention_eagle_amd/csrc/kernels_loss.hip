// In-place masked softmax-loss gradient (bandwidth-bound).
//
// The SpecForge paper review (§3 "Memory-efficient gradient computation", §4 "Masked softmax
// loss" and "In-place backward") computes, per token row of the draft logits z [N, V] with
// target distribution p and upstream gradient g:
//   pi = softmax(z),  L = -sum_i p_i log pi_i,  s = sum_i p_i g,  z <- -(p g - pi s)
// and stores the gradient over the logits, so no second [N, V] buffer exists.  g is one
// weight per row (the loss mask and normaliser of the token), broadcast along the row.
//
// One workgroup per row.  The cached variant keeps the row's z and p in registers between
// the statistics and the write, so HBM sees one read of z and p and one write of z (the
// minimum); the streaming variant (vocabularies too long to hold) reads the row twice.  The
// cached variant is held to 128 registers (bf16 rows up to 32768 columns, fp32 up to 16384) so that
// two rows (16 waves) share a CU: one row's reductions and exponentials overlap the other's
// memory traffic; longer rows get 256 registers and one row per CU.
#include "launch.h"

namespace ttt {

constexpr int LT = 512;  // threads per row
constexpr int NW = LT / 64;  // waves per row

// 8 consecutive elements of a row, kept in their storage type (bf16: 4 registers), loaded with
// the non-temporal hint (each row is read once, or twice in a row by one workgroup).
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
  }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <> struct Vec8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* in) { store_vec<T, 8>(p, in); }

// Block-wide reductions over the LT threads (NW waves): wave shuffles, then one LDS round.
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ void block_sum3(float& a, float& b, float& c, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[w] = a;
    red[NW + w] = b;
    red[2 * NW + w] = c;
  }
  __syncthreads();
  a = b = c = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    a += red[i];
    b += red[NW + i];
    c += red[2 * NW + i];
  }
  __syncthreads();
}

// Row statistics to the gradient: lse (natural log), then the loss and s.
struct RowStats {
  float lse2;  // lse * log2(e)
  float s;     // g * sum p
  float g;
  float loss;
};

__device__ __forceinline__ RowStats finish_row(float m, float sum_e, float sum_p, float sum_pz,
                                               float g) {
  RowStats r;
  const float lse = m + __log2f(sum_e) * kLn2;  // sum_e >= 1: the max element gives exp(0)
  r.lse2 = lse * kLog2e;
  r.loss = lse * sum_p - sum_pz;                 // -sum p (z - lse)
  r.s = g * sum_p;
  r.g = g;
  return r;
}

// NV vectors of 8 elements per thread stay in registers (V <= LT * 8 * NV).
template <typename T, int NV>
__global__ __launch_bounds__(LT, NV * sizeof(T) <= 16 ? 4 : 2) void loss_grad_cached_kernel(T* __restrict__ z,
                                                              const T* __restrict__ p,
                                                              const float* __restrict__ g,
                                                              float* __restrict__ loss, int V) {
  __shared__ float red[3 * NW];
  const size_t row = blockIdx.x;
  T* zr = z + row * (size_t)V;
  const T* pr = p + row * (size_t)V;
  const int nvec = V / 8;
  Vec8<T> zv[NV], pv[NV];
  float m = kNegInf;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = j * LT + threadIdx.x;
    if (vi < nvec) {
      zv[j].load(zr + 8 * vi);
      pv[j].load(pr + 8 * vi);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, zv[j][e]);
    }
  }
  m = block_max(m, red);
  const float m2 = m * kLog2e;
  float se = 0.f, sp = 0.f, spz = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    if (j * LT + threadIdx.x < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zz = zv[j][e], pp = pv[j][e];
        se += exp2_fast(__builtin_fmaf(zz, kLog2e, -m2));
        sp += pp;
        spz += pp * zz;
      }
    }
  }
  block_sum3(se, sp, spz, red);
  const RowStats r = finish_row(m, se, sp, spz, g[row]);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = j * LT + threadIdx.x;
    if (vi < nvec) {
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pi = exp2_fast(__builtin_fmaf(zv[j][e], kLog2e, -r.lse2));
        out[e] = pi * r.s - pv[j][e] * r.g;  // -(p g - pi s)
      }
      store8<T>(zr + 8 * vi, out);
    }
  }
  if (loss && threadIdx.x == 0) loss[row] = r.loss;
}

// Any V (multiple of 8): statistics with a running max per thread, then a second read of z
// and p for the write.
template <typename T>
__global__ __launch_bounds__(LT) void loss_grad_stream_kernel(T* __restrict__ z,
                                                              const T* __restrict__ p,
                                                              const float* __restrict__ g,
                                                              float* __restrict__ loss, int V) {
  __shared__ float red[3 * NW];
  const size_t row = blockIdx.x;
  T* zr = z + row * (size_t)V;
  const T* pr = p + row * (size_t)V;
  const int nvec = V / 8;
  float m = kNegInf, se = 0.f, sp = 0.f, spz = 0.f;
  for (int vi = threadIdx.x; vi < nvec; vi += LT) {
    Vec8<T> zv, pv;
    zv.load(zr + 8 * vi);
    pv.load(pr + 8 * vi);
    float mv = zv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mv = fmaxf(mv, zv[e]);
    const float m_new = fmaxf(m, mv);
    se *= exp2_fast((m - m_new) * kLog2e);  // 0 on the first vector (m = -inf)
    m = m_new;
    const float m2 = m * kLog2e;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      se += exp2_fast(__builtin_fmaf(zv[e], kLog2e, -m2));
      sp += pv[e];
      spz += pv[e] * zv[e];
    }
  }
  const float mb = block_max(m, red);
  se = (m == kNegInf) ? 0.f : se * exp2_fast((m - mb) * kLog2e);  // threads with no vector
  block_sum3(se, sp, spz, red);
  const RowStats r = finish_row(mb, se, sp, spz, g[row]);
  for (int vi = threadIdx.x; vi < nvec; vi += LT) {
    Vec8<T> zv, pv;
    float out[8];
    zv.load(zr + 8 * vi);
    pv.load(pr + 8 * vi);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      out[e] = exp2_fast(__builtin_fmaf(zv[e], kLog2e, -r.lse2)) * r.s - pv[e] * r.g;
    store8<T>(zr + 8 * vi, out);
  }
  if (loss && threadIdx.x == 0) loss[row] = r.loss;
}

// Largest vocabulary the cached variant holds in registers (bf16: 16 vectors of z and p per
// thread, 128 registers; fp32 twice the registers per vector, so half as many).
template <typename T> constexpr int loss_cached_max_vectors() { return sizeof(T) == 2 ? 16 : 8; }

template <typename T>
hipError_t launch_loss_grad(int64_t rows, int V, T* z, const T* p, const float* g, float* loss,
                            hipStream_t st) {
  const dim3 grid((unsigned)rows);
  const int nv = (V / 8 + LT - 1) / LT;
  LaunchTimer timer("loss_grad", st);
  if (nv <= 1)
    loss_grad_cached_kernel<T, 1><<<grid, LT, 0, st>>>(z, p, g, loss, V);
  else if (nv <= 2)
    loss_grad_cached_kernel<T, 2><<<grid, LT, 0, st>>>(z, p, g, loss, V);
  else if (nv <= 4)
    loss_grad_cached_kernel<T, 4><<<grid, LT, 0, st>>>(z, p, g, loss, V);
  else if (nv <= 8)
    loss_grad_cached_kernel<T, 8><<<grid, LT, 0, st>>>(z, p, g, loss, V);
  else if (nv <= loss_cached_max_vectors<T>())
    loss_grad_cached_kernel<T, loss_cached_max_vectors<T>()><<<grid, LT, 0, st>>>(z, p, g, loss, V);
  else
    loss_grad_stream_kernel<T><<<grid, LT, 0, st>>>(z, p, g, loss, V);
  return hipGetLastError();
}
template hipError_t launch_loss_grad<float>(int64_t, int, float*, const float*, const float*,
                                            float*, hipStream_t);
template hipError_t launch_loss_grad<bf16>(int64_t, int, bf16*, const bf16*, const float*, float*,
                                           hipStream_t);

}  // namespace ttt

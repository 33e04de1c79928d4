// Peak probes: bf16 matrix-core rate and HBM stream-copy rate on the plainest workloads.
#include "common.cuh"
#include "ttt_attn.h"
#include "ttt_probe.h"

namespace ttt {

// Four independent accumulation chains per wave keep the matrix core busy without waiting on
// a result; the operands depend on the lane (and on iters, via the loop) so nothing folds.
__global__ __launch_bounds__(256, 2) void probe_mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (bf16)(0.001f * (lane + j));
    b[j] = (bf16)(0.002f * (lane - j));
  }
  f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Each workgroup copies one contiguous 16 KB chunk: every lane issues its four 16-byte loads
// (each one a coalesced 4 KB row of the chunk across the workgroup) before its four stores, so
// the grid keeps the whole buffer's worth of requests flowing with no loop.  Plain loads and
// stores: on this chip they stream faster than the non-temporal forms for a pure copy
// (5.8 against 4.4-5.3 TB/s for 16-32 KB chunks).
__global__ __launch_bounds__(256) void probe_copy_kernel(const f32x4* __restrict__ src,
                                                         f32x4* __restrict__ dst, size_t n) {
  const size_t base = (size_t)blockIdx.x * 1024 + threadIdx.x;
  f32x4 r[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (base + 256 * u < n) r[u] = src[base + 256 * u];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (base + 256 * u < n) dst[base + 256 * u] = r[u];
}

}  // namespace ttt

extern "C" {

int ttt_probe_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, void* stream) {
  if (!sink) return TTT_E_NULL;
  if (workgroups < 1 || iters < 1) return TTT_E_SHAPE;
  if ((uintptr_t)sink & 15) return TTT_E_ALIGN;
  ttt::probe_mfma_kernel<<<dim3(workgroups), 256, 0, (hipStream_t)stream>>>(sink, iters);
  return hipGetLastError() == hipSuccess ? TTT_OK : TTT_E_HIP;
}

int ttt_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return TTT_E_NULL;
  if (bytes == 0 || bytes % 16) return TTT_E_SHAPE;
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return TTT_E_ALIGN;
  const size_t n = bytes / 16, wgs = (n + 1023) / 1024;
  if (wgs >= (1ull << 31)) return TTT_E_SHAPE;
  ttt::probe_copy_kernel<<<dim3((unsigned)wgs), 256, 0, (hipStream_t)stream>>>(
      (const f32x4*)src, (f32x4*)dst, n);
  return hipGetLastError() == hipSuccess ? TTT_OK : TTT_E_HIP;
}

}  // extern "C"

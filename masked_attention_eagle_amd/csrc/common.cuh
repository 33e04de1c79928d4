// Device-side helpers shared by the TTT attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace ttt {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Problem sizes as the kernels see them.
struct Shape {
  int B, Hq, Hkv, L, D, step, G, KV;  // KV = (step + 1) * L
  float scale;                        // multiplies q.k
  float scale_log2;                   // scale * log2(e): logits in base-2 units
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clamp_T(const int32_t* seq_T, int b, int L) {
  int t = seq_T[b];
  return t < 0 ? 0 : (t > L ? L : t);
}

// One 32x32x16 bf16 matrix-core step: acc += A(32x16) * B(16x32).
// Operand layout (per lane l, h = l / 32): A row l % 32 holds k = 8h .. 8h+7,
// B column l % 32 holds k = 8h .. 8h+7.  Result: lane l owns column l % 32 and
// rows 8*(i/4) + 4*h + (i%4) for accumulator element i = 0..15.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator that element i of lane-half h holds.
__device__ __forceinline__ constexpr int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// Within each group of 16 positions along a contraction axis, the accumulator of a
// 32x32 tile hands element j of lane-half h (k-chunk c) the logical index
// 16c + 8*(j/4) + 4h + j%4.  Operands staged in memory along that axis are stored with
// bits 2 and 3 of the in-group index swapped, so that lane-half h finds its 8 values
// contiguous at 16c + 8h.  The map is its own inverse.
__device__ __forceinline__ constexpr int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes (every lane of the group receives it).
__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror: pairs quad 0 with 1, 2 with 3
  x += dpp_mov<0x140>(x);  // row_mirror: pairs the two half rows
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Element loads/stores with conversion to/from fp32.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Load N consecutive elements (N * sizeof(T) bytes, naturally aligned) as fp32.
template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* p, float* out) {
  if constexpr (sizeof(T) == 2 && N == 8) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (float)v[j];
  } else if constexpr (sizeof(T) == 2 && N == 4) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (float)v[j];
  } else if constexpr (sizeof(T) == 4 && N % 4 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      f32x4 v = *reinterpret_cast<const f32x4*>(p + j);
      out[j] = v[0]; out[j + 1] = v[1]; out[j + 2] = v[2]; out[j + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = to_f32(p[j]);
  }
}

template <typename T, int N>
__device__ __forceinline__ void store_vec(T* p, const float* in) {
  if constexpr (sizeof(T) == 2 && N == 8) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16)in[j];
    *reinterpret_cast<bf16x8*>(p) = v;
  } else if constexpr (sizeof(T) == 2 && N == 4) {
    bf16x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (bf16)in[j];
    *reinterpret_cast<bf16x4*>(p) = v;
  } else if constexpr (sizeof(T) == 4 && N % 4 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      f32x4 v = {in[j], in[j + 1], in[j + 2], in[j + 3]};
      *reinterpret_cast<f32x4*>(p + j) = v;
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) p[j] = from_f32<T>(in[j]);
  }
}

// Asynchronous global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane l of the wave writes lds_base + 16 * l; lds_base must be the same for the whole wave.
__device__ __forceinline__ void g2lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Wait until this wave's outstanding vector-memory operations (incl. global -> LDS copies)
// have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Splits a grid of units * ranks workgroups into (unit, rank).  A unit is an
// independent slice of work (a head, a KV group); rank 0 is its heaviest piece.  The
// dispatcher deals workgroups to the 8 XCDs round robin, so when units % 8 == 0 each
// XCD is given a contiguous range of units (their shared K/V stay in that XCD's L2)
// and every XCD starts on its heaviest ranks.
__device__ __forceinline__ void map_block(int bid, int units, int& unit, int& rank) {
  if (units % 8 == 0) {
    const int x = bid % 8, slot = bid / 8, ux = units / 8;
    rank = slot / ux;
    unit = x * ux + slot % ux;
  } else {
    rank = bid / units;
    unit = bid % units;
  }
}

}  // namespace ttt

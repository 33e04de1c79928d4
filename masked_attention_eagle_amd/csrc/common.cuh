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
  // TTT steps whose queries one launch covers: 1, or (whole-TTT backward: row-dot, dK/dV of
  // block 0 and its reduction) all of them, stacked step after step (B*Hq*L rows per step)
  int nst;
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

// Element j of a bf16x8 as fp32 (exact): the bf16 is the high half of the fp32 pattern, so
// each packed pair gives its two values with one shift and one mask.
__device__ __forceinline__ float bf16x8_elem_f32(const bf16x8& x, int j) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = __builtin_bit_cast(u32x4, x);
  const unsigned word = w[j >> 1];
  return __uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
}

// Elements 2j, 2j + 1 of a bf16x8 (one 32-bit register of it).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2 bf16x8_pair(const bf16x8& x, int j) {
  return bf16x2{x[2 * j], x[2 * j + 1]};
}

// Elements off .. off + 7 of an accumulator, rounded to bf16 in pairs.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& a, int off) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  const f32x8 x = {a[off], a[off + 1], a[off + 2], a[off + 3],
                   a[off + 4], a[off + 5], a[off + 6], a[off + 7]};
  return __builtin_convertvector(x, bf16x8);
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

// Reductions over the two halves of a wave (lane l with lane l ^ 32) on the vector ALU:
// v_permlane32_swap exchanges the halves, leaving {x[l], x[l ^ 32]} in the two results.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Load N consecutive elements (N * sizeof(T) bytes, naturally aligned) as fp32; NT: with the
// non-temporal hint (data read once), for the 16-byte forms.
template <typename T, int N, bool NT = false>
__device__ __forceinline__ void load_vec(const T* p, float* out) {
  if constexpr (sizeof(T) == 2 && N == 8) {
    bf16x8 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p))
                  : *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (float)v[j];
  } else if constexpr (sizeof(T) == 2 && N == 4) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (float)v[j];
  } else if constexpr (sizeof(T) == 4 && N % 4 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      f32x4 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + j))
                   : *reinterpret_cast<const f32x4*>(p + j);
      out[j] = v[0]; out[j + 1] = v[1]; out[j + 2] = v[2]; out[j + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = to_f32(p[j]);
  }
}

// Store N fp32 values as N consecutive elements; NT: with the non-temporal hint (data not read
// again soon), for the 16-byte bf16 form.
template <typename T, int N, bool NT = false>
__device__ __forceinline__ void store_vec(T* p, const float* in) {
  if constexpr (sizeof(T) == 2 && N == 8) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16)in[j];
    if (NT)
      __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
    else
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

// A pointer the whole wave agrees on, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// Buffer resource for raw loads of `bytes` bytes starting at `base` (wave-uniform); loads at
// offsets past `bytes` return zero instead of reading memory.  0x00020000 is the gfx9 third
// descriptor word for untyped 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Asynchronous global -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane l
// reads byte offset voff of the buffer and writes lds_base + 16 * l; lds_base must be the same
// for the whole wave.  The buffer form (rather than global_load_lds) lets the compiler keep
// counting LDS reads precisely while the copy is in flight: it treats the global form like a
// flat access and then waits for every outstanding LDS read.
__device__ __forceinline__ void g2lds16(__amdgpu_buffer_rsrc_t rs, unsigned voff, void* lds_base,
                                        int soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voff, soff, 0, 0);
}

// Same, 4 bytes per lane (buffer_load_dword ... lds): lane l writes lds_base + 4 * l.
__device__ __forceinline__ void g2lds4(__amdgpu_buffer_rsrc_t rs, unsigned voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 4,
                                           voff, 0, 0, 0);
}

// 16-byte load from global memory at base + off (base wave-uniform, off per lane), kept a
// global_load for the same reason as the store below.
__device__ __forceinline__ bf16x8 load16_global(const void* base, unsigned off) {
  typedef const __attribute__((address_space(1))) char gchar;
  typedef const __attribute__((address_space(1))) bf16x8 gvec;
  return *(gvec*)((gchar*)base + off);
}

// The same load with the non-temporal hint, for data read once (it then displaces less of what
// the caches hold for other reads).
__device__ __forceinline__ bf16x8 load16_global_nt(const void* base, unsigned off) {
  typedef const __attribute__((address_space(1))) char gchar;
  typedef const __attribute__((address_space(1))) bf16x8 gvec;
  return __builtin_nontemporal_load((gvec*)((gchar*)base + off));
}

// 16-byte streaming store to global memory at base + off (base wave-uniform, off per lane).
// The explicit global address space keeps it a global_store: a flat store could alias LDS,
// and the compiler would first wait for every copy into LDS still in flight.  The
// non-temporal hint keeps data that is read back only by a later kernel from displacing
// the caller's working set in the caches.
__device__ __forceinline__ void store16_global_nt(void* base, unsigned off, const bf16x8& v) {
  typedef __attribute__((address_space(1))) char gchar;
  typedef __attribute__((address_space(1))) bf16x8 gvec;
  __builtin_nontemporal_store(v, (gvec*)((gchar*)base + off));
}

// Wait until this wave's outstanding vector-memory operations (incl. global -> LDS copies)
// have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N (< 16) of this wave's vector-memory operations are outstanding
// (s_waitcnt vmcnt(N); the LDS and export counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// ---------------------------------------------------------------------------------------
// LDS tiles of 128 bf16 per row (256 bytes).  The 16-byte chunk c of row r is stored at
// chunk c ^ swz(r).  Two read patterns hit these tiles:
//   row reads   : 16 lanes take 16 consecutive rows at one chunk       -> swz bijective on
//                 any aligned block of 16 rows;
//   column reads: 16 lanes take 4 consecutive rows x 2 adjacent chunks -> the 4 rows must
//                 differ in bits 2-3 of swz.
// swz(r) = 4*(r mod 4) + (r/4 mod 4) satisfies both, so neither pattern has bank conflicts.
__device__ __forceinline__ constexpr int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ constexpr int tile_off(int r, int col) {
  return r * 128 + ((((col >> 3) ^ swz(r))) << 3) + (col & 7);
}

// Copies rows [0, NROWS) of a [rows][128] bf16 matrix (row stride `ld` elements) into a
// swizzled LDS tile, global -> LDS directly; each wave instruction moves 4 rows (1 KB).
// `g` and `wave` are wave-uniform.  Wave w copies the 4-row groups i = w, w + NWAVES, ...;
// with NWAVES a multiple of 4, row r = 4i + lane/16 has swz(r) = 4*(lane/16) + w % 4 for
// every i, so one 32-bit lane offset serves all of the wave's copies.
template <int NROWS, int NWAVES>
__device__ __forceinline__ void load_tile(const bf16* g, int ld, bf16* lds, int wave, int lane) {
  static_assert(NWAVES % 4 == 0, "swizzle term must be constant per wave");
  const int rl = lane >> 4;
  const unsigned lane_off = (unsigned)(rl * ld + (((lane & 15) ^ ((rl << 2) | (wave & 3))) << 3));
  // Scalar resource (the tile's rows) + 32-bit per-lane byte offset: the copies hold no
  // 64-bit per-lane addresses in vector registers.
  const auto rs = buffer_rsrc(uniform_ptr(g), 2u * NROWS * ld);
  static_assert((NROWS / 4) % NWAVES == 0, "whole 4-row groups per wave");
#pragma unroll
  for (int r = 0; r < NROWS / 4 / NWAVES; ++r) {  // a fixed count: no branches per copy
    const int i = wave + r * NWAVES;
    unsigned off = 2u * ((unsigned)(4 * i * ld) + lane_off);
    asm volatile("" : "+v"(off));  // keeps the 32-bit offset form (no 64-bit copies to hold)
    g2lds16(rs, off, lds + i * 512);
  }
}

// load_tile with one per-lane offset register for all of the wave's copies: the 4-row group's
// offset goes into the buffer instruction's scalar offset instead.  For kernels short of
// vector registers (in the forward the scalar form measured slower).
template <int NROWS, int NWAVES>
__device__ __forceinline__ void load_tile_soff(const bf16* g, int ld, bf16* lds, int wave, int lane) {
  static_assert(NWAVES % 4 == 0, "swizzle term must be constant per wave");
  static_assert((NROWS / 4) % NWAVES == 0, "whole 4-row groups per wave");
  const int rl = lane >> 4;
  unsigned off = 2u * (unsigned)(rl * ld + (((lane & 15) ^ ((rl << 2) | (wave & 3))) << 3));
  asm volatile("" : "+v"(off));
  const auto rs = buffer_rsrc(uniform_ptr(g), 2u * NROWS * ld);
#pragma unroll
  for (int r = 0; r < NROWS / 4 / NWAVES; ++r) {
    const int i = wave + r * NWAVES;
    g2lds16(rs, off, lds + i * 512, 8 * i * ld);
  }
}

// Index of the calling wave inside its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Per-lane byte offsets of the matrix-core operand reads from a swizzled tile.  With the
// swizzle above, the offset of chunk pair t of a row read is row0 ^ 32t and that of column
// block u of a column read is col0[k] ^ 64u (the swizzle only flips bits 5-7 of a byte
// offset that has no carries into them), so three registers describe every read; tile base,
// 32-row block and 16-row chunk add multiples of 256 bytes.
struct FragOffsets {
  int row0;     // row l32, chunk hi (t = 0)
  int col0[2];  // column block 0, rows 4h.. (k = 0) and 4h + 8.. (k = 1)
};

__device__ __forceinline__ FragOffsets make_frag_offsets(int lane) {
  FragOffsets f;
  const int l32 = lane & 31, hi = lane >> 5, sl = lane & 15;
  f.row0 = 2 * (l32 * 128 + (((hi ^ swz(l32))) << 3));
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = 4 * hi + 8 * k + (sl >> 2);
    const int col = 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
    f.col0[k] = 2 * tile_off(r, col);
  }
  return f;
}

// A copy of the offsets the compiler cannot see through: called at the top of a loop body,
// it keeps the derived per-read offsets inside the body instead of hoisting them (and the
// registers they would hold) out of the loop.
__device__ __forceinline__ FragOffsets opaque(FragOffsets f) {
  asm volatile("" : "+v"(f.row0), "+v"(f.col0[0]), "+v"(f.col0[1]));
  return f;
}

// Matrix-core operand with the contraction along the row (d) axis: rows rb + l32 (rb a
// multiple of 32), elements 16t + 8*hi .. +7.
__device__ __forceinline__ bf16x8 frag_row(const bf16* tile, int rb, int t, const FragOffsets& f) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile + rb * 128) + (f.row0 ^ (32 * t)));
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// receives element i % 4 of the 4-element pieces addressed by lanes i/4, 4 + i/4, 8 + i/4
// and 12 + i/4.  With lane s addressing row r0 + s/4, column c0 + 4*(s % 4), lane i gets
// rows r0..r0+3 of column c0 + i.
__device__ __forceinline__ bf16x4 lds_tr4(const void* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// Matrix-core operand with the contraction along the token (row) axis, taken from a
// row-major tile: the lane holds column 32u + (lane % 32) and rows 16c + 4h .. +3 then
// 16c + 8 + 4h .. +3 (h = lane / 32), the token order in which a 32x32 accumulator hands over
// its values.  Rows 16c.. share the swizzle of rows 0.., so c only moves the base.
__device__ __forceinline__ bf16x8 frag_col(const bf16* tile, int c, int u, const FragOffsets& f) {
  const char* base = reinterpret_cast<const char*>(tile + 16 * c * 128);
  const bf16x4 a = lds_tr4(base + (f.col0[0] ^ (64 * u)));
  const bf16x4 b = lds_tr4(base + (f.col0[1] ^ (64 * u)));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Splits a grid of units * ranks workgroups into (unit, rank).  A unit is an independent
// slice of work (a head, a KV group share); rank 0 is its heaviest piece.  Units come in
// groups of `per_group` that read the same K/V (the heads or head splits of one KV group).
// The dispatcher deals workgroups to the 8 XCDs round robin, so when the number of groups is
// a multiple of 8 each XCD is given every 8th group: a group's K/V stay in one XCD's L2, and
// every XCD gets groups of every sequence, so sequences of different lengths load the XCDs
// evenly.  Every XCD starts on its heaviest ranks.
__device__ __forceinline__ void map_block(int bid, int units, int per_group, int& unit, int& rank) {
  const int groups = units / per_group;
  if (groups % 8 == 0) {
    const int x = bid % 8, slot = bid / 8, ux = units / 8;
    rank = slot / ux;
    const int k = slot % ux;  // unit index within XCD x
    unit = (x + 8 * (k / per_group)) * per_group + k % per_group;
  } else if (units % 8 == 0) {
    const int x = bid % 8, slot = bid / 8, ux = units / 8;
    rank = slot / ux;
    unit = x * ux + slot % ux;
  } else {
    rank = bid / units;
    unit = bid % units;
  }
}

}  // namespace ttt

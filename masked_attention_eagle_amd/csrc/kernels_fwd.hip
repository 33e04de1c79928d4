// Forward kernels of TTT sparse tree attention.
//
// The mask is the BlockMask construction of the SpecForge paper review (§3 "Sparse Tree
// Attention", §4 "BlockMask construction"): query i of the current TTT step sees keys
// 0..min(i, T-1) of block 0 (the causal prefix) and, if i < T, key t*Q_LEN + i of each later
// block t.  The causal part is dense-tileable and runs on the matrix cores; the suffix is one
// key per query and block, so it is gathered row by row and merged into the softmax state.
#include "launch.h"

namespace ttt {

// ----------------------------------------------------------------------------------------
// Causal block-0 forward, bf16 MFMA, head_dim 128.
//
// Workgroup = 4 waves = 128 queries (32 per wave); the loop streams 64-key tiles of block 0
// through LDS.  Per wave and tile:
//   S^T[64 keys x 32 queries] = K Q^T     (A = K rows from LDS, B = Q kept in registers)
//   online softmax on S^T (each lane owns one query; its keys sit in this lane and lane^32)
//   O^T[128 x 32] += V^T P^T              (A = V columns from LDS through transposing
//                                          reads, B = P^T straight from S^T)
// Tiles past min(q0 + 128, T) are never loaded (the BlockMask "skip" class); only tiles that
// straddle the diagonal or the T edge evaluate the mask ("partial"); the rest are "full".
// On partial tiles of waves whose rows see fewer than 64 keys, P is split into bf16 hi + lo
// parts so that rows with few keys (where one rounding of P would show in O) keep fp32-level
// accuracy.  Elsewhere P is rounded to bf16 once, and O is normalised by the sum of those
// rounded values (lse by the fp32 sum of the unrounded ones), so that O stays a convex
// combination of V rows whose error is small where a few keys carry most of the weight.
// With FINAL and k > 0 the kernel also merges the suffix keys (one per block 1..k for rows
// i < T; their K and V rows pass through the same LDS stages before the causal tiles) and
// writes the final o and lse; without FINAL it writes the fp32 causal state for the
// standalone suffix kernel.
//
// K and V tiles are copied global -> LDS without passing through registers (two stages),
// which keeps the wave under 256 registers: two workgroups share a CU and the matrix cores
// of one overlap the softmax of the other.  Operand fragments are read from LDS ahead of
// their products so that no product waits for its own read: the K fragments two to three
// products ahead (scheduling groups), the V fragments four ahead in register slots, the
// first four of them while the softmax runs.
// ----------------------------------------------------------------------------------------
constexpr int FD = 128;  // head dim
constexpr int FBM = 128; // queries per workgroup
constexpr int FBN = 64;  // keys per tile
constexpr float kRescaleLog2 = 8.f;  // headroom of the unnormalised probabilities (base 2)
constexpr float kFastSumLimit = 65536.f;  // fast path: largest per-lane tile sum of P kept

// DIAG (measurement variant, with FINAL): instead of the per-lane gather, the diagonal keys
// of blocks 1..k go through the matrix cores the way a BlockMask-driven kernel handles them:
// block t's key rows [t*Q_LEN + q0, t*Q_LEN + q0 + 128) form two extra 64-key tiles after the
// causal ones, processed as partial tiles whose mask keeps key row t*Q_LEN + i for query i.
// Each such tile meets the queries of two of the four waves; the other two skip it.
template <bool FINAL, bool DIAG>
__global__ __launch_bounds__(256, 2) void fwd_causal_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ seq_T, void* __restrict__ o_out, float* __restrict__ lse_out,
    Shape s) {
  // Two stages in distinct arrays: the compiler can then tell the copy into one stage from
  // the reads of the other and does not wait for the copy before computing.  A stage holds a
  // K tile and a V tile of 64 rows, or 128 rows of one suffix block (see below).
  __shared__ __attribute__((aligned(1024))) bf16 sKV0[2 * FBN * FD];
  __shared__ __attribute__((aligned(1024))) bf16 sKV1[2 * FBN * FD];
  bf16* const sK0 = sKV0;
  bf16* const sV0 = sKV0 + FBN * FD;
  bf16* const sK1 = sKV1;
  bf16* const sV1 = sKV1 + FBN * FD;

  const int n_qt = s.L / FBM;
  int bh, rank;
  map_block(blockIdx.x, s.B * s.Hq, s.G, bh, rank);
  const int qt = n_qt - 1 - rank;  // the last query tile sees the most keys: run it first
  const int b = bh / s.Hq, h = bh % s.Hq, g = h / s.G;
  const int T = clamp_T(seq_T, b, s.L);
  const int q0 = qt * FBM;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;

  bf16x8 qf[8];
  {
    const bf16* qrow = q + ((size_t)bh * s.L + my_q) * FD + 8 * hi;
#pragma unroll
    for (int t = 0; t < 8; ++t) qf[t] = *reinterpret_cast<const bf16x8*>(qrow + 16 * t);
  }
  const bf16* kb = k + (size_t)(b * s.Hkv + g) * s.KV * FD;
  const bf16* vb = v + (size_t)(b * s.Hkv + g) * s.KV * FD;

  const int kv_end = min(q0 + FBM, T);
  const int ncausal = (kv_end + FBN - 1) / FBN;
  // DIAG: two diagonal tiles per block t = 1..k, unless no row of this workgroup is live
  const int ntiles = ncausal + ((DIAG && q0 < T) ? 2 * s.step : 0);
  // first key row of tile j in k/v, and its first key index in block-local coordinates
  auto tile_row = [&](int j) -> size_t {
    if (!DIAG || j < ncausal) return (size_t)j * FBN;
    const int d = j - ncausal;
    return (size_t)(1 + d / 2) * s.L + q0 + FBN * (d & 1);
  };

  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{};
  // running max of the raw logits q.k; the softmax sum of the unrounded P (for lse); and the
  // sum of the P that enter the P V products, bf16-rounded on the full and wide tiles, which
  // normalises o (o is then a convex combination of V rows: the rounding errors of P cancel
  // out of the rows dominated by a few keys, where they would otherwise move o by up to
  // 2^-9 |o|)
  float m = kNegInf, l = 0.f, lt = 0.f;
  const float c2 = s.scale_log2;
  const FragOffsets fo = make_frag_offsets(lane);

  auto issue = [&](int j, bf16* dK, bf16* dV) {
    load_tile<FBN, 4>(kb + tile_row(j) * FD, FD, dK, wave, lane);
    load_tile<FBN, 4>(vb + tile_row(j) * FD, FD, dV, wave, lane);
  };

  // One tile: prefetch tile j + 1 into (nK, nV) while computing tile j from (cK, cV).
  auto body = [&](int j, const bf16* cK, const bf16* cV, bf16* nK, bf16* nV) {
    const FragOffsets fl = opaque(fo);
    if (j + 1 < ntiles) issue(j + 1, nK, nV);
    const bool diag = DIAG && j >= ncausal;  // a diagonal tile of block t >= 1
    // block-local index of the tile's first key
    const int k0 = diag ? q0 + FBN * ((j - ncausal) & 1) : j * FBN;
    if (diag ? (k0 <= qw + 31 && qw <= k0 + FBN - 1) : (k0 <= qw + 31)) {  // the wave sees a key
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
          sacc[st] = mfma32(frag_row(cK, st * 32, t, fl), qf[t], sacc[st]);
      }
      // K fragment reads kept two products ahead of the products
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
      // the first four V fragments of the P V products, read while P is formed
      bf16x8 vf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) vf[c] = frag_col(cV, c, 0, fl);
      const bool full = !diag && (k0 + FBN - 1 <= qw) && (k0 + FBN <= T);
      // every row of the wave sees at least 64 keys of block 0 (rows i < T see min(i + 1, T),
      // rows i >= T see T): one bf16 rounding of P then costs O no more than on full tiles
      const bool wide = !diag && qw >= FBN - 1 && T >= FBN;
      if (diag) {  // key row t*Q_LEN + key serves query key only, and only for rows < T
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + st * 32 + acc_row(i, hi);
            if (key != my_q || my_q >= T) sacc[st][i] = kNegInf;
          }
        }
      } else if (!full) {
        // key > my_q or key >= T  <=>  key > min(my_q, T - 1); with key = k0 + 32 st +
        // acc_row(i, hi) that is a compile-time constant against one per-lane value
        const int lim = min(my_q, T - 1) - k0 - 4 * hi;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (st * 32 + acc_row(i, 0) > lim) sacc[st][i] = kNegInf;
        }
      }
      // Fast path (full tiles and tiles whose rows all see >= 64 keys, once every row of the
      // wave has a reference max): P against the current reference max, no tile max.  Each P
      // of a lane is at most the lane's sum over its 32 keys, so the sum alone shows whether
      // some probability has grown past 2^16 (or overflowed); only then is the tile redone
      // through the max-and-rescale path below.  The sum stays fp32 over the unrounded P
      // (a sum of the bf16-rounded P would move lse by up to 2^-9 on short rows).
      float lsum = 0.f;
      bf16x8 pf[4], pl[4];
      bool fast = (full || wide) && __all(m != kNegInf);
      if (fast) {
        const float mc = m * c2;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float pv = exp2_fast(__builtin_fmaf(sacc[c >> 1][8 * (c & 1) + jj], c2, -mc));
            if (jj & 1) s1 += pv; else s0 += pv;
            pf[c][jj] = (bf16)pv;
          }
        }
        lsum = s0 + s1;
        fast = !__any(!(lsum <= kFastSumLimit));
      }
      if (!fast) {
        float rmax = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int i = 1; i < 15; i += 2) rmax = fmaxf(fmaxf(rmax, sacc[st][i]), sacc[st][i + 1]);
          rmax = fmaxf(rmax, sacc[st][15]);
        }
        rmax = half_max(rmax);
        // The reference max m of a row moves only when the tile's max exceeds it by more than
        // kRescaleLog2 in base-2 units.  Until then the tile's probabilities exp2((s - m) c2)
        // stay below 2^kRescaleLog2, which fp32 sums and bf16 P carry with the same relative
        // precision as values below 1, so the accumulator is rescaled only on the rare tiles
        // where some row's logits jump that far (always on a row's first visible key).
        const bool grow = rmax * c2 > m * c2 + kRescaleLog2;
        if (__any(grow)) {
          const float m_new = grow ? rmax : m;
          const float alpha = grow ? exp2_fast((m - m_new) * c2) : 1.f;
          l *= alpha;
          lt *= alpha;
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] *= alpha;
          m = m_new;
        }
        const float mc = (m == kNegInf) ? 0.f : m * c2;
        lsum = 0.f;
        if (full || wide) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const float pv = exp2_fast(__builtin_fmaf(sacc[c >> 1][8 * (c & 1) + jj], c2, -mc));
              lsum += pv;
              pf[c][jj] = (bf16)pv;
            }
          }
        } else {  // P = hi + lo in bf16, the sum in fp32
#pragma unroll
          for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const float pv = exp2_fast(__builtin_fmaf(sacc[c >> 1][8 * (c & 1) + jj], c2, -mc));
              lsum += pv;
              const bf16 ph = (bf16)pv;
              pf[c][jj] = ph;
              pl[c][jj] = (bf16)(pv - (float)ph);
            }
          }
        }
      }
      // the sum of the P the products take: bf16 pairs through packed dot products with 1
      // (exact products, fp32 sums); hi + lo (the partial tiles) carries P to 2^-17
      float rsum = lsum;
      if (full || wide) {
        const bf16x2 one2 = {(bf16)1.f, (bf16)1.f};
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int e2 = 0; e2 < 4; e2 += 2) {
            r0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x8_pair(pf[c], e2), one2, r0, false);
            r1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x8_pair(pf[c], e2 + 1), one2, r1, false);
          }
        }
        rsum = r0 + r1;
      }
      if (full || wide) {
        // four V fragments in flight: slot c is refilled with column block u + 1 right
        // after product (u, c) is issued, four products before it is needed
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[u] = mfma32(vf[c], pf[c], acc[u]);
            if (u < 3) vf[c] = frag_col(cV, c, u + 1, fl);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {  // both parts of P go through the same V operands (same four slots)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[u] = mfma32(vf[c], pf[c], acc[u]);
            acc[u] = mfma32(vf[c], pl[c], acc[u]);
            if (u < 3) vf[c] = frag_col(cV, c, u + 1, fl);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      l += half_sum(lsum);
      lt += half_sum(rsum);
    }
    wait_vmem();
    __syncthreads();
  };

  // Suffix keys t*Q_LEN + i (t = 1..k) of the workgroup's rows i in [q0, q0 + 128), merged
  // before the causal tiles (the softmax state is order-independent).  They are the rows
  // [t*Q_LEN + q0, t*Q_LEN + q0 + 128) of k and v: per block t, one pipeline slot copies the
  // 128 K rows into a stage while the lanes take their logits from the other, and one slot
  // does the same for the V rows.  A lane reads its own row i: the same half of the K row as
  // of q (d = 16c + 8*hi ..) and the same half of the V row as of O (d = 32u + 8*b4 + 4*hi ..);
  // the logit is the sum over the lane pair.  P stays fp32.  Rows i >= T see no suffix key.
  const int nsuf = (FINAL && !DIAG && q0 < T) ? s.step : 0;
  auto issue_rows = [&](const bf16* base, int t, bf16* dst) {  // rows t*Q_LEN + q0 .. + 127
    load_tile<2 * FBN, 4>(base + ((size_t)t * s.L + q0) * FD, FD, dst, wave, lane);
  };
  if (nsuf > 0)
    issue_rows(kb, 1, sKV0);
  else if (ntiles > 0)
    issue(0, sK0, sV0);
  wait_vmem();
  __syncthreads();
  if (nsuf > 0) {
    const int row = wave * 32 + l32;                      // this lane's row in the slot
    const int swz = 4 * (row & 3) + ((row >> 2) & 3);     // chunk swizzle of that row
    const bool live = my_q < T;
    float p = 0.f;
    for (int t = 1; t <= nsuf; ++t) {
      issue_rows(vb, t, sKV1);
      if (live) {
        bf16x8 kk[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          kk[c] = *reinterpret_cast<const bf16x8*>(sKV0 + row * FD + 8 * ((2 * c + hi) ^ swz));
        // q.k over the lane's 64 elements: packed bf16 pairs, products exact, fp32 sums
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            dot = __builtin_amdgcn_fdot2_f32_bf16(bf16x8_pair(qf[c], e2), bf16x8_pair(kk[c], e2),
                                                  dot, false);
        dot = half_sum(dot);
        // the same lazy rescaling as the tiles below: m moves only when the logit exceeds it
        // by more than kRescaleLog2 (base 2), always on the first key (m = -inf)
        const bool grow = dot * c2 > m * c2 + kRescaleLog2;
        if (__any(grow)) {
          const float m_new = grow ? dot : m;
          const float alpha = grow ? exp2_fast((m - m_new) * c2) : 1.f;  // 0 while m = -inf
          l *= alpha;
          lt *= alpha;
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] *= alpha;
          m = m_new;
        }
        p = exp2_fast((dot - m) * c2);
        l += p;
        lt += p;
      }
      wait_vmem();
      __syncthreads();
      if (t < nsuf)
        issue_rows(kb, t + 1, sKV0);
      else if (ntiles > 0)
        issue(0, sK0, sV0);
      if (live) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const bf16x4 vv = *reinterpret_cast<const bf16x4*>(
                sKV1 + row * FD + 8 * ((4 * u + b4) ^ swz) + 4 * hi);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[u][4 * b4 + e] = __builtin_fmaf(p, (float)vv[e], acc[u][4 * b4 + e]);
          }
        }
      }
      wait_vmem();
      __syncthreads();
    }
  }
  for (int j = 0; j < ntiles; j += 2) {
    body(j, sK0, sV0, sK1, sV1);
    if (j + 1 < ntiles) body(j + 1, sK1, sV1, sK0, sV0);
  }

  const float inv_l = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = l > 0.f ? (m * c2 + __log2f(l)) * kLn2 : kNegInf;
  const size_t row = (size_t)bh * s.L + my_q;
  if (hi == 0) lse_out[row] = lse;
  // lane owns O[my_q][32u + 8*b4 + 4*hi + e] in acc[u][4*b4 + e]
  if constexpr (FINAL) {
    bf16* orow = reinterpret_cast<bf16*>(o_out) + row * FD + 4 * hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[u][4 * b4 + e] * inv_l);
        *reinterpret_cast<bf16x4*>(orow + 32 * u + 8 * b4) = w;
      }
    }
  } else {
    float* orow = reinterpret_cast<float*>(o_out) + row * FD + 4 * hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[u][4 * b4 + e] * inv_l;
        *reinterpret_cast<f32x4*>(orow + 32 * u + 8 * b4) = w;
      }
    }
  }
}

hipError_t launch_fwd_causal_mfma(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                                  const int32_t* seq_T, void* o, float* lse, bool final_out,
                                  bool dense_diagonal, hipStream_t st) {
  const dim3 grid(s.B * s.Hq * (s.L / FBM));
  if (dense_diagonal && final_out && s.step > 0) {
    LaunchTimer timer("fwd_dense_diag_mfma", st);
    fwd_causal_mfma_kernel<true, true><<<grid, 256, 0, st>>>(q, k, v, seq_T, o, lse, s);
    return hipGetLastError();
  }
  LaunchTimer timer("fwd_causal_mfma", st);
  if (final_out)
    fwd_causal_mfma_kernel<true, false><<<grid, 256, 0, st>>>(q, k, v, seq_T, o, lse, s);
  else
    fwd_causal_mfma_kernel<false, false><<<grid, 256, 0, st>>>(q, k, v, seq_T, o, lse, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Causal block-0 forward on the vector ALUs (fp32, and bf16 shapes outside the matrix-core
// tiling; arithmetic in fp32).  One wave per query row: lanes take
// 64 keys at a time for the logits, then split the head dimension for P V.
// ----------------------------------------------------------------------------------------
template <typename T, int D, bool FINAL>
__global__ __launch_bounds__(64) void fwd_causal_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ seq_T, void* __restrict__ o_out, float* __restrict__ lse_out,
    Shape s) {
  __shared__ float sq[D];
  __shared__ float sp[64];
  constexpr int E = D / 64;
  const int bh = blockIdx.x / s.L, i = blockIdx.x % s.L;
  const int b = bh / s.Hq, h = bh % s.Hq, g = h / s.G;
  const int Tlen = clamp_T(seq_T, b, s.L);
  const int lane = threadIdx.x;
  const size_t row = (size_t)bh * s.L + i;
  for (int e = lane; e < D; e += 64) sq[e] = to_f32(q[row * D + e]);
  __syncthreads();
  const int n = (i < Tlen) ? i + 1 : Tlen;  // keys 0..n-1 of block 0
  const T* kb = k + (size_t)(b * s.Hkv + g) * s.KV * D;
  const T* vb = v + (size_t)(b * s.Hkv + g) * s.KV * D;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float m = kNegInf, l = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int j = c0 + lane;
    float x = kNegInf;
    if (j < n) {
      float dot = 0.f;
      for (int e = 0; e < D; ++e) dot += sq[e] * to_f32(kb[(size_t)j * D + e]);
      x = dot * s.scale_log2;
    }
    const float m_new = fmaxf(m, wave_max(x));  // finite: key c0 is visible
    const float alpha = exp2_fast(m - m_new);
    const float p = exp2_fast(x - m_new);
    l = l * alpha + wave_sum(p);
    m = m_new;
    sp[lane] = p;
    __syncthreads();
    const int cnt = min(64, n - c0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = acc[e] * alpha;
      const int dd = lane + 64 * e;
      for (int jj = 0; jj < cnt; ++jj) a += sp[jj] * to_f32(vb[(size_t)(c0 + jj) * D + dd]);
      acc[e] = a;
    }
    __syncthreads();
  }
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  if (lane == 0) lse_out[row] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int dd = lane + 64 * e;
    if constexpr (FINAL)
      reinterpret_cast<T*>(o_out)[row * D + dd] = from_f32<T>(acc[e] * inv_l);
    else
      reinterpret_cast<float*>(o_out)[row * D + dd] = acc[e] * inv_l;
  }
}

template <typename T>
hipError_t launch_fwd_causal_valu(const Shape& s, const T* q, const T* k, const T* v,
                                  const int32_t* seq_T, void* o, float* lse, bool final_out,
                                  hipStream_t st) {
  const dim3 grid(s.B * s.Hq * s.L);
  LaunchTimer timer("fwd_causal_valu", st);
  if (s.D == 64) {
    if (final_out) fwd_causal_valu_kernel<T, 64, true><<<grid, 64, 0, st>>>(q, k, v, seq_T, o, lse, s);
    else fwd_causal_valu_kernel<T, 64, false><<<grid, 64, 0, st>>>(q, k, v, seq_T, o, lse, s);
  } else {
    if (final_out) fwd_causal_valu_kernel<T, 128, true><<<grid, 64, 0, st>>>(q, k, v, seq_T, o, lse, s);
    else fwd_causal_valu_kernel<T, 128, false><<<grid, 64, 0, st>>>(q, k, v, seq_T, o, lse, s);
  }
  return hipGetLastError();
}
template hipError_t launch_fwd_causal_valu<float>(const Shape&, const float*, const float*,
                                                  const float*, const int32_t*, void*, float*,
                                                  bool, hipStream_t);
template hipError_t launch_fwd_causal_valu<bf16>(const Shape&, const bf16*, const bf16*,
                                                 const bf16*, const int32_t*, void*, float*, bool,
                                                 hipStream_t);

// ----------------------------------------------------------------------------------------
// Suffix forward: the diagonal keys t*Q_LEN + i (t = 1..k) of query row i < T.
//
// One aligned group of 16 lanes per (b, KV group, row i); each lane holds D/16 contiguous
// elements of a row, so one K or V row is a single 256-byte coalesced read that serves every
// query head of the group.  The causal result arrives normalised (o_c, lse_c), which is the
// same softmax state as (m = lse_c, l = 1, acc = o_c); each diagonal logit is merged in with
// the usual rescaling, then o = acc / l and lse = m + log l.  Rows i >= T only convert o_c.
// ----------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_suffix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ seq_T, const float* __restrict__ oc,
    const float* __restrict__ lsec, T* __restrict__ o, float* __restrict__ lse, Shape s) {
  constexpr int E = D / 16;
  const int sub = threadIdx.x & 15;
  const int blocks_per_bg = (s.L + 15) / 16;
  const int bg = blockIdx.x / blocks_per_bg;
  const int i = (blockIdx.x % blocks_per_bg) * 16 + (threadIdx.x >> 4);
  if (i >= s.L) return;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int Tlen = clamp_T(seq_T, b, s.L);
  const size_t kv_base = (size_t)bg * s.KV * D + (size_t)i * D + sub * E;
  for (int h = g * s.G; h < (g + 1) * s.G; ++h) {
    const size_t row = (size_t)(b * s.Hq + h) * s.L + i;
    float acc[E];
    load_vec<float, E>(oc + row * D + sub * E, acc);
    const float lc = lsec[row];
    float m = lc * kLog2e;
    float l = (lc == kNegInf) ? 0.f : 1.f;
    if (i < Tlen) {
      float qv[E];
      load_vec<T, E>(q + row * D + sub * E, qv);
      for (int t = 1; t <= s.step; ++t) {
        float kv[E], vv[E];
        load_vec<T, E>(k + kv_base + (size_t)t * s.L * D, kv);
        load_vec<T, E>(v + kv_base + (size_t)t * s.L * D, vv);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot += qv[e] * kv[e];
        const float x = sum16(dot) * s.scale_log2;
        const float m_new = fmaxf(m, x);
        const float alpha = exp2_fast(m - m_new), beta = exp2_fast(x - m_new);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + beta * vv[e];
        l = l * alpha + beta;
        m = m_new;
      }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float ov[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ov[e] = acc[e] * inv;
    store_vec<T, E>(o + row * D + sub * E, ov);
    if (sub == 0) lse[row] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
  }
}

// Same computation with the step loop outside and every head of the group in registers: each
// diagonal K/V row is read once per (row, group), and step t + 1's rows are in flight while
// step t is merged.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void fwd_suffix_g_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ seq_T, const float* __restrict__ oc,
    const float* __restrict__ lsec, T* __restrict__ o, float* __restrict__ lse, Shape s) {
  constexpr int E = D / 16;
  const int sub = threadIdx.x & 15;
  const int blocks_per_bg = (s.L + 15) / 16;
  const int bg = blockIdx.x / blocks_per_bg;
  const int i = (blockIdx.x % blocks_per_bg) * 16 + (threadIdx.x >> 4);
  if (i >= s.L) return;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int Tlen = clamp_T(seq_T, b, s.L);
  const size_t kv_base = (size_t)bg * s.KV * D + (size_t)i * D + sub * E;
  const size_t row0 = (size_t)(b * s.Hq + g * G) * s.L + i;  // row of head g*G; heads are L rows apart

  float acc[G][E], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t row = row0 + (size_t)h * s.L;
    load_vec<float, E>(oc + row * D + sub * E, acc[h]);
    const float lc = lsec[row];
    m[h] = lc * kLog2e;
    l[h] = (lc == kNegInf) ? 0.f : 1.f;
  }
  if (i < Tlen && s.step > 0) {
    float qv[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) load_vec<T, E>(q + (row0 + (size_t)h * s.L) * D + sub * E, qv[h]);
    float kc[E], vc[E];
    load_vec<T, E>(k + kv_base + (size_t)s.L * D, kc);
    load_vec<T, E>(v + kv_base + (size_t)s.L * D, vc);
    for (int t = 1; t <= s.step; ++t) {
      float kn[E], vn[E];
      if (t < s.step) {
        load_vec<T, E>(k + kv_base + (size_t)(t + 1) * s.L * D, kn);
        load_vec<T, E>(v + kv_base + (size_t)(t + 1) * s.L * D, vn);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot += qv[h][e] * kc[e];
        const float x = sum16(dot) * s.scale_log2;
        const float m_new = fmaxf(m[h], x);
        const float alpha = exp2_fast(m[h] - m_new), beta = exp2_fast(x - m_new);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = acc[h][e] * alpha + beta * vc[e];
        l[h] = l[h] * alpha + beta;
        m[h] = m_new;
      }
      if (t < s.step) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kc[e] = kn[e];
          vc[e] = vn[e];
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t row = row0 + (size_t)h * s.L;
    const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
    float ov[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ov[e] = acc[h][e] * inv;
    store_vec<T, E>(o + row * D + sub * E, ov);
    if (sub == 0) lse[row] = l[h] > 0.f ? (m[h] + __log2f(l[h])) * kLn2 : kNegInf;
  }
}

template <typename T, int D>
static hipError_t fwd_suffix_dispatch(const Shape& s, dim3 grid, hipStream_t st, const T* q,
                                      const T* k, const T* v, const int32_t* seq_T,
                                      const float* oc, const float* lsec, T* o, float* lse) {
  switch (s.G) {
    case 1: fwd_suffix_g_kernel<T, D, 1><<<grid, 256, 0, st>>>(q, k, v, seq_T, oc, lsec, o, lse, s); break;
    case 2: fwd_suffix_g_kernel<T, D, 2><<<grid, 256, 0, st>>>(q, k, v, seq_T, oc, lsec, o, lse, s); break;
    case 4: fwd_suffix_g_kernel<T, D, 4><<<grid, 256, 0, st>>>(q, k, v, seq_T, oc, lsec, o, lse, s); break;
    case 8: fwd_suffix_g_kernel<T, D, 8><<<grid, 256, 0, st>>>(q, k, v, seq_T, oc, lsec, o, lse, s); break;
    default: fwd_suffix_kernel<T, D><<<grid, 256, 0, st>>>(q, k, v, seq_T, oc, lsec, o, lse, s); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd_suffix(const Shape& s, const T* q, const T* k, const T* v,
                             const int32_t* seq_T, const float* oc, const float* lsec, T* o,
                             float* lse, hipStream_t st) {
  const dim3 grid(s.B * s.Hkv * ((s.L + 15) / 16));
  LaunchTimer timer("fwd_suffix", st);
  if (s.D == 64) return fwd_suffix_dispatch<T, 64>(s, grid, st, q, k, v, seq_T, oc, lsec, o, lse);
  return fwd_suffix_dispatch<T, 128>(s, grid, st, q, k, v, seq_T, oc, lsec, o, lse);
}
template hipError_t launch_fwd_suffix<float>(const Shape&, const float*, const float*,
                                             const float*, const int32_t*, const float*,
                                             const float*, float*, float*, hipStream_t);
template hipError_t launch_fwd_suffix<bf16>(const Shape&, const bf16*, const bf16*, const bf16*,
                                            const int32_t*, const float*, const float*, bf16*,
                                            float*, hipStream_t);

}  // namespace ttt

// Backward kernels of TTT sparse tree attention.
//
// Nothing but lse is saved by the forward (the review's §3 "Sparse Tree Attention": streamed
// FlashAttention-style, no logits kept), so every kernel recomputes P = exp(scale q.k - lse)
// and applies the softmax Jacobian dS = P * (dP - D), D = rowsum(dO * O), dP = dO V^T.
// Block-0 (causal) keys are handled by two matrix-core kernels:
//   dkdv: one workgroup owns 128 keys of one KV group and walks every query tile and every
//         query head of the group that can see them, so dK/dV need no atomics and sum the
//         heads in a fixed order (bitwise reproducible);
//   dq:   one workgroup owns 128 query rows of one head and walks the key tiles they see.
// The diagonal suffix keys of blocks 1..k are gathered by a bandwidth-bound kernel that also
// finalises dQ.
#include "launch.h"

namespace ttt {

constexpr int BD = 128;  // head dim of the matrix-core path

// ----------------------------------------------------------------------------------------
// dK, dV of block 0, bf16 MFMA.  Workgroup = 4 waves x 32 keys = 128 keys; K and V of each
// wave's keys are held in registers; query tiles of 32 rows (of every query head of the group
// that sees the keys) stream through LDS.  Per wave and tile:
//   S  = Q K^T,  dP = dO V^T          (M = queries, N = the wave's 32 keys; A = Q / dO rows)
//   P  = exp2(S * scale*log2e - lse*log2e), dS = P * (dP - D)   (lse*log2e precomputed)
//   dV += P^T dO,  dK += dS^T Q       (A operands straight from the S/dP accumulators,
//                                      B = dO / Q columns through transposing LDS reads)
// With s.nst > 1 (whole TTT) the query tiles of every step pass through the same workgroup,
// step after step.  With nsplit > 1 the query heads of the group are split over nsplit
// workgroups (each takes its heads at every step, so all workgroups work on the same step at
// about the same time) that write fp32 partial sums, reduced afterwards in split order.
// ----------------------------------------------------------------------------------------
constexpr int KBN = 128;  // keys per tile
constexpr int KBM = 32;   // queries per tile

// dS hand-over between the dK/dV kernel and the dQ kernel.  dS of one head is kept in
// 32 x 32 blocks (32 query rows x 32 keys of block 0); only blocks on or below the diagonal
// exist, packed row after row (query block r holds key blocks 0..r).
__device__ __forceinline__ size_t ds_block_index(const Shape& s, int bh, int qb, int kb) {
  const int n = s.L / 32;
  return (size_t)bh * ((size_t)n * (n + 1) / 2) + (size_t)qb * (qb + 1) / 2 + kb;
}
// Inside a 2 KB block, the dK/dV lane holding key l32 and query rows acc_row(0..15, hi) has
// its 16 values as 4-row pieces (8 bytes) in accumulator order; pieces 0-1 go to the first
// KB and pieces 2-3 to the second, each as a 16-byte chunk at slot 2*l32 + hi (slot bit 3
// flipped in the second KB).  Each of the two stores then fills one KB contiguously, and
// the transposing reads below touch every LDS bank once per half wave.
__device__ __forceinline__ unsigned ds_store_offset(int lane, int half) {
  const int slot = 2 * (lane & 31) + (lane >> 5);
  return (unsigned)(1024 * half + 16 * (slot ^ (8 * half)));
}
// Byte offset for lds_tr4 that gives lane (query n = lane % 32, half h) keys
// 16c + 8r + 4h .. +3 of its row: in each 16-lane group, lane s addresses the piece of key
// 16c + 8r + 4h + s/4 that holds queries 16(group % 2) + 4(s % 4) .. +3, i.e. piece
// 2(group % 2) + (s % 4)/2 of the writer lane of that key in half (s % 4) % 2.
__device__ __forceinline__ unsigned ds_read_offset(int lane, int c, int r) {
  const int s16 = lane & 15, a = s16 & 3, j = s16 >> 2;
  const int h = lane >> 5, qh = (lane >> 4) & 1;
  const int key = 16 * c + 8 * r + 4 * h + j;
  const int slot = 2 * key + (a & 1);
  return (unsigned)(1024 * qh + 16 * (slot ^ (8 * qh)) + 8 * (a >> 1));
}

// Diagonal keys of the suffix blocks for the query rows [r0, r0 + nrows) (NEXT-1 in the
// backward: the dK/dV workgroup of a block-0 key tile also owns the key rows t*Q_LEN + i of
// blocks t = 1..k for the same i).  16 lanes per row, 16 rows per round; each lane holds 8 of
// the 128 elements.  Two passes, so that neither the step count nor the group size sets the
// register footprint:
//   dQ:    per head, dq_suf[h, i] = scale * sum_t ds_t k_t (fp32, for the dQ kernel to add);
//   dK/dV: per block t, dK_t = scale * sum_h ds_h q_h and dV_t = sum_h p_h dO_h, written once
//          (this workgroup is the only writer of these rows).
// with p = exp2(scale*log2(e) q.k_t - lse*log2(e)), ds = p (dO.v_t - D).  Rows i >= T get no
// suffix key: zero dK/dV rows and a zero dQ term.  q and dO rows are read twice (the second
// time mostly from L2).
__device__ __forceinline__ void dkdv_suffix_rows(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ Dd,
    float* __restrict__ dq_suf, bf16* __restrict__ dk, bf16* __restrict__ dv, const Shape& s,
    int b, int bg, int hg0, int T, int r0, int nrows) {
  constexpr int E = BD / 16;
  const int sub = threadIdx.x & 15;
  for (int rr = threadIdx.x >> 4; rr < nrows; rr += 16) {
    const int i = r0 + rr;
    const bool live = i < T;
    const size_t kv_base = ((size_t)bg * s.KV + i) * BD + sub * E;
    // dQ term, head by head
    for (int h = 0; h < s.G; ++h) {
      const size_t row = (size_t)(b * s.Hq + hg0 + h) * s.L + i;
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = 0.f;
      if (live) {
        float qv[E], ov[E];
        load_vec<bf16, E>(q + row * BD + sub * E, qv);
        load_vec<bf16, E>(dO + row * BD + sub * E, ov);
        const float l2 = lse2[row], Di = Dd[row];
        for (int t = 1; t <= s.step; ++t) {
          float kc[E], vc[E];
          load_vec<bf16, E>(k + kv_base + (size_t)t * s.L * BD, kc);
          load_vec<bf16, E>(v + kv_base + (size_t)t * s.L * BD, vc);
          float sd = 0.f, pd = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            sd += qv[e] * kc[e];
            pd += ov[e] * vc[e];
          }
          const float p = exp2_fast(sum16(sd) * s.scale_log2 - l2);
          const float ds = p * (sum16(pd) - Di);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] += ds * kc[e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= s.scale;
      }
      store_vec<float, E>(dq_suf + row * BD + sub * E, acc);
    }
    // dK, dV of the key rows t*Q_LEN + i, block by block
    for (int t = 1; t <= s.step; ++t) {
      float aK[E], aV[E];
#pragma unroll
      for (int e = 0; e < E; ++e) aK[e] = aV[e] = 0.f;
      if (live) {
        float kc[E], vc[E];
        load_vec<bf16, E>(k + kv_base + (size_t)t * s.L * BD, kc);
        load_vec<bf16, E>(v + kv_base + (size_t)t * s.L * BD, vc);
        for (int h = 0; h < s.G; ++h) {
          const size_t row = (size_t)(b * s.Hq + hg0 + h) * s.L + i;
          float qv[E], ov[E];
          load_vec<bf16, E>(q + row * BD + sub * E, qv);
          load_vec<bf16, E>(dO + row * BD + sub * E, ov);
          float sd = 0.f, pd = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            sd += qv[e] * kc[e];
            pd += ov[e] * vc[e];
          }
          const float p = exp2_fast(sum16(sd) * s.scale_log2 - lse2[row]);
          const float ds = p * (sum16(pd) - Dd[row]);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            aV[e] += p * ov[e];
            aK[e] += ds * qv[e];
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) aK[e] *= s.scale;
      }
      store_vec<bf16, E, true>(dk + kv_base + (size_t)t * s.L * BD, aK);
      store_vec<bf16, E, true>(dv + kv_base + (size_t)t * s.L * BD, aV);
    }
  }
}

// Key tile kt is seen by every query row >= 128 * kt (padded rows see every key < T), so the
// work of tile kt falls linearly with kt and is zero from T on.  Workgroups take (key tile,
// head share) units from a queue in that order, heaviest first, until it is empty, so that
// one that finishes early takes the next unit (with sequences of different lengths, fixed
// pairs of tiles would leave some workgroups little or no work).  The queue is a counter in
// the workspace per XCD (when the KV groups or units spread evenly over the 8 XCDs, so that a
// group's Q/dO stay in one L2) or one for all; the row-dot kernel, launched just before on
// the same stream, sets it to zero.  Each unit's dK/dV (or split partial) is summed in the
// same order whichever workgroup takes it, so the results do not depend on the schedule.
// The kernel sits at the scalar-register limit, and scalars spilled into vector registers
// would cost the tile loop its operand read-ahead: the queue's address is kept in an LDS
// word and the tile position in 32-bit indices.
// The register file is full (dK/dV accumulators 128, K/V fragments 64 of 256), so operand
// reads run only as far ahead as the spare registers allow: the dO fragments of the dP
// products two ahead, the dO and Q fragments of the dV and dK products four ahead.
// DIAG (measurement variant of the backward, the way a BlockMask-driven kernel handles the
// suffix): after the workgroups of block 0, one workgroup per (b, KV group, block t = 1..k,
// 128-key tile) takes the key rows [t*Q_LEN + k0, t*Q_LEN + k0 + 128) and the query rows
// [k0, k0 + 128) of every head of the group as masked tiles whose mask keeps key row
// t*Q_LEN + i for query i < T; each 32-query tile meets the keys of one wave, the other three
// skip it.  These workgroups write their dK/dV rows directly (no split, no dS hand-over).
// SUF: the workgroup also takes the suffix key rows of its key tiles (dkdv_suffix_rows), with
// the dQ term written to dq_suf.
template <bool DIAG, bool SUF>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ Dd,
    const int32_t* __restrict__ seq_T, bf16* __restrict__ dk, bf16* __restrict__ dv,
    float* __restrict__ part, int nsplit, bf16* __restrict__ ds_out, float* __restrict__ dq_suf,
    unsigned* __restrict__ sched, Shape s) {
  // Two stages in distinct arrays (the copy into one never stalls reads of the other).
  __shared__ __attribute__((aligned(1024))) bf16 sQ0[KBM * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sO0[KBM * BD];
  __shared__ __attribute__((aligned(256))) float sLD0[2 * KBM];  // lse * log2(e), then D
  __shared__ __attribute__((aligned(1024))) bf16 sQ1[KBM * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sO1[KBM * BD];
  __shared__ __attribute__((aligned(256))) float sLD1[2 * KBM];

  __shared__ int sUnit;
  __shared__ unsigned* sQueue;  // this workgroup's queue counter (kept out of the registers)
  const int nkt = s.L / KBN;
  const int groups = s.B * s.Hkv, n_units = groups * nsplit;
  // the queue's workgroups: one per pair of key tiles of a unit (two units each on average)
  const int n_pair_wgs = n_units * ((nkt + 1) / 2);
  const bool dwg = DIAG && (int)blockIdx.x >= n_pair_wgs;  // a diagonal tile of a block t >= 1
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const float c2 = s.scale_log2;
  const FragOffsets fo = make_frag_offsets(lane);
  const int kd0 = wave * 32 + l32 - 4 * hi;  // my_key - k0 - 4 hi: the mask's per-lane term
  // this workgroup's queue (the dispatcher deals workgroups to the XCDs round robin)
  const bool per_xcd = groups % 8 == 0 || n_units % 8 == 0;
  const int queue = per_xcd ? (int)blockIdx.x % 8 : 0;
  const int qunits = per_xcd ? n_units / 8 : n_units;  // (KV group, split) units per queue
  if (tid == 0) sQueue = sched + 32 * queue;

#pragma nounroll
  for (int round = 0;; ++round) {
    int unit, kt, tblk = 0, nsp = nsplit;
    if (dwg) {
      if (round > 0) break;
      const int d = (int)blockIdx.x - n_pair_wgs;
      unit = d % groups;
      kt = (d / groups) % nkt;
      tblk = 1 + d / (groups * nkt);
      nsp = 1;
    } else {
      if (tid == 0) sUnit = (int)atomicAdd(sQueue, 1u);
      __syncthreads();
      const int uq = sUnit;
      __syncthreads();  // read by all before the next round overwrites it
      if (uq >= qunits * nkt) break;
      kt = uq / qunits;  // key tiles in order: the heaviest first
      const int x = uq % qunits;
      if (groups % 8 == 0)  // KV groups queue, queue + 8, ... with all their splits
        unit = (queue + 8 * (x / nsplit)) * nsplit + x % nsplit;
      else
        unit = queue * qunits + x;
    }
    const int split = unit % nsp, bg = unit / nsp;
    const int b = bg / s.Hkv;
    const int T = clamp_T(seq_T, b, s.L);
    const int hps = s.G / nsp;              // query heads of this unit, at every step
    const int hg0 = (bg % s.Hkv) * s.G;     // the group's first query head
    const int hh_begin = split * hps;
    const size_t krow0 = (size_t)tblk * s.L;  // first K/V row of the block
    const int k0 = kt * KBN;
    const int kw = k0 + wave * 32;
    const int my_key = kw + l32;

    bf16x8 kf[8], vf[8];
    {
      const bf16* kr = k + ((size_t)bg * s.KV + krow0 + my_key) * BD + 8 * hi;
      const bf16* vr = v + ((size_t)bg * s.KV + krow0 + my_key) * BD + 8 * hi;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        kf[t] = *reinterpret_cast<const bf16x8*>(kr + 16 * t);
        vf[t] = *reinterpret_cast<const bf16x8*>(vr + 16 * t);
      }
    }
    f32x16 dKacc[4], dVacc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) dKacc[u] = dVacc[u] = f32x16{};

    // Queries that see keys [k0, k0 + 128): rows >= k0 (rows >= T see every key < T); for a
    // diagonal tile, rows [k0, k0 + 128) only.
    const int q_first = (k0 < T) ? k0 : s.L;
    const int q_end = dwg ? k0 + KBN : s.L;
    const int nq = max(q_end - q_first, 0) / KBM;
    const int total = nq * hps * s.nst;

    // Tile `it` is (pair p = it / nq, query rows q_first + (it % nq) * KBM ..), where pair p is
    // step j = p / hps and head hg0 + hh_begin + p % hps; the loop carries that position and
    // steps it without dividing.
    struct Pos {
      int j, hh, q0;
      unsigned row0;   // ((j * B + b) * Hq + hg0 + hh) * L + q0
      unsigned dsrow;  // dS block index of (step j, that head, query block q0 / 32, key block 0)
    };
    auto make_pos = [&](int j, int hh, int q0) -> Pos {
      const int sbh = (j * s.B + b) * s.Hq + hg0 + hh;
      return Pos{j, hh, q0, (unsigned)((size_t)sbh * s.L + q0),
                 (unsigned)ds_block_index(s, sbh, q0 / 32, 0)};
    };
    auto next_pos = [&](Pos p) -> Pos {
      if (p.q0 + KBM >= q_end)
        return p.hh + 1 < hh_begin + hps ? make_pos(p.j, p.hh + 1, q_first)
                                         : make_pos(p.j + 1, hh_begin, q_first);
      p.dsrow += p.q0 / 32 + 1;  // query block r holds r + 1 key blocks
      p.q0 += KBM;
      p.row0 += KBM;
      return p;
    };
    auto issue = [&](Pos p, bf16* dQ, bf16* dOt, float* dLD) {
      const size_t row0 = p.row0;
      load_tile_soff<KBM, 4>(q + row0 * BD, BD, dQ, wave, lane);
      load_tile_soff<KBM, 4>(dO + row0 * BD, BD, dOt, wave, lane);
      if (wave < 2 && lane < KBM) {  // wave 0: lse * log2(e) of the 32 rows to dLD[0, 32); wave 1: D to dLD[32, 64)
        unsigned off = 4u * lane;
        asm volatile("" : "+v"(off));
        g2lds4(buffer_rsrc(uniform_ptr((wave == 0 ? lse2 : Dd) + row0), 4u * KBM), off,
               dLD + KBM * wave);
      }
    };

    auto body = [&](int it, Pos p, const bf16* cQ, const bf16* cO, const float* cLD, bf16* nQ,
                    bf16* nO, float* nLD) {
      const FragOffsets fl = opaque(fo);
      const int q0 = p.q0;
      const bool live = kw < T && (dwg ? q0 == kw : q0 + KBM - 1 >= kw);
      if (!live && it + 1 < total) issue(next_pos(p), nQ, nO, nLD);
      if (live) {
        // S, then P (kept in bf16 only), then dP: one accumulator tile live at a time.  The
        // next tile's copy is issued after the S products, so that nothing waited for before
        // them (K fragments the allocator parks in scratch) waits for that copy too.
        f32x16 acc = f32x16{};
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = mfma32(frag_row(cQ, 0, t, fl), kf[t], acc);
        if (it + 1 < total) issue(next_pos(p), nQ, nO, nLD);
        // P in place of S (the row offsets arrive as lse * log2(e)); only tiles that straddle
        // the diagonal or the T edge (a wave-uniform test) evaluate the mask:
        // key > query row q0 + acc_row(i, hi)  <=>  dkey > acc_row(i, 0) (a constant)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(&cLD[8 * i4 + 4 * hi]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[4 * i4 + e] = exp2_fast(__builtin_fmaf(acc[4 * i4 + e], c2, -L4[e]));
        }
        const bool full = !dwg && (kw + 31 <= q0) && (kw + 32 <= T);
        if (dwg) {  // key row t*Q_LEN + my_key serves query my_key only (q0 == kw), if < T
          const int dkey = my_key >= T ? KBM : kd0 + (k0 - q0);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (dkey != acc_row(i, 0)) acc[i] = 0.f;
        } else if (!full) {
          const int dkey = my_key >= T ? KBM : kd0 + (k0 - q0);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (dkey > acc_row(i, 0)) acc[i] = 0.f;
        }
        bf16x8 pb[2], dsb[2];
        pb[0] = to_bf16x8(acc, 0);
        pb[1] = to_bf16x8(acc, 8);
        acc = f32x16{};
        // dO fragments 2 products ahead (slot t % 2 refilled right after product t issues)
        bf16x8 ofr[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) ofr[t] = frag_row(cO, 0, t, fl);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          acc = mfma32(ofr[t % 2], vf[t], acc);
          if (t + 2 < 8) ofr[t % 2] = frag_row(cO, 0, t + 2, fl);
          __builtin_amdgcn_sched_barrier(0);
        }
        // dS from the bf16 P that the dV product uses
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(&cLD[KBM + 8 * i4 + 4 * hi]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * i4 + e;
            acc[i] = bf16x8_elem_f32(pb[i >> 3], i & 7) * (acc[i] - D4[e]);
          }
        }
        dsb[0] = to_bf16x8(acc, 0);
        dsb[1] = to_bf16x8(acc, 8);
        if (ds_out && !dwg) {  // hand dS to the dQ kernel (layout: ds_store_offset)
          const size_t blk = (size_t)p.dsrow + kw / 32;
          char* dst = reinterpret_cast<char*>(const_cast<void*>(uniform_ptr(ds_out + blk * 1024)));
          // ds_store_offset(lane, 1) = 1024 + (ds_store_offset(lane, 0) ^ 128)
          unsigned off0 = ds_store_offset(lane, 0);
          asm volatile("" : "+v"(off0));
          store16_global_nt(dst, off0, dsb[0]);
          store16_global_nt(dst + 1024, off0 ^ 128u, dsb[1]);
        }
        // dV then dK products, i = 0..15 (i < 8: dV, (u, c) = (i / 2, i % 2) from the dO
        // tile; then dK from the Q tile); operand fragments four products ahead in slots i % 4
        auto frag_dvk = [&](int i) {
          return frag_col(i < 8 ? cO : cQ, i & 1, (i >> 1) & 3, fl);
        };
        bf16x8 fr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fr[i] = frag_dvk(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int u = (i >> 1) & 3, c = i & 1;
          if (i < 8)
            dVacc[u] = mfma32(pb[c], fr[i & 3], dVacc[u]);
          else
            dKacc[u] = mfma32(dsb[c], fr[i & 3], dKacc[u]);
          if (i + 4 < 16) fr[i & 3] = frag_dvk(i + 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_vmem();
      __syncthreads();
    };

    Pos pos = make_pos(0, hh_begin, q_first);
    if (total > 0) issue(pos, sQ0, sO0, sLD0);
    wait_vmem();
    __syncthreads();
    for (int it = 0; it < total; it += 2) {
      body(it, pos, sQ0, sO0, sLD0, sQ1, sO1, sLD1);
      pos = next_pos(pos);
      if (it + 1 < total) body(it + 1, pos, sQ1, sO1, sLD1, sQ0, sO0, sLD0);
      pos = next_pos(pos);
    }

    // lane owns d = 32u + l32 of key rows kw + acc_row(i, hi).  The lane index goes through
    // an opaque copy so that the output offsets are formed here rather than hoisted out of
    // the tile loop, where they would hold registers.
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const int ohi = lo >> 5, ol32 = lo & 31;
    if (nsp == 1) {
      bf16* dkp = dk + ((size_t)bg * s.KV + krow0 + kw) * BD;
      bf16* dvp = dv + ((size_t)bg * s.KV + krow0 + kw) * BD;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o = acc_row(i, ohi) * BD + 32 * u + ol32;
          dkp[o] = (bf16)(dKacc[u][i] * s.scale);
          dvp[o] = (bf16)dVacc[u][i];
        }
      }
    } else {
      const size_t plane = (size_t)s.B * s.Hkv * s.L * BD;
      float* pk = part + (size_t)split * 2 * plane + ((size_t)bg * s.L + kw) * BD;
      float* pv = pk + plane;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o = acc_row(i, ohi) * BD + 32 * u + ol32;
          pk[o] = dKacc[u][i] * s.scale;
          pv[o] = dVacc[u][i];
        }
      }
    }
    // the suffix key rows t*Q_LEN + [k0, k0 + 128), split by rows over the nsp workgroups
    // that share this key tile
    if constexpr (SUF && !DIAG) {
      const int per = KBN / nsp;
      dkdv_suffix_rows(q, k, v, dO, lse2, Dd, dq_suf, dk, dv, s, b, bg, hg0, T, k0 + split * per,
                       per);
    }
  }
}

hipError_t launch_bwd_dkdv_mfma(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                                const bf16* dout, const float* lse2, const float* Dd,
                                const int32_t* seq_T, bf16* dk, bf16* dv, float* part,
                                int nsplit, bf16* ds_out, bool dense_diagonal, float* dq_suf,
                                unsigned* sched, hipStream_t st) {
  const int pairs = s.B * s.Hkv * nsplit * ((s.L / KBN + 1) / 2);
  LaunchTimer timer(dq_suf ? "bwd_dkdv_suffix_mfma" : "bwd_dkdv_mfma", st);
  if (dense_diagonal && s.step > 0) {
    const dim3 grid(pairs + s.B * s.Hkv * (s.L / KBN) * s.step);
    bwd_dkdv_mfma_kernel<true, false><<<grid, 256, 0, st>>>(q, k, v, dout, lse2, Dd, seq_T, dk, dv,
                                                            part, nsplit, nullptr, nullptr, sched, s);
    return hipGetLastError();
  }
  if (dq_suf && s.step > 0)
    bwd_dkdv_mfma_kernel<false, true><<<dim3(pairs), 256, 0, st>>>(
        q, k, v, dout, lse2, Dd, seq_T, dk, dv, part, nsplit, ds_out, dq_suf, sched, s);
  else
    bwd_dkdv_mfma_kernel<false, false><<<dim3(pairs), 256, 0, st>>>(
        q, k, v, dout, lse2, Dd, seq_T, dk, dv, part, nsplit, ds_out, nullptr, sched, s);
  return hipGetLastError();
}

// Sum of the nsplit partial dK/dV planes, in split order, into block 0 of dk/dv.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part,
                                                          int nsplit, bf16* __restrict__ dk,
                                                          bf16* __restrict__ dv, Shape s) {
  const size_t plane = (size_t)s.B * s.Hkv * s.L * BD;
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= 2 * plane) return;
  const bool is_v = e0 >= plane;
  const size_t e = is_v ? e0 - plane : e0;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + (is_v ? plane : 0) + e);
  for (int sp = 1; sp < nsplit; ++sp)
    acc += *reinterpret_cast<const f32x4*>(part + (size_t)sp * 2 * plane + (is_v ? plane : 0) + e);
  const size_t bg = e / ((size_t)s.L * BD), rem = e % ((size_t)s.L * BD);
  bf16x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = (bf16)acc[j];
  *reinterpret_cast<bf16x4*>((is_v ? dv : dk) + bg * s.KV * BD + rem) = w;
}

hipError_t launch_bwd_dkdv_reduce(const Shape& s, const float* part, int nsplit, bf16* dk,
                                  bf16* dv, hipStream_t st) {
  const size_t n4 = (size_t)s.B * s.Hkv * s.L * BD * 2 / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256));
  LaunchTimer timer("bwd_dkdv_reduce", st);
  dkdv_reduce_kernel<<<grid, 256, 0, st>>>(part, nsplit, dk, dv, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// dQ of block 0, bf16 MFMA.  Workgroup = 4 waves x 32 queries = 128 queries of one head;
// 64-key tiles of block 0 stream through LDS.  Per wave and tile:
//   S^T = K Q^T, dP^T = V dO^T      (A = K, V rows from LDS; B = Q, dO in registers)
//   dS^T = P^T * (dP^T - D)         (each lane owns one query: one lse, one D)
//   dQ^T += K^T dS^T                (A = K columns through transposing LDS reads,
//                                    B = dS^T from the accumulator)
// ----------------------------------------------------------------------------------------
constexpr int QBM = 128;
constexpr int QBN = 64;

// DIAG (measurement variant, with FINAL): the diagonal keys of blocks 1..k go through the
// matrix cores as masked tiles, the way a BlockMask-driven kernel handles them: block t's key
// rows [t*Q_LEN + q0, t*Q_LEN + q0 + 128) form two extra 64-key tiles after the causal ones,
// whose mask keeps key row t*Q_LEN + i for query i < T; dQ then covers every key and is final.
template <bool FINAL, bool DIAG>
__global__ __launch_bounds__(256, 2) void bwd_dq_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int32_t* __restrict__ seq_T, void* __restrict__ dq_out, Shape s) {
  // Two stages in distinct arrays (the copy into one never stalls reads of the other).
  __shared__ __attribute__((aligned(1024))) bf16 sK0[QBN * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[QBN * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[QBN * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[QBN * BD];

  const int n_qt = s.L / QBM;
  int bh, rank;
  map_block(blockIdx.x, s.B * s.Hq, s.G, bh, rank);
  const int qtile = n_qt - 1 - rank;
  const int b = bh / s.Hq, h = bh % s.Hq, g = h / s.G;
  const int bg = b * s.Hkv + g;
  const int T = clamp_T(seq_T, b, s.L);
  const int q0 = qtile * QBM;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;
  const size_t row = (size_t)bh * s.L + my_q;
  const float c2 = s.scale_log2;

  bf16x8 qf[8], df[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    qf[t] = *reinterpret_cast<const bf16x8*>(q + row * BD + 16 * t + 8 * hi);
    df[t] = *reinterpret_cast<const bf16x8*>(dO + row * BD + 16 * t + 8 * hi);
  }
  const float lse2 = lse[row] * kLog2e;
  const float Dq = Dd[row];
  const FragOffsets fo = make_frag_offsets(lane);

  const bf16* kb = k + (size_t)bg * s.KV * BD;
  const bf16* vb = v + (size_t)bg * s.KV * BD;
  const int kv_end = min(q0 + QBM, T);
  const int ncausal = (kv_end + QBN - 1) / QBN;
  // DIAG: two diagonal tiles per block t = 1..k, unless no row of this workgroup is live
  const int ntiles = ncausal + ((DIAG && q0 < T) ? 2 * s.step : 0);
  auto tile_row = [&](int j) -> size_t {  // first key row of tile j in k/v
    if (!DIAG || j < ncausal) return (size_t)j * QBN;
    const int d = j - ncausal;
    return (size_t)(1 + d / 2) * s.L + q0 + QBN * (d & 1);
  };

  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{};

  auto issue = [&](int j, bf16* dK, bf16* dV) {
    load_tile<QBN, 4>(kb + tile_row(j) * BD, BD, dK, wave, lane);
    load_tile<QBN, 4>(vb + tile_row(j) * BD, BD, dV, wave, lane);
  };

  auto body = [&](int j, const bf16* cK, const bf16* cV, bf16* nK, bf16* nV) {
    const FragOffsets fl = opaque(fo);
    if (j + 1 < ntiles) issue(j + 1, nK, nV);
    const bool diag = DIAG && j >= ncausal;  // a diagonal tile of block t >= 1
    // block-local index of the tile's first key
    const int k0 = diag ? q0 + QBN * ((j - ncausal) & 1) : j * QBN;
    if (diag ? (k0 <= qw + 31 && qw <= k0 + QBN - 1) : (k0 <= qw + 31)) {
      f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
      // product i = 4t + 2st + (0: S from K, 1: dP from V); its K or V fragment is read
      // four products ahead into slot i % 4
      auto frag_sp = [&](int i) {
        return frag_row((i & 1) ? cV : cK, ((i >> 1) & 1) * 32, i >> 2, fl);
      };
      bf16x8 fr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fr[i] = frag_sp(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int t = i >> 2, st = (i >> 1) & 1;
        if (i & 1)
          pacc[st] = mfma32(fr[i & 3], df[t], pacc[st]);
        else
          sacc[st] = mfma32(fr[i & 3], qf[t], sacc[st]);
        if (i + 4 < 32) fr[i & 3] = frag_sp(i + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool full = !diag && (k0 + QBN - 1 <= qw) && (k0 + QBN <= T);
      bf16x8 dsb[4];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = exp2_fast(__builtin_fmaf(sacc[st][i], c2, -lse2));
          if (diag) {  // key row t*Q_LEN + key serves query key only, and only for rows < T
            const int key = k0 + st * 32 + acc_row(i, hi);
            if (key != my_q || my_q >= T) pv = 0.f;
          } else if (!full) {
            const int key = k0 + st * 32 + acc_row(i, hi);
            if (key > my_q || key >= T) pv = 0.f;
          }
          dsb[2 * st + (i >> 3)][i & 7] = (bf16)(pv * (pacc[st][i] - Dq));
        }
      }
      // K fragments four products ahead: slot c refilled with column block u + 1 right after
      // product (u, c) is issued
      bf16x8 kfr[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kfr[c] = frag_col(cK, c, 0, fl);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[u] = mfma32(kfr[c], dsb[c], acc[u]);
          if (u < 3) kfr[c] = frag_col(cK, c, u + 1, fl);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };

  if (ntiles > 0) issue(0, sK0, sV0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    body(j, sK0, sV0, sK1, sV1);
    if (j + 1 < ntiles) body(j + 1, sK1, sV1, sK0, sV0);
  }

  // lane owns dQ[my_q][32u + 8*b4 + 4*hi + e] in acc[u][4*b4 + e]
  if constexpr (FINAL) {
    bf16* orow = reinterpret_cast<bf16*>(dq_out) + row * BD + 4 * hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[u][4 * b4 + e] * s.scale);
        *reinterpret_cast<bf16x4*>(orow + 32 * u + 8 * b4) = w;
      }
    }
  } else {
    float* orow = reinterpret_cast<float*>(dq_out) + row * BD + 4 * hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[u][4 * b4 + e] * s.scale;
        *reinterpret_cast<f32x4*>(orow + 32 * u + 8 * b4) = w;
      }
    }
  }
}

hipError_t launch_bwd_dq_mfma(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                              const bf16* dout, const float* lse, const float* Dd,
                              const int32_t* seq_T, void* dq, bool final_out,
                              bool dense_diagonal, hipStream_t st) {
  const dim3 grid(s.B * s.Hq * (s.L / QBM));
  LaunchTimer timer("bwd_dq_mfma", st);
  if (dense_diagonal)  // every key of the row: the final dq
    bwd_dq_mfma_kernel<true, true><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq, s);
  else if (final_out)
    bwd_dq_mfma_kernel<true, false><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq, s);
  else
    bwd_dq_mfma_kernel<false, false><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// dQ of block 0 from the dS blocks the dK/dV kernel stored: dQ = scale dS K, one product per
// tile instead of three.  Workgroup = 4 waves x 32 queries of one head, 64-key tiles.
//   dQ^T += K^T dS^T    (A = K columns through transposing LDS reads, B = dS^T through
//                        transposing reads of the stored 4-query pieces)
// The kernel streams dS from HBM once, so it is bound by how many bytes are in flight: K tiles
// go global -> LDS through three stages and each wave's dS (4 KB per tile) through two
// register sets, both two tiles ahead; the wave copies its dS into a private LDS slot right
// before reading it transposed.  Every tile issues the same 8 loads per wave (indices past the
// end are clamped to a valid tile), so "the loads of the tile after next may still be in
// flight" is the constant wait vmcnt(8).
// Only blocks the wave's rows can see enter the products: key block kb <= the wave's query
// block and 32 kb < T; masked entries inside them were stored as zero.
// ----------------------------------------------------------------------------------------
// With FINAL and dq_add set, the fp32 dQ term in dq_add (the diagonal keys' part, written by
// the dK/dV kernel that also owns the suffix rows) is added before the bf16 write.
template <bool FINAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_ds_kernel(const bf16* __restrict__ k,
                                                           const bf16* __restrict__ ds,
                                                           const int32_t* __restrict__ seq_T,
                                                           void* __restrict__ dq_out,
                                                           const float* __restrict__ dq_add,
                                                           Shape s) {
  __shared__ __attribute__((aligned(1024))) bf16 sK0[QBN * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[QBN * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sK2[QBN * BD];
  __shared__ __attribute__((aligned(1024))) bf16 sS[4 * 2048];  // per wave: 2 blocks of a tile

  const int n_qt = s.L / QBM;
  int bh, rank;
  map_block(blockIdx.x, s.B * s.Hq, s.G, bh, rank);
  const int qtile = n_qt - 1 - rank;
  const int b = bh / s.Hq, h = bh % s.Hq, g = h / s.G;
  const int bg = b * s.Hkv + g;
  const int T = clamp_T(seq_T, b, s.L);
  const int q0 = qtile * QBM;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, hi = lane >> 5;
  const int qb = (q0 >> 5) + wave;             // this wave's query block
  const int nkb = min(qb + 1, (T + 31) >> 5);  // key blocks it reads
  const char* srow = reinterpret_cast<const char*>(ds + ds_block_index(s, bh, qb, 0) * 1024);
  const FragOffsets fo = make_frag_offsets(lane);
  const unsigned rd0 = ds_read_offset(lane, 0, 0);
  char* mine = reinterpret_cast<char*>(sS + wave * 2048);

  const bf16* kb = k + (size_t)bg * s.KV * BD;
  const int kv_end = min(q0 + QBM, T);
  const int ntiles = (kv_end + QBN - 1) / QBN;

  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{};

  auto issue_k = [&](int j, bf16* dst) {
    load_tile<QBN, 4>(kb + (size_t)min(j, ntiles - 1) * QBN * BD, BD, dst, wave, lane);
  };
  // 4 KB of this wave's dS for tile j: blocks 2j and 2j + 1, 1 KB per load (read once:
  // non-temporal, so the stream leaves the K tiles in the caches).
  auto load_ds = [&](int j, bf16x8 (&r)[4]) {
    unsigned off = 16u * lane;
    asm volatile("" : "+v"(off));
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int blk = max(min(2 * j + (x >> 1), nkb - 1), 0);
      r[x] = load16_global_nt(uniform_ptr(srow + (size_t)blk * 2048 + (x & 1) * 1024), off);
    }
  };

  auto put_ds = [&](const bf16x8 (&r)[4]) {  // this wave's dS of one tile into its LDS slot
    unsigned wr = 16u * lane;
    asm volatile("" : "+v"(wr));
#pragma unroll
    for (int x = 0; x < 4; ++x) *reinterpret_cast<bf16x8*>(mine + x * 1024 + wr) = r[x];
  };

  // Tile j: its dS is already in the LDS slot and `r` (which held it) takes tile j + 2;
  // `rn` holds tile j + 1 and goes to the slot once this tile's reads are issued (LDS
  // operations of one wave complete in order).
  auto body = [&](int j, const bf16* cK, bf16* nK, bf16x8 (&r)[4], const bf16x8 (&rn)[4]) {
    const FragOffsets fl = opaque(fo);
    unsigned rd = rd0;
    asm volatile("" : "+v"(rd));
    issue_k(j + 2, nK);
    load_ds(j + 2, r);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      if (2 * j + cc < nkb) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const char* blk = mine + cc * 2048 + 512 * c2;
          const bf16x4 x0 = lds_tr4(blk + rd);
          const bf16x4 x1 = lds_tr4(blk + 256 + rd);
          const bf16x8 bop = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] = mfma32(frag_col(cK, 2 * cc + c2, u, fl), bop, acc[u]);
        }
      }
    }
    wait_vmem_n<8>();  // tile j + 1 has landed; tile j + 2 may still be in flight
    put_ds(rn);
    asm volatile("s_barrier" ::: "memory");
  };

  if (ntiles > 0) {
    bf16x8 ra[4], rb[4];
    issue_k(0, sK0);
    load_ds(0, ra);
    issue_k(1, sK1);
    load_ds(1, rb);
    wait_vmem_n<8>();
    put_ds(ra);
    asm volatile("s_barrier" ::: "memory");
    // Six tiles per trip (3 K stages x 2 register sets); the early exits keep the loop's
    // back edge after the sixth tile only.
    for (int j = 0;; j += 6) {
      body(j, sK0, sK2, ra, rb);
      if (j + 1 >= ntiles) break;
      body(j + 1, sK1, sK0, rb, ra);
      if (j + 2 >= ntiles) break;
      body(j + 2, sK2, sK1, ra, rb);
      if (j + 3 >= ntiles) break;
      body(j + 3, sK0, sK2, rb, ra);
      if (j + 4 >= ntiles) break;
      body(j + 4, sK1, sK0, ra, rb);
      if (j + 5 >= ntiles) break;
      body(j + 5, sK2, sK1, rb, ra);
      if (j + 6 >= ntiles) break;
    }
    wait_vmem();  // nothing stays in flight past the loop
  }

  // lane owns dQ[query][32u + 8*b4 + 4*hi + e] in acc[u][4*b4 + e]
  const size_t row = (size_t)bh * s.L + q0 + 32 * wave + (lane & 31);
  if constexpr (FINAL) {
    bf16* orow = reinterpret_cast<bf16*>(dq_out) + row * BD + 4 * hi;
    const float* arow = dq_add ? dq_add + row * BD + 4 * hi : nullptr;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (arow) a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(arow + 32 * u + 8 * b4));
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[u][4 * b4 + e] * s.scale + a[e]);
        *reinterpret_cast<bf16x4*>(orow + 32 * u + 8 * b4) = w;
      }
    }
  } else {
    float* orow = reinterpret_cast<float*>(dq_out) + row * BD + 4 * hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[u][4 * b4 + e] * s.scale;
        *reinterpret_cast<f32x4*>(orow + 32 * u + 8 * b4) = w;
      }
    }
  }
}

hipError_t launch_bwd_dq_ds(const Shape& s, const bf16* k, const bf16* ds, const int32_t* seq_T,
                            void* dq, bool final_out, const float* dq_add, hipStream_t st) {
  const dim3 grid(s.B * s.Hq * (s.L / QBM));
  LaunchTimer timer("bwd_dq_ds", st);
  if (final_out)
    bwd_dq_ds_kernel<true><<<grid, 256, 0, st>>>(k, ds, seq_T, dq, dq_add, s);
  else
    bwd_dq_ds_kernel<false><<<grid, 256, 0, st>>>(k, ds, seq_T, dq, nullptr, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Vector-ALU backward of block 0 (fp32, and bf16 shapes outside the matrix-core tiling;
// arithmetic in fp32).
// dkdv: one wave per key row j of block 0; lanes take 64 queries at a time for p and ds,
//       then split the head dimension for dV += p dO and dK += ds q (heads in order).
// dq:   one wave per query row; lanes take 64 keys at a time, then split d for dQ += ds k.
// ----------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_dkdv_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int32_t* __restrict__ seq_T, T* __restrict__ dk, T* __restrict__ dv, Shape s) {
  __shared__ float skv[2][D];
  __shared__ float sp[2][64];
  constexpr int E = D / 64;
  const int bg = blockIdx.x / s.L, j = blockIdx.x % s.L;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int Tlen = clamp_T(seq_T, b, s.L);
  const int lane = threadIdx.x;
  const size_t krow = (size_t)bg * s.KV + j;
  for (int e = lane; e < D; e += 64) {
    skv[0][e] = to_f32(k[krow * D + e]);
    skv[1][e] = to_f32(v[krow * D + e]);
  }
  __syncthreads();
  float aK[E], aV[E];
#pragma unroll
  for (int e = 0; e < E; ++e) aK[e] = aV[e] = 0.f;
  if (j < Tlen) {
    for (int h = g * s.G; h < (g + 1) * s.G; ++h) {
      const size_t bh = (size_t)b * s.Hq + h;
      for (int c0 = j; c0 < s.L; c0 += 64) {  // queries i >= j see key j
        const int i = c0 + lane;
        float p = 0.f, ds = 0.f;
        if (i < s.L) {
          const T* qr = q + (bh * s.L + i) * D;
          const T* dr = dO + (bh * s.L + i) * D;
          float sd = 0.f, pd = 0.f;
          for (int e = 0; e < D; ++e) {
            sd += to_f32(qr[e]) * skv[0][e];
            pd += to_f32(dr[e]) * skv[1][e];
          }
          p = exp2_fast(sd * s.scale_log2 - lse[bh * s.L + i] * kLog2e);
          ds = p * (pd - Dd[bh * s.L + i]);
        }
        sp[0][lane] = p;
        sp[1][lane] = ds;
        __syncthreads();
        const int cnt = min(64, s.L - c0);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int dd = lane + 64 * e;
          float av = aV[e], ak = aK[e];
          for (int ii = 0; ii < cnt; ++ii) {
            const size_t r = (bh * s.L + c0 + ii) * D + dd;
            av += sp[0][ii] * to_f32(dO[r]);
            ak += sp[1][ii] * to_f32(q[r]);
          }
          aV[e] = av;
          aK[e] = ak;
        }
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int dd = lane + 64 * e;
    dk[krow * D + dd] = from_f32<T>(aK[e] * s.scale);
    dv[krow * D + dd] = from_f32<T>(aV[e]);
  }
}

template <typename T>
hipError_t launch_bwd_dkdv_valu(const Shape& s, const T* q, const T* k, const T* v,
                                const T* dout, const float* lse, const float* Dd,
                                const int32_t* seq_T, T* dk, T* dv, hipStream_t st) {
  const dim3 grid(s.B * s.Hkv * s.L);
  LaunchTimer timer("bwd_dkdv_valu", st);
  if (s.D == 64)
    bwd_dkdv_valu_kernel<T, 64><<<grid, 64, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dk, dv, s);
  else
    bwd_dkdv_valu_kernel<T, 128><<<grid, 64, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dk, dv, s);
  return hipGetLastError();
}
template hipError_t launch_bwd_dkdv_valu<float>(const Shape&, const float*, const float*,
                                                const float*, const float*, const float*,
                                                const float*, const int32_t*, float*, float*,
                                                hipStream_t);
template hipError_t launch_bwd_dkdv_valu<bf16>(const Shape&, const bf16*, const bf16*,
                                               const bf16*, const bf16*, const float*,
                                               const float*, const int32_t*, bf16*, bf16*,
                                               hipStream_t);

template <typename T, int D, bool FINAL>
__global__ __launch_bounds__(64) void bwd_dq_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int32_t* __restrict__ seq_T, void* __restrict__ dq_out, Shape s) {
  __shared__ float sq[2][D];
  __shared__ float sds[64];
  constexpr int E = D / 64;
  const int bh = blockIdx.x / s.L, i = blockIdx.x % s.L;
  const int b = bh / s.Hq, h = bh % s.Hq, g = h / s.G;
  const int Tlen = clamp_T(seq_T, b, s.L);
  const int lane = threadIdx.x;
  const size_t row = (size_t)bh * s.L + i;
  for (int e = lane; e < D; e += 64) {
    sq[0][e] = to_f32(q[row * D + e]);
    sq[1][e] = to_f32(dO[row * D + e]);
  }
  __syncthreads();
  const float lse2 = lse[row] * kLog2e, Di = Dd[row];
  const int n = (i < Tlen) ? i + 1 : Tlen;
  const T* kb = k + (size_t)(b * s.Hkv + g) * s.KV * D;
  const T* vb = v + (size_t)(b * s.Hkv + g) * s.KV * D;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int j = c0 + lane;
    float ds = 0.f;
    if (j < n) {
      float sd = 0.f, pd = 0.f;
      for (int e = 0; e < D; ++e) {
        sd += sq[0][e] * to_f32(kb[(size_t)j * D + e]);
        pd += sq[1][e] * to_f32(vb[(size_t)j * D + e]);
      }
      const float p = exp2_fast(sd * s.scale_log2 - lse2);
      ds = p * (pd - Di);
    }
    sds[lane] = ds;
    __syncthreads();
    const int cnt = min(64, n - c0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      float a = acc[e];
      for (int jj = 0; jj < cnt; ++jj) a += sds[jj] * to_f32(kb[(size_t)(c0 + jj) * D + dd]);
      acc[e] = a;
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int dd = lane + 64 * e;
    if constexpr (FINAL)
      reinterpret_cast<T*>(dq_out)[row * D + dd] = from_f32<T>(acc[e] * s.scale);
    else
      reinterpret_cast<float*>(dq_out)[row * D + dd] = acc[e] * s.scale;
  }
}

template <typename T>
hipError_t launch_bwd_dq_valu(const Shape& s, const T* q, const T* k, const T* v, const T* dout,
                              const float* lse, const float* Dd, const int32_t* seq_T, void* dq,
                              bool final_out, hipStream_t st) {
  const dim3 grid(s.B * s.Hq * s.L);
  LaunchTimer timer("bwd_dq_valu", st);
  if (s.D == 64) {
    if (final_out) bwd_dq_valu_kernel<T, 64, true><<<grid, 64, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq, s);
    else bwd_dq_valu_kernel<T, 64, false><<<grid, 64, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq, s);
  } else {
    if (final_out) bwd_dq_valu_kernel<T, 128, true><<<grid, 64, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq, s);
    else bwd_dq_valu_kernel<T, 128, false><<<grid, 64, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq, s);
  }
  return hipGetLastError();
}
template hipError_t launch_bwd_dq_valu<float>(const Shape&, const float*, const float*,
                                              const float*, const float*, const float*,
                                              const float*, const int32_t*, void*, bool,
                                              hipStream_t);
template hipError_t launch_bwd_dq_valu<bf16>(const Shape&, const bf16*, const bf16*, const bf16*,
                                             const bf16*, const float*, const float*,
                                             const int32_t*, void*, bool, hipStream_t);

// ----------------------------------------------------------------------------------------
// Suffix backward + dQ finalisation.  One group of 16 lanes per (b, KV group, row i).
// For i < T and t = 1..k (key row r = t*Q_LEN + i), per query head h of the group:
//   p = exp(scale q_h.k_r - lse_h), dp = dO_h.v_r, ds = p (dp - D_h)
//   dV_r = sum_h p dO_h,  dK_r = scale sum_h ds q_h,  dQ_h += scale ds k_r.
// Rows i >= T get no suffix key: dK_r = dV_r = 0 and dQ_h is the block-0 part alone.
// Two passes (dQ head by head, then dK/dV key row by key row) keep the register footprint
// independent of the group size; the second pass re-reads q/dO from cache.
// ----------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_suffix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int32_t* __restrict__ seq_T, const float* __restrict__ dq_acc, T* __restrict__ dq,
    T* __restrict__ dk, T* __restrict__ dv, Shape s) {
  constexpr int E = D / 16;
  const int sub = threadIdx.x & 15;
  const int blocks_per_bg = (s.L + 15) / 16;
  const int bg = blockIdx.x / blocks_per_bg;
  const int i = (blockIdx.x % blocks_per_bg) * 16 + (threadIdx.x >> 4);
  if (i >= s.L) return;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int Tlen = clamp_T(seq_T, b, s.L);
  const size_t kv_base = (size_t)bg * s.KV * D + (size_t)i * D + sub * E;
  const bool live = i < Tlen;

  // pass 1: dQ
  for (int h = g * s.G; h < (g + 1) * s.G; ++h) {
    const size_t row = (size_t)(b * s.Hq + h) * s.L + i;
    float acc[E];
    load_vec<float, E>(dq_acc + row * D + sub * E, acc);
    if (live) {
      float qv[E], dv_[E];
      load_vec<T, E>(q + row * D + sub * E, qv);
      load_vec<T, E>(dO + row * D + sub * E, dv_);
      const float lse2 = lse[row] * kLog2e, Di = Dd[row];
      for (int t = 1; t <= s.step; ++t) {
        float kv[E], vv[E];
        load_vec<T, E>(k + kv_base + (size_t)t * s.L * D, kv);
        load_vec<T, E>(v + kv_base + (size_t)t * s.L * D, vv);
        float sd = 0.f, pd = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          sd += qv[e] * kv[e];
          pd += dv_[e] * vv[e];
        }
        sd = sum16(sd);
        pd = sum16(pd);
        const float p = exp2_fast(sd * s.scale_log2 - lse2);
        const float ds = p * (pd - Di) * s.scale;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += ds * kv[e];
      }
    }
    store_vec<T, E>(dq + row * D + sub * E, acc);
  }

  // pass 2: dK, dV of the suffix key rows t*Q_LEN + i
  for (int t = 1; t <= s.step; ++t) {
    float aK[E], aV[E];
#pragma unroll
    for (int e = 0; e < E; ++e) aK[e] = aV[e] = 0.f;
    if (live) {
      float kv[E], vv[E];
      load_vec<T, E>(k + kv_base + (size_t)t * s.L * D, kv);
      load_vec<T, E>(v + kv_base + (size_t)t * s.L * D, vv);
      for (int h = g * s.G; h < (g + 1) * s.G; ++h) {
        const size_t row = (size_t)(b * s.Hq + h) * s.L + i;
        float qv[E], dv_[E];
        load_vec<T, E>(q + row * D + sub * E, qv);
        load_vec<T, E>(dO + row * D + sub * E, dv_);
        float sd = 0.f, pd = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          sd += qv[e] * kv[e];
          pd += dv_[e] * vv[e];
        }
        sd = sum16(sd);
        pd = sum16(pd);
        const float p = exp2_fast(sd * s.scale_log2 - lse[row] * kLog2e);
        const float ds = p * (pd - Dd[row]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          aV[e] += p * dv_[e];
          aK[e] += ds * qv[e];
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) aK[e] *= s.scale;
    }
    store_vec<T, E>(dk + kv_base + (size_t)t * s.L * D, aK);
    store_vec<T, E>(dv + kv_base + (size_t)t * s.L * D, aV);
  }
}

// Single pass with the step loop outside and every head of the group in registers: each
// diagonal K/V row is read once per (row, group) and its dK/dV row is written right away
// (every input is read once and every output written once, with the non-temporal hint);
// dQ of all heads accumulates in registers and is written at the end.  With H = 2 a row takes
// 32 lanes: each half of them holds G/2 of the heads, the halves' dK/dV sums meet through one
// lane exchange, and one half writes the dK row, the other the dV row.
template <typename T, int D, int G, int H>
__global__ __launch_bounds__(256) void bwd_suffix_g_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int32_t* __restrict__ seq_T, const float* __restrict__ dq_acc, T* __restrict__ dq,
    T* __restrict__ dk, T* __restrict__ dv, Shape s) {
  constexpr int E = D / 16;
  constexpr int GH = G / H;          // heads per half
  constexpr int RPB = 16 / H;        // rows per workgroup
  const int sub = threadIdx.x & 15;
  const int half = H == 1 ? 0 : (threadIdx.x >> 4) & (H - 1);
  const int blocks_per_bg = (s.L + RPB - 1) / RPB;
  const int bg = blockIdx.x / blocks_per_bg;
  const int i = (blockIdx.x % blocks_per_bg) * RPB + (threadIdx.x >> 4) / H;
  if (i >= s.L) return;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int Tlen = clamp_T(seq_T, b, s.L);
  const size_t kv_base = (size_t)bg * s.KV * D + (size_t)i * D + sub * E;
  const size_t row0 = (size_t)(b * s.Hq + g * G + half * GH) * s.L + i;
  const bool live = i < Tlen;
  T* const dkv = half == 0 ? dk : dv;  // (H = 2) the row this half writes

  float dqa[GH][E];
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) dqa[h][e] = 0.f;

  if (live) {
    float qv[GH][E], ov[GH][E], l2[GH], Dh[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const size_t row = row0 + (size_t)h * s.L;
      load_vec<T, E, true>(q + row * D + sub * E, qv[h]);
      load_vec<T, E, true>(dO + row * D + sub * E, ov[h]);
      l2[h] = lse[row] * kLog2e;
      Dh[h] = Dd[row];
    }
    float kc[E], vc[E];
    load_vec<T, E, true>(k + kv_base + (size_t)s.L * D, kc);
    load_vec<T, E, true>(v + kv_base + (size_t)s.L * D, vc);
    for (int t = 1; t <= s.step; ++t) {
      float kn[E], vn[E];
      if (t < s.step) {
        load_vec<T, E, true>(k + kv_base + (size_t)(t + 1) * s.L * D, kn);
        load_vec<T, E, true>(v + kv_base + (size_t)(t + 1) * s.L * D, vn);
      }
      float aK[E], aV[E];
#pragma unroll
      for (int e = 0; e < E; ++e) aK[e] = aV[e] = 0.f;
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        float sd = 0.f, pd = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          sd += qv[h][e] * kc[e];
          pd += ov[h][e] * vc[e];
        }
        sd = sum16(sd);
        pd = sum16(pd);
        const float p = exp2_fast(sd * s.scale_log2 - l2[h]);
        const float ds = p * (pd - Dh[h]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          aV[e] += p * ov[h][e];
          aK[e] += ds * qv[h][e];
          dqa[h][e] += ds * kc[e];
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) aK[e] *= s.scale;
      if constexpr (H == 1) {
        store_vec<T, E, true>(dk + kv_base + (size_t)t * s.L * D, aK);
        store_vec<T, E, true>(dv + kv_base + (size_t)t * s.L * D, aV);
      } else {
        // half 0 writes dK, half 1 dV: each sends the other the sum it lacks
        float w[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float mine = half == 0 ? aK[e] : aV[e];
          w[e] = mine + __shfl_xor(half == 0 ? aV[e] : aK[e], 16);
        }
        store_vec<T, E, true>(dkv + kv_base + (size_t)t * s.L * D, w);
      }
      if (t < s.step) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kc[e] = kn[e];
          vc[e] = vn[e];
        }
      }
    }
  } else {  // rows no query sees: zero
    float z[E];
#pragma unroll
    for (int e = 0; e < E; ++e) z[e] = 0.f;
    for (int t = 1; t <= s.step; ++t) {
      if constexpr (H == 1) {
        store_vec<T, E, true>(dk + kv_base + (size_t)t * s.L * D, z);
        store_vec<T, E, true>(dv + kv_base + (size_t)t * s.L * D, z);
      } else {
        store_vec<T, E, true>(dkv + kv_base + (size_t)t * s.L * D, z);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    const size_t row = row0 + (size_t)h * s.L;
    float a[E];
    load_vec<float, E, true>(dq_acc + row * D + sub * E, a);
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] += s.scale * dqa[h][e];
    store_vec<T, E, true>(dq + row * D + sub * E, a);
  }
}

template <typename T, int D>
static hipError_t bwd_suffix_dispatch(const Shape& s, dim3 grid, hipStream_t st, const T* q,
                                      const T* k, const T* v, const T* dout, const float* lse,
                                      const float* Dd, const int32_t* seq_T, const float* dq_acc,
                                      T* dq, T* dk, T* dv) {
  const dim3 grid2(s.B * s.Hkv * ((s.L + 7) / 8));  // 8 rows of 32 lanes per workgroup
  switch (s.G) {
    case 1: bwd_suffix_g_kernel<T, D, 1, 1><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk, dv, s); break;
    case 2: bwd_suffix_g_kernel<T, D, 2, 1><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk, dv, s); break;
    case 4: bwd_suffix_g_kernel<T, D, 4, 1><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk, dv, s); break;
    case 8: bwd_suffix_g_kernel<T, D, 8, 2><<<grid2, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk, dv, s); break;
    default: bwd_suffix_kernel<T, D><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk, dv, s); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_suffix(const Shape& s, const T* q, const T* k, const T* v, const T* dout,
                             const float* lse, const float* Dd, const int32_t* seq_T,
                             const float* dq_acc, T* dq, T* dk, T* dv, hipStream_t st) {
  const dim3 grid(s.B * s.Hkv * ((s.L + 15) / 16));
  LaunchTimer timer("bwd_suffix", st);
  if (s.D == 64)
    return bwd_suffix_dispatch<T, 64>(s, grid, st, q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk, dv);
  return bwd_suffix_dispatch<T, 128>(s, grid, st, q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk, dv);
}
template hipError_t launch_bwd_suffix<float>(const Shape&, const float*, const float*,
                                             const float*, const float*, const float*,
                                             const float*, const int32_t*, const float*, float*,
                                             float*, float*, hipStream_t);
template hipError_t launch_bwd_suffix<bf16>(const Shape&, const bf16*, const bf16*, const bf16*,
                                            const bf16*, const float*, const float*,
                                            const int32_t*, const float*, bf16*, bf16*, bf16*,
                                            hipStream_t);

// ----------------------------------------------------------------------------------------
// Whole-TTT suffix backward (bf16, d = 128): one group of 16 lanes per (b, KV group, row i)
// takes the diagonal keys r = t*Q_LEN + i of every block t = 1..K-1 for the queries of every
// step k >= t (same per-key terms as the per-step kernels above).  Blocks go in chunks of
// NB whose dK/dV rows accumulate in registers over the steps and heads and are written once;
// steps run in the outer loop, so a step's dQ row (its fp32 block-0 part from dq_acc plus the
// diagonal terms) is complete in the chunk that holds its last block k, and goes back to
// dq_acc in fp32 from the chunks before that one.
// Layouts: q, dO, dq [K, B, Hq, Q_LEN, d]; lse, Dd [K, B, Hq, Q_LEN]; dq_acc of steps
// 1..K-1 [K-1, B, Hq, Q_LEN, d] fp32; k, v, dk, dv the cache [B, Hkv, K*Q_LEN, d]; s.step =
// K-1, s.KV = K*Q_LEN.  dQ of step 0 has no diagonal term and is not touched.
// ----------------------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(256) void bwd_suffix_sweep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int32_t* __restrict__ seq_T, float* __restrict__ dq_acc, bf16* __restrict__ dq,
    bf16* __restrict__ dk, bf16* __restrict__ dv, Shape s) {
  constexpr int E = BD / 16;
  const int sub = threadIdx.x & 15;
  const int blocks_per_bg = (s.L + 15) / 16;
  const int bg = blockIdx.x / blocks_per_bg;
  const int i = (blockIdx.x % blocks_per_bg) * 16 + (threadIdx.x >> 4);
  if (i >= s.L) return;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const bool live = i < clamp_T(seq_T, b, s.L);
  const size_t kv_base = ((size_t)bg * s.KV + i) * BD + sub * E;
  const size_t step_rows = (size_t)s.B * s.Hq * s.L;
  const size_t row_g = (size_t)(b * s.Hq + g * s.G) * s.L + i;  // head g*G, step 0
  const int nblk = s.step;

  for (int t0 = 1; t0 <= nblk; t0 += NB) {
    const int nb = min(NB, nblk - t0 + 1);  // blocks t0 .. t0 + nb - 1
    float aK[NB][E], aV[NB][E];
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int e = 0; e < E; ++e) aK[c][e] = aV[c][e] = 0.f;
    // (step, head) pairs (kk, h), kk = t0..K-1: steps k >= t0 reach blocks t0 .. min(k, t0 +
    // nb - 1).  The rows of the next pair are loaded while the current one computes (read
    // once: non-temporal; the diagonal K/V rows, read for every pair, stay cached).
    struct RowIn {
      bf16x8 qr, orw;
      float l2, Di;
      f32x4 a0, a1;
    };
    auto load_in = [&](int kk, int h, RowIn& r) {
      const size_t hrow = row_g + (size_t)h * s.L;
      const size_t row = (size_t)kk * step_rows + hrow;
      const float* accp = dq_acc + ((size_t)(kk - 1) * step_rows + hrow) * BD + sub * E;
      r.a0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(accp));
      r.a1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(accp + 4));
      if (live) {
        r.qr = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(q + row * BD + sub * E));
        r.orw = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(dO + row * BD + sub * E));
        r.l2 = lse[row] * kLog2e;
        r.Di = Dd[row];
      }
    };
    RowIn cur, nxt;
    load_in(t0, 0, cur);
    for (int kk = t0, h = 0;;) {
      int kn = kk, hn = h + 1;
      if (hn == s.G) {
        hn = 0;
        ++kn;
      }
      const bool more = kn <= nblk;
      if (more) load_in(kn, hn, nxt);
      const int reach = min(kk - t0 + 1, nb);
      const bool last = kk < t0 + nb;  // no later chunk holds a block <= kk
      {
        const size_t hrow = row_g + (size_t)h * s.L;
        const size_t row = (size_t)kk * step_rows + hrow;
        float* accp = dq_acc + ((size_t)(kk - 1) * step_rows + hrow) * BD + sub * E;
        float dqa[E];  // sum over the chunk's blocks of ds * k (the per-step kernels' order)
#pragma unroll
        for (int e = 0; e < E; ++e) dqa[e] = 0.f;
        if (live) {
          float qv[E], ov[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            qv[e] = (float)cur.qr[e];
            ov[e] = (float)cur.orw[e];
          }
          const float l2 = cur.l2, Di = cur.Di;
#pragma unroll
          for (int c = 0; c < NB; ++c) {
            if (c < reach) {
              float kc[E], vc[E];
              load_vec<bf16, E>(k + kv_base + (size_t)(t0 + c) * s.L * BD, kc);
              load_vec<bf16, E>(v + kv_base + (size_t)(t0 + c) * s.L * BD, vc);
              float sd = 0.f, pd = 0.f;
#pragma unroll
              for (int e = 0; e < E; ++e) {
                sd += qv[e] * kc[e];
                pd += ov[e] * vc[e];
              }
              sd = sum16(sd);
              pd = sum16(pd);
              const float p = exp2_fast(sd * s.scale_log2 - l2);
              const float ds = p * (pd - Di);
#pragma unroll
              for (int e = 0; e < E; ++e) {
                aV[c][e] += p * ov[e];
                aK[c][e] += ds * qv[e];
                dqa[e] += ds * kc[e];
              }
            }
          }
        }
        float a[E] = {cur.a0[0], cur.a0[1], cur.a0[2], cur.a0[3],
                      cur.a1[0], cur.a1[1], cur.a1[2], cur.a1[3]};
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] += s.scale * dqa[e];
        if (last)
          store_vec<bf16, E, true>(dq + row * BD + sub * E, a);
        else
          store_vec<float, E>(accp, a);
      }
      if (!more) break;
      cur = nxt;
      kk = kn;
      h = hn;
    }
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if (c < nb) {
#pragma unroll
        for (int e = 0; e < E; ++e) aK[c][e] *= s.scale;
        store_vec<bf16, E, true>(dk + kv_base + (size_t)(t0 + c) * s.L * BD, aK[c]);
        store_vec<bf16, E, true>(dv + kv_base + (size_t)(t0 + c) * s.L * BD, aV[c]);
      }
    }
  }
}

hipError_t launch_bwd_suffix_sweep(const Shape& s, const bf16* q, const bf16* k, const bf16* v,
                                   const bf16* dout, const float* lse, const float* Dd,
                                   const int32_t* seq_T, float* dq_acc, bf16* dq, bf16* dk,
                                   bf16* dv, hipStream_t st) {
  const dim3 grid(s.B * s.Hkv * ((s.L + 15) / 16));
  LaunchTimer timer("bwd_suffix_sweep", st);
  bwd_suffix_sweep_kernel<6><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dd, seq_T, dq_acc, dq, dk,
                                                   dv, s);
  return hipGetLastError();
}

}  // namespace ttt

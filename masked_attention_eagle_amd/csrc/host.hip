// C ABI of the TTT sparse tree attention library: validation, workspace layout, dispatch.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "launch.h"
#include "ttt_attn.h"
#include "ttt_loss.h"

namespace ttt {

// ------------------------------------------------------------------ per-launch timing hook
// Launches from several threads may be timed at once: all state below is guarded by g_mu, and a
// timer keeps its own events until its launch is done, so a read or reset from another thread
// never takes events that a launch still uses.
namespace {
struct TimingRecord {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_mu;
std::atomic<bool> g_timing_on{false};
void* g_flush_buf = nullptr;  // with timing on: overwritten before every timed launch
size_t g_flush_bytes = 0;
std::vector<TimingRecord> g_free;  // event pairs ready for reuse
std::vector<TimingRecord> g_done;  // launches whose stop event is recorded, not yet read

struct Accum {
  char name[48];
  int launches;
  double ms;
};
std::vector<Accum> g_accum;
}  // namespace

LaunchTimer::LaunchTimer(const char* name, hipStream_t st)
    : name_(name), st_(st), start_(nullptr), stop_(nullptr), on_(false) {
  if (!g_timing_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_free.empty()) {
    start_ = g_free.back().start;
    stop_ = g_free.back().stop;
    g_free.pop_back();
  } else {
    if (hipEventCreate(&start_) != hipSuccess) return;
    if (hipEventCreate(&stop_) != hipSuccess) {
      hipEventDestroy(start_);
      return;
    }
  }
  on_ = true;
  if (g_flush_buf) launch_flush_fill(g_flush_buf, g_flush_bytes, st);  // outside the timed span
  hipEventRecord(start_, st);
}

LaunchTimer::~LaunchTimer() {
  if (!on_) return;
  hipEventRecord(stop_, st_);
  std::lock_guard<std::mutex> lock(g_mu);
  g_done.push_back(TimingRecord{name_, start_, stop_});
}

static void accumulate(const char* name, double ms) {
  for (auto& a : g_accum) {
    if (strncmp(a.name, name, sizeof(a.name)) == 0) {
      a.launches += 1;
      a.ms += ms;
      return;
    }
  }
  Accum a{};
  strncpy(a.name, name, sizeof(a.name) - 1);
  a.launches = 1;
  a.ms = ms;
  g_accum.push_back(a);
}

// ------------------------------------------------------------------ validation and layout
namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// bf16 shapes the matrix-core kernels tile (head_dim 128, q_len a multiple of 128); other
// bf16 shapes and all fp32 ones run on the vector-ALU kernels.
bool mfma_path(const ttt_attn_params* p) {
  return p->dtype == TTT_DTYPE_BF16 && p->head_dim == 128 && p->q_len % 128 == 0;
}

// bf16 at head_dim 64 with q_len a multiple of 128 (per-step calls with a workspace): the same
// kernels through head_dim-128 copies of the rows whose upper half is zero.  The zero half adds
// exact zeros to every dot product, so the logits, P, lse and the lower halves of o and of
// every gradient are those of the head_dim-64 problem, at twice its matrix-core work; the
// copies sit in the caller's workspace ahead of the kernels' own regions.
bool pad64_path(const ttt_attn_params* p) {
  return p->dtype == TTT_DTYPE_BF16 && p->head_dim == 64 && p->q_len % 128 == 0;
}
ttt_attn_params widened(const ttt_attn_params* p) {
  ttt_attn_params w = *p;
  w.head_dim = 128;
  return w;
}

int validate(const ttt_attn_params* p) {
  if (!p) return TTT_E_NULL;
  if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->q_len <= 0 ||
      p->head_dim <= 0 || p->ttt_step < 0)
    return TTT_E_SHAPE;
  if (p->heads_q % p->heads_kv != 0) return TTT_E_SHAPE;
  if (!isfinite(p->scale) || !(p->scale > 0.f)) return TTT_E_SHAPE;
  const int64_t kv = ((int64_t)p->ttt_step + 1) * p->q_len;  // widened before the add
  if (kv > INT32_MAX) return TTT_E_SHAPE;
  // Thread counts of the largest grids must stay below 2^32 and element counts below 2^40.
  const int64_t rows_q = (int64_t)p->batch * p->heads_q * p->q_len;
  const int64_t rows_kv = (int64_t)p->batch * p->heads_kv * kv;
  if (rows_q * p->head_dim > (1ll << 40) || rows_kv * p->head_dim > (1ll << 40)) return TTT_E_SHAPE;
  if (p->dtype != TTT_DTYPE_F32 && p->dtype != TTT_DTYPE_BF16) return TTT_E_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return TTT_E_UNSUPPORTED;
  if (mfma_path(p) || pad64_path(p)) {
    if ((int64_t)p->batch * p->heads_kv * p->q_len * 16 >= (1ll << 32)) return TTT_E_SHAPE;
  } else {
    // one 64-lane workgroup per query row (per key row in the dK/dV kernel)
    if (rows_q * 64 >= (1ll << 32) || (int64_t)p->batch * p->heads_kv * p->q_len * 64 >= (1ll << 32))
      return TTT_E_SHAPE;
  }
  if (p->flags & ~(TTT_FLAG_SEPARATE_SUFFIX | TTT_FLAG_RECOMPUTE_DQ | TTT_FLAG_DENSE_DIAGONAL |
                   TTT_FLAG_FUSED_SUFFIX_BWD))
    return TTT_E_UNSUPPORTED;
  if ((p->flags & TTT_FLAG_SEPARATE_SUFFIX) && (p->flags & TTT_FLAG_DENSE_DIAGONAL))
    return TTT_E_UNSUPPORTED;
  // the fused backward suffix hands its dQ term to the stored-dS dQ kernel
  if ((p->flags & TTT_FLAG_FUSED_SUFFIX_BWD) &&
      (p->flags & (TTT_FLAG_RECOMPUTE_DQ | TTT_FLAG_DENSE_DIAGONAL)))
    return TTT_E_UNSUPPORTED;
  return TTT_OK;
}

// Whole-TTT calls: the matrix-core shapes only, and the step-stacked q/o/dout/dq tensors
// (K times the per-step rows) within the same element and grid limits.
int validate_sweep(const ttt_attn_params* p) {
  const int rc = validate(p);
  if (rc != TTT_OK) return rc;
  if (!mfma_path(p) && !pad64_path(p)) return TTT_E_UNSUPPORTED;
  const int64_t rows_all = ((int64_t)p->ttt_step + 1) * p->batch * p->heads_q * p->q_len;
  if (rows_all * p->head_dim > (1ll << 40) || rows_all / 16 >= (1ll << 31)) return TTT_E_SHAPE;
  return TTT_OK;
}

// bf16 backward with the diagonal keys as masked matrix-core tiles (measurement variant).
bool dense_bwd(const ttt_attn_params* p) {
  return mfma_path(p) && (p->flags & TTT_FLAG_DENSE_DIAGONAL) && p->ttt_step > 0;
}
// bf16 backward: the dQ kernel reads dS stored by the dK/dV kernel unless asked to recompute
// (the dense-diagonal backward always recomputes: its dQ kernel also takes the diagonal tiles).
bool stored_ds(const ttt_attn_params* p) {
  return mfma_path(p) && !(p->flags & TTT_FLAG_RECOMPUTE_DQ) && !dense_bwd(p);
}
// bf16 backward whose dK/dV kernel also takes the suffix key rows (no suffix kernel).
bool fused_bwd_suffix(const ttt_attn_params* p) {
  return mfma_path(p) && (p->flags & TTT_FLAG_FUSED_SUFFIX_BWD) && p->ttt_step > 0;
}
// The forward merges the suffix inside the causal kernel unless asked for the separate
// suffix kernel; the vector-ALU path always runs it.
bool fused_fwd(const ttt_attn_params* p) {
  return mfma_path(p) && !(p->flags & TTT_FLAG_SEPARATE_SUFFIX);
}

Shape make_shape(const ttt_attn_params* p) {
  Shape s;
  s.B = p->batch;
  s.Hq = p->heads_q;
  s.Hkv = p->heads_kv;
  s.L = p->q_len;
  s.D = p->head_dim;
  s.step = p->ttt_step;
  s.G = p->heads_q / p->heads_kv;
  s.KV = (p->ttt_step + 1) * p->q_len;
  s.scale = p->scale;
  s.scale_log2 = p->scale * kLog2e;
  s.nst = 1;
  return s;
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Number of shares the query heads of one KV group are split into in the dK/dV kernel (its
// queue holds one unit per share and 128-key tile, and its grid one workgroup per two units):
// doubled while the grid is below two workgroups per CU and the group still splits evenly.
int dkdv_nsplit(const Shape& s) {
  const int64_t base = (int64_t)s.B * s.Hkv * ((s.L / 128 + 1) / 2);
  int n = 1;
  while (base * n < 512 && n < s.G && s.G % (2 * n) == 0) n *= 2;
  return n;
}

struct FwdLayout {
  size_t oc = 0, lsec = 0, total = 0;
};
FwdLayout fwd_layout(const Shape& s, bool fused) {
  FwdLayout w;
  size_t off = 0;
  const size_t rows_q = (size_t)s.B * s.Hq * s.L;
  if (s.step > 0 && !fused) {
    w.oc = off;
    off += round_up(rows_q * s.D * 4);
    w.lsec = off;
    off += round_up(rows_q * 4);
  }
  w.total = off;
  return w;
}

struct BwdLayout {
  size_t Dd = 0, lse2 = 0, sched = 0, part = 0, ds = 0, dqacc = 0, total = 0;
  int nsplit = 1;
};
// D; (bf16) lse * log2(e) for the dK/dV kernel and the split dK/dV partials (heads of a group
// over several workgroups); the dS blocks of block 0 when the dQ kernel reads them; for k > 0
// the fp32 dQ accumulator that the suffix kernel finalises.  D, lse * log2(e) and dS are held
// for each of the s.nst steps, and (whole TTT) the dQ accumulators of steps 1..nst-1.
size_t ds_step_elems(const Shape& s) {
  const size_t n = s.L / 32;
  return (size_t)s.B * s.Hq * (n * (n + 1) / 2) * 32 * 32;
}
BwdLayout bwd_layout(const Shape& s, bool mfma, bool with_ds, bool dense = false) {
  BwdLayout w;
  const size_t rows_1 = (size_t)s.B * s.Hq * s.L;
  const size_t rows_q = rows_1 * s.nst;
  size_t off = 0;
  w.Dd = off;
  off += round_up(rows_q * 4);
  if (mfma) {
    w.lse2 = off;
    off += round_up(rows_q * 4);
    w.sched = off;  // the dK/dV kernel's queue counters, one per 128-byte line
    off += round_up(8 * 128);
    w.nsplit = dkdv_nsplit(s);
    if (w.nsplit > 1) {
      w.part = off;
      off += round_up((size_t)w.nsplit * 2 * s.B * s.Hkv * s.L * s.D * 4);
    }
  }
  if (with_ds) {
    w.ds = off;
    off += round_up(ds_step_elems(s) * s.nst * 2);
  }
  if (s.step > 0 && !dense) {
    w.dqacc = off;
    off += round_up(rows_1 * s.D * 4 * (s.nst > 1 ? s.nst - 1 : 1));
  }
  w.total = off;
  return w;
}

// The head_dim-128 copies of a head_dim-64 call (pad64_path), in bytes from the workspace start:
// q, k, v and (forward output, backward input) o; for the backward also dO, dq, dk, dv; the
// kernels' own workspace follows at `inner`.
struct PadLayout {
  size_t q = 0, k = 0, v = 0, o = 0, dout = 0, dq = 0, dk = 0, dv = 0, inner = 0;
};
// rows_q: rows of q (o, dO, dq); rows_kv: rows of k (v, dk, dv)
PadLayout pad_regions(size_t rows_q, size_t rows_kv, bool bwd) {
  PadLayout w;
  const size_t rq = round_up(rows_q * 128 * 2);
  const size_t rkv = round_up(rows_kv * 128 * 2);
  size_t off = 0;
  w.q = off; off += rq;
  w.k = off; off += rkv;
  w.v = off; off += rkv;
  w.o = off; off += rq;
  if (bwd) {
    w.dout = off; off += rq;
    w.dq = off; off += rq;
    w.dk = off; off += rkv;
    w.dv = off; off += rkv;
  }
  w.inner = off;
  return w;
}
PadLayout pad_layout(const Shape& s, bool bwd) {
  return pad_regions((size_t)s.B * s.Hq * s.L, (size_t)s.B * s.Hkv * s.KV, bwd);
}

int hip_status(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_E_HIP; }

// ------------------------------------------------------------------ no-allocation scratch
// The backward's scratch for ttt_attn_bwd_noalloc: a file-scope device array, one copy per
// GPU.  Host code never uses the array's name as an address (on the host it only names the
// symbol); the device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and is what the kernels receive.
static __device__ __align__(256) char scratch[TTT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TTT_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TTT_E_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return TTT_OK;
}

}  // namespace
}  // namespace ttt

using namespace ttt;

extern "C" {

int ttt_attn_version(void) { return 104; }

const char* ttt_attn_status_string(int status) {
  switch (status) {
    case TTT_OK: return "ok";
    case TTT_E_NULL: return "null pointer argument";
    case TTT_E_SHAPE: return "invalid shape (non-positive size, heads_q % heads_kv != 0, ttt_step < 0, scale not finite and positive, or size overflow)";
    case TTT_E_UNSUPPORTED: return "unsupported configuration (head_dim other than 64 or 128, unknown dtype, unknown or conflicting flags, or a whole-TTT call outside bf16 with head_dim 128 and q_len % 128 == 0)";
    case TTT_E_ALIGN: return "pointer not 16-byte aligned";
    case TTT_E_WORKSPACE: return "workspace smaller than required";
    case TTT_E_HIP: return "HIP kernel launch failed";
    case TTT_E_SCRATCH: return "the no-allocation backward needs more scratch than its fixed maximum (TTT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t ttt_attn_fwd_workspace_size(const ttt_attn_params* p) {
  if (validate(p) != TTT_OK) return 0;
  if (pad64_path(p)) {
    const ttt_attn_params w = widened(p);
    return pad_layout(make_shape(p), false).inner + fwd_layout(make_shape(&w), fused_fwd(&w)).total;
  }
  return fwd_layout(make_shape(p), fused_fwd(p)).total;
}

size_t ttt_attn_bwd_workspace_size(const ttt_attn_params* p) {
  if (validate(p) != TTT_OK) return 0;
  if (pad64_path(p)) {
    const ttt_attn_params w = widened(p);
    return pad_layout(make_shape(p), true).inner +
           bwd_layout(make_shape(&w), true, stored_ds(&w), dense_bwd(&w)).total;
  }
  return bwd_layout(make_shape(p), mfma_path(p), stored_ds(p), dense_bwd(p)).total;
}

}  // extern "C"

namespace ttt {
namespace {

// Vector-ALU steps (fp32, and bf16 shapes outside the matrix-core tiling): element loads
// convert to fp32, all arithmetic is fp32, outputs are rounded once on the write.
template <typename T>
hipError_t fwd_valu(const Shape& s, const void* q, const void* k, const void* v,
                    const int32_t* seq_T, void* o, float* lse, float* oc, float* lsec,
                    bool final_causal, hipStream_t st) {
  const T* qt = (const T*)q;
  const T* kt = (const T*)k;
  const T* vt = (const T*)v;
  hipError_t e = launch_fwd_causal_valu<T>(s, qt, kt, vt, seq_T, final_causal ? o : (void*)oc,
                                           lsec, final_causal, st);
  if (e != hipSuccess || final_causal) return e;
  return launch_fwd_suffix<T>(s, qt, kt, vt, seq_T, oc, lsec, (T*)o, lse, st);
}

template <typename T>
hipError_t bwd_valu(const Shape& s, const void* q, const void* k, const void* v,
                    const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                    void* dq, void* dk, void* dv, float* Dd, float* dqacc, bool final_causal,
                    hipStream_t st) {
  const T* qt = (const T*)q;
  const T* kt = (const T*)k;
  const T* vt = (const T*)v;
  const T* dot = (const T*)dout;
  hipError_t e;
  if ((e = launch_bwd_rowdot<T>(s, (const T*)o, dot, Dd, nullptr, nullptr, nullptr, st)) !=
      hipSuccess)
    return e;
  if ((e = launch_bwd_dkdv_valu<T>(s, qt, kt, vt, dot, lse, Dd, seq_T, (T*)dk, (T*)dv, st)) !=
      hipSuccess)
    return e;
  if ((e = launch_bwd_dq_valu<T>(s, qt, kt, vt, dot, lse, Dd, seq_T,
                                 final_causal ? dq : (void*)dqacc, final_causal, st)) != hipSuccess)
    return e;
  if (final_causal) return e;
  return launch_bwd_suffix<T>(s, qt, kt, vt, dot, lse, Dd, seq_T, dqacc, (T*)dq, (T*)dk, (T*)dv,
                              st);
}

// One forward step on validated arguments (s.KV is the row stride of k and v per KV group).
int run_fwd(const ttt_attn_params* p, const Shape& s, const void* q, const void* k,
            const void* v, const int32_t* seq_T, void* o, float* lse, char* ws, hipStream_t st) {
  const bool fused = fused_fwd(p);
  const FwdLayout w = fwd_layout(s, fused);
  const bool final_causal = s.step == 0 || fused;
  float* oc = final_causal ? nullptr : (float*)(ws + w.oc);
  float* lsec = final_causal ? lse : (float*)(ws + w.lsec);
  hipError_t e;
  if (mfma_path(p)) {
    const bf16* qb = (const bf16*)q;
    const bf16* kb = (const bf16*)k;
    const bf16* vb = (const bf16*)v;
    // final_causal with k > 0: the kernel merges the suffix keys itself
    e = launch_fwd_causal_mfma(s, qb, kb, vb, seq_T, final_causal ? o : (void*)oc, lsec,
                               final_causal, (p->flags & TTT_FLAG_DENSE_DIAGONAL) != 0, st);
    if (e != hipSuccess) return TTT_E_HIP;
    if (!final_causal)
      e = launch_fwd_suffix<bf16>(s, qb, kb, vb, seq_T, oc, lsec, (bf16*)o, lse, st);
  } else if (p->dtype == TTT_DTYPE_BF16) {
    e = fwd_valu<bf16>(s, q, k, v, seq_T, o, lse, oc, lsec, final_causal, st);
  } else {
    e = fwd_valu<float>(s, q, k, v, seq_T, o, lse, oc, lsec, final_causal, st);
  }
  return hip_status(e);
}

// One backward step on validated arguments.
int run_bwd(const ttt_attn_params* p, const Shape& s, const void* q, const void* k,
            const void* v, const int32_t* seq_T, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, char* ws, hipStream_t st) {
  const bool with_ds = stored_ds(p);
  const bool dense = dense_bwd(p);
  const BwdLayout w = bwd_layout(s, mfma_path(p), with_ds, dense);
  float* Dd = (float*)(ws + w.Dd);
  const bool final_causal = s.step == 0 || dense;
  float* dqacc = final_causal ? nullptr : (float*)(ws + w.dqacc);
  hipError_t e;
  if (mfma_path(p)) {
    const bf16* qb = (const bf16*)q;
    const bf16* kb = (const bf16*)k;
    const bf16* vb = (const bf16*)v;
    const bf16* dob = (const bf16*)dout;
    float* part = w.nsplit > 1 ? (float*)(ws + w.part) : nullptr;
    bf16* dsb = with_ds ? (bf16*)(ws + w.ds) : nullptr;
    void* dq_causal = final_causal ? dq : (void*)dqacc;
    float* lse2 = (float*)(ws + w.lse2);
    unsigned* sched = (unsigned*)(ws + w.sched);
    if ((e = launch_bwd_rowdot<bf16>(s, (const bf16*)o, dob, Dd, lse, lse2, sched, st)) !=
        hipSuccess)
      return TTT_E_HIP;
    // fused: the dK/dV kernel writes the suffix rows and the suffix dQ term (into the dQ
    // accumulator's space), and the dQ kernel adds that term and writes the final dq
    const bool fused = fused_bwd_suffix(p);
    if ((e = launch_bwd_dkdv_mfma(s, qb, kb, vb, dob, lse2, Dd, seq_T, (bf16*)dk, (bf16*)dv, part,
                                  w.nsplit, dsb, dense, fused ? dqacc : nullptr, sched, st)) !=
        hipSuccess)
      return TTT_E_HIP;
    if (w.nsplit > 1 &&
        (e = launch_bwd_dkdv_reduce(s, part, w.nsplit, (bf16*)dk, (bf16*)dv, st)) != hipSuccess)
      return TTT_E_HIP;
    if (fused)
      e = launch_bwd_dq_ds(s, kb, dsb, seq_T, dq, true, dqacc, st);
    else if (with_ds)
      e = launch_bwd_dq_ds(s, kb, dsb, seq_T, dq_causal, final_causal, nullptr, st);
    else
      e = launch_bwd_dq_mfma(s, qb, kb, vb, dob, lse, Dd, seq_T, dq_causal, final_causal, dense,
                             st);
    if (e != hipSuccess) return TTT_E_HIP;
    if (!final_causal && !fused)
      e = launch_bwd_suffix<bf16>(s, qb, kb, vb, dob, lse, Dd, seq_T, dqacc, (bf16*)dq, (bf16*)dk,
                                  (bf16*)dv, st);
  } else if (p->dtype == TTT_DTYPE_BF16) {
    e = bwd_valu<bf16>(s, q, k, v, seq_T, o, lse, dout, dq, dk, dv, Dd, dqacc, final_causal, st);
  } else {
    e = bwd_valu<float>(s, q, k, v, seq_T, o, lse, dout, dq, dk, dv, Dd, dqacc, final_causal, st);
  }
  return hip_status(e);
}

// Whole-TTT sweep: p->ttt_step = K - 1, K steps over one cache of K*Q_LEN rows per KV group.
// Shape of step k: its own step index and the cache's row stride.
Shape sweep_shape(const ttt_attn_params* p, int k) {
  Shape s = make_shape(p);
  s.step = k;  // s.KV stays (K) * Q_LEN: the row stride of the cache
  return s;
}
size_t sweep_fwd_ws(const ttt_attn_params* p) {
  size_t m = 0;
  for (int k = 0; k <= p->ttt_step; ++k) m = std::max(m, fwd_layout(sweep_shape(p, k), fused_fwd(p)).total);
  return m;
}
// The whole-TTT backward ignores TTT_FLAG_DENSE_DIAGONAL and TTT_FLAG_FUSED_SUFFIX_BWD (its
// dK/dV sums over the steps go through its own suffix kernel): its paths and workspace follow
// the flags without those bits.
ttt_attn_params sweep_bwd_params(const ttt_attn_params* p) {
  ttt_attn_params q = *p;
  q.flags &= ~(TTT_FLAG_DENSE_DIAGONAL | TTT_FLAG_FUSED_SUFFIX_BWD);
  return q;
}
// The whole-TTT backward's shape for the launches that cover every step at once (row-dot,
// dK/dV of block 0, its reduction).
Shape sweep_all_shape(const ttt_attn_params* p) {
  Shape s = make_shape(p);
  s.nst = p->ttt_step + 1;
  return s;
}

// Whole-TTT forward and backward on validated arguments (head_dim-128 rows: the head_dim-64
// calls pass their zero-padded copies).
int run_fwd_sweep(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                  const int32_t* seq_T, void* o, float* lse, char* ws, hipStream_t st) {
  const size_t qel = (size_t)p->batch * p->heads_q * p->q_len * p->head_dim;  // per step
  const size_t rows = (size_t)p->batch * p->heads_q * p->q_len;
  for (int kk = 0; kk <= p->ttt_step; ++kk) {
    const int rc = run_fwd(p, sweep_shape(p, kk), (const bf16*)q + kk * qel, k, v, seq_T,
                           (bf16*)o + kk * qel, lse + kk * rows, ws, st);
    if (rc != TTT_OK) return rc;
  }
  return TTT_OK;
}
size_t sweep_bwd_ws(const ttt_attn_params* p) {
  const ttt_attn_params pb = sweep_bwd_params(p);
  return bwd_layout(sweep_all_shape(p), true, stored_ds(&pb)).total;
}
int run_bwd_sweep(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                  const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, char* ws, hipStream_t st) {
  const ttt_attn_params pb = sweep_bwd_params(p);
  const bool with_ds = stored_ds(&pb);
  const Shape sa = sweep_all_shape(p);
  const BwdLayout w = bwd_layout(sa, true, with_ds);
  const size_t qel = (size_t)p->batch * p->heads_q * p->q_len * p->head_dim;
  const size_t rows = (size_t)p->batch * p->heads_q * p->q_len;
  const bf16* qb = (const bf16*)q;
  const bf16* kb = (const bf16*)k;
  const bf16* vb = (const bf16*)v;
  const bf16* dob = (const bf16*)dout;
  float* Dd = (float*)(ws + w.Dd);
  float* lse2 = (float*)(ws + w.lse2);
  float* part = w.nsplit > 1 ? (float*)(ws + w.part) : nullptr;
  bf16* dsb = with_ds ? (bf16*)(ws + w.ds) : nullptr;
  float* dqacc = (float*)(ws + w.dqacc);
  hipError_t e;
  // Block 0: one row-dot launch, one dK/dV launch and one reduction over the queries of all
  // steps (the keys of block 0 are seen by every step), which writes its dk/dv rows.
  unsigned* sched = (unsigned*)(ws + w.sched);
  if ((e = launch_bwd_rowdot<bf16>(sa, (const bf16*)o, dob, Dd, lse, lse2, sched, st)) != hipSuccess)
    return TTT_E_HIP;
  if ((e = launch_bwd_dkdv_mfma(sa, qb, kb, vb, dob, lse2, Dd, seq_T, (bf16*)dk, (bf16*)dv, part,
                                w.nsplit, dsb, false, nullptr, sched, st)) != hipSuccess)
    return TTT_E_HIP;
  if (w.nsplit > 1 &&
      (e = launch_bwd_dkdv_reduce(sa, part, w.nsplit, (bf16*)dk, (bf16*)dv, st)) != hipSuccess)
    return TTT_E_HIP;
  // Per step, the block-0 dQ: final for step 0, into its fp32 accumulator for the others.
  for (int kk = 0; kk <= p->ttt_step; ++kk) {
    const Shape s = sweep_shape(p, kk);
    void* dq_causal = kk == 0 ? (void*)((bf16*)dq) : (void*)(dqacc + (kk - 1) * qel);
    if (with_ds)
      e = launch_bwd_dq_ds(s, kb, dsb + kk * ds_step_elems(s), seq_T, dq_causal, kk == 0, nullptr,
                           st);
    else
      e = launch_bwd_dq_mfma(s, qb + kk * qel, kb, vb, dob + kk * qel, lse + kk * rows,
                             Dd + kk * rows, seq_T, dq_causal, kk == 0, false, st);
    if (e != hipSuccess) return TTT_E_HIP;
  }
  // Blocks 1..K-1 and the diagonal part of dQ: one launch over every step.
  if (p->ttt_step > 0 &&
      (e = launch_bwd_suffix_sweep(sa, qb, kb, vb, dob, lse, Dd, seq_T, dqacc, (bf16*)dq,
                                   (bf16*)dk, (bf16*)dv, st)) != hipSuccess)
    return TTT_E_HIP;
  return TTT_OK;
}
// The head_dim-128 copies of a whole-TTT head_dim-64 call: q, o (dO, dq) of every step and the
// cache k, v (dk, dv).
PadLayout sweep_pad(const ttt_attn_params* p, bool bwd) {
  const size_t K = (size_t)p->ttt_step + 1;
  return pad_regions(K * p->batch * p->heads_q * p->q_len, K * p->batch * p->heads_kv * p->q_len,
                     bwd);
}

}  // namespace
}  // namespace ttt

extern "C" {

int ttt_attn_fwd(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                 const int32_t* seq_T, void* o, float* lse, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int rc = validate(p);
  if (rc != TTT_OK) return rc;
  if (!q || !k || !v || !seq_T || !o || !lse) return TTT_E_NULL;
  const Shape s = make_shape(p);
  const size_t need = ttt_attn_fwd_workspace_size(p);
  if (need > 0 && !workspace) return TTT_E_NULL;
  if (workspace_bytes < need) return TTT_E_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(seq_T) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(workspace))
    return TTT_E_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  if (pad64_path(p)) {
    const ttt_attn_params p2 = widened(p);
    const PadLayout w = pad_layout(s, false);
    char* ws = (char*)workspace;
    const size_t rq = (size_t)s.B * s.Hq * s.L, rkv = (size_t)s.B * s.Hkv * s.KV;
    if (launch_pad64(q, ws + w.q, rq, st) != hipSuccess ||
        launch_pad64(k, ws + w.k, rkv, st) != hipSuccess ||
        launch_pad64(v, ws + w.v, rkv, st) != hipSuccess)
      return TTT_E_HIP;
    rc = run_fwd(&p2, make_shape(&p2), ws + w.q, ws + w.k, ws + w.v, seq_T, ws + w.o, lse,
                 ws + w.inner, st);
    if (rc != TTT_OK) return rc;
    return hip_status(launch_unpad64(ws + w.o, o, rq, st));
  }
  return run_fwd(p, s, q, k, v, seq_T, o, lse, (char*)workspace, st);
}

int ttt_attn_bwd(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                 const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int rc = validate(p);
  if (rc != TTT_OK) return rc;
  if (!q || !k || !v || !seq_T || !o || !lse || !dout || !dq || !dk || !dv) return TTT_E_NULL;
  const Shape s = make_shape(p);
  const size_t need = ttt_attn_bwd_workspace_size(p);
  if (need > 0 && !workspace) return TTT_E_NULL;
  if (workspace_bytes < need) return TTT_E_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(seq_T) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(workspace))
    return TTT_E_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  if (pad64_path(p)) {
    const ttt_attn_params p2 = widened(p);
    const PadLayout w = pad_layout(s, true);
    char* ws = (char*)workspace;
    const size_t rq = (size_t)s.B * s.Hq * s.L, rkv = (size_t)s.B * s.Hkv * s.KV;
    if (launch_pad64(q, ws + w.q, rq, st) != hipSuccess ||
        launch_pad64(k, ws + w.k, rkv, st) != hipSuccess ||
        launch_pad64(v, ws + w.v, rkv, st) != hipSuccess ||
        launch_pad64(o, ws + w.o, rq, st) != hipSuccess ||
        launch_pad64(dout, ws + w.dout, rq, st) != hipSuccess)
      return TTT_E_HIP;
    rc = run_bwd(&p2, make_shape(&p2), ws + w.q, ws + w.k, ws + w.v, seq_T, ws + w.o, lse,
                 ws + w.dout, ws + w.dq, ws + w.dk, ws + w.dv, ws + w.inner, st);
    if (rc != TTT_OK) return rc;
    if (launch_unpad64(ws + w.dq, dq, rq, st) != hipSuccess ||
        launch_unpad64(ws + w.dk, dk, rkv, st) != hipSuccess ||
        launch_unpad64(ws + w.dv, dv, rkv, st) != hipSuccess)
      return TTT_E_HIP;
    return TTT_OK;
  }
  return run_bwd(p, s, q, k, v, seq_T, o, lse, dout, dq, dk, dv, (char*)workspace, st);
}

int ttt_attn_bwd_noalloc(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                         const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, void* stream) {
  int rc = validate(p);
  if (rc != TTT_OK) return rc;
  if (!q || !k || !v || !seq_T || !o || !lse || !dout || !dq || !dk || !dv) return TTT_E_NULL;
  ttt_attn_params pr = *p;
  pr.flags |= TTT_FLAG_RECOMPUTE_DQ;  // no logits-sized dS buffer
  const Shape s = make_shape(&pr);
  // bf16 head_dim 64 takes the zero-padded copies as ttt_attn_bwd does (same kernels, same bits);
  // they sit at the start of the scratch array, ahead of the head_dim-128 call's regions
  const bool pad = pad64_path(&pr);
  const ttt_attn_params p2 = pad ? widened(&pr) : pr;
  const PadLayout pl = pad ? pad_layout(s, true) : PadLayout{};
  const BwdLayout w = bwd_layout(make_shape(&p2), mfma_path(&p2), stored_ds(&p2), dense_bwd(&p2));
  if (pl.inner + w.total > TTT_NOALLOC_SCRATCH_BYTES) return TTT_E_SCRATCH;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(seq_T) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return TTT_E_ALIGN;
  char* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws)) != TTT_OK) return rc;
  const hipStream_t st = (hipStream_t)stream;
  if (!pad) return run_bwd(&pr, s, q, k, v, seq_T, o, lse, dout, dq, dk, dv, ws, st);
  const size_t rq = (size_t)s.B * s.Hq * s.L, rkv = (size_t)s.B * s.Hkv * s.KV;
  if (launch_pad64(q, ws + pl.q, rq, st) != hipSuccess ||
      launch_pad64(k, ws + pl.k, rkv, st) != hipSuccess ||
      launch_pad64(v, ws + pl.v, rkv, st) != hipSuccess ||
      launch_pad64(o, ws + pl.o, rq, st) != hipSuccess ||
      launch_pad64(dout, ws + pl.dout, rq, st) != hipSuccess)
    return TTT_E_HIP;
  rc = run_bwd(&p2, make_shape(&p2), ws + pl.q, ws + pl.k, ws + pl.v, seq_T, ws + pl.o, lse,
               ws + pl.dout, ws + pl.dq, ws + pl.dk, ws + pl.dv, ws + pl.inner, st);
  if (rc != TTT_OK) return rc;
  if (launch_unpad64(ws + pl.dq, dq, rq, st) != hipSuccess ||
      launch_unpad64(ws + pl.dk, dk, rkv, st) != hipSuccess ||
      launch_unpad64(ws + pl.dv, dv, rkv, st) != hipSuccess)
    return TTT_E_HIP;
  return TTT_OK;
}

size_t ttt_attn_fwd_sweep_workspace_size(const ttt_attn_params* p) {
  if (validate_sweep(p) != TTT_OK) return 0;
  if (pad64_path(p)) {
    const ttt_attn_params w = widened(p);
    return sweep_pad(p, false).inner + sweep_fwd_ws(&w);
  }
  return sweep_fwd_ws(p);
}
size_t ttt_attn_bwd_sweep_workspace_size(const ttt_attn_params* p) {
  if (validate_sweep(p) != TTT_OK) return 0;
  if (pad64_path(p)) {
    const ttt_attn_params w = widened(p);
    return sweep_pad(p, true).inner + sweep_bwd_ws(&w);
  }
  return sweep_bwd_ws(p);
}

int ttt_attn_fwd_sweep(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_T, void* o, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = validate_sweep(p);
  if (rc != TTT_OK) return rc;
  if (!q || !k || !v || !seq_T || !o || !lse) return TTT_E_NULL;
  const size_t need = ttt_attn_fwd_sweep_workspace_size(p);
  if (need > 0 && !workspace) return TTT_E_NULL;
  if (workspace_bytes < need) return TTT_E_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(seq_T) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(workspace))
    return TTT_E_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  if (pad64_path(p)) {
    const ttt_attn_params p2 = widened(p);
    const PadLayout w = sweep_pad(p, false);
    char* ws = (char*)workspace;
    const size_t K = (size_t)p->ttt_step + 1;
    const size_t rq = K * p->batch * p->heads_q * p->q_len;
    const size_t rkv = K * p->batch * p->heads_kv * p->q_len;
    if (launch_pad64(q, ws + w.q, rq, st) != hipSuccess ||
        launch_pad64(k, ws + w.k, rkv, st) != hipSuccess ||
        launch_pad64(v, ws + w.v, rkv, st) != hipSuccess)
      return TTT_E_HIP;
    rc = run_fwd_sweep(&p2, ws + w.q, ws + w.k, ws + w.v, seq_T, ws + w.o, lse, ws + w.inner, st);
    if (rc != TTT_OK) return rc;
    return hip_status(launch_unpad64(ws + w.o, o, rq, st));
  }
  return run_fwd_sweep(p, q, k, v, seq_T, o, lse, (char*)workspace, st);
}

int ttt_attn_bwd_sweep(const ttt_attn_params* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_T, const void* o, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = validate_sweep(p);
  if (rc != TTT_OK) return rc;
  if (!q || !k || !v || !seq_T || !o || !lse || !dout || !dq || !dk || !dv) return TTT_E_NULL;
  if (!workspace) return TTT_E_NULL;
  if (workspace_bytes < ttt_attn_bwd_sweep_workspace_size(p)) return TTT_E_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(seq_T) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(workspace))
    return TTT_E_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  if (pad64_path(p)) {
    const ttt_attn_params p2 = widened(p);
    const PadLayout w = sweep_pad(p, true);
    char* ws = (char*)workspace;
    const size_t K = (size_t)p->ttt_step + 1;
    const size_t rq = K * p->batch * p->heads_q * p->q_len;
    const size_t rkv = K * p->batch * p->heads_kv * p->q_len;
    if (launch_pad64(q, ws + w.q, rq, st) != hipSuccess ||
        launch_pad64(k, ws + w.k, rkv, st) != hipSuccess ||
        launch_pad64(v, ws + w.v, rkv, st) != hipSuccess ||
        launch_pad64(o, ws + w.o, rq, st) != hipSuccess ||
        launch_pad64(dout, ws + w.dout, rq, st) != hipSuccess)
      return TTT_E_HIP;
    rc = run_bwd_sweep(&p2, ws + w.q, ws + w.k, ws + w.v, seq_T, ws + w.o, lse, ws + w.dout,
                       ws + w.dq, ws + w.dk, ws + w.dv, ws + w.inner, st);
    if (rc != TTT_OK) return rc;
    if (launch_unpad64(ws + w.dq, dq, rq, st) != hipSuccess ||
        launch_unpad64(ws + w.dk, dk, rkv, st) != hipSuccess ||
        launch_unpad64(ws + w.dv, dv, rkv, st) != hipSuccess)
      return TTT_E_HIP;
    return TTT_OK;
  }
  return run_bwd_sweep(p, q, k, v, seq_T, o, lse, dout, dq, dk, dv, (char*)workspace, st);
}

int ttt_loss_grad_inplace(const ttt_loss_params* p, void* z, const void* target, const float* g,
                          float* loss, void* stream) {
  if (!p) return TTT_E_NULL;
  if (p->rows < 1 || p->vocab < 1 || p->rows >= (1ll << 31) ||
      p->rows * (int64_t)p->vocab >= (1ll << 40))
    return TTT_E_SHAPE;
  if (p->vocab % 8 != 0 || (p->dtype != TTT_DTYPE_BF16 && p->dtype != TTT_DTYPE_F32))
    return TTT_E_UNSUPPORTED;
  if (!z || !target || !g) return TTT_E_NULL;
  if (!aligned16(z) || !aligned16(target) || ((uintptr_t)g & 3) || ((uintptr_t)loss & 3))
    return TTT_E_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (p->dtype == TTT_DTYPE_BF16)
    e = launch_loss_grad<bf16>(p->rows, p->vocab, (bf16*)z, (const bf16*)target, g, loss, st);
  else
    e = launch_loss_grad<float>(p->rows, p->vocab, (float*)z, (const float*)target, g, loss, st);
  return hip_status(e);
}

int ttt_attn_timing_enable(int on) {
  return g_timing_on.exchange(on != 0) ? 1 : 0;
}

int ttt_attn_timing_read(ttt_attn_kernel_time* out, int max_entries) {
  std::lock_guard<std::mutex> lock(g_mu);
  int status = TTT_OK;
  for (const auto& r : g_done) {
    float ms = 0.f;
    if (status == TTT_OK && (hipEventSynchronize(r.stop) != hipSuccess ||
                             hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess))
      status = TTT_E_HIP;
    if (status == TTT_OK) accumulate(r.name, ms);
    g_free.push_back(r);
  }
  g_done.clear();
  if (status != TTT_OK) return status;
  int n = 0;
  for (const auto& a : g_accum) {
    if (n >= max_entries) break;
    if (out) {
      memset(&out[n], 0, sizeof(out[n]));
      strncpy(out[n].name, a.name, sizeof(out[n].name) - 1);
      out[n].launches = a.launches;
      out[n].total_ms = a.ms;
    }
    ++n;
  }
  return n;
}

int ttt_attn_timing_flush(void* buf, size_t bytes) {
  if (buf && (((uintptr_t)buf & 15) || bytes % 16 || bytes == 0)) return TTT_E_ALIGN;
  std::lock_guard<std::mutex> lock(g_mu);
  g_flush_buf = buf;
  g_flush_bytes = buf ? bytes : 0;
  return TTT_OK;
}

void ttt_attn_timing_reset(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (const auto& r : g_done) {
    hipEventSynchronize(r.stop);
    g_free.push_back(r);
  }
  g_done.clear();
  g_accum.clear();
}

}  // extern "C"

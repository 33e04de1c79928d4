"""Benchmark of the TTT sparse tree attention hot path on one MI355X.

One step = one TTT sweep of a draft layer: the forward of every TTT step k = 0..K-1 (KV length
(k+1) * Q_LEN) followed by the backward of every step in reverse order, i.e. all kernels of the
path (tile classification, causal MFMA forward, suffix gather/merge, backward row dot, causal
MFMA dK/dV and dQ, suffix backward with dQ finalisation).  Inputs are seeded synthetic tensors
already resident in HBM; outputs and workspaces are preallocated, so the timed region only
launches kernels.

value = unmasked TFLOP/s = sum over steps of 14 * d * |M| * B * Hq (4d forward + 10d backward
per unmasked (query, key) pair) / step time.  tokens/s = B * Q_LEN / step time.
pct_roofline = t_roof / step time, t_roof = causal flops at the bf16 matrix-core peak plus the
suffix's marginal K/V bytes and the backward preprocessing bytes at the HBM peak.

Prints one JSON line.  ``--gpus`` above 1 is refused: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT-attn fwd+bwd unmasked TFLOP/s + tokens/s at Q_LEN=4096, TTT=7; % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
# Scaled FETCH_SIZE + WRITE_SIZE counter readings per kernel launch, taken with rocprofv3 on the
# same workload; used only while the kernel's source is unchanged since they were taken.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
TRAFFIC_TAG = {2: "llama31_8b", 3: "padding_heavy", 4: "llama33_70b", 5: "qwen3_30b_a3b"}
CSRC = os.path.join(ROOT, "masked_attention_eagle_amd", "csrc")


def kernel_source(name: str) -> str:
    if name.startswith("fwd_"):
        return "kernels_fwd.hip"
    return "kernels_aux.hip" if name == "bwd_rowdot" else "kernels_bwd.hip"


def source_digest(files) -> str:
    """sha256 (16 hex digits) of the code in the given csrc files with comments and white space
    removed, so that the digest moves with the compiled code and not with its comments."""
    import hashlib
    import re
    h = hashlib.sha256()
    for fn in files:
        with open(os.path.join(CSRC, fn)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config: int, name: str):
    """HBM bytes per launch of kernel `name` from the committed counter summary, or None when
    there is none for this workload or the kernel's code has changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f)[TRAFFIC_TAG[config]]["kernels"][name]
    except (OSError, KeyError, ValueError):
        return None
    if source_digest((kernel_source(name), "common.cuh")) != entry.get("code_digest"):
        return None
    return int(entry["bytes_per_launch"])


def run_traffic(config: int, name: str, sweep: bool, dq_mode: str, suffix: str):
    """measured_traffic for this run's dominant kernel, or None when the run takes other paths
    than the counters were taken on (per-step calls, stored dS, fused suffix): the whole-TTT
    dK/dV launch covers every step, and the other dQ and suffix paths run the kernels
    differently (no dS stores, for one)."""
    if sweep or dq_mode != "stored" or suffix != "fused":
        return None
    return measured_traffic(config, name)


def causal_pairs(L: int, T: int) -> int:
    """|M_causal| for one (batch, head): T(T+1)/2 over rows i < T plus T keys for each of the
    L - T padded rows."""
    return T * (T + 1) // 2 + (L - T) * T


def total_pairs(L: int, step: int, T: int) -> int:
    """|M| for one (batch, head) at TTT step `step`: the causal part plus one diagonal key per
    later block for every row i < T."""
    return causal_pairs(L, T) + step * T


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload number (2: the 8B draft layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra measurement of the step captured in a HIP graph")
    ap.add_argument("--suffix", choices=("fused", "separate", "dense"), default="fused",
                    help="diagonal keys of blocks 1..k: merged inside the causal forward kernel, "
                         "the forward's standalone suffix kernel, or (measurement variant, forward "
                         "and backward) masked diagonal matrix-core tiles")
    ap.add_argument("--sweep", action="store_true",
                    help="time the whole-TTT calls (one forward and one backward call over one KV "
                         "cache, dK/dV summed over the steps) instead of the per-step calls")
    ap.add_argument("--dq-mode", choices=("stored", "recompute", "fused-suffix"), default="stored",
                    help="dS handed from the dK/dV kernel to the dQ kernel through the workspace, "
                         "or recomputed in the dQ kernel, or handed over with the diagonal keys' "
                         "rows taken by the dK/dV kernel (no suffix kernel)")
    ap.add_argument("--loss", action="store_true",
                    help="measure the in-place masked softmax-loss gradient on the draft LM head "
                         "of one TTT step (N = 8192 tokens, V = 32000, bf16) instead")
    ap.add_argument("--no-also", action="store_true",
                    help="with the default workload, skip the sub-records of the other workloads "
                         "(the Llama-3.3-70B-shaped layer, the padding-heavy batch and the "
                         "long-TTT Qwen3-shaped layer)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured matrix-core and stream-copy peaks")
    ap.add_argument("--cold-steps", type=int, default=2,
                    help="steps timed again with the caches flushed before every launch "
                         "(per-kernel cold-cache averages; 0 to skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run one plain device-to-device copy of MIB MiB (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    """One plain copy of known size, so that HBM byte counters can be scaled by what they read
    for it (expected: mib MiB fetched and mib MiB written)."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "bytes": 2 * n}))


def sweep_step(args, w, T, blocks, lib, A, dev, t_setup):
    """Resident inputs of the whole-TTT calls: one KV cache [B, Hkv, K*L, d], step-major q
    and dO; returns the step function (forward sweep, then backward sweep)."""
    import torch
    bf = torch.bfloat16
    steps = list(w.steps)
    K = len(steps)
    kc = torch.cat([torch.from_numpy(b[0]) for b in blocks], 2).to(dev, bf)
    vc = torch.cat([torch.from_numpy(b[1]) for b in blocks], 2).to(dev, bf)
    qa = torch.stack([torch.from_numpy(inputs_mod().q_at(w, k)) for k in steps]).to(dev, bf)
    da = torch.stack([torch.from_numpy(inputs_mod().do_at(w, k)) for k in steps]).to(dev, bf)
    Td = torch.as_tensor(T, device=dev)
    oa, la = torch.empty_like(qa), torch.empty(qa.shape[:4], dtype=torch.float32, device=dev)
    dqa, dkc, dvc = torch.empty_like(qa), torch.empty_like(kc), torch.empty_like(vc)
    p = A.make_params(w.B, w.Hq, w.Hkv, w.L, w.d, steps[-1], w.scale, A.TTT_DTYPE_BF16,
                      A.path_flags(args.suffix, args.dq_mode))
    nb = max(int(lib.ttt_attn_fwd_sweep_workspace_size(ctypes.byref(p))),
             int(lib.ttt_attn_bwd_sweep_workspace_size(ctypes.byref(p))))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    fa = (ctypes.byref(p), qa.data_ptr(), kc.data_ptr(), vc.data_ptr(), Td.data_ptr(),
          oa.data_ptr(), la.data_ptr(), ws.data_ptr(), nb)
    ba = (ctypes.byref(p), qa.data_ptr(), kc.data_ptr(), vc.data_ptr(), Td.data_ptr(),
          oa.data_ptr(), la.data_ptr(), da.data_ptr(), dqa.data_ptr(), dkc.data_ptr(),
          dvc.data_ptr(), ws.data_ptr(), nb)
    keep = (kc, vc, qa, da, Td, oa, la, dqa, dkc, dvc, ws, p)

    def one_step():
        _ = keep
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # the caller's stream
        for fn, a in ((lib.ttt_attn_fwd_sweep, fa), (lib.ttt_attn_bwd_sweep, ba)):
            rc = fn(*a, sp)
            if rc:
                raise A.TTTError(rc, A.status_string(rc))
    return one_step, setup_s


def inputs_mod():
    from masked_attention_eagle_amd import inputs
    return inputs


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the TTT attention path needs no collective (every "
              "(sequence, KV group) is independent under data parallelism), so each GPU runs its "
              "share at these shapes; multi-GPU runs are not supported here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from masked_attention_eagle_amd import inputs
    from masked_attention_eagle_amd import ttt_attn as A

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.loss:
        bench_loss(args)
        return
    A.load()
    torch.cuda.set_device(torch.device("cuda", 0))
    peaks = None if args.no_peaks else measure_peaks()
    out = measure(args, args.config, peaks)
    if args.config == 2 and not args.no_also:
        # the metric's other headline workload (4), then the padding-heavy (3) and long-TTT (5)
        # workloads, timed the same way in the same run
        out["also"] = {}
        for cfg in (4, 3, 5):
            torch.cuda.empty_cache()
            sub = measure(args, cfg, peaks)
            out["also"][sub["config"]["workload"]] = {
                k: sub[k] for k in ("value", "unit", "ms_per_step", "tokens_per_s",
                                    "valid_tokens_per_s", "step_ms", "pct_roofline", "roofline",
                                    "config", "unmasked_flop_per_step", "kernels") if k in sub}
    if peaks is not None:
        out["peaks_measured"] = peaks
    if not args.no_cpu_baseline:
        w = inputs.WORKLOADS[args.config]
        out["cpu_baseline"] = cpu_baseline(w, inputs.seq_lengths(w), list(w.steps))
    print(json.dumps(out))


def measure_peaks():
    """The chip's attainable peaks on the plainest workloads, from the library's probes: bf16
    matrix-core TFLOP/s (2048 workgroups = 8 waves per CU, operands in registers) and HBM
    stream-copy GB/s (1 GiB copied, read + write bytes), best of 5 runs each."""
    import torch
    from masked_attention_eagle_amd import ttt_attn as A
    wgs, iters = 2048, 4096
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    src = torch.ones(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return min(ts)

    t_mfma = best(lambda: A.probe_mfma_bf16(sink, wgs, iters))
    t_copy = best(lambda: A.probe_copy(src, dst))
    mfma = wgs * 4 * iters * 8 * 32768 / t_mfma / 1e12
    copy = 2 * src.numel() * 2 / t_copy / 1e9
    return {"mfma_bf16_tflops": round(mfma, 1), "mfma_frac_of_spec": round(mfma / PEAK_BF16_TFLOPS, 4),
            "copy_gbs": round(copy, 1), "copy_frac_of_spec": round(copy / PEAK_HBM_GBS, 4),
            "how": "library probes: 32x32x16 bf16 MFMA on 4 register chains per wave, 8 waves "
                   "per CU; 1 GiB device copy, 16 KB per workgroup, 16-byte loads/stores; best of 5"}


def measure(args, config, peaks=None):
    """Times the sweep of one workload; returns the JSON record (without the CPU baseline)."""
    import torch
    from masked_attention_eagle_amd import inputs
    from masked_attention_eagle_amd import ttt_attn as A
    lib = A.load()
    dev = torch.device("cuda", 0)
    w = inputs.WORKLOADS[config]
    assert w.dtype == "bf16"
    T = inputs.seq_lengths(w)
    steps = list(w.steps)
    K = len(steps)

    # ---------------------------------------------------------------- resident inputs
    t_setup = time.time()
    bf = torch.bfloat16
    blocks = [inputs.kv_block(w, t) for t in range(K)]
    if args.sweep:
        one_step, setup_s = sweep_step(args, w, T, blocks, lib, A, dev, t_setup)
        blocks = []
    kv = []
    for k in (steps if not args.sweep else []):
        kk = np.concatenate([blocks[t][0] for t in range(k + 1)], axis=2)
        vv = np.concatenate([blocks[t][1] for t in range(k + 1)], axis=2)
        kv.append((torch.from_numpy(kk).to(dev, bf), torch.from_numpy(vv).to(dev, bf)))
        del kk, vv
    if not args.sweep:
        qs = [torch.from_numpy(inputs.q_at(w, k)).to(dev, bf) for k in steps]
        dos = [torch.from_numpy(inputs.do_at(w, k)).to(dev, bf) for k in steps]
        Td = torch.as_tensor(T, device=dev)
        os_ = [torch.empty_like(q) for q in qs]
        lses = [torch.empty(q.shape[:3], dtype=torch.float32, device=dev) for q in qs]
        dqs = [torch.empty_like(q) for q in qs]
        dks = [torch.empty_like(kv[i][0]) for i in range(K)]
        dvs = [torch.empty_like(kv[i][1]) for i in range(K)]
        params = [A.make_params(w.B, w.Hq, w.Hkv, w.L, w.d, k, w.scale, A.TTT_DTYPE_BF16,
                                A.path_flags(args.suffix, args.dq_mode)) for k in steps]
        ws_bytes = max(max(A.fwd_workspace_size(p), A.bwd_workspace_size(p)) for p in params)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        setup_s = time.time() - t_setup

        fwd_args = [(ctypes.byref(params[i]), qs[i].data_ptr(), kv[i][0].data_ptr(), kv[i][1].data_ptr(),
                     Td.data_ptr(), os_[i].data_ptr(), lses[i].data_ptr(), ws.data_ptr(), ws_bytes)
                    for i in range(K)]
        bwd_args = [(ctypes.byref(params[i]), qs[i].data_ptr(), kv[i][0].data_ptr(), kv[i][1].data_ptr(),
                     Td.data_ptr(), os_[i].data_ptr(), lses[i].data_ptr(), dos[i].data_ptr(),
                     dqs[i].data_ptr(), dks[i].data_ptr(), dvs[i].data_ptr(), ws.data_ptr(), ws_bytes)
                    for i in range(K)]

        def one_step():
            sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # the caller's stream
            for i in range(K):
                rc = lib.ttt_attn_fwd(*fwd_args[i], sp)
                if rc:
                    raise A.TTTError(rc, A.status_string(rc))
            for i in reversed(range(K)):
                rc = lib.ttt_attn_bwd(*bwd_args[i], sp)
                if rc:
                    raise A.TTTError(rc, A.status_string(rc))

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    # events between the steps (on the stream every kernel is launched on) give the per-step
    # spread; the value itself is the wall clock over all timed steps.  No per-kernel events
    # here: they add a few microseconds to every launch.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        one_step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    sec = (t1 - t0) / args.steps

    # ---------------------------------------------------------------- kernel-timed region
    # the same K steps again with every launch bracketed by hipEvents on its stream: the
    # per-kernel averages (and the roofline of the dominant kernel) come from here
    kernels = {}
    sec_events = None
    if not args.no_kernel_timing:
        A.timing_reset()
        A.timing_enable(True)
        torch.cuda.synchronize()
        e0 = time.perf_counter()
        for _ in range(args.steps):
            one_step()
        torch.cuda.synchronize()
        sec_events = (time.perf_counter() - e0) / args.steps
        A.timing_enable(False)
        kernels = A.timing_read()

    # per-kernel averages with the caches flushed (1 GiB overwritten) before every launch: the
    # bandwidth-bound kernels then read everything from HBM, none of it from the last-level
    # cache that the kernel before them filled
    kernels_cold = {}
    if args.cold_steps > 0 and not args.no_kernel_timing:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        A.timing_reset()
        A.timing_flush(flush)
        A.timing_enable(True)
        for _ in range(args.cold_steps):
            one_step()
        torch.cuda.synchronize()
        A.timing_enable(False)
        A.timing_flush(None)
        kernels_cold = A.timing_read()
        del flush

    # the same step captured once in a HIP graph and replayed (launch gaps removed); reported
    # beside the eager figure, which stays the headline
    graph_sec = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_sec = (time.perf_counter() - g0) / args.steps
        del graph

    # ---------------------------------------------------------------- accounting
    pairs_step = [sum(total_pairs(w.L, k, int(t)) for t in T) * w.Hq for k in steps]
    causal = sum(causal_pairs(w.L, int(t)) for t in T) * w.Hq  # per launch of a causal kernel
    flops = sum(14 * w.d * p for p in pairs_step)
    value = flops / sec / 1e12
    tokens = w.B * w.L / sec
    # algorithmic matrix-core flops of each causal kernel per TTT step: dK/dV kernel does the
    # S, dP, dV and dK products (8d per pair), dQ kernel the dQ product (2d), forward 4d.  The
    # rate is the kernel's flops per sweep over its time per sweep: per launch for the
    # per-step calls (one launch per step), and the same for the whole-TTT dK/dV launch, which
    # covers every step.
    alg = {"bwd_dkdv_mfma": 8 * w.d * causal, "bwd_dkdv_suffix_mfma": 8 * w.d * causal,
           "bwd_dq_mfma": 2 * w.d * causal,
           "bwd_dq_ds": 2 * w.d * causal, "fwd_causal_mfma": 4 * w.d * causal}
    nsteps = len(steps)
    rows_q = w.B * w.Hq * w.L
    live_q = int(sum(int(t) for t in T)) * w.Hq
    live_kv = int(sum(int(t) for t in T)) * w.Hkv
    kk = [k for k in steps if k > 0]
    L32 = w.L // 32
    # algorithmic HBM bytes per launch of the bandwidth-bound kernels, averaged over the steps
    # each one runs at
    alg_bytes = {}
    if kk:
        # forward standalone suffix kernel: q of the live rows, the fp32 causal state (o_c,
        # lse_c), the diagonal K/V rows; o and lse written
        alg_bytes["fwd_suffix"] = np.mean([live_q * w.d * 2 + rows_q * (w.d * 4 + 4) +
                                           live_kv * k * 2 * w.d * 2 + rows_q * (w.d * 2 + 4)
                                           for k in kk])
        # suffix backward: q, dO, lse, D of the live rows, the fp32 dQ accumulator read and dq
        # written, the diagonal K/V rows read and all dK/dV rows of blocks 1..k written
        alg_bytes["bwd_suffix"] = np.mean([2 * live_q * w.d * 2 + 2 * live_q * 4 + rows_q * w.d * 4 +
                                           rows_q * w.d * 2 + live_kv * k * 2 * w.d * 2 +
                                           w.B * w.Hkv * k * w.L * 2 * w.d * 2 for k in kk])
        # whole TTT, one launch: the same rows for every step k >= 1, the diagonal K/V rows of
        # every block t = 1..K-1 read once and its dK/dV rows written once
        alg_bytes["bwd_suffix_sweep"] = (
            len(kk) * (2 * live_q * w.d * 2 + 2 * live_q * 4 + rows_q * w.d * 4 + rows_q * w.d * 2) +
            max(kk) * (live_kv * 2 * w.d * 2 + w.B * w.Hkv * w.L * 2 * w.d * 2))
    # stored-dS dQ kernel: the 2 KB dS blocks it reads (key block kb <= query block qb, 32 kb <
    # T), K of block 0 once per KV group, dQ written (fp32 accumulator for k >= 1, bf16 at k = 0)
    blocks = w.Hq * sum(min(qb + 1, -(-int(t) // 32)) for t in T for qb in range(L32))
    alg_bytes["bwd_dq_ds"] = np.mean([blocks * 2048 + w.B * w.Hkv * w.L * w.d * 2 +
                                      rows_q * w.d * (4 if k else 2) for k in steps])
    # row dot: o and dO read, D and lse * log2(e) written (lse read)
    alg_bytes["bwd_rowdot"] = rows_q * (2 * w.d * 2 + 12)

    def annotate(raw, nstep):
        st = {name: {"launches": n, "avg_ms": ms / n, "total_ms_per_step": ms / nstep}
              for name, (n, ms) in raw.items()}
        for n in alg:
            if n in st:
                a = nsteps * alg[n] / (st[n]["total_ms_per_step"] / 1e3) / 1e12
                st[n]["alg_tflops"] = round(a, 1)
                st[n]["frac_mfma_peak"] = round(a / PEAK_BF16_TFLOPS, 4)
        for n, b in alg_bytes.items():
            if n in st:
                gbs = b / (st[n]["avg_ms"] / 1e3) / 1e9
                st[n].update(alg_bytes=int(b), alg_gbs=round(gbs, 1),
                             frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))
        return st

    kstats = annotate(kernels, args.steps)
    kcold = annotate(kernels_cold, args.cold_steps) if kernels_cold else None
    roofline = None
    if kstats:
        mfma = {n: s for n, s in kstats.items() if n in alg}
        dom = max(mfma, key=lambda n: mfma[n]["total_ms_per_step"])
        achieved = nsteps * alg[dom] / (mfma[dom]["total_ms_per_step"] / 1e3) / 1e12
        traffic = run_traffic(config, dom, args.sweep, args.dq_mode, args.suffix)
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
        if peaks:
            roofline["frac_of_measured_peak"] = round(achieved / peaks["mfma_bf16_tflops"], 4)

    # % roofline of the whole sweep: the time the causal flops would take at the matrix-core
    # peak, plus the suffix's marginal bytes (diagonal K/V rows read by the forward, read and
    # their dK/dV written by the backward) and the backward preprocessing (read o and dO, write
    # D) at the HBM peak, over the measured step time
    live_kv_rows = int(sum(int(t) for t in T)) * w.Hkv
    f_causal = sum(14 * w.d * causal for _ in steps)
    b_suffix = sum(3 * live_kv_rows * k * 2 * w.d * 2 for k in steps)
    b_pre = len(steps) * w.B * w.Hq * w.L * (2 * w.d * 2 + 4)
    t_roof = f_causal / (PEAK_BF16_TFLOPS * 1e12) + (b_suffix + b_pre) / (PEAK_HBM_GBS * 1e9)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "Q_LEN": w.L,
                   "T": [int(t) for t in T] if w.T_fixed is None else w.T_fixed,
                   "ttt_steps": f"k=0..{steps[-1]}", "global_batch": w.B, "seq_len": w.L,
                   "parallelism": "single GPU"},
        "dq_mode": args.dq_mode, "suffix": args.suffix,
        "api": "sweep" if args.sweep else "per-step",
        "tokens_per_s": round(tokens, 1),
        # tokens inside the sequences' lengths (sum of T over the batch), per second
        "valid_tokens_per_s": round(float(sum(int(t) for t in T)) / sec, 1),
        "pct_roofline": {"t_roof_ms": round(t_roof * 1e3, 4), "frac": round(t_roof / sec, 4),
                         "causal_flop": f_causal, "suffix_bytes": b_suffix, "preprocess_bytes": b_pre},
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "min": round(step_ms[0], 4),
                    "max": round(step_ms[-1], 4)},
        "ms_per_step_kernel_timed": None if sec_events is None else round(sec_events * 1e3, 4),
        "graph_replay": None if graph_sec is None else {
            "ms_per_step": round(graph_sec * 1e3, 4), "value": round(flops / graph_sec / 1e12, 2),
            "tokens_per_s": round(w.B * w.L / graph_sec, 1)},
        "unmasked_flop_per_step": flops,
        "roofline": roofline,
        "kernels": kstats,
        "kernels_cold_cache": kcold,
        "setup_s": round(setup_s, 1),
    }
    return out


def bench_loss(args):
    """One step = one in-place loss-gradient call over the whole [N, V] logits of a TTT step.
    value = algorithmic HBM bytes (read z and p, write z; read g, write the loss) / time."""
    import torch
    from masked_attention_eagle_amd import inputs
    from masked_attention_eagle_amd import ttt_attn as A
    name = "llama3.1-8b-draft-lmhead N8192 V32000"
    N, V = inputs.LOSS_WORKLOADS[name]
    A.load()
    z, p, g = inputs.loss_case_device(11, N, V, "bf16")
    loss = torch.empty((N,), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        A.loss_grad_inplace(z, p, g, loss)
    torch.cuda.synchronize()
    timing = not args.no_kernel_timing
    if timing:
        A.timing_reset()
        A.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        A.loss_grad_inplace(z, p, g, loss)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    kernels = {}
    if timing:
        A.timing_enable(False)
        kernels = A.timing_read()
    alg = 3 * N * V * 2 + 2 * N * 4
    roofline = None
    if "loss_grad" in kernels:
        n, ms = kernels["loss_grad"]
        avg = ms / n / 1e3
        gbs = alg / avg / 1e9
        roofline = {"kernel": "loss_grad", "bound": "hbm", "achieved": round(gbs, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic_loss("loss_grad")}
    out = {"metric": "in-place masked softmax-loss gradient, algorithmic HBM GB/s", "value": round(alg / sec / 1e9, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": name, "rows": N, "vocab": V}, "alg_bytes_per_step": alg,
           "roofline": roofline}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_loss(V)
    print(json.dumps(out))


def measured_traffic_loss(name):
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f)["lmhead"]["kernels"][name]
    except (OSError, KeyError, ValueError):
        return None
    if source_digest(("kernels_loss.hip", "common.cuh")) != entry.get("code_digest"):
        return None
    return int(entry["bytes_per_launch"])


def cpu_baseline_loss(V):
    """The fp64 oracle on 1024 rows of the same shape, in the same unit (GB/s of the kernel's
    algorithmic bytes for those rows)."""
    from masked_attention_eagle_amd import inputs
    from oracle import loss_oracle as LO
    rows = 1024
    z, p, g = inputs.loss_case(11, rows, V, "bf16")
    t0 = time.perf_counter()
    LO.loss_and_grad(z, p, g)
    sec = time.perf_counter() - t0
    host = host_cores()
    return {"value": round((3 * rows * V * 2 + 2 * rows * 4) / sec / 1e9, 4), "unit": "GB/s",
            "cores": host["threads"], "kind": "oracle", "host": host, "seconds": round(sec, 3),
            "sample": f"loss and gradient of {rows} rows x {V} columns"}


CPU_SAMPLE_SECONDS = 25.0


def host_cores() -> dict:
    """The host side of the CPU baseline: cores this process may run on (its affinity), the
    machine's logical CPU count, the BLAS threads the oracle's matrix products use (the cores
    actually used), and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [affinity])
    except Exception:
        threads = affinity
    return {"affinity_cores": affinity, "logical_cpus": os.cpu_count(), "threads": threads,
            "cpu_model": model}


def cpu_baseline(w, T, steps):
    """The CPU oracle (fp64 NumPy, dense masked) on a bounded sample of the same workload:
    forward + backward of one KV group (all of its query heads) of sequence 0 at TTT steps
    0, 1, 2, ... in order, stopping after the step during which the elapsed time passes
    CPU_SAMPLE_SECONDS.  Reported in the same unit (unmasked TFLOP/s over the sample's own
    pairs)."""
    from masked_attention_eagle_amd import inputs
    from oracle import ttt_oracle as O
    G = w.Hq // w.Hkv
    host = host_cores()
    sec, flops, done, ks, vs = 0.0, 0, [], [], []
    for k in steps:
        q = inputs.q_at(w, k)[0:1, 0:G]
        kb, vb = inputs.kv_block(w, k)  # block k of the cache, KV group 0 of sequence 0
        ks.append(kb[0:1, 0:1])
        vs.append(vb[0:1, 0:1])
        kk, vv = np.concatenate(ks, axis=2), np.concatenate(vs, axis=2)
        do = inputs.do_at(w, k)[0:1, 0:G]
        t0 = time.perf_counter()
        o, _ = O.forward(q, kk, vv, T[0:1], w.scale)
        O.backward(q, kk, vv, T[0:1], w.scale, do, o)
        sec += time.perf_counter() - t0
        flops += 14 * w.d * total_pairs(w.L, k, int(T[0])) * G
        done.append(k)
        if sec > CPU_SAMPLE_SECONDS:
            break
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": host["threads"],
            "kind": "oracle", "host": host, "seconds": round(sec, 2),
            "sample": f"fwd+bwd of KV group 0 ({G} query heads) of sequence 0 at TTT steps "
                      f"{done[0]}..{done[-1]}"}


if __name__ == "__main__":
    main()

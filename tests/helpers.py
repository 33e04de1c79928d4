"""Shared helpers of the GPU parity tests: device transfer, the HIP calls, and the tolerance checks.

Tolerances (max-abs for o and lse, normalised max error max|d|/max|ref| for gradients):
  fp32 tiny workload : 1e-5 max-abs on every output;
  other fp32 shapes  : 1e-5 * max(1, max|ref|) per output (fp32 sums of up to a few hundred
                       terms of magnitude ~|ref| carry a relative error of a few 1e-7);
  bf16 workloads     : o 1e-2, lse 1e-3, dq/dk/dv 2e-2 normalised.
The o bound holds where bf16 can hold it: from |o| = 4 on, half a bf16 step (2^-6 at [4, 8))
alone exceeds 1e-2, so there an element may be off by that half step plus one bf16 rounding of
P (2^-9 |o|) (o_bound).
Set TTT_ERRLOG to a file path to append every measured error as a JSON line.
"""
import json
import os

import numpy as np

TOL_F32 = 1e-5
TOL_O, TOL_LSE, TOL_GRAD = 1e-2, 1e-3, 2e-2


def to_dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=dtype).contiguous()


def to_np(t):
    import torch
    return t.detach().to(dtype=torch.float64).cpu().numpy()


def gpu_fwd_bwd(lib, q, k, v, do, T, scale, dtype_name, with_bwd=True, dq_mode="stored",
                suffix="fused"):
    import torch
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    Td = torch.as_tensor(np.asarray(T, dtype=np.int32), device="cuda")
    o, lse = lib.ttt_attn_fwd(qd, kd, vd, Td, scale, suffix=suffix)
    out = {"o": to_np(o), "lse": to_np(lse)}
    if with_bwd:
        dq, dk, dv = lib.ttt_attn_bwd(qd, kd, vd, Td, o, lse, dod, scale, dq_mode=dq_mode,
                                      suffix=suffix)
        out.update(dq=to_np(dq), dk=to_np(dk), dv=to_np(dv))
    torch.cuda.synchronize()
    return out


def o_bound(ref, o_tol=TOL_O):
    """Per-element bound on |o - ref| for a bf16 o: o_tol, or from |ref| = 4 on (where half a
    bf16 step, 2^(e-8) at [2^e, 2^(e+1)), passes 1e-2) that half step plus 2^-9 |ref|."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    half_step = np.exp2(np.floor(np.log2(np.maximum(a, 1e-30))) - 8)
    return np.where(a >= 4.0, np.maximum(o_tol, half_step + a * 2.0 ** -9), o_tol)


def _lse_err(got, ref):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "empty-row lse must be -inf on both sides"
    return float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0


def errors(got, ref):
    d = np.abs(got["o"] - ref["o"])
    e = {"o": float(d.max()) if d.size else 0.0,
         # largest error of an element with |ref| < 4, and largest error / bound over all
         "o_small": float(d[np.abs(ref["o"]) < 4.0].max()) if (np.abs(ref["o"]) < 4.0).any() else 0.0,
         "lse": _lse_err(got["lse"], ref["lse"])}
    e["o_ratio"] = float((d / o_bound(ref["o"])).max()) if d.size else 0.0
    for name in ("dq", "dk", "dv"):
        if name in got and name in ref:
            den = np.abs(ref[name]).max()
            diff = np.abs(got[name] - ref[name]).max()
            e[name + "_abs"] = float(diff)
            e[name] = float(diff / den) if den > 0 else float(diff)
    return e


def check(got, ref, dtype_name, label="", f32_relative=False, o_tol=TOL_O):
    e = errors(got, ref)
    log = os.environ.get("TTT_ERRLOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": label, "dtype": dtype_name, **e}) + "\n")
    if dtype_name == "f32":
        for name in ("o", "lse", "dq_abs", "dk_abs", "dv_abs"):
            if name in e:
                key = name.replace("_abs", "")
                tol = TOL_F32
                if f32_relative and key in ref:
                    fin = ref[key][np.isfinite(ref[key])]
                    tol = TOL_F32 * max(1.0, float(np.abs(fin).max()) if fin.size else 1.0)
                assert e[name] <= tol, f"{label} {name} max-abs error {e[name]:.3g} > {tol:.3g}"
    else:
        d = np.abs(got["o"] - ref["o"])
        bound = o_bound(ref["o"], o_tol)
        worst = np.unravel_index(int(np.argmax(d - bound)), d.shape) if d.size else None
        assert not d.size or (d <= bound).all(), (
            f"{label} o error {d[worst]:.4g} at {worst} (|ref| {abs(float(ref['o'][worst])):.4g}) "
            f"exceeds its bound {bound[worst]:.4g}")
        assert e["lse"] <= TOL_LSE, f"{label} lse max-abs error {e['lse']:.4g}"
        for name in ("dq", "dk", "dv"):
            if name in e:
                assert e[name] <= TOL_GRAD, f"{label} {name} normalised error {e[name]:.4g}"
    return e

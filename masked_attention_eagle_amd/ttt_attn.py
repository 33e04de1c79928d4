"""Python binding of the C ABI in ``include/ttt_attn.h`` and ``include/ttt_loss.h`` (ctypes;
argument marshalling only).

Every step of the computation runs in the HIP library ``libttt_attn.so``; this module only
checks tensor metadata, allocates outputs and workspace with torch, and passes pointers and
the current HIP stream.  There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttt_attn.so")

TTT_DTYPE_F32 = 0
TTT_DTYPE_BF16 = 1
TTT_FLAG_SEPARATE_SUFFIX = 1
TTT_FLAG_RECOMPUTE_DQ = 2
TTT_FLAG_DENSE_DIAGONAL = 4
TTT_FLAG_FUSED_SUFFIX_BWD = 8
SUFFIX_PATHS = {"fused": 0, "separate": TTT_FLAG_SEPARATE_SUFFIX, "dense": TTT_FLAG_DENSE_DIAGONAL}
# backward paths: "stored" (dS handed from the dK/dV kernel to the dQ kernel, suffix kernel for
# the diagonal keys), "recompute" (the dQ kernel recomputes S and dP), "fused-suffix" (stored dS,
# and the dK/dV kernel also takes the diagonal keys' rows; no suffix kernel)
DQ_MODES = {"stored": 0, "recompute": TTT_FLAG_RECOMPUTE_DQ, "fused-suffix": TTT_FLAG_FUSED_SUFFIX_BWD}

STATUS = {
    0: "TTT_OK", -1: "TTT_E_NULL", -2: "TTT_E_SHAPE", -3: "TTT_E_UNSUPPORTED",
    -4: "TTT_E_ALIGN", -5: "TTT_E_WORKSPACE", -6: "TTT_E_HIP", -7: "TTT_E_SCRATCH",
}

# Every symbol the header declares.
EXPORTS = (
    "ttt_attn_fwd_workspace_size", "ttt_attn_bwd_workspace_size", "ttt_attn_fwd", "ttt_attn_bwd",
    "ttt_attn_fwd_sweep_workspace_size", "ttt_attn_bwd_sweep_workspace_size",
    "ttt_attn_fwd_sweep", "ttt_attn_bwd_sweep",
    "ttt_attn_status_string", "ttt_attn_version", "ttt_attn_timing_enable",
    "ttt_attn_timing_read", "ttt_attn_timing_reset", "ttt_attn_timing_flush",
    "ttt_attn_bwd_noalloc",
)
LOSS_EXPORTS = ("ttt_loss_grad_inplace",)
PROBE_EXPORTS = ("ttt_probe_mfma_bf16", "ttt_probe_copy")


class TTTError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(f"{STATUS.get(code, code)}: {text}")
        self.code = code


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("q_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ttt_step", ctypes.c_int32),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
    ]


class LossParams(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m masked_attention_eagle_amd.build`")
    # torch's ROCm wheel carries its own HIP runtime.  Loaded first, that runtime is the one the
    # library's libamdhip64 dependency binds to; loaded later, the process would hold two HIP
    # runtimes, and the streams and memory torch hands over would be foreign to the library's.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Params)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.ttt_attn_fwd_workspace_size.argtypes = [P]
    lib.ttt_attn_fwd_workspace_size.restype = sz
    lib.ttt_attn_bwd_workspace_size.argtypes = [P]
    lib.ttt_attn_bwd_workspace_size.restype = sz
    lib.ttt_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ttt_attn_fwd.restype = ctypes.c_int
    lib.ttt_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ttt_attn_bwd.restype = ctypes.c_int
    lib.ttt_attn_fwd_sweep_workspace_size.argtypes = [P]
    lib.ttt_attn_fwd_sweep_workspace_size.restype = sz
    lib.ttt_attn_bwd_sweep_workspace_size.argtypes = [P]
    lib.ttt_attn_bwd_sweep_workspace_size.restype = sz
    lib.ttt_attn_fwd_sweep.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ttt_attn_fwd_sweep.restype = ctypes.c_int
    lib.ttt_attn_bwd_sweep.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ttt_attn_bwd_sweep.restype = ctypes.c_int
    lib.ttt_attn_status_string.argtypes = [ctypes.c_int]
    lib.ttt_attn_status_string.restype = ctypes.c_char_p
    lib.ttt_attn_version.argtypes = []
    lib.ttt_attn_version.restype = ctypes.c_int
    lib.ttt_attn_timing_enable.argtypes = [ctypes.c_int]
    lib.ttt_attn_timing_enable.restype = ctypes.c_int
    lib.ttt_attn_timing_read.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int]
    lib.ttt_attn_timing_read.restype = ctypes.c_int
    lib.ttt_attn_timing_reset.argtypes = []
    lib.ttt_attn_timing_reset.restype = None
    lib.ttt_attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ttt_attn_bwd_noalloc.restype = ctypes.c_int
    lib.ttt_attn_timing_flush.argtypes = [vp, sz]
    lib.ttt_attn_timing_flush.restype = ctypes.c_int
    lib.ttt_probe_mfma_bf16.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
    lib.ttt_probe_mfma_bf16.restype = ctypes.c_int
    lib.ttt_probe_copy.argtypes = [vp, vp, sz, vp]
    lib.ttt_probe_copy.restype = ctypes.c_int
    lib.ttt_loss_grad_inplace.argtypes = [ctypes.POINTER(LossParams), vp, vp, vp, vp, vp]
    lib.ttt_loss_grad_inplace.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().ttt_attn_status_string(code).decode()


def _check(code: int) -> None:
    if code != 0:
        raise TTTError(code, status_string(code))


def make_params(B: int, Hq: int, Hkv: int, L: int, d: int, step: int, scale: float, dtype: int,
                flags: int = 0) -> Params:
    return Params(B, Hq, Hkv, L, d, step, float(scale), dtype, flags)


def path_flags(suffix: str = "fused", dq_mode: str = "stored") -> int:
    """ttt_attn_params.flags for a forward suffix path ("fused" | "separate" | "dense") and a backward
    dQ mode ("stored": dS handed from the dK/dV kernel to the dQ kernel | "recompute" |
    "fused-suffix": stored dS with the diagonal keys taken by the dK/dV kernel)."""
    if suffix not in SUFFIX_PATHS:
        raise ValueError(f"suffix must be one of {sorted(SUFFIX_PATHS)}, not {suffix!r}")
    if dq_mode not in DQ_MODES:
        raise ValueError(f"dq_mode must be one of {sorted(DQ_MODES)}, not {dq_mode!r}")
    return SUFFIX_PATHS[suffix] | DQ_MODES[dq_mode]


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return TTT_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return TTT_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _params_from(q, k, scale, flags: int = 0) -> Params:
    B, Hq, L, d = q.shape
    Bk, Hkv, KV, dk = k.shape
    if Bk != B or dk != d or KV % L != 0:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q shape {tuple(q.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return make_params(B, Hq, Hkv, L, d, KV // L - 1, scale, _dtype_code(q), flags)


def _require(t, name, dtype=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fwd_workspace_size(p: Params) -> int:
    return int(load().ttt_attn_fwd_workspace_size(ctypes.byref(p)))


def bwd_workspace_size(p: Params) -> int:
    return int(load().ttt_attn_bwd_workspace_size(ctypes.byref(p)))


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def ttt_attn_fwd(q, k, v, seq_T, scale: Optional[float] = None, out=None, lse=None,
                 workspace=None, suffix: str = "fused") -> Tuple["torch.Tensor", "torch.Tensor"]:
    """o, lse = masked attention of q [B,Hq,L,d] over k, v [B,Hkv,(step+1)L,d].

    seq_T: int32 [B] on the GPU.  The TTT step is k.shape[2] // L - 1.  suffix "fused"
    merges the diagonal keys of blocks 1..k inside the causal kernel (bf16); "separate" runs
    the standalone suffix kernel on an fp32 causal state; "dense" (measurement variant) runs
    them through the matrix cores as masked diagonal tiles.
    """
    import torch
    lib = load()
    p = _params_from(q, k, scale, path_flags(suffix))
    _require(q, "q")
    _require(k, "k", q.dtype)
    _require(v, "v", q.dtype, k.shape)
    _require(seq_T, "seq_T", torch.int32, (q.shape[0],))
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o, "out", q.dtype, q.shape)
    _require(lse_t, "lse", torch.float32, q.shape[:3])
    need = fwd_workspace_size(p)
    if need == 0 and p.dtype not in (TTT_DTYPE_F32, TTT_DTYPE_BF16):
        raise TTTError(-3, "unsupported")
    ws = _workspace(need, q.device) if workspace is None else workspace
    _check(lib.ttt_attn_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            seq_T.data_ptr(), o.data_ptr(), lse_t.data_ptr(), ws.data_ptr(),
                            ws.numel(), _stream()))
    return o, lse_t


def ttt_attn_bwd(q, k, v, seq_T, o, lse, dout, scale: Optional[float] = None, dq=None, dk=None,
                 dv=None, workspace=None, dq_mode: str = "stored", suffix: str = "fused"):
    """dq, dk, dv: gradients of sum(dout * o) for the o/lse of ttt_attn_fwd.

    dq_mode "stored": the dK/dV kernel hands dS of block 0 to the dQ kernel through the
    workspace (one matrix product per tile there); "recompute": a small workspace, and the dQ
    kernel recomputes S and dP.  suffix "dense" (measurement variant) takes the diagonal keys of
    blocks 1..k through the matrix-core kernels as masked tiles (dQ recomputed) instead of the
    suffix kernel; "fused" and "separate" give the same backward.
    """
    import torch
    lib = load()
    p = _params_from(q, k, scale, path_flags(suffix, dq_mode))
    _require(q, "q")
    _require(k, "k", q.dtype)
    _require(v, "v", q.dtype, k.shape)
    _require(seq_T, "seq_T", torch.int32, (q.shape[0],))
    _require(o, "o", q.dtype, q.shape)
    _require(lse, "lse", torch.float32, q.shape[:3])
    _require(dout, "dout", q.dtype, q.shape)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", q.dtype, q.shape)
    _require(dk, "dk", q.dtype, k.shape)
    _require(dv, "dv", q.dtype, k.shape)
    need = bwd_workspace_size(p)
    ws = _workspace(need, q.device) if workspace is None else workspace
    _check(lib.ttt_attn_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            seq_T.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                            _stream()))
    return dq, dk, dv


def ttt_attn_bwd_noalloc(q, k, v, seq_T, o, lse, dout, scale: Optional[float] = None, dq=None,
                         dk=None, dv=None):
    """The backward on the library's own scratch array (no workspace; the dQ kernel recomputes S
    and dP).  Outputs are allocated here unless given, so code that cannot allocate passes
    dq, dk, dv.  Returns (dq, dk, dv)."""
    import torch
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    p = _params_from(q, k, scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _require(t, name, like.dtype, tuple(like.shape))
    _check(lib.ttt_attn_bwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    seq_T.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    _stream()))
    return dq, dk, dv


def _sweep_params(q, k, scale, flags: int) -> Params:
    """Params of a whole-TTT sweep: q [K, B, Hq, L, d] over the cache k [B, Hkv, K*L, d]."""
    if q.dim() != 5:
        raise ValueError(f"q must be [K, B, Hq, L, d], got {tuple(q.shape)}")
    K = q.shape[0]
    if k.dim() != 4 or k.shape[2] != K * q.shape[3]:
        raise ValueError(f"k must be [B, Hkv, K*L, d] with K = {K}, got {tuple(k.shape)}")
    return _params_from(q[0], k, scale, flags)


def ttt_attn_fwd_sweep(q, k, v, seq_T, scale: Optional[float] = None, suffix: str = "fused",
                       workspace=None):
    """o [K,B,Hq,L,d], lse [K,B,Hq,L] of the K steps of a TTT unroll: step k's queries q[k]
    attend rows [0, (k+1)L) of the cache k, v [B,Hkv,K*L,d] (bf16)."""
    import torch
    lib = load()
    p = _sweep_params(q, k, scale, path_flags(suffix))
    _require(q, "q")
    _require(k, "k", q.dtype)
    _require(v, "v", q.dtype, k.shape)
    _require(seq_T, "seq_T", torch.int32, (q.shape[1],))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:4], dtype=torch.float32, device=q.device)
    need = int(lib.ttt_attn_fwd_sweep_workspace_size(ctypes.byref(p)))
    ws = _workspace(need, q.device) if workspace is None else workspace
    _check(lib.ttt_attn_fwd_sweep(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  seq_T.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream()))
    return o, lse


def ttt_attn_bwd_sweep(q, k, v, seq_T, o, lse, dout, scale: Optional[float] = None,
                       dq_mode: str = "stored", workspace=None):
    """dq [K,B,Hq,L,d] of every step and dk, dv [B,Hkv,K*L,d]: the gradient of the cache
    summed over the steps (fp32 inside, rounded once)."""
    import torch
    lib = load()
    p = _sweep_params(q, k, scale, path_flags("fused", dq_mode))
    _require(q, "q")
    _require(k, "k", q.dtype)
    _require(v, "v", q.dtype, k.shape)
    _require(seq_T, "seq_T", torch.int32, (q.shape[1],))
    _require(o, "o", q.dtype, q.shape)
    _require(lse, "lse", torch.float32, q.shape[:4])
    _require(dout, "dout", q.dtype, q.shape)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = int(lib.ttt_attn_bwd_sweep_workspace_size(ctypes.byref(p)))
    ws = _workspace(need, q.device) if workspace is None else workspace
    _check(lib.ttt_attn_bwd_sweep(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  seq_T.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream()))
    return dq, dk, dv


def timing_enable(on: bool) -> bool:
    return bool(load().ttt_attn_timing_enable(1 if on else 0))


def timing_reset() -> None:
    load().ttt_attn_timing_reset()


def timing_flush(buf) -> None:
    """With timing enabled, overwrite the uint8 device tensor `buf` before every timed launch
    (cold caches for each kernel); None turns it off."""
    if buf is None:
        _check(load().ttt_attn_timing_flush(None, 0))
    else:
        _check(load().ttt_attn_timing_flush(buf.data_ptr(), buf.numel() * buf.element_size()))


def probe_mfma_bf16(sink, workgroups: int, iters: int) -> None:
    """Enqueue the bf16 matrix-core probe (flops = workgroups * 4 * iters * 8 * 32768) on the
    current stream; sink is an fp32 device tensor of at least workgroups * 256 elements."""
    if sink.dtype.itemsize != 4 or sink.numel() < workgroups * 256 or not sink.is_cuda:
        raise ValueError("sink: fp32 device tensor of workgroups * 256 elements")
    _check(load().ttt_probe_mfma_bf16(sink.data_ptr(), workgroups, iters, _stream()))


def probe_copy(src, dst) -> None:
    """Enqueue the stream-copy probe dst <- src (same byte size, device tensors) on the current
    stream; moves 2 * nbytes."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (src.is_cuda and dst.is_cuda):
        raise ValueError("src and dst: device tensors of the same byte size")
    _check(load().ttt_probe_copy(src.data_ptr(), dst.data_ptr(), n, _stream()))


def timing_read() -> dict:
    """{kernel name: (launches, total ms)} accumulated since the last reset."""
    arr = (KernelTime * 64)()
    n = load().ttt_attn_timing_read(arr, 64)
    if n < 0:
        raise TTTError(n, status_string(n))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


def _autograd_fn():
    import torch

    class TTTAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, seq_T, scale):
            o, lse = ttt_attn_fwd(q, k, v, seq_T, scale)
            ctx.save_for_backward(q, k, v, seq_T, o, lse)
            ctx.scale = scale
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, seq_T, o, lse = ctx.saved_tensors
            dq, dk, dv = ttt_attn_bwd(q, k, v, seq_T, o, lse, do.contiguous(), ctx.scale)
            return dq, dk, dv, None, None

    return TTTAttentionFn


def ttt_attention(q, k, v, seq_T, scale: Optional[float] = None):
    """Autograd-aware wrapper: returns o; backward runs ttt_attn_bwd."""
    return _autograd_fn().apply(q, k, v, seq_T, scale)


fwd = ttt_attn_fwd
bwd = ttt_attn_bwd


def loss_grad_inplace(z, target, g, loss=None, want_loss: bool = True):
    """In-place masked softmax-loss gradient (``ttt_loss_grad_inplace``): z [N, V] logits are
    overwritten with -(p g - softmax(z) s), s = g sum(p); returns the per-row loss [N] fp32
    (or None when ``want_loss`` is False and no ``loss`` tensor is given)."""
    import torch
    _require(z, "z")
    N, V = z.shape
    _require(target, "target", z.dtype, (N, V))
    _require(g, "g", torch.float32, (N,))
    if loss is None and want_loss:
        loss = torch.empty((N,), dtype=torch.float32, device=z.device)
    if loss is not None:
        _require(loss, "loss", torch.float32, (N,))
    p = LossParams(N, V, _dtype_code(z))
    _check(load().ttt_loss_grad_inplace(ctypes.byref(p), z.data_ptr(), target.data_ptr(), g.data_ptr(),
                                        loss.data_ptr() if loss is not None else None, _stream()))
    return loss

"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds workload shapes and random-number recipes only: none of the
attention arithmetic lives here, so both the HIP path and the CPU oracle can
consume the same arrays without sharing any of the method's code.

Recipe (one NumPy ``default_rng(SeedSequence([config, index, slot]))`` stream per
tensor):
  * K block t (rows [t*L, (t+1)*L) of the stacked KV): ``[cfg, t, 1]``;
    V block t: ``[cfg, t, 2]``.  Blocks are generated once per t, so the KV
    tensor at TTT step k is the concatenation of blocks 0..k (an append-only
    cache, as the TTT unroll produces it).
  * q at step k: ``[cfg, k, 0]``; dO at step k: ``[cfg, k, 3]``.
  * per-sequence valid lengths of the padding-heavy workload:
    ``[cfg, 99, 4]``, integers uniform on [256, 2048] inclusive.
  * values are N(0, 1) in fp32, rounded to nearest-even bf16 for bf16 workloads.

Inputs of the in-place masked softmax-loss gradient (``loss_case``), one stream
``[seed, 200, slot]`` per tensor: logits z = 2 * N(0, 1) (slot 0); target
distribution p = a row of E**6 draws (E standard exponential) divided by its sum
(a peaked distribution: a few columns carry most of the mass, slot 1); per-row upstream weight g = mask / (number
of unmasked rows) with 10% of the rows masked (slot 2).  z and p are rounded to
bf16 for bf16 cases.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    steps: tuple
    dtype: str  # "f32" or "bf16"
    T_fixed: int | None  # None: drawn per sequence from the seed

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def kv_len(self, step: int) -> int:
        return (step + 1) * self.L


WORKLOADS = {
    1: Workload(1, "tiny-fp32 B1 Hq2 Hkv1 d64 L128 T100", 1, 2, 1, 64, 128, (0, 1, 2), "f32", 100),
    2: Workload(2, "llama3.1-8b-draft B2 Hq32 Hkv8 d128 L4096 T4096", 2, 32, 8, 128, 4096,
                tuple(range(7)), "bf16", 4096),
    3: Workload(3, "padding-heavy B8 Hq32 Hkv8 d128 L2048 T~U[256,2048]", 8, 32, 8, 128, 2048,
                tuple(range(7)), "bf16", None),
    4: Workload(4, "llama3.3-70b-draft B1 Hq64 Hkv8 d128 L4096 T4096", 1, 64, 8, 128, 4096,
                tuple(range(7)), "bf16", 4096),
    5: Workload(5, "qwen3-30b-a3b-draft-long-ttt B1 Hq32 Hkv4 d128 L4096 T3500", 1, 32, 4, 128, 4096,
                tuple(range(13)), "bf16", 3500),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); result kept in fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _normal(seed: List[int], shape, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def seq_lengths(w: Workload) -> np.ndarray:
    if w.T_fixed is not None:
        return np.full((w.B,), w.T_fixed, dtype=np.int32)
    rng = np.random.default_rng(np.random.SeedSequence([w.cfg, 99, 4]))
    return rng.integers(256, 2049, size=w.B).astype(np.int32)


def kv_block(w: Workload, t: int):
    shape = (w.B, w.Hkv, w.L, w.d)
    return _normal([w.cfg, t, 1], shape, w.dtype), _normal([w.cfg, t, 2], shape, w.dtype)


def kv_stack(w: Workload, step: int):
    ks, vs = zip(*(kv_block(w, t) for t in range(step + 1)))
    return np.concatenate(ks, axis=2), np.concatenate(vs, axis=2)


def q_at(w: Workload, step: int) -> np.ndarray:
    return _normal([w.cfg, step, 0], (w.B, w.Hq, w.L, w.d), w.dtype)


def do_at(w: Workload, step: int) -> np.ndarray:
    return _normal([w.cfg, step, 3], (w.B, w.Hq, w.L, w.d), w.dtype)


def make_case(seed: int, B: int, Hq: int, Hkv: int, d: int, L: int, step: int, T, dtype: str,
              q_mult: float = 1.0):
    """Free-form case for tests: returns q, k, v, do (fp32 arrays) and T (int32 [B]).

    ``q_mult`` scales q before rounding (a "peaky" variant that stresses the
    online-softmax rescaling).
    """
    T = np.broadcast_to(np.asarray(T, dtype=np.int32), (B,)).copy()
    q = _normal([seed, step, 10], (B, Hq, L, d), "f32") * np.float32(q_mult)
    q = round_to_bf16(q) if dtype == "bf16" else q
    k = _normal([seed, step, 11], (B, Hkv, (step + 1) * L, d), dtype)
    v = _normal([seed, step, 12], (B, Hkv, (step + 1) * L, d), dtype)
    do = _normal([seed, step, 13], (B, Hq, L, d), dtype)
    return q, k, v, do, T


# Loss-gradient workload: the draft LM head of one TTT step of the Llama-3.1-8B-shaped
# layer (B * Q_LEN = 2 * 4096 tokens) over a 32,000-entry draft vocabulary.
LOSS_WORKLOADS = {
    "llama3.1-8b-draft-lmhead N8192 V32000": (8192, 32000),
}


def loss_case(seed: int, N: int, V: int, dtype: str, mask_frac: float = 0.1):
    """z [N, V], p [N, V] (fp32 arrays, bf16-rounded for bf16) and g [N] fp32."""
    z = _normal([seed, 200, 0], (N, V), "f32") * np.float32(2.0)
    rng = np.random.default_rng(np.random.SeedSequence([seed, 200, 1]))
    p = np.empty((N, V), dtype=np.float32)
    for r0 in range(0, N, 256):  # row chunks bound the fp64 temporaries (same stream)
        r1 = min(N, r0 + 256)
        w = rng.standard_exponential(size=(r1 - r0, V), dtype=np.float32) ** 6
        p[r0:r1] = w / w.sum(axis=1, keepdims=True, dtype=np.float64)
    rng = np.random.default_rng(np.random.SeedSequence([seed, 200, 2]))
    keep = rng.uniform(size=N) >= mask_frac
    keep[0] = True
    if N > 1:
        keep[-1] = False
    g = (keep / keep.sum()).astype(np.float32)
    if dtype == "bf16":
        z, p = round_to_bf16(z), round_to_bf16(p)
    return z, p, g


def loss_case_device(seed: int, N: int, V: int, dtype: str, device="cuda", mask_frac: float = 0.1):
    """The loss_case recipe drawn with torch's seeded generator on the device (for the full-size
    workload, where the host draws take tens of seconds).  Returns torch tensors z, p (dtype)
    and g (fp32); tests copy the rows they check to the host before the in-place call."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 200)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    z = (2.0 * torch.randn((N, V), generator=gen, device=device)).to(dt)
    p = torch.empty((N, V), dtype=dt, device=device)
    for r0 in range(0, N, 1024):
        r1 = min(N, r0 + 1024)
        w = torch.empty((r1 - r0, V), device=device).exponential_(generator=gen) ** 6
        p[r0:r1] = (w / w.sum(dim=1, keepdim=True, dtype=torch.float64).float()).to(dt)
    keep = torch.rand((N,), generator=gen, device=device) >= mask_frac
    keep[0] = True
    if N > 1:
        keep[-1] = False
    g = (keep.float() / keep.sum().float()).contiguous()
    return z.contiguous(), p.contiguous(), g

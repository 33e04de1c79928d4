"""The four bf16 draft-layer workloads at full size, through the C ABI in the same launch
configuration the benchmark times.

* one KV group (all of its query heads) per sequence is compared element by element with the
  oracle (a whole group is needed: dK/dV sum over its heads): the group is chosen from the seed,
  for one sequence chosen from the seed, or for every sequence of the padding-heavy workload
  (each of its eight sequences has its own valid length);
* over every group: sum_j dK[b,g,j] = 0 (rows of dS sum to zero) and sum_j dV[b,g,j] =
  sum of dO over the group's non-empty query rows (rows of P sum to one), to fp32 rounding
  relative to sum|dK| and sum|dV|;
* block-0 key rows >= T and suffix rows t*Q_LEN + i with i >= T get exactly zero gradient;
* the backward pass is bitwise reproducible.
"""
import numpy as np
import pytest

from masked_attention_eagle_amd import inputs
from oracle import ttt_oracle as O
from tests.helpers import check, to_dev, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CASES = [(2, 0), (2, 3), (2, 6), (3, 0), (3, 6), (4, 0), (4, 6), (5, 3), (5, 12)]


def _run(lib, w, step, dq_mode="stored", suffix="fused"):
    import torch
    q = inputs.q_at(w, step)
    k, v = inputs.kv_stack(w, step)
    do = inputs.do_at(w, step)
    T = inputs.seq_lengths(w)
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    Td = torch.as_tensor(T, device="cuda")
    o, lse = lib.ttt_attn_fwd(qd, kd, vd, Td, w.scale, suffix=suffix)
    dq, dk, dv = lib.ttt_attn_bwd(qd, kd, vd, Td, o, lse, dod, w.scale, dq_mode=dq_mode)
    torch.cuda.synchronize()
    return (q, k, v, do, T), (qd, kd, vd, dod, Td), (o, lse, dq, dk, dv)


# The default path merges the suffix inside the causal forward kernel and hands dS from the
# dK/dV kernel to the dQ kernel; the extra cases run the backward whose dQ kernel recomputes
# S and dP (small workspace), the forward's standalone suffix kernel, and the backward whose
# dK/dV kernel also takes the diagonal keys' rows (heads split over workgroups at the 70B shape).
@pytest.mark.parametrize("cfg,step,dq_mode,suffix", [c + ("stored", "fused") for c in CASES] +
                         [(2, 6, "recompute", "fused"), (3, 6, "recompute", "fused"),
                          (2, 6, "stored", "separate"), (5, 12, "stored", "separate"),
                          (2, 6, "fused-suffix", "fused"), (3, 6, "fused-suffix", "fused"),
                          (4, 6, "fused-suffix", "fused"), (5, 12, "fused-suffix", "fused")])
def test_workload_sampled_group_and_properties(gpu_lib, cfg, step, dq_mode, suffix):
    import torch
    w = inputs.WORKLOADS[cfg]
    print(f"workload {w.name} step {step} dq {dq_mode} suffix {suffix}", flush=True)
    (q, k, v, do, T), dev, (o, lse, dq, dk, dv) = _run(gpu_lib, w, step, dq_mode, suffix)
    G, L = w.Hq // w.Hkv, w.L

    # properties over every KV group (fp64 on the GPU)
    dk64, dv64, do64 = dk.double(), dv.double(), dev[3].double()
    colsum_k = dk64.sum(dim=2)
    scale_k = dk64.abs().sum(dim=2)
    assert float((colsum_k.abs() / scale_k.clamp_min(1e-30)).max()) < 1e-2
    want_v = do64.view(w.B, w.Hkv, G, L, w.d).sum(dim=(2, 3))
    want_v[torch.as_tensor(T, device="cuda") == 0] = 0
    err_v = (dv64.sum(dim=2) - want_v).abs() / dv64.abs().sum(dim=2).clamp_min(1e-30)
    assert float(err_v.max()) < 1e-2
    for b in range(w.B):
        rows = torch.arange(w.kv_len(step), device="cuda") % L >= int(T[b])
        assert not bool(dk[b][:, rows].any()) and not bool(dv[b][:, rows].any())

    # KV groups against the oracle: one per sequence for the padding-heavy workload (every
    # valid length), else one sequence
    rng = np.random.default_rng(np.random.SeedSequence([cfg, step, 77]))
    seqs = list(range(w.B)) if len(set(int(t) for t in T)) > 1 else [int(rng.integers(w.B))]
    for b in seqs:
        g = int(rng.integers(w.Hkv))
        hs = slice(g * G, (g + 1) * G)
        qs, ks, vs, dos = q[b:b + 1, hs], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], do[b:b + 1, hs]
        ro, rlse = O.forward(qs, ks, vs, T[b:b + 1], w.scale)
        rdq, rdk, rdv = O.backward(qs, ks, vs, T[b:b + 1], w.scale, dos, ro)
        got = dict(o=to_np(o[b:b + 1, hs]), lse=to_np(lse[b:b + 1, hs]), dq=to_np(dq[b:b + 1, hs]),
                   dk=to_np(dk[b:b + 1, g:g + 1]), dv=to_np(dv[b:b + 1, g:g + 1]))
        e = check(got, dict(o=ro, lse=rlse, dq=rdq, dk=rdk, dv=rdv), "bf16",
                  f"cfg={cfg} step={step} b={b} g={g} T={int(T[b])}")
        print("errors", b, g, int(T[b]), e, flush=True)


@pytest.mark.parametrize("cfg", [4, 3])
def test_backward_bitwise_reproducible_full_size(gpu_lib, cfg):
    """The dK/dV workgroups take their (key tile, head share) units from a queue, so which
    workgroup computes a unit changes from run to run; each unit sums in a fixed order and the
    split partials are reduced in split order, so two runs agree bit for bit.  Workload 4 splits
    the heads of a KV group over two units per key tile; the padding-heavy workload has
    sequences of different lengths, whose units differ most in size."""
    import torch
    w = inputs.WORKLOADS[cfg]
    _, (qd, kd, vd, dod, Td), (o, lse, dq, dk, dv) = _run(gpu_lib, w, 2)
    dq2, dk2, dv2 = gpu_lib.ttt_attn_bwd(qd, kd, vd, Td, o, lse, dod, w.scale)
    torch.cuda.synchronize()
    for a, c in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))

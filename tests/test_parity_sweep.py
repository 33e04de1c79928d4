"""Whole-TTT sweep (ttt_attn_fwd_sweep / ttt_attn_bwd_sweep): K steps over one KV cache.

* small shapes against the oracle: o, lse, dq of every step, and dk, dv of the cache as the
  sum over the steps of each step's oracle gradient (block t gets the diagonal gradients of
  every step k >= t, block 0 the causal gradient of all steps);
* full size (the Llama-3.1-8B-shaped layer, k = 0..6): o, lse, dq bitwise equal to the
  per-step calls on copies of the cache prefix (same kernels, same inputs), dk/dv equal to
  the sum of the per-step gradients up to their bf16 rounding.
"""
import numpy as np
import pytest

from masked_attention_eagle_amd import inputs
from oracle import ttt_oracle as O
from tests.helpers import TOL_GRAD, TOL_LSE, o_bound, to_dev, to_np

pytestmark = pytest.mark.gpu


def _sweep_case(seed, B, Hq, Hkv, d, L, K, T):
    T = np.broadcast_to(np.asarray(T, dtype=np.int32), (B,)).copy()
    q = np.stack([inputs.round_to_bf16(inputs._normal([seed, s, 20], (B, Hq, L, d), "f32"))
                  for s in range(K)])
    kc = inputs._normal([seed, 99, 21], (B, Hkv, K * L, d), "bf16")
    vc = inputs._normal([seed, 99, 22], (B, Hkv, K * L, d), "bf16")
    do = np.stack([inputs._normal([seed, s, 23], (B, Hq, L, d), "bf16") for s in range(K)])
    return q, kc, vc, do, T


def _norm_err(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


@pytest.mark.parametrize("dq_mode", ["stored", "recompute"])
@pytest.mark.parametrize("B,Hq,Hkv,L,K,T", [(2, 4, 2, 256, 4, (256, 140)), (1, 8, 2, 128, 3, 77),
                                             (2, 2, 1, 256, 2, (0, 255)),
                                             # more diagonal blocks than the suffix kernel keeps
                                             # in registers at once (6): two and three chunks
                                             (1, 4, 1, 128, 9, 100), (2, 2, 1, 128, 14, (128, 37)),
                                             # a single step: block 0 only, no suffix launch
                                             (1, 4, 2, 128, 1, 100)])
def test_sweep_against_oracle(gpu_lib, B, Hq, Hkv, L, K, T, dq_mode):
    _sweep_vs_oracle(gpu_lib, 128, B, Hq, Hkv, L, K, T, dq_mode)


# head_dim 64: the same kernels through zero-padded head_dim-128 copies of every step's rows
@pytest.mark.parametrize("dq_mode", ["stored", "recompute"])
@pytest.mark.parametrize("B,Hq,Hkv,L,K,T", [(2, 4, 2, 256, 4, (256, 140)), (1, 8, 2, 128, 3, 77)])
def test_sweep_head_dim_64_against_oracle(gpu_lib, B, Hq, Hkv, L, K, T, dq_mode):
    _sweep_vs_oracle(gpu_lib, 64, B, Hq, Hkv, L, K, T, dq_mode)


def _sweep_vs_oracle(gpu_lib, d, B, Hq, Hkv, L, K, T, dq_mode):
    import torch
    q, kc, vc, do, Tarr = _sweep_case(B * 100 + K, B, Hq, Hkv, d, L, K, T)
    print(f"sweep d={d} B={B} Hq={Hq} Hkv={Hkv} L={L} K={K} T={list(Tarr)} dq={dq_mode}", flush=True)
    bf = torch.bfloat16
    qd, kd, vd, dod = to_dev(q, bf), to_dev(kc, bf), to_dev(vc, bf), to_dev(do, bf)
    Td = torch.as_tensor(Tarr, device="cuda")
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.ttt_attn_fwd_sweep(qd, kd, vd, Td, scale)
    dq, dk, dv = gpu_lib.ttt_attn_bwd_sweep(qd, kd, vd, Td, o, lse, dod, scale, dq_mode=dq_mode)
    torch.cuda.synchronize()
    dk_ref = np.zeros(kc.shape, dtype=np.float64)
    dv_ref = np.zeros(vc.shape, dtype=np.float64)
    for s in range(K):
        n = (s + 1) * L
        ks, vs = kc[:, :, :n], vc[:, :, :n]
        ro, rlse = O.forward(q[s], ks, vs, Tarr, scale)
        rdq, rdk, rdv = O.backward(q[s], ks, vs, Tarr, scale, do[s], ro)
        dk_ref[:, :, :n] += rdk
        dv_ref[:, :, :n] += rdv
        assert (np.abs(to_np(o[s]) - ro) <= o_bound(ro)).all()
        got_lse, fin = to_np(lse[s]), np.isfinite(rlse)
        assert np.array_equal(np.isneginf(got_lse), np.isneginf(rlse))
        if fin.any():
            assert float(np.abs(got_lse[fin] - rlse[fin]).max()) <= TOL_LSE
        if np.abs(rdq).max() > 0:
            assert _norm_err(to_np(dq[s]), rdq) <= TOL_GRAD
    if np.abs(dk_ref).max() > 0:
        assert _norm_err(to_np(dk), dk_ref) <= TOL_GRAD
        assert _norm_err(to_np(dv), dv_ref) <= TOL_GRAD
    else:
        assert not bool(dk.any()) and not bool(dv.any())


@pytest.mark.slow
def test_sweep_matches_per_step_calls_full_size(gpu_lib):
    import torch
    w = inputs.WORKLOADS[2]
    K = len(w.steps)
    T = inputs.seq_lengths(w)
    bf = torch.bfloat16
    blocks = [inputs.kv_block(w, t) for t in range(K)]
    kc = torch.cat([torch.from_numpy(b[0]) for b in blocks], 2).to("cuda", bf)
    vc = torch.cat([torch.from_numpy(b[1]) for b in blocks], 2).to("cuda", bf)
    del blocks
    qd = torch.stack([torch.from_numpy(inputs.q_at(w, s)) for s in w.steps]).to("cuda", bf)
    dod = torch.stack([torch.from_numpy(inputs.do_at(w, s)) for s in w.steps]).to("cuda", bf)
    Td = torch.as_tensor(T, device="cuda")
    o, lse = gpu_lib.ttt_attn_fwd_sweep(qd, kc, vc, Td, w.scale)
    dq, dk, dv = gpu_lib.ttt_attn_bwd_sweep(qd, kc, vc, Td, o, lse, dod, w.scale)
    dk_sum = torch.zeros(kc.shape, dtype=torch.float32, device="cuda")
    dv_sum = torch.zeros_like(dk_sum)
    step_max = {"k": 0.0, "v": 0.0}  # sum over the steps of max|per-step gradient|
    L = w.L
    for s in w.steps:
        n = (s + 1) * L
        ks, vs = kc[:, :, :n].contiguous(), vc[:, :, :n].contiguous()
        os_, ls = gpu_lib.ttt_attn_fwd(qd[s], ks, vs, Td, w.scale)
        assert torch.equal(os_.view(torch.int16), o[s].view(torch.int16))
        assert torch.equal(ls, lse[s])
        dqs, dks, dvs = gpu_lib.ttt_attn_bwd(qd[s], ks, vs, Td, o[s], lse[s], dod[s], w.scale)
        assert torch.equal(dqs.view(torch.int16), dq[s].view(torch.int16))
        dk_sum[:, :, :n] += dks.float()
        dv_sum[:, :, :n] += dvs.float()
        step_max["k"] += float(dks.float().abs().max())
        step_max["v"] += float(dvs.float().abs().max())
        del ks, vs, dqs, dks, dvs, os_, ls
    torch.cuda.synchronize()
    # The per-step outputs are each rounded to bf16 (relative 2^-9) before being summed here;
    # the sweep rounds its fp32 sum once.  Besides fp32 summation order, the difference is
    # bounded by 2^-9 * (sum_k max|step k| + max|sum|), taken with a factor 2 of margin for
    # the fp32 sums inside the kernels.
    for name, got, ref in (("k", dk, dk_sum), ("v", dv, dv_sum)):
        err = float((got.float() - ref).abs().max())
        bound = 2 * 2 ** -9 * (step_max[name] + float(ref.abs().max()))
        print(f"sweep d{name} vs per-step sum: max-abs {err:.3g}, bound {bound:.3g}", flush=True)
        assert err <= bound

"""In-place masked softmax-loss gradient on the GPU (through the C ABI) against the fp64 oracle.

Tolerances, from the arithmetic: the kernel works in fp32 on the exact input values, so the
softmax statistics carry a relative error of order 1e-6; the gradient is then rounded once to
the storage type.  Per element: |got - ref| <= 2^-8 |ref| + 1e-5 max_row|ref| for bf16 (the
rounding is at most 2^-9 |ref|), 1e-5 (|ref| + max_row|ref|) for fp32.  The per-row loss is an
fp32 sum of V terms: |got - ref| <= 1e-5 (sum_i |p_i z_i| + |lse| sum_i p_i) + 1e-6.
"""
import numpy as np
import pytest

from masked_attention_eagle_amd import inputs
from oracle import loss_oracle as LO

pytestmark = pytest.mark.gpu


def _run(lib, z, p, g, dtype):
    import torch
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    zd = torch.from_numpy(z).to("cuda", dt).contiguous()
    pd = torch.from_numpy(p).to("cuda", dt).contiguous()
    gd = torch.from_numpy(g).to("cuda", torch.float32)
    loss = lib.loss_grad_inplace(zd, pd, gd)
    torch.cuda.synchronize()
    return zd, loss


def _check(z, p, g, got_grad, got_loss, dtype, label):
    ref_loss, ref = LO.loss_and_grad(z, p, g)
    rowmax = np.abs(ref).max(axis=1, keepdims=True)
    if dtype == "bf16":
        tol = 2.0 ** -8 * np.abs(ref) + 1e-5 * rowmax
    else:
        tol = 1e-5 * (np.abs(ref) + rowmax)
    err = np.abs(got_grad - ref)
    bad = err > tol
    assert not bad.any(), f"{label}: gradient off at {np.argwhere(bad)[:3]}, max err {err.max():.3g}"
    z64, p64 = z.astype(np.float64), p.astype(np.float64)
    m = z64.max(axis=1)
    lse = m + np.log(np.exp(z64 - m[:, None]).sum(axis=1))
    ltol = 1e-5 * (np.abs(p64 * z64).sum(axis=1) + np.abs(lse) * p64.sum(axis=1)) + 1e-6
    lerr = np.abs(got_loss - ref_loss)
    assert (lerr <= ltol).all(), f"{label}: loss max err {lerr.max():.3g}"
    return float((err / np.maximum(rowmax, 1e-30)).max()), float(lerr.max())


@pytest.mark.parametrize("N,V,dtype", [
    (5, 8, "f32"), (33, 1000, "f32"), (7, 32768, "f32"), (3, 40000, "f32"),
    (64, 4000, "bf16"), (16, 32000, "bf16"), (6, 65536, "bf16"), (3, 131072, "bf16"),
])
def test_loss_grad_matches_oracle(gpu_lib, N, V, dtype):
    """Register-resident rows (every vector count up to the limit) and the streaming path."""
    z, p, g = inputs.loss_case(N + V, N, V, dtype)
    print(f"loss case N={N} V={V} {dtype}", flush=True)
    zd, loss = _run(gpu_lib, z, p, g, dtype)
    e = _check(z, p, g, zd.double().cpu().numpy(), loss.double().cpu().numpy(), dtype, f"N={N} V={V} {dtype}")
    print("errors", e)


def test_loss_grad_edge_cases(gpu_lib):
    """One-hot targets, a masked row, large and equal logits, targets summing to less than 1."""
    N, V = 6, 1024
    z, p, g = inputs.loss_case(3, N, V, "f32")
    p[0] = 0.0
    p[0, 17] = 1.0                   # one-hot
    z[1] *= 40.0                     # peaky logits (exp underflows for most columns)
    z[2] = 3.0                       # equal logits
    p[3] *= 0.25                     # targets summing to 1/4
    g[4] = 0.0                       # masked row
    zd, loss = _run(gpu_lib, z, p, g, "f32")
    got = zd.double().cpu().numpy()
    _check(z, p, g, got, loss.double().cpu().numpy(), "f32", "edge cases")
    assert not got[4].any()


def test_loss_grad_without_loss_output(gpu_lib):
    import torch
    z, p, g = inputs.loss_case(8, 4, 512, "bf16")
    zd = torch.from_numpy(z).to("cuda", torch.bfloat16)
    pd = torch.from_numpy(p).to("cuda", torch.bfloat16)
    gd = torch.from_numpy(g).to("cuda")
    assert gpu_lib.loss_grad_inplace(zd, pd, gd, want_loss=False) is None
    torch.cuda.synchronize()
    ref = LO.grad_inplace(z, p, g)
    assert np.abs(zd.double().cpu().numpy() - ref).max() <= 2.0 ** -8 * np.abs(ref).max() + 1e-6


@pytest.mark.slow
def test_loss_grad_full_size_lm_head(gpu_lib):
    """The draft LM head of one TTT step (N = 8192 tokens, V = 32000, bf16), in the launch the
    benchmark times: 64 sampled rows against the oracle, every row for the closed-form
    properties (gradient rows sum to zero; masked rows are zero)."""
    import torch
    N, V = inputs.LOSS_WORKLOADS["llama3.1-8b-draft-lmhead N8192 V32000"]
    zd, pd, gd = inputs.loss_case_device(11, N, V, "bf16")
    rows = np.random.default_rng(5).choice(N, size=64, replace=False)
    rows = np.union1d(rows, [0, N - 1])
    ri = torch.as_tensor(rows, device="cuda")
    z, p, g = (zd[ri].double().cpu().numpy(), pd[ri].double().cpu().numpy(),
               gd[ri].double().cpu().numpy())
    g_all = gd.clone()
    loss = gpu_lib.loss_grad_inplace(zd, pd, gd)
    torch.cuda.synchronize()
    e = _check(z, p, g, zd[ri].double().cpu().numpy(), loss[ri].double().cpu().numpy(), "bf16",
               "full size")
    print("sampled errors", e)
    gz = zd.double()
    rs = gz.sum(dim=1).abs() / gz.abs().sum(dim=1).clamp_min(1e-30)
    assert float(rs.max()) < 1e-2
    assert not bool(zd[g_all == 0].any())

"""One TTT step (forward, then backward) captured in a HIP graph replays to the eager results.

Every kernel of the library goes on the caller's stream, and the library itself never
allocates, frees, synchronises or clears memory with a memset, so a training loop can capture
the step once and replay it.  The graph is replayed several times with eager work between the
replays (the outputs are overwritten by fill kernels first), and every replay must match the
eager call bitwise: the kernels are deterministic (fixed summation orders, no atomics).
"""
import numpy as np
import pytest

from masked_attention_eagle_amd import inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


# head_dim 64 runs on the matrix-core kernels through zero-padded copies (copy kernels too)
@pytest.mark.parametrize("suffix,dq_mode,d", [("fused", "stored", 128), ("separate", "recompute", 128),
                                              ("fused", "stored", 64)])
def test_step_replays_in_a_graph(gpu_lib, suffix, dq_mode, d):
    import torch
    A = gpu_lib
    B, Hq, Hkv, L, step = 2, 4, 2, 512, 2
    q, k, v, do, T = inputs.make_case(31, B, Hq, Hkv, d, L, step, [500, 300], "bf16")
    print(f"graph case suffix={suffix} dq={dq_mode} d={d} B={B} Hq={Hq} Hkv={Hkv} L={L} step={step}",
          flush=True)
    bf = torch.bfloat16
    qd, kd, vd, dod = (to_dev(x, bf) for x in (q, k, v, do))
    Td = torch.as_tensor(T, device="cuda")
    scale = 1.0 / np.sqrt(d)

    o_e, lse_e = A.ttt_attn_fwd(qd, kd, vd, Td, scale, suffix=suffix)
    dq_e, dk_e, dv_e = A.ttt_attn_bwd(qd, kd, vd, Td, o_e, lse_e, dod, scale, dq_mode=dq_mode)
    torch.cuda.synchronize()

    # static outputs and workspaces, allocated before the capture
    p_f = A._params_from(qd, kd, scale, A.path_flags(suffix))
    p_b = A._params_from(qd, kd, scale, A.path_flags("fused", dq_mode))
    ws_f = torch.empty(max(A.fwd_workspace_size(p_f), 1), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(A.bwd_workspace_size(p_b), 1), dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(o_e), torch.empty_like(lse_e)
    dq, dk, dv = torch.empty_like(dq_e), torch.empty_like(dk_e), torch.empty_like(dv_e)

    def step_fn():
        A.ttt_attn_fwd(qd, kd, vd, Td, scale, out=o, lse=lse, workspace=ws_f, suffix=suffix)
        A.ttt_attn_bwd(qd, kd, vd, Td, o, lse, dod, scale, dq=dq, dk=dk, dv=dv, workspace=ws_b,
                       dq_mode=dq_mode)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_fn()
    torch.cuda.synchronize()

    outs = (o, lse, dq, dk, dv)
    refs = (o_e, lse_e, dq_e, dk_e, dv_e)
    for rep in range(3):
        for t in outs:
            t.fill_(7.0)  # eager work between replays; the replay must overwrite all of it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), outs, refs):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"


def test_sweep_replays_in_a_graph(gpu_lib):
    """The whole-TTT calls (forward and backward over every step, one KV cache) captured once
    and replayed: each replay matches the eager calls bitwise.  Outputs and workspaces come from
    the capture's memory pool, so they stay in place across replays."""
    import torch
    from tests.test_parity_sweep import _sweep_case
    A = gpu_lib
    B, Hq, Hkv, d, L, K = 2, 4, 2, 128, 256, 3
    q, kc, vc, do, T = _sweep_case(77, B, Hq, Hkv, d, L, K, (256, 140))
    print(f"graph sweep case B={B} Hq={Hq} Hkv={Hkv} L={L} K={K} T={list(T)}", flush=True)
    bf = torch.bfloat16
    qd, kd, vd, dod = (to_dev(x, bf) for x in (q, kc, vc, do))
    Td = torch.as_tensor(T, device="cuda")
    scale = 1.0 / np.sqrt(d)
    o_e, lse_e = A.ttt_attn_fwd_sweep(qd, kd, vd, Td, scale)
    refs = (o_e, lse_e) + tuple(A.ttt_attn_bwd_sweep(qd, kd, vd, Td, o_e, lse_e, dod, scale))
    torch.cuda.synchronize()

    def step_fn():
        o, lse = A.ttt_attn_fwd_sweep(qd, kd, vd, Td, scale)
        return (o, lse) + tuple(A.ttt_attn_bwd_sweep(qd, kd, vd, Td, o, lse, dod, scale))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step_fn()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), outs, refs):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"

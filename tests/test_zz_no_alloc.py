"""The no-allocation backward (ttt_attn_bwd_noalloc) against ttt_attn_bwd on the same path (the
dQ kernel recomputing S and dP): the same kernels run on the library's fixed scratch array
instead of a caller workspace, so dq, dk and dv must be bitwise equal.  Calls in a row share
the array and each starts from what the previous one left there: the full-size
Llama-3.1-8B-shaped step first, then smaller shapes (matrix-core at head_dim 128 and 64,
vector-ALU bf16 and fp32 paths), then the first shape again."""
import ctypes

import numpy as np
import pytest

from masked_attention_eagle_amd import inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def _noalloc(lib, qd, kd, vd, Td, o, lse, dod, scale):
    import torch
    from masked_attention_eagle_amd import ttt_attn as A
    p = A._params_from(qd, kd, scale)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    rc = A.load().ttt_attn_bwd_noalloc(ctypes.byref(p), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                       Td.data_ptr(), o.data_ptr(), lse.data_ptr(), dod.data_ptr(),
                                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == 0, A.status_string(rc)
    return dq, dk, dv


def _case(label, q, k, v, do, T, dtype):
    import torch
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    return label, (qd, kd, vd, torch.as_tensor(np.asarray(T, dtype=np.int32), device="cuda"), dod)


def test_noalloc_backward_matches_workspace_backward(gpu_lib):
    import torch
    w = inputs.WORKLOADS[2]
    full = _case("llama3.1-8b step 6", inputs.q_at(w, 6), *inputs.kv_stack(w, 6), inputs.do_at(w, 6),
                 inputs.seq_lengths(w), "bf16")
    cases = [full,
             _case("bf16 B2 Hq8 Hkv2 L512 k3", *inputs.make_case(81, 2, 8, 2, 128, 512, 3, (512, 301), "bf16"), "bf16"),
             _case("bf16 B1 Hq4 Hkv1 L256 k1", *inputs.make_case(82, 1, 4, 1, 128, 256, 1, 200, "bf16"), "bf16"),
             _case("bf16 d64 B2 Hq4 Hkv2 L192 k2", *inputs.make_case(83, 2, 4, 2, 64, 192, 2, (150, 192), "bf16"), "bf16"),
             # head_dim 64 on the matrix-core kernels: zero-padded copies in the scratch array
             _case("bf16 d64 B2 Hq8 Hkv2 L256 k2", *inputs.make_case(85, 2, 8, 2, 64, 256, 2, (256, 97), "bf16"), "bf16"),
             _case("f32 B1 Hq2 Hkv1 L128 k2", *inputs.make_case(84, 1, 2, 1, 64, 128, 2, 100, "f32"), "f32"),
             full]
    for label, (qd, kd, vd, Td, dod) in cases:
        print("case", label, flush=True)
        scale = 1.0 / np.sqrt(qd.shape[-1])
        o, lse = gpu_lib.ttt_attn_fwd(qd, kd, vd, Td, scale)
        want = gpu_lib.ttt_attn_bwd(qd, kd, vd, Td, o, lse, dod, scale, dq_mode="recompute")
        got = _noalloc(gpu_lib, qd, kd, vd, Td, o, lse, dod, scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            bits = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(a.view(bits), b.view(bits)), f"{label}: {name} differs"


def test_noalloc_backward_replays_in_a_graph(gpu_lib):
    """The use the no-allocation backward is for: captured in a HIP graph (after one eager call,
    which looks up the scratch array's address) with caller-owned outputs and no workspace, then
    replayed three times with eager fills of the outputs between the replays; every replay
    matches the eager call bitwise."""
    import torch
    q, k, v, do, T = inputs.make_case(85, 2, 8, 2, 128, 512, 3, (512, 377), "bf16")
    print("graph no-alloc case B=2 Hq=8 Hkv=2 L=512 k=3", flush=True)
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    Td = torch.as_tensor(T, device="cuda")
    o, lse = gpu_lib.ttt_attn_fwd(qd, kd, vd, Td)
    refs = gpu_lib.ttt_attn_bwd_noalloc(qd, kd, vd, Td, o, lse, dod)
    torch.cuda.synchronize()
    outs = tuple(torch.empty_like(r) for r in refs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu_lib.ttt_attn_bwd_noalloc(qd, kd, vd, Td, o, lse, dod, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu_lib.ttt_attn_bwd_noalloc(qd, kd, vd, Td, o, lse, dod, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("dq", "dk", "dv"), outs, refs):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep}: {name}"

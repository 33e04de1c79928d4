"""Backward calls in flight at once on two streams, each with its own workspace (the dK/dV
kernel's work-queue counters live in the workspace, so such calls share no state): every
result equals that of the same call made alone, bit for bit."""
import numpy as np
import pytest

from masked_attention_eagle_amd import inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dq_mode", ["stored", "recompute"])
def test_backward_on_two_streams_matches_serial_calls(gpu_lib, dq_mode):
    import torch
    bf = torch.bfloat16
    cases = []
    for seed, (B, Hq, Hkv, L, step, T) in enumerate([(2, 8, 2, 512, 2, (512, 301)),
                                                      (1, 16, 4, 384, 1, (200,))]):
        q, k, v, do, Tn = inputs.make_case(700 + seed, B, Hq, Hkv, 128, L, step, T, "bf16")
        qd, kd, vd, dod = (to_dev(x, bf) for x in (q, k, v, do))
        Td = torch.as_tensor(Tn, device="cuda")
        o, lse = gpu_lib.ttt_attn_fwd(qd, kd, vd, Td)
        cases.append((qd, kd, vd, Td, o, lse, dod))
    torch.cuda.synchronize()
    ref = [gpu_lib.ttt_attn_bwd(*c, dq_mode=dq_mode) for c in cases]
    torch.cuda.synchronize()
    print(f"two streams, dq={dq_mode}", flush=True)
    streams = [torch.cuda.Stream() for _ in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [[] for _ in cases]
    for rep in range(3):  # several calls per stream, interleaved on the host
        for i, (s, c) in enumerate(zip(streams, cases)):
            with torch.cuda.stream(s):
                got[i].append(gpu_lib.ttt_attn_bwd(*c, dq_mode=dq_mode))
    for s in streams:
        s.synchronize()
    for i in range(len(cases)):
        for out in got[i]:
            for a, b in zip(out, ref[i]):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16))

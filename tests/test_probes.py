"""The measurement helpers on the GPU: the peak probes do their work (the copy moves every byte,
the matrix-core probe writes finite sums), and cold-cache timing (a caller buffer overwritten
before every timed launch) leaves the attention results untouched."""
import numpy as np
import pytest

from masked_attention_eagle_amd import inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def test_copy_probe_copies_every_byte(gpu_lib):
    import torch
    n = (1 << 20) + 3 * 8  # not a whole number of 16 KB chunks: the last one is partial
    src = torch.arange(n, dtype=torch.int64, device="cuda")
    dst = torch.zeros_like(src)
    gpu_lib.probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_mfma_probe_writes_finite_sums(gpu_lib):
    import torch
    wgs = 64
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.probe_mfma_bf16(sink, wgs, 16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())


def test_cold_cache_timing_keeps_results(gpu_lib):
    import torch
    q, k, v, do, T = inputs.make_case(91, 2, 4, 2, 128, 256, 2, (256, 190), "bf16")
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    Td = torch.as_tensor(T, device="cuda")
    o, lse = gpu_lib.ttt_attn_fwd(qd, kd, vd, Td)
    ref = gpu_lib.ttt_attn_bwd(qd, kd, vd, Td, o, lse, dod)
    flush = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    gpu_lib.timing_reset()
    gpu_lib.timing_flush(flush)
    gpu_lib.timing_enable(True)
    try:
        o2, lse2 = gpu_lib.ttt_attn_fwd(qd, kd, vd, Td)
        got = gpu_lib.ttt_attn_bwd(qd, kd, vd, Td, o2, lse2, dod)
        torch.cuda.synchronize()
    finally:
        gpu_lib.timing_enable(False)
        gpu_lib.timing_flush(None)
    times = gpu_lib.timing_read()
    assert "fwd_causal_mfma" in times and "bwd_dkdv_mfma" in times
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert bool((flush == 0).all())  # the flush wrote zeros over the whole buffer


def test_timing_counts_launches_from_two_threads(gpu_lib):
    """Timed launches from two threads on their own streams: every launch is counted once and
    the results are those of an untimed call."""
    import threading
    import torch
    q, k, v, _, T = inputs.make_case(92, 2, 4, 2, 128, 256, 2, (256, 170), "bf16")
    qd, kd, vd = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    Td = torch.as_tensor(T, device="cuda")
    ref_o, ref_lse = gpu_lib.ttt_attn_fwd(qd, kd, vd, Td)
    torch.cuda.synchronize()
    n_calls, results, errors = 6, {}, []

    def worker(tag):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [gpu_lib.ttt_attn_fwd(qd, kd, vd, Td) for _ in range(n_calls)]
            s.synchronize()
            results[tag] = outs
        except Exception as e:  # reported below, in the test's thread
            errors.append(e)

    gpu_lib.timing_reset()
    gpu_lib.timing_enable(True)
    try:
        threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
    finally:
        gpu_lib.timing_enable(False)
    torch.cuda.synchronize()
    assert not errors, errors
    times = gpu_lib.timing_read()
    assert times["fwd_causal_mfma"][0] == 2 * n_calls
    assert times["fwd_causal_mfma"][1] > 0
    for outs in results.values():
        for o, lse in outs:
            assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
            assert torch.equal(lse, ref_lse)
    assert gpu_lib.timing_read()["fwd_causal_mfma"][0] == 2 * n_calls  # nothing read twice

"""The FFN entry point that allocates nothing (its workspace is a file-scope device array) against
moe_slot_ffn on the same routed, ensured and copied calls: outputs and residual streams bit for bit,
and the oracle's output within tolerance.  Two calls in a row, the second with fewer tokens; then a
call whose workspace would exceed the array is rejected before any launch."""
import numpy as np
import pytest
import torch

import expert_offload_slot_amd as m
import oracle
import synth
from gpu_harness import GpuLayer, make_layer_inputs, row_rel_err, to_dev, to_np, TOL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wdt,E,S,k,H,F,Ts,shared", [
    (1, 32, 10, 4, 512, 256, [24, 1], False),    # batch kernels, then the single-token kernels
    (2, 64, 12, 2, 256, 256, [80, 9, 3], True),  # fp8 grouped GEMM (> 64 tokens; 9 tokens: 0.28 pairs per
                                                 # expert, the GEMM too), then a 3-token decode batch (0.09)
    (0, 8, 4, 2, 64, 128, [6, 3], False),        # fp32 kernels
    (3, 16, 8, 4, 256, 512, [40, 2], True),      # MXFP4: 40 tokens take the GEMM, 2 the decode kernels
])
def test_noalloc_ffn_matches_slot_ffn(wdt, E, S, k, H, F, Ts, shared):
    print("noalloc wdt=%d E=%d S=%d k=%d H=%d F=%d Ts=%s shared=%s" % (wdt, E, S, k, H, F, Ts, shared), flush=True)
    host, wr, b, sh = make_layer_inputs(41, 0, E, H, F, wdt, 1.2, shared)
    gl = GpuLayer(E, S, k, H, F, wdt, max(Ts), host, wr, b, shared=sh)
    ol = oracle.Layer(E, S, k, H, F, wdt, host, wr, b, shared=sh)
    xs = synth.tokens(41, 3, max(Ts), H, len(Ts), 0.0, wdt)
    adt = torch.float32 if wdt == 0 else torch.bfloat16
    try:
        for i, T in enumerate(Ts):
            x = np.ascontiguousarray(xs[i][:T])
            xd = to_dev(x)
            gl.route(xd, T)
            gl.ensure(T)
            gl.copy()
            y_ref = torch.zeros((T, H), dtype=adt, device="cuda")
            xn_ref = torch.zeros((T, H), dtype=adt, device="cuda")
            y_na = torch.full((T, H), 7.0, dtype=adt, device="cuda")
            xn_na = torch.full((T, H), 7.0, dtype=adt, device="cuda")
            s = torch.cuda.current_stream()
            m.moe_slot_ffn(gl.h, xd, gl.slot_ids, gl.w, T, gl.shared, y_ref, None, xn_ref, s)
            m.moe_slot_ffn_noalloc(gl.h, xd, gl.slot_ids, gl.w, T, gl.shared, y_na, None, xn_na, s)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(y_na), to_np(y_ref)), (i, T)
            assert np.array_equal(to_np(xn_na), to_np(xn_ref)), (i, T)
            r = ol.step(x)
            assert np.array_equal(to_np(gl.slot_ids[:T]), r["slot_ids"])
            assert row_rel_err(to_np(y_na), r["y64"], wdt) <= TOL[wdt]
        assert gl.stats()["error"] == 0
    finally:
        gl.close()


def test_noalloc_rejects_calls_beyond_the_scratch():
    # DeepSeek-V3-sized rows: 2048 tokens x (8 + 1) rows of (2048 x 2 + 7168 x 4) bytes is far above 32 MiB
    E, S, k, H, F, T = 16, 8, 8, 7168, 2048, 2048
    h = m.moe_offload_create(E, S, H, F, k, m.FP8, T, 0, 0)
    try:
        x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
        sid = torch.zeros((T, k), dtype=torch.int32, device="cuda")
        w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
        y = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(m.MoeError) as ei:
            m.moe_slot_ffn_noalloc(h, x, sid, w, T, None, y)
        assert ei.value.code == m.EINVAL and "scratch" in str(ei.value)
        with pytest.raises(m.MoeError) as ei:
            m.moe_slot_ffn_noalloc(h, x, sid, w, 0, None, y)
        assert ei.value.code == m.EINVAL
        torch.cuda.synchronize()
        assert m.moe_offload_stats(h)["error"] == 0
    finally:
        m.moe_offload_destroy(h)

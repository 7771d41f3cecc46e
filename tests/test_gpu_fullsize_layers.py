"""GPU parity of single layers at the full sizes of two workloads, through the
entry points (route, ensure or prefill stage, copy, FFN).

* Mixtral-8x7B shape: 8 experts, top-2, hidden 4096, ffn 14336 (352 MB per
  expert), slots 2, 4 and 6, decode batches 1 to 64 plus one call above 64
  tokens (the matrix-core FFN kernels), uniform router.
* DeepSeek-V3 shape: fp8 e4m3 with 128x128 block scales, 256 experts plus a
  shared expert, top-8, hidden 7168, ffn 2048, 26 slots; decode batch 16, a
  2048-token prefill that stages the whole layer, then decode batch 16 again
  from an empty cache in split mode (a measured share of the staged misses
  computed by the host CPU).

Every call is checked bit for bit on ids, slot ids, the copy list and the slot
table (weights within 1e-5); a few token rows per call are computed one by one
by the oracle straight from the host records of the routed experts and must be
within 2e-2 of its double sums.
"""
import numpy as np
import pytest
import torch

import expert_offload_slot_amd as m
import oracle
import synth
from gpu_harness import GpuLayer, d2h, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

BF16, FP8 = 1, 2


def log(*a):
    print(*a, flush=True)


def fill_layer(gl, seed, E, H, F, wdt):
    p, stride, _ = m.moe_offload_host_records(gl.h)
    synth.fill_records(seed, 0, 0, E, H, F, wdt, p, stride)
    return m.host_array(gl.h, E)


def check_call(gl, cache, x, T, wr, b, wdt, H, F, host, toks, shared=None, prefill=False):
    ids, w, _ = oracle.route(x, wr, b, gl.k, wdt)
    assert np.array_equal(to_np(gl.ids[:T]), ids)
    assert np.abs(to_np(gl.w[:T]) - w).max() <= 1e-5
    if prefill and oracle.distinct(ids, gl.E) > gl.S:
        sid, mode, pairs = cache.stage_all(ids)
    else:
        sid, mode, pairs = cache.ensure(ids)
    assert np.array_equal(to_np(gl.slot_ids[:T]), sid)
    gmode, gpairs = gl.copy_list()
    assert gmode == mode and np.array_equal(gpairs, pairs), (gmode, gpairs, mode, pairs)
    so, eo, lu = gl.table()
    oso, oeo, olu, _ = cache.state()
    assert np.array_equal(so, oso) and np.array_equal(eo, oeo) and np.array_equal(lu, olu)
    toks = sorted(set(t for t in toks if t < T))
    _, y64 = oracle.ffn(x[toks], wdt, H, F, oracle.host_records(host, ids[toks]), w[toks], shared, want_f64=True)
    err = row_rel_err(to_np(gl.y[:T])[toks], y64, wdt)
    assert err <= 2e-2, err
    return mode, err


@pytest.mark.parametrize("S", [2, 4, 6])
def test_mixtral_shape_decode(S):
    E, k, H, F, wdt, seed = 8, 2, 4096, 14336, BF16, 7
    wr, b = synth.router(seed, 0, E, H, wdt, zipf_s=0.0)  # uniform router
    gl = GpuLayer(E, S, k, H, F, wdt, 96, None, wr, b)
    try:
        host = fill_layer(gl, seed, E, H, F, wdt)
        cache = oracle.Cache(E, S)
        modes, worst = set(), 0.0
        for i, T in enumerate([1, 2, 4, 8, 16, 32, 64, 3, 80]):
            log("mixtral S=%d call %d T=%d" % (S, i, T))
            x = np.ascontiguousarray(synth.tokens(seed, 20 + i, T, H, 1, 0.0, wdt)[0])
            gl.step(to_dev(x), T)
            mode, err = check_call(gl, cache, x, T, wr, b, wdt, H, F, host, (0, T // 2, T - 1))
            modes.add(mode)
            worst = max(worst, err)
        assert m.moe_offload_stats(gl.h)["error"] == 0
        log("mixtral S=%d: modes %s, sampled rows within %.2e" % (S, sorted(modes), worst))
    finally:
        gl.close()


def test_deepseek_shape_fp8_decode_and_prefill():
    E, k, H, F, S, wdt, seed = 256, 8, 7168, 2048, 26, FP8, 9
    wr, b = synth.router(seed, 0, E, H, BF16, zipf_s=1.2)
    shared = synth.records(seed, 0, 1, H, F, wdt, shared=True)[0]
    gl = GpuLayer(E, S, k, H, F, wdt, 2048, None, wr, b, shared=shared)
    try:
        host = fill_layer(gl, seed, E, H, F, wdt)
        cache = oracle.Cache(E, S)
        worst = 0.0
        for s in range(16):
            log("deepseek decode step %d (T=16)" % s)
            x = np.ascontiguousarray(synth.tokens(seed, 30 + s, 16, H, 1, 0.0, BF16)[0])
            gl.step(to_dev(x), 16)
            _, err = check_call(gl, cache, x, 16, wr, b, wdt, H, F, host, (s % 16, 15 - s % 16), shared)
            worst = max(worst, err)
        log("deepseek prefill T=2048")
        T = 2048
        x = np.ascontiguousarray(synth.tokens(seed, 40, T, H, 1, 0.0, BF16)[0])
        xd = to_dev(x)
        gl.route(xd, T)
        staged = m.moe_prefill_stage(gl.h, gl.ids, T, gl.slot_ids, torch.cuda.current_stream())
        assert staged == 1
        gl.ffn(xd, T)
        torch.cuda.synchronize()
        mode, err = check_call(gl, cache, x, T, wr, b, wdt, H, F, host, (0, 1, 777, 1500, 2047), shared, prefill=True)
        assert mode == oracle.STAGED_ALL
        worst = max(worst, err)
        for e in (0, 100, 255):
            got = d2h(gl.info["staging"] + e * gl.info["record_stride"], gl.info["record_bytes"])
            assert np.array_equal(got, host[e, :gl.info["record_bytes"]])
        assert m.moe_offload_stats(gl.h)["error"] == 0
        log("deepseek: decode + prefill bit-exact routing/slots, sampled rows within %.2e" % worst)
        # split mode from an empty cache: the share q measured on this machine; each overflowing call sends
        # that share of its staged misses to the host CPU (records listed at S + E + e) and copies the rest
        st = torch.cuda.current_stream()
        m.moe_offload_reset(gl.h, st)
        cache = oracle.Cache(E, S)
        q, cpu_us, link_us = m.moe_offload_set_cold(gl.h, m.COLD_SPLIT, st)
        cache.set_split(q)
        log("deepseek split: host %.1f us, link %.1f us per record -> q %d" % (cpu_us, link_us, q))
        before = m.moe_offload_stats(gl.h)
        host_seen = 0
        try:
            for s in range(8):
                log("deepseek split decode step %d (T=16)" % s)
                x = np.ascontiguousarray(synth.tokens(seed, 50 + s, 16, H, 1, 0.0, BF16)[0])
                xd = to_dev(x)
                gl.route(xd, 16)
                gl.ensure(16)
                gl.copy()
                m.moe_slot_ffn_host_cold(gl.h, xd, gl.slot_ids, gl.w, 16, gl.shared, gl.y, None, None, st)
                torch.cuda.synchronize()
                _, err = check_call(gl, cache, x, 16, wr, b, wdt, H, F, host, (s % 16, 15 - s % 16), shared)
                worst = max(worst, err)
                _, pairs = gl.copy_list()
                host_seen += int((pairs[:, 1] >= S + E).sum()) if len(pairs) else 0
        finally:
            m.moe_offload_set_cold(gl.h, m.COLD_OFF, st)
        after = m.moe_offload_stats(gl.h)
        c = cache.counters()
        assert after["error"] == 0
        for key in ("calls", "hits", "misses", "staged_calls", "staged_copies"):
            assert after[key] - before[key] == c[key], key
        assert after["cold_misses"] - before["cold_misses"] == c["cold"] == host_seen > 0
        log("deepseek split: 8 calls bit-exact, %d host-computed records, sampled rows within %.2e" % (host_seen, worst))
    finally:
        gl.close()

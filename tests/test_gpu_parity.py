"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: router ids, slot ids, copy lists, slot tables, slot bytes.
Within tolerance: routing weights (1e-5) and layer outputs (per token row,
||y - ref||_inf <= tol * ||ref||_inf with tol 1e-5 for fp32 and 2e-2 for
bf16/fp8; ref = the oracle's double sums).
Sizes span several kernel tiles, ragged token counts, staging, and more than
one 64-token pass per expert.
"""
import numpy as np
import pytest
import torch

import expert_offload_slot_amd as m
import oracle
import synth
from gpu_harness import (TOL, GpuLayer, compare_call, d2h, h2d, make_layer_inputs, oracle_policy, row_rel_err,
                         to_dev, to_np)

pytestmark = pytest.mark.gpu


def run_sequence(E, S, k, H, F, wdt, zipf, seed, steps, Ts, shared=False, flags=m.FLAG_AUDIT, pins=None,
                 gemm_waves=0):
    print("case E=%d S=%d k=%d H=%d F=%d wdt=%d zipf=%s seed=%d Ts=%s shared=%s" %
          (E, S, k, H, F, wdt, zipf, seed, Ts, shared), flush=True)
    host, wr, b, sh = make_layer_inputs(seed, 0, E, H, F, wdt, zipf, shared)
    maxT = max(Ts)
    gl = GpuLayer(E, S, k, H, F, wdt, maxT, host, wr, b, flags=flags, shared=sh)
    m.moe_offload_set_gemm_waves(gl.h, gemm_waves)
    ol = oracle.Layer(E, S, k, H, F, wdt, host, wr, b, shared=sh,
                      policy=oracle_policy(flags))
    xs = synth.tokens(seed, 7, maxT, H, steps, 0.0, wdt)
    modes, errs = [], []
    try:
        for s in range(steps):
            if pins and s in pins:  # a new pinned set before this step, on both sides
                P = np.array(pins[s], np.int32)
                m.moe_offload_pin(gl.h, to_dev(P) if len(P) else None, len(P), torch.cuda.current_stream())
                want = ol.cache.pin(P)
                ol.cache.copy(0, want)
                mode, got = gl.copy_list()
                assert mode == 0 and np.array_equal(got, want), (s, got, want)
                assert np.array_equal(gl.pinned(), ol.cache.pinned()), s
            T = Ts[s % len(Ts)]
            x = np.ascontiguousarray(xs[s][:T])
            xd = to_dev(x)
            gl.step(xd, T)
            r = ol.step(x)
            errs.append(compare_call(gl, r, T, r["y64"], oracle_cache=ol.cache))
            modes.append(r["mode"])
            # residual output: round(x + y) from the GPU's own y
            xn = to_np(gl.xn[:T])
            assert np.array_equal(xn, oracle.residual(x, to_np(gl.y[:T]), wdt))
        st = gl.stats()
        c = ol.cache.counters()
        assert st["error"] == 0
        for key in ("calls", "hits", "misses", "staged_calls", "staged_copies"):
            assert st[key] == c[key], key
        # every resident slot holds its expert's host bytes
        so, eo, lu = gl.table()
        rb = oracle.record_bytes(wdt, H, F)
        for s_ in range(S):
            if eo[s_] >= 0:
                assert np.array_equal(gl.slot_bytes(s_, rb), host[eo[s_], :rb])
    finally:
        gl.close()
    return modes, max(errs)


def test_c1_tiny_fp32_config():
    # 8 experts, top-2, hidden 64, ffn 128, 4 slots, 32 steps of batch 4, Zipf(1.2)-ranked bias
    for seed in range(4):
        run_sequence(8, 4, 2, 64, 128, 0, 1.2, seed, 32, [4])


@pytest.mark.parametrize("S", [2, 3, 4, 8])
def test_c1_variants_slots_and_batches(S):
    modes, _ = run_sequence(8, S, 2, 64, 128, 0, 0.0, 11 + S, 24, [1, 2, 4, 8])
    if S < 8:
        assert 1 in modes and 0 in modes  # both slot calls and staged calls ran


@pytest.mark.parametrize("S,zipf", [(4, 0.0), (6, 1.2), (16, 0.0)])
def test_bf16_multi_tile(S, zipf):
    run_sequence(16, S, 4, 256, 384, 1, zipf, 21, 20, [1, 3, 8, 17])


def test_bf16_many_tokens_per_expert():
    # > 64 tokens on an expert: several passes over each weight tile
    run_sequence(8, 8, 2, 128, 256, 1, 1.2, 5, 4, [300, 77])


@pytest.mark.parametrize("S", [4, 12])
def test_fp8_block_scaled_with_shared_expert(S):
    # 256 x 384 fp8 records are 294,984 bytes: not a multiple of 16 (the scales sit in the tail)
    run_sequence(12, S, 3, 256, 384, 2, 0.0, 31, 12, [1, 5, 16], shared=True)


def test_fp8_prefill_gemm_ragged_tiles():
    # > 64 tokens per call: the grouped GEMM; records with partial 64-pair tiles,
    # several K slices and row tiles, the shared expert's own tiles
    run_sequence(12, 6, 3, 256, 384, 2, 1.2, 33, 3, [100, 130, 65], shared=True)


@pytest.mark.parametrize("wdt", [1, 2, 3])
@pytest.mark.parametrize("waves", [4, 8])
def test_prefill_gemm_several_tiles_per_record(wdt, waves):
    # the grouped GEMM at H = F = 512 (8 row tiles each way with 4 wavefronts per workgroup, 4 and 2
    # with 8) in bf16, fp8 and MXFP4; Zipf routing gives records several 64-pair token tiles and a
    # ragged last one
    run_sequence(8, 8, 2, 512, 512, wdt, 1.2, 80 + wdt, 3, [300, 129, 70], shared=(wdt != 1), gemm_waves=waves)


@pytest.mark.parametrize("wdt", [1, 2, 3])
def test_prefill_gemm_automatic_workgroup_size(wdt):
    """A call just large enough for the automatic rule to give gate/up 8-wavefront workgroups: T * k / 64 =
    32 token tiles times F / 128 = 32 row tiles = 1024 items (down, H / 256 = 1 row tile, keeps 4).  The
    automatic choice, 4 forced and 8 forced give the same bits, within tolerance of the oracle."""
    E, k, H, F, T = 16, 2, 256, 4096, 1024
    print("gemm automatic workgroup size wdt=%d T=%d" % (wdt, T), flush=True)
    host, wr, b, sh = make_layer_inputs(75, 0, E, H, F, wdt, 0.0, wdt == 2)
    x = np.ascontiguousarray(synth.tokens(76, 0, T, H, 1, 0.0, wdt)[0])
    gl = GpuLayer(E, E, k, H, F, wdt, T, host, wr, b, shared=sh)
    try:
        xd = to_dev(x)
        gl.route(xd, T)
        gl.ensure(T)
        gl.copy()
        ids, w = to_np(gl.ids[:T]), to_np(gl.w[:T])
        toks = [0, 1, 63, 64, 500, 777, 1022, 1023]  # sampled rows: the oracle's plain sums, one by one
        _, y64 = oracle.ffn(x[toks], wdt, H, F, oracle.host_records(host, ids[toks]), w[toks].astype(np.float64),
                            shared=sh, want_f64=True)
        ys = []
        for waves in (0, 4, 8):
            m.moe_offload_set_gemm_waves(gl.h, waves)
            gl.ffn(xd, T)
            ys.append(to_np(gl.y[:T]))
            assert row_rel_err(ys[-1][toks], y64, wdt) <= TOL[wdt], waves
        assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
        assert gl.stats()["error"] == 0
    finally:
        gl.close()


@pytest.mark.parametrize("wdt", [1, 2])
def test_prefill_gemm_down_rows_not_a_multiple_of_256(wdt):
    # H = 640 with 8-wavefront workgroups forced: gate/up row tiles of 128 rows (F = 384, three per
    # matrix), down keeps 4 wavefronts (five tiles of 128 rows); fp8 with the shared expert
    run_sequence(8, 8, 2, 640, 384, wdt, 1.2, 90 + wdt, 3, [300, 129, 70], shared=(wdt == 2), gemm_waves=8)


def test_bf16_prefill_gemm_one_hot_record():
    # every token routed to the same experts (k = E = S): one long record per expert
    run_sequence(2, 2, 2, 128, 256, 1, 0.0, 34, 2, [257, 64])


@pytest.mark.parametrize("H,F", [(2048, 512), (1024, 768), (768, 1024), (512, 128), (384, 2048), (1792, 256),
                                 (128, 384)])
@pytest.mark.parametrize("wdt", [1, 2])
def test_single_token_every_pass_width(H, F, wdt):
    # one-token calls stream each weight row in passes of 16, 8, 6, 4, 3, 2 or 1 K blocks of 128 (the
    # largest that divides the row): these shapes reach every width in gate/up (H / 128 blocks) and
    # in down (F / 128), bf16 and fp8 with the shared expert
    run_sequence(8, 4, 3, H, F, wdt, 1.2, 40 + H // 128, 6, [1], shared=(wdt == 2))


@pytest.mark.parametrize("H,F", [(4096, 256), (2048, 1536), (1536, 2048), (1024, 4096), (768, 512), (512, 768),
                                 (256, 1024)])
def test_mxfp4_single_token_every_pass_width(H, F):
    # MXFP4 K blocks hold 256 weights: H / 256 blocks for gate/up, F / 256 for down; these shapes
    # reach pass widths 16, 8, 6, 4, 3, 2 and 1 in each, with the shared expert
    run_sequence(8, 4, 3, H, F, 3, 1.2, 50 + H // 256, 6, [1], shared=True)


@pytest.mark.parametrize("S", [4, 12])
def test_mxfp4_decode_batches_with_shared_expert(S):
    run_sequence(16, S, 4, 512, 768, 3, 1.2, 61, 12, [1, 2, 5, 17, 64], shared=True)


def test_mxfp4_prefill_gemm_ragged_tiles():
    # > 64 tokens per call: the grouped GEMM with E2M1 codes widened (scale folded in) into registers
    run_sequence(12, 6, 3, 256, 512, 3, 1.2, 62, 3, [100, 130, 65], shared=True)


@pytest.mark.parametrize("wdt", [1, 2, 3])
def test_prefill_gemm_tile_boundaries(wdt):
    """Records whose pair counts sit on every GEMM tile boundary: a record's pairs form 64-pair tiles
    and a last tile of up to 80 (1 to 5 blocks of 16), so the counts 1, 15, 16, 17, 63 to 65, 79 to 81,
    96, 144, 145, 160 and 161 reach one-tile records of every width, the first count that splits, and
    two-tile records with the widest and narrowest last tile.  Choice 0 of each token names the record;
    choice 1 names expert 15, a record of every token (19 tiles, a 35-pair last one).  Tokens are
    shuffled, so every tile gathers rows from all over the call."""
    counts = [1, 15, 16, 17, 63, 64, 65, 79, 80, 81, 96, 144, 145, 160, 161]
    E, k, H, F = 16, 2, 256, 512  # MXFP4 needs multiples of 256
    T = sum(counts)
    rng = np.random.default_rng(70 + wdt)
    first = rng.permutation(np.repeat(np.arange(len(counts)), counts)).astype(np.int32)
    ids = np.stack([first, np.full(T, E - 1, np.int32)], axis=1)
    w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    shared = wdt == 2
    print("tile boundaries wdt=%d T=%d" % (wdt, T), flush=True)
    host, wr, b, sh = make_layer_inputs(71, 0, E, H, F, wdt, 0.0, shared)
    x = np.ascontiguousarray(synth.tokens(72, 0, T, H, 1, 0.0, wdt)[0])
    gl = GpuLayer(E, E, k, H, F, wdt, T, host, wr, b, shared=sh)
    try:
        m.moe_offload_set_ffn_path(gl.h, m.FFN_GEMM)
        gl.w[:T].copy_(torch.from_numpy(w))
        gl.ensure(T, ids=to_dev(ids))
        gl.copy()
        _, y64 = oracle.ffn(x, wdt, H, F, oracle.host_records(host, ids), w.astype(np.float64), shared=sh,
                            want_f64=True)
        # workgroups of 4 wavefronts, and of 8 (token rows two K slices ahead; down's single
        # 256-row tile spans two fp8 scale blocks): the same bits
        ys = []
        for waves in (4, 8):
            m.moe_offload_set_gemm_waves(gl.h, waves)
            gl.ffn(to_dev(x), T)
            ys.append(to_np(gl.y[:T]))
            assert row_rel_err(ys[-1], y64, wdt) <= TOL[wdt], waves
        assert np.array_equal(ys[0], ys[1])
        assert gl.stats()["error"] == 0
    finally:
        gl.close()


@pytest.mark.parametrize("E,S,k,Ts", [(16, 6, 4, [1, 2, 3]), (32, 10, 4, [1, 4, 9]), (64, 12, 8, [1, 2])])
def test_scored_eviction_parity(E, S, k, Ts):
    # scored eviction: slot tables, usage scores, copy lists and counters bit-exact against the oracle,
    # with Zipf routing (repeat customers) and batches that overflow the cache
    run_sequence(E, S, k, 256, 256, 1, 1.2, 70 + E, 30, Ts, flags=m.FLAG_AUDIT | m.FLAG_SCORED)


@pytest.mark.parametrize("E,S,k,Ts", [(16, 6, 4, [1, 2, 3]), (32, 10, 4, [1, 4, 9]), (64, 12, 8, [1, 2])])
def test_activation_aware_eviction_parity(E, S, k, Ts):
    # activation-aware eviction: slot tables, per-expert activation counts, copy lists and counters
    # bit-exact against the oracle, with Zipf routing and batches that overflow the cache
    run_sequence(E, S, k, 256, 256, 1, 1.2, 75 + E, 30, Ts, flags=m.FLAG_AUDIT | m.FLAG_FREQ)


@pytest.mark.parametrize("flags", [m.FLAG_AUDIT, m.FLAG_AUDIT | m.FLAG_SCORED, m.FLAG_AUDIT | m.FLAG_FREQ])
def test_pinned_placement_parity(flags):
    # pinned sets replaced mid-stream (overlapping, then empty); with 3 of 6 slots pinned a batch of 3
    # overflows although |D| <= S
    # (flat routing: 5-6 distinct experts per 3-token call against 3 unpinned slots)
    pins = {0: [1, 4, 9], 12: [4, 2], 24: []}
    modes, _ = run_sequence(16, 6, 2, 256, 256, 1, 0.0, 90, 32, [1, 2, 3], flags=flags, pins=pins)
    assert 1 in modes and 0 in modes


def test_fp8_without_shared_expert():
    run_sequence(10, 5, 2, 128, 256, 2, 1.2, 32, 10, [2, 7])


def test_placement_invariance_bitwise():
    """The same token stream at every slot count (slot calls, decode staging) and
    with whole-layer staging on every overflowing call: identical y bits."""
    E, k, H, F, wdt = 16, 4, 256, 256, 1
    host, wr, b, _ = make_layer_inputs(41, 0, E, H, F, wdt, 0.0)
    xs = synth.tokens(41, 3, 8, H, 12, 0.0, wdt)
    outs = {}
    staged_seen = set()
    for S in [4, 5, 9, 16, "prefill"]:
        gl = GpuLayer(E, 4 if S == "prefill" else S, k, H, F, wdt, 8, host, wr, b)
        ys = []
        for s in range(12):
            T = [1, 8, 3, 5][s % 4]
            xd = to_dev(np.ascontiguousarray(xs[s][:T]))
            gl.route(xd, T)
            if S == "prefill":
                staged_seen.add(m.moe_prefill_stage(gl.h, gl.ids, T, gl.slot_ids, torch.cuda.current_stream()))
            else:
                gl.ensure(T)
                gl.copy()
                staged_seen.add(("mode", gl.copy_list()[0]))
            gl.ffn(xd, T)
            ys.append(to_np(gl.y[:T]).copy())
        outs[S] = ys
        gl.close()
    assert {0, 1} <= staged_seen and ("mode", 0) in staged_seen and ("mode", 1) in staged_seen
    for S in outs:
        for a, b_ in zip(outs[S], outs[4]):
            assert np.array_equal(a, b_), S


def test_prefill_whole_layer_staging():
    E, S, k, H, F, wdt = 16, 4, 4, 256, 256, 1
    host, wr, b, _ = make_layer_inputs(51, 0, E, H, F, wdt, 0.0)
    T = 40
    gl = GpuLayer(E, S, k, H, F, wdt, T, host, wr, b)
    ol = oracle.Layer(E, S, k, H, F, wdt, host, wr, b)
    try:
        x = synth.tokens(51, 1, T, H, 1, 0.0, wdt)[0]
        xd = to_dev(x)
        gl.route(xd, T)
        staged = m.moe_prefill_stage(gl.h, gl.ids, T, gl.slot_ids)
        assert staged == 1
        gl.ffn(xd, T)
        r = ol.step(x, stage_all=True)
        compare_call(gl, r, T, r["y64"], oracle_cache=ol.cache)
        for e in range(E):
            assert np.array_equal(gl.staging_bytes(e, host.shape[1]), host[e])
        # a small call afterwards takes the slot path
        x1 = synth.tokens(51, 2, 1, H, 1, 0.0, wdt)[0]
        x1d = to_dev(x1)
        gl.route(x1d, 1)
        assert m.moe_prefill_stage(gl.h, gl.ids, 1, gl.slot_ids) == 0
        gl.ffn(x1d, 1)
        r = ol.step(x1)
        compare_call(gl, r, 1, r["y64"], oracle_cache=ol.cache)
    finally:
        gl.close()


def test_bad_id_is_a_noop_with_sticky_error():
    E, S, k, H, F = 8, 4, 2, 128, 128
    host, wr, b, _ = make_layer_inputs(61, 0, E, H, F, 1, 1.2)
    gl = GpuLayer(E, S, k, H, F, 1, 4, host, wr, b)
    try:
        x = to_dev(synth.tokens(61, 1, 2, H, 1, 0.0, 1)[0])
        gl.step(x, 2)
        before = gl.table()
        bad = torch.tensor([[1, 2], [3, E]], dtype=torch.int32, device="cuda")
        m.moe_slot_ensure(gl.h, bad, 2, gl.slot_ids)
        gl.copy()
        after = gl.table()
        assert all(np.array_equal(p, q) for p, q in zip(before, after))
        assert gl.copy_list()[1].shape[0] == 0
        st = gl.stats()
        assert st["error"] & m.DEV_ERR_BAD_ID
        with pytest.raises(m.MoeError):
            m.moe_prefill_stage(gl.h, bad, 2, gl.slot_ids)
        m.moe_offload_reset(gl.h)
        assert gl.stats()["error"] == 0 and gl.stats()["tick"] == 0
    finally:
        gl.close()


def test_pin_rejects_bad_sets():
    E, S, k, H, F = 8, 4, 2, 128, 128
    host, wr, b, _ = make_layer_inputs(62, 0, E, H, F, 1, 1.2)
    gl = GpuLayer(E, S, k, H, F, 1, 4, host, wr, b)
    try:
        with pytest.raises(m.MoeError) as ei:  # more than S - k pinned experts
            m.moe_offload_pin(gl.h, to_dev(np.array([0, 1, 2], np.int32)), 3)
        assert ei.value.code == m.EINVAL
        m.moe_offload_pin(gl.h, to_dev(np.array([5, 1], np.int32)), 2)
        torch.cuda.synchronize()
        before = gl.table() + (gl.pinned(),)
        assert gl.pinned().sum() == 2
        for bad in ([3, 3], [2, E]):  # repeated or out of range: nothing changes, sticky bad-id bit
            m.moe_offload_pin(gl.h, to_dev(np.array(bad, np.int32)), 2)
            torch.cuda.synchronize()
            after = gl.table() + (gl.pinned(),)
            assert all(np.array_equal(p, q) for p, q in zip(before, after))
            assert gl.stats()["error"] & m.DEV_ERR_BAD_ID
            m.moe_offload_reset(gl.h)
            m.moe_offload_pin(gl.h, to_dev(np.array([5, 1], np.int32)), 2)
            torch.cuda.synchronize()
            before = gl.table() + (gl.pinned(),)
        m.moe_offload_pin(gl.h, None, 0)  # the empty set unpins everything
        torch.cuda.synchronize()
        assert gl.pinned().sum() == 0 and gl.stats()["error"] == 0
    finally:
        gl.close()


def test_nan_logit_sets_error():
    E, S, k, H, F = 8, 4, 2, 128, 128
    host, wr, b, _ = make_layer_inputs(62, 0, E, H, F, 1, 1.2)
    gl = GpuLayer(E, S, k, H, F, 1, 4, host, wr, b)
    try:
        x = synth.tokens(62, 1, 1, H, 1, 0.0, 1)[0].copy()
        x[0, 5] = 0x7FC0
        gl.route(to_dev(x), 1)
        assert gl.stats()["error"] & m.DEV_ERR_NAN
    finally:
        gl.close()


def test_audit_flags_a_corrupted_table():
    E, S, k, H, F = 8, 4, 2, 128, 128
    host, wr, b, _ = make_layer_inputs(63, 0, E, H, F, 1, 1.2)
    gl = GpuLayer(E, S, k, H, F, 1, 4, host, wr, b)
    try:
        x = to_dev(synth.tokens(63, 1, 2, H, 1, 0.0, 1)[0])
        gl.step(x, 2)
        assert gl.stats()["error"] == 0
        so, eo, lu = gl.table()
        e = int(eo[0])
        bad = so.copy()
        bad[e] = 1 if so[e] != 1 else 2  # expert points at a slot that does not hold it
        h2d(gl.info["slot_of"], bad)
        gl.step(x, 2)
        assert gl.stats()["error"] & m.DEV_ERR_AUDIT
    finally:
        gl.close()


def test_create_rejects_bad_shapes():
    with pytest.raises(m.MoeError) as ei:
        m.moe_offload_create(8, 1, 128, 128, 2, 1, 4)  # S < k
    assert ei.value.code == m.EINVAL
    with pytest.raises(m.MoeError) as ei:
        m.moe_offload_create(8, 4, 128, 128, 2, 7, 4)  # unknown dtype
    assert ei.value.code == m.EUNSUPPORTED
    with pytest.raises(m.MoeError) as ei:
        m.moe_offload_create(8, 4, 100, 128, 2, 1, 4)  # hidden not a multiple of 128
    assert ei.value.code == m.EUNSUPPORTED
    for H, F in ((384, 256), (256, 128)):  # MXFP4: hidden and ffn must be multiples of 256
        with pytest.raises(m.MoeError) as ei:
            m.moe_offload_create(8, 4, H, F, 2, m.MXFP4, 4)
        assert ei.value.code == m.EUNSUPPORTED
    m.moe_offload_destroy(m.moe_offload_create(8, 4, 256, 256, 2, m.MXFP4, 4))
    with pytest.raises(m.MoeError) as ei:
        m.moe_offload_create(8, 4, 128, 128, 2, 1, 4, device=99)
    assert ei.value.code == m.EINVAL


@pytest.mark.parametrize("wdt,zipf", [(1, 0.0), (2, 1.2)])
def test_maximum_experts_and_top_k(wdt, zipf):
    """The largest expert count and top-k the library accepts (1024 experts, top-16), 96 slots,
    bf16 records under a uniform router (calls wider than the cache) and fp8 records with the
    shared expert under a Zipf-skewed router (mostly hits): single tokens (one work item per
    choice), decode batches, 512 pairs (the control workgroup's limit) and a call of 65 tokens
    (1040 pairs, the grouped GEMM), every call against the oracle."""
    modes, err = run_sequence(1024, 96, 16, 256, 256, wdt, zipf, 95 + wdt, 8, [1, 8, 32, 65],
                              shared=(wdt == 2))
    if zipf == 0.0:
        assert max(modes) >= 1  # some calls wider than the cache
    assert err <= 2e-2


@pytest.mark.parametrize("wdt,S,zipf", [(0, 1, 0.0), (1, 1, 0.0), (1, 8, 1.2), (2, 2, 0.0)])
def test_degenerate_top1_and_slot_counts(wdt, S, zipf):
    """Top-1 routing (every weight exactly 1) with a single slot under a uniform router (calls
    touching two experts are wider than the cache), with every expert resident (S = E), and fp8
    records with two slots; fp32, bf16 and fp8, batches 1 to 5, every call against the oracle."""
    modes, err = run_sequence(8, S, 1, 128, 256, wdt, zipf, 120 + 10 * wdt + S, 12, [1, 2, 5],
                              shared=(wdt == 2))
    if S == 1:
        assert max(modes) >= 1
    assert err <= (1e-5 if wdt == 0 else 2e-2)


def test_calls_reject_bad_sizes_and_null_pointers():
    """Call-level argument checks on a live handle: T outside [1, max_tokens], null tensors and
    install budgets outside [0, S] return EINVAL with a message and leave the state untouched."""
    E, S, k, H, F, maxT = 8, 4, 2, 128, 128, 4
    print("case call-level argument checks", flush=True)
    h = m.moe_offload_create(E, S, H, F, k, m.BF16, maxT)
    try:
        dev = torch.device("cuda", 0)
        x = torch.zeros((maxT + 1, H), dtype=torch.bfloat16, device=dev)
        wr = torch.zeros((E, H), dtype=torch.bfloat16, device=dev)
        b = torch.zeros(E, dtype=torch.float32, device=dev)
        ids = torch.zeros((maxT + 1, k), dtype=torch.int32, device=dev)
        w = torch.zeros((maxT + 1, k), dtype=torch.float32, device=dev)
        sid = torch.zeros_like(ids)
        y = torch.zeros_like(x)
        for T in (0, -1, maxT + 1):
            for call in (lambda: m.moe_route_topk(h, x, wr, b, T, ids, w),
                         lambda: m.moe_slot_ensure(h, ids, T, sid),
                         lambda: m.moe_slot_ffn(h, x, sid, w, T, None, y),
                         lambda: m.moe_prefill_stage(h, ids, T, sid),
                         lambda: m.moe_prefetch_install(h, ids, T, 1)):
                with pytest.raises(m.MoeError) as ei:
                    call()
                assert ei.value.code == m.EINVAL and "T=" in str(ei.value), (T, str(ei.value))
        for call in (lambda: m.moe_route_topk(h, None, wr, b, 1, ids, w),
                     lambda: m.moe_route_topk(h, x, wr, None, 1, ids, w),
                     lambda: m.moe_slot_ensure(h, ids, 1, None),
                     lambda: m.moe_slot_ffn(h, x, sid, w, 1, None, None),
                     lambda: m.moe_prefill_stage(h, None, 1, sid),
                     lambda: m.moe_prefetch_install(h, None, 1, 1)):
            with pytest.raises(m.MoeError) as ei:
                call()
            assert ei.value.code == m.EINVAL and "null" in str(ei.value)
        for n in (-1, S + 1):
            with pytest.raises(m.MoeError) as ei:
                m.moe_prefetch_install(h, ids, 1, n)
            assert ei.value.code == m.EINVAL
        torch.cuda.synchronize()
        st = m.moe_offload_stats(h)
        assert st["calls"] == 0 and st["resident"] == 0 and st["error"] == 0, st
    finally:
        m.moe_offload_destroy(h)


def test_graph_replay_matches_eager():
    """Two layers captured once in a HIP graph (via torch.cuda.graph) and replayed."""
    E, S, k, H, F, wdt, T = 16, 6, 4, 256, 256, 1, 3
    L = 2
    ins = [make_layer_inputs(71, l, E, H, F, wdt, 1.2) for l in range(L)]
    xs = synth.tokens(71, 4, T, H, 6, 0.9, wdt)

    def build():
        return [GpuLayer(E, S, k, H, F, wdt, T, *ins[l][:3]) for l in range(L)]

    def step(layers, x0):
        x = x0
        for gl in layers:
            gl.step(x, T)
            x = gl.xn
        return x

    eager = build()
    ref = []
    for s in range(6):
        xo = step(eager, to_dev(xs[s]))
        ref.append((to_np(xo[:T]).copy(), [gl.table() for gl in eager]))
    graphed = build()
    x_static = to_dev(xs[0])
    # warm-up on a side stream is not needed: nothing here allocates
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        out = step(graphed, x_static)
    # the capture did not execute: state is still empty
    for s in range(6):
        x_static.copy_(to_dev(xs[s]))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(out[:T]), ref[s][0]), s
        for gl, tab in zip(graphed, ref[s][1]):
            assert all(np.array_equal(p, q) for p, q in zip(gl.table(), tab))
    for gl in eager + graphed:
        gl.close()


def test_auto_slots_fill_free_memory_up_to_the_reserve():
    """moe_offload_auto_slots on the device's own free memory: `layers` handles created with the
    returned slot count (sharing one staging buffer) leave at least the reserve free, and one more
    slot per layer would not have fitted."""
    E, H, F, k, L, T = 64, 1024, 512, 4, 4, 8
    stride = 3 * H * F * 2  # bf16, a multiple of 4096
    # threshold of the rule from its arithmetic-only mode: free bytes giving exactly k slots per layer
    lo, hi = 1, 1 << 44
    while lo < hi:
        mid = (lo + hi) // 2
        try:
            m.moe_offload_auto_slots(E, H, F, k, m.BF16, T, L, 0, mid)
            hi = mid
        except m.MoeError:
            lo = mid + 1
    # the runtime's own first-use allocations (code objects, the library's device scratch array, kernel
    # resources) come with the first handle on a device: take them before measuring
    m.moe_offload_destroy(m.moe_offload_create(E, k, H, F, k, m.BF16, T, 0, 0))
    torch.cuda.synchronize()
    free_now = torch.cuda.mem_get_info()[0]
    reserve = free_now - lo - 10 * L * stride - stride // 2  # room for k + 10 slots per layer, not k + 11
    S = m.moe_offload_auto_slots(E, H, F, k, m.BF16, T, L, reserve)
    assert S == k + 10, S
    hs = []
    try:
        for l in range(L):
            hs.append(m.moe_offload_create(E, S, H, F, k, m.BF16, T, 0, 0, hs[0] if l else None,
                                           hs[0] if l else None))
        torch.cuda.synchronize()
        # allocation granularity aside (a few MiB per allocation), the reserve is still free
        assert torch.cuda.mem_get_info()[0] >= reserve - 64 * (1 << 20)
    finally:
        for h in reversed(hs):
            m.moe_offload_destroy(h)


@pytest.mark.parametrize("wdt,E,S,k,H,F,Ts,shared", [
    (1, 32, 8, 4, 512, 256, [1, 3, 9, 2], False),   # single-token and batch kernels around the host's pairs
    (2, 16, 6, 4, 256, 256, [2, 5, 70], True),      # fp8 + shared expert; 70 tokens: the grouped GEMM
    (3, 16, 8, 4, 256, 512, [1, 4], True),          # MXFP4
    (0, 8, 4, 2, 64, 128, [4, 1], False),           # fp32
])
def test_host_cold_experts_parity(wdt, E, S, k, H, F, Ts, shared):
    """Cold mode switched on mid-stream and off again: ids, slot ids, copy lists (mode COLD, index
    S + E + e), tables, scores and activation counts bit-exact against the oracle's cold rule; layer
    outputs (GPU hits + host-computed misses) within tolerance; resident slots keep their bytes."""
    print("cold wdt=%d E=%d S=%d k=%d H=%d F=%d Ts=%s" % (wdt, E, S, k, H, F, Ts), flush=True)
    host, wr, b, sh = make_layer_inputs(51, 0, E, H, F, wdt, 0.0, shared)  # flat routing: misses in every phase
    gl = GpuLayer(E, S, k, H, F, wdt, max(Ts), host, wr, b, shared=sh)
    ol = oracle.Layer(E, S, k, H, F, wdt, host, wr, b, shared=sh)
    steps = 16
    xs = synth.tokens(51, 7, max(Ts), H, steps, 0.0, wdt)
    st = torch.cuda.current_stream()
    cold_seen = 0
    try:
        for s in range(steps):
            if s == 4:
                chosen, _, _ = m.moe_offload_set_cold(gl.h, m.COLD_ON, st)
                assert chosen == 1
                ol.cache.set_cold(True)
            if s == 12:
                assert m.moe_offload_set_cold(gl.h, m.COLD_OFF, st)[0] == 0
                ol.cache.set_cold(False)
            cold = 4 <= s < 12
            T = Ts[s % len(Ts)]
            x = np.ascontiguousarray(xs[s][:T])
            xd = to_dev(x)
            gl.route(xd, T)
            gl.ensure(T)
            gl.copy()
            if cold:
                with pytest.raises(m.MoeError) as ei:
                    gl.ffn(xd, T)
                assert ei.value.code == m.EINVAL
                m.moe_slot_ffn_host_cold(gl.h, xd, gl.slot_ids, gl.w, T, gl.shared, gl.y, None, gl.xn, st)
            else:
                gl.ffn(xd, T)
            r = ol.step(x)
            assert r["mode"] == (oracle.COLD if cold else r["mode"])
            if cold:
                cold_seen += len(r["pairs"])
            compare_call(gl, r, T, r["y64"], oracle_cache=ol.cache)
            assert np.array_equal(to_np(gl.xn[:T]), oracle.residual(x, to_np(gl.y[:T]), wdt))
        stt = gl.stats()
        c = ol.cache.counters()
        assert stt["error"] == 0 and stt["cold_misses"] == c["cold"] == cold_seen and cold_seen > 0
        for key in ("calls", "hits", "misses", "staged_calls", "staged_copies"):
            assert stt[key] == c[key], key
        so, eo, lu = gl.table()
        rb = oracle.record_bytes(wdt, H, F)
        for s_ in range(S):
            if eo[s_] >= 0:
                assert np.array_equal(gl.slot_bytes(s_, rb), host[eo[s_], :rb])
    finally:
        gl.close()


@pytest.mark.parametrize("wdt,E,S,k,H,F,Ts,shared,q", [
    (1, 32, 8, 4, 512, 256, [9, 3, 16, 1], False, 128),   # half of the staged misses on the host
    (2, 16, 6, 4, 256, 256, [5, 70, 2], True, 256),       # fp8 + shared; every staged miss on the host
    (3, 16, 8, 4, 256, 512, [8, 4], True, 77),            # MXFP4
    (0, 8, 4, 2, 64, 128, [4, 1], False, 0),              # fp32; q = 0: the link carries every staged miss
    (1, 32, 8, 4, 512, 256, [12, 6], False, None),         # q from the measured host and link times
])
def test_split_mode_parity(wdt, E, S, k, H, F, Ts, shared, q):
    """Split mode switched on mid-stream and off again: of each overflowing call's staged misses the last
    share q/256 (ascending id) is computed on the host (index S + E + e), the rest is staged over the link;
    ids, slot ids, copy lists, tables, scores, activation counts and counters bit-exact against the
    oracle's split rule; layer outputs within tolerance; staged and resident records hold their bytes."""
    print("split wdt=%d E=%d S=%d k=%d H=%d F=%d Ts=%s q=%s" % (wdt, E, S, k, H, F, Ts, q), flush=True)
    host, wr, b, sh = make_layer_inputs(53, 0, E, H, F, wdt, 0.0, shared)
    gl = GpuLayer(E, S, k, H, F, wdt, max(Ts), host, wr, b, shared=sh)
    ol = oracle.Layer(E, S, k, H, F, wdt, host, wr, b, shared=sh)
    steps = 14
    xs = synth.tokens(53, 9, max(Ts), H, steps, 0.0, wdt)
    st = torch.cuda.current_stream()
    rb = oracle.record_bytes(wdt, H, F)
    host_seen = staged_seen = 0
    try:
        for s in range(steps):
            if s == 3:
                if q is None:
                    qq, cpu_us, link_us = m.moe_offload_set_cold(gl.h, m.COLD_SPLIT, st)
                    print("split: host FFN %.1f us, link %.1f us per record -> q %d" % (cpu_us, link_us, qq),
                          flush=True)
                    assert cpu_us > 0 and link_us > 0 and 0 <= qq <= 256
                    assert qq == int(np.floor(256.0 * link_us / (cpu_us + link_us) + 0.5)) or \
                        abs(qq - 256.0 * link_us / (cpu_us + link_us)) <= 0.5 + 1e-9
                else:
                    qq = q
                    m.moe_offload_set_split(gl.h, q, st)
                ol.cache.set_split(qq)
            if s == 11:
                assert m.moe_offload_set_cold(gl.h, m.COLD_OFF, st)[0] == 0
                ol.cache.set_cold(False)
            split = 3 <= s < 11
            T = Ts[s % len(Ts)]
            x = np.ascontiguousarray(xs[s][:T])
            xd = to_dev(x)
            gl.route(xd, T)
            gl.ensure(T)
            gl.copy()
            if split:
                with pytest.raises(m.MoeError) as ei:
                    gl.ffn(xd, T)
                assert ei.value.code == m.EINVAL
                m.moe_slot_ffn_host_cold(gl.h, xd, gl.slot_ids, gl.w, T, gl.shared, gl.y, None, gl.xn, st)
            else:
                gl.ffn(xd, T)
            r = ol.step(x)
            if split:
                recs = [int(p_[1]) for p_ in r["pairs"]]
                host_seen += sum(1 for v in recs if v >= S + E)
                staged_seen += sum(1 for v in recs if S <= v < S + E)
            compare_call(gl, r, T, r["y64"], oracle_cache=ol.cache)
            assert np.array_equal(to_np(gl.xn[:T]), oracle.residual(x, to_np(gl.y[:T]), wdt))
            if r["mode"] == oracle.STAGED:  # the staged records crossed the link, the host's did not need to
                for e_, v in r["pairs"]:
                    if S <= v < S + E:
                        assert np.array_equal(gl.staging_bytes(int(e_), rb), host[int(e_), :rb])
        stt = gl.stats()
        c = ol.cache.counters()
        assert stt["error"] == 0 and stt["cold_misses"] == c["cold"] == host_seen
        for key in ("calls", "hits", "misses", "staged_calls", "staged_copies"):
            assert stt[key] == c[key], key
        if q == 256:
            assert host_seen > 0 and staged_seen == 0
        elif q == 0:
            assert host_seen == 0 and staged_seen > 0
        elif q is not None:
            assert host_seen > 0 and staged_seen > 0
        for s_ in range(S):
            so, eo, lu = gl.table()
            if eo[s_] >= 0:
                assert np.array_equal(gl.slot_bytes(s_, rb), host[eo[s_], :rb])
    finally:
        gl.close()


def test_split_mode_small_calls_take_the_plain_ffn():
    """Split mode: a call of at most S - P pairs (P pinned experts) cannot overflow, so
    moe_slot_ffn_host_cold runs it with no host round trip: outputs bit for bit those of a twin layer
    with the mode off, tables and lists bit-exact against the oracle's split rule.  With P = 3 pinned,
    3-token calls (6 pairs > S - P = 5) take the host path again and stay within tolerance."""
    E, S, k, H, F, wdt = 16, 8, 2, 256, 512, 1
    host, wr, b, _ = make_layer_inputs(58, 0, E, H, F, wdt, 1.2)
    split = GpuLayer(E, S, k, H, F, wdt, 4, host, wr, b)
    plain = GpuLayer(E, S, k, H, F, wdt, 4, host, wr, b)
    ol = oracle.Layer(E, S, k, H, F, wdt, host, wr, b)
    st = torch.cuda.current_stream()
    Ts = [1, 2, 4, 1, 3, 4, 2, 3, 2, 3]
    xs = synth.tokens(58, 2, 4, H, len(Ts), 0.0, wdt)
    try:
        m.moe_offload_set_split(split.h, 128, st)
        ol.cache.set_split(128)
        for s, T in enumerate(Ts):
            if s == 6:  # pin 3 experts on both layers and in the oracle: S - P = 5
                P = np.array([0, 5, 9], np.int32)
                for gl in (split, plain):
                    m.moe_offload_pin(gl.h, to_dev(P), len(P), st)
                ol.cache.copy(0, ol.cache.pin(P))
            x = np.ascontiguousarray(xs[s][:T])
            xd = to_dev(x)
            for gl in (split, plain):
                gl.route(xd, T)
                gl.ensure(T)
                gl.copy()
            m.moe_slot_ffn_host_cold(split.h, xd, split.slot_ids, split.w, T, None, split.y, None, split.xn, st)
            plain.ffn(xd, T)
            r = ol.step(x)
            compare_call(split, r, T, r["y64"], oracle_cache=ol.cache)
            if T * k <= S - (3 if s >= 6 else 0):
                assert np.array_equal(to_np(split.y[:T]), to_np(plain.y[:T])), (s, T)
                assert np.array_equal(to_np(split.xn[:T]), to_np(plain.xn[:T])), (s, T)
        assert split.stats()["error"] == 0
    finally:
        split.close()
        plain.close()


@pytest.mark.parametrize("wdt,E,S,k,H,F,Ts,shared", [
    (1, 8, 4, 2, 512, 256, [8, 16, 20, 48], False),   # bf16: the automatic rule takes the GEMM from 5 pairs per expert
    (2, 64, 12, 2, 256, 256, [2, 3, 4, 16], True),    # fp8 + shared: from 1/8
    (3, 16, 8, 4, 256, 512, [2, 3, 4, 12], False),    # MXFP4: from 1
])
def test_ffn_path_choice_parity(wdt, E, S, k, H, F, Ts, shared):
    """The same calls through the decode kernels, the grouped GEMM and the automatic choice: each within
    tolerance of the oracle; the automatic choice bitwise equal to the pair its rule names; and under the
    automatic choice the outputs at S slots bitwise equal those of a layer holding every expert."""
    print("ffn path wdt=%d E=%d S=%d k=%d H=%d F=%d Ts=%s" % (wdt, E, S, k, H, F, Ts), flush=True)
    host, wr, b, sh = make_layer_inputs(57, 0, E, H, F, wdt, 0.0, shared)
    st = torch.cuda.current_stream()
    layers = [GpuLayer(E, S_, k, H, F, wdt, max(Ts), host, wr, b, shared=sh) for S_ in (S, E)]
    ol = oracle.Layer(E, E, k, H, F, wdt, host, wr, b, shared=sh)
    xs = synth.tokens(57, 3, max(Ts), H, len(Ts), 0.0, wdt)
    c8 = {1: 40, 2: 1, 3: 8}[wdt]  # the GEMM from c8 / 8 pairs per expert
    try:
        for s, T in enumerate(Ts):
            x = np.ascontiguousarray(xs[s][:T])
            xd = to_dev(x)
            r = ol.step(x)
            outs = {}
            for li, gl in enumerate(layers):
                gl.route(xd, T)
                gl.ensure(T)
                gl.copy()
                for path in (m.FFN_DECODE, m.FFN_GEMM, m.FFN_AUTO):
                    m.moe_offload_set_ffn_path(gl.h, path)
                    gl.ffn(xd, T)
                    y = to_np(gl.y[:T])
                    assert row_rel_err(y, r["y64"], wdt) <= TOL[wdt], (T, li, path)
                    outs[(li, path)] = y
            want = m.FFN_GEMM if 8 * T * k >= c8 * E else m.FFN_DECODE
            assert np.array_equal(outs[(0, m.FFN_AUTO)], outs[(0, want)]), T
            for path in (m.FFN_DECODE, m.FFN_GEMM, m.FFN_AUTO):  # slot-count invariance on every path
                assert np.array_equal(outs[(0, path)], outs[(1, path)]), (T, path)
        for gl in layers:
            assert gl.stats()["error"] == 0
        with pytest.raises(m.MoeError):
            m.moe_offload_set_ffn_path(layers[0].h, 3)
        for bad in (-1, 1, 2, 5, 16):
            with pytest.raises(m.MoeError):
                m.moe_offload_set_gemm_waves(layers[0].h, bad)
    finally:
        for gl in layers:
            gl.close()


def test_host_cold_policy_measures_both_paths():
    """MOE_COLD_AUTO: the host FFN of one record against one record over the link, measured on this machine;
    the layer goes cold exactly when the host is faster, and the device flag follows (the next ensure
    lists its misses as cold or loads them)."""
    E, S, k, H, F = 16, 4, 4, 2048, 768
    host, wr, b, _ = make_layer_inputs(52, 0, E, H, F, 1, 1.2)
    gl = GpuLayer(E, S, k, H, F, 1, 4, host, wr, b)
    st = torch.cuda.current_stream()
    try:
        chosen, cpu_us, link_us = m.moe_offload_set_cold(gl.h, m.COLD_AUTO, st)
        print("cold policy: host FFN %.1f us, link %.1f us per record -> %s" %
              (cpu_us, link_us, "host" if chosen else "link"), flush=True)
        assert cpu_us > 0 and link_us > 0 and chosen == int(cpu_us < link_us)
        x = to_dev(synth.tokens(52, 1, 4, H, 1, 0.0, 1)[0])
        gl.route(x, 4)
        gl.ensure(4)
        mode, pairs = gl.copy_list()
        assert len(pairs) > 0 and (mode == m.MODE_COLD) == bool(chosen)
    finally:
        gl.close()

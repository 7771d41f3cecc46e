"""GPU parity of the Qwen3-30B-A3B-shaped decode chain at full size, in the
launch configuration the benchmark times: 48 layers x 128 experts, top-8,
hidden 2048, moe ffn 768, 26 slots per layer, bf16, every layer's 128 records
(58 GB) in pinned host memory, the whole decode step replayed as one HIP graph
at batch 1, 8 and 32, and the router-lookahead prefetch variant (4 installs
per layer); and the same chain with MXFP4 records at batch 1.

Every call is teacher-forced (the oracle routes the GPU's own block input) and
checked bit for bit on ids, slot ids, copy lists, prefetch lists, slot tables
and counters; weights within 1e-5.  Expert outputs are sampled (a few token
rows of a few calls, computed one by one by the oracle straight from the host
records of the routed experts, independent of any slot map) and must be within
2e-2 of the oracle's double sums; the residual stream is checked bitwise on
every layer, and the slot bytes of two layers against the host records.
"""
import time

import numpy as np
import pytest
import torch

import expert_offload_slot_amd as m
import oracle
import synth
from gpu_harness import d2h, hip, row_rel_err, to_dev

pytestmark = pytest.mark.gpu

BF16, FP8, MXFP4 = 1, 2, 3


def log(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------------------------- Qwen3-30B chain

class Qwen3Model:
    L, E, k, H, F, S, MAX_T = 48, 128, 8, 2048, 768, 26, 32

    def __init__(self, seed=0, wdt=BF16):
        t0 = time.time()
        self.seed, self.wdt = seed, wdt  # weight format; activations and routers are bf16
        self.handles = []
        for l in range(self.L):
            self.handles.append(m.moe_offload_create(self.E, self.S, self.H, self.F, self.k, wdt, self.MAX_T, 0,
                                                     m.FLAG_AUDIT, None, self.handles[0] if l else None))
        self.info = [m.moe_offload_query(h) for h in self.handles]
        self.stride = self.info[0]["record_stride"]
        self.rb = self.info[0]["record_bytes"]
        for l, h in enumerate(self.handles):
            p, _, _ = m.moe_offload_host_records(h)
            synth.fill_records(seed, l, 0, self.E, self.H, self.F, wdt, p, self.stride)
        self.hosts = [m.host_array(h, self.E) for h in self.handles]
        self.routers = [synth.router(seed, l, self.E, self.H, BF16, zipf_s=1.2) for l in range(self.L)]
        self.wr = [to_dev(w) for w, _ in self.routers]
        self.b = [to_dev(b) for _, b in self.routers]
        log("qwen3 model: %d layers, %.1f GB host store, %.0f s" % (self.L, self.L * self.E * self.stride / 1e9,
                                                                     time.time() - t0))

    def reset(self):
        for h in self.handles:
            m.moe_offload_reset(h)
        torch.cuda.synchronize()
        return [oracle.Cache(self.E, self.S) for _ in range(self.L)]

    def close(self):
        for h in reversed(self.handles):
            m.moe_offload_destroy(h)


class Chain:
    def __init__(self, model, T, prefetch_n, tag):
        self.mo, self.T, self.pf = model, T, prefetch_n
        self.c = m.moe_chain_create(model.handles, model.wr, model.b, T, prefetch_n)
        self.bufs = m.moe_chain_get_buffers(self.c)
        self.xs = synth.tokens(model.seed, tag, T, model.H, 64, 0.9, BF16)

    def run(self, s):
        xd = to_dev(np.ascontiguousarray(self.xs[s]))
        torch.cuda.synchronize()
        assert hip().hipMemcpy(self.bufs["x"], xd.data_ptr(), xd.numel() * 2, 3) == 0
        m.moe_chain_run(self.c, torch.cuda.current_stream())
        torch.cuda.synchronize()

    def snapshot(self):
        L, T, H, k = self.mo.L, self.T, self.mo.H, self.mo.k
        return dict(
            x=d2h(self.bufs["x"], (L + 1) * T * H * 2, np.uint16).reshape(L + 1, T, H),
            xn=d2h(self.bufs["xn"], L * T * H * 2, np.uint16).reshape(L, T, H),
            y=d2h(self.bufs["y"], L * T * H * 2, np.uint16).reshape(L, T, H),
            ids=d2h(self.bufs["ids"], L * T * k * 4, np.int32).reshape(L, T, k),
            w=d2h(self.bufs["w"], L * T * k * 4, np.float32).reshape(L, T, k),
            sid=d2h(self.bufs["slot_ids"], L * T * k * 4, np.int32).reshape(L, T, k),
        )

    def close(self):
        m.moe_chain_destroy(self.c)


def layer_lists(mo, l):
    i = mo.info[l]
    lst = d2h(i["copy_list"], 4 * (2 + 2 * max(mo.S, mo.E)), np.int32)
    pf = d2h(i["prefetch_list"], 4 * (2 + 2 * mo.S), np.int32)
    so = d2h(i["slot_of"], 4 * mo.E, np.int32)
    eo = d2h(i["expert_of"], 4 * mo.S, np.int32)
    lu = d2h(i["last_use"], 8 * mo.S, np.uint64)
    sc = d2h(i["score"], 4 * mo.S, np.uint32)
    return (int(lst[0]), lst[2:2 + 2 * lst[1]].reshape(-1, 2)), pf[2:2 + 2 * pf[1]].reshape(-1, 2), (so, eo, lu, sc)


def replay_step(mo, caches, snap, T, prefetch_n, ffn_layers=(), ffn_tokens=()):
    """Teacher-forced oracle for one chain step over all layers; returns the largest sampled row error."""
    worst = 0.0
    installs = {}
    for l in range(mo.L):
        xn = snap["xn"][l]
        ref_xn = oracle.rmsnorm(snap["x"][l], BF16)
        assert np.array_equal(xn, ref_xn), l
        wr, b = mo.routers[l]
        ids, w, _ = oracle.route(xn, wr, b, mo.k, BF16)
        assert np.array_equal(ids, snap["ids"][l]), (l, ids, snap["ids"][l])
        assert np.abs(snap["w"][l] - w).max() <= 1e-5, l
        sid, mode, pairs = caches[l].ensure(ids)
        assert np.array_equal(sid, snap["sid"][l]), l
        (gmode, gpairs), gpf, (so, eo, lu, sc) = layer_lists(mo, l)
        assert gmode == mode and np.array_equal(gpairs, pairs), (l, gmode, gpairs, mode, pairs)
        if l in installs:
            assert np.array_equal(gpf, installs[l]), (l, gpf, installs[l])
        if prefetch_n and l + 1 < mo.L:
            pred, _, _ = oracle.route(xn, mo.routers[l + 1][0], mo.routers[l + 1][1], mo.k, BF16)
            installs[l + 1] = caches[l + 1].install(pred, prefetch_n)
        oso, oeo, olu, _ = caches[l].state()
        assert np.array_equal(so, oso) and np.array_equal(eo, oeo) and np.array_equal(lu, olu), l
        assert np.array_equal(sc, caches[l].scores()), l
        if l in ffn_layers:
            toks = [t for t in ffn_tokens if t < T]
            _, y64 = oracle.ffn(xn[toks], mo.wdt, mo.H, mo.F, oracle.host_records(mo.hosts[l], ids[toks]),
                                w[toks], want_f64=True)
            err = row_rel_err(snap["y"][l][toks], y64, BF16)
            assert err <= 2e-2, (l, err)
            worst = max(worst, err)
        assert np.array_equal(snap["x"][l + 1], oracle.residual(snap["x"][l], snap["y"][l], BF16)), l
    return worst


def check_counters(mo, caches):
    for l, h in enumerate(mo.handles):
        st = m.moe_offload_stats(h)
        c = caches[l].counters()
        assert st["error"] == 0, (l, st["error"])
        for key in ("calls", "hits", "misses", "staged_calls", "staged_copies", "prefetch_installs", "prefetch_hits"):
            assert st[key] == c[key], (l, key, st[key], c[key])


def check_slot_bytes(mo, layers):
    for l in layers:
        eo = d2h(mo.info[l]["expert_of"], 4 * mo.S, np.int32)
        for s in range(mo.S):
            if eo[s] >= 0:
                got = d2h(mo.info[l]["slots"] + s * mo.stride, mo.rb)
                assert np.array_equal(got, mo.hosts[l][eo[s], :mo.rb]), (l, s, eo[s])


def test_qwen3_mxfp4_chain_full_size():
    """The same 48-layer chain with MXFP4 expert records (2.5 MB each, 15 GB host store), batch 1.  It runs
    before the module's bf16 model exists and frees its own: both host stores at once exceed what the host
    lets a process pin."""
    mo = Qwen3Model(seed=1, wdt=MXFP4)
    try:
        caches = mo.reset()
        ch = Chain(mo, 1, 0, 401)
        try:
            worst = 0.0
            for s in range(12):
                log("qwen3 mxfp4 chain step %d" % s)
                ch.run(s)
                snap = ch.snapshot()
                sample = s in (0, 6, 11)
                worst = max(worst, replay_step(mo, caches, snap, 1, 0, (0, 17, 47) if sample else (), (0,)))
            log("qwen3 mxfp4 chain: 12 steps bit-exact, sampled rows within %.2e" % worst)
        finally:
            ch.close()
        check_counters(mo, caches)
        check_slot_bytes(mo, (0, 47))
    finally:
        mo.close()


@pytest.fixture(scope="module")
def qwen3():
    mo = Qwen3Model()
    yield mo
    mo.close()


def test_qwen3_chain_full_size_batches_1_8_32(qwen3):
    mo = qwen3
    caches = mo.reset()
    plan = [(1, 20, set(range(20)), (0, 1, 23, 47), (0,)),
            (8, 16, set(range(16)), (0, 47), (0, 7)),
            (32, 16, set(range(16)), (0, 31), (0, 13, 31))]
    for T, steps, ffn_steps, ffn_layers, toks in plan:
        ch = Chain(mo, T, 0, 200 + T)
        try:
            worst = 0.0
            for s in range(steps):
                log("qwen3 chain T=%d step %d" % (T, s))
                ch.run(s)
                snap = ch.snapshot()
                sample = s in ffn_steps
                # sampled rows move over the batch step by step, so every token row is checked somewhere
                rows = tuple(sorted({(t + s) % T for t in toks}))
                worst = max(worst, replay_step(mo, caches, snap, T, 0, ffn_layers if sample else (), rows))
            log("qwen3 chain T=%d: %d steps bit-exact, sampled rows within %.2e" % (T, steps, worst))
        finally:
            ch.close()
    check_counters(mo, caches)
    check_slot_bytes(mo, (0, 47))


def test_qwen3_chain_host_computed_full_size(qwen3):
    """The 48-layer chain with every layer in cold mode (the cache warmed over the link for 8 steps, then
    frozen; the chain's host thread computes every miss): batch 1 and 8, ids, slot ids (S + E + e for the
    host's pairs), copy lists, tables and counters bit-exact against the oracle's cold rule, sampled
    output rows within tolerance, the graph captured again when the mode switches."""
    mo = qwen3
    st = torch.cuda.current_stream()
    for T, toks in ((1, (0,)), (8, (0, 7))):
        caches = mo.reset()
        for cache in caches:
            cache.set_cold(False)
        ch = Chain(mo, T, 0, 400 + T)
        host_pairs = 0
        try:
            worst = 0.0
            for s in range(14):
                if s == 8:
                    for l, h in enumerate(mo.handles):
                        assert m.moe_offload_set_cold(h, m.COLD_ON, st)[0] == 1
                        caches[l].set_cold(True)
                log("qwen3 chain host-computed T=%d step %d" % (T, s))
                ch.run(s)
                snap = ch.snapshot()
                host_pairs += int((snap["sid"] >= mo.S + mo.E).sum())
                rows = tuple(sorted({(t + s) % T for t in toks}))
                worst = max(worst, replay_step(mo, caches, snap, T, 0, (0, 23, 47) if s >= 8 else (), rows))
            for l, h in enumerate(mo.handles):
                stt = m.moe_offload_stats(h)
                assert stt["cold_misses"] == caches[l].counters()["cold"], l
            check_counters(mo, caches)
            assert host_pairs > 0
            log("qwen3 chain host-computed T=%d: 14 steps bit-exact, %d host pairs, sampled rows within %.2e" %
                (T, host_pairs, worst))
        finally:
            for l, h in enumerate(mo.handles):
                m.moe_offload_set_cold(h, m.COLD_OFF, st)
            ch.close()


def test_qwen3_lookahead_prefetch_full_size(qwen3):
    mo = qwen3
    T, steps = 1, 16
    outs, misses = {}, {}
    for n in (4, 0):
        caches = mo.reset()
        ch = Chain(mo, T, n, 300)
        try:
            xs_out = []
            for s in range(steps):
                log("qwen3 prefetch=%d step %d" % (n, s))
                ch.run(s)
                snap = ch.snapshot()
                replay_step(mo, caches, snap, T, n, (0, 47) if s in (0, steps - 1) else (), (0,))
                xs_out.append(snap["x"].copy())
            outs[n] = xs_out
        finally:
            ch.close()
        check_counters(mo, caches)
        misses[n] = sum(m.moe_offload_stats(h)["misses"] for h in mo.handles)
        if n:
            st = [m.moe_offload_stats(h) for h in mo.handles]
            log("prefetch: installs %d, prefetch hits %d" % (sum(x["prefetch_installs"] for x in st),
                                                            sum(x["prefetch_hits"] for x in st)))
    for a, b in zip(outs[4], outs[0]):
        assert np.array_equal(a, b)
    log("demand misses over %d steps: %d without prefetch, %d with" % (steps, misses[0], misses[4]))
    assert misses[4] <= misses[0]



def test_qwen3_slot_fractions_bitwise_identical_full_size(qwen3):
    """The pages' invariant at full size: the first 4 layers of the Qwen3 shape at 13, 26, 52 and 128 slots
    (10 / 20 / 40 / 100 %), each from an empty cache on the same token stream, read the same host records
    (one shared store) and must give bitwise identical block inputs and outputs on every layer and step,
    while the smallest cache misses more often than the larger ones."""
    mo = qwen3
    L, steps, T = 4, 48, 1
    xs = synth.tokens(mo.seed, 500, T, mo.H, steps, 0.9, BF16)
    runs, misses = {}, {}
    for S in (13, 26, 52, 128):
        hs = []
        try:
            for l in range(L):
                hs.append(m.moe_offload_create(mo.E, S, mo.H, mo.F, mo.k, BF16, 1, 0, m.FLAG_AUDIT, mo.handles[l],
                                               mo.handles[0]))
            c = m.moe_chain_create(hs, mo.wr[:L], mo.b[:L], T, 0)
            try:
                bufs = m.moe_chain_get_buffers(c)
                out = []
                for s in range(steps):
                    xd = to_dev(np.ascontiguousarray(xs[s]))
                    torch.cuda.synchronize()
                    assert hip().hipMemcpy(bufs["x"], xd.data_ptr(), xd.numel() * 2, 3) == 0
                    m.moe_chain_run(c, torch.cuda.current_stream())
                    torch.cuda.synchronize()
                    out.append((d2h(bufs["x"], (L + 1) * T * mo.H * 2, np.uint16),
                                d2h(bufs["y"], L * T * mo.H * 2, np.uint16),
                                d2h(bufs["slot_ids"], L * T * mo.k * 4, np.int32)))
                runs[S] = out
            finally:
                m.moe_chain_destroy(c)
            misses[S] = sum(m.moe_offload_stats(h)["misses"] for h in hs)
            assert all(m.moe_offload_stats(h)["error"] == 0 for h in hs)
        finally:
            for h in reversed(hs):
                m.moe_offload_destroy(h)
        log("slots %d: %d misses over %d steps x %d layers" % (S, misses[S], steps, L))
    for S in (13, 52, 128):
        for s in range(steps):
            assert np.array_equal(runs[S][s][0], runs[26][s][0]), (S, s, "x")
            assert np.array_equal(runs[S][s][1], runs[26][s][1]), (S, s, "y")
    # over these 48 steps 26 slots may already hold every expert the 4 layers use: then only the
    # compulsory misses remain from 26 slots up
    assert misses[13] > misses[26] >= misses[52] >= misses[128]


def test_qwen3_split_mode_full_size(qwen3):
    """Split and cold mode at full size: the first 8 layers of the Qwen3 shape at batch 32 (nearly every call
    wider than its 26 slots), entry-point calls per layer; 6 steps with the share q measured per layer
    (MOE_COLD_SPLIT), then 3 steps with the warmed cache frozen and every miss on the host (MOE_COLD_ON).
    Teacher-forced: block inputs, ids, slot ids, copy lists (staged records at S + e, host-computed ones at
    S + E + e), slot tables and counters bit-exact against the oracle's split and cold rules; sampled output
    rows within 2e-2 of the plain definition from the host records; the residual stream bitwise."""
    mo = qwen3
    L, T, steps, split_steps = 8, 32, 9, 6
    caches = mo.reset()
    st = torch.cuda.current_stream()
    dev = torch.device("cuda", 0)
    x = [torch.empty((T, mo.H), dtype=torch.bfloat16, device=dev) for _ in range(L + 1)]
    xn = [torch.empty_like(x[0]) for _ in range(L)]
    y = [torch.empty_like(x[0]) for _ in range(L)]
    ids = torch.empty((T, mo.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, mo.k), dtype=torch.float32, device=dev)
    sid = torch.empty_like(ids)
    xs = synth.tokens(mo.seed, 321, T, mo.H, steps, 0.9, BF16)
    host_seen = 0
    try:
        for l in range(L):
            q, cpu_us, link_us = m.moe_offload_set_cold(mo.handles[l], m.COLD_SPLIT, st)
            caches[l].set_split(q)
            log("layer %d: host %.1f us, link %.1f us per record -> q %d" % (l, cpu_us, link_us, q))
        worst = 0.0
        for s in range(steps):
            if s == split_steps:  # freeze the warmed cache: every miss on the host from here on
                for l in range(L):
                    assert m.moe_offload_set_cold(mo.handles[l], m.COLD_ON, st)[0] == 1
                    caches[l].set_cold(True)
            log("qwen3 split T=%d step %d" % (T, s))
            x[0].copy_(to_dev(np.ascontiguousarray(xs[s])))
            for l in range(L):
                h = mo.handles[l]
                m.moe_rmsnorm(x[l], xn[l], T, mo.H, BF16, stream=st)
                m.moe_route_topk(h, xn[l], mo.wr[l], mo.b[l], T, ids, w, st)
                m.moe_slot_ensure(h, ids, T, sid, st)
                m.moe_copy_misses(h, st)
                m.moe_slot_ffn_host_cold(h, xn[l], sid, w, T, None, y[l], x[l], x[l + 1], st)
                torch.cuda.synchronize()
                # teacher-forced oracle for this layer
                gx = d2h(x[l].data_ptr(), T * mo.H * 2, np.uint16).reshape(T, mo.H)
                gxn = d2h(xn[l].data_ptr(), T * mo.H * 2, np.uint16).reshape(T, mo.H)
                assert np.array_equal(gxn, oracle.rmsnorm(gx, BF16)), (s, l)
                wr, b = mo.routers[l]
                oids, ow, _ = oracle.route(gxn, wr, b, mo.k, BF16)
                assert np.array_equal(oids, d2h(ids.data_ptr(), T * mo.k * 4, np.int32).reshape(T, mo.k)), (s, l)
                assert np.abs(d2h(w.data_ptr(), T * mo.k * 4, np.float32).reshape(T, mo.k) - ow).max() <= 1e-5
                osid, mode, pairs = caches[l].ensure(oids)
                assert np.array_equal(osid, d2h(sid.data_ptr(), T * mo.k * 4, np.int32).reshape(T, mo.k)), (s, l)
                (gmode, gpairs), _, (so, eo, lu, sc) = layer_lists(mo, l)
                assert gmode == mode and np.array_equal(gpairs, pairs), (s, l, gmode, mode)
                host_seen += int((pairs[:, 1] >= mo.S + mo.E).sum()) if len(pairs) else 0
                oso, oeo, olu, _ = caches[l].state()
                assert np.array_equal(so, oso) and np.array_equal(eo, oeo) and np.array_equal(lu, olu), (s, l)
                gy = d2h(y[l].data_ptr(), T * mo.H * 2, np.uint16).reshape(T, mo.H)
                if l in (0, 5):
                    toks = sorted({(t + 5 * s) % T for t in (0, 11, 31)})
                    _, y64 = oracle.ffn(gxn[toks], BF16, mo.H, mo.F, oracle.host_records(mo.hosts[l], oids[toks]),
                                        ow[toks], want_f64=True)
                    err = row_rel_err(gy[toks], y64, BF16)
                    assert err <= 2e-2, (s, l, err)
                    worst = max(worst, err)
                gx1 = d2h(x[l + 1].data_ptr(), T * mo.H * 2, np.uint16).reshape(T, mo.H)
                assert np.array_equal(gx1, oracle.residual(gx, gy, BF16)), (s, l)
        for l in range(L):
            stt = m.moe_offload_stats(mo.handles[l])
            c = caches[l].counters()
            assert stt["error"] == 0
            for key in ("calls", "hits", "misses", "staged_calls", "staged_copies"):
                assert stt[key] == c[key], (l, key)
            assert stt["cold_misses"] == c["cold"], l
        assert host_seen > 0
        log("qwen3 split/cold: %d steps x %d layers bit-exact, %d host-computed records, sampled rows within %.2e"
            % (steps, L, host_seen, worst))
    finally:
        for l in range(L):
            m.moe_offload_set_cold(mo.handles[l], m.COLD_OFF, st)
        mo.reset()

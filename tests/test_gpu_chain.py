"""GPU parity of the decode-step chain (norm, route, ensure, copy, FFN + residual
per layer, captured in one HIP graph) and of its router-lookahead prefetch variant.

Per step and layer the oracle is teacher-forced with the GPU's own block input
xn_l (so the bit-exact routing comparison is on identical inputs), keeps its own
cache per layer (with installs for the prefetch variant), and must match ids,
slot ids, demand and prefetch copy lists, and slot tables bit for bit, and the
outputs within 2e-2.
"""
import numpy as np
import pytest
import torch

import expert_offload_slot_amd as m
import oracle
import synth
from gpu_harness import act_f64, d2h, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def test_rmsnorm_parity():
    for wdt, H, T in [(1, 2048, 5), (1, 256, 33), (0, 64, 7), (1, 7168, 3), (0, 2048, 2)]:
        x = synth.tokens(91, 1, T, H, 1, 0.0, wdt)[0] * (3 if wdt == 0 else 1)
        x = np.ascontiguousarray(x)
        xd = to_dev(x)
        out = torch.empty_like(xd)
        m.moe_rmsnorm(xd, out, T, H, wdt, stream=torch.cuda.current_stream())
        got = to_np(out)
        ref = oracle.rmsnorm(x, wdt)
        assert np.array_equal(got, ref), (wdt, H, T)  # one binary32 order on both sides: the same codes


class ChainModel:
    def __init__(self, L, E, S, k, H, F, wdt, T, seed, prefetch_n=0, zipf=1.2, rho=0.9, shared=False, scored=False,
                 policy_flag=0):
        self.L, self.E, self.S, self.k, self.H, self.F, self.wdt, self.T = L, E, S, k, H, F, wdt, T
        self.hosts, self.routers, self.handles, self.shared = [], [], [], []
        rdt = 1 if wdt >= 2 else wdt  # fp8 and MXFP4 layers take a bf16 router and bf16 activations
        for l in range(L):
            self.hosts.append(synth.records(seed, l, E, H, F, wdt))
            self.routers.append(synth.router(seed, l, E, H, rdt, zipf_s=zipf))
            self.shared.append(synth.records(seed, l, 1, H, F, wdt, shared=True)[0] if shared else None)
            h = m.moe_offload_create(E, S, H, F, k, wdt, T, 0,
                                     m.FLAG_AUDIT | (m.FLAG_SCORED if scored else 0) | policy_flag,
                                     None, self.handles[0] if l else None)
            m.host_array(h, E)[:, :self.hosts[l].shape[1]] = self.hosts[l]
            self.handles.append(h)
        self.wr = [to_dev(w) for w, _ in self.routers]
        self.b = [to_dev(b) for _, b in self.routers]
        self.sh = [to_dev(s) for s in self.shared] if shared else None
        self.chain = m.moe_chain_create(self.handles, self.wr, self.b, T, prefetch_n, self.sh)
        self.bufs = m.moe_chain_get_buffers(self.chain)
        self.info = [m.moe_offload_query(h) for h in self.handles]
        self.xs = synth.tokens(seed, 5, T, H, 64, rho, rdt)
        self.act = 4 if wdt == 0 else 2

    def run(self, s, graph=True):
        xd = to_dev(np.ascontiguousarray(self.xs[s]))
        torch.cuda.synchronize()
        from gpu_harness import hip
        hip().hipMemcpy(self.bufs["x"], xd.data_ptr(), self.T * self.H * self.act, 3)
        (m.moe_chain_run if graph else m.moe_chain_run_eager)(self.chain, torch.cuda.current_stream())
        torch.cuda.synchronize()

    def snapshot(self):
        L, T, H, k = self.L, self.T, self.H, self.k
        dt = np.float32 if self.wdt == 0 else np.uint16  # activations are bf16 for fp8 layers
        return dict(
            x=d2h(self.bufs["x"], (L + 1) * T * H * self.act, dt).reshape(L + 1, T, H),
            xn=d2h(self.bufs["xn"], L * T * H * self.act, dt).reshape(L, T, H),
            y=d2h(self.bufs["y"], L * T * H * self.act, dt).reshape(L, T, H),
            ids=d2h(self.bufs["ids"], L * T * k * 4, np.int32).reshape(L, T, k),
            sid=d2h(self.bufs["slot_ids"], L * T * k * 4, np.int32).reshape(L, T, k),
        )

    def lists(self, l):
        i = self.info[l]
        lst = d2h(i["copy_list"], 4 * (2 + 2 * max(self.S, self.E)), np.int32)
        pf = d2h(i["prefetch_list"], 4 * (2 + 2 * self.S), np.int32)
        so = d2h(i["slot_of"], 4 * self.E, np.int32)
        eo = d2h(i["expert_of"], 4 * self.S, np.int32)
        lu = d2h(i["last_use"], 8 * self.S, np.uint64)
        sc = d2h(i["score"], 4 * self.S, np.uint32)
        return (int(lst[0]), lst[2:2 + 2 * lst[1]].reshape(-1, 2)), pf[2:2 + 2 * pf[1]].reshape(-1, 2), (so, eo, lu, sc)

    def activations(self, l):
        return d2h(self.info[l]["act"], 4 * self.E, np.uint32)

    def close(self):
        m.moe_chain_destroy(self.chain)
        for h in reversed(self.handles):
            m.moe_offload_destroy(h)


def oracle_replay_step(cm, caches, snap, prefetch_n, check_ffn=True):
    """Teacher-forced oracle for one chain step; asserts parity for every layer."""
    L = cm.L
    adt = 1 if cm.wdt >= 2 else cm.wdt  # activation / router format
    for l in range(L):
        xn = snap["xn"][l]
        # the block input itself: the norm of the GPU stream, the same codes as the oracle's
        ref_xn = oracle.rmsnorm(snap["x"][l], adt)
        assert np.array_equal(xn, ref_xn), l
        ids, w, _ = oracle.route(xn, cm.routers[l][0], cm.routers[l][1], cm.k, adt)
        assert np.array_equal(ids, snap["ids"][l]), (l, ids, snap["ids"][l])
        sid, mode, pairs = caches[l].ensure(ids)
        caches[l].copy(mode, pairs)
        assert np.array_equal(sid, snap["sid"][l]), l
        if prefetch_n and l + 1 < L:
            pred, _, _ = oracle.route(xn, cm.routers[l + 1][0], cm.routers[l + 1][1], cm.k, adt)
            inst = caches[l + 1].install(pred, prefetch_n)
            caches[l + 1].copy(0, inst)
        if check_ffn:
            y, y64 = oracle.ffn(xn, cm.wdt, cm.H, cm.F, caches[l].records(sid), w, cm.shared[l], want_f64=True)
            assert row_rel_err(snap["y"][l], y64, cm.wdt) <= (1e-5 if cm.wdt == 0 else 2e-2), l
            assert np.array_equal(snap["x"][l + 1], oracle.residual(snap["x"][l], snap["y"][l], cm.wdt))
    # lists and tables of every layer after the step (each handle's last call)
    for l in range(L):
        (mode, pairs), pf, (so, eo, lu, sc) = cm.lists(l)
        oso, oeo, olu, _ = caches[l].state()
        assert np.array_equal(so, oso) and np.array_equal(eo, oeo) and np.array_equal(lu, olu), l
        assert np.array_equal(sc, caches[l].scores()), l
        assert np.array_equal(cm.activations(l), caches[l].activations()), l


@pytest.mark.parametrize("prefetch_n", [0, 2])
def test_chain_graph_matches_eager_and_oracle(prefetch_n):
    L, E, S, k, H, F, T = 4, 16, 6, 4, 256, 256, 2
    print("chain L=%d E=%d S=%d k=%d H=%d F=%d T=%d prefetch=%d" % (L, E, S, k, H, F, T, prefetch_n), flush=True)
    cg = ChainModel(L, E, S, k, H, F, 1, T, 81, prefetch_n)
    ce = ChainModel(L, E, S, k, H, F, 1, T, 81, prefetch_n)
    caches = [oracle.Cache(E, S, cg.hosts[l], oracle.record_bytes(1, H, F)) for l in range(L)]
    try:
        for s in range(12):
            cg.run(s, graph=True)
            ce.run(s, graph=False)
            sg, se = cg.snapshot(), ce.snapshot()
            for key in sg:
                assert np.array_equal(sg[key], se[key]), (s, key)
            oracle_replay_step(cg, caches, sg, prefetch_n)
        st = [m.moe_offload_stats(h) for h in cg.handles]
        assert all(x["error"] == 0 for x in st)
        if prefetch_n:
            assert sum(x["prefetch_installs"] for x in st) > 0
    finally:
        cg.close()
        ce.close()


def test_prefetch_keeps_outputs_identical():
    """Same token stream with and without lookahead prefetch: identical outputs, identical routing."""
    L, E, S, k, H, F, T = 6, 32, 8, 4, 256, 256, 1
    a = ChainModel(L, E, S, k, H, F, 1, T, 83, 0)
    b = ChainModel(L, E, S, k, H, F, 1, T, 83, 4)
    try:
        for s in range(24):
            a.run(s)
            b.run(s)
            sa, sb = a.snapshot(), b.snapshot()
            assert np.array_equal(sa["x"], sb["x"]) and np.array_equal(sa["ids"], sb["ids"]), s
        ma = sum(m.moe_offload_stats(h)["misses"] for h in a.handles)
        stb = [m.moe_offload_stats(h) for h in b.handles]
        mb = sum(x["misses"] for x in stb)
        print("demand misses without / with prefetch: %d / %d, installs %d, prefetch hits %d" %
              (ma, mb, sum(x["prefetch_installs"] for x in stb), sum(x["prefetch_hits"] for x in stb)), flush=True)
        assert mb <= ma
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("case", [
    # (E, S, k, H, F, wdt, T, prefetch, shared): the fused router launch with a shared expert and fp8 records,
    # the same with MXFP4 records,
    # the batch limits of that fusion (8 fused, 9 not), 256 experts, and more than 512 (t, j) pairs (separate
    # kernels and the predictor stream for the lookahead)
    (16, 6, 4, 256, 256, 2, 3, 2, True),
    (16, 6, 4, 256, 256, 1, 8, 2, True),
    (16, 6, 4, 256, 256, 1, 9, 0, False),
    (256, 20, 8, 256, 256, 1, 2, 3, False),
    (32, 12, 8, 128, 256, 1, 72, 2, False),
    (16, 6, 4, 256, 512, 3, 3, 2, True),
])
def test_chain_variants_match_eager_and_oracle(case):
    E, S, k, H, F, wdt, T, prefetch_n, shared = case
    L = 3
    print("chain variant E=%d S=%d k=%d H=%d F=%d wdt=%d T=%d prefetch=%d shared=%s" % case, flush=True)
    cg = ChainModel(L, E, S, k, H, F, wdt, T, 85, prefetch_n, shared=shared)
    ce = ChainModel(L, E, S, k, H, F, wdt, T, 85, prefetch_n, shared=shared)
    rb = oracle.record_bytes(wdt, H, F)
    caches = [oracle.Cache(E, S, cg.hosts[l], rb) for l in range(L)]
    try:
        for s in range(5):
            cg.run(s, graph=True)
            ce.run(s, graph=False)
            sg, se = cg.snapshot(), ce.snapshot()
            for key in sg:
                assert np.array_equal(sg[key], se[key]), (s, key)
            oracle_replay_step(cg, caches, sg, prefetch_n)
        assert all(m.moe_offload_stats(h)["error"] == 0 for h in cg.handles)
    finally:
        cg.close()
        ce.close()


@pytest.mark.parametrize("wdt,T,mode", [(1, 1, "cold"), (1, 4, "cold"), (2, 2, "cold"), (3, 1, "cold"),
                                         (1, 8, "split"), (1, 1, "split")])
def test_chain_with_host_computed_layers(wdt, T, mode):
    """Layers in cold or split mode inside the decode chain: the graph publishes each call with
    host-computed pairs to the chain's host thread and waits for its rows.  Steps 0-2 run over the link,
    steps 3-5 with every layer in the mode, steps 6-8 with layer 1 switched back (the graph is captured
    again each time the set changes).  Graph and eager runs bitwise identical; ids, slot ids (index
    S + E + e for the host's pairs), tables and counters bit-exact against the oracle teacher-forced, its
    outputs within tolerance.  Split mode at one token (4 pairs <= S) never involves the host."""
    L, E, S, k, H, F = 3, 16, 6, 4, 256, 512
    print("chain host-computed wdt=%d T=%d mode=%s" % (wdt, T, mode), flush=True)
    cg = ChainModel(L, E, S, k, H, F, wdt, T, 86)
    ce = ChainModel(L, E, S, k, H, F, wdt, T, 86)
    rb = oracle.record_bytes(wdt, H, F)
    caches = [oracle.Cache(E, S, cg.hosts[l], rb) for l in range(L)]
    st = torch.cuda.current_stream()
    cold_seen = 0
    try:
        for s in range(9):
            if s in (3, 6):
                for l in (range(L) if s == 3 else [1]):
                    for cm in (cg, ce):
                        if s == 6:
                            assert m.moe_offload_set_cold(cm.handles[l], m.COLD_OFF, st)[0] == 0
                        elif mode == "cold":
                            assert m.moe_offload_set_cold(cm.handles[l], m.COLD_ON, st)[0] == 1
                        else:
                            m.moe_offload_set_split(cm.handles[l], 128, st)
                    if s == 6:
                        caches[l].set_cold(False)
                    elif mode == "cold":
                        caches[l].set_cold(True)
                    else:
                        caches[l].set_split(128)
            cg.run(s, graph=True)
            ce.run(s, graph=False)
            sg, se = cg.snapshot(), ce.snapshot()
            for key in sg:
                assert np.array_equal(sg[key], se[key]), (s, key)
            cold_seen += int((sg["sid"] >= S + E).sum())
            oracle_replay_step(cg, caches, sg, 0)
        for cm in (cg, ce):
            assert all(m.moe_offload_stats(h)["error"] == 0 for h in cm.handles)
        if mode == "cold" or T * k > S:
            assert cold_seen > 0
        else:
            assert cold_seen == 0
    finally:
        cg.close()
        ce.close()


@pytest.mark.parametrize("prefetch_n,T", [(0, 1), (3, 2)])
def test_chain_scored_eviction(prefetch_n, T):
    """Scored eviction in the decode chain, with and without lookahead installs (usage 0, first out)."""
    L, E, S, k, H, F = 3, 32, 8, 4, 256, 256
    print("chain scored eviction prefetch=%d T=%d" % (prefetch_n, T), flush=True)
    cg = ChainModel(L, E, S, k, H, F, 1, T, 87, prefetch_n, scored=True)
    caches = [oracle.Cache(E, S, cg.hosts[l], oracle.record_bytes(1, H, F), policy=oracle.SCORED) for l in range(L)]
    try:
        for s in range(10):
            cg.run(s, graph=True)
            oracle_replay_step(cg, caches, cg.snapshot(), prefetch_n)
        assert all(m.moe_offload_stats(h)["error"] == 0 for h in cg.handles)
    finally:
        cg.close()


@pytest.mark.parametrize("prefetch_n,T", [(0, 1), (3, 2), (0, 8)])
def test_chain_activation_aware_eviction(prefetch_n, T):
    """Activation-aware eviction in the decode chain, with and without lookahead installs."""
    L, E, S, k, H, F = 3, 32, 8, 4, 256, 256
    print("chain activation-aware eviction prefetch=%d T=%d" % (prefetch_n, T), flush=True)
    cg = ChainModel(L, E, S, k, H, F, 1, T, 88, prefetch_n, policy_flag=m.FLAG_FREQ)
    caches = [oracle.Cache(E, S, cg.hosts[l], oracle.record_bytes(1, H, F), policy=oracle.FREQ) for l in range(L)]
    try:
        for s in range(12):
            cg.run(s, graph=True)
            oracle_replay_step(cg, caches, cg.snapshot(), prefetch_n)
        assert all(m.moe_offload_stats(h)["error"] == 0 for h in cg.handles)
    finally:
        cg.close()


def test_chain_with_pinned_experts():
    """Each layer pins its own hot set before the decode chain runs (eager pin calls between graph replays)."""
    L, E, S, k, H, F, T = 3, 32, 8, 4, 256, 256, 1
    cg = ChainModel(L, E, S, k, H, F, 1, T, 89, 2)
    caches = [oracle.Cache(E, S, cg.hosts[l], oracle.record_bytes(1, H, F)) for l in range(L)]
    try:
        for l in range(L):
            P = np.array([(3 * l + j) % E for j in range(3)], np.int32)
            m.moe_offload_pin(cg.handles[l], to_dev(P), len(P), torch.cuda.current_stream())
            caches[l].copy(0, caches[l].pin(P))
        torch.cuda.synchronize()
        for s in range(10):
            cg.run(s, graph=True)
            oracle_replay_step(cg, caches, cg.snapshot(), 2)
        for l in range(L):
            so, eo, lu, sc = cg.lists(l)[2]
            pinned = d2h(cg.info[l]["pinned"], 4 * S, np.int32)
            assert np.array_equal(pinned, caches[l].pinned()) and pinned.sum() == 3
        assert all(m.moe_offload_stats(h)["error"] == 0 for h in cg.handles)
    finally:
        cg.close()


@pytest.mark.parametrize("wdt,shared,prefetch_n,H,F,T", [
    # single tokens: small passes for each format, the lookahead beside it, and the 16- and 8-block passes
    # (read through at half the width) for bf16, fp8 and MXFP4; batches of 4 and 8 (calls wider than the
    # 6 slots read their overflow through into staging) for each format, with and without the lookahead
    (1, False, 0, 256, 512, 1), (2, True, 0, 256, 512, 1), (3, True, 0, 256, 512, 1), (1, False, 2, 256, 512, 1),
    (1, False, 0, 2048, 256, 1), (2, False, 0, 1024, 1024, 1), (3, True, 0, 2048, 512, 1),
    (1, False, 0, 256, 512, 4), (2, True, 0, 256, 512, 8), (3, True, 0, 512, 512, 4), (1, False, 2, 2048, 256, 8),
    # 16 and 32 tokens: records with more than 8 tokens read the host once and their later token groups
    # read back what the first one stored
    (1, False, 0, 256, 512, 16), (2, True, 0, 512, 256, 32), (3, False, 0, 512, 512, 32), (1, False, 2, 256, 512, 32)])
def test_chain_read_through_matches_copy_kernel(wdt, shared, prefetch_n, H, F, T):
    """Read-through (the FFN fills missed slots, and the staging records of calls wider than the cache, from
    the host store; no copy launch) against the same chain with the copy kernel: identical outputs, routing,
    tables and counters on every step, every occupied slot byte-identical to its expert's host record, and
    the oracle replay; the two chains swap modes after six steps (graph dropped and captured again)."""
    L, E, S, k = 3, 16, 6, 4
    print("chain read-through wdt=%d shared=%s prefetch=%d H=%d F=%d T=%d" % (wdt, shared, prefetch_n, H, F, T),
          flush=True)
    rt = ChainModel(L, E, S, k, H, F, wdt, T, 93, prefetch_n, shared=shared)
    cp = ChainModel(L, E, S, k, H, F, wdt, T, 93, prefetch_n, shared=shared)
    # only the decode kernels read through; at 8 to 32 tokens over 16 experts the automatic choice would take
    # the grouped GEMM for some formats, so both chains are held to the decode kernels (set before capture)
    for h in rt.handles + cp.handles:
        m.moe_offload_set_ffn_path(h, m.FFN_DECODE)
    m.moe_chain_set_read_through(cp.chain, 0)
    rb = oracle.record_bytes(wdt, H, F)
    caches = [oracle.Cache(E, S, rt.hosts[l], rb) for l in range(L)]
    try:
        for s in range(10):
            if s == 6:  # swap the modes mid-stream: both graphs are dropped and captured again
                m.moe_chain_set_read_through(rt.chain, 0)
                m.moe_chain_set_read_through(cp.chain, 1)
            graph = s % 3 != 2  # mostly graph replays, every third step eager
            rt.run(s, graph=graph)
            cp.run(s, graph=graph)
            sr, sc = rt.snapshot(), cp.snapshot()
            for key in sr:
                assert np.array_equal(sr[key], sc[key]), (s, key)
            for l in range(L):
                assert all(np.array_equal(a, b) for a, b in zip(rt.lists(l)[2], cp.lists(l)[2])), (s, l)
                eo = rt.lists(l)[2][1]
                for slot in range(S):
                    if eo[slot] >= 0:
                        got = d2h(rt.info[l]["slots"] + slot * rt.info[l]["record_stride"], rb, np.uint8)
                        assert np.array_equal(got, rt.hosts[l][eo[slot], :rb]), (s, l, slot, int(eo[slot]))
            oracle_replay_step(rt, caches, sr, prefetch_n)
        sa = [m.moe_offload_stats(h) for h in rt.handles]
        sb = [m.moe_offload_stats(h) for h in cp.handles]
        assert sa == sb and all(x["error"] == 0 for x in sa)
        assert sum(x["misses"] for x in sa) > 0
    finally:
        rt.close()
        cp.close()

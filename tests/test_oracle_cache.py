"""Pins for the oracle's per-layer LRU slot cache and prefetch install.

  * textbook LRU: for one id per call the miss count at every capacity S is
    given by Mattson stack distances (Mattson, Gecsei, Slutz, Traiger, 1970),
    and the resident set after every call equals an OrderedDict LRU;
  * a brute-force re-statement of the batched rules (tie order, staging,
    install) compared exactly on random traces;
  * invariants after every call (maps inverse, D resident, misses = D \\ R,
    free slots first, staging iff |D| > S; a call wider than the cache
    leaves every slot holding one of its experts, the most used ones);
  * a hand-worked example of the threshold, the overflow claim order and
    the LRU ties;
  * capacity >= distinct experts ever seen: only compulsory misses.
"""
from collections import OrderedDict

import numpy as np
import pytest


def mattson_misses(trace, S):
    stack, misses = [], 0
    for e in trace:
        if e in stack:
            d = stack.index(e) + 1  # stack distance (1 = most recent)
            stack.remove(e)
        else:
            d = None  # first reference: infinite distance
        stack.insert(0, e)
        if d is None or d > S:
            misses += 1
    return misses


@pytest.mark.parametrize("seed", range(5))
def test_single_id_calls_match_mattson_and_textbook_lru(orc, seed):
    rng = np.random.default_rng(seed)
    E = 16
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    trace = rng.choice(E, size=400, p=p / p.sum()).astype(np.int32)
    for S in range(1, E + 1):
        c = orc.Cache(E, S)
        lru = OrderedDict()
        misses = 0
        for e in trace:
            _, mode, pairs = c.ensure(np.array([[e]], np.int32))
            assert mode == orc.SLOTS
            misses += len(pairs)
            hit = e in lru
            assert (len(pairs) == 0) == hit
            if hit:
                lru.move_to_end(e)
            else:
                if len(lru) == S:
                    lru.popitem(last=False)
                lru[e] = True
            so, eo, _, _ = c.state()
            assert set(int(v) for v in eo if v >= 0) == set(lru.keys())
        assert misses == mattson_misses(list(trace), S)
        assert c.counters()["misses"] == misses


class BruteCache:
    """The batched rules restated plainly (sorted(), dicts), independently of the C code.
    scored=True: least-used slots go first (usage = calls since loaded, capped), then LRU.
    freq=True: slots installed and not used since go first, then the expert activated by the fewest
    calls since the cache was created (kept across evictions, capped), then LRU."""

    def __init__(self, E, S, scored=False, cap=(1 << 20) - 1, freq=False, cold=False, split=None):
        self.E, self.S = E, S
        self.held = [None] * S
        self.home = {}
        self.used = [0] * S
        self.uses = [0] * S
        self.fired = [0] * E  # activations per expert
        self.clock = 0
        self.scored, self.cap, self.freq, self.cold, self.split = scored, cap, freq, cold, split
        self.pinned = set()

    def _victims(self, protect):
        cands = [s for s in range(self.S)
                 if s not in self.pinned and (self.held[s] is None or self.held[s] not in protect)]
        if self.scored:
            return sorted(cands, key=lambda s: (self.held[s] is not None, self.uses[s], self.used[s], s))
        if self.freq:
            def key(s):
                if self.held[s] is None:
                    return (0, 0, 0, 0, s)
                return (1, self.used[s] != 0, self.fired[self.held[s]], self.used[s], s)
            return sorted(cands, key=key)
        return sorted(cands, key=lambda s: (self.held[s] is not None, self.used[s], s))

    def _put(self, e, s):
        if self.held[s] is not None:
            del self.home[self.held[s]]
        self.held[s] = e
        self.home[e] = s
        self.uses[s] = 0

    def ensure(self, ids, k):
        self.clock += 1
        D = sorted(set(ids))
        miss = [e for e in D if e not in self.home]
        if self.cold:  # nothing loads; misses are read at S + E + e from the host
            for e in D:
                if e in self.home:
                    self.used[self.home[e]] = self.clock
                    self.uses[self.home[e]] = min(self.uses[self.home[e]] + 1, self.cap)
                self.fired[e] = min(self.fired[e] + 1, self.cap)
            rec = lambda e: self.home.get(e, self.S + self.E + e)
            return [rec(e) for e in ids], 3, [(e, rec(e)) for e in miss]
        claim = miss
        victims = self._victims(set(D))
        over = len(miss) > len(victims)
        if over:  # more misses than victims: the most used misses claim them
            count = {e: ids.count(e) for e in D}
            best = {e: min(i % k for i, x in enumerate(ids) if x == e) for e in D}
            claim = sorted(miss, key=lambda e: (-count[e], best[e], e))
        for e, s in zip(claim, victims):
            self._put(e, s)
        for e in D:
            if e in self.home:
                self.used[self.home[e]] = self.clock
                self.uses[self.home[e]] = min(self.uses[self.home[e]] + 1, self.cap)
            self.fired[e] = min(self.fired[e] + 1, self.cap)
        host = set()
        if over and self.split is not None:  # the host's share of all misses, from the last staged ones
            staged = sorted(e for e in miss if e not in self.home)
            n_host = min(len(staged), (len(miss) * self.split + 128) // 256)
            host = set(staged[len(staged) - n_host:])
        rec = lambda e: self.home.get(e, self.S + self.E + e if e in host else self.S + e)
        return [rec(e) for e in ids], int(over), [(e, rec(e)) for e in miss]

    def pin(self, P):
        P = list(P)
        self.pinned = {self.home[e] for e in P if e in self.home}
        loads = []
        for e, s in zip(sorted(e for e in P if e not in self.home), self._victims(set(P))):
            self._put(e, s)
            self.used[s] = self.clock
            self.pinned.add(s)
            loads.append((e, s))
        return loads

    def install(self, pred, n_max):
        T, k = len(pred), len(pred[0])
        count, best = {}, {}
        for row in pred:
            for j, e in enumerate(row):
                count[e] = count.get(e, 0) + 1
                best[e] = min(best.get(e, k), j)
        cand = sorted((e for e in count if e not in self.home), key=lambda e: (-count[e], best[e], e))
        vict = self._victims(set(count))
        n = max(0, min(n_max, len(cand), len(vict)))
        pairs = list(zip(cand[:n], vict[:n]))
        for e, s in pairs:
            self._put(e, s)
            self.used[s] = 0
        return pairs


def _check_invariants(c, ids, slot_ids, mode, pairs, before, pinned0=None):
    so, eo, lu, tick = c.state()
    S, E = c.S, c.E
    pinned0 = np.zeros(S, np.int32) if pinned0 is None else pinned0
    for s in range(S):
        if eo[s] >= 0:
            assert so[eo[s]] == s
    for e in range(E):
        if so[e] >= 0:
            assert eo[so[e]] == e
    D = sorted(set(ids.reshape(-1).tolist()))
    so0, eo0, lu0, tick0 = before
    R0 = set(int(v) for v in eo0 if v >= 0)
    assert tick == tick0 + 1
    eligible = [s for s in range(S) if not pinned0[s] and (eo0[s] < 0 or eo0[s] not in D)]
    if len([e for e in D if e not in R0]) > len(eligible):
        assert mode == 1
        assert [int(p[0]) for p in pairs] == [e for e in D if e not in R0]
        # residents stay; every slot not pinned now holds an expert of D, last used now
        for e in D:
            if so0[e] >= 0:
                assert so[e] == so0[e]
        assert all(eo[s] in D and lu[s] == tick for s in range(S) if not pinned0[s])
        # the misses that got a slot were used by at least as many pairs as those staged
        n_of = {e: int((ids == e).sum()) for e in D}
        got = [int(p[0]) for p in pairs if p[1] < S]
        staged = [int(p[0]) for p in pairs if p[1] >= S]
        assert len(got) + len(staged) == len(pairs) and len(staged) > 0
        if got:
            assert min(n_of[e] for e in got) >= max(n_of[e] for e in staged)
        for p in pairs:
            assert p[1] == (so[p[0]] if p[1] < S else S + p[0])
        for i, e in np.ndenumerate(ids):
            assert slot_ids[i] == (so[e] if so[e] >= 0 else S + e)
        return
    assert mode == 0
    assert [int(p[0]) for p in pairs] == [e for e in D if e not in R0]  # misses ascending
    for e in D:
        assert so[e] >= 0 and lu[so[e]] == tick
    for i, e in np.ndenumerate(ids):
        assert slot_ids[i] == so[e]
    # no expert of D was evicted; free slots were used before any eviction
    free0 = [s for s in range(S) if eo0[s] < 0]
    used = [int(p[1]) for p in pairs]
    assert used[:len(free0)] == free0[:len(used)]
    for s in used:
        assert (eo0[s] < 0 or eo0[s] not in D) and not pinned0[s]


@pytest.mark.parametrize("policy", ["lru", "scored", "freq"])
@pytest.mark.parametrize("seed", range(8))
def test_batched_calls_match_brute_force(orc, seed, policy):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.choice([8, 16, 32]))
    k = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(k, E + 1))
    c = orc.Cache(E, S, policy={"lru": orc.LRU, "scored": orc.SCORED, "freq": orc.FREQ}[policy])
    b = BruteCache(E, S, scored=policy == "scored", freq=policy == "freq")
    p = 1.0 / np.arange(1, E + 1) ** rng.uniform(0.3, 1.5)
    for step in range(200):
        T = int(rng.integers(1, 6))
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
        before = c.state()
        if rng.random() < 0.2:
            pred = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
            n = int(rng.integers(0, 5))
            got = c.install(pred, n)
            exp = b.install(pred.tolist(), n)
            assert [tuple(map(int, r)) for r in got] == exp
            before = c.state()
        if rng.random() < 0.05:  # a new pinned set (at most S - k experts, so every call fits)
            P = rng.choice(E, size=int(rng.integers(0, S - k + 1)), replace=False).astype(np.int32)
            assert [tuple(map(int, r)) for r in c.pin(P)] == b.pin(P.tolist())
            assert [int(v) for v in c.pinned()] == [int(s_ in b.pinned) for s_ in range(S)]
            before = c.state()
        pinned0 = c.pinned()
        slot_ids, mode, pairs = c.ensure(ids)
        es, em, ep = b.ensure(ids.reshape(-1).tolist(), k)
        assert slot_ids.reshape(-1).tolist() == es
        assert mode == em
        assert [tuple(map(int, r)) for r in pairs] == ep
        assert c.scores().tolist() == b.uses
        assert c.activations().tolist() == b.fired
        _check_invariants(c, ids, slot_ids, mode, pairs, before, pinned0)


def test_enough_capacity_gives_only_compulsory_misses(orc):
    rng = np.random.default_rng(9)
    E, k = 32, 4
    trace = [np.stack([rng.choice(12, size=k, replace=False) for _ in range(2)]).astype(np.int32) for _ in range(100)]
    for S in (12, 20, 32):
        c = orc.Cache(E, S)
        total = sum(len(c.ensure(ids)[2]) for ids in trace)
        assert total == len(set(np.concatenate([t.reshape(-1) for t in trace]).tolist()))


def test_staging_threshold_and_free_first(orc):
    c = orc.Cache(8, 3)
    # three distinct experts fit: misses ascending into the free slots 0, 1, 2
    sid, mode, pairs = c.ensure(np.array([[5, 1], [1, 7]], np.int32))
    assert mode == 0 and pairs.tolist() == [[1, 0], [5, 1], [7, 2]] and sid.tolist() == [[1, 0], [0, 2]]
    # four distinct do not.  Hits 5 (slot 1) and 1 (slot 0) stay; slot 2 (expert 7, not routed) is
    # the one eligible victim.  Misses 2 and 3 are each routed once; 3 is at top-k position 0 and 2
    # at position 1, so 3 claims slot 2 and 2 is staged at S + 2 = 5.
    sid, mode, pairs = c.ensure(np.array([[5, 2], [3, 1]], np.int32))
    assert mode == 1 and pairs.tolist() == [[2, 5], [3, 2]]
    assert sid.tolist() == [[1, 5], [2, 0]]
    so, eo, lu, tick = c.state()
    assert eo.tolist() == [1, 5, 3] and lu.tolist() == [2, 2, 2] and tick == 2 and so[7] == -1 and so[2] == -1
    cnt = c.counters()
    assert (cnt["hits"], cnt["misses"], cnt["staged_calls"], cnt["staged_copies"]) == (2, 4, 1, 1)
    # all slots last used at tick 2: misses 4, 7 take the lowest slots
    sid, mode, pairs = c.ensure(np.array([[4, 7]], np.int32))
    assert mode == 0 and pairs.tolist() == [[4, 0], [7, 1]]
    sid, mode, pairs = c.ensure(np.array([[6, 4]], np.int32))
    assert pairs.tolist() == [[6, 2]]  # slot 2 (tick 2) is older than slot 1 (tick 3)
    # an overflow call whose misses outnumber the eligible slots by count: expert 0 is routed by
    # both tokens, so it claims the one eligible slot (slot 1, expert 7) ahead of experts 1, 2, 3
    c2 = orc.Cache(8, 2)
    c2.ensure(np.array([[6, 7]], np.int32))
    sid, mode, pairs = c2.ensure(np.array([[3, 0, 6], [0, 1, 2]], np.int32))
    assert mode == 1 and pairs.tolist() == [[0, 1], [1, 3], [2, 4], [3, 5]]
    assert sid.tolist() == [[5, 1, 0], [1, 3, 4]]


def test_invalid_id_leaves_state_untouched(orc):
    c = orc.Cache(8, 4)
    c.ensure(np.array([[1, 2]], np.int32))
    before = c.state()
    for bad in (8, -1, 1 << 20):
        with pytest.raises(ValueError):
            c.ensure(np.array([[1, bad]], np.int32))
        after = c.state()
        assert all(np.array_equal(a, b) for a, b in zip(before[:3], after[:3])) and after[3] == before[3]


def test_perfect_prediction_turns_misses_into_prefetch_hits(orc):
    rng = np.random.default_rng(3)
    E, S, k = 32, 12, 4
    with_pf, without = orc.Cache(E, S), orc.Cache(E, S)
    demand_pf = demand_plain = 0
    for step in range(100):
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(2)]).astype(np.int32)
        installed = with_pf.install(ids, 4)  # the predictor is exact
        _, m1, p1 = with_pf.ensure(ids)
        _, m0, p0 = without.ensure(ids)
        if m1 == 0:
            # every installed expert is a hit of the very next call
            assert set(installed[:, 0].tolist()) <= set(ids.reshape(-1).tolist())
            assert not (set(p1[:, 0].tolist()) & set(installed[:, 0].tolist()))
            if step == 0:  # cold: the installs cover part of the compulsory misses
                assert len(p1) == len(p0) - len(installed)
        demand_pf += len(p1) if m1 == 0 else 0
        demand_plain += len(p0) if m0 == 0 else 0
    cnt = with_pf.counters()
    assert cnt["prefetch_hits"] == cnt["prefetch_installs"]
    assert demand_pf < demand_plain


def test_install_budget_zero_changes_nothing(orc):
    rng = np.random.default_rng(4)
    a, b = orc.Cache(16, 6), orc.Cache(16, 6)
    for _ in range(100):
        ids = np.stack([rng.choice(16, size=2, replace=False) for _ in range(2)]).astype(np.int32)
        assert len(a.install(ids[::-1], 0)) == 0
        ra, rb = a.ensure(ids), b.ensure(ids)
        assert np.array_equal(ra[0], rb[0]) and ra[1] == rb[1] and np.array_equal(ra[2], rb[2])


def test_scored_eviction_prefers_the_least_used_slot(orc):
    # two slots; expert 0 is routed three times, expert 1 once but more recently: LRU evicts expert 0
    # (slot 0, last used at tick 3), scored eviction evicts expert 1 (slot 1, used once since loaded)
    calls = [[[0, 1]], [[0]], [[0]], [[1]], [[2]]]
    victims = {}
    for policy in (orc.LRU, orc.SCORED):
        c = orc.Cache(4, 2, policy=policy)
        for ids in calls:
            _, _, pairs = c.ensure(np.array(ids, np.int32))
        victims[policy] = pairs.tolist()
        so, eo, lu, tick = c.state()
        if policy == orc.SCORED:
            assert eo.tolist() == [0, 2] and c.scores().tolist() == [3, 1] and lu.tolist() == [3, 5]
    assert victims[orc.LRU] == [[2, 0]] and victims[orc.SCORED] == [[2, 1]]


def test_scored_installs_start_at_zero_and_go_first(orc):
    c = orc.Cache(8, 3, policy=orc.SCORED)
    c.ensure(np.array([[0, 1]], np.int32))
    c.ensure(np.array([[0]], np.int32))
    inst = c.install(np.array([[5]], np.int32), 1)  # into the free slot, at usage 0
    assert inst.tolist() == [[5, 2]] and c.scores().tolist() == [2, 1, 0]
    _, _, pairs = c.ensure(np.array([[7, 0]], np.int32))
    assert pairs.tolist() == [[7, 2]]  # the installed, never used slot goes before expert 1 (used once)
    # with a budget of two, the second install takes the least used occupied slot (expert 1, not expert 0)
    c2 = orc.Cache(8, 3, policy=orc.SCORED)
    c2.ensure(np.array([[0, 1]], np.int32))
    c2.ensure(np.array([[0]], np.int32))
    assert c2.install(np.array([[5, 6]], np.int32), 2).tolist() == [[5, 2], [6, 1]]
    assert c2.scores().tolist() == [2, 0, 0]


def test_pinned_experts_are_never_evicted(orc):
    c = orc.Cache(8, 3)
    assert c.pin(np.array([5], np.int32)).tolist() == [[5, 0]]  # free slot 0, pinned
    assert c.pinned().tolist() == [1, 0, 0]
    for e, want in ((1, [[1, 1]]), (2, [[2, 2]]), (3, [[3, 1]]), (4, [[4, 2]])):
        _, mode, pairs = c.ensure(np.array([[e]], np.int32))
        assert mode == 0 and pairs.tolist() == want  # slots 1 and 2 take turns; slot 0 keeps expert 5
    # two experts need slots and only two are eligible (slot 0 is pinned): they fit, expert 5 stays
    _, mode, pairs = c.ensure(np.array([[6, 7]], np.int32))
    assert mode == 0 and pairs.tolist() == [[6, 1], [7, 2]]
    # three misses, two eligible slots: the call overflows although |D| = 3 = S
    _, mode, pairs = c.ensure(np.array([[0, 1, 2]], np.int32))
    assert mode == 1 and len(pairs) == 3 and sum(1 for p in pairs if p[1] >= 3) == 1
    assert c.state()[1][0] == 5
    # unpinning gives slot 0 back to the cache: last used at the pin (tick 0), it is the next victim
    assert c.pin(np.array([], np.int32)).tolist() == [] and c.pinned().tolist() == [0, 0, 0]
    _, _, pairs = c.ensure(np.array([[3]], np.int32))
    assert pairs.tolist() == [[3, 0]]
    with pytest.raises(ValueError):
        c.pin(np.array([1, 1], np.int32))  # repeated id: nothing changes


def test_activation_aware_eviction_keeps_the_most_activated_expert(orc):
    # two slots, four experts.  Expert 0 is routed by three calls, evicted by a call that needs both
    # slots, and reloaded; expert 1 is loaded once and routed twice.  At the last call both slots were
    # used at the same tick: LRU takes the lower slot (expert 0), scored eviction takes expert 0 as
    # well (used once since its reload, against twice for expert 1), the activation-aware cache keeps
    # expert 0 (four activations, expert 1 two) and evicts expert 1.
    calls = [[[0]], [[0]], [[0]], [[1, 2]], [[0, 1]], [[3]]]
    last = {}
    for policy in (orc.LRU, orc.SCORED, orc.FREQ):
        c = orc.Cache(4, 2, policy=policy)
        for ids in calls:
            _, mode, pairs = c.ensure(np.array(ids, np.int32))
            assert mode == orc.SLOTS
        last[policy] = pairs.tolist()
        if policy == orc.FREQ:
            so, eo, lu, tick = c.state()
            assert eo.tolist() == [0, 3] and c.activations().tolist() == [4, 2, 1, 1] and lu.tolist() == [5, 6]
    assert last[orc.LRU] == [[3, 0]] and last[orc.SCORED] == [[3, 0]] and last[orc.FREQ] == [[3, 1]]


def test_activation_aware_installs_go_first(orc):
    # an installed expert with a long history is still the first victim until a call uses it
    c = orc.Cache(4, 2, policy=orc.FREQ)
    for ids in ([[0]], [[0]], [[0]], [[1, 2]]):
        c.ensure(np.array(ids, np.int32))
    # slots hold 2 (slot 0) and 1 (slot 1); expert 0 has three activations and is installed over one of them
    assert c.install(np.array([[0]], np.int32), 1).tolist() == [[0, 0]]
    _, _, pairs = c.ensure(np.array([[3]], np.int32))
    assert pairs.tolist() == [[3, 0]]  # the installed, unused expert 0 goes first despite its count
    assert c.activations().tolist() == [3, 1, 1, 1]


@pytest.mark.parametrize("seed", range(6))
def test_cold_mode_matches_brute_force_and_never_moves_weights(orc, seed):
    """Host-computed cold experts: calls in cold mode load nothing (the slot maps never change), hits
    are used in place, misses are listed at S + E + e; switching the mode on and off mid-trace."""
    rng = np.random.default_rng(300 + seed)
    E = int(rng.choice([8, 16, 32]))
    k = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(k, E + 1))
    policy = [orc.LRU, orc.SCORED, orc.FREQ][seed % 3]
    c = orc.Cache(E, S, policy=policy)
    b = BruteCache(E, S, scored=policy == orc.SCORED, freq=policy == orc.FREQ)
    p = 1.0 / np.arange(1, E + 1) ** rng.uniform(0.3, 1.5)
    cold_total = 0
    for step in range(150):
        if step % 25 == 0:
            on = bool(rng.integers(0, 2))
            c.set_cold(on)
            b.cold = on
        T = int(rng.integers(1, 6))
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
        before = c.state()
        slot_ids, mode, pairs = c.ensure(ids)
        es, em, ep = b.ensure(ids.reshape(-1).tolist(), k)
        assert slot_ids.reshape(-1).tolist() == es and mode == em
        assert [tuple(map(int, r)) for r in pairs] == ep
        assert c.scores().tolist() == b.uses and c.activations().tolist() == b.fired
        if b.cold:
            so, eo, lu, tick = c.state()
            assert np.array_equal(so, before[0]) and np.array_equal(eo, before[1]) and tick == before[3] + 1
            cold_total += len(pairs)
        else:
            _check_invariants(c, ids, slot_ids, mode, pairs, before)
    assert c.counters()["cold"] == cold_total


def test_cold_mode_hand_example(orc):
    c = orc.Cache(8, 3)
    c.ensure(np.array([[1, 2]], np.int32))  # slots 0, 1 hold experts 1, 2 (tick 1)
    c.set_cold(True)
    sid, mode, pairs = c.ensure(np.array([[2, 5], [6, 1]], np.int32))
    assert mode == orc.COLD and pairs.tolist() == [[5, 16], [6, 17]]  # S + E + e = 3 + 8 + e
    assert sid.tolist() == [[1, 16], [17, 0]]
    so, eo, lu, tick = c.state()
    assert eo.tolist() == [1, 2, -1] and lu.tolist() == [2, 2, 0] and tick == 2
    cnt = c.counters()
    assert (cnt["hits"], cnt["misses"], cnt["cold"]) == (2, 2, 2)
    assert c.activations().tolist() == [0, 2, 2, 0, 0, 1, 1, 0]


@pytest.mark.parametrize("seed", range(6))
def test_split_mode_matches_brute_force(orc, seed):
    """Split mode: calls wider than the cache hand the last share of their staged misses to the host
    (index S + E + e); everything else, slot claims included, is unchanged."""
    rng = np.random.default_rng(400 + seed)
    E = int(rng.choice([16, 32]))
    k = int(rng.choice([2, 4]))
    S = int(rng.integers(k, E // 2))
    q = int(rng.choice([0, 64, 115, 200, 256]))
    c = orc.Cache(E, S)
    c.set_split(q)
    b = BruteCache(E, S, split=q)
    host_total = staged_total = 0
    for step in range(120):
        T = int(rng.integers(1, 8))
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        before = c.state()
        slot_ids, mode, pairs = c.ensure(ids)
        es, em, ep = b.ensure(ids.reshape(-1).tolist(), k)
        assert slot_ids.reshape(-1).tolist() == es and mode == em, (step, q)
        assert [tuple(map(int, r)) for r in pairs] == ep
        assert c.scores().tolist() == b.uses and c.activations().tolist() == b.fired
        host_total += sum(1 for p_ in pairs if p_[1] >= S + E)
        staged_total += sum(1 for p_ in pairs if S <= p_[1] < S + E)
        so, eo, lu, tick = c.state()
        for s_ in range(S):  # the maps stay mutually inverse
            if eo[s_] >= 0:
                assert so[eo[s_]] == s_
    cnt = c.counters()
    assert cnt["cold"] == host_total and cnt["staged_copies"] == staged_total
    if q == 0:
        assert host_total == 0
    if q == 256:
        assert staged_total == 0 and host_total > 0


def test_split_mode_hand_example(orc):
    # 3 slots hold experts 1, 2, 3; a call needs 1, 4, 5, 6, 7 (|D| = 5 > 3): experts 2 and 3 are the two
    # eligible victims; the misses 4..7 are routed once each at positions 1, 2 (token 0) and 0, 1 (token 1)
    # after 1, so 6 (position 0) and 4 (position 1, lower id than 7) claim slots 1 and 2; 5 and 7 are staged.
    # The host's share counts all 4 misses: q = 64 (a quarter) is one of them, the last staged one, 7;
    # q = 128 (half) is two, both staged ones; q = 256 would be four, capped at the two staged.
    for q, host in ((64, {7}), (128, {5, 7}), (256, {5, 7})):
        c = orc.Cache(8, 3)
        c.ensure(np.array([[1, 2, 3]], np.int32))
        c.set_split(q)
        sid, mode, pairs = c.ensure(np.array([[1, 4, 5], [6, 7, 1]], np.int32))
        assert mode == orc.STAGED
        rec = {e: (3 + 8 + e if e in host else 3 + e) for e in (5, 7)}  # host S + E + e, staged S + e
        assert pairs.tolist() == [[4, 2], [5, rec[5]], [6, 1], [7, rec[7]]], q
        assert sid.tolist() == [[0, 2, rec[5]], [1, rec[7], 0]], q
        cnt = c.counters()
        assert (cnt["staged_copies"], cnt["cold"]) == (2 - len(host), len(host)), q

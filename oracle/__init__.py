"""CPU ORACLE for the offloaded MoE layer step (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The GPU library never does, and this package
never imports the GPU library: the two share only the seeded input bytes
written by `synth`.

The arithmetic lives in `moe_oracle.c` (plain C, double precision, router
logits in a fixed binary32 order); this module only marshals numpy arrays and
keeps the per-layer state objects together:

* `route`            router logits, top-k ids, renormalised softmax weights
* `Cache`            the per-layer LRU slot table (ensure, whole-layer stage,
                     prefetch install) plus the oracle's own slot and staging
                     bytes, so a wrong slot map gives wrong outputs
* `ffn`              the expert FFN and top-k weighted combine

Sources: xinfer-ai 0.14.6 docs/moe_offload.md ("How it works": Decode,
Prefill, slot tensors; the opening paragraph on placement invariance) and
FreeToken issue #677 ("Proposal": Lookahead, Install, Correctness constraint).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libmoe_oracle.so")
_lib = None

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3
LRU, SCORED, FREQ = 0, 1, 2  # eviction policies
SCORE_MAX = (1 << 20) - 1
SLOTS, STAGED, STAGED_ALL, COLD = 0, 1, 2, 3


def build():
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                           "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32, u64, sz, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = f64
        L.orc_f64_to_bf16.argtypes = [f64]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_fp8_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_fp8_to_f64.restype = f64
        L.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_to_f64.restype = f64
        L.orc_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_f64.restype = f64
        L.orc_record_bytes.argtypes = [i32, i32, i32]
        L.orc_record_bytes.restype = sz
        L.orc_router_logits.argtypes = [vp, vp, i32, vp, i32, i32, i32, vp]
        L.orc_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        L.orc_topk.restype = i32
        L.orc_cache_new.argtypes = [i32, i32]
        L.orc_cache_new.restype = vp
        L.orc_cache_free.argtypes = [vp]
        L.orc_cache_set_policy.argtypes = [vp, i32]
        L.orc_cache_scores.argtypes = [vp, vp]
        L.orc_cache_act.argtypes = [vp, vp]
        L.orc_cache_set_cold.argtypes = [vp, i32]
        L.orc_cache_set_split.argtypes = [vp, i32]
        L.orc_cache_pinned.argtypes = [vp, vp]
        L.orc_pin.argtypes = [vp, vp, i32, vp]
        L.orc_pin.restype = i32
        L.orc_cache_state.argtypes = [vp, vp, vp, vp, vp]
        L.orc_cache_counters.argtypes = [vp, vp]
        L.orc_ensure.argtypes = [vp, vp, i32, i32, vp, vp]
        L.orc_ensure.restype = i32
        L.orc_stage_all.argtypes = [vp, vp, i32, vp, vp]
        L.orc_stage_all.restype = i32
        L.orc_distinct.argtypes = [vp, i32, i32]
        L.orc_distinct.restype = i32
        L.orc_install.argtypes = [vp, vp, i32, i32, i32, vp]
        L.orc_install.restype = i32
        L.orc_copy.argtypes = [vp, i32, vp, sz, vp, vp, sz, sz]
        L.orc_ffn.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_resolve.argtypes = [vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.orc_residual.argtypes = [vp, vp, i32, sz, vp]
        L.orc_rmsnorm.argtypes = [vp, i32, i32, i32, f64, vp]
        L.orc_threads.argtypes = []
        L.orc_threads.restype = i32
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


def threads():
    """OpenMP threads the oracle's parallel loops run on."""
    return int(lib().orc_threads())


def set_threads(n):
    """Run the oracle's parallel loops on n threads from now on (n < 1: all processors)."""
    lib().orc_set_threads(int(n))


def _p(a):
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return ctypes.c_void_p(a.ctypes.data)
    return ctypes.c_void_p(int(a))


def _act_dtype(wdt):
    return np.float32 if wdt == F32 else np.uint16


# ---------------------------------------------------------------- formats

def bf16_to_f64(bits):
    return lib().orc_bf16_to_f64(int(bits))


def f64_to_bf16(v):
    return lib().orc_f64_to_bf16(float(v))


def fp8_to_f64(code):
    return lib().orc_fp8_to_f64(int(code))


def e2m1_to_f64(code):
    return lib().orc_e2m1_to_f64(int(code))


def e8m0_to_f64(code):
    return lib().orc_e8m0_to_f64(int(code))


def record_bytes(wdt, H, F):
    return int(lib().orc_record_bytes(wdt, H, F))


# ---------------------------------------------------------------- router

def router_logits(x, wr, bias, wdt):
    """x [T,H] (fp32, or bf16 bits as uint16), wr [E,H], bias [E] fp32 -> logits [T,E] fp32."""
    x = np.ascontiguousarray(x)
    wr = np.ascontiguousarray(wr)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(_p(x), _p(wr), wdt, _p(bias), T, E, H, _p(out))
    return out


def topk(logits, k):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    rc = lib().orc_topk(_p(logits), T, E, k, _p(ids), _p(w))
    if rc != 0:
        raise ValueError("NaN router logit")
    return ids, w


def route(x, wr, bias, k, wdt):
    """-> ids [T,k] int32, w [T,k] float64, logits [T,E] fp32."""
    lg = router_logits(x, wr, bias, wdt)
    ids, w = topk(lg, k)
    return ids, w, lg


# ---------------------------------------------------------------- cache

class Cache:
    """Per-layer LRU slot table with the oracle's own slot (and staging) bytes.

    host: uint8 [E, stride] expert records (the bytes `synth` wrote).
    staging: optional shared uint8 [E, stride] array; allocated on first use.
    """

    def __init__(self, E, S, host=None, record_bytes_=None, staging=None, keep_bytes=True, policy=LRU):
        self.E, self.S = E, S
        self._c = lib().orc_cache_new(E, S)
        if not self._c:
            raise ValueError("bad cache shape E=%d S=%d" % (E, S))
        lib().orc_cache_set_policy(self._c, policy)
        self.host = host
        self.keep_bytes = keep_bytes and host is not None
        if self.keep_bytes:
            self.stride = host.shape[1]
            self.rb = record_bytes_ if record_bytes_ is not None else self.stride
            self.slots = np.zeros((S, self.stride), dtype=np.uint8)
            self.staging = staging
        self.max_pairs = max(S, E)

    def __del__(self):
        if getattr(self, "_c", None):
            lib().orc_cache_free(self._c)
            self._c = None

    def _desc(self):
        return np.zeros(2 + 2 * self.max_pairs, dtype=np.int32)

    @staticmethod
    def _unpack(desc):
        n = int(desc[1])
        return int(desc[0]), desc[2:2 + 2 * n].reshape(n, 2).copy()

    def ensure(self, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        slot_ids = np.empty_like(ids)
        desc = self._desc()
        k = ids.shape[-1] if ids.ndim > 1 else max(ids.size, 1)
        rc = lib().orc_ensure(self._c, _p(ids), ids.size, k, _p(slot_ids), _p(desc))
        if rc != 0:
            raise ValueError("expert id out of range")
        mode, pairs = self._unpack(desc)
        return slot_ids, mode, pairs

    def stage_all(self, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        slot_ids = np.empty_like(ids)
        desc = self._desc()
        rc = lib().orc_stage_all(self._c, _p(ids), ids.size, _p(slot_ids), _p(desc))
        if rc != 0:
            raise ValueError("expert id out of range")
        mode, pairs = self._unpack(desc)
        return slot_ids, mode, pairs

    def install(self, pred_ids, max_n):
        pred = np.ascontiguousarray(pred_ids, dtype=np.int32)
        T, k = pred.shape
        desc = self._desc()
        rc = lib().orc_install(self._c, _p(pred), T, k, max_n, _p(desc))
        if rc != 0:
            raise ValueError("expert id out of range")
        return self._unpack(desc)[1]

    def copy(self, mode, pairs):
        """Apply a copy list to the oracle's own slot/staging bytes."""
        if not self.keep_bytes or len(pairs) == 0 or mode == COLD:  # cold experts are never copied
            return
        pairs = pairs[pairs[:, 1] < self.S + self.E]  # split mode: host-computed entries move nothing
        if len(pairs) == 0:
            return
        if self.staging is None and (pairs[:, 1] >= self.S).any():
            self.staging = np.zeros((self.E, self.stride), dtype=np.uint8)
        desc = np.zeros(2 + 2 * len(pairs), dtype=np.int32)
        desc[0], desc[1] = mode, len(pairs)
        desc[2:] = pairs.reshape(-1)
        st = self.staging if self.staging is not None else np.zeros((1, self.stride), np.uint8)
        lib().orc_copy(_p(desc), self.S, _p(self.host), self.stride, _p(self.slots), _p(st), self.stride, self.rb)

    def records(self, slot_ids):
        """Pointers to the records that each (t, j) reads (slots, staging, or host records of cold experts)."""
        sid = np.ascontiguousarray(slot_ids, dtype=np.int32).reshape(-1)
        recs = (ctypes.c_void_p * sid.size)()
        st = self.staging if self.staging is not None else self.slots
        lib().orc_resolve(_p(sid), sid.size, self.S, self.E, _p(self.slots), _p(st), _p(self.host), self.stride, recs)
        return recs

    def set_cold(self, on):
        """Cold mode: later ensure calls load nothing; misses are read from their host records."""
        lib().orc_cache_set_cold(self._c, 1 if on else 0)

    def set_split(self, q):
        """Split mode: a call wider than the cache reads min(n_staged, round(n_misses * q / 256)) of its staged
        misses, the last in ascending id, from their host records instead."""
        lib().orc_cache_set_split(self._c, int(q))

    def state(self):
        so = np.empty(self.E, np.int32)
        eo = np.empty(self.S, np.int32)
        lu = np.empty(self.S, np.uint64)
        tick = np.zeros(1, np.uint64)
        lib().orc_cache_state(self._c, _p(so), _p(eo), _p(lu), _p(tick))
        return so, eo, lu, int(tick[0])

    def pin(self, experts):
        """Pin the distinct experts (replacing the pinned set); returns the load list [(expert, slot)]."""
        ex = np.ascontiguousarray(experts, dtype=np.int32).reshape(-1)
        desc = self._desc()
        if lib().orc_pin(self._c, _p(ex), ex.size, _p(desc)) != 0:
            raise ValueError("bad pin set")
        return self._unpack(desc)[1]

    def pinned(self):
        out = np.empty(self.S, np.int32)
        lib().orc_cache_pinned(self._c, _p(out))
        return out

    def scores(self):
        out = np.empty(self.S, np.uint32)
        lib().orc_cache_scores(self._c, _p(out))
        return out

    def activations(self):
        out = np.empty(self.E, np.uint32)
        lib().orc_cache_act(self._c, _p(out))
        return out

    def counters(self):
        out = np.zeros(8, np.uint64)
        lib().orc_cache_counters(self._c, _p(out))
        keys = ("calls", "hits", "misses", "staged_calls", "staged_copies", "prefetch_installs", "prefetch_hits",
                "cold")
        return dict(zip(keys, (int(v) for v in out)))


def distinct(ids, E):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    return int(lib().orc_distinct(_p(ids), ids.size, E))


# ---------------------------------------------------------------- FFN

def ffn(x, wdt, H, F, recs, w, shared=None, want_f64=False):
    """x [T,H]; recs: ctypes pointer array of T*k records; w [T,k] float64.
    -> y [T,H] rounded to the activation dtype (and the double sums)."""
    x = np.ascontiguousarray(x)
    T = x.shape[0]
    w = np.ascontiguousarray(w, dtype=np.float64)
    k = w.shape[1]
    y = np.empty((T, H), dtype=_act_dtype(wdt))
    y64 = np.empty((T, H), dtype=np.float64) if want_f64 else None
    lib().orc_ffn(_p(x), wdt, H, F, T, k, recs, _p(w), _p(shared), _p(y), _p(y64))
    return (y, y64) if want_f64 else y


def host_records(host, ids):
    """Pointers straight to host records (the brute-force, cache-free path)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    recs = (ctypes.c_void_p * ids.size)()
    base = host.ctypes.data
    for i, e in enumerate(ids):
        recs[i] = base + int(e) * host.shape[1]
    return recs


def residual(x, y, wdt):
    x = np.ascontiguousarray(x)
    y = np.ascontiguousarray(y)
    out = np.empty_like(x)
    lib().orc_residual(_p(x), _p(y), wdt, x.size, _p(out))
    return out


RMS_EPS = 1e-6


def rmsnorm(x, wdt, eps=RMS_EPS):
    """Per-token RMS normalisation of a [T, H] stream (the MoE block input)."""
    x = np.ascontiguousarray(x)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), wdt, x.shape[0], x.shape[1], eps, _p(out))
    return out


# ---------------------------------------------------------------- one layer call

class Layer:
    """One MoE layer as the oracle sees it: router + cache + FFN."""

    def __init__(self, E, S, k, H, F, wdt, host, wr, bias, shared=None, staging=None, policy=None):
        self.E, self.S, self.k, self.H, self.F, self.wdt = E, S, k, H, F, wdt
        self.wr, self.bias, self.shared = wr, bias, shared
        self.cache = Cache(E, S, host, record_bytes(wdt, H, F), staging, policy=LRU if policy is None else policy)

    def step(self, x, stage_all=False, compute_ffn=True):
        ids, w, _ = route(x, self.wr, self.bias, self.k, self.wdt)
        if stage_all:
            slot_ids, mode, pairs = self.cache.stage_all(ids)
        else:
            slot_ids, mode, pairs = self.cache.ensure(ids)
        self.cache.copy(mode, pairs)
        y = y64 = None
        if compute_ffn:
            y, y64 = ffn(x, self.wdt, self.H, self.F, self.cache.records(slot_ids), w, self.shared, want_f64=True)
        return dict(ids=ids, w=w, slot_ids=slot_ids, mode=mode, pairs=pairs, y=y, y64=y64)

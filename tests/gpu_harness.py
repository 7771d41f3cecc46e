"""Helpers for the GPU parity tests: drive the C ABI through the binding and
compare every output with the CPU oracle on the same seeded inputs."""
import ctypes

import numpy as np
import torch

import expert_offload_slot_amd as m
import oracle
import synth

_hip = None


def hip():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    return _hip


def d2h(ptr, nbytes, dtype=np.uint8):
    """Copy device memory at a raw address to a new numpy array (synchronises)."""
    torch.cuda.synchronize()
    out = np.empty(nbytes, dtype=np.uint8)
    rc = hip().hipMemcpy(out.ctypes.data, ptr, nbytes, 2)
    assert rc == 0, rc
    return out.view(dtype)


def h2d(ptr, arr):
    torch.cuda.synchronize()
    arr = np.ascontiguousarray(arr)
    rc = hip().hipMemcpy(ptr, arr.ctypes.data, arr.nbytes, 1)
    assert rc == 0, rc


def to_dev(a):
    """numpy -> cuda tensor (bf16 bits as uint16 become torch.bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_np(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def act_f64(a, wdt):
    if wdt == 0:
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_rel_err(y_gpu, y64, wdt):
    """max over tokens of ||y - ref||_inf / ||ref||_inf"""
    g = act_f64(y_gpu, wdt)
    num = np.abs(g - y64).max(axis=1)
    den = np.maximum(np.abs(y64).max(axis=1), 1e-30)
    return float((num / den).max())


TOL = {0: 1e-5, 1: 2e-2, 2: 2e-2, 3: 2e-2}


class GpuLayer:
    """One handle plus its device-side router, buffers and a mirror of its host store."""

    def __init__(self, E, S, k, H, F, wdt, max_tokens, host, wr, bias, flags=m.FLAG_AUDIT, shared=None,
                 share_host=None, share_staging=None):
        self.E, self.S, self.k, self.H, self.F, self.wdt, self.max_tokens = E, S, k, H, F, wdt, max_tokens
        self.h = m.moe_offload_create(E, S, H, F, k, wdt, max_tokens, 0, flags,
                                      share_host.h if share_host else None,
                                      share_staging.h if share_staging else None)
        self.info = m.moe_offload_query(self.h)
        if host is not None and share_host is None:
            hv = m.host_array(self.h, E)
            hv[:, :host.shape[1]] = host
        self.wr = to_dev(wr)
        self.bias = to_dev(bias)
        self.shared = to_dev(shared) if shared is not None else None
        adt = torch.float32 if wdt == 0 else torch.bfloat16
        self.ids = torch.zeros((max_tokens, k), dtype=torch.int32, device="cuda")
        self.w = torch.zeros((max_tokens, k), dtype=torch.float32, device="cuda")
        self.slot_ids = torch.zeros((max_tokens, k), dtype=torch.int32, device="cuda")
        self.y = torch.zeros((max_tokens, H), dtype=adt, device="cuda")
        self.xn = torch.zeros((max_tokens, H), dtype=adt, device="cuda")

    def close(self):
        if self.h:
            m.moe_offload_destroy(self.h)
            self.h = None

    # every call goes to torch's current stream (the capture stream inside torch.cuda.graph)
    def route(self, x, T, stream=None):
        m.moe_route_topk(self.h, x, self.wr, self.bias, T, self.ids, self.w, stream or torch.cuda.current_stream())

    def ensure(self, T, stream=None, ids=None):
        m.moe_slot_ensure(self.h, self.ids if ids is None else ids, T, self.slot_ids,
                          stream or torch.cuda.current_stream())

    def copy(self, stream=None):
        m.moe_copy_misses(self.h, stream or torch.cuda.current_stream())

    def ffn(self, x, T, stream=None, x_next=True, residual=None):
        m.moe_slot_ffn(self.h, x, self.slot_ids, self.w, T, self.shared, self.y, residual,
                       self.xn if x_next else None, stream or torch.cuda.current_stream())

    def step(self, x, T):
        self.route(x, T)
        self.ensure(T)
        self.copy()
        self.ffn(x, T)

    def copy_list(self):
        n = 2 + 2 * max(self.S, self.E)
        lst = d2h(self.info["copy_list"], 4 * n, np.int32)
        mode, cnt = int(lst[0]), int(lst[1])
        return mode, lst[2:2 + 2 * cnt].reshape(cnt, 2).copy()

    def prefetch_list(self):
        lst = d2h(self.info["prefetch_list"], 4 * (2 + 2 * self.S), np.int32)
        cnt = int(lst[1])
        return lst[2:2 + 2 * cnt].reshape(cnt, 2).copy()

    def table(self):
        so = d2h(self.info["slot_of"], 4 * self.E, np.int32)
        eo = d2h(self.info["expert_of"], 4 * self.S, np.int32)
        lu = d2h(self.info["last_use"], 8 * self.S, np.uint64)
        return so, eo, lu

    def scores(self):
        return d2h(self.info["score"], 4 * self.S, np.uint32)

    def pinned(self):
        return d2h(self.info["pinned"], 4 * self.S, np.int32)

    def activations(self):
        return d2h(self.info["act"], 4 * self.E, np.uint32)

    def stats(self):
        return m.moe_offload_stats(self.h)

    def slot_bytes(self, s, nbytes):
        return d2h(self.info["slots"] + s * self.info["record_stride"], nbytes)

    def staging_bytes(self, e, nbytes):
        return d2h(self.info["staging"] + e * self.info["record_stride"], nbytes)


def oracle_policy(flags):
    """The oracle's eviction policy for a handle's create flags."""
    if flags & m.FLAG_SCORED:
        return oracle.SCORED
    if flags & m.FLAG_FREQ:
        return oracle.FREQ
    return oracle.LRU


def make_layer_inputs(seed, layer, E, H, F, wdt, zipf_s, shared=False):
    host = synth.records(seed, layer, E, H, F, wdt)
    wr, b = synth.router(seed, layer, E, H, wdt, zipf_s=zipf_s)
    sh = synth.records(seed, layer, 1, H, F, wdt, shared=True)[0] if shared else None
    return host, wr, b, sh


def compare_call(gl, ol_step, T, y64=None, check_table=True, oracle_cache=None):
    """Bit-exact: ids, slot ids, copy list, table; weights within 1e-5; y within TOL."""
    ids = to_np(gl.ids[:T])
    assert np.array_equal(ids, ol_step["ids"]), (ids, ol_step["ids"])
    w = to_np(gl.w[:T])
    assert np.abs(w - ol_step["w"]).max() <= 1e-5
    sid = to_np(gl.slot_ids[:T])
    assert np.array_equal(sid, ol_step["slot_ids"]), (sid, ol_step["slot_ids"])
    mode, pairs = gl.copy_list()
    assert mode == ol_step["mode"] and np.array_equal(pairs, ol_step["pairs"]), (mode, pairs, ol_step["mode"],
                                                                                 ol_step["pairs"])
    if check_table and oracle_cache is not None:
        so, eo, lu = gl.table()
        oso, oeo, olu, _ = oracle_cache.state()
        assert np.array_equal(so, oso) and np.array_equal(eo, oeo) and np.array_equal(lu, olu)
        assert np.array_equal(gl.scores(), oracle_cache.scores())
        assert np.array_equal(gl.pinned(), oracle_cache.pinned())
        assert np.array_equal(gl.activations(), oracle_cache.activations())
    if y64 is not None:
        err = row_rel_err(to_np(gl.y[:T]), y64, gl.wdt)
        assert err <= TOL[gl.wdt], err
        return err
    return None

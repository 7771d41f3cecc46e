"""Python binding of libmoe_offload.so — the offloaded MoE layer step on MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors may be passed as torch tensors (their data_ptr() is used) or
as integer addresses; streams as torch streams, integers or None (null stream).
The functions keep the C names; a non-zero return code raises MoeError with
the library's message.  The library must have been built
(``python -m expert_offload_slot_amd.build`` or ``__graft_entry__.build()``);
there is no fallback path.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmoe_offload.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe_offload.h")

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3
MODE_SLOTS, MODE_STAGED, MODE_STAGED_ALL = 0, 1, 2
FLAG_AUDIT, FLAG_HOST_COHERENT, FLAG_SCORED, FLAG_FREQ = 1, 2, 4, 8
DEV_ERR_BAD_ID, DEV_ERR_NAN, DEV_ERR_AUDIT, DEV_ERR_HOST_TIMEOUT = 1, 2, 4, 8
EINVAL, ENOMEM, EHIP, EUNSUPPORTED, EDEVICE = -1, -2, -3, -4, -5


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("num_slots", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("top_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("device", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("share_host", ctypes.c_void_p), ("share_staging", ctypes.c_void_p)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("calls", "hits", "misses", "staged_calls", "staged_copies",
                                               "prefetch_installs", "prefetch_hits", "bytes_copied", "tick")] + \
               [("error", ctypes.c_int32), ("resident", ctypes.c_int32), ("cold_misses", ctypes.c_uint64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


KERNEL_KINDS = ("logits", "topk", "decide", "ensure", "install", "copy", "prefetch_copy", "group", "gateup",
                "down", "combine", "stage")


class KernelTimes(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * len(KERNEL_KINDS)), ("launches", ctypes.c_uint64 * len(KERNEL_KINDS))]


class Info(ctypes.Structure):
    _fields_ = [("slot_of", ctypes.c_void_p), ("expert_of", ctypes.c_void_p), ("last_use", ctypes.c_void_p),
                ("copy_list", ctypes.c_void_p), ("prefetch_list", ctypes.c_void_p), ("slots", ctypes.c_void_p),
                ("staging", ctypes.c_void_p), ("host", ctypes.c_void_p), ("host_dev", ctypes.c_void_p),
                ("ffn_h", ctypes.c_void_p), ("ffn_part", ctypes.c_void_p), ("ffn_groups", ctypes.c_void_p),
                ("record_bytes", ctypes.c_size_t), ("record_stride", ctypes.c_size_t)] + \
               [(n, ctypes.c_int32) for n in ("E", "S", "H", "F", "k", "dtype", "max_tokens", "device")] + \
               [("score", ctypes.c_void_p), ("pinned", ctypes.c_void_p), ("act", ctypes.c_void_p)]


class ChainBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "xn", "y", "ids", "w", "slot_ids", "pred")] + \
               [("act_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """Load libmoe_offload.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_offload.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
        sig = {
            "moe_offload_create": ([P(Desc), P(vp)], i32),
            "moe_offload_destroy": ([vp], None),
            "moe_offload_auto_slots": ([P(Desc), i32, i32, ctypes.c_uint64, ctypes.c_uint64, P(ctypes.c_int32)], i32),
            "moe_offload_host_records": ([vp, P(vp), P(ctypes.c_size_t), P(ctypes.c_size_t)], i32),
            "moe_route_topk": ([vp, vp, vp, vp, i32, vp, vp, vp], i32),
            "moe_slot_ensure": ([vp, vp, i32, vp, vp], i32),
            "moe_copy_misses": ([vp, vp], i32),
            "moe_slot_ffn": ([vp, vp, vp, vp, i32, vp, vp, vp, vp, vp], i32),
            "moe_slot_ffn_noalloc": ([vp, vp, vp, vp, i32, vp, vp, vp, vp, vp], i32),
            "moe_slot_ffn_host_cold": ([vp, vp, vp, vp, i32, vp, vp, vp, vp, vp], i32),
            "moe_offload_set_cold": ([vp, i32, vp, P(ctypes.c_int32), P(ctypes.c_double), P(ctypes.c_double)], i32),
            "moe_offload_set_split": ([vp, i32, vp], i32),
            "moe_offload_set_ffn_path": ([vp, i32], i32),
            "moe_offload_set_gemm_waves": ([vp, i32], i32),
            "moe_rmsnorm": ([vp, vp, i32, i32, i32, ctypes.c_float, vp], i32),
            "moe_prefill_stage": ([vp, vp, i32, vp, P(ctypes.c_int32), vp], i32),
            "moe_prefetch_install": ([vp, vp, i32, i32, vp], i32),
            "moe_offload_pin": ([vp, vp, i32, vp], i32),
            "moe_copy_prefetch": ([vp, vp], i32),
            "moe_offload_stats": ([vp, P(Stats)], i32),
            "moe_offload_reset": ([vp, vp], i32),
            "moe_offload_query": ([vp, P(Info)], i32),
            "moe_offload_last_error": ([], ctypes.c_char_p),
            "moe_offload_profile": ([vp, i32], i32),
            "moe_offload_kernel_times": ([vp, P(KernelTimes)], i32),
            "moe_chain_create": ([P(vp), i32, P(vp), P(vp), P(vp), i32, i32, P(vp)], i32),
            "moe_chain_get_buffers": ([vp, P(ChainBuffers)], i32),
            "moe_chain_run": ([vp, vp], i32),
            "moe_chain_run_eager": ([vp, vp], i32),
            "moe_chain_set_read_through": ([vp, i32], i32),
            "moe_chain_destroy": ([vp], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def header_functions():
    """Names of the functions declared in include/moe_offload.h."""
    import re
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def _addr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    raise TypeError("cannot take the address of %r" % type(t))


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc):
    if rc != 0:
        raise MoeError(rc, lib().moe_offload_last_error().decode())
    return rc


def moe_offload_create(E, S, H, F, k, dtype, max_tokens, device=0, flags=0, share_host=None, share_staging=None):
    d = Desc(E, S, H, F, k, dtype, max_tokens, device, flags, share_host, share_staging)
    h = ctypes.c_void_p()
    _check(lib().moe_offload_create(ctypes.byref(d), ctypes.byref(h)))
    return h.value


def moe_offload_auto_slots(E, H, F, k, dtype, max_tokens, layers, reserve_bytes, free_bytes=0, share_staging=True,
                           device=0, flags=0):
    """Slots per layer that `layers` handles of this shape can take from free device memory, leaving
    reserve_bytes (free_bytes = 0: the device's free memory now)."""
    d = Desc(E, k, H, F, k, dtype, max_tokens, device, flags, None, None)
    out = ctypes.c_int32()
    _check(lib().moe_offload_auto_slots(ctypes.byref(d), layers, 1 if share_staging else 0, reserve_bytes,
                                        free_bytes, ctypes.byref(out)))
    return out.value


def moe_offload_destroy(h):
    lib().moe_offload_destroy(h)


def moe_offload_host_records(h):
    """-> (host address, record_stride, record_bytes)"""
    p, st, rb = ctypes.c_void_p(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_offload_host_records(h, ctypes.byref(p), ctypes.byref(st), ctypes.byref(rb)))
    return p.value, st.value, rb.value


def moe_route_topk(h, x, w_router, bias, T, ids, w, stream=None):
    return _check(lib().moe_route_topk(h, _addr(x), _addr(w_router), _addr(bias), T, _addr(ids), _addr(w),
                                       _stream(stream)))


def moe_slot_ensure(h, ids, T, slot_ids, stream=None):
    return _check(lib().moe_slot_ensure(h, _addr(ids), T, _addr(slot_ids), _stream(stream)))


def moe_copy_misses(h, stream=None):
    return _check(lib().moe_copy_misses(h, _stream(stream)))


def moe_slot_ffn(h, x, slot_ids, w, T, shared_record, y, residual=None, x_next=None, stream=None):
    return _check(lib().moe_slot_ffn(h, _addr(x), _addr(slot_ids), _addr(w), T, _addr(shared_record), _addr(y),
                                     _addr(residual), _addr(x_next), _stream(stream)))


def moe_slot_ffn_noalloc(h, x, slot_ids, w, T, shared_record, y, residual=None, x_next=None, stream=None):
    return _check(lib().moe_slot_ffn_noalloc(h, _addr(x), _addr(slot_ids), _addr(w), T, _addr(shared_record),
                                             _addr(y), _addr(residual), _addr(x_next), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20

COLD_OFF, COLD_ON, COLD_AUTO, COLD_SPLIT = 0, 1, 2, 3
MODE_COLD = 3


def moe_offload_set_cold(h, mode, stream=None):
    """-> (chosen: 0/1, or the host share q for COLD_SPLIT; host FFN us per record, link us per record); the
    times are measured for COLD_AUTO and COLD_SPLIT only."""
    chosen, cpu, link = ctypes.c_int32(), ctypes.c_double(), ctypes.c_double()
    _check(lib().moe_offload_set_cold(h, mode, _stream(stream), ctypes.byref(chosen), ctypes.byref(cpu),
                                      ctypes.byref(link)))
    return chosen.value, cpu.value, link.value


FFN_AUTO, FFN_DECODE, FFN_GEMM = 0, 1, 2


def moe_offload_set_ffn_path(h, path):
    return _check(lib().moe_offload_set_ffn_path(h, path))


def moe_offload_set_gemm_waves(h, waves):
    return _check(lib().moe_offload_set_gemm_waves(h, waves))


def moe_offload_set_split(h, q, stream=None):
    return _check(lib().moe_offload_set_split(h, q, _stream(stream)))


def moe_slot_ffn_host_cold(h, x, slot_ids, w, T, shared_record, y, residual=None, x_next=None, stream=None):
    return _check(lib().moe_slot_ffn_host_cold(h, _addr(x), _addr(slot_ids), _addr(w), T, _addr(shared_record),
                                               _addr(y), _addr(residual), _addr(x_next), _stream(stream)))

RMS_EPS = 1e-6


def moe_rmsnorm(x, out, T, H, dtype, eps=RMS_EPS, stream=None):
    return _check(lib().moe_rmsnorm(_addr(x), _addr(out), T, H, dtype, eps, _stream(stream)))


def moe_prefill_stage(h, ids, T, slot_ids, stream=None):
    """-> 1 if the whole layer was staged, else 0."""
    out = ctypes.c_int32(-1)
    _check(lib().moe_prefill_stage(h, _addr(ids), T, _addr(slot_ids), ctypes.byref(out), _stream(stream)))
    return out.value


def moe_offload_pin(h, experts_dev, n, stream=None):
    return _check(lib().moe_offload_pin(h, _addr(experts_dev) if n else None, n, _stream(stream)))


def moe_prefetch_install(h, pred_ids, T, max_n, stream=None):
    return _check(lib().moe_prefetch_install(h, _addr(pred_ids), T, max_n, _stream(stream)))


def moe_copy_prefetch(h, stream=None):
    return _check(lib().moe_copy_prefetch(h, _stream(stream)))


def moe_offload_profile(h, enable):
    return _check(lib().moe_offload_profile(h, int(bool(enable))))


def moe_offload_kernel_times(h):
    """{kind: (summed ms, timed launches)} for the kinds of KERNEL_KINDS."""
    t = KernelTimes()
    _check(lib().moe_offload_kernel_times(h, ctypes.byref(t)))
    return {k: (t.ms[i], t.launches[i]) for i, k in enumerate(KERNEL_KINDS)}


def moe_offload_stats(h):
    s = Stats()
    _check(lib().moe_offload_stats(h, ctypes.byref(s)))
    return s.as_dict()


def moe_offload_reset(h, stream=None):
    return _check(lib().moe_offload_reset(h, _stream(stream)))


def moe_offload_query(h):
    i = Info()
    _check(lib().moe_offload_query(h, ctypes.byref(i)))
    return {n: getattr(i, n) for n, _ in Info._fields_}


def host_array(h, E):
    """The handle's pinned host store as a numpy uint8 array [E, record_stride] (no copy)."""
    p, stride, _ = moe_offload_host_records(h)
    buf = (ctypes.c_uint8 * (E * stride)).from_address(p)
    return np.frombuffer(buf, dtype=np.uint8).reshape(E, stride)


def moe_chain_create(layers, w_router, bias, T, prefetch_n=0, shared_records=None):
    """layers: handles; w_router, bias, shared_records: per-layer tensors/addresses (shared entries may be None)."""
    L = len(layers)
    arr = lambda xs: (ctypes.c_void_p * L)(*[_addr(v) for v in xs])
    out = ctypes.c_void_p()
    sh = arr(shared_records) if shared_records is not None else None
    _check(lib().moe_chain_create(arr(layers), L, arr(w_router), arr(bias), sh, T, prefetch_n, ctypes.byref(out)))
    return out.value


def moe_chain_get_buffers(c):
    b = ChainBuffers()
    _check(lib().moe_chain_get_buffers(c, ctypes.byref(b)))
    return {n: getattr(b, n) for n, _ in ChainBuffers._fields_}


def moe_chain_run(c, stream=None):
    return _check(lib().moe_chain_run(c, _stream(stream)))


def moe_chain_run_eager(c, stream=None):
    return _check(lib().moe_chain_run_eager(c, _stream(stream)))


def moe_chain_set_read_through(c, on):
    return _check(lib().moe_chain_set_read_through(c, 1 if on else 0))


def moe_chain_destroy(c):
    lib().moe_chain_destroy(c)

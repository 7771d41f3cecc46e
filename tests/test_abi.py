"""The C-ABI library loads without a GPU and exports every function include/moe_offload.h declares.
No compute calls here."""
import ctypes
import subprocess

import expert_offload_slot_amd as m


def test_library_exports_every_header_function():
    names = m.header_functions()
    assert len(names) >= 14
    L = m.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_exported_symbols_are_plain_c():
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in m.header_functions():
        assert n in exported  # unmangled extern "C" names


def test_struct_sizes_match_the_header_layout():
    # moe_offload_desc: 9 x 32-bit fields + 2 pointers; moe_stats: 9 x u64 + 2 x i32 + 1 x u64
    assert ctypes.sizeof(m.Desc) == 9 * 4 + 4 + 2 * 8
    assert ctypes.sizeof(m.Stats) == 9 * 8 + 2 * 4 + 8
    # moe_kernel_times: MOE_K_N doubles + MOE_K_N u64
    assert ctypes.sizeof(m.KernelTimes) == 2 * 8 * len(m.KERNEL_KINDS)


def test_kernel_kinds_match_the_header_enum():
    import re
    text = open(m.HEADER).read()
    kinds = dict((n, int(v)) for n, v in re.findall(r"MOE_K_(\w+)\s*=\s*(\d+)", text))
    assert kinds.pop("N") == len(m.KERNEL_KINDS)
    assert sorted(kinds.values()) == list(range(len(m.KERNEL_KINDS)))


def test_last_error_is_empty_string_initially():
    assert isinstance(m.lib().moe_offload_last_error(), bytes)


def test_null_handles_are_rejected_before_any_device_call():
    """Every per-handle call checks its handle first and returns EINVAL with a message; destroy
    calls are null-safe.  No HIP call is reached, so this runs without a GPU."""
    L = m.lib()
    calls = {
        "moe_route_topk": (None, None, None, None, 1, None, None, None),
        "moe_slot_ensure": (None, None, 1, None, None),
        "moe_copy_misses": (None, None),
        "moe_slot_ffn": (None, None, None, None, 1, None, None, None, None, None),
        "moe_prefill_stage": (None, None, 1, None, None, None),
        "moe_prefetch_install": (None, None, 1, 1, None),
        "moe_offload_pin": (None, None, 0, None),
        "moe_copy_prefetch": (None, None),
        "moe_offload_stats": (None, None),
        "moe_offload_reset": (None, None),
        "moe_offload_query": (None, None),
        "moe_offload_profile": (None, 1),
        "moe_offload_kernel_times": (None, None),
        "moe_offload_host_records": (None, None, None, None),
        "moe_chain_run": (None, None),
        "moe_chain_run_eager": (None, None),
        "moe_chain_set_read_through": (None, 1),
        "moe_chain_get_buffers": (None, None),
        "moe_slot_ffn_host_cold": (None, None, None, None, 1, None, None, None, None, None),
        "moe_slot_ffn_noalloc": (None, None, None, None, 1, None, None, None, None, None),
        "moe_offload_set_cold": (None, 1, None, None, None, None),
        "moe_offload_set_split": (None, 128, None),
        "moe_offload_set_ffn_path": (None, 0),
        "moe_offload_set_gemm_waves": (None, 0),
    }
    for name, args in calls.items():
        rc = getattr(L, name)(*args)
        assert rc == m.EINVAL, (name, rc)
        assert L.moe_offload_last_error(), name
    assert L.moe_offload_create(None, None) == m.EINVAL
    assert b"null" in L.moe_offload_last_error()
    assert L.moe_chain_create(None, 0, None, None, None, 1, 0, None) == m.EINVAL
    assert L.moe_rmsnorm(None, None, 1, 64, m.BF16, 1e-6, None) == m.EINVAL
    L.moe_offload_destroy(None)
    L.moe_chain_destroy(None)


def test_rmsnorm_rejects_bad_sizes_without_a_device():
    import numpy as np
    L = m.lib()
    buf = np.zeros(64, np.float32)
    p = buf.ctypes.data
    for T, H, eps in ((0, 64, 1e-6), (1, 60, 1e-6), (1, 4, 1e-6), (1, 64, 0.0), (1, 64, -1.0)):
        assert L.moe_rmsnorm(p, p, T, H, m.F32, eps, None) == m.EINVAL, (T, H, eps)


def test_exclusive_eviction_flags_are_rejected_before_any_device_call():
    """Scored and activation-aware eviction are two victim orders: asking for both is EINVAL, decided
    from the descriptor alone (no device is touched, so this runs without a GPU)."""
    L = m.lib()
    d = m.Desc(8, 4, 128, 128, 2, m.BF16, 4, 0, m.FLAG_SCORED | m.FLAG_FREQ, None, None)
    out = ctypes.c_void_p()
    assert L.moe_offload_create(ctypes.byref(d), ctypes.byref(out)) == m.EINVAL
    assert b"exclusive" in L.moe_offload_last_error() and not out.value

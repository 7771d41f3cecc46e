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
    # moe_offload_desc: 9 x 32-bit fields + 2 pointers; moe_stats: 9 x u64 + 2 x i32
    assert ctypes.sizeof(m.Desc) == 9 * 4 + 4 + 2 * 8
    assert ctypes.sizeof(m.Stats) == 9 * 8 + 2 * 4
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

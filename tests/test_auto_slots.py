"""Automatic slot sizing (xinfer-ai docs, "Options", auto): the slot count every layer gets from a
given amount of free device memory.  With free_bytes given the call is arithmetic only, so these run
without a GPU.  Pinned to the rule's own structure: one more slot per layer costs exactly
layers x record_stride; the reserve and a shared staging buffer shift the thresholds by exactly their
size; the count never leaves [top_k, E]."""
import pytest

import expert_offload_slot_amd as m

GB = 1 << 30
QWEN = dict(E=128, H=2048, F=768, k=8, dtype=m.BF16, max_tokens=32)
STRIDE = 9437184  # 3 x 2048 x 768 x 2 bytes, already a multiple of 4096


def auto(free, layers=48, reserve=0, share=True, shape=QWEN):
    return m.moe_offload_auto_slots(shape["E"], shape["H"], shape["F"], shape["k"], shape["dtype"],
                                    shape["max_tokens"], layers, reserve, free, share)


def threshold(layers=48, reserve=0, share=True):
    """smallest free byte count that gives top_k slots per layer (binary search)"""
    lo, hi = 1, 1 << 44
    while lo < hi:
        mid = (lo + hi) // 2
        try:
            auto(mid, layers, reserve, share)
            hi = mid
        except m.MoeError as e:
            assert e.code == m.ENOMEM
            lo = mid + 1
    return lo


def test_each_slot_costs_one_record_per_layer():
    f0 = threshold()
    assert auto(f0) == QWEN["k"]
    with pytest.raises(m.MoeError) as ei:
        auto(f0 - 1)
    assert ei.value.code == m.ENOMEM
    for j in (1, 5, 18, 100):
        step = 48 * STRIDE
        got = auto(f0 + j * step)
        assert got == min(QWEN["E"], QWEN["k"] + j)
        assert auto(f0 + j * step - 1) == min(QWEN["E"], QWEN["k"] + j - 1)


def test_threshold_is_slots_plus_staging_plus_state():
    f0 = threshold()
    staging = QWEN["E"] * STRIDE
    state = (f0 - QWEN["k"] * 48 * STRIDE - staging) / 48
    assert 0 < state < 64 << 20  # tables, lists and the 32-token workspaces of one layer


def test_reserve_and_staging_shift_the_threshold_exactly():
    f0 = threshold()
    r = 3 * GB + 12345
    assert threshold(reserve=r) == f0 + r
    # one staging buffer per layer instead of one shared buffer: 47 more [E, stride] buffers
    assert threshold(share=False) == f0 + 47 * QWEN["E"] * STRIDE


def test_count_is_clamped_to_the_expert_count():
    assert auto(1 << 44) == QWEN["E"]  # 16 TiB: every expert resident
    assert auto(1 << 44, layers=1) == QWEN["E"]


def test_bad_descriptors_are_rejected():
    with pytest.raises(m.MoeError) as ei:
        auto(GB, layers=0)
    assert ei.value.code == m.EINVAL
    bad = dict(QWEN, H=100)
    with pytest.raises(m.MoeError) as ei:
        auto(GB, shape=bad)
    assert ei.value.code == m.EUNSUPPORTED

"""GPU routing parity on inputs built to hit the top-k's tie rules.

Router rows are repeated so that many logits are exactly equal (the oracle and
the kernel both take every logit in the same binary32 order), and biases of
-inf make whole groups of experts tie at -inf.  Expert ids must match the
oracle bit for bit (order: logit descending, id ascending); weights within
1e-5 relative.  Expert counts cover one to sixteen 64-lane registers per lane,
with and without a ragged last register.
"""
import numpy as np
import pytest
import torch

import expert_offload_slot_amd as m
import oracle
from gpu_harness import to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (100, 16), (128, 8), (256, 8), (1000, 16), (1024, 4)])
def test_topk_ties_and_infinities(E, k):
    print("case E=%d k=%d" % (E, k), flush=True)
    T, H, F = 5, 64, 64
    rng = np.random.default_rng(E * 31 + k)
    x = rng.standard_normal((T, H)).astype(np.float32)
    base = rng.standard_normal((4, H)).astype(np.float32)
    wr = np.ascontiguousarray(base[np.arange(E) % 4])          # four distinct logits per token
    bias = np.zeros(E, dtype=np.float32)
    bias[np.arange(E) % 7 == 3] = -np.inf                      # groups tied at -inf
    if E >= 100:
        bias[np.arange(E) % 2 == 1] = -np.inf                  # fewer finite than some k
        bias[(np.arange(E) % 2 == 0) & (np.arange(E) >= 2 * k // 3)] = -np.inf
    ids_ref, w_ref, _ = oracle.route(x, wr, bias, k, 0)
    h = m.moe_offload_create(E, k, H, F, k, m.F32, T)
    try:
        xd, wd, bd = to_dev(x), to_dev(wr), to_dev(bias)
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        m.moe_route_topk(h, xd, wd, bd, T, ids, w)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(ids), ids_ref)
        np.testing.assert_allclose(to_np(w), w_ref, rtol=1e-5, atol=1e-7)
        assert m.moe_offload_stats(h)["error"] == 0
    finally:
        m.moe_offload_destroy(h)

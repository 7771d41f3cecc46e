"""The host-CPU expert FFN of cold and split mode (csrc/host_ffn.cpp), on the CPU: every pair whose record
index is S + E + e is computed from expert e's host record and must match the oracle's plain definition of
that expert's output (fp64) within the GPU path's tolerance; every other row of the output is left alone.
Token counts above the 8 rows a pass holds, several cold experts per call, every weight format."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_offload_slot_amd", "csrc")


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host_ffn") / "libhostffn.so")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", "-ffp-contract=off",
                           "-I", CSRC, os.path.join(ROOT, "tests", "host_ffn_shim.cpp"),
                           os.path.join(CSRC, "host_ffn.cpp"), "-o", out])
    L = ctypes.CDLL(out)
    vp = ctypes.c_void_p
    L.shim_host_cold_ffn.argtypes = [vp, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int,
                                     ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp]
    L.shim_host_cold_ffn.restype = ctypes.c_int
    return L


TOL = {0: 1e-5, 1: 2e-2, 2: 2e-2, 3: 2e-2}


@pytest.mark.parametrize("wdt,H,F", [(0, 128, 192), (1, 256, 384), (2, 256, 256), (3, 256, 512)])
@pytest.mark.parametrize("T", [1, 5, 11])
def test_host_ffn_matches_the_plain_definition(shim, wdt, H, F, T):
    E, S, k = 8, 3, 2
    rng = np.random.default_rng(100 * wdt + T)
    host = synth.records(17, wdt, E, H, F, wdt)
    x = synth.tokens(17, 3 + T, T, H, 1, 0.0, wdt)[0]
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    cold = rng.random((T, k)) < 0.6
    cold[0, 0] = True
    # cold pairs at S + E + e; the rest at a slot or a staging record (not the host's to compute)
    sid = np.where(cold, S + E + ids, np.where(rng.random((T, k)) < 0.5, ids % S, S + ids)).astype(np.int32)
    out = np.full((T * k, H), np.float32(12345.0))
    n = shim.shim_host_cold_ffn(host.ctypes.data, host.shape[1], wdt, H, F, x.ctypes.data, T, k, sid.ctypes.data, S,
                                E, out.ctypes.data)
    assert n >= 1
    worst = 0.0
    for t in range(T):
        for j in range(k):
            row = out[t * k + j]
            if not cold[t, j]:
                assert np.all(row == np.float32(12345.0)), (t, j)
                continue
            _, ref = oracle.ffn(x[t:t + 1], wdt, H, F, oracle.host_records(host, ids[t:t + 1, j:j + 1]),
                                np.ones((1, 1)), want_f64=True)
            err = np.abs(row.astype(np.float64) - ref[0]).max() / max(np.abs(ref[0]).max(), 1e-30)
            assert err <= TOL[wdt], (t, j, err)
            worst = max(worst, err)
    # the host keeps h in fp32 and sums in fp32: far inside the GPU path's tolerance
    assert worst <= 1e-4, worst


def test_host_ffn_one_expert_shared_by_many_tokens(shim):
    """19 tokens on one cold expert (three passes of at most 8 rows), bf16: each token's row is that expert's
    output for that token alone."""
    E, S, k, H, F, wdt, T = 4, 2, 1, 256, 256, 1, 19
    host = synth.records(23, 0, E, H, F, wdt)
    x = synth.tokens(23, 1, T, H, 1, 0.0, wdt)[0]
    sid = np.full((T, k), S + E + 3, np.int32)
    out = np.zeros((T, H), np.float32)
    shim.shim_host_cold_ffn(host.ctypes.data, host.shape[1], wdt, H, F, x.ctypes.data, T, k, sid.ctypes.data, S, E,
                            out.ctypes.data)
    _, ref = oracle.ffn(x, wdt, H, F, oracle.host_records(host, np.full((T, 1), 3)), np.ones((T, 1)), want_f64=True)
    err = (np.abs(out.astype(np.float64) - ref).max(axis=1) / np.abs(ref).max(axis=1)).max()
    assert err <= 1e-4, err

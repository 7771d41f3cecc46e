"""Pins for the oracle's expert FFN and combine.

  * numpy float64 matrix products on records decoded with torch's own
    bf16 / float8_e4m3fn / float8_e8m0fnu dtypes and the E2M1 bit-field
    formula (the brute force; no cache involved) agree with the oracle to
    1e-12 relative;
  * an MXFP4 record and a bf16 record holding the same weights (every MXFP4
    weight is a bf16 value) give bitwise identical oracle outputs;
  * placement invariance: outputs through the oracle's own slot copies are
    bitwise identical at every slot count S = k..E and with every call
    staged, and equal the cache-free result (the pages' point that which
    slot an expert occupies affects neither the routing nor the arithmetic);
  * special cases: x = 0 gives y = 0; k = 1 gives one expert's output;
    zero down-projection gives 0.
"""
import numpy as np
import pytest
import torch


def e2m1_closed_form(code):
    # OCP MX v1.0 E2M1 bit fields: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def _decode_mx(rec_codes, rec_scales, R, C):
    # codes: two per byte, element 2i in the low nibble; scales: E8M0, one per 32 of a row
    b = np.frombuffer(rec_codes[:R * C // 2].tobytes(), np.uint8)
    codes = np.stack([b & 15, b >> 4], axis=1).reshape(-1)
    lut = np.array([e2m1_closed_form(c) for c in range(16)])
    sc = torch.from_numpy(np.frombuffer(rec_scales[:R * C // 32].tobytes(), np.uint8).copy()).view(
        torch.float8_e8m0fnu).double().numpy()
    return lut[codes].reshape(R, C) * np.repeat(sc.reshape(R, C // 32), 32, axis=1)


def _decode(raw, wdt, n):
    if wdt == 0:
        return np.frombuffer(raw[:4 * n].tobytes(), np.float32).astype(np.float64)
    if wdt == 1:
        return torch.from_numpy(np.frombuffer(raw[:2 * n].tobytes(), np.int16).copy()).view(torch.bfloat16).double().numpy()
    return torch.from_numpy(np.frombuffer(raw[:n].tobytes(), np.uint8).copy()).view(torch.float8_e4m3fn).double().numpy()


def expert_mats(rec, wdt, H, F):
    n = H * F
    if wdt == 3:
        sc0 = 3 * n // 2
        return (_decode_mx(rec[0:], rec[sc0:], F, H), _decode_mx(rec[n // 2:], rec[sc0 + n // 32:], F, H),
                _decode_mx(rec[n:], rec[sc0 + 2 * n // 32:], H, F))
    esz = {0: 4, 1: 2, 2: 1}[wdt]
    g = _decode(rec[0:], wdt, n).reshape(F, H)
    u = _decode(rec[esz * n:], wdt, n).reshape(F, H)
    d = _decode(rec[2 * esz * n:], wdt, n).reshape(H, F)
    if wdt == 2:
        nb = (H // 128) * (F // 128)
        sc = np.frombuffer(rec[3 * n:3 * n + 12 * nb].tobytes(), np.float32).astype(np.float64)
        blk = np.ones((128, 128))
        g = g * np.kron(sc[:nb].reshape(F // 128, H // 128), blk)
        u = u * np.kron(sc[nb:2 * nb].reshape(F // 128, H // 128), blk)
        d = d * np.kron(sc[2 * nb:].reshape(H // 128, F // 128), blk)
    return g, u, d


def act_f64(x, wdt):
    if wdt == 0:
        return x.astype(np.float64)
    return torch.from_numpy(x.astype(np.int16)).view(torch.bfloat16).double().numpy()


def brute_layer(x, host, ids, w, wdt, H, F, shared=None):
    xv = act_f64(x, wdt)
    y = np.zeros((x.shape[0], H))
    cache = {}
    for t in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = expert_mats(host[e], wdt, H, F)
            g, u, d = cache[e]
            a, b = g @ xv[t], u @ xv[t]
            y[t] += w[t, j] * (d @ (a / (1.0 + np.exp(-a)) * b))
        if shared is not None:
            g, u, d = expert_mats(shared, wdt, H, F)
            a, b = g @ xv[t], u @ xv[t]
            y[t] += d @ (a / (1.0 + np.exp(-a)) * b)
    return y


CASES = [  # wdt, E, k, H, F, T
    (0, 8, 2, 64, 128, 4),
    (1, 16, 4, 128, 64, 3),
    (2, 6, 2, 256, 256, 2),
    (3, 6, 2, 256, 512, 2),
]


@pytest.mark.parametrize("wdt,E,k,H,F,T", CASES)
def test_ffn_matches_numpy_brute_force(orc, syn, wdt, E, k, H, F, T):
    host = syn.records(21, 0, E, H, F, wdt)
    wr, b = syn.router(21, 0, E, H, wdt, zipf_s=0.0)
    x = syn.tokens(21, 9, T, H, 1, 0.0, wdt)[0]
    ids, w, _ = orc.route(x, wr, b, k, wdt)
    shared = syn.records(21, 0, 1, H, F, wdt, shared=True)[0] if wdt >= 2 else None
    y, y64 = orc.ffn(x, wdt, H, F, orc.host_records(host, ids), w, shared, want_f64=True)
    ref = brute_layer(x, host, ids, w, wdt, H, F, shared)
    assert np.max(np.abs(y64 - ref)) <= 1e-12 * np.max(np.abs(ref))
    # output is the double sum rounded once to the activation dtype
    if wdt == 0:
        assert np.array_equal(y, y64.astype(np.float32))
    else:
        assert np.array_equal(y, np.array([orc.f64_to_bf16(v) for v in y64.reshape(-1)], np.uint16).reshape(y.shape))


@pytest.mark.parametrize("wdt,E,k,H,F,T", CASES[:2])
def test_placement_invariance_in_the_oracle(orc, syn, wdt, E, k, H, F, T):
    host = syn.records(5, 0, E, H, F, wdt)
    wr, b = syn.router(5, 0, E, H, wdt, zipf_s=0.0)  # flat routing: many misses and evictions
    xs = syn.tokens(5, 3, T, H, 12, 0.0, wdt)
    ref = [orc.ffn(xs[s], wdt, H, F, orc.host_records(host, orc.route(xs[s], wr, b, k, wdt)[0]),
                   orc.route(xs[s], wr, b, k, wdt)[1]) for s in range(len(xs))]
    modes = set()
    for S in list(range(k, E + 1)) + ["stage_all"]:
        L = orc.Layer(E, E if S == "stage_all" else S, k, H, F, wdt, host, wr, b)
        for s in range(len(xs)):
            r = L.step(xs[s], stage_all=(S == "stage_all"))
            modes.add(r["mode"])
            assert np.array_equal(r["y"], ref[s]), (S, s)
    assert modes == {0, 1, 2}  # slots, decode staging and whole-layer staging all exercised
    # split mode: of a wide call's staged misses, half are read from their host records at S + E + e
    for S in (k, (k + E) // 2):
        L = orc.Layer(E, S, k, H, F, wdt, host, wr, b)
        L.cache.set_split(128)
        for s in range(len(xs)):
            r = L.step(xs[s])
            assert np.array_equal(r["y"], ref[s]), ("split", S, s)
    # host-computed cold experts: the misses are read from their host records at S + E + e
    for S in (k, (k + E) // 2):
        L = orc.Layer(E, S, k, H, F, wdt, host, wr, b)
        for s in range(len(xs)):
            if s == 4:
                L.cache.set_cold(True)
            r = L.step(xs[s])
            assert r["mode"] == (orc.COLD if s >= 4 else r["mode"])
            assert np.array_equal(r["y"], ref[s]), ("cold", S, s)


def test_wrong_slot_map_would_change_the_output(orc, syn):
    # the oracle reads its own slot copies: pointing (t, j) at another slot changes y
    E, k, H, F, wdt = 8, 2, 64, 128, 0
    host = syn.records(6, 0, E, H, F, wdt)
    wr, b = syn.router(6, 0, E, H, wdt, zipf_s=0.0)
    x = syn.tokens(6, 1, 2, H, 1, 0.0, wdt)[0]
    L = orc.Layer(E, 4, k, H, F, wdt, host, wr, b)
    r = L.step(x)
    bad = r["slot_ids"].copy()
    bad[0, 0] = (bad[0, 0] + 1) % 4
    y_bad = orc.ffn(x, wdt, H, F, L.cache.records(bad), r["w"])
    assert not np.array_equal(y_bad[0], r["y"][0]) and np.array_equal(y_bad[1], r["y"][1])


def test_special_cases(orc, syn):
    E, k, H, F, wdt = 8, 2, 64, 128, 0
    host = syn.records(8, 0, E, H, F, wdt)
    w = np.array([[0.7, 0.3]])
    ids = np.array([[3, 5]], np.int32)
    # x = 0 -> y = 0 (silu(0) * 0 = 0)
    y = orc.ffn(np.zeros((1, H), np.float32), wdt, H, F, orc.host_records(host, ids), w)
    assert np.all(y == 0)
    # k = 1, weight 1 -> the single expert's output
    x = syn.tokens(8, 1, 1, H, 1, 0.0, wdt)[0]
    y1, y64 = orc.ffn(x, wdt, H, F, orc.host_records(host, ids[:, :1]), np.ones((1, 1)), want_f64=True)
    g, u, d = expert_mats(host[3], wdt, H, F)
    a, bb = g @ x[0].astype(np.float64), u @ x[0].astype(np.float64)
    assert np.allclose(y64[0], d @ (a / (1 + np.exp(-a)) * bb), rtol=1e-13, atol=0)
    # zeroed down projection -> 0
    h2 = host.copy()
    h2[3, 2 * 4 * H * F:3 * 4 * H * F] = 0
    h2[5, 2 * 4 * H * F:3 * 4 * H * F] = 0
    assert np.all(orc.ffn(x, wdt, H, F, orc.host_records(h2, ids), w) == 0)


def test_residual_rounds_once(orc):
    x = np.array([0x3F80, 0x3F80], np.uint16)         # 1.0, 1.0
    y = np.array([0x3B80, 0x3B81], np.uint16)         # 2^-8 (tie -> 1.0), 2^-8(1 + 2^-7) (-> 1 + 2^-7)
    assert orc.residual(x, y, 1).tolist() == [0x3F80, 0x3F81]


def test_rmsnorm_matches_numpy(orc, syn):
    """The norm is computed in binary32 in one fixed order; against the fp64 definition every bf16 code
    is the correctly rounded one except where the exact value lies within the binary32 error bound
    (2^-19 relative, well above the ~20 roundings of the chain) of a rounding midpoint, and there it is one
    of the two neighbours; fp32 outputs are within that bound.  Hidden sizes with one chunk per partial
    sum (2048), several (7168), and fewer chunks than partials (64, 256)."""
    bound = 2.0 ** -19
    for H, T in ((256, 6), (2048, 5), (7168, 3), (64, 4)):
        x = syn.tokens(13, 2 + H, T, H, 1, 0.0, 1)[0].copy()
        x[0] = 0x3F80  # a constant row of 1.0 -> all ones
        xv = act_f64(x, 1)
        ref = xv / np.sqrt((xv ** 2).mean(axis=1, keepdims=True) + 1e-6)
        got = orc.rmsnorm(x, 1)
        assert np.all(got[0] == 0x3F80)
        lo = np.array([orc.f64_to_bf16(v) for v in (ref * (1 - bound)).reshape(-1)], np.uint16)
        hi = np.array([orc.f64_to_bf16(v) for v in (ref * (1 + bound)).reshape(-1)], np.uint16)
        g = got.reshape(-1)
        assert np.all((g == lo) | (g == hi)), H
        exact = np.array([orc.f64_to_bf16(v) for v in ref.reshape(-1)], np.uint16)
        # away from midpoints the code is the correctly rounded one, and that is nearly every element
        assert np.array_equal(g[lo == hi], exact[lo == hi]) and (lo == hi).mean() > 0.99, H
    xf = syn.tokens(13, 3, 3, 64, 1, 0.0, 0)[0] * 3
    reff = xf.astype(np.float64) / np.sqrt((xf.astype(np.float64) ** 2).mean(axis=1, keepdims=True) + 1e-6)
    gotf = orc.rmsnorm(xf, 0).astype(np.float64)
    assert np.all(np.abs(gotf - reff) <= bound * np.abs(reff))
    # a partial-sum slip (a chunk dropped or counted twice) moves the result far outside that bound
    x1 = np.full((1, 2048), 0x3F80, np.uint16)
    x1[0, :8] = 0x4080  # the first chunk is 4.0: mean square 1 + 120/2048, inv 0.9719 (0.31 steps from a midpoint)
    want = 1.0 / np.sqrt(1.0 + 120.0 / 2048 + 1e-6)
    assert orc.rmsnorm(x1, 1)[0, 100] == orc.f64_to_bf16(want)


def test_prenorm_chain_stays_bounded(orc, syn):
    """48 chained blocks at hidden 2048 / ffn 768 with N(0, 0.02) experts: without a norm on the
    block input the stream's RMS grows super-linearly (the reason for the pre-norm reading);
    with x <- x + MoE(rmsnorm(x)) it stays O(1)."""
    E, k, H, F, L = 8, 2, 2048, 768, 48
    layers = []
    for l in range(L):
        host = syn.records(3, l, E, H, F, 1)
        wr, b = syn.router(3, l, E, H, 1, zipf_s=1.2)
        layers.append((host, wr, b))
    rms = {}
    for norm in (False, True):
        x = syn.tokens(3, 1, 1, H, 1, 0.9, 1)[0]
        try:
            for host, wr, b in layers:
                lay = orc.Layer(E, E, k, H, F, 1, host, wr, b)
                r = lay.step(orc.rmsnorm(x, 1) if norm else x)
                x = orc.residual(x, r["y"], 1)
            xv = act_f64(x, 1)
            rms[norm] = np.sqrt((xv ** 2).mean()) if np.all(np.isfinite(xv)) else np.inf
        except ValueError:  # the stream overflowed and a router logit became NaN
            rms[norm] = np.inf
    assert rms[True] < 2.0
    assert rms[False] > 2 * rms[True]


def test_mxfp4_equals_bf16_record_of_the_same_weights(orc, syn):
    E, k, H, F, T = 4, 2, 256, 256, 3
    mx = syn.records(23, 0, E, H, F, 3)
    bf = np.zeros((E, orc.record_bytes(1, H, F)), np.uint8)
    for e in range(E):
        g, u, d = expert_mats(mx[e], 3, H, F)
        w = np.concatenate([g.reshape(-1), u.reshape(-1), d.reshape(-1)])
        bits = torch.from_numpy(w).to(torch.bfloat16)
        assert np.array_equal(bits.double().numpy(), w)  # each weight is exactly a bf16 value
        bf[e] = bits.view(torch.int16).numpy().view(np.uint8)
    wr, b = syn.router(23, 0, E, H, 1, zipf_s=0.0)
    x = syn.tokens(23, 4, T, H, 1, 0.0, 1)[0]
    ids, w, _ = orc.route(x, wr, b, k, 1)
    y3, y3_64 = orc.ffn(x, 3, H, F, orc.host_records(mx, ids), w, want_f64=True)
    y1, y1_64 = orc.ffn(x, 1, H, F, orc.host_records(bf, ids), w, want_f64=True)
    assert np.array_equal(y3_64, y1_64) and np.array_equal(y3, y1)

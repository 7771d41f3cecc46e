#!/usr/bin/env python3
"""MoE-layer decode throughput of the offloaded MoE layer step on one MI355X.

Default workload (one JSON line on stdout): Qwen3-30B-A3B-shaped decode in
bf16 — 48 MoE layers, each 128 experts, top-8 with renormalised softmax,
hidden 2048, moe ffn 768, 26 GPU slots per layer (20 %), batch 1, token hidden
states from an AR(1) process (rho 0.9) per sequence, router bias ranked by a
seeded Zipf(1.2) permutation.  Every expert of every layer (58 GB) sits in
pinned, device-mapped host memory; a decode step = for each layer: router
top-k, LRU slot ensure, miss copy from host memory, expert FFN + residual,
all 48 layers replayed as one captured HIP graph.

Measured: tokens/s over the timed steps; the dominant kernel's roofline (miss
copy against the host link, HIP events around each copy launch in an eager
pass over the same stream); the FFN against HBM; batch 8 and 32 runs; the CPU
oracle on a bounded sample of the same workload.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

E, K_TOP, H, F, SLOTS, LAYERS = 128, 8, 2048, 768, 26, 48
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
LINK_PEAK_GBPS = 64.0           # PCIe 5.0 x16, one direction, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=224)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the batch 8/32 runs and the link/FFN rooflines")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import expert_offload_slot_amd as m
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    L, T0 = args.layers, args.batch
    max_T = max(32, T0)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    hip.hipMemcpyAsync.restype = ctypes.c_int

    # ---------------- layers: pinned host stores, slots, routers
    t0 = time.time()
    handles = []
    for l in range(L):
        handles.append(m.moe_offload_create(E, SLOTS, H, F, K_TOP, m.BF16, max_T, 0, 0, None,
                                            handles[0] if l else None))
    info0 = m.moe_offload_query(handles[0])
    rb, stride = info0["record_bytes"], info0["record_stride"]
    for l, h in enumerate(handles):
        p, _, _ = m.moe_offload_host_records(h)
        synth.fill_records(args.seed, l, 0, E, H, F, synth.BF16, p, stride)
        if l % 8 == 7:
            log("host store: %d/%d layers filled (%.0f s)" % (l + 1, L, time.time() - t0))
    routers = [synth.router(args.seed, l, E, H, synth.BF16, zipf_s=1.2) for l in range(L)]
    wr_d = [torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev) for w, _ in routers]
    b_d = [torch.from_numpy(b).to(dev) for _, b in routers]
    log("setup %.0f s: %d layers, %.1f GB pinned host store" % (time.time() - t0, L, L * E * stride / 1e9))

    stream = torch.cuda.current_stream()

    def stats_sum():
        tot = {}
        for h in handles:
            for kk, v in m.moe_offload_stats(h).items():
                tot[kk] = tot.get(kk, 0) + v
        return tot

    def run_decode(T, warm, steps, tag):
        """graph replays of the whole step; returns (tok/s, ms/step, stats delta, chain, token stream)"""
        xs = synth.tokens(args.seed, 100 + T, T, H, warm + steps + 24, 0.9, synth.BF16)
        xs_d = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
        c = m.moe_chain_create(handles, wr_d, b_d, T)
        bufs = m.moe_chain_get_buffers(c)
        nbytes = T * H * 2

        def step(s):
            rc = hip.hipMemcpyAsync(bufs["x"], xs_d[s].data_ptr(), nbytes, 3, stream.cuda_stream)
            assert rc == 0
            m.moe_chain_run(c, stream)

        for s in range(warm):
            step(s)
        torch.cuda.synchronize()
        before = stats_sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(warm, warm + steps):
            step(s)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        after = stats_sum()
        delta = {kk: after[kk] - before[kk] for kk in after}
        assert after["error"] == 0, "device error %d" % after["error"]
        log("%s: batch %d, %d steps in %.1f ms: %.1f tok/s, misses/token %.2f, staged calls %d/%d" %
            (tag, T, steps, ms, T * steps * 1e3 / ms, delta["misses"] / (T * steps), delta["staged_calls"],
             delta["calls"]))
        return T * steps * 1e3 / ms, ms / steps, delta, c, bufs, xs_d

    tok_s, ms_step, delta, chain, bufs, xs_d = run_decode(T0, args.warmup, args.steps, "decode")

    # ---------------- eager profile pass on the same stream: HIP events around every call
    T = T0
    n_prof = 16
    act = 2
    xb, xnb, yb = bufs["x"], bufs["xn"], bufs["y"]
    ev = lambda: torch.cuda.Event(enable_timing=True)
    copy_ms = ffn_ms = other_ms = 0.0
    copy_launches = ffn_launches = 0
    before = stats_sum()
    pairs = []
    s0 = args.warmup + args.steps
    for s in range(s0, s0 + n_prof):
        hip.hipMemcpyAsync(xb, xs_d[s].data_ptr(), T * H * act, 3, stream.cuda_stream)
        for l, h in enumerate(handles):
            xl = xb + l * T * H * act
            xnl = xnb + l * T * H * act
            off = l * T * K_TOP * 4
            a, b_, c_, d_ = ev(), ev(), ev(), ev()
            a.record(stream)
            m.moe_rmsnorm(xl, xnl, T, H, m.BF16, m.RMS_EPS, stream)
            m.moe_route_topk(h, xnl, wr_d[l], b_d[l], T, bufs["ids"] + off, bufs["w"] + off, stream)
            m.moe_slot_ensure(h, bufs["ids"] + off, T, bufs["slot_ids"] + off, stream)
            b_.record(stream)
            m.moe_copy_misses(h, stream)
            c_.record(stream)
            m.moe_slot_ffn(h, xnl, bufs["slot_ids"] + off, bufs["w"] + off, T, None, yb + l * T * H * act,
                           xl, xl + T * H * act, stream)
            d_.record(stream)
            pairs.append((a, b_, c_, d_))
    torch.cuda.synchronize()
    for a, b_, c_, d_ in pairs:
        other_ms += a.elapsed_time(b_)
        copy_ms += b_.elapsed_time(c_)
        ffn_ms += c_.elapsed_time(d_)
        copy_launches += 1
        ffn_launches += 1
    after = stats_sum()
    prof_bytes = after["bytes_copied"] - before["bytes_copied"]
    prof_misses = after["misses"] - before["misses"] + after["staged_copies"] - before["staged_copies"]
    copy_avg_us = copy_ms * 1e3 / copy_launches
    copy_gbps = prof_bytes / (copy_ms * 1e-3) / 1e9 if copy_ms > 0 else 0.0
    ffn_avg_us = ffn_ms * 1e3 / ffn_launches
    log("eager profile (%d steps): copy %.1f ms (%d launches, avg %.1f us, %.2f GB/s over %.1f MB), ffn %.1f ms "
        "(avg %.1f us), route+ensure %.1f ms" % (n_prof, copy_ms, copy_launches, copy_avg_us, copy_gbps,
                                                  prof_bytes / 1e6, ffn_ms, ffn_avg_us, other_ms))

    result = {
        "metric": "MoE-layer decode tokens/s at 20% slots (Qwen3-30B-A3B-shaped, 48 layers, bf16)",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox: N(0,0.02) experts/router, Zipf(1.2)-ranked bias, AR(1) rho 0.9 tokens)",
        "config": {"workload": "qwen3-30b-a3b-shaped offloaded MoE decode: 48 layers x 128 experts, top-8, "
                               "hidden 2048, moe ffn 768, 26 slots/layer, batch %d, HIP-graph step" % T0,
                   "layers": L, "experts": E, "top_k": K_TOP, "hidden": H, "ffn": F, "slots": SLOTS,
                   "batch": T0, "host_store_GB": round(L * E * stride / 1e9, 2)},
        "decode_stats": {"misses_per_token": round(delta["misses"] / (T0 * args.steps), 4),
                         "staged_calls": delta["staged_calls"], "calls": delta["calls"],
                         "staged_copies_per_token": round(delta["staged_copies"] / (T0 * args.steps), 4),
                         "hit_rate": round(delta["hits"] / max(1, delta["hits"] + delta["misses"]), 4)},
        "eager_profile": {"steps": n_prof, "copy_ms": round(copy_ms, 3), "ffn_ms": round(ffn_ms, 3),
                          "route_ensure_ms": round(other_ms, 3), "copy_bytes": prof_bytes,
                          "copied_records": prof_misses},
    }
    copy_roof = {"bound": "host_link", "kernel": "k_copy (moe_copy_misses)", "achieved": round(copy_gbps, 2),
                 "peak": LINK_PEAK_GBPS, "unit": "GB/s", "frac": round(copy_gbps / LINK_PEAK_GBPS, 4),
                 "traffic": None, "avg_launch_us": round(copy_avg_us, 2), "launches": copy_launches,
                 "bytes": prof_bytes}
    result["roofline"] = copy_roof

    if not args.no_extra:
        # FFN against HBM: 8 distinct resident records per call at batch 1
        ffn_bytes_per_call = None
        if T0 == 1:
            ffn_bytes_per_call = K_TOP * rb + 3 * H * 2
            gbps = ffn_bytes_per_call / (ffn_avg_us * 1e-6) / 1e9
            result["roofline_ffn"] = {"bound": "hbm", "kernel": "moe_slot_ffn (group + gate/up + down)",
                                      "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                      "frac": round(gbps / HBM_PEAK_GBPS, 4), "avg_call_us": round(ffn_avg_us, 2),
                                      "bytes_per_call": ffn_bytes_per_call, "traffic": None}
        # host link: SDMA copy of 1 GiB pinned -> device, and the copy kernel moving 128 records (1.2 GB)
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        a, b_ = ev(), ev()
        a.record(stream)
        for _ in range(3):
            dst.copy_(src, non_blocking=True)
        b_.record(stream)
        torch.cuda.synchronize()
        sdma = 3 * n / (a.elapsed_time(b_) * 1e-3) / 1e9
        del src, dst
        hl = m.moe_offload_create(E, SLOTS, H, F, K_TOP, m.BF16, 16, 0, 0, handles[0], handles[0])
        ids_all = torch.arange(E, dtype=torch.int32, device=dev).reshape(16, K_TOP)
        sid = torch.empty_like(ids_all)
        kern = []
        for r in range(4):
            m.moe_offload_reset(hl, stream)
            m.moe_slot_ensure(hl, ids_all, 16, sid, stream)  # 128 distinct > 26 slots: all 128 staged
            a, b_ = ev(), ev()
            a.record(stream)
            m.moe_copy_misses(hl, stream)
            b_.record(stream)
            torch.cuda.synchronize()
            kern.append(E * rb / (a.elapsed_time(b_) * 1e-3) / 1e9)
        m.moe_offload_destroy(hl)
        kernel_link = max(kern[1:])
        link = max(sdma, kernel_link)
        result["host_link"] = {"sdma_GBps": round(sdma, 2), "copy_kernel_1p2GB_GBps": round(kernel_link, 2),
                               "measured_link_GBps": round(link, 2),
                               "decode_copy_frac_of_measured_link": round(copy_gbps / link, 4)}
        log("host link: SDMA %.2f GB/s, copy kernel %.2f GB/s; decode copies at %.1f %% of measured link" %
            (sdma, kernel_link, 100 * copy_gbps / link))
        # other batch sizes (same layers, caches carry over)
        for T in (8, 32):
            if T == T0:
                continue
            steps = 64 if T == 8 else 32
            ts, msps, d, c2, _, _ = run_decode(T, 8, steps, "decode-b%d" % T)
            result["batch%d" % T] = {"tokens_per_s": round(ts, 2), "ms_per_step": round(msps, 3), "steps": steps,
                                     "misses_per_token": round(d["misses"] / (T * steps), 4),
                                     "staged_calls": d["staged_calls"], "calls": d["calls"],
                                     "staged_copies_per_token": round(d["staged_copies"] / (T * steps), 4)}
            m.moe_chain_destroy(c2)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, handles, routers, stride, rb, T0)

    print(json.dumps(result), flush=True)
    m.moe_chain_destroy(chain)
    for h in reversed(handles):
        m.moe_offload_destroy(h)


def cpu_baseline(args, handles, routers, stride, rb, T):
    """The CPU oracle, as it stands, on the first decode steps of the same token stream (all layers)."""
    import numpy as np

    import expert_offload_slot_amd as m
    import oracle
    import synth

    L = len(handles)
    xs = synth.tokens(args.seed, 100 + T, T, H, args.warmup + args.steps, 0.9, synth.BF16)
    staging = np.zeros((E, stride), dtype=np.uint8)
    layers = [oracle.Layer(E, SLOTS, K_TOP, H, F, oracle.BF16, m.host_array(h, E), routers[l][0], routers[l][1],
                           staging=staging) for l, h in enumerate(handles)]
    t0 = time.time()
    steps = 0
    while steps < len(xs):
        x = xs[steps]
        for lay in layers:
            r = lay.step(oracle.rmsnorm(x, oracle.BF16))
            x = oracle.residual(x, r["y"], oracle.BF16)
        steps += 1
        if time.time() - t0 > args.cpu_seconds:
            break
    dt = time.time() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    log("cpu oracle: %d steps x %d layers in %.1f s" % (steps, L, dt))
    return {"value": round(T * steps / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d decode steps (batch %d, all %d layers) of the same token stream, from a cold cache"
                      % (steps, T, L)}


if __name__ == "__main__":
    main()

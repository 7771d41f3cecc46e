#!/usr/bin/env python3
"""MoE-layer decode throughput of the offloaded MoE layer step on one MI355X.

Workload of `value` (one JSON line on stdout): Qwen3-30B-A3B-shaped decode in
bf16 -- 48 MoE layers, each 128 experts, top-8 with renormalised softmax,
hidden 2048, moe ffn 768, 26 GPU slots per layer (20 %), batch 1, token hidden
states from an AR(1) process (rho 0.9), router bias ranked by a seeded
Zipf(1.2) permutation.  Every expert of every layer (58 GB) sits in pinned,
device-mapped host memory.  A step = for each layer: router logits, one
control workgroup (top-k, LRU slot ensure, grouping), the miss copy from host
memory (read through by the FFN launches), the expert FFN with combine and
residual; all 48 layers replayed as one captured HIP graph.  Inputs are
resident in HBM before the timed region.

`value` times exactly the --steps replays that follow --warmup untimed
replays, from empty caches.  The same line carries, measured in the same run:
  * steady_state: a fixed untimed warm-up of 32 replays from empty caches,
    then 224 timed replays (steps 32-255), and the summed link + HBM roofline;
    the same with the copy kernel instead of read-through; batch 8 and 32;
  * per-kernel average durations from HIP events on the launch stream
    (library profiling switch) over an eager pass of the same chain; the
    gate/up kernel's HBM roofline, the down kernel's and the miss copy's
    host-link fraction;
  * a 256 MiB device-to-device copy (HBM reference) and the host link (SDMA
    copy of 1 GiB pinned memory, the copy kernel over 128 records);
  * router-lookahead prefetch against none, LRU against scored eviction and
    pinned placement, decode at 10/20/40/100 % slots (outputs bitwise
    identical at every fraction);
  * misses computed on the host CPU (split and cold mode) at batch 1, 8 and
    32, through the entry points and inside the graph (the chain's host
    thread);
  * the MXFP4 records (over the link, and with a profile-guided hot set and
    every miss on the host), the Mixtral-8x7B-shaped layer at 2/4/6 slots and
    the DeepSeek-V3-shaped fp8 layer (decode at batch 16 over the link and in
    split mode, the 2048-token prefill: staging copy, FFN TFLOP/s and the
    fraction of its attainable roofline);
  * the CPU oracle on a bounded sample of the same workload.
--quick keeps only the batch-1 window, its steady state, the eager profile
and the host link.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

E, K_TOP, H, F, SLOTS, LAYERS = 128, 8, 2048, 768, 26, 48
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
LINK_PEAK_GBPS = 64.0           # PCIe 5.0 x16, one direction, published
COUNTERS = os.path.join(ROOT, "profiles", "k_gateup_one_decode_b1_counters.md")
TRACE = os.path.join(ROOT, "profiles", "decode_qwen3_30b_b1_kernel_trace.md")
GU_KERNEL_TRACE_NAME = "k_gateup_one<1, 16, false>"
SS_WARM, SS_STEPS = 32, 224     # steady state: untimed cache warm-up from an empty cache, then timed replays
FFN_SRC = os.path.join(ROOT, "expert_offload_slot_amd", "csrc", "k_ffn.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_sha256(path):
    """sha256 of a C++ source with its comments and whitespace removed (comment edits keep the hash)."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, if taken on the current kernel code."""
    if not os.path.exists(COUNTERS):
        return None
    text = open(COUNTERS).read()
    sha = code_sha256(FFN_SRC)
    got = dict(re.findall(r"^(\w+):\s*(\S+)\s*$", text, re.M))
    if got.get("source_sha256") != sha:
        return None
    try:
        return int(got["fetch_bytes_per_launch"]) + int(got["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traced_avg_us(path, kernel):
    """Average duration of `kernel` in the committed rocprofv3 summary of this command: its dispatches in the
    eager profile pass (the ones this run times with HIP events), from the trace's start and end timestamps."""
    if not os.path.exists(path):
        return None
    m_ = re.search(r"^trace_avg_us\[%s\]:\s*(\S+)\s*$" % re.escape(kernel), open(path).read(), re.M)
    return float(m_.group(1)) if m_ else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=224)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prof-steps", type=int, default=16)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--quick", action="store_true",
                    help="only the batch-1 window, its steady state, the eager profile and the host link")
    ap.add_argument("--no-cpu-rates", action="store_true",
                    help="skip the CPU oracle's own rates on all threads and one (about 15 s)")
    ap.add_argument("--prefetch-only", action="store_true",
                    help="only the lookahead-prefetch comparison on the 48-layer workload (its own JSON line)")
    ap.add_argument("--counters-only", action="store_true",
                    help="only eager passes of the copy-kernel chain at batch 1 (no graph), --prof-steps steps from "
                         "an empty cache, and the 256 MiB device copy: the workload of the FETCH_SIZE / WRITE_SIZE "
                         "counter passes (its own JSON line)")
    ap.add_argument("--mixtral-only", action="store_true",
                    help="only the Mixtral-8x7B-shaped layer (its own JSON line)")
    ap.add_argument("--split-only", action="store_true",
                    help="only the eager comparison of the link, split and host-cold modes at batch 1, 8 and 32 (its own JSON line)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--mxfp4-only", action="store_true",
                    help="only the same decode chain with MXFP4 expert records (prints its own JSON line)")
    ap.add_argument("--deepseek-only", action="store_true",
                    help="only the DeepSeek-V3-shaped layer: fp8 decode at batch 16 and the 2048-token prefill "
                         "(prints its own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (requested --gpus %d)" % args.gpus,
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
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    if args.deepseek_only:
        print(json.dumps({"workload": "deepseek-v3-shaped offloaded MoE layer, fp8 e4m3 experts with 128x128 "
                                      "scales: 256 experts + shared, top-8, hidden 7168, moe ffn 2048, 26 slots",
                          "deepseek_v3_layer": deepseek_layer(args, m, torch)}), flush=True)
        return

    if args.mixtral_only:
        print(json.dumps({"workload": "mixtral-8x7b-shaped offloaded MoE layer: 8 experts, top-2, hidden 4096, "
                                      "moe ffn 14336, bf16, 2/4/6 slots",
                          "mixtral_8x7b_layer": mixtral_layer(args, m, torch)}), flush=True)
        return

    if args.mxfp4_only:
        routers = [synth.router(args.seed, l, E, H, synth.BF16, zipf_s=1.2) for l in range(L)]
        wr_d = [torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev) for w, _ in routers]
        b_d = [torch.from_numpy(b).to(dev) for _, b in routers]
        out = qwen3_mxfp4(args, m, torch, hip, wr_d, b_d)
        print(json.dumps({"workload": "qwen3-30b-a3b-shaped offloaded MoE decode, MXFP4 expert records: %d layers x "
                                      "128 experts, top-8, hidden 2048, moe ffn 768, 26 slots/layer, batch 1, "
                                      "HIP-graph step" % L, "qwen3_mxfp4": out}), flush=True)
        return

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

    # ---------------- known-size device copy: HBM reference and counter scale
    n_cal = 256 << 20
    a_cal = torch.empty(n_cal, dtype=torch.uint8, device=dev)
    b_cal = torch.empty(n_cal, dtype=torch.uint8, device=dev)
    b_cal.copy_(a_cal)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(3):
        b_cal.copy_(a_cal)
    e1.record(stream)
    torch.cuda.synchronize()
    hbm_copy_gbps = 3 * 2 * n_cal / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a_cal, b_cal
    log("device copy 256 MiB: %.0f GB/s (read + write)" % hbm_copy_gbps)

    def stats_sum(hs=None):
        tot = {}
        for h in hs or handles:
            for kk, v in m.moe_offload_stats(h).items():
                tot[kk] = tot.get(kk, 0) + v
        return tot

    def token_stream(T, n):
        xs = synth.tokens(args.seed, 100 + T, T, H, n, 0.9, synth.BF16)
        return torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)

    def run_decode(T, warm, steps, tag, prefetch_n=0, xs_d=None, hs=None, cold=None, read_through=True, fresh=True):
        """graph replays of the whole step; returns (tok/s, ms/step, stats delta, chain, buffers, tokens).
        fresh: the graph is captured and replayed once outside the timed window and every layer's cache is
        emptied again, so the warm-up replays start from an empty cache (fresh=False keeps the caches as
        they are: the capture replay is then step 0 and the warm-up covers steps 1..warm-1).
        With a dict `cold`, the warm-up replays are timed into it."""
        hs = hs or handles
        if xs_d is None:
            xs_d = token_stream(T, warm + steps + args.prof_steps)
        c = m.moe_chain_create(hs, wr_d, b_d, T, prefetch_n)
        if not read_through:
            m.moe_chain_set_read_through(c, 0)
        bufs = m.moe_chain_get_buffers(c)
        nbytes = T * H * 2

        def step(s):
            rc = hip.hipMemcpyAsync(bufs["x"], xs_d[s].data_ptr(), nbytes, 3, stream.cuda_stream)
            assert rc == 0
            m.moe_chain_run(c, stream)

        step(0)  # capture + instantiate outside the timed window
        torch.cuda.synchronize()
        if fresh:
            for h in hs:
                m.moe_offload_reset(h, stream)
            torch.cuda.synchronize()
        if cold is not None:
            c0, c1 = ev(), ev()
            c0.record(stream)
        for s in range(0 if fresh else 1, warm):
            step(s)
        if cold is not None:
            c1.record(stream)
        torch.cuda.synchronize()
        if cold is not None:
            st = stats_sum(hs)
            cms = c0.elapsed_time(c1)
            cold.update({"steps": "0-%d" % (warm - 1), "tokens_per_s": round(T * warm * 1e3 / cms, 2),
                         "ms_per_step": round(cms / warm, 4),
                         "misses_per_token": round(st["misses"] / (T * warm), 4),
                         "staged_copies_per_token": round(st["staged_copies"] / (T * warm), 4)})
            log("%s cold start (steps 0-%d from an empty cache): %.1f tok/s, %.2f copies/token" %
                (tag, warm - 1, T * warm * 1e3 / cms, (st["misses"] + st["staged_copies"]) / (T * warm)))
        before = stats_sum(hs)
        a, b_ = ev(), ev()
        torch.cuda.synchronize()
        a.record(stream)
        for s in range(warm, warm + steps):
            step(s)
        b_.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b_)
        after = stats_sum(hs)
        delta = {kk: after[kk] - before[kk] for kk in after}
        assert after["error"] == 0, "device error %d" % after["error"]
        log("%s: batch %d, %d steps in %.1f ms: %.1f tok/s, copies/token %.2f (%.2f into slots), staged calls %d/%d" %
            (tag, T, steps, ms, T * steps * 1e3 / ms, (delta["misses"] + delta["staged_copies"]) / (T * steps),
             delta["misses"] / (T * steps), delta["staged_calls"], delta["calls"]))
        return T * steps * 1e3 / ms, ms / steps, delta, c, bufs, xs_d

    if args.prefetch_only:
        print(json.dumps({"workload": "qwen3-30b-a3b-shaped offloaded MoE decode, 48 layers, batch 1: router-"
                                      "lookahead prefetch (4 installs per layer) against none",
                          "prefetch": prefetch_compare(args, m, hip, handles, run_decode, token_stream)}), flush=True)
        for h in reversed(handles):
            m.moe_offload_destroy(h)
        return

    if args.counters_only:
        c = m.moe_chain_create(handles, wr_d, b_d, T0, 0)
        m.moe_chain_set_read_through(c, 0)
        bufs = m.moe_chain_get_buffers(c)
        xs_c = token_stream(T0, args.prof_steps)
        for s in range(args.prof_steps):
            hip.hipMemcpyAsync(bufs["x"], xs_c[s].data_ptr(), T0 * H * 2, 3, stream.cuda_stream)
            m.moe_chain_run_eager(c, stream)
        torch.cuda.synchronize()
        st = stats_sum()
        assert st["error"] == 0
        m.moe_chain_destroy(c)
        print(json.dumps({"workload": "qwen3-30b-a3b-shaped offloaded MoE decode, 48 layers, batch %d: eager passes "
                                      "of the copy-kernel chain from an empty cache" % T0,
                          "eager_steps": args.prof_steps, "calls": st["calls"], "misses": st["misses"]}), flush=True)
        for h in reversed(handles):
            m.moe_offload_destroy(h)
        return

    if args.split_only:
        print(json.dumps({"workload": "qwen3-30b-a3b-shaped offloaded MoE decode, 48 layers, batch 1, 8 and 32, eager "
                                      "entry-point calls: misses over the link, split with the host CPU, or on "
                                      "the host (from an empty cache, or after a warm-up over the link)",
                          "host_split": host_split_compare(args, m, torch, handles, wr_d, b_d, token_stream),
                          "host_chain": host_chain_compare(args, m, torch, hip, handles, wr_d, b_d, token_stream)}),
              flush=True)
        for h in reversed(handles):
            m.moe_offload_destroy(h)
        return

    # ---------------- the timed window: --warmup untimed replays from an empty cache, then --steps timed
    # replays (the headline value; cold start included when the window is short)
    tok_s, ms_step, delta, chain, bufs, xs_d = run_decode(T0, args.warmup, args.steps, "decode-window")
    m.moe_chain_destroy(chain)

    # ---------------- steady state: a fixed untimed cache warm-up of SS_WARM replays from an empty cache,
    # then SS_STEPS timed replays (steps SS_WARM .. SS_WARM + SS_STEPS - 1 of the same token stream)
    for h in handles:
        m.moe_offload_reset(h, stream)
    cold = {}
    ss_tok, ss_ms, ss_d, chain, bufs, xs_ss = run_decode(T0, SS_WARM, SS_STEPS, "decode-steady", cold=cold)

    # ---------------- the same stream from empty caches with the misses moved by the copy kernel before the FFN
    for h in handles:
        m.moe_offload_reset(h, stream)
    m.moe_chain_destroy(chain)
    tok_cp, ms_cp, delta_cp, chain, bufs, _ = run_decode(T0, SS_WARM, SS_STEPS, "decode-steady-copy-kernel",
                                                         xs_d=xs_ss, read_through=False)
    assert delta_cp["misses"] == ss_d["misses"] and delta_cp["staged_copies"] == ss_d["staged_copies"]

    # ---------------- eager pass of the copy-kernel chain with per-kernel HIP events on the launch stream:
    # each kernel's bytes come from one memory (the FFN from HBM, the copy over the host link)
    T = T0
    for h in handles:
        m.moe_offload_profile(h, 1)
    before = stats_sum()
    s0 = SS_WARM + SS_STEPS
    gu_bytes = dn_bytes = 0
    distinct = 0  # distinct records the FFN reads, summed over the profiled calls
    sid_host = np.empty((L, T, K_TOP), dtype=np.int32)
    for s in range(s0, s0 + args.prof_steps):
        hip.hipMemcpyAsync(bufs["x"], xs_ss[s].data_ptr(), T * H * 2, 3, stream.cuda_stream)
        m.moe_chain_run_eager(chain, stream)
        torch.cuda.synchronize()
        # algorithmic bytes of this step's FFN launches: distinct records of each call
        assert hip.hipMemcpy(sid_host.ctypes.data, bufs["slot_ids"], sid_host.nbytes, 2) == 0
        for l in range(L):
            nrec = len(np.unique(sid_host[l]))
            distinct += nrec
            gu_bytes += nrec * 2 * F * H * 2 + T * H * 2 + T * K_TOP * F * 2
            dn_bytes += nrec * F * H * 2 + T * K_TOP * F * 2 + T * K_TOP * H * 4
    kt = {}
    for h in handles:
        for kind, (ms_, n_) in m.moe_offload_kernel_times(h).items():
            a_ms, a_n = kt.get(kind, (0.0, 0))
            kt[kind] = (a_ms + ms_, a_n + n_)
        m.moe_offload_profile(h, 0)
    after = stats_sum()
    copy_bytes = after["bytes_copied"] - before["bytes_copied"]
    kernels = {kind: {"avg_us": round(ms_ * 1e3 / n_, 3), "launches": n_, "total_ms": round(ms_, 3)}
               for kind, (ms_, n_) in kt.items() if n_}
    log("eager profile (%d steps): " % args.prof_steps +
        ", ".join("%s %.2f us" % (k_, v["avg_us"]) for k_, v in kernels.items()))
    gu_ms, gu_n = kt["gateup"]
    dn_ms, dn_n = kt["down"]
    cp_ms, cp_n = kt["copy"]
    gu_gbps = gu_bytes / (gu_ms * 1e-3) / 1e9
    dn_gbps = dn_bytes / (dn_ms * 1e-3) / 1e9
    cp_gbps = copy_bytes / (cp_ms * 1e-3) / 1e9 if cp_ms > 0 else 0.0
    traffic = measured_traffic()
    gu_alg = int(gu_bytes // gu_n)
    traced = traced_avg_us(TRACE, GU_KERNEL_TRACE_NAME)

    def hit_rate(d):
        return round(d["hits"] / max(1, d["hits"] + d["misses"] + d["staged_copies"]), 4)

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
                   "batch": T0, "host_store_GB": round(L * E * stride / 1e9, 2),
                   "window": "value times steps %d-%d of the token stream, replayed from empty caches after "
                             "%d untimed replays" % (args.warmup, args.warmup + args.steps - 1, args.warmup),
                   "steady_state_warmup_steps": SS_WARM, "steady_state_timed_steps": SS_STEPS},
        "window_stats": {"misses_per_token": round(delta["misses"] / (T0 * args.steps), 4),
                         "staged_calls": delta["staged_calls"], "calls": delta["calls"],
                         "staged_copies_per_token": round(delta["staged_copies"] / (T0 * args.steps), 4),
                         "hit_rate": hit_rate(delta)},
        "steady_state": {"batch": T0, "steps": "%d-%d" % (SS_WARM, SS_WARM + SS_STEPS - 1),
                         "untimed_cache_warmup_steps": SS_WARM,
                         "tokens_per_s": round(ss_tok, 2), "ms_per_step": round(ss_ms, 4),
                         "misses_per_token": round(ss_d["misses"] / (T0 * SS_STEPS), 4),
                         "staged_copies_per_token": round(ss_d["staged_copies"] / (T0 * SS_STEPS), 4),
                         "hit_rate": hit_rate(ss_d)},
        "cold_start": cold,
        "read_through": {"on_tokens_per_s": round(ss_tok, 2), "off_tokens_per_s": round(tok_cp, 2),
                         "on_ms_per_step": round(ss_ms, 4), "off_ms_per_step": round(ms_cp, 4),
                         "speedup": round(ss_tok / tok_cp, 4), "steps": "%d-%d steady state" % (SS_WARM, SS_WARM + SS_STEPS - 1)},
        "roofline": {"bound": "hbm", "kernel": "k_gateup_one<bf16, 16, false> (gate/up + SiLU, single-token decode, records read in place)",
                     "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else traffic,
                     "avg_launch_us": round(gu_ms * 1e3 / gu_n, 3), "launches": gu_n,
                     "algorithmic_bytes_per_launch": gu_alg,
                     "duration_source": "HIP start/stop events recorded with each dispatch on its launch stream "
                                        "(hipExtLaunchKernelGGL), eager pass of %d steps in this run" % args.prof_steps,
                     "traffic_source": None if traffic is None else
                     "scaled FETCH_SIZE + WRITE_SIZE per launch from %s (taken on this kernel source)" %
                     os.path.relpath(COUNTERS, ROOT),
                     "rocprof": None if traced is None else
                     {"avg_launch_us": traced, "frac": round(gu_alg / (traced * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                      "source": "%s (rocprofv3 --kernel-trace --stats of this command: the kernel's dispatches "
                                "in the eager pass, from the trace's own start and end timestamps)" %
                                os.path.relpath(TRACE, ROOT)}},
        "roofline_down": {"bound": "hbm", "kernel": "k_down_one<bf16, 6, false>", "achieved": round(dn_gbps, 1),
                          "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dn_gbps / HBM_PEAK_GBPS, 4),
                          "avg_launch_us": round(dn_ms * 1e3 / dn_n, 3),
                          "algorithmic_bytes_per_launch": int(dn_bytes // dn_n)},
        "roofline_copy": {"bound": "host_link", "kernel": "k_copy (demand misses)", "achieved": round(cp_gbps, 2),
                          "peak": LINK_PEAK_GBPS, "unit": "GB/s", "frac": round(cp_gbps / LINK_PEAK_GBPS, 4),
                          "avg_launch_us": round(cp_ms * 1e3 / max(1, cp_n), 3), "launches": cp_n,
                          "bytes": copy_bytes},
        "kernels_us": kernels,
        "hbm_copy_256MiB_GBps": round(hbm_copy_gbps, 1),
    }

    # ---------------- host link: SDMA copy of 1 GiB pinned -> device, and the copy kernel moving 128 records
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
        m.moe_slot_ensure(hl, ids_all, 16, sid, stream)  # cold cache: all 128 experts miss (26 to slots, 102 staged)
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
                           "decode_copy_frac_of_measured_link": round(cp_gbps / link, 4)}
    log("host link: SDMA %.2f GB/s, copy kernel %.2f GB/s; decode copies at %.1f %% of measured link" %
        (sdma, kernel_link, 100 * cp_gbps / link))

    # ---------------- summed roofline of the steady-state steps: every copied record over the measured host
    # link, every distinct record the FFN reads once from HBM at the datasheet rate
    def summed(d, steps, ms, T_, distinct_per_step):
        copies_step = (d["misses"] + d["staged_copies"]) / steps
        bound_ms = (copies_step * rb / (link * 1e9) + distinct_per_step * rb / (HBM_PEAK_GBPS * 1e9)) * 1e3
        return {"ms_per_step": round(bound_ms, 4), "tokens_per_s": round(T_ * 1e3 / bound_ms, 2),
                "frac": round(bound_ms / ms, 4), "copied_records_per_step": round(copies_step, 3),
                "distinct_records_per_step": round(distinct_per_step, 3), "record_bytes": rb,
                "link_GBps": round(link, 2), "hbm_GBps": HBM_PEAK_GBPS}

    result["steady_state"]["summed_roofline"] = summed(ss_d, SS_STEPS, ss_ms, T0, distinct / args.prof_steps)
    log("steady state: %.1f tok/s = %.1f %% of the summed roofline (%.1f tok/s)" %
        (ss_tok, 100 * result["steady_state"]["summed_roofline"]["frac"],
         result["steady_state"]["summed_roofline"]["tokens_per_s"]))
    m.moe_chain_destroy(chain)

    if not args.quick:
        result["steady_state_batches"] = {}
        for T, steps in ((8, 64), (32, 32)):
            if T == T0:
                continue
            for h in handles:
                m.moe_offload_reset(h, stream)
            ts, msps, d, c2, b2, _ = run_decode(T, SS_WARM, steps, "decode-steady-b%d" % T)
            nd = distinct_records(hip, b2, L, T, SS_WARM + steps - 1)
            m.moe_chain_destroy(c2)
            result["steady_state_batches"]["batch%d" % T] = {
                "tokens_per_s": round(ts, 2), "ms_per_step": round(msps, 3),
                "steps": "%d-%d" % (SS_WARM, SS_WARM + steps - 1), "untimed_cache_warmup_steps": SS_WARM,
                "misses_per_token": round(d["misses"] / (T * steps), 4),
                "staged_calls": d["staged_calls"], "calls": d["calls"],
                "staged_copies_per_token": round(d["staged_copies"] / (T * steps), 4),
                "summed_roofline": summed(d, steps, msps, T, nd)}
        result["prefetch"] = prefetch_compare(args, m, hip, handles, run_decode, token_stream)
        result["eviction"] = eviction_compare(args, m, hip, torch, handles, wr_d, b_d, run_decode, token_stream)
        result["slot_fractions"] = slot_fraction_compare(args, m, hip, handles, run_decode, token_stream)
        result["host_split"] = host_split_compare(args, m, torch, handles, wr_d, b_d, token_stream)
        result["host_chain"] = host_chain_compare(args, m, torch, hip, handles, wr_d, b_d, token_stream)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, handles, routers, stride, T0)
        if not args.no_cpu_rates and not args.quick:
            result["cpu_oracle"] = cpu_oracle_rates(args)

    for h in reversed(handles):
        m.moe_offload_destroy(h)
    if not args.quick:  # after the bf16 layers' host stores are released
        result["qwen3_mxfp4"] = qwen3_mxfp4(args, m, torch, hip, wr_d, b_d)
        result["mixtral_8x7b_layer"] = mixtral_layer(args, m, torch)
        result["deepseek_v3_layer"] = deepseek_layer(args, m, torch)
    print(json.dumps(result), flush=True)


def distinct_records(hip, bufs, L, T, step):
    """Distinct records each layer's FFN read in the chain's last step, summed over the layers."""
    import numpy as np
    sid = np.empty((L, T, K_TOP), dtype=np.int32)
    assert hip.hipMemcpy(sid.ctypes.data, bufs["slot_ids"], sid.nbytes, 2) == 0
    return sum(len(np.unique(sid[l])) for l in range(L))


def qwen3_mxfp4(args, m, torch, hip, wr_d, b_d):
    """The batch-1 decode chain of the default workload with MXFP4 expert records (2.5 MB instead of 9.4 MB):
    same layers, slots, routers and token stream; graph replays timed, then an eager pass with per-kernel events."""
    import numpy as np
    import synth
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    L, T, t0 = args.layers, 1, time.time()
    hs = []
    for l in range(L):
        hs.append(m.moe_offload_create(E, SLOTS, H, F, K_TOP, m.MXFP4, 32, 0, 0, None, hs[0] if l else None))
    info = m.moe_offload_query(hs[0])
    rb, stride = info["record_bytes"], info["record_stride"]
    for l, h in enumerate(hs):
        p, _, _ = m.moe_offload_host_records(h)
        synth.fill_records(args.seed, l, 0, E, H, F, synth.MXFP4, p, stride)
        if l % 16 == 15:
            log("mxfp4 host store: %d/%d layers filled (%.0f s)" % (l + 1, L, time.time() - t0))
    warm, steps, prof = SS_WARM, SS_STEPS, args.prof_steps
    xs = synth.tokens(args.seed, 100 + T, T, H, warm + steps + prof, 0.9, synth.BF16)
    xs_d = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
    c = m.moe_chain_create(hs, wr_d, b_d, T, 0)
    bufs = m.moe_chain_get_buffers(c)

    def step(s, run):
        assert hip.hipMemcpyAsync(bufs["x"], xs_d[s].data_ptr(), T * H * 2, 3, stream.cuda_stream) == 0
        run(c, stream)

    def stats():
        tot = {}
        for h in hs:
            for kk, v in m.moe_offload_stats(h).items():
                tot[kk] = tot.get(kk, 0) + v
        return tot

    for s in range(warm):
        step(s, m.moe_chain_run)
    torch.cuda.synchronize()
    before = stats()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for s in range(warm, warm + steps):
        step(s, m.moe_chain_run)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    d = {kk: v - before[kk] for kk, v in stats().items()}
    assert d["error"] == 0
    # the same replays from empty caches with the copy kernel moving the misses before the FFN; the eager
    # profile below runs this way too, so that each kernel's bytes come from one memory
    m.moe_chain_set_read_through(c, 0)
    for h in hs:
        m.moe_offload_reset(h, stream)
    for s in range(warm):
        step(s, m.moe_chain_run)
    a.record(stream)
    for s in range(warm, warm + steps):
        step(s, m.moe_chain_run)
    b.record(stream)
    torch.cuda.synchronize()
    ms_off = a.elapsed_time(b)
    for h in hs:
        m.moe_offload_profile(h, 1)
    gu_bytes = dn_bytes = 0
    sid = np.empty((L, T, K_TOP), dtype=np.int32)
    cb0 = stats()["bytes_copied"]
    for s in range(warm + steps, warm + steps + prof):
        step(s, m.moe_chain_run_eager)
        torch.cuda.synchronize()
        assert hip.hipMemcpy(sid.ctypes.data, bufs["slot_ids"], sid.nbytes, 2) == 0
        for l in range(L):
            nrec = len(np.unique(sid[l]))
            gu_bytes += nrec * 2 * (F * H // 2 + F * H // 32) + T * H * 2 + T * K_TOP * F * 2
            dn_bytes += nrec * (F * H // 2 + F * H // 32) + T * K_TOP * F * 2 + T * K_TOP * H * 4
    kt = {}
    for h in hs:
        for kind, (ms_, n_) in m.moe_offload_kernel_times(h).items():
            x0, n0 = kt.get(kind, (0.0, 0))
            kt[kind] = (x0 + ms_, n0 + n_)
        m.moe_offload_profile(h, 0)
    copy_bytes = stats()["bytes_copied"] - cb0
    m.moe_chain_destroy(c)
    # host-computed misses with MXFP4 records (the host FFN widens E2M1 codes): each layer pins its S - k most
    # routed experts of a separate profiling stream, the warm-up fills the other k slots over the link, then
    # every miss is computed on the host inside the graph (as the bf16 chain's cold_profile mode)
    cnt = routing_profile(args, m, hip, torch, hs, wr_d, b_d, T, 256)
    for l, h in enumerate(hs):
        m.moe_offload_reset(h, stream)
        top = np.ascontiguousarray(np.argsort(-cnt[l], kind="stable")[:SLOTS - K_TOP].astype(np.int32))
        m.moe_offload_pin(h, torch.from_numpy(top).to(dev), len(top), stream)
    c = m.moe_chain_create(hs, wr_d, b_d, T, 0)
    bufs = m.moe_chain_get_buffers(c)
    try:
        for s in range(warm):
            step(s, m.moe_chain_run)
        torch.cuda.synchronize()
        for h in hs:
            m.moe_offload_set_cold(h, m.COLD_ON, stream)
        step(warm, m.moe_chain_run)  # untimed: the graph is captured again
        torch.cuda.synchronize()
        before_c = stats()
        done = torch.cuda.Event(blocking=True)
        tc = time.perf_counter()
        for s in range(warm + 1, warm + 1 + steps):
            step(s, m.moe_chain_run)
        done.record(stream)
        done.synchronize()
        dt_cold = time.perf_counter() - tc
        dc = {kk: v - before_c[kk] for kk, v in stats().items()}
        assert dc["error"] == 0
    finally:
        m.moe_chain_destroy(c)
        for h in hs:
            m.moe_offload_set_cold(h, m.COLD_OFF, stream)
            m.moe_offload_pin(h, None, 0, stream)
    cold_profile = {"tokens_per_s": round(T * steps / dt_cold, 2), "ms_per_step": round(dt_cold * 1e3 / steps, 4),
                    "host_records_per_token": round(dc["cold_misses"] / (T * steps), 3),
                    "link_records_per_token": round((dc["misses"] + dc["staged_copies"]) / (T * steps), 3),
                    "steps": "%d-%d after %d untimed (+1 after the mode switch), wall clock" %
                             (warm + 1, warm + steps, warm)}
    log("qwen3 mxfp4 decode, profile-guided hot set, misses on the host: %.1f tok/s, %.2f host records/token" %
        (cold_profile["tokens_per_s"], cold_profile["host_records_per_token"]))
    for h in reversed(hs):
        m.moe_offload_destroy(h)
    (gu_ms, gu_n), (dn_ms, dn_n), (cp_ms, cp_n) = kt["gateup"], kt["down"], kt["copy"]
    out = {"tokens_per_s": round(T * steps * 1e3 / ms, 2), "ms_per_step": round(ms / steps, 4), "steps": steps,
           "copy_kernel_tokens_per_s": round(T * steps * 1e3 / ms_off, 2),
           "record_bytes": rb, "host_store_GB": round(L * E * stride / 1e9, 2),
           "copies_per_token": round((d["misses"] + d["staged_copies"]) / (T * steps), 4),
           "copy_GBps": round(copy_bytes / (cp_ms * 1e-3) / 1e9, 2) if cp_ms > 0 else 0.0,
           "roofline_gateup": {"kernel": "k_gateup_one<mxfp4, 8, false>", "avg_launch_us": round(gu_ms * 1e3 / gu_n, 3),
                               "algorithmic_bytes_per_launch": int(gu_bytes // gu_n),
                               "achieved": round(gu_bytes / (gu_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                               "unit": "GB/s", "frac": round(gu_bytes / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
           "roofline_down": {"kernel": "k_down_one<mxfp4, 3, false>", "avg_launch_us": round(dn_ms * 1e3 / dn_n, 3),
                             "algorithmic_bytes_per_launch": int(dn_bytes // dn_n),
                             "achieved": round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": round(dn_bytes / (dn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
           "kernels_us": {kind: round(v * 1e3 / n, 3) for kind, (v, n) in kt.items() if n},
           "host_cold_profile": cold_profile}
    log("qwen3 mxfp4 decode: %.1f tok/s (copy kernel: %.1f), %.2f copies/token of %.2f MB, gateup %.2f us, "
        "down %.2f us" % (out["tokens_per_s"], out["copy_kernel_tokens_per_s"], out["copies_per_token"], rb / 1e6,
                          out["roofline_gateup"]["avg_launch_us"], out["roofline_down"]["avg_launch_us"]))
    return out


def layer_steps(m, torch, h, wr, b, shared, xs, T, steps, warm, split=False):
    """Entry-point decode calls (route, ensure, copy, FFN) of one layer: tok/s over the timed calls, and the
    per-kernel event averages of the same calls.  split: the layer in split mode (MOE_COLD_SPLIT, the share
    measured when it is switched on), the FFN through moe_slot_ffn_host_cold, so calls wider than the cache
    send that share of their staged misses to the host CPU; the cache starts empty."""
    dev = torch.device("cuda", 0)
    st = torch.cuda.current_stream()
    H = xs.shape[-1]
    k = m.moe_offload_query(h)["k"]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    sid = torch.empty_like(ids)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    q = None
    if split:
        m.moe_offload_reset(h, st)
        q = m.moe_offload_set_cold(h, m.COLD_SPLIT, st)
    ffn = m.moe_slot_ffn_host_cold if split else m.moe_slot_ffn

    def call(s):
        x = xs[s]
        m.moe_route_topk(h, x, wr, b, T, ids, w, st)
        m.moe_slot_ensure(h, ids, T, sid, st)
        m.moe_copy_misses(h, st)
        ffn(h, x, sid, w, T, shared, y, None, None, st)

    for s in range(warm):
        call(s)
    torch.cuda.synchronize()
    before = m.moe_offload_stats(h)
    m.moe_offload_profile(h, 1)
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for s in range(warm, warm + steps):
        call(s)
    b_.record(st)
    torch.cuda.synchronize()
    kt = m.moe_offload_kernel_times(h)
    m.moe_offload_profile(h, 0)
    after = m.moe_offload_stats(h)
    ms = a.elapsed_time(b_)
    d = {kk: after[kk] - before[kk] for kk in after}
    extra = {}
    if split:
        m.moe_offload_set_cold(h, m.COLD_OFF, st)
        m.moe_offload_reset(h, st)
        torch.cuda.synchronize()
        extra = {"host_share_of_256": q[0], "host_us_per_record": round(q[1], 1), "link_us_per_record": round(q[2], 1),
                 "host_records_per_call": round(d["cold_misses"] / steps, 3)}
    return {**extra, "tokens_per_s": round(T * steps * 1e3 / ms, 2), "ms_per_call": round(ms / steps, 3), "calls": steps,
            "misses_per_call": round(d["misses"] / steps, 3), "staged_calls": d["staged_calls"],
            "staged_copies_per_call": round(d["staged_copies"] / steps, 3),
            "copy_GBps": round(d["bytes_copied"] / (kt["copy"][0] * 1e-3) / 1e9, 2) if kt["copy"][0] > 0 else None,
            "kernels_us": {kind: round(v[0] * 1e3 / v[1], 2) for kind, v in kt.items() if v[1]}}


def mixtral_layer(args, m, torch):
    """Mixtral-8x7B-shaped layer (8 experts, top-2, hidden 4096, ffn 14336, bf16, uniform router): decode at
    2, 4 and 6 slots, and at 6 slots both FFN kernel pairs on calls of 8 to 64 tokens."""
    import numpy as np
    import synth
    E, k, H, F, seed = 8, 2, 4096, 14336, args.seed + 7
    dev = torch.device("cuda", 0)
    wr, b = synth.router(seed, 0, E, H, synth.BF16, zipf_s=0.0)
    wr_d = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).to(dev)
    b_d = torch.from_numpy(b).to(dev)
    out = {}
    for S in (2, 4, 6):
        h = m.moe_offload_create(E, S, H, F, k, m.BF16, 64, 0, 0)
        p, stride, rb = m.moe_offload_host_records(h)
        synth.fill_records(seed, 0, 0, E, H, F, synth.BF16, p, stride)
        for T in (1, 8, 64):
            xs = synth.tokens(seed, 50 + T, T, H, 24, 0.9, synth.BF16)
            xs_d = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
            r = layer_steps(m, torch, h, wr_d, b_d, None, xs_d, T, 16, 8)
            out["S%d_T%d" % (S, T)] = r
            log("mixtral S=%d T=%d: %.1f tok/s, %.3f misses/call, copy %s GB/s" %
                (S, T, r["tokens_per_s"], r["misses_per_call"], r["copy_GBps"]))
        if S == 6:
            # the pair-dot decode kernels against the grouped MFMA GEMM on the same calls (2 to 16 pairs per
            # expert): FFN kernel time (grouping, gate/up, down) per pair
            paths = {}
            for T in (8, 16, 24, 32, 64):
                xs = synth.tokens(seed, 50 + T, T, H, 24, 0.9, synth.BF16)
                xs_d = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
                row = {"pairs_per_expert": T * k / E}
                for name, path in (("pairdot", m.FFN_DECODE), ("mfma", m.FFN_GEMM)):
                    m.moe_offload_set_ffn_path(h, path)
                    r = layer_steps(m, torch, h, wr_d, b_d, None, xs_d, T, 8, 4)
                    row[name + "_us_per_pair"] = round(sum(r["kernels_us"].get(kk, 0) for kk in
                                                           ("group", "gateup", "down")) / (T * k), 3)
                m.moe_offload_set_ffn_path(h, m.FFN_AUTO)
                row["auto"] = "mfma" if T * k >= 5 * E else "pairdot"
                paths["T%d" % T] = row
                log("mixtral T=%d: pair-dot %.2f us/pair, MFMA %.2f us/pair (auto: %s)" %
                    (T, row["pairdot_us_per_pair"], row["mfma_us_per_pair"], row["auto"]))
            out["ffn_paths_S6"] = paths
        m.moe_offload_destroy(h)
    return out


def prefill_ffn(m, torch, h, wr_d, b_d, sh_d, x, mfma_dtype):
    """Route a prefill call, stage the layer (host-synchronising), then time the FFN (5 repetitions):
    TFLOP/s and the fraction of its attainable roofline (the slower of streaming the distinct records once
    at 8 TB/s and the dense bf16 MFMA rate)."""
    import numpy as np
    info = m.moe_offload_query(h)
    E, k, H, F, rb = info["E"], info["k"], info["H"], info["F"], info["record_bytes"]
    T = x.shape[0]
    dev = torch.device("cuda", 0)
    st = torch.cuda.current_stream()
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    sid = torch.empty_like(ids)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    m.moe_route_topk(h, xd, wr_d, b_d, T, ids, w, st)
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    staged = m.moe_prefill_stage(h, ids, T, sid, st)
    b_.record(st)
    torch.cuda.synchronize()
    stage_ms = a.elapsed_time(b_)
    m.moe_slot_ffn(h, xd, sid, w, T, sh_d, y, None, None, st)  # warm
    torch.cuda.synchronize()
    reps = 5
    m.moe_offload_profile(h, 1)
    a.record(st)
    for _ in range(reps):
        m.moe_slot_ffn(h, xd, sid, w, T, sh_d, y, None, None, st)
    b_.record(st)
    torch.cuda.synchronize()
    kt = m.moe_offload_kernel_times(h)
    m.moe_offload_profile(h, 0)
    ffn_ms = a.elapsed_time(b_) / reps
    flop_gu = 2 * (T * k + T) * 2 * F * H
    flop_dn = 2 * (T * k + T) * F * H
    cnt = np.bincount(ids.cpu().numpy().reshape(-1), minlength=E)
    wbytes = (int((cnt > 0).sum()) + 1) * rb
    gu_us = kt["gateup"][0] * 1e3 / kt["gateup"][1]
    dn_us = kt["down"][0] * 1e3 / kt["down"][1]
    bound_ms = max(wbytes / 8e12, (flop_gu + flop_dn) / 2.5e15) * 1e3
    r = {"staged": staged, "stage_ms": round(stage_ms, 2), "stage_GBps": round(E * rb / (stage_ms * 1e-3) / 1e9, 2),
         "record_bytes": rb, "ffn_ms": round(ffn_ms, 3),
         "ffn_TFLOPs": round((flop_gu + flop_dn) / (ffn_ms * 1e-3) / 1e12, 1),
         "gateup_us": round(gu_us, 1), "gateup_TFLOPs": round(flop_gu / (gu_us * 1e-6) / 1e12, 1),
         "down_us": round(dn_us, 1), "down_TFLOPs": round(flop_dn / (dn_us * 1e-6) / 1e12, 1),
         "mfma_peak_TFLOPs": 2500.0, "mfma_dtype": mfma_dtype,
         "frac_of_mfma_peak": round((flop_gu + flop_dn) / (ffn_ms * 1e-3) / 1e12 / 2500.0, 4),
         "hbm_bound_ms": round(wbytes / 8e12 * 1e3, 3), "attainable_bound_ms": round(bound_ms, 3),
         "frac_of_attainable": round(bound_ms / ffn_ms, 4),
         "tokens_per_expert_max": int(cnt.max()), "experts_used": int((cnt > 0).sum())}
    log("prefill T=%d (%s records of %.1f MB): stage %.1f ms (%.1f GB/s), ffn %.2f ms = %.1f TFLOP/s, %.1f %% of "
        "attainable" % (T, "fp8" if rb > 30e6 else "mxfp4", rb / 1e6, stage_ms, r["stage_GBps"], ffn_ms,
                        r["ffn_TFLOPs"], 100 * r["frac_of_attainable"]))
    return r


def deepseek_layer(args, m, torch):
    """DeepSeek-V3-shaped layer (fp8 e4m3 + 128x128 scales, 256 experts + shared, top-8, hidden 7168, ffn 2048,
    26 slots): decode at batch 16, and a 2048-token prefill that stages the whole layer; the same prefill with
    MXFP4 records."""
    import numpy as np
    import synth
    E, k, H, F, S, seed = 256, 8, 7168, 2048, 26, args.seed + 9
    dev = torch.device("cuda", 0)
    st = torch.cuda.current_stream()
    h = m.moe_offload_create(E, S, H, F, k, m.FP8, 2048, 0, 0)
    p, stride, rb = m.moe_offload_host_records(h)
    synth.fill_records(seed, 0, 0, E, H, F, synth.FP8, p, stride)
    wr, b = synth.router(seed, 0, E, H, synth.BF16, zipf_s=1.2)
    wr_d = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).to(dev)
    b_d = torch.from_numpy(b).to(dev)
    sh_d = torch.from_numpy(synth.records(seed, 0, 1, H, F, synth.FP8, shared=True)[0]).to(dev)
    out = {}
    xs = synth.tokens(seed, 60, 16, H, 72, 0.0, synth.BF16)
    xs_d = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
    out["decode_T16"] = layer_steps(m, torch, h, wr_d, b_d, sh_d, xs_d, 16, 64, 8)
    log("deepseek decode T=16: %.1f tok/s, %d/%d calls staged" % (out["decode_T16"]["tokens_per_s"],
                                                                  out["decode_T16"]["staged_calls"], 64))
    # the same calls from an empty cache in split mode: the measured share of each call's staged misses is
    # computed by the host CPU from host memory while the rest cross the link
    out["decode_T16_split"] = layer_steps(m, torch, h, wr_d, b_d, sh_d, xs_d, 16, 64, 8, split=True)
    log("deepseek decode T=16, split with the host: %.1f tok/s, %.2f records per call on the host (share %s/256)" %
        (out["decode_T16_split"]["tokens_per_s"], out["decode_T16_split"]["host_records_per_call"],
         out["decode_T16_split"]["host_share_of_256"]))
    T = 2048
    x = synth.tokens(seed, 70, T, H, 1, 0.0, synth.BF16)[0]
    out["prefill_T2048"] = prefill_ffn(m, torch, h, wr_d, b_d, sh_d, x, "bf16 (fp8 codes widened exactly)")
    m.moe_offload_destroy(h)
    # the same prefill with MXFP4 expert records (E2M1 codes + E8M0 scale per 32, widened with the scale folded in)
    h = m.moe_offload_create(E, S, H, F, k, m.MXFP4, 2048, 0, 0)
    p, stride, rb = m.moe_offload_host_records(h)
    synth.fill_records(seed, 0, 0, E, H, F, synth.MXFP4, p, stride)
    sh_mx = torch.from_numpy(synth.records(seed, 0, 1, H, F, synth.MXFP4, shared=True)[0]).to(dev)
    out["prefill_T2048_mxfp4"] = prefill_ffn(m, torch, h, wr_d, b_d, sh_mx, x,
                                             "bf16 (E2M1 codes widened exactly, E8M0 scale folded in)")
    m.moe_offload_destroy(h)
    return out


def host_split_compare(args, m, torch, handles, wr_d, b_d, token_stream, batches=(1, 8, 32), warm=24, steps=8):
    """Eager decode over the layers with entry-point calls (norm, route, ensure, copy, FFN per layer) at
    batch 1, 8 and 32, the same `steps` timed steps of one token stream after `warm` untimed ones, each mode
    from empty caches:
      link       every miss over the host link (the method as it stands);
      split      calls wider than the cache send the share of their staged misses measured per layer
                 (MOE_COLD_SPLIT) to the host CPU;
      split_all  the same with every staged miss on the host (share 256/256): the misses that claim
                 slots still cross the link, so the cache keeps learning;
      cold       every miss computed on the host from the start (nothing is ever loaded);
      cold_warm  the warm-up steps with the link (the cache learns), then every miss on the host.
    Wall-clock tok/s."""
    import numpy as np
    dev = torch.device("cuda", 0)
    st = torch.cuda.current_stream()
    out = {}
    for T in batches:
        ids = torch.empty((T, K_TOP), dtype=torch.int32, device=dev)
        w = torch.empty((T, K_TOP), dtype=torch.float32, device=dev)
        sid = torch.empty_like(ids)
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        xa, xb, xn = torch.empty_like(y), torch.empty_like(y), torch.empty_like(y)
        xs = token_stream(T, warm + steps)
        res = {}
        qs = []
        try:
            for mode in ("link", "split", "split_all", "cold", "cold_warm"):
                for h in handles:
                    m.moe_offload_set_cold(h, m.COLD_OFF, st)
                    m.moe_offload_reset(h, st)
                if mode == "split":
                    qs = [m.moe_offload_set_cold(h, m.COLD_SPLIT, st) for h in handles]
                elif mode == "split_all":
                    for h in handles:
                        m.moe_offload_set_split(h, 256, st)
                elif mode == "cold":
                    for h in handles:
                        m.moe_offload_set_cold(h, m.COLD_ON, st)
                cold_ffn = [mode in ("split", "split_all", "cold")]

                def step(s):
                    a, b = xa, xb
                    a.copy_(xs[s])
                    ffn = m.moe_slot_ffn_host_cold if cold_ffn[0] else m.moe_slot_ffn
                    for l, h in enumerate(handles):  # the decode chain's block: pre-norm, MoE, residual
                        m.moe_rmsnorm(a, xn, T, H, m.BF16, stream=st)
                        m.moe_route_topk(h, xn, wr_d[l], b_d[l], T, ids, w, st)
                        m.moe_slot_ensure(h, ids, T, sid, st)
                        m.moe_copy_misses(h, st)
                        ffn(h, xn, sid, w, T, None, y, a, b, st)
                        a, b = b, a

                for s in range(warm):
                    step(s)
                torch.cuda.synchronize()
                if mode == "cold_warm":
                    for h in handles:
                        m.moe_offload_set_cold(h, m.COLD_ON, st)
                    cold_ffn[0] = True
                before = [m.moe_offload_stats(h) for h in handles]
                t0 = time.perf_counter()
                for s in range(warm, warm + steps):
                    step(s)
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
                after = [m.moe_offload_stats(h) for h in handles]
                assert all(a_["error"] == 0 for a_ in after), [a_["error"] for a_ in after]
                d = {kk: sum(a_[kk] - b_[kk] for a_, b_ in zip(after, before)) for kk in after[0]}
                res[mode] = {"tokens_per_s": round(T * steps / dt, 2), "ms_per_step": round(dt * 1e3 / steps, 3),
                             "link_records_per_token": round((d["misses"] + d["staged_copies"]) / (T * steps), 3),
                             "host_records_per_token": round(d["cold_misses"] / (T * steps), 3),
                             "staged_calls": d["staged_calls"], "calls": d["calls"]}
                log("host-offload b%d %s: %.1f tok/s, %.2f records/token over the link, %.2f on the host" %
                    (T, mode, res[mode]["tokens_per_s"], res[mode]["link_records_per_token"],
                     res[mode]["host_records_per_token"]))
        finally:
            for h in handles:
                m.moe_offload_set_cold(h, m.COLD_OFF, st)
                m.moe_offload_reset(h, st)
            torch.cuda.synchronize()
        if qs:
            q = sorted(x[0] for x in qs)
            res["split_share_q256"] = {"median": q[len(q) // 2], "min": q[0], "max": q[-1],
                                       "host_us_per_record_median": round(float(np.median([x[1] for x in qs])), 1),
                                       "link_us_per_record_median": round(float(np.median([x[2] for x in qs])), 1)}
        res["steps"] = "%d-%d after %d untimed" % (warm, warm + steps - 1, warm)
        out["batch%d" % T] = res
    return out


def host_chain_compare(args, m, torch, hip, handles, wr_d, b_d, token_stream, batches=(1, 8, 32), warm=24, steps=8):
    """The same comparison inside the decode chain (one HIP graph per step; the host's share runs on the
    chain's host thread, with no host synchronisation): batch 1, 8 and 32, each mode from empty caches,
    `warm` untimed steps, one more untimed step after a mode switch (the graph is captured again), then
    `steps` timed ones, waited for with a blocking event (the calling thread sleeps rather than spins, so
    the host FFN has every core):
      link          every miss over the host link (read-through);
      split         calls wider than the cache send the measured share of their staged misses to the host;
      cold_warm     the warm-up over the link (the cache learns), then every miss on the host;
      cold_profile  a profile-guided hot set (npu-offload's placement from a routing profile): each layer
                    pins its S - k most routed experts of a separate profiling stream (256 tokens, at
                    least 16 steps), the warm-up fills the other k slots over the link, then every miss
                    on the host.
    Wall-clock tok/s."""
    import numpy as np
    out = {}
    st = torch.cuda.current_stream()
    for T in batches:
        xs = token_stream(T, warm + steps + 1)
        res = {}
        for mode in ("link", "split", "cold_warm", "cold_profile"):
            for h in handles:
                m.moe_offload_set_cold(h, m.COLD_OFF, st)
                m.moe_offload_pin(h, None, 0, st)
                m.moe_offload_reset(h, st)
            if mode == "split":
                for h in handles:
                    m.moe_offload_set_cold(h, m.COLD_SPLIT, st)
            if mode == "cold_profile":
                cnt = routing_profile(args, m, hip, torch, handles, wr_d, b_d, T, max(16, 256 // T))
                for l, h in enumerate(handles):
                    m.moe_offload_reset(h, st)
                    top = np.ascontiguousarray(np.argsort(-cnt[l], kind="stable")[:SLOTS - K_TOP].astype(np.int32))
                    m.moe_offload_pin(h, torch.from_numpy(top).to(st.device), len(top), st)
                torch.cuda.synchronize()
            c = m.moe_chain_create(handles, wr_d, b_d, T, 0)
            bufs = m.moe_chain_get_buffers(c)
            try:
                def step(s_):
                    assert hip.hipMemcpyAsync(bufs["x"], xs[s_].data_ptr(), T * H * 2, 3, st.cuda_stream) == 0
                    m.moe_chain_run(c, st)

                for s_ in range(warm):
                    step(s_)
                torch.cuda.synchronize()
                if mode in ("cold_warm", "cold_profile"):
                    for h in handles:
                        m.moe_offload_set_cold(h, m.COLD_ON, st)
                step(warm)  # untimed: a switched mode captures the graph again
                torch.cuda.synchronize()
                before = [m.moe_offload_stats(h) for h in handles]
                done = torch.cuda.Event(blocking=True)  # this thread sleeps: every core is left to the host FFN
                t0 = time.perf_counter()
                for s_ in range(warm + 1, warm + 1 + steps):
                    step(s_)
                done.record(st)
                done.synchronize()
                dt = time.perf_counter() - t0
                after = [m.moe_offload_stats(h) for h in handles]
            finally:
                m.moe_chain_destroy(c)
            assert all(a_["error"] == 0 for a_ in after), [a_["error"] for a_ in after]
            d = {kk: sum(a_[kk] - b_[kk] for a_, b_ in zip(after, before)) for kk in after[0]}
            res[mode] = {"tokens_per_s": round(T * steps / dt, 2), "ms_per_step": round(dt * 1e3 / steps, 3),
                         "link_records_per_token": round((d["misses"] + d["staged_copies"]) / (T * steps), 3),
                         "host_records_per_token": round(d["cold_misses"] / (T * steps), 3)}
            log("host-offload chain b%d %s: %.1f tok/s, %.2f records/token over the link, %.2f on the host" %
                (T, mode, res[mode]["tokens_per_s"], res[mode]["link_records_per_token"],
                 res[mode]["host_records_per_token"]))
        for h in handles:
            m.moe_offload_set_cold(h, m.COLD_OFF, st)
            m.moe_offload_pin(h, None, 0, st)
            m.moe_offload_reset(h, st)
        torch.cuda.synchronize()
        res["steps"] = "%d-%d after %d untimed (+1 after a mode switch)" % (warm + 1, warm + steps, warm)
        out["batch%d" % T] = res
    return out


def torch_stream():
    import torch
    return torch.cuda.current_stream()


def prefetch_compare(args, m, hip, handles, run_decode, token_stream):
    """Router-lookahead prefetch (up to 4 experts per layer) against none, each from an empty cache on the
    same token stream; the last step's output stream must be bitwise identical."""
    import numpy as np
    T, warm, steps = 1, 16, 128
    xs_d = token_stream(T, warm + steps + args.prof_steps)
    out, last = {}, {}
    for n in (0, 4):
        for h in handles:
            m.moe_offload_reset(h)
        ts, msps, d, c, bufs, _ = run_decode(T, warm, steps, "prefetch-%d" % n, prefetch_n=n, xs_d=xs_d)
        xl = np.empty((T, H), dtype=np.uint16)  # the last layer's output stream x[L] of the last step
        assert hip.hipMemcpy(xl.ctypes.data, bufs["x"] + len(handles) * T * H * 2, xl.nbytes, 2) == 0
        last[n] = xl
        # per-kernel event times of a few eager steps of the same chain
        stream = torch_stream()
        for h in handles:
            m.moe_offload_profile(h, 1)
        for s_ in range(warm + steps, warm + steps + 8):
            assert hip.hipMemcpyAsync(bufs["x"], xs_d[s_].data_ptr(), T * H * 2, 3, stream.cuda_stream) == 0
            m.moe_chain_run_eager(c, stream)
        kt = {}
        for h in handles:
            for kind, (ms_, n_) in m.moe_offload_kernel_times(h).items():
                a_, b2 = kt.get(kind, (0.0, 0))
                kt[kind] = (a_ + ms_, b2 + n_)
            m.moe_offload_profile(h, 0)
        kernels = {kind: round(v * 1e3 / k_, 3) for kind, (v, k_) in kt.items() if k_}
        out["prefetch_%d" % n] = {"tokens_per_s": round(ts, 2), "ms_per_step": round(msps, 3),
                                  "demand_misses_per_token": round(d["misses"] / (T * steps), 4),
                                  "prefetch_installs_per_token": round(d["prefetch_installs"] / (T * steps), 4),
                                  "prefetch_hits_per_token": round(d["prefetch_hits"] / (T * steps), 4),
                                  "eager_kernels_us": kernels}
        m.moe_chain_destroy(c)
    out["outputs_identical"] = bool(np.array_equal(last[0], last[4]))
    return out


def slot_fraction_compare(args, m, hip, handles, run_decode, token_stream):
    """Decode at batch 1 with 10, 20, 40 and 100 % of each layer's experts in slots (13, 26, 52, 128 of 128),
    each from an empty cache on the same token stream; the other fractions' layers share the 20 % layers' host
    stores.  Every layer's output of the last step must be bitwise identical at every fraction."""
    import numpy as np
    T, warm, steps = 1, 16, 128
    xs_d = token_stream(T, warm + steps + args.prof_steps)
    out, last = {}, {}
    for S in (13, SLOTS, 52, E):
        hs = handles if S == SLOTS else [m.moe_offload_create(E, S, H, F, K_TOP, m.BF16, 32, 0, 0, h, handles[0])
                                         for h in handles]
        try:
            for h in hs:
                m.moe_offload_reset(h)
            ts, msps, d, c, bufs, _ = run_decode(T, warm, steps, "slots-%d" % S, xs_d=xs_d, hs=hs)
            xl = np.empty((len(hs) + 1, T, H), dtype=np.uint16)  # every layer's input stream x[0..L]
            assert hip.hipMemcpy(xl.ctypes.data, bufs["x"], xl.nbytes, 2) == 0
            last[S] = xl
            out["slots_%d" % S] = {"slot_fraction": round(S / E, 4), "tokens_per_s": round(ts, 2),
                                   "ms_per_step": round(msps, 3),
                                   "misses_per_token": round(d["misses"] / (T * steps), 4)}
            m.moe_chain_destroy(c)
        finally:
            if hs is not handles:
                for h in reversed(hs):
                    m.moe_offload_destroy(h)
    out["outputs_identical"] = bool(all(np.array_equal(last[S], last[SLOTS]) for S in last))
    assert out["outputs_identical"], "outputs differ between slot fractions"
    return out


def routing_profile(args, m, hip, torch, handles, wr_d, b_d, T, steps):
    """Expert counts per layer over `steps` decode steps of a separate profiling token stream."""
    import numpy as np
    import synth
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    xs = synth.tokens(args.seed, 900 + T, T, H, steps, 0.9, synth.BF16)
    xs_d = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
    c = m.moe_chain_create(handles, wr_d, b_d, T, 0)
    bufs = m.moe_chain_get_buffers(c)
    L = len(handles)
    ids = np.empty((L, T, K_TOP), dtype=np.int32)
    cnt = np.zeros((L, E), dtype=np.int64)
    for s in range(steps):
        assert hip.hipMemcpyAsync(bufs["x"], xs_d[s].data_ptr(), T * H * 2, 3, stream.cuda_stream) == 0
        m.moe_chain_run(c, stream)
        torch.cuda.synchronize()
        assert hip.hipMemcpy(ids.ctypes.data, bufs["ids"], ids.nbytes, 2) == 0
        for l in range(L):
            cnt[l] += np.bincount(ids[l].reshape(-1), minlength=E)
    m.moe_chain_destroy(c)
    return cnt


def eviction_compare(args, m, hip, torch, handles, wr_d, b_d, run_decode, token_stream):
    """LRU against scored eviction (least used first, then LRU), activation-aware eviction (least activated
    expert first, counts kept across evictions, then LRU) and profile-guided placement (each
    layer's SLOTS // 2 most routed experts of a separate profiling stream pinned, LRU for the rest), each from
    an empty cache on the same token stream; the scored layers share the LRU layers' host stores.  Outputs
    must be bitwise identical."""
    import numpy as np
    T, warm, steps = 1, 16, 128
    xs_d = token_stream(T, warm + steps + args.prof_steps)
    scored = [m.moe_offload_create(E, SLOTS, H, F, K_TOP, m.BF16, 32, 0, m.FLAG_SCORED, h, handles[0])
              for h in handles]
    freq = [m.moe_offload_create(E, SLOTS, H, F, K_TOP, m.BF16, 32, 0, m.FLAG_FREQ, h, handles[0])
            for h in handles]
    out, last = {}, {}
    try:
        for name, hs in (("lru", handles), ("scored", scored), ("activation_aware", freq), ("pinned", handles)):
            for h in hs:
                m.moe_offload_reset(h)
            if name == "pinned":
                cnt = routing_profile(args, m, hip, torch, handles, wr_d, b_d, T, 64)
                for h in hs:
                    m.moe_offload_reset(h)
                for l, h in enumerate(hs):
                    hot = np.argsort(-cnt[l], kind="stable")[:SLOTS // 2].astype(np.int32)
                    m.moe_offload_pin(h, torch.from_numpy(hot).to("cuda"), len(hot), torch.cuda.current_stream())
                torch.cuda.synchronize()
            ts, msps, d, c, bufs, _ = run_decode(T, warm, steps, "eviction-" + name, xs_d=xs_d, hs=hs,
                                                 fresh=name != "pinned")
            xl = np.empty((T, H), dtype=np.uint16)
            assert hip.hipMemcpy(xl.ctypes.data, bufs["x"] + len(hs) * T * H * 2, xl.nbytes, 2) == 0
            last[name] = xl
            out[name] = {"tokens_per_s": round(ts, 2), "ms_per_step": round(msps, 3),
                         "misses_per_token": round(d["misses"] / (T * steps), 4)}
            m.moe_chain_destroy(c)
    finally:
        for h in reversed(scored + freq):
            m.moe_offload_destroy(h)
    for h in handles:  # unpin: the default layers go back to plain LRU
        m.moe_offload_pin(h, None, 0, torch.cuda.current_stream())
    torch.cuda.synchronize()
    out["pinned"]["pinned_per_layer"] = SLOTS // 2
    out["outputs_identical"] = bool(all(np.array_equal(last["lru"], last[n]) for n in last))
    return out


def cpu_baseline(args, handles, routers, stride, T):
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
    threads = oracle.threads()
    log("cpu oracle: %d steps x %d layers in %.1f s on %d threads" % (steps, L, dt, threads))
    return {"value": round(T * steps / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d decode steps (batch %d, all %d layers) of the same token stream, from a cold cache"
                      % (steps, T, L),
            "host": host_cpu()}


def cpu_oracle_rates(args):
    """The oracle's own rates on the host, on all its threads and on one: the tiny fp32 layer's decode
    tokens/s, one Qwen3-shaped layer step at batch 1 (route, ensure, copy of its misses from a cold cache,
    FFN), the copy of 26 records into its slot arrays, and its FFN over 16 tokens x top-8."""
    import numpy as np
    import oracle
    import synth

    def c1():
        E, k, Hs, Fs, S, T, steps = 8, 2, 64, 128, 4, 4, 32
        host = synth.records(args.seed, 0, E, Hs, Fs, synth.F32)
        wr, b = synth.router(args.seed, 0, E, Hs, synth.F32, zipf_s=1.2)
        lay = oracle.Layer(E, S, k, Hs, Fs, oracle.F32, host, wr, b)
        xs = synth.tokens(args.seed, 7, T, Hs, steps, 0.0, synth.F32)
        t0 = time.time()
        for s in range(steps):
            lay.step(xs[s])
        return T * steps / (time.time() - t0)

    host = synth.records(args.seed, 0, E, H, F, synth.BF16)
    rb = oracle.record_bytes(oracle.BF16, H, F)
    wr, b = synth.router(args.seed, 0, E, H, synth.BF16, zipf_s=1.2)
    xs = synth.tokens(args.seed, 8, 1, H, 8, 0.9, synth.BF16)
    x16 = synth.tokens(args.seed, 9, 16, H, 1, 0.0, synth.BF16)[0]
    ids16 = np.arange(16 * K_TOP, dtype=np.int32).reshape(16, K_TOP) % E
    w16 = np.full((16, K_TOP), 1.0 / K_TOP)

    def layer_step_ms():
        lay = oracle.Layer(E, SLOTS, K_TOP, H, F, oracle.BF16, host, wr, b)
        t0 = time.time()
        for s in range(len(xs)):
            lay.step(xs[s])
        return (time.time() - t0) * 1e3 / len(xs)

    def copy_gbps():
        cache = oracle.Cache(E, SLOTS, host, rb)
        pairs = np.array([[e, e] for e in range(SLOTS)], dtype=np.int32)
        cache.copy(0, pairs)  # first touch of the slot arrays
        t0 = time.time()
        cache.copy(0, pairs)
        return SLOTS * rb / (time.time() - t0) / 1e9

    def ffn_gflops():
        recs = oracle.host_records(host, ids16)
        t0 = time.time()
        oracle.ffn(x16, oracle.BF16, H, F, recs, w16)
        return 6.0 * H * F * 16 * K_TOP / (time.time() - t0) / 1e9

    full = oracle.threads()
    out = {"threads": full, "host": host_cpu()}
    for label, n in (("all_threads", full), ("one_thread", 1)):
        oracle.set_threads(n)
        out[label] = {"tiny_fp32_decode_tokens_per_s": round(c1(), 1),
                      "qwen3_layer_step_b1_ms": round(layer_step_ms(), 2),
                      "copy_26_records_GBps": round(copy_gbps(), 2),
                      "ffn_16x8_GFLOPs": round(ffn_gflops(), 2)}
        log("cpu oracle on %d thread(s): %s" % (n, out[label]))
    oracle.set_threads(full)
    return out


def host_cpu():
    """nproc, the CPU model, sockets and hardware threads of the host, from /proc/cpuinfo."""
    model, sockets, logical = None, set(), 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "processor":
                    logical += 1
                elif key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    sockets.add(val)
    except OSError:
        pass
    return {"nproc": len(os.sched_getaffinity(0)), "model": model, "sockets": len(sockets) or None,
            "threads": logical or os.cpu_count()}


if __name__ == "__main__":
    main()

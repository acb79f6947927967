#!/usr/bin/env python3
"""Benchmark of one sparse decode step over a host-offloaded latent cache.

Workload: 32K context, 16 requests, one query token per step, 64x128 fp8
indexer, top-2048, 128-head absorbed MLA over 576-wide bf16 latents, a hot
pool of 8192 slots per request, latents in pinned host memory.  One step =
indexer scores -> top-k with the slot lookup -> pool update -> gather +
attention over the selected rows (+ combine), for all 16 requests; the
gather reads each miss from host memory inside the attention kernel and
writes it to its pool slot from the tile.  All per-step inputs (the drifting indexer queries and
the absorbed queries) are staged in device memory before the timed region;
the pool's first fill runs before the warm-up steps.

The headline figure times whole steps through the one-call entry point
(ess_decode_step) with nothing recorded between its kernels.  A second pass
runs the same steps stage by stage through the per-stage entry points with
HIP events between the stages for the breakdown and the rooflines.  Prints
one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
PCIE5_X16_GBPS = 64.0          # published host-link rate per direction


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=32)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--workload", default="32k-b16")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="budget for the oracle CPU baseline (0 = skip)")
    p.add_argument("--quiet", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the 128K and multi-layer prefetch measurements")
    p.add_argument("--layers", type=int, default=16,
                   help="layers of the 16-layer configuration to run (16 = all)")
    p.add_argument("--extra-only", choices=["prefill_pipeline", "eviction_replay",
                                            "fp8_entries", "growing_context", "multilayer"],
                   help="only run one extra measurement and print its JSON (for "
                        "profiling it alone)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy (known "
                        "bytes) for scaling the HBM traffic counters")
    p.add_argument("--trace-summary", metavar="CSV",
                   help="summarise a rocprofv3 kernel_trace.csv or "
                        "counter_collection.csv of a run with the same "
                        "--steps/--warmup: per kernel, the dispatches of the "
                        "timed steps only (all dispatches if the file holds no "
                        "timed window), then exit")
    return p.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def host_machine():
    """The host the oracle runs on: logical CPUs, the ones this process may
    use, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model}


def cpu_baseline(wl, seconds, requests=None, layers=1):
    """The oracle, as is, on the same workload: (layer, request) sequences in
    order - layers 0.. of requests 0, 1, ... (or the given requests) - each
    run from its fill through its steps, until about `seconds` of step time
    (fill and input generation excluded) have been spent.  A workload step
    is B * layers request-layer-steps of oracle work for B * m query
    tokens, so query-tok/s = m * (request-layer-steps per second) / layers;
    with sampled requests or layers the figure is extrapolated that way."""
    from oracle import decode as odecode
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    requests = list(range(wl.batch)) if requests is None else list(requests)
    n, spent, seqs = 0, 0.0, []
    for b in requests:
        for layer in range(layers):
            it = odecode.run_workload_request(wl, layer, b, check_pool=False)
            next(it)                              # the fill (untimed)
            seqs.append((layer, b))
            while spent < seconds:
                t0 = time.perf_counter()
                try:
                    next(it)
                except StopIteration:
                    break
                spent += time.perf_counter() - t0
                n += 1
            if spent >= seconds:
                break
        if spent >= seconds:
            break
    sampled = layers > 1 or len(seqs) < wl.batch * layers
    return {"value": wl.mtp * n / spent / layers, "unit": "query-tok/s",
            "cores": int(cores), "kind": "oracle",
            "steps_per_s": n / spent / (wl.batch * layers),
            "extrapolated": sampled,
            "sample": f"{n} request-layer-steps of {wl.name} over (layer, request) "
                      f"{seqs[0]}..{seqs[-1]} ({len(seqs)} sequences, fills excluded), "
                      f"{spent:.1f} s of step time"
                      + (f"; one step = {wl.batch} requests x {layers} layers, "
                         "scaled from the sample" if sampled else "")}


# Kernels whose counters give roofline.traffic, with the source each is
# built from; a recorded figure only counts while that source is unchanged.
def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")


KERNEL_SOURCES = {
    "index_scores_kernel": "index_scores.hip",
    "topk_kernel": "topk.hip",
    "topk_level_kernel": "topk.hip",
    "topk_final_kernel": "topk.hip",
    "topk_split_kernel": "topk.hip",
    "split_clear_kernel": "topk.hip",
    "select_update_kernel": "topk.hip",
    "pool_update_kernel": "pool_update.hip",
    "pool_reset_kernel": "pool_update.hip",
    "pool_status_kernel": "pool_update.hip",
    "miss_copy_kernel": "miss_copy.hip",
    "entry_copy_kernel": "miss_copy.hip",
    "append_tokens_kernel": "tail.hip",
    "sparse_mla_kernel": "sparse_mla.hip",
    "mla_combine_kernel": "sparse_mla.hip",
    "append_rows_kernel": "prefill.hip",
    "column_sums_kernel": "prefill.hip",
    "column_sums_reduce_kernel": "prefill.hip",
}


def source_digest(kernel):
    """Digest of the kernel's source file together with every header of the
    kernel sources (any of which it may include)."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "decode_lightning_indexer_amd", "csrc")
    h = hashlib.sha256()
    for path in [os.path.join(csrc, KERNEL_SOURCES[kernel])] + sorted(glob.glob(os.path.join(csrc, "*.h"))):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE scaled by a known-size copy),
    or None when there is none or the kernel's source has changed since."""
    try:
        with open(traffic_file(workload)) as f:
            for line in f:
                w = line.split()
                if len(w) == 4 and w[0] == "traffic" and w[1] == kernel:
                    return float(w[2]) if w[3] == source_digest(kernel) else None
    except OSError:
        pass
    return None


def trace_summary(path, steps, warmup):
    """Per-kernel mean duration (and mean value of each counter, for a
    counter run) over the timed steps: the window from the first timed
    step's index_scores_kernel to the next one after the timed steps
    (dispatch 0 is the pool's first fill).  A counter file has one row per
    (dispatch, counter)."""
    import csv
    import re
    rows = list(csv.DictReader(open(path)))
    # One record per dispatch: name, start, end and its counters.
    disp = {}
    for r in rows:
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Start_Timestamp"])
        d = disp.setdefault(key, {"name": r["Kernel_Name"], "t0": int(r["Start_Timestamp"]),
                                  "t1": int(r["End_Timestamp"]), "ctr": {}})
        if "Counter_Name" in r:
            d["ctr"][r["Counter_Name"]] = d["ctr"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ds = sorted(disp.values(), key=lambda d: d["t0"])

    def short(n):
        m = re.match(r"_ZN3ess12_GLOBAL__N_1(\d+)", n)   # names left mangled
        if m:
            ln = int(m.group(1))
            base = n[m.end():m.end() + ln]
            t = re.match(r"I((?:L[ib]\d+E)+)E", n[m.end() + ln:])
            if not t:
                return base
            args = [("false", "true")[int(v)] if k == "b" else v
                    for k, v in re.findall(r"L([ib])(\d+)E", t.group(1))]
            return base + "<" + ", ".join(args) + ">"
        n = n.replace("ess::(anonymous namespace)::", "").replace("void ", "")
        return n.split("(")[0]
    starts = [d["t0"] for d in ds if short(d["name"]).startswith("index_scores_kernel")]
    windowed = len(starts) > warmup + steps + 1
    if windowed:
        lo, hi = starts[warmup + 1], starts[warmup + steps + 1]
        ds = [d for d in ds if lo <= d["t0"] < hi]
    ctrs = sorted({c for d in ds for c in d["ctr"]})
    agg = {}
    for d in ds:
        a = agg.setdefault(short(d["name"]), {"n": 0, "us": 0.0, "ctr": {}})
        a["n"] += 1
        a["us"] += (d["t1"] - d["t0"]) / 1e3
        for c, v in d["ctr"].items():
            a["ctr"][c] = a["ctr"].get(c, 0.0) + v
    print(f"# {'timed steps' if windowed else 'all dispatches'}: {path}")
    head = f"{'kernel':48s} {'dispatches':>10s} {'mean_us':>9s}"
    for c in ctrs:
        head += f" {c:>26s}"
    print(head)
    for name, a in sorted(agg.items(), key=lambda kv: -kv[1]["us"]):
        if windowed and a["n"] < steps:
            continue                  # not a per-step kernel
        line = f"{name[:48]:48s} {a['n']:10d} {a['us'] / a['n']:9.2f}"
        for c in ctrs:
            line += f" {a['ctr'].get(c, 0.0) / a['n']:26.1f}"
        print(line)
    for name in KERNEL_SOURCES:
        print(f"# source {name} {source_digest(name)}")
    return 0


def staged_inputs(wl, layer, dev):
    """Index queries and absorbed queries of every step of one layer, in
    device memory (the timed region then reads nothing from the host but
    the misses)."""
    import numpy as np
    import torch
    from synth import gen
    q_all, w, n_vis = gen.index_inputs(wl, layer)
    qi = torch.from_numpy(q_all).to(dev)
    qa = torch.empty((wl.steps, wl.batch, wl.mtp, wl.mla_heads, 576),
                     dtype=torch.int16, device=dev)
    for t in range(wl.steps):
        qa[t].copy_(torch.from_numpy(gen.abs_query(wl, layer, t).view(np.int16)))
    return qi, qa, w, n_vis


def run_steps(args, name, n_layers, modes, K, W, resident=False, store="bf16"):
    """Whole steps of a workload through ess_decode_step: per mode, from the
    same first fill, W warm-up steps then K timed steps.  Returns per-mode
    step times, misses of the last step, and the last step's miss copies
    replayed alone (the host-link time a step needs).  store="entries": the
    host store holds the latents as 656-byte fp8 entries."""
    import numpy as np
    import torch
    from decode_lightning_indexer_amd import ess
    from decode_lightning_indexer_amd.session import HostStore, LayerBuffers, dims_of
    from synth import gen, get_workload

    from concurrent.futures import ThreadPoolExecutor

    dev = "cuda"
    wl = get_workload(name).with_(steps=W + K)
    d = dims_of(wl)
    B, m, L, k = wl.batch, wl.mtp, wl.ctx_len, wl.topk
    t0 = time.perf_counter()
    hosts, lbs, qis, qas = [], [], [], []
    n_vis = None
    for l in range(n_layers):
        if store == "entries":
            h = HostStore((B, L, 656), np.uint8)

            def enc(b, h=h, l=l):
                h.array[b] = gen.encode_entries(gen.latents(wl, l, b))
            with ThreadPoolExecutor(max_workers=8) as ex:
                list(ex.map(enc, range(B)))
            lb = LayerBuffers(d, None, entries=h)
        else:
            h = HostStore((B, L, 576))
            gen.fill_latents(wl, l, h.array)
            lb = LayerBuffers(d, h)
        kb = np.empty((B, L, wl.idx_dim), np.uint8)
        gen.fill_index_keys(wl, l, kb)
        lb.k_idx.copy_(torch.from_numpy(kb))
        del kb
        qi, qa, w, nv = staged_inputs(wl, l, dev)
        lb.w_idx.copy_(torch.from_numpy(w))
        n_vis = torch.from_numpy(nv).to(dev)
        hosts.append(h); lbs.append(lb); qis.append(qi); qas.append(qa)
    torch.cuda.synchronize()
    log(args, f"{name}: {n_layers} layer(s) ready in {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()              # default priority

    def ios(t):
        out = []
        for l, lb in enumerate(lbs):
            io = lb.io()
            io.q_idx = qis[l][t].data_ptr()
            io.q_abs = qas[l][t].data_ptr()
            out.append(io)
        return out

    steps = [ios(t) for t in range(W + K)]
    res = {}
    n_miss_steps = torch.zeros(K, dtype=torch.int64, device=dev)
    for mode in modes:
        for lb in lbs:
            lb.reset(stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        ess.ess_decode_step(d, steps[0], n_vis, ess.ESS_MODE_FILL, stream)
        ev[1].record(stream)
        for t in range(W):
            ess.ess_decode_step(d, steps[t], n_vis, mode, stream, side)
        torch.cuda.synchronize()
        res.setdefault("fill", ev[0].elapsed_time(ev[1]) * 1e-3)
        t1 = time.perf_counter()
        for i in range(K):
            ess.ess_decode_step(d, steps[W + i], n_vis, mode, stream, side)
        torch.cuda.synchronize()
        res[mode] = (time.perf_counter() - t1) / K
        if mode == modes[0]:
            # Misses per timed step (the same steps again, counted: the
            # timed pass records nothing between its calls).
            for lb in lbs:
                lb.reset(stream)
            ess.ess_decode_step(d, steps[0], n_vis, ess.ESS_MODE_FILL, stream)
            for t in range(W + K):
                ess.ess_decode_step(d, steps[t], n_vis, mode, stream, side)
                if t >= W:
                    n_miss_steps[t - W] = sum(lb.n_miss.sum() for lb in lbs)
            torch.cuda.synchronize()
            res["misses_per_step"] = float(n_miss_steps.double().mean())
    n_miss = sum(int(lb.n_miss.sum()) for lb in lbs)
    # The last step's miss lists copied again, alone: host-link time of a step.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for lb in lbs:
        if store == "entries":
            ess.ess_miss_copy_entries(d, m * k, lb.miss_pos, lb.miss_slot,
                                      lb.n_miss, lb.entries.dev, lb.pool, stream)
        else:
            ess.ess_miss_copy(d, m * k, lb.miss_pos, lb.miss_slot, lb.n_miss,
                              lb.host.dev, lb.pool, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    t_copy = ev[0].elapsed_time(ev[1]) * 1e-3
    if resident:
        # The last step again: every row it selects is now in the pool, so
        # this is the same step with no misses (selection, update and
        # attention all run; nothing crosses the host link).
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ess.ess_decode_step(d, steps[W + K - 1], n_vis, ess.ESS_MODE_INLINE, stream, side)
        ev[0].record(stream)
        for _ in range(4):
            ess.ess_decode_step(d, steps[W + K - 1], n_vis, ess.ESS_MODE_INLINE, stream, side)
        ev[1].record(stream)
        torch.cuda.synchronize()
        res["resident"] = ev[0].elapsed_time(ev[1]) * 1e-3 / 4
        res["resident_misses"] = sum(int(lb.n_miss.sum()) for lb in lbs)
    for h in hosts:
        h.free()
    return res, n_miss, t_copy, wl


def overlap_split(d, lb, qi, qa, n_vis, ts, stream, host_dev):
    """The pages' OverlapRatio (FlashOffloading analysis, "numbers: 1.03x to
    1.27x") on steps ts, each selected through the per-stage calls, then its
    gather + attention timed three ways with HIP events on the launch
    stream: T_fused = the call with per-row writer slots (the misses read
    from host memory inside the attention kernel and written to their
    slots), T_copy = the step's miss list copied host -> pool alone, T_attn
    = the attention with every row read from the pool.  Returns the mean
    times (us), the ratio (T_copy + T_attn - T_fused) / T_copy, its physical
    bound min(1, T_attn / T_copy) and the misses per step."""
    import numpy as np
    import torch
    from decode_lightning_indexer_amd import ess
    m, k = d.mtp, d.topk
    sel_pos, sel_slot = lb.rows(lb.sel_pos, k, m), lb.rows(lb.sel_slot, k, m)
    row_dst, post = lb.rows(lb.row_dst, k, m), lb.rows(lb.sel_slot_post, k, m)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in ts]
    n_miss = torch.zeros(len(ts), dtype=torch.int64, device=lb.n_miss.device)
    for i, t in enumerate(ts):
        ess.ess_index_scores(d, qi[t], lb.w_idx, lb.k_idx, n_vis, lb.scores, stream)
        ess.ess_topk_lookup(d, k, m, lb.scores, n_vis, lb.cache_slots, sel_pos, sel_slot,
                            lb.n_sel, lb.ws, lb.ws_bytes, stream)
        ess.ess_pool_update(d, k, m, sel_pos, lb.n_sel, lb.cache_slots, lb.slot_pos, lb.lru,
                            lb.miss_pos, lb.miss_slot, lb.n_miss, lb.n_evict, row_dst, post,
                            stream)
        e = evs[i]
        e[0].record(stream)
        ess.ess_sparse_mla_decode(d, qa[t], sel_pos, sel_slot, row_dst, lb.n_sel, lb.pool,
                                  host_dev, lb.out, lb.lse, lb.ws, lb.ws_bytes, stream)
        e[1].record(stream)
        ess.ess_miss_copy(d, m * k, lb.miss_pos, lb.miss_slot, lb.n_miss, host_dev,
                          lb.pool, stream)
        e[2].record(stream)
        ess.ess_sparse_mla_decode(d, qa[t], sel_pos, post, None, lb.n_sel, lb.pool,
                                  host_dev, lb.out, lb.lse, lb.ws, lb.ws_bytes, stream)
        e[3].record(stream)
        n_miss[i] = lb.n_miss.sum()
    torch.cuda.synchronize()
    tt = np.zeros(3)
    for e in evs:
        tt += [e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
    t_fused, t_copy, t_attn = tt / len(ts) * 1e3
    return {"t_copy_us": t_copy, "t_attn_us": t_attn, "t_fused_us": t_fused,
            "ratio": (t_copy + t_attn - t_fused) / t_copy if t_copy > 0 else None,
            "bound": min(1.0, t_attn / t_copy) if t_copy > 0 else None,
            "misses_per_step": float(n_miss.double().mean())}


def single_layer_config(args, name, K=16, burn=16, n_ov=8, index_flush=False):
    """One single-layer workload through ess_decode_step: the first fill
    (event-timed), `burn` untimed steps, K timed steps (misses counted per
    step), then n_ov further steps split for the OverlapRatio; optionally
    the indexer alone over rotating copies of the index cache (from HBM).
    Steps/s are reported without and with the fill over the workload's own
    step count."""
    import numpy as np
    import torch
    from decode_lightning_indexer_amd import ess
    from decode_lightning_indexer_amd.session import HostStore, LayerBuffers, dims_of
    from synth import gen, get_workload

    dev = "cuda"
    base = get_workload(name)
    wl = base.with_(steps=burn + K + n_ov)
    d = dims_of(wl)
    B, m, L, k = wl.batch, wl.mtp, wl.ctx_len, wl.topk
    t0 = time.perf_counter()
    host = HostStore((B, L, 576))
    gen.fill_latents(wl, 0, host.array)
    lb = LayerBuffers(d, host)
    kb = np.empty((B, L, wl.idx_dim), np.uint8)
    gen.fill_index_keys(wl, 0, kb)
    lb.k_idx.copy_(torch.from_numpy(kb))
    del kb
    qi, qa, w, nv = staged_inputs(wl, 0, dev)
    lb.w_idx.copy_(torch.from_numpy(w))
    n_vis = torch.from_numpy(nv).to(dev)
    torch.cuda.synchronize()
    log(args, f"{name}: ready in {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    n_miss_all = torch.zeros((wl.steps, B), dtype=torch.int32, device=dev)

    def io(t):
        x = lb.io()
        x.q_idx, x.q_abs = qi[t].data_ptr(), qa[t].data_ptr()
        x.n_miss = n_miss_all[t].data_ptr()
        return [x]
    ios = [io(t) for t in range(wl.steps)]
    lb.reset(stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    ess.ess_decode_step(d, ios[0], n_vis, ess.ESS_MODE_FILL, stream)
    ev[1].record(stream)
    for t in range(burn):
        ess.ess_decode_step(d, ios[t], n_vis, ess.ESS_MODE_INLINE, stream)
    torch.cuda.synchronize()
    t_fill = ev[0].elapsed_time(ev[1]) * 1e-3
    t1 = time.perf_counter()
    for i in range(K):
        ess.ess_decode_step(d, ios[burn + i], n_vis, ess.ESS_MODE_INLINE, stream)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t1) / K
    misses = n_miss_all[burn:burn + K].double().sum(dim=1)
    T = base.steps
    out = {"steps_per_s": 1 / t_step, "query_tok_s": B * m / t_step,
           "us_per_step": t_step * 1e6, "rho": wl.rho,
           "burn_in_steps": burn, "timed_steps": K,
           "fill_us": t_fill * 1e6,
           "steps_per_s_incl_fill": T / (t_fill + T * t_step),
           "query_tok_s_incl_fill": B * m * T / (t_fill + T * t_step),
           "workload_steps": T,
           "misses_per_step": float(misses.mean()),
           "miss_rate": float(misses.mean()) / (B * m * k)}
    if n_ov > 0:
        out["overlap"] = overlap_split(d, lb, qi, qa, n_vis,
                                       range(burn + K, burn + K + n_ov), stream, host.dev)
    if index_flush:
        cold, warm, n_copies = indexer_alone(d, lb, qi[burn + K - 1], n_vis, stream)
        idx_bytes = B * L * wl.idx_dim + B * m * L * 4 + B * m * wl.idx_heads * (wl.idx_dim + 4)
        out["indexer"] = {"bytes_per_launch": idx_bytes, "us_from_hbm": cold * 1e6,
                          "gbps_from_hbm": idx_bytes / cold / 1e9,
                          "frac_of_hbm_peak": idx_bytes / cold / 1e9 / HBM_PEAK_GBPS,
                          "index_cache_copies": n_copies,
                          "same_cache_back_to_back_gbps": idx_bytes / warm / 1e9}
    host.free()
    del lb, qi, qa
    torch.cuda.empty_cache()
    log(args, f"{name}: {out}")
    return out


def multilayer(args, n_layers=16, K=16, W=16):
    """The 16-layer configuration (64K context, 32 requests per layer) over
    n_layers layers: inline against side-stream prefetch, the host link's
    busy share, and the multi-layer overlap of the miss transfer."""
    from decode_lightning_indexer_amd import ess
    t0 = time.perf_counter()
    name = "64k-b32-16layer"
    res, n_miss, t_copy, wl = run_steps(
        args, name, n_layers, [ess.ESS_MODE_INLINE, ess.ESS_MODE_PREFETCH], K, W,
        resident=True)
    ti, tp = res[ess.ESS_MODE_INLINE], res[ess.ESS_MODE_PREFETCH]
    t_res = res["resident"]
    # Prefetch hides the next layer's selection under this layer's copy and
    # attention: the share of the step's non-copy work that disappears, and
    # how much of each step the host link is busy.
    T = 16
    res_out = {"layers_timed": n_layers, "burn_in_steps": W, "timed_steps": K,
               "inline_us_per_step": ti * 1e6, "prefetch_us_per_step": tp * 1e6,
               "steps_per_s": 1 / tp, "query_tok_s": wl.batch * wl.mtp / tp,
               "query_tok_s_prefetch": wl.batch * wl.mtp / tp,
               "query_tok_s_inline": wl.batch * wl.mtp / ti,
               "fill_us": res["fill"] * 1e6,
               "steps_per_s_incl_fill": T / (res["fill"] + T * tp),
               "misses_per_step": res["misses_per_step"],
               "miss_rate": res["misses_per_step"] / (n_layers * wl.batch * wl.mtp * wl.topk),
               "misses_last_step": n_miss,
               "miss_copy_us_last_step": t_copy * 1e6,
               "link_busy_inline": t_copy / ti, "link_busy_prefetch": t_copy / tp,
               # The multi-layer overlap of the miss transfer: (sum of the
               # step's copies + the step with every row resident - the
               # pipelined step) / the copies, with its bound.
               "resident_us_per_step": t_res * 1e6,
               "resident_step_misses": res["resident_misses"],
               "overlap_prefetch": (t_copy + t_res - tp) / t_copy,
               "overlap_inline": (t_copy + t_res - ti) / t_copy,
               "overlap_bound": min(1.0, t_res / t_copy),
               "hidden_noncopy_fraction": (ti - tp) / (ti - t_copy) if ti > t_copy else None}
    res_out["wall_s"] = time.perf_counter() - t0
    log(args, f"{name} over {n_layers} layers: {res_out}")
    return res_out


def config_measurements(args):
    """Every workload other than the headline one: the 4K oracle-sized
    decode, the 128K / MTP=2 configuration at its three query-drift rates
    (each with its OverlapRatio), the 1M-token single request at both pool
    sizes, and the 16-layer configuration (all of its layers unless
    --layers says fewer) with and without side-stream prefetch.  The
    indexer alone from HBM at 128K and 1M."""
    out = {}
    for name, flush in (("tiny-4k", False), ("128k-b8-mtp2-r099", False),
                        ("128k-b8-mtp2-r095", True), ("128k-b8-mtp2-r080", False),
                        ("1m-b1-c8k", False), ("1m-b1-c16k", True)):
        out[name] = single_layer_config(args, name, index_flush=flush)
    out["64k-b32-16layer"] = multilayer(args, n_layers=args.layers)
    return out


def fp8_entries(args, names=("32k-b16", "128k-b8-mtp2-r099")):
    """The same steps with the host store holding 656-byte fp8 entries: the
    misses cross the host link as entries, read inside the attention kernel,
    which dequantizes each in its tile and writes the bf16 row to its slot.
    Step time and the last step's entry copy replayed alone, beside the
    bf16 store's figures (bytes per miss 656 against 1152)."""
    from decode_lightning_indexer_amd import ess
    out = {}
    K, W = 16, 4
    for name in names:
        per = {}
        for store in ("bf16", "entries"):
            res, n_miss, t_copy, wl = run_steps(args, name, 1, [ess.ESS_MODE_INLINE],
                                                K, W, store=store)
            t = res[ess.ESS_MODE_INLINE]
            nbytes = n_miss * (656 if store == "entries" else 1152)
            per[store] = {"us_per_step": t * 1e6,
                          "query_tok_s": wl.batch * wl.mtp / t,
                          "misses_last_step": n_miss,
                          "host_bytes_last_step": nbytes,
                          "miss_copy_us_last_step": t_copy * 1e6,
                          "miss_copy_gbps": nbytes / t_copy * 1e-9 if t_copy > 0 else None}
        per["speedup"] = per["bf16"]["us_per_step"] / per["entries"]["us_per_step"]
        out[name] = per
        log(args, f"fp8 entries {name}: {per}")
    return out


def growing_context(args, name="32k-b16", block=64, K=32, W=8):
    """Whole steps with the context growing by one token per request per
    step (ess_append_tokens before each ess_decode_step, tail blocks of
    `block` tokens written back to the host store on their own stream),
    against the same steps over a fixed context: the cost of the append
    and of reading the newest positions from the tail."""
    import numpy as np
    import torch
    from decode_lightning_indexer_amd import ess
    from decode_lightning_indexer_amd.session import HostStore, LayerBuffers, dims_of
    from synth import gen, get_workload

    dev = "cuda"
    wl = get_workload(name).with_(steps=W + K)
    d = dims_of(wl)
    B, m, L = wl.batch, wl.mtp, wl.ctx_len
    L0 = L - (W + K) * m
    host = HostStore((B, L, 576))
    gen.fill_latents(wl, 0, host.array)
    T = W + K
    # New tokens per step as contiguous [B][m][...] blocks: [T][B][m][...].
    lat_new = torch.from_numpy(np.ascontiguousarray(
        host.array[:, L0:].reshape(B, T, m, 576).transpose(1, 0, 2, 3)).view(np.int16)).to(dev)
    lb = LayerBuffers(d, host)
    kb = np.empty((B, L, wl.idx_dim), np.uint8)
    gen.fill_index_keys(wl, 0, kb)
    keys_new = torch.from_numpy(np.ascontiguousarray(
        kb[:, L0:].reshape(B, T, m, wl.idx_dim).transpose(1, 0, 2, 3))).to(dev)
    lb.k_idx.copy_(torch.from_numpy(kb))
    del kb
    qi, qa, w, _ = staged_inputs(wl, 0, dev)
    lb.w_idx.copy_(torch.from_numpy(w))
    n_vis = torch.empty((B, m), dtype=torch.int32, device=dev)
    rows = torch.empty((B, 2 * block, 576), dtype=torch.int16, device=dev)
    state = torch.empty(3 * B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    side, d2h = torch.cuda.Stream(), torch.cuda.Stream()
    out = {}
    for grow in (False, True):
        n_vis.copy_(torch.tensor([[L0 - m + 1 + j for j in range(m)]] * B, dtype=torch.int32))
        lb.reset(stream)
        io = lb.io()
        io.q_idx, io.q_abs = qi[0].data_ptr(), qa[0].data_ptr()
        ess.ess_decode_step(d, [io], n_vis, ess.ESS_MODE_FILL, stream)
        tail = ess.ess_tail_init(d, rows, block, [L0] * B, state, stream)
        if not grow:        # the fixed context: every step sees L0 + 1 positions
            n_vis.copy_(torch.tensor([[L0 + 1 + j for j in range(m)]] * B, dtype=torch.int32))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        misses = 0
        for t in range(W + K):
            if t == W:
                torch.cuda.synchronize()
                ev[0].record(stream)
            if grow:
                ess.ess_append_tokens(d, tail, keys_new[t], lat_new[t], lb.k_idx, n_vis,
                                      host.host, stream, d2h)
            io = lb.io()
            io.q_idx, io.q_abs = qi[t].data_ptr(), qa[t].data_ptr()
            if grow:
                io.tail_rows, io.tail_start, io.tail_block = rows.data_ptr(), tail.start_dev, block
            ess.ess_decode_step(d, [io], n_vis, ess.ESS_MODE_INLINE, stream, side)
        ev[1].record(stream)
        torch.cuda.synchronize()
        misses = int(lb.n_miss.sum())
        ess.ess_tail_release(tail)
        t_step = ev[0].elapsed_time(ev[1]) * 1e-3 / K
        out["growing" if grow else "fixed"] = {
            "us_per_step": t_step * 1e6, "query_tok_s": B * m / t_step,
            "misses_last_step": misses}
    out["block"] = block
    out["written_back_per_block_mb"] = B * block * 1152 / 1e6
    # Device-resident latent bytes of the layer against a fully resident
    # cache: B (C + 2b) 1152 against B L 1152 (the K/V term of M_decode).
    out["device_latent_mb"] = B * (wl.pool_slots + 2 * block) * 1152 / 1e6
    out["full_resident_latent_mb"] = B * L * 1152 / 1e6
    out["resident_fraction"] = (wl.pool_slots + 2 * block) / L
    out["context_start"] = L0
    host.free()
    log(args, f"growing context {name}: {out}")
    return out


def replay_curves(args, name="128k-b8-mtp2-r095", T=32,
                  capacities=(8192, 12288, 16384, 24576)):
    """The pages' offline eviction-policy comparison on traces of our own
    decode: T steps of the workload run on the GPU (fill, then inline steps
    with the workload's pool), every step's scores and selections copied to
    host memory, then each request replayed through ess_replay_evictions
    under LRU, Random and Score at several pool sizes.  The LRU replay at the
    workload's own pool size must reproduce the GPU pool update's miss count
    of every request and step."""
    import numpy as np
    import torch
    from decode_lightning_indexer_amd import ess
    from decode_lightning_indexer_amd.session import HostStore, LayerBuffers, dims_of
    from synth import gen, get_workload

    dev = "cuda"
    wl = get_workload(name).with_(steps=T)
    d = dims_of(wl)
    B, m, L, k, C = wl.batch, wl.mtp, wl.ctx_len, wl.topk, wl.pool_slots
    h = HostStore((B, L, 576))
    gen.fill_latents(wl, 0, h.array)
    lb = LayerBuffers(d, h)
    kb = np.empty((B, L, wl.idx_dim), np.uint8)
    gen.fill_index_keys(wl, 0, kb)
    lb.k_idx.copy_(torch.from_numpy(kb))
    del kb
    qi, qa, w, nv = staged_inputs(wl, 0, dev)
    lb.w_idx.copy_(torch.from_numpy(w))
    n_vis = torch.from_numpy(nv).to(dev)
    stream = torch.cuda.current_stream()
    scores = np.empty((B, T, m, L), np.float32)
    sel = np.empty((B, T, m, k), np.int32)
    n_sel = np.empty((B, T, m), np.int32)
    gpu_miss = np.empty((B, T), np.int32)
    lb.reset(stream)
    io = lb.io()
    io.q_idx = qi[0].data_ptr()
    ess.ess_decode_step(d, [io], n_vis, ess.ESS_MODE_FILL, stream)
    for t in range(T):
        io = lb.io()
        io.q_idx = qi[t].data_ptr()
        io.q_abs = qa[t].data_ptr()
        ess.ess_decode_step(d, [io], n_vis, ess.ESS_MODE_INLINE, stream)
        scores[:, t] = lb.scores.cpu().numpy()
        sel[:, t] = lb.rows(lb.sel_pos, k, m).cpu().numpy()
        n_sel[:, t] = lb.n_sel.cpu().numpy()
        gpu_miss[:, t] = lb.n_miss.cpu().numpy()
    h.free()
    del lb, qi, qa
    torch.cuda.empty_cache()

    codes = {"lru": ess.ESS_EVICT_LRU, "random": ess.ESS_EVICT_RANDOM,
             "score": ess.ESS_EVICT_SCORE}
    t0 = time.perf_counter()
    misses = {p: {} for p in codes}
    n_replays = 0
    for pol, code in codes.items():
        for cap in capacities:
            tot = 0
            for b in range(B):
                nm, _ = ess.ess_replay_evictions(code, cap, scores[b], sel[b], n_sel[b],
                                                 seed=1, request=b)
                n_replays += 1
                if pol == "lru" and cap == C and not np.array_equal(nm, gpu_miss[b]):
                    raise AssertionError(f"LRU replay differs from the GPU pool at request {b}")
                tot += int(nm.sum())
            misses[pol][cap] = tot
    t_replay = time.perf_counter() - t0
    per = B * T
    lo, hi = min(capacities), 16384
    return {
        "workload": name, "steps": T, "requests": B,
        # (per request and step; the pool's contents are compared with the
        # oracle, step by step, by the full-size parity tests)
        "lru_replay_miss_counts_equal_gpu_pool": True,
        "misses_per_request_step": {p: {str(c): v / per for c, v in d_.items()}
                                    for p, d_ in misses.items()},
        f"miss_cut_{lo}_to_{hi}": {p: 1 - misses[p][hi] / misses[p][lo] for p in codes},
        f"score_vs_lru_at_{hi}": 1 - misses["score"][hi] / misses["lru"][hi],
        f"random_vs_lru_at_{hi}": 1 - misses["random"][hi] / misses["lru"][hi],
        "replay_steps_per_s": n_replays * T / t_replay,
    }


def prefill_pipeline(args, NL=16, n_hist=32768, n_new=2048, ratios=(0.5, 1.0, 2.0)):
    """The four-buffer prefill pipeline (ess_prefill_layers) over NL layers
    of n_hist history rows + n_new new rows of 576 bf16: per layer, the
    history load (H2D) and the new rows' write-back (D2H) timed alone on
    their streams, the stand-in compute timed alone (layer 0 resident), and
    whole pipelined passes (median of five, one at a time) with the compute
    window set to about ratio x the load time.  Exposed time = pipelined - compute only, against the pages'
    per-layer bound max(0, tau_H2D - d_on tau_compute) (d_on = 2 layers for
    the default prefetch) and the serial-link bound."""
    import numpy as np
    import torch
    from decode_lightning_indexer_amd import ess
    from decode_lightning_indexer_amd.session import HostStore

    rows = n_hist + n_new
    dev = "cuda"
    store = HostStore((NL, rows, 576))
    rng = np.random.default_rng(7)
    block = rng.integers(-8, 9, (1024, 576)).astype(np.int16)
    table = np.array([0xC100, 0xC0E0, 0xC0C0, 0xC0A0, 0xC080, 0xC040, 0xC000, 0xBF80,
                      0x0000, 0x3F80, 0x4000, 0x4040, 0x4080, 0x40A0, 0x40C0, 0x40E0,
                      0x4100], np.uint16)                # bf16 of -8 .. 8
    pat = table[block + 8]
    for r0 in range(0, rows, 1024):
        r1 = min(rows, r0 + 1024)
        store.array[:, r0:r1] = pat[:r1 - r0]
    new = torch.from_numpy(table[rng.integers(-8, 9, (NL, n_new, 576)) + 8].view(np.int16)).to(dev)
    bufs = torch.zeros((4, rows, 576), dtype=torch.int16, device=dev)
    bufs[0, :n_hist] = torch.from_numpy(store.array[0, :n_hist].view(np.int16)).to(dev)
    out = torch.zeros((NL, 576), dtype=torch.float32, device=dev)
    ws = torch.empty(ess.ess_prefill_ws_bytes(rows), dtype=torch.uint8, device=dev)
    sc, sh, sd = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    row_b = 576 * 2

    def timed(stream, fn, reps=3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        stream.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        stream.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps * 1e-3

    # The per-layer transfers alone, through the library's copy call (one
    # HIP runtime in the process).
    def h2d():
        ess.ess_copy_async(bufs[1].data_ptr(), store.host + row_b * rows, n_hist * row_b, sh)

    def d2h():
        ess.ess_copy_async(store.host + row_b * (rows + n_hist), bufs[1][n_hist:].data_ptr(),
                           n_new * row_b, sd)

    def call(n_layers, reps):
        with torch.cuda.stream(sc):
            ess.ess_prefill_layers(n_layers, rows, n_hist, n_new, store.host, new, bufs,
                                   out, ws, compute_reps=reps, compute=sc, h2d=sh, d2h=sd)

    t_h2d = timed(sh, h2d)
    t_d2h = timed(sd, d2h)
    # One layer (layer 0, resident): compute + its write-back; two rep counts
    # give the time per on-chip repetition of the stand-in compute and its
    # fixed part (one pass over the buffer, the launches, the write-back).
    call(NL, 1)                              # first use: events, kernels loaded
    torch.cuda.synchronize()
    ta = timed(sc, lambda: call(1, 64), reps=5)
    tb = timed(sc, lambda: call(1, 1064), reps=5)
    per_rep = max(1e-9, (tb - ta) / 1000)
    fixed = max(0.0, ta - 64 * per_rep)
    # A discarded pass at the shortest window first: the first pipelined
    # runs in a process were up to 25 % slower (12-13.7 ms against
    # 10.7-10.9 ms at compute/load 0.56, with or without write-backs), so
    # the link and clocks are brought out of idle before anything is timed.
    def reps_for(ratio):
        return max(1, int(round((ratio * t_h2d + t_d2h - fixed) / per_rep)))
    timed(sc, lambda: call(NL, reps_for(min(ratios))), reps=3)
    runs = []
    for ratio in ratios:
        reps = reps_for(ratio)
        t_layer = timed(sc, lambda: call(1, reps))           # compute + write-back
        t_c = max(1e-9, t_layer - t_d2h)
        # One prefill pass per timing (each after the previous has finished;
        # passes issued back to back measured 1-1.6 ms slower each, the next
        # pass's first loads waiting on the previous pass's last layers);
        # the median of five.
        t_pipe = float(np.median([timed(sc, lambda: call(NL, reps), reps=1) for _ in range(5)]))
        t_only = NL * t_c + t_d2h
        exposed = max(0.0, t_pipe - t_only)
        loads = (NL - 1) * t_h2d
        runs.append({
            "compute_reps": reps, "tau_compute_ms": t_c * 1e3,
            "compute_over_load": t_c / t_h2d,
            "t_pipelined_ms": t_pipe * 1e3, "t_compute_only_ms": t_only * 1e3,
            "exposed_ms": exposed * 1e3,
            "bound_pages_ms": (NL - 1) * max(0.0, t_h2d - 2 * t_c) * 1e3,
            "bound_serial_link_ms": max(0.0, loads + t_c - NL * t_c) * 1e3,
            "load_hidden_fraction": 1 - exposed / loads,
        })
    store.free()
    return {"layers": NL, "history_rows": n_hist, "new_rows": n_new,
            "layer_bytes": n_hist * row_b,
            "tau_h2d_ms": t_h2d * 1e3, "h2d_gbps": n_hist * row_b / t_h2d / 1e9,
            "tau_d2h_ms": t_d2h * 1e3, "d2h_gbps": n_new * row_b / t_d2h / 1e9,
            "runs": runs}


def indexer_alone(d, lb, q_idx, n_vis, stream, reps=16):
    """Indexer kernel time alone, launches back to back with events only
    around the whole run: over copies of the index cache taken in turn,
    enough of them (>= 512 MB) that each launch finds its keys evicted from
    the 256 MB last-level cache (the 16-layer shape's situation: every
    layer's cache is read once per step), and over the one cache again and
    again (which then stays in the last-level cache)."""
    import torch
    from decode_lightning_indexer_amd import ess
    key_bytes = lb.k_idx.numel()
    n_copies = max(2, -(-(512 << 20) // key_bytes))
    copies = [lb.k_idx.clone() for _ in range(n_copies)]
    reps = max(reps, 2 * n_copies)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for i in range(n_copies):          # warm-up: one pass over the copies
        ess.ess_index_scores(d, q_idx, lb.w_idx, copies[i], n_vis, lb.scores, stream)
    ev[0].record(stream)
    for i in range(reps):
        ess.ess_index_scores(d, q_idx, lb.w_idx, copies[i % n_copies], n_vis, lb.scores, stream)
    ev[1].record(stream)
    ev[2].record(stream)
    for _ in range(reps):
        ess.ess_index_scores(d, q_idx, lb.w_idx, lb.k_idx, n_vis, lb.scores, stream)
    ev[3].record(stream)
    torch.cuda.synchronize()
    cold = ev[0].elapsed_time(ev[1]) / reps
    warm = ev[2].elapsed_time(ev[3]) / reps
    del copies
    torch.cuda.empty_cache()
    return cold * 1e-3, warm * 1e-3, n_copies


def main():
    args = parse()
    if args.trace_summary:
        return trace_summary(args.trace_summary, args.steps, args.warmup)
    if args.extra_only:
        import torch
        torch.cuda.set_device(0)
        fn = {"prefill_pipeline": prefill_pipeline, "eviction_replay": replay_curves,
              "fp8_entries": lambda a: fp8_entries(a, (a.workload,)),
              "growing_context": lambda a: growing_context(a, a.workload),
              "multilayer": lambda a: multilayer(a, a.layers)}
        print(json.dumps({args.extra_only: fn[args.extra_only](args)}), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not "
              "supported (requests shard across GPUs with no exchange; see "
              "the design notes)", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    if args.copy_calibration:
        torch.cuda.set_device(0)
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel(), "copy_bytes_written": b.numel(),
                          "launches": 4}), flush=True)
        return 0

    from decode_lightning_indexer_amd import ess
    from decode_lightning_indexer_amd.session import HostStore, LayerBuffers, dims_of
    from synth import gen, get_workload

    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup
    # Untimed steps after the first fill: at least 16 whatever --warmup is,
    # so that the timed steps see the pool's steady state (misses per step
    # grow over the first steps after the fill).
    burn = max(16, W)
    n_ov = min(8, K)                       # extra steps for the overlap split
    base = get_workload(args.workload)
    wl = base.with_(steps=burn + K + n_ov)
    B, m, L, k, C, H = wl.batch, wl.mtp, wl.ctx_len, wl.topk, wl.pool_slots, wl.mla_heads
    d = dims_of(wl)
    dev = "cuda"

    t_gen = time.perf_counter()
    host = HostStore((B, L, 576))
    gen.fill_latents(wl, 0, host.array)
    lb = LayerBuffers(d, host)
    kb = np.empty((B, L, wl.idx_dim), np.uint8)
    gen.fill_index_keys(wl, 0, kb)
    lb.k_idx.copy_(torch.from_numpy(kb))
    del kb
    q_all, w, n_vis_np = gen.index_inputs(wl, 0)
    lb.w_idx.copy_(torch.from_numpy(w))
    q_idx = torch.from_numpy(q_all).to(dev)                     # [T][B][m][HI][dI]
    q_abs = torch.empty((wl.steps, B, m, H, 576), dtype=torch.int16, device=dev)
    for t in range(wl.steps):
        q_abs[t].copy_(torch.from_numpy(gen.abs_query(wl, 0, t).view(np.int16)))
    n_vis = torch.from_numpy(n_vis_np).to(dev)
    torch.cuda.synchronize()
    log(args, f"inputs ready in {time.perf_counter() - t_gen:.1f} s")

    stream = torch.cuda.current_stream()
    lists = m * k
    sel_pos = lb.rows(lb.sel_pos, k, m)
    sel_slot = lb.rows(lb.sel_slot, k, m)
    row_dst = lb.rows(lb.row_dst, k, m)
    post = lb.rows(lb.sel_slot_post, k, m)

    n_miss_all = torch.zeros((wl.steps, B), dtype=torch.int32, device=dev)

    # Misses are read from host memory inside the attention kernel and
    # written to their slots from the tile.
    names = ["index_scores", "topk_lookup", "pool_update", "gather_attention"]
    n_st = len(names)

    def step(t, ev=None):
        if ev is not None:
            ev[0].record(stream)
        ess.ess_index_scores(d, q_idx[t], lb.w_idx, lb.k_idx, n_vis, lb.scores, stream)
        if ev is not None:
            ev[1].record(stream)
        ess.ess_topk_lookup(d, k, m, lb.scores, n_vis, lb.cache_slots, sel_pos,
                            sel_slot, lb.n_sel, lb.ws, lb.ws_bytes, stream)
        if ev is not None:
            ev[2].record(stream)
        ess.ess_pool_update(d, k, m, sel_pos, lb.n_sel, lb.cache_slots, lb.slot_pos,
                            lb.lru, lb.miss_pos, lb.miss_slot, n_miss_all[t], lb.n_evict,
                            row_dst, post, stream)
        if ev is not None:
            ev[3].record(stream)
        ess.ess_sparse_mla_decode(d, q_abs[t], sel_pos, sel_slot, row_dst, lb.n_sel,
                                  lb.pool, host.dev, lb.out, lb.lse, lb.ws,
                                  lb.ws_bytes, stream)
        if ev is not None:
            ev[4].record(stream)

    # First fill (top-C of token 0 at step 0 into the empty pool), untimed.
    lb.reset(stream)
    lb.q_idx.copy_(q_idx[0])
    ess.ess_decode_step(d, [lb.io()], n_vis, ess.ESS_MODE_FILL, stream)
    torch.cuda.synchronize()

    for t in range(burn):
        step(t)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_st + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(burn + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = np.zeros(n_st)
    for e in evs:
        for s in range(n_st):
            stage_ms[s] += e[s].elapsed_time(e[s + 1])
    stage_us = stage_ms / K * 1e3
    n_miss_tot = int(n_miss_all[burn:burn + K].sum())

    # The same steps without the per-stage events, as one ess_decode_step
    # call per step: the headline figure.  Each step's miss counts go to a
    # buffer of their own (no work added between the calls).
    n_miss_plain = torch.zeros((wl.steps, B), dtype=torch.int32, device=dev)
    ios = []
    for t in range(burn + K):
        io = lb.io()
        io.q_idx = q_idx[t].data_ptr()
        io.q_abs = q_abs[t].data_ptr()
        io.n_miss = n_miss_plain[t].data_ptr()
        ios.append([io])
    lb.reset(stream)
    ev_fill = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev_fill[0].record(stream)
    ess.ess_decode_step(d, ios[0], n_vis, ess.ESS_MODE_FILL, stream)
    ev_fill[1].record(stream)
    for t in range(burn):
        ess.ess_decode_step(d, ios[t], n_vis, ess.ESS_MODE_INLINE, stream)
    torch.cuda.synchronize()
    t_fill = ev_fill[0].elapsed_time(ev_fill[1]) * 1e-3
    t1 = time.perf_counter()
    for i in range(K):
        ess.ess_decode_step(d, ios[burn + i], n_vis, ess.ESS_MODE_INLINE, stream)
    torch.cuda.synchronize()
    wall_plain = time.perf_counter() - t1
    miss_plain = n_miss_plain[burn:burn + K].double().sum(dim=1)

    # Overlap on further steps (the pages' OverlapRatio): T_fused, T_copy
    # and T_attn of each step's gather + attention.
    ov = overlap_split(d, lb, q_idx, q_abs, n_vis, range(burn + K, burn + K + n_ov),
                       stream, host.dev)
    t_fused, t_copy, t_attn = ov["t_fused_us"], ov["t_copy_us"], ov["t_attn_us"]

    # Host-link ceiling: the copy kernel over every row of the pool.
    ev_h = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    all_pos = torch.arange(C, dtype=torch.int32, device=dev).repeat(B)
    all_n = torch.full((B,), C, dtype=torch.int32, device=dev)
    ev_h[0].record(stream)
    ess.ess_miss_copy(d, C, all_pos, all_pos, all_n, host.dev, lb.pool, stream)
    ev_h[1].record(stream)
    torch.cuda.synchronize()
    host_gbps = B * C * 1152 / (ev_h[0].elapsed_time(ev_h[1]) * 1e-3) / 1e9

    t_idx_cold, t_idx_warm, n_idx_copies = indexer_alone(d, lb, q_idx[burn + K - 1], n_vis, stream)

    # Algorithmic bytes / flops per launch.
    idx_bytes = B * L * wl.idx_dim + B * m * L * 4 + B * m * wl.idx_heads * (wl.idx_dim + 4)
    idx_flop = 2 * B * m * wl.idx_heads * wl.idx_dim * L
    sel_bytes = B * m * k * 1152
    attn_flop = 2 * B * m * H * k * (576 + 512)
    attn_bytes = sel_bytes + B * m * H * (576 * 2 + 512 * 4)
    miss_bytes = n_miss_tot * 1152 / K
    t_gather = float(stage_us[names.index("gather_attention")])
    # The attention's own HBM and MFMA rates: timed alone with every row in
    # the pool (the fused call is paced by the host link).
    t_attn_st = float(t_attn)
    attn_kernels = "sparse_mla_kernel+mla_combine_kernel"
    roofs = {
        # achieved: launches back to back, each reading its keys from HBM
        # (a different copy of the index cache each time); beside it the
        # same launches over one cache (last-level-cache resident) and the
        # event-timed stage inside the step (with its dispatch gap).
        "index_scores": {"kernel": "index_scores_kernel", "bound": "hbm",
                         "achieved": idx_bytes / t_idx_cold / 1e9,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "bytes_per_launch": idx_bytes,
                         "us_from_hbm": t_idx_cold * 1e6,
                         "index_cache_copies": n_idx_copies,
                         "same_cache_back_to_back_gbps": idx_bytes / t_idx_warm / 1e9,
                         "in_step_event_timed_gbps": idx_bytes / (stage_us[0] * 1e3)},
    }
    attn_view = {"attention_us": t_attn_st,
                 "hbm_gbps": attn_bytes / (t_attn_st * 1e3),
                 "hbm_bytes_per_launch": attn_bytes,
                 "hbm_frac": attn_bytes / (t_attn_st * 1e3) / HBM_PEAK_GBPS,
                 "tflops": attn_flop / (t_attn_st * 1e6),
                 "mfma_frac": attn_flop / (t_attn_st * 1e6) / BF16_PEAK_TFLOPS}
    # The host link sets the pace of the fused call: its misses cross it
    # while the attention's HBM reads and MFMA work run.
    roofs["gather_attention"] = {
        "kernel": attn_kernels, "bound": "host-link",
        "achieved": miss_bytes / (t_gather * 1e3), "peak": PCIE5_X16_GBPS,
        "unit": "GB/s", "bytes_per_launch": miss_bytes,
        "measured_ceiling": host_gbps, **attn_view}
    for r in roofs.values():
        r["frac"] = r["achieved"] / r["peak"]
    dom = int(np.argmax(stage_us))
    roof = dict(roofs.get(names[dom], {"kernel": names[dom], "bound": "alu",
                                        "achieved": None, "peak": None,
                                        "unit": "us", "frac": None}))
    parts = [recorded_traffic(kn, base.name) for kn in roof["kernel"].split("+")
             if kn in KERNEL_SOURCES]
    roof["traffic"] = (sum(parts) if parts and all(x is not None for x in parts)
                       and len(parts) == len(roof["kernel"].split("+")) else None)

    res = {
        "metric": "sparse decode steps/s & query-tok/s at 32K/128K; indexer HBM GB/s; miss-fetch GB/s",
        "value": B * m * K / wall_plain,
        "unit": "query-tok/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": wall_plain / K * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": base.name,
                   "batch": B, "mtp": m, "ctx_len": L, "idx_heads": wl.idx_heads,
                   "idx_dim": wl.idx_dim, "topk": k, "mla_heads": H,
                   "pool_slots": C, "rho": wl.rho,
                   "miss_mode": "in-kernel"},
        "steps_per_s": K / wall_plain,
        "burn_in_steps": burn,
        "misses_per_step_timed": float(miss_plain.mean()),
        "miss_rate_timed": float(miss_plain.mean()) / (B * m * k),
        "fill_us": t_fill * 1e6,
        "steps_per_s_incl_fill": base.steps / (t_fill + base.steps * wall_plain / K),
        "query_tok_s_incl_fill": B * m * base.steps / (t_fill + base.steps * wall_plain / K),
        "steps_per_s_staged": K / wall,
        "stage_us": {n: round(float(v), 2) for n, v in zip(names, stage_us)},
        "indexer_gbps": idx_bytes / t_idx_cold / 1e9,
        "indexer_gbps_in_step": idx_bytes / (stage_us[0] * 1e-6) / 1e9,
        "attention_tflops": attn_view["tflops"],
        "misses_per_step": n_miss_tot / K,
        "miss_rate": n_miss_tot / (K * B * m * k),
        "miss_fetch_gbps": miss_bytes / (t_gather * 1e3),
        "gather_us": t_gather,
        "host_link_gbps_measured": host_gbps,
        "overlap": ov,
        "roofline": roof,
        "rooflines": roofs,
    }
    host.free()
    del lb, q_idx, q_abs
    torch.cuda.empty_cache()
    if not args.no_extra:
        # The prefill pipeline first: after the 16-layer configuration has
        # pinned and released 38.7 GB of host memory its host-to-device
        # loads ran slower and unevenly (14-28 ms against 11-23 ms alone).
        res["extra"] = {}
        res["extra"]["prefill_pipeline"] = prefill_pipeline(args)
        res["configs"] = config_measurements(args)
        res["extra"]["eviction_replay"] = replay_curves(args)
        res["extra"]["fp8_entries"] = fp8_entries(args)
        res["extra"]["growing_context"] = growing_context(args)
    if args.cpu_seconds > 0:
        log(args, "timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(base, args.cpu_seconds)
        res["cpu_baseline"]["machine"] = host_machine()
        if not args.no_extra:
            # Every other workload, a shorter sample each; the 16-layer one
            # on its first and last requests over all its layers.
            short = max(1.0, args.cpu_seconds / 4)
            per = {}
            for name in ("tiny-4k", "128k-b8-mtp2-r099", "128k-b8-mtp2-r095",
                         "128k-b8-mtp2-r080", "1m-b1-c8k", "1m-b1-c16k"):
                per[name] = cpu_baseline(get_workload(name), short)
            w16 = get_workload("64k-b32-16layer")
            per[w16.name] = cpu_baseline(w16, short, requests=[0, w16.batch - 1],
                                         layers=w16.layers)
            res["cpu_baselines"] = per
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

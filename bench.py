"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (moe_layer_forward: routing, grouping,
the owned experts' FFN and the combine, with the results of the four calls
moe_route, moe_group_tokens, moe_expert_forward, moe_combine) over one batch of
synthetic input that is already resident in device memory.

The headline workload is single-token decode (T=1, H=4096, 256 experts,
I=2048, top-8, 2-bit gate/up/down, Q8_0 router, fp32 activations).  Every step
routes a different token from a pool of distinct tokens, so successive steps
touch different experts and the 76.6 MB a step reads mostly misses the 256 MB
last-level cache, as real decode does.  The same JSON line also carries the
other workloads (batched decode, prefill on bf16 matrix cores, one expert-
parallel share) measured the same way, under "workloads".

Kernel times come from HIP events that the library records around every
eighth launch of the named kernel during the timed region (on the stream the
kernel runs on).  The timed region is also cut into ten chunks, whose per-step
times give p10 / median / p90.  For the decode-like workloads two more numbers
are taken, each labelled: cold (a 512 MB buffer written between steps, outside
the timed steps, so nothing of the step's weights survives in the 256 MB last-
level cache) and warm (the same batch every step, its experts' weights served
from that cache).  Fractions are given against the published peaks and against
a measured device copy.
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores

WORKLOADS = {
    "decode": 2,
    "batched_decode": 3,
    "prefill": 4,
    "ep_share": 5,
    "table_batched": 3,
    "decode_shared": 2,
}
TABLE_V = 8192   # rows of the synthetic token-id routing table


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_layer(cfg_id, share=None):
    """Device layer for a workload (the owned share's stack when share is given)."""
    import synth
    import quantized_moe_routed_amd as moe
    from quantized_moe_routed_amd.layer import MoELayer
    wl = synth.make(cfg_id, T=1)
    fm = (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)
    g2l = None
    gate, up, down = wl.gate, wl.up, wl.down
    if share is not None:
        owner = moe.place_lpt(wl.load_hist, 2)
        g2l, l2g = moe.share_tables(owner, share)
        gate, up, down = gate[l2g], up[l2g], down[l2g]
    layer = MoELayer(wl.H, wl.I, wl.E, wl.k, wl.cfg.router_fmt, wl.router[0], wl.bias, fm, gate, up, down,
                     g2l=g2l)
    return wl, layer


def input_pool(wl, n_batches, torch):
    """n_batches distinct device batches of the workload's T tokens."""
    import synth
    T = wl.cfg.T
    toks = synth.tokens(0, T * n_batches, wl.H)
    if wl.cfg.act == "bf16":
        bits = synth.f32_to_bf16_bits(toks)
        xs = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xs = torch.from_numpy(toks).cuda()
    return [xs[i * T:(i + 1) * T] for i in range(n_batches)], toks


TRACE_EVERY = 8  # the kernel events of the timed region sample one launch in this many
N_CHUNKS = 10    # the timed region in this many chunks, for percentiles of the step time


def time_layer(layer, xs, steps, warmup, kernel, torch, run=None, route=None):
    """Run warmup + steps layer calls cycling through xs; returns the step time
    (ms), the average duration of `kernel` (ms), and per batch the mean number
    of owned experts and of slots on small tiles and on large tiles.  run(i, b) and route(i, b)
    replace the layer call and the routing of batch i (table routing)."""
    import quantized_moe_routed_amd as moe
    from quantized_moe_routed_amd.layer import act_code
    b = layer.buffers(xs[0].shape[0], act_code(xs[0]))
    run = run or (lambda i, b: layer.run(xs[i], b))
    route = route or (lambda i, b: layer.route(xs[i], b))
    for i in range(warmup):
        run(i % len(xs), b)
    torch.cuda.synchronize()
    # events around every TRACE_EVERY-th launch of the kernel only: each pair of events costs the
    # stream a few microseconds, which would otherwise be charged to every step
    trace = moe.KernelTrace(kernel, (steps + TRACE_EVERY - 1) // TRACE_EVERY, TRACE_EVERY)
    n_chunks = min(N_CHUNKS, steps)
    bounds = [round(steps * c / n_chunks) for c in range(n_chunks + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    torch.cuda.synchronize()
    with trace:
        evs[0].record()
        for c in range(n_chunks):
            for i in range(bounds[c], bounds[c + 1]):
                run((warmup + i) % len(xs), b)
            evs[c + 1].record()
    torch.cuda.synchronize()
    ms_step = evs[0].elapsed_time(evs[-1]) / steps
    chunk_ms = [evs[c].elapsed_time(evs[c + 1]) / (bounds[c + 1] - bounds[c]) for c in range(n_chunks)]
    kms = trace.times_ms()
    # per-step loads, outside the timed region: replay the routing of each batch and count the
    # owned experts and slots on each kind of tile
    T = xs[0].shape[0]
    large_min = moe.large_tile_min(T) or 1 << 30   # experts of this many slots or more run on large tiles
    owned = None if layer.g2l is None else (layer.g2l >= 0).cpu().numpy()
    d_small, s_small, d_large, s_large = [], [], [], []
    for i in range(min(steps, len(xs))):
        route((warmup + i) % len(xs), b)
        layer.group(b)
        c = b.counts.cpu().numpy()
        if owned is not None:
            c = c * owned
        small = (c > 0) & (c < large_min)
        d_small.append(int(small.sum()))
        s_small.append(int(c[small].sum()))
        d_large.append(int((c >= large_min).sum()))
        s_large.append(int(c[c >= large_min].sum()))
    torch.cuda.synchronize()
    pct = {f"ms_{q}": float(np.percentile(chunk_ms, v)) for q, v in (("p10", 10), ("median", 50), ("p90", 90))}
    return (ms_step, float(np.mean(kms)), float(np.mean(d_small)), float(np.mean(s_small)), float(np.mean(d_large)),
            float(np.mean(s_large)), pct)


FLUSH_BYTES = 512 << 20   # written between cold steps: twice the last-level cache


def time_cold_warm(layer, xs, reps, torch, run=None):
    """Per-step times (median ms) of single steps: cold, with FLUSH_BYTES written to a scratch
    buffer before each step (outside its events), and warm, the same batch repeated."""
    from quantized_moe_routed_amd.layer import act_code
    b = layer.buffers(xs[0].shape[0], act_code(xs[0]))
    run = run or (lambda i, b: layer.run(xs[i], b))
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for r in range(reps):
        flush.fill_(r & 0xFF)
        evs[r][0].record()
        run(r % len(xs), b)
        evs[r][1].record()
    torch.cuda.synchronize()
    cold = float(np.median([s.elapsed_time(e) for s, e in evs]))
    for _ in range(5):
        run(0, b)
    for r in range(reps):
        evs[r][0].record()
        run(0, b)
        evs[r][1].record()
    torch.cuda.synchronize()
    warm = float(np.median([s.elapsed_time(e) for s, e in evs]))
    del flush
    return cold, warm


def copy_ceiling_gbs(torch, nbytes=1 << 30, reps=10):
    """Measured device copy rate (bytes read + written per second, GB/s) over nbytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (s.elapsed_time(e) * 1e-3) / 1e9
    del src, dst
    return gbs


def traffic_record(kernel):
    """HBM bytes per launch of `kernel` measured with hardware counters (profiles/), or None when
    the kernel's source has changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return rec if h.hexdigest() == rec["sources_sha256"] else None


def measure(name, steps, warmup, torch, copy_gbs=None):
    cfg_id = WORKLOADS[name]
    share = 0 if name == "ep_share" else None
    log(f"{name}: generating weights and inputs")
    wl, layer = build_layer(cfg_id, share)
    T, H, I, k = wl.cfg.T, wl.H, wl.I, wl.k
    n_batches = 1 if name == "prefill" else max(1, 1024 // T)
    xs, _ = input_pool(wl, n_batches, torch)
    per_expert = layer.expert_bytes() // layer.E_local
    gateup_per_expert = (layer.gate.nbytes() + layer.up.nbytes()) // layer.E_local
    bf16 = wl.cfg.act == "bf16"
    kernel = "ffn_gateup_large" if name == "prefill" else "ffn_gateup"
    run = route = None
    if name == "decode_shared":
        # the routed layer, then a Q8_0 shared expert of the routed experts' shapes added to its
        # output (two gate/up launches a step: the sampled launches 0, 8, 16, ... are the routed ones)
        import synth
        from quantized_moe_routed_amd.layer import SharedExpert
        shared = SharedExpert(H, I, 1, *synth.shared_expert(0, H, I))
        run = lambda i, b: (layer.run(xs[i], b), shared.add_to(xs[i], b.out))
    if name == "table_batched":
        # table routing: each batch's token ids index a seeded [TABLE_V, k] table of distinct experts
        import synth
        table = torch.from_numpy(synth.route_table(0, TABLE_V, wl.E, k)).cuda()
        tok = torch.from_numpy(synth.token_ids(0, T * len(xs), TABLE_V)).cuda()
        tids = [tok[i * T:(i + 1) * T] for i in range(len(xs))]
        run = lambda i, b: layer.run_table(xs[i], b, tids[i], table)
        route = lambda i, b: layer.route_table(xs[i], b, tids[i], table)
    log(f"{name}: timing {steps} steps")
    ms, kms, d_small, s_small, d_large, s_large, pct = time_layer(layer, xs, steps, warmup, kernel, torch, run, route)
    slots = s_small + s_large
    router_bytes = layer.router.nbytes()
    x_bytes = T * H * (2 if bf16 else 4)
    flops = 6.0 * H * I * slots
    # whole-layer bytes: every touched owned expert's weights, the router, x in and the output
    layer_bytes = (d_small + d_large) * per_expert + router_bytes + x_bytes + T * H * 4
    if name == "decode_shared":
        layer_bytes += shared.nbytes()
    res = {
        "tokens_per_s": T / (ms * 1e-3),
        "ms_per_step": ms,
        **pct,
        "T": T,
        "owned_slots": slots,
        "distinct_experts": d_small + d_large,
        "small_tile_experts": d_small,
        "small_tile_slots": s_small,
        "large_tile_slots": s_large,
        "layer_bytes": layer_bytes,
        "layer_gbs": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_tflops": flops / (ms * 1e-3) / 1e12,
        "mfma_frac_of_bf16_peak": (flops / (ms * 1e-3) / 1e12) / BF16_PEAK_TFLOPS if bf16 else None,
    }
    # the whole layer against its binding roofline (HBM, or the matrix cores for prefill)
    if name == "prefill":
        res["layer_roofline"] = {"bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                 "algorithmic_flops_per_step": flops}
    else:
        res["layer_roofline"] = {"bound": "hbm", "achieved": res["layer_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": res["layer_gbs"] / HBM_PEAK_GBS, "algorithmic_bytes_per_step": layer_bytes}
        if copy_gbs:
            res["layer_roofline"]["copy_ceiling_gbs"] = copy_gbs
            res["layer_roofline"]["frac_of_copy_ceiling"] = res["layer_gbs"] / copy_gbs
    if name in ("decode", "batched_decode", "ep_share"):
        log(f"{name}: cold and warm single steps")
        cold, warm = time_cold_warm(layer, xs, 30, torch, run)
        res["cold"] = {"ms_per_step": cold, "layer_gbs": layer_bytes / (cold * 1e-3) / 1e9,
                       "note": f"{FLUSH_BYTES >> 20} MB written before each step, outside its events"}
        res["warm"] = {"ms_per_step": warm, "layer_gbs": layer_bytes / (warm * 1e-3) / 1e9,
                       "note": "the same batch every step: its experts' weights come from the last-level cache"}
    if name == "prefill":
        # large-tile gate/up: 2 matrices x 2 flops x H x I per slot on large tiles
        kflops = 4.0 * H * I * s_large
        rec = traffic_record(kernel + ":" + name)
        res["roofline"] = {"bound": "mfma", "achieved": kflops / (kms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": kflops / (kms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                           "traffic": rec["bytes_per_launch"] if rec else None, "algorithmic_flops_per_launch": kflops}
    else:
        # small-tile gate/up, algorithmic bytes as for the layer: the gate/up weights of the experts
        # on small tiles and the activations x; the implementation's own traffic (the prepared
        # operand read per slot, hi + lo, and h written per slot, hi + lo) is reported beside it
        kbytes = d_small * gateup_per_expert + x_bytes
        impl = s_small * (H * 4 + I * 4)
        rec = traffic_record(kernel + ":" + name)
        res["roofline"] = {"bound": "hbm", "achieved": kbytes / (kms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": kbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "traffic": rec["bytes_per_launch"] if rec else None,
                           "algorithmic_bytes_per_launch": kbytes, "implementation_bytes_per_launch": impl}
    res["roofline"]["kernel"] = kernel
    res["roofline"]["avg_launch_ms"] = kms
    return wl, res


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(budget_s=15.0, single_budget_s=8.0, max_tokens=1600):
    """The CPU oracle, as it stands, on a bounded sample of the decode workload: on every thread its
    OpenMP runtime uses, then on one thread."""
    import ctypes
    import oracle
    import synth
    wl = synth.make(2, T=1)
    fm = (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)
    pool = synth.tokens(0, max_tokens, wl.H)

    def run(budget, limit):
        done = 0
        t0 = time.perf_counter()
        while done < limit and time.perf_counter() - t0 < budget:
            xs = pool[done:done + 8]
            oracle.layer(xs, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k, fm, wl.gate, wl.up, wl.down)
            done += len(xs)
        return done, time.perf_counter() - t0

    gomp = ctypes.CDLL("libgomp.so.1")   # the oracle's OpenMP runtime (already loaded with it)
    threads = int(gomp.omp_get_max_threads())
    done, dt = run(budget_s, max_tokens)
    gomp.omp_set_num_threads(1)
    try:
        done1, dt1 = run(single_budget_s, max_tokens)
    finally:
        gomp.omp_set_num_threads(threads)
    return {"value": done / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"{done} single-token decode layer evaluations (route + 8 experts + combine, fp64 FFN) "
                      f"in {dt:.1f} s on {threads} OpenMP threads",
            "single_thread": {"value": done1 / dt1, "unit": "tokens/s",
                              "sample": f"{done1} evaluations in {dt1:.1f} s on one thread"}}


# Kernels whose HBM traffic is recorded from hardware counters, by workload, with the sources that
# define them (the record is ignored once any of them changes).
_FFN_SOURCES = ["quantized_moe_routed_amd/csrc/ffn.hip", "quantized_moe_routed_amd/csrc/ffn.h",
                "quantized_moe_routed_amd/csrc/fmt.h", "quantized_moe_routed_amd/csrc/device.h",
                "quantized_moe_routed_amd/csrc/smallsel.h", "quantized_moe_routed_amd/csrc/select.h",
                "quantized_moe_routed_amd/csrc/launch.h"]
TRAFFIC_KERNELS = {
    "decode": ("ffn_gateup", "moe::ffn_small_kernel<2, 2, true, 0, true, true, false, false>", _FFN_SOURCES),
    "batched_decode": ("ffn_gateup", "moe::ffn_small_kernel<2, 2, true, 0, false, false, false, true>", _FFN_SOURCES),
    "ep_share": ("ffn_gateup", "moe::ffn_small_kernel<2, 2, true, 0, false, false, false, true>", _FFN_SOURCES),
    "prefill": ("ffn_gateup_large", "moe::ffn_large_kernel<2, 2, false, 0, 1, 2, 4>",
                ["quantized_moe_routed_amd/csrc/ffn_large.hip", "quantized_moe_routed_amd/csrc/ffn.h",
                 "quantized_moe_routed_amd/csrc/fmt.h", "quantized_moe_routed_amd/csrc/device.h",
                 "quantized_moe_routed_amd/csrc/launch.h"]),
}
COPY_BYTES = 256 << 20   # the calibration copy: reads and writes this many bytes


def calibration_copy(torch):
    """A plain device copy of known size, for scaling the memory counters."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def record_traffic(workload, fetch_dir, write_dir):
    """profiles/traffic.json entry for the workload's kernel, from a FETCH_SIZE run and a WRITE_SIZE
    run of rocprofv3 (counter_collection.csv under the given directories).  Each counter is scaled
    by what it reads for the calibration copy of COPY_BYTES."""
    import csv
    import glob
    import hashlib
    key, kname, sources = TRAFFIC_KERNELS[workload]

    def per_launch(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        vals = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        mine = [v for k, v in vals.items() if k.startswith("void " + kname) or k.startswith(kname)]
        copy = [v for k, v in vals.items() if "copy" in k.lower()]
        assert mine and copy, (counter, list(vals)[:8])
        copy_v = max(max(v) for v in copy)   # the calibration copy (the other copies are small)
        return float(np.mean(mine[0])), float(copy_v)

    fk, fc = per_launch(fetch_dir, "FETCH_SIZE")
    wk, wc = per_launch(write_dir, "WRITE_SIZE")
    fetch_bytes = fk * COPY_BYTES / fc
    write_bytes = wk * COPY_BYTES / wc
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec[key + ":" + workload] = {
        "kernel": kname, "bytes_per_launch": fetch_bytes + write_bytes, "fetch_bytes": fetch_bytes,
        "write_bytes": write_bytes, "fetch_counter_per_launch": fk, "write_counter_per_launch": wk,
        "copy_fetch_counter": fc, "copy_write_counter": wc, "copy_bytes": COPY_BYTES,
        "sources": sources, "sources_sha256": h.hexdigest()}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec[key + ":" + workload]))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode",
                    help="workload of the headline value (default: single-token decode)")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain copy of known size (for scaling memory counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs (no GPU work)")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer's expert-parallel "
              "path is designed, not built, for more than one GPU)", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    copy_gbs = None
    if args.calibration_copy:
        # (a counter run: the only large copy is the calibration one, which scales the counters)
        calibration_copy(torch)
    else:
        copy_gbs = copy_ceiling_gbs(torch)
        log(f"device copy: {copy_gbs:.0f} GB/s (read + write)")
    wl, head = measure(args.workload, args.steps, args.warmup, torch, copy_gbs)
    others = {}
    if not args.only:
        for name in ("batched_decode", "prefill", "ep_share", "table_batched", "decode_shared", "decode"):
            if name == args.workload:
                continue
            steps = {"prefill": 20, "batched_decode": 100, "ep_share": 50, "table_batched": 100, "decode_shared": 200,
                     "decode": 200}[name]
            _, r = measure(name, steps, 5, torch, copy_gbs)
            others[name] = r
    T = head["T"]
    cfg = wl.cfg
    desc = {
        "decode": "single-token decode: T=1, H=4096, E=256 routed experts, I=2048, top-8, Q2SM (2-bit) "
                  "gate/up/down, Q8_0 router, fp32 activations, distinct tokens cycled",
        "batched_decode": "batched decode: T=32, H=4096, E=256, I=2048, top-8, Q2SM gate/up, Q8_0 down, "
                          "router bias N(0,0.5), fp32 activations",
        "prefill": "prefill: T=2048, H=4096, E=256, I=2048, top-8, Q2SM gate/up, Q8_0 down, Zipf(1.1) router "
                   "bias, bf16 activations on matrix cores",
        "ep_share": "expert-parallel share: T=128, 128 of 256 experts owned (LPT), H=4096, I=2048, top-8, "
                    "Q2SM gate/up, Q8_0 down, fp32 activations; partial output",
        "decode_shared": "single-token decode plus a Q8_0 shared expert (I=2048) added to the routed output",
        "table_batched": "batched decode with table routing: T=32, experts from a seeded 8192-row token-id table "
                         "of 8 distinct experts, shapes and formats of batched decode",
    }[args.workload]
    result = {
        "metric": "MoE layer tokens/s at 1 MI355X; decode HBM GB/s and prefill MFMA % of peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": desc, "global_batch": T, "parallelism": "none (1 GPU)"},
        "ms_p10": head["ms_p10"],
        "ms_median": head["ms_median"],
        "ms_p90": head["ms_p90"],
        "layer_gbs": head["layer_gbs"],
        "layer_bytes_per_step": head["layer_bytes"],
        "distinct_experts_per_step": head["distinct_experts"],
        "roofline": head["roofline"],
        "layer_roofline": head["layer_roofline"],
        "measured_copy_gbs": copy_gbs,
    }
    for key in ("cold", "warm"):
        if key in head:
            result[key] = head[key]
    if head["mfma_frac_of_bf16_peak"] is not None:
        result["mfma_frac_of_bf16_peak"] = head["mfma_frac_of_bf16_peak"]
    if others:
        result["workloads"] = others
    if not args.no_cpu_baseline and args.workload == "decode":
        log("cpu baseline (oracle on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

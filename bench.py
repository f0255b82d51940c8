"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (moe_route, moe_group_tokens,
moe_expert_forward, moe_combine) over one batch of synthetic input that is
already resident in device memory.  The default workload is single-token
decode (T=1, H=4096, 256 experts, I=2048, top-8, 2-bit gate/up/down, Q8_0
router, fp32 activations): every step routes a different token from a pool of
distinct tokens, so successive steps touch different experts and the 76.6 MB
each step reads mostly misses the 256 MB last-level cache, as real decode does.

Prints one JSON line.  The dominant kernel's time comes from HIP events the
library records around each of its launches during the timed region.
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

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(wl, layer_bytes_per_expert, D, T):
    """Bytes the layer must move once: the distinct touched experts' weights, the
    router, the activations in and the output out."""
    router = wl.router[0].nbytes if wl.cfg.router_fmt != 0 else wl.E * wl.H * 4
    x_bytes = T * wl.H * (2 if wl.cfg.act == "bf16" else 4)
    return D * layer_bytes_per_expert + router + x_bytes + T * wl.H * 4


def cpu_baseline(wl_cfg, pool_tokens, budget_s=15.0, max_tokens=400):
    """The CPU oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    import synth
    wl = synth.make(wl_cfg, T=1)
    fm = (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)
    done = 0
    t0 = time.perf_counter()
    while done < max_tokens and time.perf_counter() - t0 < budget_s:
        n = 8
        xs = pool_tokens[done:done + n]
        oracle.layer(xs, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k, fm, wl.gate, wl.up, wl.down)
        done += len(xs)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": done / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} single-token decode layer evaluations (route + 8 experts + combine, fp64 FFN) "
                      f"in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pool", type=int, default=1024, help="distinct tokens cycled through (decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer's expert-parallel "
              "path is designed, not built, for more than one GPU)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import quantized_moe_routed_amd as moe
    from quantized_moe_routed_amd.layer import MoELayer

    assert torch.cuda.is_available()
    cfg_id = 2
    log("generating decode workload (256 experts, 2-bit)")
    wl = synth.make(cfg_id, T=1)
    fm = (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)
    layer = MoELayer(wl.H, wl.I, wl.E, wl.k, wl.cfg.router_fmt, wl.router[0], wl.bias, fm, wl.gate, wl.up,
                     wl.down)
    bytes_per_expert = layer.expert_bytes() // wl.E
    gateup_bytes_per_expert = (layer.gate.nbytes() + layer.up.nbytes()) // wl.E
    pool = synth.tokens(0, args.pool, wl.H)
    x_pool = torch.from_numpy(pool).cuda()
    xs = [x_pool[i:i + 1] for i in range(args.pool)]
    b = layer.buffers(1, moe.ACT_F32)
    log("warmup")
    for i in range(args.warmup):
        layer.run(xs[i % args.pool], b)
    torch.cuda.synchronize()

    K = args.steps
    dom = "gemv_gateup"
    trace = moe.KernelTrace(dom, K)
    distinct = []
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"timing {K} steps")
    with trace:
        start.record()
        for i in range(K):
            layer.run(xs[(args.warmup + i) % args.pool], b)
        end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / K
    dom_ms = trace.times_ms()
    dom_avg_ms = float(np.mean(dom_ms))
    D = int(np.count_nonzero(b.counts.cpu().numpy()))
    distinct.append(D)

    T = 1
    layer_bytes = algorithmic_bytes(wl, bytes_per_expert, D, T)
    # gate/up kernel: gate + up weights of the touched experts, x read once per slot, h written
    dom_bytes = D * gateup_bytes_per_expert + T * wl.k * wl.H * 4 + T * wl.k * wl.I * 4
    dom_gbs = dom_bytes / (dom_avg_ms * 1e-3) / 1e9
    result = {
        "metric": "MoE layer tokens/s at 1 MI355X; decode HBM GB/s and prefill MFMA % of peak",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "single-token decode: T=1, H=4096, E=256 routed experts, I=2048, top-8, "
                               "Q2SM (2-bit) gate/up/down, Q8_0 router, fp32 activations, "
                               f"{args.pool} distinct tokens cycled",
                   "global_batch": T, "parallelism": "none (1 GPU)"},
        "layer_gbs": layer_bytes / (ms_step * 1e-3) / 1e9,
        "layer_bytes_per_step": layer_bytes,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dom_gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": dom_avg_ms},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline(cfg_id, pool)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

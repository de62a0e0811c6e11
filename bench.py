"""Benchmark of the routed-expert MoE decode layer on one MI355X.

One step = one moe_decode_forward call over one batch of M tokens (router GEMV, softmax top-k,
dispatch compaction, gate/up SwiGLU, down projection, weighted combine with the shared expert),
with all inputs already resident in HBM.  The timed steps are replayed from a hipGraph and rotate
over L complete copies of the layer's weights (same values, distinct addresses) so that each
step's expert weights come from HBM, not from the 256 MB Infinity Cache ("Chasing the Batch-1
Floor", section "Fixing the ruler before fixing the machine": a looped kernel keeps its weights
cache-resident and runs optimistically).

Prints one JSON line.  Roofline: algorithmic bytes per step (router + each unique expert once +
shared expert + activations in/out + routing outputs) over the measured time, against 8 TB/s.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer µs/step + achieved HBM GB/s (% of peak), Ling shapes, M=1/6/16"
PEAK_HBM_GBPS = 8000.0
KERNEL_SOURCES = ["moe_speculative_decode_amd/csrc/moe_layer.hip", "moe_speculative_decode_amd/csrc/moe_internal.h"]


def algorithmic_bytes(cfg, U: int) -> int:
    """Bytes the layer must move once: router weight, each unique routed expert once, the shared
    expert, x in, y out, top-k ids and weights out."""
    from moe_speculative_decode_amd import synth
    H, E, k, I, Is, M = cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter, cfg.shared_inter, cfg.M
    ab = 4 if cfg.act_fmt == synth.F32 else 2

    def mat(rows, cols):
        if cfg.weight_fmt == synth.MXFP4:
            return rows * cols // 2 + rows * cols // 32
        return rows * cols * (4 if cfg.weight_fmt == synth.F32 else 2)

    expert = 2 * mat(I, H) + mat(H, I)
    shared = (2 * mat(Is, H) + mat(H, Is)) if Is else 0
    return E * H * ab + U * expert + shared + 2 * M * H * ab + 8 * M * k


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per step from the committed counter summary, if it was taken on the current
    kernels; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("bytes_per_step")


def cpu_baseline(cfg, layer, x, budget_s: float):
    """The fp64 oracle on the host cores, on a bounded sample: whole steps of the same workload
    repeated until about budget_s seconds have passed."""
    from oracle import oracle as O
    O.build(force=False)
    d = O.layer_desc(cfg)
    W = O.layer_weights(layer)
    threads = len(os.sched_getaffinity(0))
    used = min(threads, cfg.M)  # the oracle parallelises over tokens
    t0 = time.perf_counter()
    n = 0
    while True:
        O.forward(d, W, x, layer.router, threads=used)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    return {"value": dt * 1e6, "unit": "us/step", "cores": used, "kind": "oracle",
            "sample": "%d whole steps of the same workload (M=%d), fp64 C loops, OpenMP over tokens" % (n, cfg.M)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="ling_bf16_m1")
    ap.add_argument("--copies", type=int, default=0, help="layer copies rotated (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true", help="run a plain 1 GiB device copy (counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer has no multi-GPU path (one GPU's share is "
              "the whole layer here)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_speculative_decode_amd as mdl
    from moe_speculative_decode_amd import device as dev
    from moe_speculative_decode_amd import synth

    torch.cuda.set_device(0)
    if args.calib_copy:
        n = 1 << 30
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "dispatches": 5}))
        return

    cfg = synth.CONFIGS[args.config]
    M = cfg.M
    t0 = time.time()
    layer = synth.Layer(cfg)
    seed = synth.accepted_hidden_seed(cfg.name)
    x_host = synth.make_hidden(cfg, seed)
    print("[bench] layer generated in %.1fs" % (time.time() - t0), file=sys.stderr, flush=True)
    base = dev.DeviceLayer(layer)
    x = dev.to_device(x_host)
    desc = dev.desc_of(cfg)
    ws = dev.workspace(desc)
    y = torch.empty((M, cfg.hidden), dtype=dev.act_dtype(cfg), device="cuda")
    ids = torch.empty((M, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, cfg.top_k), dtype=torch.float32, device="cuda")
    disp = dev.DispatchOut(M, cfg.top_k, cfg.num_experts)

    # U of this workload, from the layer itself
    mdl.moe_decode_forward(desc, M, x, base.router, base.weights(), y, ws, topk_ids=ids, topk_w=w,
                           disp=disp.struct())
    torch.cuda.synchronize()
    U = int(disp.unit_count.item())
    B = algorithmic_bytes(cfg, U)
    L = args.copies or max(1, -(-(1 << 30) // B))
    copies = [base] + [base.clone() for _ in range(L - 1)]
    weights = [c.weights() for c in copies]
    routers = [c.router for c in copies]
    torch.cuda.synchronize()
    print("[bench] %s U=%d B_alg=%d L=%d copies (%.1f GB)" % (cfg.name, U, B, L, L * base.nbytes() / 1e9),
          file=sys.stderr, flush=True)

    K, W = args.steps, args.warmup

    def step(i, stream):
        j = i % L
        mdl.moe_decode_forward(desc, M, x, routers[j], weights[j], y, ws, topk_ids=ids, topk_w=w, stream=stream)

    s = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    # warmup: W eager steps
    for i in range(W):
        step(i, cur)
    torch.cuda.synchronize()
    # capture exactly K steps (rotating copies) in one graph
    s.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(K):
                step(i, s)
    cur.wait_stream(s)
    g.replay()  # graph upload; untimed
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(cur)
    g.replay()
    ev1.record(cur)
    torch.cuda.synchronize()
    t_step_us = ev0.elapsed_time(ev1) * 1e3 / K

    # eager stream launches, events around every step on the launch stream (not graded)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        starts[i].record(cur)
        step(i, cur)
        ends[i].record(cur)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends))
    eager_med_us = per[len(per) // 2]

    achieved = B / (t_step_us * 1e-6) / 1e9
    traffic = traffic_from_profiles(cfg.name)
    out = {
        "metric": METRIC, "value": round(t_step_us, 3), "unit": "us/step", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(t_step_us / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": synth.FORMAT_NAMES[cfg.weight_fmt], "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "hidden": cfg.hidden, "experts": cfg.num_experts,
                   "top_k": cfg.top_k, "inter": cfg.inter, "shared_inter": cfg.shared_inter,
                   "weights": synth.FORMAT_NAMES[cfg.weight_fmt], "unique_experts": U,
                   "algorithmic_bytes": B, "cold_copies": L, "timing": "hipGraph of K steps, rotating copies"},
        "tokens_per_s": round(M / (t_step_us * 1e-6), 1),
        "hbm_GBps": round(achieved, 1), "hbm_frac": round(achieved / PEAK_HBM_GBPS, 4),
        "eager_median_us": round(eager_med_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, layer, np.ascontiguousarray(x_host), args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the routed-expert MoE decode layer on one MI355X.

One step = one moe_decode_forward call over one batch of M tokens (router GEMV, softmax top-k,
dispatch compaction, gate/up SwiGLU, down projection, weighted combine with the shared expert),
with all inputs already resident in HBM.

Timing ("Chasing the Batch-1 Floor", section "Fixing the ruler before fixing the machine": a
looped kernel keeps its weights cache-resident and runs optimistically; time the cold case, and
keep the counter pass separate from the timing):
  * cold: K steps captured in one hipGraph rotate over L complete copies of the layer's weights
    (same values, distinct addresses; L * bytes >= 1 GiB, four times the 256 MB Infinity Cache),
    so every step's weights come from HBM.  The graph is replayed `trials` (>= 10) times; each
    replay is one sample of us/step; the median, p10 and p90 are reported.
  * hot: the same with L = 1 (the weights stay in the caches between steps); not graded.
  * eager: stream launches with events around each step; not graded.
  * stream ceiling: a plain streaming read of the same number of bytes, cold and graph-replayed
    the same way: what one launch can read from HBM in that time on this GPU.

Prints ONE JSON line.  The headline is the first workload (bf16, one token).  `workloads` holds
every Ling configuration (bf16, MXFP4 and FP8 weights at M = 1, 6, 16) with its unique-expert count
U, algorithmic bytes B_alg (router + each unique routed expert once + the shared expert + x in,
y out + routing outputs), the roofline fraction B_alg / t / 8 TB/s and the HBM traffic the
committed counter pass measured on the current kernel (null otherwise), and the LM head GEMV
(157,184 x 2,560, bf16 and FP8 weights, M = 1 and 6) measured the same way.  The CPU baseline is
the fp64 oracle on the host's cores.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer µs/step + achieved HBM GB/s (% of peak), Ling shapes, M=1/6/16"
PEAK_HBM_GBPS = 8000.0
# the sources of each kernel: counter summaries taken on other sources are stale
KERNEL_SOURCES = {"k_layer": ["moe_speculative_decode_amd/csrc/moe_layer.hip",
                              "moe_speculative_decode_amd/csrc/moe_internal.h"],
                  "k_lm_head": ["moe_speculative_decode_amd/csrc/lm_head.hip"]}
HEADLINE = "ling_bf16_m1"
WORKLOADS = ["ling_bf16_m1", "ling_bf16_m6", "ling_bf16_m16_ragged", "ling_mxfp4_m1", "ling_mxfp4_m6",
             "ling_mxfp4_m16_ragged", "ling_fp8_m1", "ling_fp8_m6", "ling_fp8_m16_ragged"]
COLD_BYTES = 1 << 30


def algorithmic_bytes(cfg, U: int) -> int:
    """Bytes the layer must move once: router weight, each unique routed expert once, the shared
    expert, x in, y out, top-k ids and weights out."""
    from moe_speculative_decode_amd import synth
    H, E, k, I, Is, M = cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter, cfg.shared_inter, cfg.M
    ab = 4 if cfg.act_fmt == synth.F32 else 2

    def mat(rows, cols):
        if cfg.weight_fmt == synth.MXFP4:
            return rows * cols // 2 + rows * cols // 32
        if cfg.weight_fmt == synth.FP8:  # one byte a code, 4 bytes a 128 x 128 block scale
            return rows * cols + 4 * (rows // synth.FP8_BLOCK) * (cols // synth.FP8_BLOCK)
        return rows * cols * (4 if cfg.weight_fmt == synth.F32 else 2)

    expert = 2 * mat(I, H) + mat(H, I)
    shared = (2 * mat(Is, H) + mat(H, Is)) if Is else 0
    return E * H * ab + U * expert + shared + 2 * M * H * ab + 8 * M * k


def kernel_of(workload: str) -> str:
    return "k_lm_head" if workload.startswith("lm_head") else "k_layer"


def kernel_hash(kernel: str = "k_layer") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per step from the committed counter summary, if it was taken on the current
    kernels; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_hash") != kernel_hash(kernel_of(workload)):
        return None
    return d.get("bytes_per_step")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, layer, x, budget_s: float):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample: whole steps of the
    same workload repeated for about budget_s seconds, once on one thread and once on every core
    this process may use (OpenMP over (token, expert) pairs)."""
    from oracle import oracle as O
    O.build(force=False)
    d = O.layer_desc(cfg)
    W = O.layer_weights(layer)
    avail = len(os.sched_getaffinity(0))
    # the oracle has M * (k + 1) independent expert outputs per step: more threads than that idle
    used_all = min(avail, cfg.M * (cfg.top_k + 1))

    def timed(threads):
        t0 = time.perf_counter()
        n = 0
        while True:
            O.forward(d, W, x, layer.router, threads=threads, **O.router_aux(layer))
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return (time.perf_counter() - t0) / n * 1e6, n

    one_us, n1 = timed(1)
    all_us, na = timed(used_all)
    return {"value": round(all_us, 1), "unit": "us/step", "cores": used_all, "kind": "oracle",
            "sample": "%d whole steps of %s (M=%d) on %d threads, %d steps on 1 thread; fp64 C loops, no BLAS"
                      % (na, cfg.name, cfg.M, used_all, n1),
            "value_1thread": round(one_us, 1), "affinity_cores": avail, "cpu_model": cpu_model()}


def pct(vals, q):
    v = sorted(vals)
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


class StreamRef:
    """The streaming-read reference (libmoe_bench.so)."""

    def __init__(self):
        path = os.path.join(ROOT, "moe_speculative_decode_amd", "libmoe_bench.so")
        if not os.path.exists(path):
            raise ImportError("libmoe_bench.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        L.moe_bench_stream_read.restype = ctypes.c_int
        L.moe_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.moe_bench_stream_read_blocks.restype = ctypes.c_int
        self.L = L

    def launch(self, src_ptr, nbytes, sink_ptr, stream):
        st = self.L.moe_bench_stream_read(src_ptr, nbytes, sink_ptr, stream)
        if st != 0:
            raise RuntimeError("moe_bench_stream_read failed (%d)" % st)


def graph_times(torch, step, K: int, trials: int, warmup: int):
    """Captures K steps step(i, stream) into one hipGraph and replays it `trials` times.
    Returns the us/step of every replay (events on the launch stream)."""
    s = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    for i in range(warmup):
        step(i, cur)
    torch.cuda.synchronize()
    s.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(K):
                step(i, s)
    cur.wait_stream(s)
    for _ in range(3):  # upload and warm the graph; untimed
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(trials)]
    for a, b in ev:
        a.record(cur)
        g.replay()
        b.record(cur)
    torch.cuda.synchronize()
    out = [a.elapsed_time(b) * 1e3 / K for a, b in ev]
    del g
    return out


def summary(samples):
    return {"median": round(pct(samples, 0.5), 3), "p10": round(pct(samples, 0.1), 3),
            "p90": round(pct(samples, 0.9), 3), "n": len(samples)}


def measure_format(torch, mdl, dev, synth, names, args, stream_ref):
    """All workloads of one weight format share one layer (the same weights): its cold copies are
    allocated once, for the workload with the fewest bytes."""
    cfgs = [synth.CONFIGS[n] for n in names]
    t0 = time.time()
    layer = synth.Layer(cfgs[0])
    print("[bench] %s layer generated in %.1fs" % (synth.FORMAT_NAMES[cfgs[0].weight_fmt], time.time() - t0),
          file=sys.stderr, flush=True)
    base = dev.DeviceLayer(layer)
    prepared = []
    for cfg in cfgs:
        seed = synth.accepted_hidden_seed(cfg.name)
        x_host = synth.make_hidden(cfg, seed)
        x = dev.to_device(x_host)
        desc = dev.desc_of(cfg, layer=base)
        ws = dev.workspace(desc)
        M = cfg.M
        y = torch.empty((M, cfg.hidden), dtype=dev.act_dtype(cfg), device="cuda")
        ids = torch.empty((M, cfg.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((M, cfg.top_k), dtype=torch.float32, device="cuda")
        disp = dev.DispatchOut(M, cfg.top_k, cfg.num_experts)
        mdl.moe_decode_forward(desc, M, x, base.router, base.weights(), y, ws, topk_ids=ids, topk_w=w,
                               disp=disp.struct())
        torch.cuda.synchronize()
        U = int(disp.unit_count.item())
        prepared.append((cfg, x_host, x, desc, ws, y, ids, w, U, algorithmic_bytes(cfg, U)))
    L = args.copies or max(1, -(-COLD_BYTES // min(p[-1] for p in prepared)))
    copies = [base] + [base.clone() for _ in range(L - 1)]
    weights = [c.weights() for c in copies]
    routers = [c.router for c in copies]
    torch.cuda.synchronize()
    print("[bench] %d copies (%.1f GB)" % (L, L * base.nbytes() / 1e9), file=sys.stderr, flush=True)
    K, W, T = args.steps, args.warmup, args.trials
    results = []
    for cfg, x_host, x, desc, ws, y, ids, w, U, B in prepared:
        M = cfg.M
        Lc = max(1, min(L, -(-COLD_BYTES // B)))  # copies this workload needs to run cold

        def step(i, stream, rot=Lc):
            j = i % rot
            mdl.moe_decode_forward(desc, M, x, routers[j], weights[j], y, ws, topk_ids=ids, topk_w=w, stream=stream)

        cold = graph_times(torch, step, K, T, W)
        hot = graph_times(torch, lambda i, s: step(i, s, 1), K, T, W)
        cur = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i, (a, b) in enumerate(ev):
            a.record(cur)
            step(i, cur)
            b.record(cur)
        torch.cuda.synchronize()
        eager = [a.elapsed_time(b) * 1e3 for a, b in ev]
        t = pct(cold, 0.5)
        achieved = B / (t * 1e-6) / 1e9
        r = {"workload": cfg.name, "M": M, "weights": synth.FORMAT_NAMES[cfg.weight_fmt], "unique_experts": U,
             "algorithmic_bytes": B, "cold_copies": Lc, "us_cold": summary(cold), "us_hot": summary(hot),
             "us_eager_median": round(pct(eager, 0.5), 3), "tokens_per_s": round(M / (t * 1e-6), 1),
             "hbm_GBps": round(achieved, 1), "frac": round(achieved / PEAK_HBM_GBPS, 4),
             "traffic": traffic_from_profiles(cfg.name)}
        if stream_ref is not None:
            r["stream_ceiling"] = stream_ceiling(torch, stream_ref, B, K, T, W)
            r["frac_of_stream"] = round(r["stream_ceiling"]["us_median"] / t, 4)
        print("[bench] %s U=%d B=%d cold %.2f us (p10 %.2f, p90 %.2f) hot %.2f us  frac %.4f" %
              (cfg.name, U, B, t, pct(cold, 0.1), pct(cold, 0.9), pct(hot, 0.5), r["frac"]),
              file=sys.stderr, flush=True)
        results.append((r, cfg, layer, x_host))
    del copies, weights, routers, base, prepared
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return results


LM_HEAD_WORKLOADS = ["lm_head_bf16_m1", "lm_head_fp8_m1", "lm_head_bf16_m6", "lm_head_fp8_m6"]


def lm_head_bytes(cfg) -> int:
    """Bytes the LM head must move once: the weight (FP8: codes and one scale per row), the token
    rows in and the fp32 logits out."""
    from moe_speculative_decode_amd import synth
    w = cfg.vocab * cfg.hidden * (1 if cfg.weight_fmt == synth.FP8 else 2)
    if cfg.weight_fmt == synth.FP8:
        w += 4 * cfg.vocab
    return w + 2 * cfg.M * cfg.hidden + 4 * cfg.M * cfg.vocab


def measure_lm_heads(torch, mdl, dev, synth, names, args, stream_ref):
    """The LM head GEMV (moe_lm_head) per workload, timed like the layer: cold copies of the weight
    rotated in a graph, hot, eager, and the streaming-read ceiling of the same bytes."""
    results = []
    cache = {}
    for name in names:
        cfg = synth.LM_HEADS[name]
        key = (cfg.weight_fmt, cfg.hidden, cfg.vocab, cfg.seed)
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            t0 = time.time()
            w, sc = synth.lm_head_weights(cfg)
            print("[bench] %s weight generated in %.1fs" % (name, time.time() - t0), file=sys.stderr, flush=True)
            B1 = lm_head_bytes(cfg)
            L = args.copies or max(1, -(-COLD_BYTES // B1))
            wd = [dev.to_device(w)]
            wd += [wd[0].clone() for _ in range(L - 1)]
            scd = None if sc is None else [dev.to_device(sc)]
            if scd is not None:
                scd += [scd[0].clone() for _ in range(L - 1)]
            cache[key] = (wd, scd, L)
            del w, sc
        wd, scd, L = cache[key]
        x = dev.to_device(synth.lm_head_hidden(cfg, 1))
        out = torch.empty((cfg.M, cfg.vocab), dtype=torch.float32, device="cuda")
        desc = mdl.moe_lm_head_desc_t(cfg.hidden, cfg.vocab, cfg.weight_fmt)
        B = lm_head_bytes(cfg)

        def step(i, stream, rot=L):
            j = i % rot
            mdl.moe_lm_head(desc, cfg.M, x, wd[j], out, w_scale=None if scd is None else scd[j], stream=stream)

        K, W, T = args.steps, args.warmup, args.trials
        cold = graph_times(torch, step, K, T, W)
        hot = graph_times(torch, lambda i, st: step(i, st, 1), K, T, W)
        t = pct(cold, 0.5)
        achieved = B / (t * 1e-6) / 1e9
        r = {"workload": name, "M": cfg.M, "weights": synth.FORMAT_NAMES[cfg.weight_fmt], "vocab": cfg.vocab,
             "hidden": cfg.hidden, "algorithmic_bytes": B, "cold_copies": L, "us_cold": summary(cold),
             "us_hot": summary(hot), "tokens_per_s": round(cfg.M / (t * 1e-6), 1), "hbm_GBps": round(achieved, 1),
             "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_from_profiles(name)}
        if stream_ref is not None:
            r["stream_ceiling"] = stream_ceiling(torch, stream_ref, B, K, T, W)
            r["frac_of_stream"] = round(r["stream_ceiling"]["us_median"] / t, 4)
        print("[bench] %s cold %.2f us (p10 %.2f, p90 %.2f) hot %.2f us  frac %.4f" %
              (name, t, pct(cold, 0.1), pct(cold, 0.9), pct(hot, 0.5), r["frac"]), file=sys.stderr, flush=True)
        results.append(r)
    cache.clear()
    torch.cuda.empty_cache()
    return results


def stream_ceiling(torch, ref, nbytes: int, K: int, T: int, W: int):
    """A plain streaming read of nbytes, cold (rotating over enough distinct buffers), graph-replayed
    like the layer."""
    nb = (nbytes + 15) // 16 * 16
    L = max(1, -(-COLD_BYTES // nb))
    buf = torch.empty(L * nb, dtype=torch.uint8, device="cuda")
    sink = torch.empty(max(1, ref.L.moe_bench_stream_read_blocks()), dtype=torch.int32, device="cuda")
    base = buf.data_ptr()

    def step(i, stream):
        ref.launch(base + (i % L) * nb, nb, sink.data_ptr(), stream.cuda_stream)

    t = graph_times(torch, step, K, T, W)
    del buf
    med = pct(t, 0.5)
    gbps = nbytes / (med * 1e-6) / 1e9
    return {"us_median": round(med, 3), "GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="steps per graph replay (K)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--trials", type=int, default=20, help="graph replays timed per workload (>= 10)")
    ap.add_argument("--config", default=None, help="measure only these workloads (comma-separated names)")
    ap.add_argument("--copies", type=int, default=0, help="layer copies rotated (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-budget", type=float, default=6.0, help="seconds per CPU-baseline timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-read reference")
    ap.add_argument("--calib-copy", action="store_true", help="run a plain 1 GiB device copy (counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer has no multi-GPU path here (one GPU holds the "
              "whole layer); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    args.trials = max(10, args.trials)

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

    names = args.config.split(",") if args.config else WORKLOADS + LM_HEAD_WORKLOADS
    layer_names = [n for n in names if n in synth.CONFIGS]
    head_names = [n for n in names if n in synth.LM_HEADS]
    stream_ref = None if args.no_stream else StreamRef()
    by_fmt = {}
    for n in layer_names:
        by_fmt.setdefault(synth.CONFIGS[n].weight_fmt, []).append(n)
    results = []
    for fmt, group in by_fmt.items():
        results += measure_format(torch, mdl, dev, synth, group, args, stream_ref)
    lm_heads = measure_lm_heads(torch, mdl, dev, synth, head_names, args, stream_ref) if head_names else []
    if not results:  # an LM-head run only
        print(json.dumps({"metric": "LM head us/step", "workloads": lm_heads}), flush=True)
        return
    head = next((r for r in results if r[0]["workload"] == HEADLINE), results[0])
    hr, hcfg, hlayer, hx = head
    t = hr["us_cold"]["median"]
    out = {
        "metric": METRIC, "value": t, "unit": "us/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": hr["weights"], "data": "synthetic",
        "config": {"workload": hr["workload"], "M": hcfg.M, "hidden": hcfg.hidden, "experts": hcfg.num_experts,
                   "top_k": hcfg.top_k, "inter": hcfg.inter, "shared_inter": hcfg.shared_inter,
                   "weights": hr["weights"], "unique_experts": hr["unique_experts"],
                   "algorithmic_bytes": hr["algorithmic_bytes"], "cold_copies": hr["cold_copies"],
                   "timing": "median of %d hipGraph replays of %d steps rotating cold copies" %
                             (args.trials, args.steps)},
        "tokens_per_s": hr["tokens_per_s"], "hbm_GBps": hr["hbm_GBps"], "hbm_frac": hr["frac"],
        "us_p10": hr["us_cold"]["p10"], "us_p90": hr["us_cold"]["p90"], "us_hot": hr["us_hot"]["median"],
        "eager_median_us": hr["us_eager_median"],
        "roofline": {"bound": "hbm", "achieved": hr["hbm_GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": hr["frac"], "traffic": hr["traffic"]},
        "stream_ceiling": hr.get("stream_ceiling"),
        "workloads": [r[0] for r in results] + lm_heads,
    }
    if not args.no_cpu_baseline:
        import numpy as np
        out["cpu_baseline"] = cpu_baseline(hcfg, hlayer, np.ascontiguousarray(hx), args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

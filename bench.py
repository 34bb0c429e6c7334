"""Benchmark of the Prox sparse SwiGLU FFN forward on one MI355X.

Default workload: one 8B-like FFN layer (d_model 4096, d_ff 14336, bf16
weights N(0, 0.02^2)), one decode token, input keep 0.5, FFN sparsity 0.7,
int8 per-row proxy.  A step is one full forward of the layer (both stages:
two kernels for one token).  Four copies of the weights and proxy (1.9 GB) are cycled so
each step streams its weights from HBM, not from the 256 MB Infinity Cache.

Prints one JSON line: µs per layer (back-to-back steps on one stream), the
layer's effective GB/s against the 8 TB/s HBM peak, per-call latency
percentiles (one event pair around each call), the dominant kernel's
roofline beside the measured stream-read ceiling (prox_read_probe over
1 GiB), the HIP-graph variant, the dense (sparsity 0) comparator, and the
CPU oracle timed on the host as a baseline (all threads and one thread, the
dense oracle FFN too, and the CPU model).

The dominant kernel's duration is measured live: a HIP graph of back-to-back
launches of that kernel alone (cycling the weight sets) is replayed between
two events on the stream it runs on, and the average per launch is taken.

    python bench.py [--steps K] [--warmup W] [--workload llama8b] [--batch 1]
                    [--sparsity 0.7] [--mode int8_row] [--no-cpu] [--copy-calibration]

--copy-calibration ends the run with a 256 MiB device-to-device copy, the
known-size kernel against which the memory-traffic counters are scaled.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "µs/FFN layer + HBM GB/s (% roofline), 4096×14336 bf16 @70% sparsity, B=1"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="llama8b", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--sparsity", type=float, default=None)
    ap.add_argument("--keep", type=float, default=None)
    ap.add_argument("--mode", default=None)
    ap.add_argument("--wformat", default="native", choices=["native", "fp8"],
                    help="exact (Stage-2) weights in the activation dtype, or FP8 E4M3 with per-row scales")
    ap.add_argument("--sets", type=int, default=4, help="weight copies cycled to defeat the Infinity Cache")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="fit the sparsity-allocation cost model from measured stage times and test its plans")
    ap.add_argument("--chain", action="store_true",
                    help="time the 32-layer chain (RMSNorm + residual between layers) at B = 1 and 8 instead")
    ap.add_argument("--diagnostics", action="store_true",
                    help="mask recall of each selection signal against the exact-state mask, and its time")
    return ap.parse_args()


def kept_union(x_f32: np.ndarray, k_in: int) -> int:
    """Number of input columns some token keeps (largest |x|, ties to the lower index)."""
    keep = np.zeros(x_f32.shape[1], bool)
    for row in x_f32:
        order = np.lexsort((np.arange(row.size), -np.abs(row.astype(np.float64))))
        keep[order[:k_in]] = True
    return int(keep.sum())


def algorithmic_bytes(d, F, B, k, k_union, bw, mode, fp8=False):
    """Bytes the method must move for one layer: x, proxy codes of the kept
    columns (the union over tokens), proxy scales, the selected gate/up/down
    rows (one byte per weight with FP8 weights, plus their scales), the mask,
    the output.  Workspace traffic (partials, scores) is not counted."""
    if mode == "int8_row":
        proxy = 2 * k_union * F
        scales = 2 * F * 4
    else:
        proxy = k_union * F  # two nibbles per byte, gate and up
        scales = (d // 128) * 2 * F * 4
    ww = 1 if fp8 else bw
    return dict(x=B * d * bw, proxy=proxy, scales=scales, gateup=2 * k * d * ww + (8 * k if fp8 else 0),
                down=k * d * ww + (4 * d if fp8 and k else 0), sel=k * 4, out=B * d * bw)


# the sources the single-token kernels (stage1_fused_kernel, stage2_rows_kernel, stage2_fused_kernel)
# are built from: the stored counter traffic is valid while these are unchanged
DIGEST_SOURCES = ("common.h", "kernels.h", "select.h", "stage1_fused.hip", "stage2.hip", "stage2_rows.hip")


def source_digest() -> str:
    h = hashlib.sha256()
    for f in DIGEST_SOURCES:
        with open(os.path.join(ROOT, "free_sparse_swiglu_stage1_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_digest") != source_digest():
        return None
    return e.get("bytes_per_launch")


def chain_bench(args, torch, P):
    """End-to-end latency of the 32-layer 4096 x 14336 bf16 FFN stack,
    h <- h + FFN_l(RMSNorm(h)) per layer through prox_chain_forward, at
    sparsity 0.7 and keep 0.5, against the same stack dense (sparsity 0).
    Weights are drawn on the GPU (torch's generator, seed = layer, N(0, 0.02)
    in binary32 rounded to bf16): 15 GB of layers would take minutes from the
    host generator, and the values do not change the time (k is fixed).
    Prints one JSON line per batch size."""
    wl = synth.WORKLOADS["llama8b_chain32"]
    d, F, n_layers = wl.d, wl.F, 32
    dev = torch.device("cuda:0")
    t0 = time.time()
    layers, proxies = [], []
    for l in range(n_layers):
        g = torch.Generator(device=dev)
        g.manual_seed(l)
        raw = [(torch.randn(shape, generator=g, device=dev) * wl.std).to(torch.bfloat16)
               for shape in ((F, d), (F, d), (d, F))]
        w = P.pack_weights(*raw)
        del raw
        layers.append(w)
        proxies.append(P.quantize_proxy(w, wl.mode))
    torch.cuda.synchronize()
    print("chain setup %.1fs" % (time.time() - t0), file=sys.stderr, flush=True)
    keep, sp = wl.input_keep, wl.sparsities[0]
    steps, warmup = max(1, min(args.steps, 40)), max(1, min(args.warmup, 4))
    for B in wl.batches:
        x_host = synth.make_x(B, d, wl.dtype, seed=0)
        h = torch.from_numpy(x_host.view(np.int16)).to(dev).view(torch.bfloat16)
        res = {}
        for name, s in (("sparse", sp), ("dense", 0.0)):
            ws = P.workspace_init(torch.empty(P.chain_workspace_size(d, F, B, wl.mode), dtype=torch.uint8,
                                              device=dev))
            for _ in range(warmup):
                P.chain_forward(h, layers, proxies, keep, s, workspace=ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                P.chain_forward(h, layers, proxies, keep, s, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            res[name] = 1000.0 * e0.elapsed_time(e1) / steps
        print(json.dumps({"metric": "us per 32-layer FFN stack (RMSNorm + residual), 4096x14336 bf16 @70% sparsity",
                          "value": round(res["sparse"], 1), "unit": "us/stack", "higher_is_better": False,
                          "steps": steps, "warmup": warmup, "dtype": "bf16", "data": "synthetic",
                          "us_per_layer": round(res["sparse"] / n_layers, 2),
                          "dense_us_per_stack": round(res["dense"], 1),
                          "dense_us_per_layer": round(res["dense"] / n_layers, 2),
                          "config": {"workload": "llama8b_chain32", "layers": n_layers, "batch": B,
                                     "d_model": d, "d_ff": F, "ffn_sparsity": sp, "input_keep": keep,
                                     "proxy": wl.mode}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import free_sparse_swiglu_stage1_amd as P

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    P.load_library()
    if args.chain:
        chain_bench(args, torch, P)
        return
    wl = synth.WORKLOADS[args.workload]
    d, F, dtype = wl.d, wl.F, wl.dtype
    B = args.batch
    if args.sparsity is not None:
        sp = args.sparsity
    else:
        sp = 0.7 if 0.7 in wl.sparsities else wl.sparsities[0]
    keep = wl.input_keep if args.keep is None else args.keep
    mode = wl.mode if args.mode is None else args.mode
    bw = 4 if dtype == "f32" else 2
    dev = torch.device("cuda:0")
    t0 = time.time()

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    wg, wu, wd = synth.make_weights(d, F, wl.std, dtype, seed=0, layer=0)
    x_host = synth.make_x(B, d, dtype, seed=0)
    fp8 = args.wformat == "fp8"
    w0 = (P.pack_weights_fp8 if fp8 else P.pack_weights)(to_dev(wg), to_dev(wu), to_dev(wd))
    p0 = P.quantize_proxy(w0, mode)
    sets = [(w0, p0)]
    for _ in range(1, args.sets):
        if fp8:
            w = P.Weights(w0.w_gu.clone(), w0.w_down_t.clone(), d, F, act_dtype=w0.act_dtype,
                          gu_scales=w0.gu_scales.clone(), down_scales=w0.down_scales.clone())
        else:
            w = P.Weights(w0.w_gu.clone(), w0.w_down_t.clone(), d, F)
        p = P.Proxy(p0.codes.clone(), p0.scales.clone(), p0.mode, d, F)
        sets.append((w, p))
    x = to_dev(x_host)
    out = torch.empty_like(x)
    ws = P.alloc_workspace(d, F, B, mode, dev)
    torch.cuda.synchronize()
    print("setup %.1fs" % (time.time() - t0), file=sys.stderr, flush=True)

    k_in, k = P.counts(d, F, keep, sp)
    k_union = kept_union(synth.to_f32(x_host), k_in)
    parts = algorithmic_bytes(d, F, B, k, k_union, bw, mode, fp8)
    layer_bytes = sum(parts.values())
    R = len(sets)

    def step(i):
        w, p = sets[i % R]
        P.ffn_forward(x, w, p, keep, sp, out=out, workspace=ws)

    # ---- eager, back to back on one stream
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    us_layer = 1000.0 * ms_total / args.steps
    print("eager %.2f us/layer" % us_layer, file=sys.stderr, flush=True)

    # ---- per-call latency: one event pair around each call, back to back
    n_t = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_t)]
    for i in range(n_t):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    lat = sorted(1000.0 * a.elapsed_time(b) for a, b in evs[n_t // 10:])
    pick = lambda q: lat[min(len(lat) - 1, int(q * len(lat)))]  # noqa: E731
    latency = dict(p10=pick(0.10), median=pick(0.50), p90=pick(0.90), p99=pick(0.99), samples=len(lat))

    # ---- HIP graph of R forwards (one per weight set), replayed
    graph_us = None
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for r in range(R):
                        step(r)
            torch.cuda.synchronize()
            ref = out.clone()
            for _ in range(max(1, args.warmup // R)):
                g.replay()
            torch.cuda.synchronize()
            e0.record()
            n_rep = max(1, args.steps // R)
            for _ in range(n_rep):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_us = 1000.0 * e0.elapsed_time(e1) / (n_rep * R)
            step(R - 1)
            torch.cuda.synchronize()
            if not torch.equal(out.view(torch.int16), ref.view(torch.int16)):
                graph_us = None
                print("graph replay output differs from eager; graph timing dropped", file=sys.stderr)
        except Exception as exc:  # pragma: no cover
            print("graph capture unavailable: %r" % (exc,), file=sys.stderr)
    print("graph %s us/layer" % graph_us, file=sys.stderr, flush=True)

    # ---- each stage alone, live: a HIP graph of back-to-back launches of
    # that stage (cycling the weight sets) replayed between two events on the
    # graph's stream.  For one token each stage is one kernel.
    sels = []
    for r in range(R):
        w, p = sets[r]
        sels.append(P.stage1_select(x, w, p, keep, sp, workspace=ws) if k not in (0, F) else None)
    torch.cuda.synchronize()
    sel_buf = torch.empty(max(k, 1), dtype=torch.int32, device=dev)
    n_l = 4 * R

    def live_us(launch):
        try:
            g1 = torch.cuda.CUDAGraph()
            s1 = torch.cuda.Stream()
            s1.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s1):
                with torch.cuda.graph(g1, stream=s1):
                    for i in range(n_l):
                        launch(i)
            torch.cuda.synchronize()
            for _ in range(3):
                g1.replay()
            torch.cuda.synchronize()
            n_rep = max(2, min(50, args.steps // n_l))
            e0.record()
            for _ in range(n_rep):
                g1.replay()
            e1.record()
            torch.cuda.synchronize()
            return 1000.0 * e0.elapsed_time(e1) / (n_rep * n_l)
        except Exception as exc:  # pragma: no cover
            print("stage graph timing unavailable (%r)" % (exc,), file=sys.stderr)
            return None

    def s1_launch(i):
        w, p = sets[i % R]
        P.stage1_select(x, w, p, keep, sp, workspace=ws, sel_out=sel_buf)

    def s2_launch(i):
        w, _ = sets[i % R]
        P.stage2_exact(x, w, sels[i % R], out=out, workspace=ws)

    has_s1 = k not in (0, F)
    kern_us = {}
    if has_s1:
        kern_us["stage1"] = live_us(s1_launch)
    kern_us["stage2"] = live_us(s2_launch) if has_s1 else live_us(lambda i: step(i))
    kern_us = {kk: v for kk, v in kern_us.items() if v is not None}
    kern_bytes = {"stage1": parts["x"] + parts["proxy"] + parts["scales"] + parts["sel"],
                  "stage2": parts["gateup"] + parts["down"] + parts["x"] + parts["out"] + parts["sel"]}
    rows = B == 1 and dtype == "bf16" and not fp8 and d in (4096, 8192) and -(-k // 256) <= 128
    one_kernel = {"stage1": "stage1_fused_kernel" if (B == 1 and d <= 8192 and F <= 16384) else None,
                  "stage2": ("stage2_rows_kernel" if rows else "stage2_fused_kernel") if B == 1 else None}
    # ---- the measured stream-read ceiling: one read of a 1 GiB buffer (four
    # times the Infinity Cache), the probe kernel's best of several reps
    read_ceiling = None
    try:
        nb = 1 << 30
        big = torch.empty(nb // 4, dtype=torch.int32, device=dev).fill_(7)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        reps = []
        for r in range(8):
            e0.record()
            P.read_probe(big, sink)
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                reps.append(nb / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        read_ceiling = {"gbps": round(max(reps), 1), "median_gbps": round(statistics.median(reps), 1),
                        "bytes": nb, "kernel": "read_probe_kernel"}
        del big
    except Exception as exc:  # pragma: no cover
        print("read probe unavailable (%r)" % (exc,), file=sys.stderr)
    dom = max(kern_us, key=kern_us.get)
    dom_us, dom_kernel = kern_us[dom], one_kernel[dom]
    dom_bytes = kern_bytes[dom]
    dom_gbps = dom_bytes / (dom_us * 1e-6) / 1e9
    wl_name = "%s_ffn_%dx%d_%s_B%d_sp%g_keep%g_%s%s" % (args.workload, d, F, dtype, B, sp, keep, mode,
                                                         "_fp8w" if fp8 else "")
    traffic = traffic_from_profiles(dom_kernel or dom, wl_name)
    roofline = {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dom_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": dom_kernel or dom,
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3),
                "measured_read_ceiling_gbps": None if read_ceiling is None else read_ceiling["gbps"],
                "frac_of_measured_ceiling": None if read_ceiling is None else round(dom_gbps / read_ceiling["gbps"], 4)}
    layer_gbps = layer_bytes / (us_layer * 1e-6) / 1e9

    # ---- dense comparator: the same library at sparsity 0 (Stage 1 skipped)
    dense_us = None
    if not args.no_dense:
        n_d = max(R, args.steps // 4)
        for i in range(R):
            w, p = sets[i % R]
            P.ffn_forward(x, w, p, keep, 0.0, out=out, workspace=ws)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n_d):
            w, p = sets[i % R]
            P.ffn_forward(x, w, p, keep, 0.0, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        dense_us = 1000.0 * e0.elapsed_time(e1) / n_d
    print("dominant %s %.2f us/launch; dense %s us/layer" % (dom_kernel or dom, dom_us, dense_us),
          file=sys.stderr, flush=True)

    # ---- sparsity-allocation cost model: stage times measured live at several
    # fractions, a straight line fitted to each, the dense layer as the unit;
    # then the library's allocation for a few targets, timed end to end
    calibration = None
    if args.calibrate:
        keeps = [0.3, 0.5, 0.7, 1.0]
        t1 = []
        for kp in keeps:
            def s1k(i, kp=kp):
                w, p = sets[i % R]
                P.stage1_select(x, w, p, kp, sp, workspace=ws, sel_out=sel_buf)
            t1.append(live_us(s1k))
        kappas = [0.1, 0.3, 0.5, 0.7, 0.9]
        t2 = []
        rng = np.random.default_rng(7)
        for kap in kappas:
            kk = int(round(kap * F))
            selk = torch.from_numpy(np.sort(rng.choice(F, kk, replace=False)).astype(np.int32)).to(dev)
            def s2k(i, selk=selk):
                w, _ = sets[i % R]
                P.stage2_exact(x, w, selk, out=out, workspace=ws)
            t2.append(live_us(s2k))
        b1, a1 = np.polyfit(keeps, t1, 1)
        b2, a2 = np.polyfit(kappas, t2, 1)
        def dense_launch(i):
            w, p = sets[i % R]
            P.ffn_forward(x, w, p, keep, 0.0, out=out, workspace=ws)
        t_dense = live_us(dense_launch)
        model = (max(a1, 0.0), max(b1, 0.0), max(a2, 0.0), b2, t_dense)
        plans = {}
        for target in (0.3, 0.4, 0.5):
            plan = P.allocate_sparsity(model, target)
            if plan is None:
                plans[str(target)] = None
                continue
            kp, spp = plan
            def fwd(i, kp=kp, spp=spp):
                w, p = sets[i % R]
                P.ffn_forward(x, w, p, kp, spp, out=out, workspace=ws)
            t_plan = live_us(fwd)
            plans[str(target)] = {"input_keep": round(kp, 4), "ffn_sparsity": round(spp, 4),
                                  "predicted_us": round((1.0 - target) * t_dense, 3), "measured_us": round(t_plan, 3),
                                  "measured_effective_sparsity": round(1.0 - t_plan / t_dense, 4)}
        calibration = {"stage1_us": dict(zip(map(str, keeps), [round(v, 3) for v in t1])),
                       "stage2_us": dict(zip(map(str, kappas), [round(v, 3) for v in t2])),
                       "dense_us": round(t_dense, 3),
                       "model": dict(zip(("stage1_fixed_us", "stage1_per_keep_us", "stage2_fixed_us",
                                          "stage2_per_kept_us", "dense_us"), [round(v, 4) for v in model])),
                       "plans": plans}
        print("calibration %s" % json.dumps(calibration), file=sys.stderr, flush=True)

    # ---- selection-signal diagnostics: each signal's mask against the ideal
    # (exact-state) mask of the same token, and the forward time with it
    diagnostics = None
    if args.diagnostics and 0 < k < F:
        masks, times = {}, {}
        for signal in ("exact_s", "s", "h", "u"):
            sel_d = torch.empty(k, dtype=torch.int32, device=dev)
            w, p = sets[0]
            P.ffn_forward(x, w, p, keep, sp, out=out, sel_out=sel_d,
                          workspace=ws, signal=signal)
            torch.cuda.synchronize()
            masks[signal] = set(sel_d.cpu().numpy().tolist())
            n_s = max(R, args.steps // 8)
            e0.record()
            for i in range(n_s):
                w, p = sets[i % R]
                P.ffn_forward(x, w, p, keep, sp, out=out, workspace=ws,
                              signal=signal)
            e1.record()
            torch.cuda.synchronize()
            times[signal] = round(1000.0 * e0.elapsed_time(e1) / n_s, 3)
        diagnostics = {sig: {"recall_vs_exact_state_mask": round(len(masks[sig] & masks["exact_s"]) / k, 4),
                             "us_per_layer": times[sig]} for sig in masks}
        print("diagnostics %s" % diagnostics, file=sys.stderr, flush=True)

    # ---- CPU oracle baseline (bounded sample on the host cores)
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        oracle.build(force=False)
        if fp8:  # the oracle's FP8 copy; the proxy is built from its binary32 values
            f8 = oracle.quantize_fp8(wg) + oracle.quantize_fp8(wu) + oracle.quantize_fp8(wd)
            proxy_q = (oracle.quantize(oracle.dequant_fp8_f32(f8[0], f8[1]), mode) +
                       oracle.quantize(oracle.dequant_fp8_f32(f8[2], f8[3]), mode))
        else:
            f8 = None
            proxy_q = oracle.quantize(wg, mode) + oracle.quantize(wu, mode)
        def sample(fn, budget_s, max_n):
            ts = []
            t_end = time.time() + budget_s
            while True:
                t = time.perf_counter()
                r = fn()
                ts.append(time.perf_counter() - t)
                if time.time() > t_end or len(ts) >= max_n:
                    return r, ts
        n_all = oracle.get_threads()
        ref, times = sample(lambda: oracle.prox_forward(x_host, wg, wu, wd, proxy_q, keep, sp, mode, fp8=f8), 6.0, 40)
        _, dense_times = sample(lambda: oracle.ffn_dense(x_host, wg, wu, wd), 4.0, 20)
        oracle.set_threads(1)
        try:
            _, times_1 = sample(lambda: oracle.prox_forward(x_host, wg, wu, wd, proxy_q, keep, sp, mode, fp8=f8),
                                8.0, 10)
        finally:
            oracle.set_threads(n_all)
        cpu_model = None
        try:
            with open("/proc/cpuinfo") as fh:
                for ln in fh:
                    if ln.startswith("model name"):
                        cpu_model = ln.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        cpu = {"value": round(1e6 * statistics.median(times), 1), "unit": "us/layer",
               "cores": n_all, "kind": "oracle",
               "sample": "%d full oracle forwards of the same layer and token (median), binary64 C loops, "
                         "%d threads" % (len(times), n_all),
               "value_1_thread": round(1e6 * statistics.median(times_1), 1),
               "sample_1_thread": "%d forwards on 1 thread (median)" % len(times_1),
               "dense_oracle_value": round(1e6 * statistics.median(dense_times), 1),
               "dense_oracle_sample": "%d dense SwiGLU FFNs (all channels, no proxy) on %d threads (median)"
                                      % (len(dense_times), n_all),
               "cpu_model": cpu_model, "host_logical_cpus": os.cpu_count()}
        # parity of the timed configuration against the oracle
        sel = torch.empty(max(k, 1), dtype=torch.int32, device=dev)
        y = P.ffn_forward(x, w0, p0, keep, sp, sel_out=sel)
        torch.cuda.synchronize()
        sel_np = sel[:k].cpu().numpy().astype(np.int64)
        ok, msg = oracle.mask_admissible(sel_np, ref["sel"], ref["score"], ref["T"], k)
        y_ref, _ = (oracle.ffn_masked(x_host, wg, wu, wd, sel_np) if f8 is None else
                    oracle.ffn_masked_fp8(x_host, f8, sel_np))
        yg = (y.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else y.cpu().numpy())
        yg = oracle.as_f64(yg)
        err = max(float(np.abs(yg[b] - y_ref[b]).max() / np.abs(y_ref[b]).max()) for b in range(B))
        parity = {"mask_admissible": bool(ok), "max_rel_err": err, "mask": msg}

    line = {
        "metric": METRIC,
        "value": round(us_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype + ("+fp8e4m3w" if fp8 else ""),
        "data": "synthetic",
        "config": {"workload": wl_name,
                   "d_model": d, "d_ff": F, "batch": B, "ffn_sparsity": sp, "input_keep": keep, "proxy": mode,
                   "exact_weights": "fp8_e4m3_row_scaled" if fp8 else dtype,
                   "k": k, "k_in": k_in, "kept_union": k_union, "weight_sets": R},
        "layer_bytes": layer_bytes,
        "layer_gbps": round(layer_gbps, 1),
        "layer_frac_of_hbm_peak": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "latency_us": {kk: round(v, 2) for kk, v in latency.items()},
        "graph_us_per_layer": None if graph_us is None else round(graph_us, 3),
        "kernels_us": {kk: round(v, 3) for kk, v in kern_us.items()},
        "kernels": {kk: one_kernel[kk] for kk in kern_us},
        "kernels_gbps": {kk: round(kern_bytes[kk] / (kern_us[kk] * 1e-6) / 1e9, 1) for kk in kern_us},
        "roofline": roofline,
        "hbm_read_ceiling": read_ceiling,
        "dense_us_per_layer": None if dense_us is None else round(dense_us, 3),
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if diagnostics is not None:
        line["diagnostics"] = diagnostics
    if calibration is not None:
        line["calibration"] = calibration
    print(json.dumps(line), flush=True)

    if args.copy_calibration:  # known-size copy for the memory-traffic counters
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print("copy calibration: 3 device copies of %d bytes" % n, file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()

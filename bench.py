#!/usr/bin/env python3
"""Benchmark: FP8 varlen attention TFLOP/s including Q/K/V quantization.

One step = the whole hot path on one batch already resident in HBM:
fp8vit_quantize_qkv (amax + scale bookkeeping in dynamic mode, e4m3
quantization of Q, K and V) followed by fp8vit_attn_varlen_ws (the attention
with a workspace, which splits the keys of grids too small to fill the GPU;
the same kernel and result as fp8vit_attn_varlen otherwise). Throughput counts
the useful attention flops 4*H*d*sum(L_i^2) per step.

Default workload: one 8192-token segment, 16 heads, head_dim 72, static scales
= 1.5 x calibrated (the MI300X AITER table of the vLLM "FP8 ViT Encoder
Attention" page uses this shape; calibration follows its Calibrate-Once Reuse
Workflow: 16 dynamic passes on calibration draws, values x 1.5 written to a
JSON scale file, read back through the library's loader).

Prints one JSON line (rank 0). Only one GPU is used: --gpus above 1 exits.
"""
import argparse
import json
import os
import re
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (published)
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E (published)
METRIC = "FP8 varlen attn TFLOP/s incl. QKV quant (hd72, L=8192); % FP8 MFMA peak"
# Page number for this metric and workload, on other hardware (context only):
# MI300X AITER FP8 call incl. Q/K/V quantization, 16 heads, hd72, L=8192: 2.364 ms.
PAGE_MI300X_TFLOPS = {"l8192_hd72_static": 4 * 16 * 72 * 8192 ** 2 / 2.364e-3 / 1e12,
                      "l16384_hd72_static": 4 * 16 * 72 * 16384 ** 2 / 8.655e-3 / 1e12,
                      "l2304_hd72_dyn": 4 * 16 * 72 * 2304 ** 2 / 0.337e-3 / 1e12}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=100, help="untimed steps just before the timed block")
    p.add_argument("--settle-s", type=float, default=2.0,
                   help="untimed clock-settle phase before the warm-up: steps run back to back for this many "
                        "seconds of wall time, whatever --warmup says (the shader clock ramps up under load)")
    p.add_argument("--repeats", type=int, default=10,
                   help="after the timed block, this many more blocks of --steps steps give the median and "
                        "p10/p90 of the time per step")
    p.add_argument("--workload", default="l8192_hd72_static")
    p.add_argument("--rotate-mb", type=float, default=600.0,
                   help="cycle through input copies totalling at least this many MB (defeats the 256 MB MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle baseline")
    p.add_argument("--static-values", default=None,
                   help="q,k,v static values to use instead of calibrating (profiling runs: no dynamic passes)")
    p.add_argument("--out", choices=("bf16", "fp8"), default="bf16",
                   help="attention output: bf16, or e4m3 with a static output descale (fused fp8 output)")
    p.add_argument("--scaling", choices=("tensor", "mx"), default="tensor",
                   help="tensor: per-tensor scales (the method); mx: block-scaled Q and K (E8M0 scale per "
                        "32-element block of head_dim), per-tensor V")
    p.add_argument("--graph", action="store_true",
                   help="also time the steps as one captured HIP graph (no host launch gaps)")
    p.add_argument("--no-hot", dest="hot", action="store_false",
                   help="skip the 'hot' figure (the same steps on a single input set, no rotation), "
                        "which is reported beside the rotated one by default")
    p.add_argument("--kernel-events-every", type=int, default=10,
                   help="bracket the quantize and attention launches with HIP events on every N-th timed step")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (for scaling HBM byte counters)")
    return p.parse_args()


def to_dev(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def calibrate_static(fv, w, dev, margin=1.5):
    """Calibrate-once: 16 dynamic passes on calibration draws, then the library
    saves margin x window max to a JSON scale file and reads it back."""
    cal = fv.new_state(dev)
    for s in w.warm_seeds:
        q, k, v = (to_dev(x, dev) for x in w.inputs(s))
        fv.quantize_qkv(q, k, v, cal, "dynamic")
    vals = fv.calibrated_values(cal, margin)
    layer = "visual.blocks.0.attn.attn"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "scales.json")
        fv.save_static_scales(path, layer, vals)
        loaded = fv.load_static_scales(path, layer)
    assert tuple(loaded) == tuple(vals)
    return [float(x) for x in loaded]


def cpu_baseline(w, qb, kb, vb, static_values, out_gpu, target_s, compare=True, mx=False):
    """The oracle, untuned, timed on this host: oracle quantization of Q, K and V
    plus fp64 oracle attention. Whole steps are repeated until about `target_s`
    seconds of CPU work are done; a workload whose single step would take more
    than 30 s is sampled instead (the first rows of every segment and head, all
    keys), its step time extrapolated linearly in query rows. The oracle rows
    computed here are also compared with the GPU output of the same input."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    H, d = qb.shape[1], qb.shape[2]
    sigma = np.float64(oracle.attention.default_softmax_scale(d))
    cu = [int(x) for x in w.cu_seqlens]
    segs = [(cu[i], cu[i + 1]) for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]

    def quantize():
        ring = oracle.scales.AmaxRing()
        if mx:
            r = oracle.pipeline.forward_mx(qb, kb, vb, None, w.mode, ring=ring, static_values=static_values,
                                           attend=False)
            return [oracle.mx.dequantize(*r.q), oracle.mx.dequantize(*r.k),
                    oracle.quant.dequantize(r.v_codes, r.v_descale)]
        codes, ds, _ = oracle.pipeline.quantize_step(qb, kb, vb, w.mode, ring=ring, static_values=static_values)
        return [oracle.quant.dequantize(c, dd) for c, dd in zip(codes, ds)]

    def attend(deq, rows):
        res = []
        for s0, s1 in segs:
            n = min(rows, s1 - s0)
            for h in range(H):
                res.append((s0, s1, n, h, oracle.attention._segment_head(
                    deq[0][s0:s0 + n, h], deq[1][s0:s1, h], deq[2][s0:s1, h], sigma)))
        return res

    t0 = time.perf_counter()
    deq = quantize()
    t_quant = time.perf_counter() - t0
    s0, s1 = segs[0]
    t0 = time.perf_counter()
    oracle.attention._segment_head(deq[0][s0:s0 + min(64, s1 - s0), 0], deq[1][s0:s1, 0], deq[2][s0:s1, 0], sigma)
    pilot = time.perf_counter() - t0
    rate = 4.0 * d * min(64, s1 - s0) * (s1 - s0) / max(pilot, 1e-9)      # flop/s of the oracle attention
    est_step = t_quant + w.flops / rate
    work_s = t_quant + pilot
    if est_step <= 30.0:
        # whole steps until target_s of CPU work, never past 30 s
        reps, elapsed = 0, 0.0
        t0 = time.perf_counter()
        while reps == 0 or (elapsed < target_s and elapsed + elapsed / reps <= 30.0):
            deq = quantize()
            rows_out = attend(deq, 1 << 30)
            reps += 1
            elapsed = time.perf_counter() - t0
        work_s += elapsed
        value = reps * w.flops / elapsed / 1e12
        sample = (f"{reps} whole step(s): oracle quantization of all {3 * qb.size} elements + fp64 attention "
                  f"over every query row of every segment and head; {work_s:.1f} s of CPU work")
        step_s = elapsed / reps
    else:
        frac = max(1e-4, (target_s - t_quant) * rate / w.flops)
        rows = max(1, int(frac * max(s1 - s0 for s0, s1 in segs)))
        t0 = time.perf_counter()
        rows_out = attend(deq, rows)
        t_attn = time.perf_counter() - t0
        work_s += t_attn
        done = sum(4.0 * d * n * (b - a) for a, b, n, _, _ in rows_out)     # flops of the sampled rows
        step_s = t_quant + t_attn * w.flops / done
        value = w.flops / step_s / 1e12
        sample = (f"oracle quantization of all {3 * qb.size} elements + fp64 attention for the first {rows} query "
                  f"rows of every segment and head (all keys); step time extrapolated linearly in query rows; "
                  f"{work_s:.1f} s of CPU work")
    if not compare:
        return {"value": value, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle", "sample": sample,
                "seconds_per_step": round(step_s, 3)}
    vmax = float(np.abs(oracle.quant.bf16_to_f32(vb)).max())
    err = max(float(np.abs(out_gpu[a:a + n, h].astype(np.float64) - o).max()) for a, _, n, h, o in rows_out)
    # the method's own error on the same rows: unquantized fp64 attention of the bf16 inputs
    fp = [oracle.quant.bf16_to_f32(x) for x in (qb, kb, vb)]
    e_gpu = e_orc = ref2 = 0.0
    for a, b, n, h, o in rows_out:
        r = oracle.attention._segment_head(*(np.asarray(x, np.float64) for x in
                                             (fp[0][a:a + n, h], fp[1][a:b, h], fp[2][a:b, h])), sigma)
        e_gpu += float(np.sum((out_gpu[a:a + n, h].astype(np.float64) - r) ** 2))
        e_orc += float(np.sum((o - r) ** 2))
        ref2 += float(np.sum(r ** 2))
    return {"value": value, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle", "sample": sample,
            "seconds_per_step": round(step_s, 3),
            "gpu_vs_oracle_max_abs_over_vmax": err / vmax if vmax > 0 else 0.0,
            "gpu_rel_rms_vs_fp64": (e_gpu / ref2) ** 0.5 if ref2 > 0 else 0.0,
            "oracle_rel_rms_vs_fp64": (e_orc / ref2) ** 0.5 if ref2 > 0 else 0.0,
            "gpu_rows_checked": int(sum(n for _, _, n, _, _ in rows_out))}


def attn_kernel_name(w, dev, out8, mx=False):
    """Name of the attention kernel instance the library launches for this
    workload, as the profiler prints it: the wide shape (256 queries per
    workgroup) is used once its workgroups cover at least half of the CUs; at
    head dim 72 it is the 32x32-block kernel attn_w32_kernel."""
    import torch
    d = w.head_dim
    T, nseg, L = w.total_tokens, len(w.seglens), max(w.seglens)
    tiles = min((T + 255) // 256 + nseg, nseg * ((L + 255) // 256))
    wide = 2 * w.heads * tiles >= torch.cuda.get_device_properties(dev).multi_processor_count
    o8 = "true" if out8 else "false"
    m = "true" if mx else "false"
    if wide and d == 72:
        return "attn_w32_kernel<%s, %s>" % (o8, m)
    return "attn_kernel<%d, %s, %s, %s>" % (d, o8, "true" if wide else "false", m)


def attn_traffic(workload, head_dim):
    """HBM bytes per attention launch from the committed counter summary
    profiles/traffic_attn_<workload>.md, or None when the summary is missing or
    was taken on a different attention kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_attn_{workload}.md")
    src = os.path.join(ROOT, "fp8_quantized_varlen_amd", "csrc", "attn.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        m = re.match(r"^- ([a-z0-9_ ]+): `?([0-9a-f.]+)`?\s*$", line.strip())
        if m:
            fields[m.group(1)] = m.group(2)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("attention kernel source sha256") != sha or "traffic bytes per launch" not in fields:
        return None
    return int(float(fields["traffic bytes per launch"]))


class ClockSampler:
    """Shader clock (MHz) of the benchmarked GPU from the SMU metrics table
    (amdsmi, the library behind amd-smi). Best effort: on any failure the
    readings are None and the reason is kept in `error`. `start()` begins
    sampling from a background thread (every ~0.5 ms while the main thread
    waits for the GPU), `stop()` returns the samples taken since."""

    def __init__(self, dev_index):
        import threading
        self.h, self.error, self._amdsmi = None, None, None
        self._lock, self._stop, self._thread, self._samples = threading.Lock(), threading.Event(), None, []
        try:
            import amdsmi
            import torch
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            props = torch.cuda.get_device_properties(dev_index)
            want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            handles = amdsmi.amdsmi_get_processor_handles()
            for h in handles:
                dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.h = h
            if self.h is None and len(handles) == 1:
                self.h = handles[0]
            if self.h is None:
                self.error = "no amdsmi handle matches the PCI address of cuda:%d" % dev_index
            else:
                self.read()
        except Exception as e:  # noqa: BLE001 - best effort only
            self.h, self.error = None, "%s: %s" % (type(e).__name__, e)

    def read(self):
        """Current shader clock in MHz (mean over the XCDs that report one)."""
        if self.h is None:
            return None
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        clks = m.get("current_gfxclks")
        if isinstance(clks, list):
            vals = [c for c in clks if isinstance(c, (int, float)) and 0 < c < 10000]
            if vals:
                return float(sum(vals)) / len(vals)
        for key in ("current_gfxclk", "average_gfxclk_frequency"):
            c = m.get(key)
            if isinstance(c, (int, float)) and 0 < c < 10000:
                return float(c)
        return None

    def safe_read(self):
        try:
            return self.read()
        except Exception as e:  # noqa: BLE001
            self.error = "%s: %s" % (type(e).__name__, e)
            return None

    def _run(self):
        while not self._stop.is_set():
            c = self.safe_read()
            if c is not None:
                with self._lock:
                    self._samples.append(c)
            self._stop.wait(0.0005)

    def start(self):
        import threading
        if self.h is None:
            return
        self._samples, self._stop = [], threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is None:
            return []
        self._stop.set()
        self._thread.join()
        self._thread = None
        with self._lock:
            return list(self._samples)


def _r(x, nd):
    return None if x is None else round(float(x), nd)


def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q)) if xs else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path has no multi-GPU mode (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import fp8_quantized_varlen_amd as fv
    from synth import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qb, kb, vb = w.inputs()
    T, H, d = qb.shape
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    max_seqlen = max(w.seglens)

    st = fv.new_state(dev)
    static_values = None
    if w.mode == "static":
        if args.static_values:
            static_values = [float(x) for x in args.static_values.split(",")]
        else:
            static_values = calibrate_static(fv, w, dev)
        fv.state_set_static(st, static_values)
    base = [to_dev(x, dev) for x in (qb, kb, vb)]
    if w.mode == "dynamic":
        for s in w.warm_seeds:            # fill the amax ring before measuring
            fv.quantize_qkv(*(to_dev(x, dev) for x in w.inputs(s)), st, "dynamic")
    in_bytes = 3 * T * H * d * 2
    n_sets = int(min(16, max(1, np.ceil(args.rotate_mb * 1e6 / max(in_bytes, 1)))))
    sets = [base] + [[torch.roll(x, shifts=(i * 997) % max(T, 1), dims=0) for x in base] for i in range(1, n_sets)]
    q8, k8, v8 = (torch.empty((T, H, d), dtype=torch.uint8, device=dev) for _ in range(3))
    out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    out8 = torch.empty((T, H, d), dtype=torch.uint8, device=dev) if args.out == "fp8" else None
    out_descale = torch.tensor([0.0025], dtype=torch.float32, device=dev)

    # workspace for the key split of grids too small to fill the GPU (0 bytes when it would not split)
    ws_bytes = fv.attn_workspace_bytes(len(w.seglens), max_seqlen, T, H, d)
    ws = fv.attn_workspace(len(w.seglens), max_seqlen, T, H, d, device=dev)

    mx = args.scaling == "mx"
    if mx and out8 is not None:
        print("--scaling mx has no fp8 output variant", file=sys.stderr)
        sys.exit(2)
    qs, ks = (torch.empty((T, H, 4), dtype=torch.uint8, device=dev) for _ in range(2))

    def quantize(q, k, v):
        if mx:
            fv.quantize_qkv_mx(q, k, v, st, w.mode, out=(q8, k8, v8, qs, ks))
        else:
            fv.quantize_qkv(q, k, v, st, w.mode, out=(q8, k8, v8))

    def attend():
        if mx:
            fv.attn_varlen_mx(q8, k8, v8, qs, ks, cu, max_seqlen, st, out=out)
        elif out8 is not None:
            fv.attn_varlen_fp8out(q8, k8, v8, cu, max_seqlen, st, out_descale, out=out8)
        else:
            fv.attn_varlen_ws(q8, k8, v8, cu, max_seqlen, st, ws, out=out)
    torch.cuda.synchronize()

    def step(i):
        q, k, v = sets[i % n_sets]
        quantize(q, k, v)
        attend()

    clock = ClockSampler(dev.index or 0)
    clock_idle = clock.safe_read()
    # Clock settle: the shader clock ramps up over some tens of ms of load, so
    # steps run back to back (in batches of 10, one wait per batch) for a fixed
    # wall time before the warm-up, whatever --warmup is.
    settle_steps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        for _ in range(10):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t0
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Per-kernel durations: HIP events around the two launches of every
    # `kernel_events_every`-th timed step (from step every // 2 on). An event
    # record costs a few us of device time here (three per step add ~11 us to a
    # ~300 us step), so the other steps run without them.
    every = max(1, args.kernel_events_every)
    sampled = [i for i in range(args.steps) if i % every == every // 2] or [0]
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clock_before = clock.safe_read()
    clock.start()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        q, k, v = sets[i % n_sets]
        e = ev.get(i)
        if e:
            e[0].record()
        quantize(q, k, v)
        if e:
            e[1].record()
        attend()
        if e:
            e[2].record()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    clock_during = clock.stop()
    clock_after = clock.safe_read()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    quant_samples = [e[0].elapsed_time(e[1]) for e in ev.values()]
    attn_samples = [e[1].elapsed_time(e[2]) for e in ev.values()]

    # Repeated blocks: `repeats` more blocks of the same steps, each bracketed
    # by its own events, give the spread of the time per step; the middle step
    # of each block also brackets its two launches (more per-kernel samples).
    block_ms = []
    for _ in range(max(0, args.repeats)):
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        mid = args.steps // 2
        b0.record()
        for i in range(args.steps):
            q, k, v = sets[i % n_sets]
            if i == mid:
                e[0].record()
            quantize(q, k, v)
            if i == mid:
                e[1].record()
            attend()
            if i == mid:
                e[2].record()
        b1.record()
        torch.cuda.synchronize()
        block_ms.append(b0.elapsed_time(b1) / args.steps)
        quant_samples.append(e[0].elapsed_time(e[1]))
        attn_samples.append(e[1].elapsed_time(e[2]))
    clock_end = clock.safe_read()
    quant_ms = float(np.mean(quant_samples))
    attn_ms = float(np.mean(attn_samples))

    # Hot: the same steps on one input set, so that its 85 MB (at L = 8192) can stay
    # in the 256 MB MALL between steps; reported beside the rotated figure.
    hot_ms = None
    if args.hot:
        q, k, v = sets[0]
        for _ in range(10):
            quantize(q, k, v)
            attend()
        torch.cuda.synchronize()
        h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0.record()
        for _ in range(args.steps):
            quantize(q, k, v)
            attend()
        h1.record()
        torch.cuda.synchronize()
        hot_ms = h0.elapsed_time(h1) / args.steps

    graph_ms = None
    if args.graph:
        # the same steps captured once and replayed: device time without launch gaps
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for i in range(args.steps):
                step(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gstart, gend = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gstart.record()
        g.replay()
        gend.record()
        torch.cuda.synchronize()
        graph_ms = gstart.elapsed_time(gend) / args.steps
        del g

    if args.calib_copy:
        a = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()

    # numerics of the benched run on a few sampled rows (cheap; full parity lives in tests/)
    assert not torch.isnan(out).any().item()
    state = fv.state_read(st)

    kname = attn_kernel_name(w, dev, args.out == "fp8", mx)
    value = w.flops / (ms_step * 1e-3) / 1e12
    attn_tflops = w.flops / (attn_ms * 1e-3) / 1e12
    quant_bytes = 3 * T * H * d * 3
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGE_MI300X_TFLOPS[w.name], 3) if w.name in PAGE_MI300X_TFLOPS else None,
        # S = Q K^T on the FP8 MFMA; P.V on the f16 MFMA in the wide kernels,
        # on the FP8 MFMA (two e4m3 terms of P) in the narrow ones. The wide
        # hd72 block-scaled kernel takes d 64..71 of S as exact scaled bf16.
        "dtype": ("fp8e4m3+f16" if kname.startswith("attn_w32") or
                  (kname.startswith("attn_kernel<128") and kname.split(", ")[2] == "true")
                  else "fp8e4m3") + ("+e8m0 block scales (Q, K)" if mx else "")
                 + ("+bf16 (S, d 64..71)" if mx and kname.startswith("attn_w32") else ""),
        "data": "synthetic",
        "config": {"workload": w.name, "segments": list(w.seglens), "heads": H, "head_dim": d, "output": args.out,
                   "key_split_workspace_bytes": ws_bytes if out8 is None and not mx else 0,
                   "scaling": ("Q, K: E8M0 per 32-element block; V: " if mx else "") + w.mode +
                              (" (1.5 x calibrated)" if w.mode == "static" else " (16-slot ring)"),
                   "outlier_frac": w.outlier_frac, "input_sets_rotated": n_sets},
        "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        # the same against the dense FP8 rate at the clock the chip held during the timed
        # block (256 CUs x 8192 FP8 flop per clock per CU x f)
        "pct_fp8_peak_at_measured_clock": (round(100 * value / (256 * 8192 * clk * 1e-6), 2)
                                           if (clk := (clock_during and _pct(clock_during, 50))) else None),
        "settle": {"seconds": round(settle_s, 3), "steps": settle_steps},
        "blocks": {"n": len(block_ms), "steps_each": args.steps,
                   "median_ms_per_step": _r(_pct(block_ms, 50), 4), "p10_ms_per_step": _r(_pct(block_ms, 10), 4),
                   "p90_ms_per_step": _r(_pct(block_ms, 90), 4),
                   "median_value": _r(w.flops / (_pct(block_ms, 50) * 1e-3) / 1e12, 2) if block_ms else None},
        "clock_mhz": {"idle": clock_idle, "before": clock_before, "after": clock_after, "end": clock_end,
                      "during_timed_block": {"n": len(clock_during), "min": _r(min(clock_during), 1),
                                             "median": _r(_pct(clock_during, 50), 1),
                                             "max": _r(max(clock_during), 1)} if clock_during else None,
                      "source": "amdsmi gpu_metrics current_gfxclks (mean over XCDs)",
                      **({"error": clock.error} if clock.error else {})},
        "kernels": {"quantize_ms": round(quant_ms, 4), "attention_ms": round(attn_ms, 4),
                    "attention_ms_median": round(_pct(attn_samples, 50), 4),
                    "quantize_ms_median": round(_pct(quant_samples, 50), 4),
                    "event_samples": len(attn_samples),
                    "quantize_GBps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                    "attention_TFLOPs": round(attn_tflops, 2)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": None if mx else attn_traffic(w.name, d),
                     "kernel": kname},
        "descale_used": state["descale_used"],
        **({"graph": {"ms_per_step": round(graph_ms, 4),
                      "value": round(w.flops / (graph_ms * 1e-3) / 1e12, 2)}} if graph_ms else {}),
        **({"hot": {"ms_per_step": round(hot_ms, 4),
                    "value": round(w.flops / (hot_ms * 1e-3) / 1e12, 2)}} if hot_ms else {}),
        "wall_s_timed_region": round(t_wall, 3),
    }
    if not args.no_cpu_baseline:
        # one more step on the unrotated input, so the oracle rows can be compared with it
        step(0)
        if out8 is not None:     # the oracle check reads the bf16 output of the same input
            fv.attn_varlen(q8, k8, v8, cu, max_seqlen, st, out=out)
        torch.cuda.synchronize()
        out_np = out.float().cpu().numpy()
        # dynamic mode: the GPU ring holds only this input's amax (the scales the oracle's
        # fresh ring gives) once 16 forwards of it have been pushed
        same_scales = w.mode == "static" or args.warmup + args.steps >= 16
        res["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, static_values, out_np, args.cpu_seconds, same_scales, mx)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

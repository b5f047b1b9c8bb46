#!/usr/bin/env python3
"""Decode-step benchmark: one JSON line on stdout.

A "step" is one decode step of the whole workload (every arm / bit-width
segment, every head) over one batch of synthetic inputs already resident in
HBM.  The default workload is the long-horizon mixed-precision stack: 24
independent Gated-DeltaNet layers x batch 512 x 32 heads, Dk = Dv = 128,
delta rule, persistent scales after a 64-step fp32 warmup, bounded
directional rounding; layers 0-3 INT8 g64, layers 4-23 INT4 g32 (two launches
per step).

value       algorithmic state-update bytes per step x steps / wall time (GB/s)
roofline    the dominant kernel (the INT4 g32 segment): its algorithmic bytes
            per launch / its mean launch time from HIP events recorded around
            each launch on the launch stream, against 8 TB/s; traffic = HBM
            bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (profiles/),
            reported only while the kernel sources match the profiled ones
valu_issue  the same launch against its arithmetic floor: its VALU instruction
            count (profiled, same condition) per second, and the launch time
            at full issue of its hot loop's instruction mix priced at this
            run's VALU probe rates
cpu_baseline  the CPU oracle on a bounded sample of the same workload (sampled
            heads, a few steps, the host threads stated), in the same unit

--workload prefill-gla times the chunkwise prefill instead: a step is one
4096-token prompt into batch 64 x 16 heads of INT4 g32 state (diagonal decay),
value = its input and state bytes / wall time; the roofline is the prefill
kernel's, with its integer matrix-core rate reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "state-update HBM GB/s (% of peak) and batch·head·steps/s, INT4 g32"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ("quantized_recurrent_state_amd/csrc/lsq_step_impl.h",
                  "quantized_recurrent_state_amd/csrc/lsq_step_q4.hip",
                  "quantized_recurrent_state_amd/csrc/lsq_step_q8.hip")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=8,
                    help="steps per lsq_decode_run call in the timed region")
    ap.add_argument("--workload", default="stack24")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--fp32-steps", type=int, default=8,
                    help="steps of the fp32-state comparison run (0 disables it)")
    ap.add_argument("--graph", action="store_true",
                    help="also replay K more steps captured in one HIP graph (launch gaps removed)")
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--ceiling-gib", type=float, default=4.0,
                    help="buffer size of the streaming-ceiling probes (0 disables them)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this benchmark measures the decode step on one GPU only; the step needs "
              "no exchange between GPUs, and runs with --gpus above 1 are not part of it",
              file=sys.stderr)
        return 2

    import torch
    import quantized_recurrent_state_amd as lsq
    from quantized_recurrent_state_amd import runner
    from quantized_recurrent_state_amd.inputs import PREFILL_WORKLOADS, WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in PREFILL_WORKLOADS:
        return bench_prefill(args, PREFILL_WORKLOADS[args.workload], dev)
    wl = WORKLOADS[args.workload]
    K, W = args.steps, args.warmup
    stream = torch.cuda.current_stream()

    # ---- set-up (untimed): handles, fp32 warmup + calibration, resident inputs
    arms = []
    shared = None
    t_setup = time.perf_counter()
    for arm in wl.arms:
        st, t_first, _ = runner.prepare(wl, arm, dev)
        cfg = st.cfg
        npl = wl.batch * wl.heads
        if wl.shared_inputs and shared is not None:
            inp = shared
        else:
            inp = runner.inputs(wl, arm, t_first, W + 2 * K + (K if args.graph else 0), npl, dev)
            if wl.shared_inputs:
                shared = inp
        o = torch.empty((cfg.n, cfg.dv), device=dev)
        o_ref = torch.empty((cfg.n, cfg.dv), device=dev) if cfg.policy == lsq.POLICY_YOKED else None
        arms.append(dict(arm=arm, st=st, cfg=cfg, inp=inp, o=o, o_ref=o_ref,
                         bytes=runner.algorithmic_bytes(cfg, o_ref is not None)))
        log(f"arm {arm.name}: {cfg} bytes/step {arms[-1]['bytes'] / 1e9:.3f} GB")
    torch.cuda.synchronize()
    log(f"set-up {time.perf_counter() - t_setup:.1f} s")
    dom = max(range(len(arms)), key=lambda i: arms[i]["bytes"])

    def launch(a, t, s=stream):
        i = a["inp"]
        lsq.lsq_decode_step(a["st"].handle, i["q"][t], i["k"][t], i["v"][t], i["alpha"][t],
                            i["beta"][t], a["o"], a["o_ref"], s)

    for t in range(W):
        for a in arms:
            launch(a, t)
    torch.cuda.synchronize()

    # ---- timed region: K steps through lsq_decode_run, in chunks of C steps per arm
    # (the library's horizon driver; the wall clock includes the launch gaps)
    C = max(1, min(args.chunk, K))

    def run_chunk(a, t, h, s=stream):
        i = a["inp"]
        lsq.lsq_decode_run(a["st"].handle, h, i["q"][t:t + h], i["k"][t:t + h], i["v"][t:t + h],
                           i["alpha"][t:t + h], i["beta"][t:t + h], a["o_run"][:h],
                           None if a["o_ref"] is None else a["o_ref_run"][:h], s)

    for a in arms:
        a["o_run"] = torch.empty((C, a["cfg"].n, a["cfg"].dv), device=dev)
        a["o_ref_run"] = torch.empty_like(a["o_run"]) if a["o_ref"] is not None else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c0 in range(W, W + K, C):
        h = min(C, W + K - c0)
        for a in arms:
            run_chunk(a, c0, h)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # ---- kernel time per launch: the next K steps one launch at a time, HIP events
    # around every launch on the launch stream (outside the wall-clock region).
    # The arms' order alternates from step to step: where arms read the same
    # inputs, the first launch of a step fetches them from HBM and the next finds
    # them in the last-level cache, so each arm takes each position half the time.
    ev_s = [[torch.cuda.Event(enable_timing=True) for _ in range(K)] for _ in arms]
    ev_e = [[torch.cuda.Event(enable_timing=True) for _ in range(K)] for _ in arms]
    torch.cuda.synchronize()
    for j, t in enumerate(range(W + K, W + 2 * K)):
        order = list(enumerate(arms))
        if j % 2:
            order.reverse()
        for i, a in order:
            ev_s[i][j].record(stream)
            launch(a, t)
            ev_e[i][j].record(stream)
    torch.cuda.synchronize()
    for i, a in enumerate(arms):
        ms = sorted(x.elapsed_time(y) for x, y in zip(ev_s[i], ev_e[i]))
        a["launch_us"] = {"median": round(ms[len(ms) // 2] * 1e3, 2),
                          "p10": round(ms[len(ms) // 10] * 1e3, 2),
                          "p90": round(ms[(9 * len(ms)) // 10] * 1e3, 2),
                          "mean": round(sum(ms) / len(ms) * 1e3, 2)}
        a["kernel_gbs"] = round(a["bytes"] / (sum(ms) / len(ms) * 1e-3) / 1e9, 2)
    kern_ms = [x.elapsed_time(y) for x, y in zip(ev_s[dom], ev_e[dom])]
    kern_ms_mean = sum(kern_ms) / len(kern_ms)

    bytes_step = sum(a["bytes"] for a in arms)
    heads_step = sum(a["cfg"].n for a in arms)
    gbs = bytes_step * K / wall / 1e9
    dom_a = arms[dom]
    dom_gbs = dom_a["bytes"] / (kern_ms_mean * 1e-3) / 1e9
    log(f"timed {K} steps (lsq_decode_run, chunks of {C}): {wall * 1e3 / K:.3f} ms/step, "
        f"{gbs:.1f} GB/s; dominant kernel {kern_ms_mean * 1e3:.1f} us, {dom_gbs:.1f} GB/s")

    # ---- optional: the next K steps captured in one HIP graph and replayed once
    # (every launch records its own inputs, step index and bypass slot at
    # capture; the state advances on replay)
    graph = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for t in range(W + 2 * K, W + 3 * K):
                for a in arms:
                    launch(a, t, cs)
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - tg0
        graph = {"steps": K, "ms_per_step": round(gwall * 1e3 / K, 4),
                 "value": round(sum(a["bytes"] for a in arms) * K / gwall / 1e9, 2)}
        log(f"graph replay of {K} steps: {gwall * 1e3 / K:.4f} ms/step")
        del g

    ceiling = None
    if args.ceiling_gib > 0:
        span_kib = runner.state_kib_per_head(dom_a["cfg"])
        ceiling = measure_ceiling(dev, stream, args.ceiling_gib, span_kib)

    traffic = None
    valu_rec = None
    sha = kernel_source_sha()
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if (tr.get("source_sha") == sha and tr.get("workload") == wl.name
                and tr.get("arm") == dom_a["arm"].name):
            traffic = int(tr["hbm_bytes_per_launch"])
            valu_rec = tr.get("valu")
            # measured bytes of the other profiled segments, attached to their arms
            for a in arms:
                a["traffic"] = traffic if a is dom_a else None
                for seg in (tr.get("int8_segment"),):
                    if seg and seg.get("arm") == a["arm"].name:
                        a["traffic"] = int(seg["hbm_bytes_per_launch"])

    # ---- copy probe for counter calibration (outside the timed region)
    if args.copy_probe_gib > 0:
        nbytes = int(args.copy_probe_gib * (1 << 30)) // 256 * 256
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)   # contents irrelevant
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: one device copy of {nbytes} bytes (read {nbytes}, written {nbytes})")
        del src, dst

    # ---- fp32-state comparison at the same shapes (the 'vs FP32 states' context)
    fp32 = None
    if args.fp32_steps > 0:
        fl = []
        for a in arms:
            f = lsq.LsqState(runner.fp32_config(a["cfg"]), device=dev).zero()
            fl.append((a, f))
        torch.cuda.synchronize()
        nf = min(args.fp32_steps, W + 2 * K)
        tf0 = time.perf_counter()
        for t in range(nf):
            for a, f in fl:
                i = a["inp"]
                lsq.lsq_decode_step(f.handle, i["q"][t], i["k"][t], i["v"][t], i["alpha"][t],
                                    i["beta"][t], a["o"], None, stream)
        torch.cuda.synchronize()
        fms = (time.perf_counter() - tf0) * 1e3 / nf
        fbytes = sum(runner.algorithmic_bytes(f.cfg) for _, f in fl)
        fp32 = {"ms_per_step": round(fms, 4), "state_bytes_per_step": fbytes,
                "speedup_of_quantised_step": round(fms / (wall * 1e3 / K), 3),
                "state_memory_ratio": round(
                    sum(f.f32.numel() * 4 for _, f in fl)
                    / sum(a["st"].codes.numel() + a["st"].scales.numel() * a["st"].scales.element_size()
                          for a in arms), 3)}
        del fl
        log(f"fp32-state step {fms:.3f} ms")

    # ---- arms on shared inputs beside a yoked arm: the stored state's Frobenius
    # norm (lsq_state_dequantize, fl(C s)) against the fp32 reference R the yoked
    # arm advances on the same inputs, after the same steps; reported, not a bound
    state_norms = None
    yoked = [a for a in arms if a["cfg"].policy == lsq.POLICY_YOKED]
    if wl.shared_inputs and yoked:
        r_norm = float(torch.linalg.vector_norm(yoked[0]["st"].ref, dtype=torch.float64))
        state_norms = {"reference": "fp32 R of the yoked arm",
                       "steps": int(yoked[0]["st"].step_index), "ratio_to_reference": {}}
        for a in arms:
            S = a["st"].dequantize()
            state_norms["ratio_to_reference"][a["arm"].name] = round(
                float(torch.linalg.vector_norm(S, dtype=torch.float64)) / r_norm, 5)
            del S
        log(f"state norm / reference norm: {state_norms['ratio_to_reference']}")

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(arms, args.cpu_seconds, W + 2 * K)

    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(wall * 1e3 / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "head_steps_per_s": round(heads_step * K / wall, 1),
        "config": {"workload": wl.name, "layers": sum(len(a["arm"].layers) for a in arms),
                   "batch_per_layer": wl.batch, "heads": wl.heads, "dk": wl.dk, "dv": wl.dv,
                   "delta": wl.delta, "decay": "diag" if wl.decay else "scalar",
                   "arms": [{"name": a["arm"].name, "bits": a["cfg"].bits,
                             "group": a["cfg"].group, "policy": a["cfg"].policy,
                             "rounding": a["cfg"].rounding, "scale_fmt": a["cfg"].scale_fmt,
                             "lrb_rank": a["cfg"].lrb_rank, "heads": a["cfg"].n,
                             "bytes_per_step": a["bytes"], "launch_us": a["launch_us"],
                             "kernel_gbs": a["kernel_gbs"],
                             "kernel_head_steps_per_s": round(
                                 a["cfg"].n / (a["launch_us"]["mean"] * 1e-6), 1),
                             "traffic_bytes_per_launch": a.get("traffic"),
                             "traffic_over_algorithmic": (
                                 round(a["traffic"] / a["bytes"], 4) if a.get("traffic") else None)}
                            for a in arms],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": f"decode step, {dom_a['arm'].name}",
                     "algorithmic_bytes_per_launch": dom_a["bytes"],
                     "launch_us_mean": round(kern_ms_mean * 1e3, 2),
                     "launch_us_min": round(min(kern_ms) * 1e3, 2),
                     "source_sha": sha,
                     "ceiling_gbs": ceiling and ceiling["copy"]["gbs"],
                     "frac_of_ceiling": ceiling and round(dom_gbs / ceiling["copy"]["gbs"], 4),
                     "pattern_ceiling_gbs": ceiling and ceiling["span_in_place"]["gbs"],
                     "frac_of_pattern_ceiling": ceiling and round(
                         dom_gbs / ceiling["span_in_place"]["gbs"], 4)},
        "ceiling": ceiling,
        "valu_issue": valu_issue(valu_rec, ceiling, kern_ms_mean, dom_a["bytes"]),
        "fp32_state": fp32,
        "graph_replay": graph,
        "state_norms": state_norms,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def valu_issue(rec, ceiling, launch_ms: float, nbytes: int):
    """The dominant launch against its arithmetic floor: its VALU instruction
    count (from the profile of the same kernel sources) over the launch time,
    and the launch time at full issue of its hot loop's instruction mix priced
    at this run's probe rates (kinds without a probe form at the med3 rate)."""
    if not rec or not ceiling or "valu" not in ceiling:
        return None
    rates = {k: v["wave_instr_per_s"] for k, v in ceiling["valu"].items()}
    loop = rec["hot_loop_per_row_iteration"]
    per_row = sum(n / rates.get(k, rates["med3"]) for k, n in loop.items())
    rows = rec["waves_per_launch"] * rec["row_iterations_per_wave"]
    floor_s = rows * per_row + rec["waves_per_launch"] * rec["setup_per_wave"] / rates["med3"]
    t = launch_ms * 1e-3
    return {"instr_per_launch": rec["instr_per_launch"],
            "achieved_wave_instr_per_s": round(rec["instr_per_launch"] / t / 1e9, 2) * 1e9,
            "fmac_probe_wave_instr_per_s": rates.get("fmac"),
            "priced_floor_us": round(floor_s * 1e6, 1),
            "frac_of_priced_floor": round(floor_s / t, 4),
            "hbm_frac_at_floor": round(nbytes / floor_s / (PEAK_HBM_GBS * 1e9), 4)}


def measure_ceiling(dev, stream, gib: float, span_kib: int) -> dict:
    """Streaming rates of hand-written probes (include/lsq_probe.h) on this GPU:
    the best read, write and copy over a few launch shapes (one pass over the
    buffer, 16-byte vectors, 1-4 per lane, with and without the non-temporal
    hint), and the in-place span walk of the decode step's own access pattern
    (one wave per span of span_kib KiB).  Best of five launches each, HIP events
    on the launch stream; GB/s counts bytes read plus bytes written.  Also the
    VALU issue rate of fma, med3, a four-and-four mix and seven more single
    instruction kinds at four waves per SIMD (lsq_probe_valu), in wave64
    instructions per second."""
    import torch
    import quantized_recurrent_state_amd as lsq

    span = span_kib * 1024
    nbytes = int(gib * (1 << 30)) // span * span
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(7)

    def timed(fn, moved):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(5)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ms = min(a.elapsed_time(b) for a, b in ev)
        return round(moved / (ms * 1e-3) / 1e9, 1)

    out = {"bytes": nbytes, "method": "best of 5 launches per shape, HIP events on the launch stream"}
    kinds = {"read": (lsq.PROBE_READ, 1), "write": (lsq.PROBE_WRITE, 1), "copy": (lsq.PROBE_COPY, 2)}
    for name, (kind, mult) in kinds.items():
        best = None
        for u in (1, 2, 4):
            for nt in (0, 1):
                g = timed(lambda: lsq.lsq_probe_stream(kind, src, dst, nbytes, u, nt, 0, stream),
                          mult * nbytes)
                if best is None or g > best["gbs"]:
                    best = {"gbs": g, "loads_per_lane": u, "nontemporal": nt, "grid": "one pass"}
        out[name] = best
    best = None
    for nt in (0, 1):
        g = timed(lambda: lsq.lsq_probe_span(src, src, nbytes, span_kib, nt, stream), 2 * nbytes)
        if best is None or g > best["gbs"]:
            best = {"gbs": g, "span_kib": span_kib, "nontemporal_loads": nt}
    out["span_in_place"] = best
    del src, dst
    # VALU issue rates of one instruction form at four waves per SIMD (the
    # reference for an arithmetic-bound kernel): wave64 instructions per second
    sink = torch.zeros(4, device=dev)
    wg, iters = 1024, 8192
    for name, form in (("fma", lsq.PROBE_VALU_FMA), ("med3", lsq.PROBE_VALU_MED3),
                       ("mixed", lsq.PROBE_VALU_MIXED), ("fmac", lsq.PROBE_VALU_FMAC),
                       ("fma_mix", lsq.PROBE_VALU_FMA_MIX), ("lshl_or", lsq.PROBE_VALU_LSHL_OR),
                       ("perm", lsq.PROBE_VALU_PERM), ("xad", lsq.PROBE_VALU_XAD),
                       ("and", lsq.PROBE_VALU_AND), ("mul", lsq.PROBE_VALU_MUL)):
        run = lambda: lsq.lsq_probe_valu(form, wg, iters, sink, stream)
        run()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(5)]
        for a, b in ev:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        ms = min(a.elapsed_time(b) for a, b in ev)
        rate = wg * 4 * iters * 8 / (ms * 1e-3)
        out.setdefault("valu", {})[name] = {"wave_instr_per_s": round(rate / 1e9, 2) * 1e9,
                                            "per_cu_per_ns": round(rate / 256 / 1e9, 3)}
    log(f"ceiling probes: {out}")
    return out


PREFILL_SOURCES = ("quantized_recurrent_state_amd/csrc/lsq_prefill.hip",
                   "quantized_recurrent_state_amd/csrc/lsq_step_impl.h")
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA


def bench_prefill(args, wl, dev) -> int:
    """Chunkwise prefill: a "step" is one prefill of the workload's T-token
    prompt into every head's state (the state carries over between steps)."""
    import torch
    import quantized_recurrent_state_amd as lsq
    from quantized_recurrent_state_amd import runner
    from quantized_recurrent_state_amd.inputs import gen_steps

    K, W = args.steps, args.warmup
    stream = torch.cuda.current_stream()
    cfg = lsq.LsqConfig(**wl.config())
    st = lsq.LsqState(cfg, device=dev).zero()
    t_setup = time.perf_counter()
    d = gen_steps(wl.recipe, cfg.n, cfg.dk, cfg.dv, [0], 0, wl.tokens, device=dev)
    inp = [d[x] for x in ("k", "v", "alpha", "beta")]
    del d
    torch.cuda.synchronize()
    log(f"prefill {cfg} T={wl.tokens}: set-up {time.perf_counter() - t_setup:.1f} s")
    nbytes = runner.prefill_algorithmic_bytes(cfg, wl.tokens)
    ops = runner.prefill_int8_ops(cfg, wl.tokens)

    def launch():
        lsq.lsq_prefill(st.handle, wl.tokens, *inp, stream)

    for _ in range(W):
        launch()
    torch.cuda.synchronize()
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(K):
        ev_s[j].record(stream)
        launch()
        ev_e[j].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in zip(ev_s, ev_e)]
    kms = sum(kern_ms) / len(kern_ms)
    gbs = nbytes * K / wall / 1e9
    kgbs = nbytes / (kms * 1e-3) / 1e9
    log(f"timed {K} prefills: {wall * 1e3 / K:.3f} ms each, {gbs:.1f} GB/s; kernel {kms * 1e3:.1f} us")

    h = hashlib.sha256()
    for rel in PREFILL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()[:16]
    traffic = None
    tf = os.path.join(ROOT, "profiles", "traffic_prefill.json")
    if os.path.exists(tf):
        tr = json.load(open(tf))
        if tr.get("source_sha") == sha and tr.get("workload") == wl.name:
            traffic = int(tr["hbm_bytes_per_launch"])

    if args.copy_probe_gib > 0:          # counter calibration, outside the timed region
        nb = int(args.copy_probe_gib * (1 << 30)) // 256 * 256
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: one device copy of {nb} bytes (read {nb}, written {nb})")
        del src, dst

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline_prefill(wl, cfg, st, inp, args.cpu_seconds, nbytes)

    line = {
        "metric": "prefill HBM GB/s of inputs and state (% of peak) and tokens/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall * 1e3 / K, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8 products, f32 state pass", "data": "synthetic",
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(cfg.n * wl.tokens * K / wall, 1),
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "dk": wl.dk,
                   "dv": wl.dv, "tokens": wl.tokens, "chunk": 64, "bits": wl.bits,
                   "group": wl.group, "policy": wl.policy,
                   "decay": "diag" if wl.decay else "scalar", "bytes_per_step": nbytes,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "prefill_kernel", "algorithmic_bytes_per_launch": nbytes,
                     "launch_us_mean": round(kms * 1e3, 2),
                     "launch_us_min": round(min(kern_ms) * 1e3, 2), "source_sha": sha},
        "mfma": {"int8_ops_per_launch": ops, "achieved_tops": round(ops / (kms * 1e-3) / 1e12, 2),
                 "peak_tops": PEAK_INT8_TOPS,
                 "frac": round(ops / (kms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline_prefill(wl, cfg, st, inp, seconds: float, nbytes: int):
    """The CPU oracle's prefill on sampled heads (same inputs and start state as
    the GPU's last prefill), threads over heads, in the benchmark's unit."""
    import concurrent.futures as cf

    import numpy as np
    import torch
    import oracle
    from tests.parity import ocfg_of, snapshot

    threads, host_cores, _ = host_threads()
    n = cfg.n

    def sample(m):
        idx = np.linspace(0, n - 1, m).astype(np.int64)
        sel = torch.as_tensor(idx, device=st.device)
        s0 = snapshot(st, heads=sel)
        xs = [x.index_select(1, sel).cpu().numpy() for x in inp]
        return s0, xs

    def run(m):
        s0, xs = sample(m)
        parts = np.array_split(np.arange(m), threads)
        jobs = []
        for p in parts:
            if len(p) == 0:
                continue
            oc = ocfg_of(cfg).replace(batch=len(p), heads=1)
            s = s0.copy()
            s.codes, s.scales = s.codes[p].copy(), s.scales[p].copy()
            jobs.append((oc, s, [x[:, p].copy() for x in xs]))
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(len(jobs)) as ex:
            list(ex.map(lambda j: oracle.prefill(j[0], j[1], *j[2], chunk=64), jobs))
        return time.perf_counter() - t0

    dt1 = run(threads)
    m = int(max(threads, min(n, threads * round(seconds / max(dt1, 1e-3)))))
    dt = run(m)
    log(f"cpu oracle prefill: {m} sampled heads x {wl.tokens} tokens in {dt:.1f} s on {threads} threads")
    return {"value": round(nbytes * m / n / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "host_cores": host_cores, "kind": "oracle", "tokens_per_s": round(m * wl.tokens / dt, 1),
            "sample": f"{m} of {n} heads (evenly spaced) x the full {wl.tokens}-token prompt, "
                      f"from the GPU's state, on the same inputs"}


def host_threads() -> tuple[int, int, int]:
    """(threads the CPU baseline uses, host cores, cores this process may run on).
    The oracle runs one worker per available core up to 16, the CPU share of
    one GPU on the machines this benchmark targets."""
    host = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = host
    return max(1, min(16, avail)), host, avail


def cpu_baseline(arms, seconds: float, steps_avail: int):
    """Time the CPU oracle on every arm of the workload (same inputs and state as
    the GPU), scaled to the benchmark's unit: all heads and all the steps that
    fit the time budget when the workload is small, else evenly spaced heads;
    with every available worker thread and with one thread."""
    import numpy as np
    import oracle
    from quantized_recurrent_state_amd import runner
    from tests.parity import ocfg_of, snapshot

    threads, host_cores, avail = host_threads()
    per_arm = seconds / max(1, len(arms))

    def sample(a, m):
        n = a["cfg"].n
        idx = np.linspace(0, n - 1, m).astype(np.int64)
        sel = __import__("torch").as_tensor(idx, device=a["st"].device)
        st = snapshot(a["st"], heads=sel)
        t_now = a["st"].step_index
        ocfg = ocfg_of(a["cfg"], step=t_now).replace(batch=m, heads=1, lrb_rank=a["cfg"].lrb_rank)
        if ocfg.lrb_rank > 0:
            cin = (t_now & 1) if a["cfg"].decay else 0
            st.lrb_a = a["st"].lrb_a.index_select(0, sel).cpu().numpy().copy()
            st.lrb_b = a["st"].lrb_b[:, cin].index_select(0, sel).cpu().numpy().copy()
        return ocfg, st, sel

    def timed(a, ocfg, st, sel, steps, nthr):
        i = a["inp"]
        x = {k: i[k][:steps].index_select(1, sel).cpu().numpy() for k in i}
        s2 = st.copy()
        t0 = time.perf_counter()
        if ocfg.lrb_rank > 0:
            # the bypass oracle steps one call at a time: split the heads over
            # threads (the oracle releases the interpreter while it runs)
            import concurrent.futures as cf
            bounds = np.linspace(0, ocfg.n, nthr + 1).astype(np.int64)

            def part(lo, hi):
                sub = oracle.OracleState(codes=s2.codes[lo:hi], scales=s2.scales[lo:hi],
                                         lrb_a=s2.lrb_a[lo:hi], lrb_b=s2.lrb_b[lo:hi])
                c = ocfg.replace(batch=int(hi - lo))
                for t in range(steps):
                    oracle.step(c.replace(step=ocfg.step + t), sub, x["q"][t][lo:hi],
                                x["k"][t][lo:hi], x["v"][t][lo:hi], x["alpha"][t][lo:hi],
                                x["beta"][t][lo:hi])

            with cf.ThreadPoolExecutor(nthr) as ex:
                list(ex.map(lambda j: part(bounds[j], bounds[j + 1]), range(nthr)))
        else:
            oracle.run(ocfg, s2, x["q"], x["k"], x["v"], x["alpha"], x["beta"], nthreads=nthr)
        return time.perf_counter() - t0

    results, tot_b, tot_hs, tot_dt, tot_b1, tot_dt1 = [], 0, 0, 0.0, 0, 0.0
    for a in arms:
        n = a["cfg"].n
        bph = runner.algorithmic_bytes(a["cfg"]) // n          # bytes per head-step
        # the rate of one step on eight heads per thread sets the sample size
        ocfg, st, sel = sample(a, min(n, 8 * threads))
        dt0 = max(timed(a, ocfg, st, sel, 1, threads), 1e-4)
        per_hs = dt0 / ocfg.n * threads                        # seconds per head-step, one thread
        budget = per_arm * threads / per_hs                    # head-steps that fit the budget
        if n * steps_avail <= budget:
            m, steps = n, steps_avail                          # the whole workload as timed
        else:
            steps = int(max(1, min(steps_avail, budget // min(n, max(threads, n // 32)))))
            m = int(max(threads, min(n, budget // steps)))
        ocfg, st, sel = sample(a, m)
        dt = timed(a, ocfg, st, sel, steps, threads)
        # one thread on a share of the same sample (1/threads of the heads)
        m1 = max(1, m // threads)
        o1, s1, sel1 = sample(a, m1)
        dt1 = timed(a, o1, s1, sel1, steps, 1)
        results.append({"arm": a["arm"].name, "heads": m, "of_heads": n, "steps": steps,
                        "seconds": round(dt, 2), "seconds_one_thread": round(dt1, 2),
                        "gbs": round(bph * m * steps / dt / 1e9, 4),
                        "head_steps_per_s": round(m * steps / dt, 1),
                        "gbs_one_thread": round(bph * m1 * steps / dt1 / 1e9, 4),
                        "head_steps_per_s_one_thread": round(m1 * steps / dt1, 1)})
        tot_b += bph * m * steps
        tot_hs += m * steps
        tot_dt += dt
        tot_b1 += bph * m1 * steps
        tot_dt1 += dt1
        log(f"cpu oracle, {a['arm'].name}: {m} of {n} heads x {steps} steps in {dt:.1f} s on "
            f"{threads} threads; {m1} heads in {dt1:.1f} s on one thread")
    # rounding statistics of one oracle step (a whole merge period for the bypass)
    # on up to 64 heads of every arm: element-steps changed by directional
    # rounding, and clamped at qmax
    rates = []
    for a in arms:
        ocfg, st, sel = sample(a, min(a["cfg"].n, 64))
        nst = max(1, ocfg.lrb_rank)
        s2, fired, clamped = st.copy(), 0, 0
        for t in range(nst):
            x = {k: a["inp"][k][t].index_select(0, sel).cpu().numpy() for k in a["inp"]}
            stats = {}
            oracle.step(ocfg.replace(step=ocfg.step + t), s2, x["q"], x["k"], x["v"], x["alpha"],
                        x["beta"], stats=stats)
            fired += stats["bdr_fired"]
            clamped += stats["clamped"]
        ne = ocfg.n * ocfg.dv * ocfg.dk * nst
        rates.append({"arm": a["arm"].name, "steps": nst, "bdr_fired_rate": round(fired / ne, 5),
                      "clamp_rate": round(clamped / ne, 5)})
    # one teacher-forced parity step per arm, untimed and after everything else:
    # the GPU takes one more step from its current state and the oracle repeats
    # it from the same state and inputs on 64 evenly spaced heads; codes, stored
    # scales and outputs are compared bit for bit (tests.parity.compare_step)
    import torch
    import quantized_recurrent_state_amd as lsq
    from tests.parity import compare_step
    parity = []
    for a in arms:
        ocfg, before, sel = sample(a, min(a["cfg"].n, 64))
        i = a["inp"]
        lsq.lsq_decode_step(a["st"].handle, i["q"][0], i["k"][0], i["v"][0], i["alpha"][0],
                            i["beta"][0], a["o"], a["o_ref"], torch.cuda.current_stream())
        torch.cuda.synchronize()
        after = snapshot(a["st"], heads=sel)
        o_gpu = a["o"].index_select(0, sel).cpu().numpy()
        o_ref_gpu = None if a["o_ref"] is None else a["o_ref"].index_select(0, sel).cpu().numpy()
        x = tuple(i[k][0].index_select(0, sel).cpu().numpy() for k in ("q", "k", "v", "alpha", "beta"))
        rep = compare_step(ocfg, before, x, after, o_gpu, o_ref_gpu)
        parity.append({"arm": a["arm"].name, "heads": int(sel.numel()), "step": int(ocfg.step),
                       "codes": rep.codes, "codes_exact": rep.exact, "codes_failed": rep.failed,
                       "scales_differ": rep.scales_differ, "outputs": rep.outputs,
                       "outputs_differ": rep.o_differ, "bit_exact": bool(rep.ok)})
    log(f"parity sample: {parity}")
    whole = all(r["heads"] == r["of_heads"] and r["steps"] == steps_avail for r in results)
    return {"value": round(tot_b / tot_dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "host_cores": host_cores, "cores_available": avail, "kind": "oracle",
            "value_one_thread": round(tot_b1 / tot_dt1 / 1e9, 4),
            "head_steps_per_s": round(tot_hs / tot_dt, 1), "arms": results,
            "rounding_stats": rates, "parity": parity,
            "sample": ("the whole workload as the GPU timed it" if whole else
                       "evenly spaced heads of every arm x the steps sized to about "
                       f"{per_arm:.0f} s per arm (" +
                       ", ".join(f"{r['seconds']} s" for r in results) + " measured)") +
                      f"; from the GPU's state, on the same inputs; {threads} worker threads "
                      "(one per available core, at most 16), and one thread on 1/"
                      f"{threads} of the heads"}


if __name__ == "__main__":
    sys.exit(main())

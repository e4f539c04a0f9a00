#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

Default workload (the one the headline metric is quoted on): one layer of d=2048, f=768,
E=512 experts, top-10, 4-bit block-32 weights with fp16 scale+min, a T=4 speculative
verify window, Zipf(1.1)-biased router logits. One step = moe_route + the decode expert
FFN (int8 activation quantization, gate/up, SwiGLU, h quantization, down, combine) for
the window's 4 tokens. Steps rotate over several independently generated layer
instances so that consecutive steps read different experts and the 256 MB Infinity
Cache cannot serve the weights (each instance is 1.51 GB; the touched experts of one
step are ~63 MB).

Reported:
  value         expert-weight bytes streamed per second over whole steps (GB/s), with
                bytes counted from each step's actual routing: every distinct touched
                expert once, 3*f*d*(bits+1)/8 bytes;
  tokens_per_s  window tokens per second (4 per step);
  roofline      the dominant kernel (gate/up projections: 2/3 of the bytes) against the
                8 TB/s HBM peak, its average duration taken from HIP events around a run
                of that kernel alone, launched back to back over the rotating instances
                (each replaying its own step's gate/up stage);
  step_us_percentiles  p10 / p50 / p90 of event-bracketed steps;
  cache_variants (configs 2 and 3) p10 / p50 / p90 of event-bracketed steps with the
                layer instances in turn, with a 1 GiB scratch write ahead of every step
                (outside its events), and warm (one instance repeated);
  seed, source  the generator seed (0), a hash of the library sources and the git commit;
  cpu_baseline  the CPU oracle on the host, on a bounded sample of the same steps: on all
                physical cores the process may use (capped by OMP_NUM_THREADS), with the
                single-thread rate and the core counts beside it;
  supplementary (default run) the other configurations, each with its own roofline:
                1 = the tiny layer; 3 = 2-bit, 64 sequences x T (T=1 and 4), uniform
                logits; 4 = 48 chained layers, one decode step, eager and as one HIP
                graph, with bytes per token; 5 = the 8192-token prefill chunk (TFLOP/s).

Single configurations: --config 1..5 (3 with --T).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("expert-weight HBM GB/s (% of peak) and MoE-layer tokens/s, T=4 decode window")
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--T", type=int, default=4, help="window size for --config 3")
    ap.add_argument("--instances", type=int, default=0,
                    help="layer instances rotated over (default: 10 for config 2, 3 for 3)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="--config 4: skip the HIP-graph replay of the 48-layer step")
    ap.add_argument("--experts", type=int, default=512, choices=[512, 256],
                    help="experts per layer (256: the pruned Coder model, still top-10)")
    ap.add_argument("--router", action="store_true",
                    help="--config 2 or 4: each layer projects its own router logits from x "
                         "(bf16 router rows) instead of taking the workload's logits")
    ap.add_argument("--shared", action="store_true",
                    help="--config 2 or 4: layers with one always-active shared expert")
    ap.add_argument("--no-supplementary", action="store_true",
                    help="default run: only the headline configuration (no configs 1, 3, 4, 5)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device-to-device copy of MIB MiB (the reference "
                         "dispatch that scales hardware byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Step:
    """Pre-built C structs of one layer instance, so the timed loop only makes C calls.
    One step is moe_layer_decode: routing fused into the first kernel, then the expert FFN."""

    def __init__(self, q, layer, lg, x, res, routing, ws):
        self.q = q
        self.layer_obj = layer  # owns the weight tensors layer_s points to
        self.layer_s = layer._struct()
        self.rout_s = routing._struct()
        self.routing = routing
        self.lg, self.x, self.res, self.ws = lg, x, res, ws
        self.n, self.E = x.shape[0], layer.n_experts
        self.k = layer.top_k
        # no logits: the layer projects them from x with its router rows
        self.lg_ptr = None if lg is None else lg.data_ptr()

    def layer(self, stream, stages):
        rc = self.q.lib.moe_layer_decode_stages(
            ctypes.byref(self.layer_s), self.lg_ptr, self.x.data_ptr(), self.n,
            ctypes.byref(self.rout_s), self.res.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
            None, stages, stream)
        assert rc == 0, rc

    def full(self, stream):
        self.layer(stream, self.q.DECODE_ALL)

    def gate_up(self, stream):
        self.layer(stream, self.q.DECODE_GATE_UP)

    def stages(self):
        q = self.q
        return [("route_prep", lambda sh: self.layer(sh, q.DECODE_PREP)),
                ("gate_up", lambda sh: self.layer(sh, q.DECODE_GATE_UP)),
                ("down_combine", lambda sh: self.layer(sh, q.DECODE_DOWN | q.DECODE_COMBINE))]


def sleep_cycles_for(torch, seconds):
    """Spin-kernel length covering `seconds` of host enqueue time (calibrated)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 2_000_000
    torch.cuda.synchronize()
    s.record()
    torch.cuda._sleep(n)
    e.record()
    torch.cuda.synchronize()
    per_cycle = max(s.elapsed_time(e) * 1e-3 / n, 1e-12)
    return int(seconds / per_cycle)


def timed_region(torch, steps, order, instrument, enqueue_estimate, call="full"):
    """Run the steps back to back on the GPU: a spin kernel holds the queue while the host
    enqueues every step, so host launch cost does not open gaps between kernels. With
    `instrument`, HIP events on the launch stream bracket each stage of every step;
    otherwise each step runs its `call` method (the whole step by default).
    Returns (total_ms, {stage label: per-step ms list} or None, host seconds, covered)."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if instrument == "step":  # one event pair per whole step
        plans = [[("step", steps[i].full)] for i in order]
    else:
        plans = [steps[i].stages() for i in order] if instrument else None
    evs = None
    if instrument:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(p) + 1)] for p in plans]
    cycles = sleep_cycles_for(torch, max(0.02, 2.0 * enqueue_estimate))
    torch.cuda.synchronize()
    torch.cuda._sleep(cycles)
    start.record()
    t0 = time.perf_counter()
    for s_idx, i in enumerate(order):
        if instrument:
            ev = evs[s_idx]
            ev[0].record()
            for j, (_, fn) in enumerate(plans[s_idx]):
                fn(sh)
                ev[j + 1].record()
        else:
            getattr(steps[i], call)(sh)
    end.record()
    host_s = time.perf_counter() - t0
    covered = not start.query()  # the spin kernel still ran when the last step was queued
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    stages = None
    if instrument:
        labels = [lab for lab, _ in plans[0]]
        stages = {lab: [ev[j].elapsed_time(ev[j + 1]) for ev in evs]
                  for j, lab in enumerate(labels)}
    return total_ms, stages, host_s, covered


def percentiles(ms_list):
    """p10 / p50 / p90 of per-step times given in ms, reported in us."""
    import numpy as np

    a = np.asarray(ms_list, np.float64) * 1e3
    return {"p10": round(float(np.percentile(a, 10)), 2),
            "p50": round(float(np.percentile(a, 50)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "steps": int(a.size),
            "how": "HIP events around every step on the launch stream (about 1 us each)"}


def event_steps(torch, steps, order, enqueue_estimate, before=None):
    """Per-step GPU times (ms) of steps[i].full for i in order, one event pair around each
    step only. `before(stream)`, if given, is enqueued ahead of each step's first event, so
    its work is not in the measured span. A spin kernel holds the queue while the host
    enqueues everything."""
    sh = torch.cuda.current_stream().cuda_stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in order]
    cycles = sleep_cycles_for(torch, max(0.02, 2.0 * enqueue_estimate))
    torch.cuda.synchronize()
    torch.cuda._sleep(cycles)
    for (e0, e1), i in zip(evs, order):
        if before is not None:
            before(sh)
        e0.record()
        steps[i].full(sh)
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def source_ids():
    """What the timed kernels were built from: a hash of the library sources (the C ABI
    header and every HIP source and header of the package), and the git commit when the
    tree is a checkout (null otherwise)."""
    import glob
    import hashlib
    import subprocess

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_routed_expert_router_amd", "csrc")
    files = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")) +
                   glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    sha = None
    try:
        res = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10)
        sha = res.stdout.strip() if res.returncode == 0 and res.stdout.strip() else None
    except (OSError, subprocess.SubprocessError):
        sha = None
    return {"library_sources_sha256_16": h.hexdigest()[:16], "git_sha": sha}


def touched_experts(routing) -> int:
    off = routing.expert_offsets.cpu()
    return int(((off[1:] - off[:-1]) > 0).sum())


def host_cores():
    """Logical CPUs, the CPUs this process may run on, and the physical cores among them
    (distinct (package, core) pairs from sysfs)."""
    logical = os.cpu_count() or 1
    allowed = sorted(os.sched_getaffinity(0))
    phys = set()
    for c in allowed:
        base = f"/sys/devices/system/cpu/cpu{c}/topology/"
        try:
            core = open(base + "core_id").read().strip()
            pkg = open(base + "physical_package_id").read().strip()
            phys.add((pkg, core))
        except OSError:
            phys.add(("?", str(c)))
    return logical, len(allowed), len(phys)


def _oracle_rate(w, instances_inputs, seconds, nthreads):
    """The oracle (as it stands) on `nthreads` host threads over config steps until about
    `seconds` of oracle time; returns (GB/s, tokens/s, steps, seconds, instances)."""
    import numpy as np

    from oracle import oracle as O
    from quantized_routed_expert_router_amd import synth

    total_t, total_b, steps = 0.0, 0, 0
    host_layers = {}
    i = 0
    while total_t < seconds and steps < 10_000:
        idx = i % len(instances_inputs)
        lg, x = instances_inputs[idx]
        ids_pre = np.argsort(-lg, axis=1, kind="stable")[:, :w.k]
        if idx not in host_layers:
            host_layers[idx] = synth.host_layer(w, idx, experts=np.unique(ids_pre))
        g, u, dn = host_layers[idx]
        om = lambda h: O.Matrix(h.codes, h.scale_min, h.rows, h.cols, h.bits)  # noqa: E731
        t0 = time.perf_counter()
        ids, wt = O.route(lg, w.k)
        O.group(ids, w.E)
        O.ffn_decode(om(g), om(u), om(dn), w.E, x, ids, wt, x, nthreads=nthreads)
        total_t += time.perf_counter() - t0
        total_b += len(np.unique(ids)) * synth.expert_bytes(w.d, w.f, w.bits)
        steps += 1
        i += 1
    return (total_b / total_t / 1e9, steps * w.n / total_t, steps, total_t,
            min(steps, len(instances_inputs)))


def cpu_baseline(w, instances_inputs, seconds):
    """The oracle on one host thread and on all physical cores this process may use
    (capped by OMP_NUM_THREADS, the machine's CPU share), each for about seconds/2."""
    from oracle import oracle as O

    logical, allowed, physical = host_cores()
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    all_threads = max(1, min(physical, cap) if cap > 0 else physical)
    gb1, tok1, st1, t1, _ = _oracle_rate(w, instances_inputs, seconds / 2, 1)
    gbn, tokn, stn, tn, inst = _oracle_rate(w, instances_inputs, seconds / 2, all_threads)
    used = O.threads(all_threads)
    return dict(value=round(gbn, 4), unit="GB/s", cores=used, kind="oracle",
                sample=f"{stn} steps of the same workload (route + decode layer, {w.n} tokens "
                       f"each) over {inst} layer instances, {tn:.1f} s of oracle time on "
                       f"{used} threads; and {st1} steps, {t1:.1f} s on 1 thread",
                tokens_per_s=round(tokn, 3),
                single_thread={"value": round(gb1, 4), "unit": "GB/s",
                               "tokens_per_s": round(tok1, 3), "steps": st1},
                host={"logical_cpus": logical, "cpus_allowed": allowed,
                      "physical_cores_allowed": physical, "omp_num_threads_cap": cap or None})


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_t4_k_gateup_traffic.md")


def measured_traffic(profile_path):
    """Calibrated HBM bytes per launch from a committed counter summary, or None when any
    source the kernel is built from has changed since the counters were taken."""
    import hashlib
    import re

    if not os.path.exists(profile_path):
        return None
    text = open(profile_path).read()
    srcs = re.findall(r"^kernel_source: (\S+)$", text, re.M)
    shas = re.findall(r"^kernel_source_sha256: ([0-9a-f]{64})$", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    if not (srcs and len(srcs) == len(shas) and val):
        return None
    for src, sha in zip(srcs, shas):
        path = os.path.join(ROOT, src)
        if not os.path.exists(path):
            return None
        if hashlib.sha256(open(path, "rb").read()).hexdigest() != sha:
            return None
    return int(val.group(1))


def bench_decode(args, torch, q, synth, workloads):
    import numpy as np

    w = synth.config(args.config, args.T, None if args.config == 1 else args.experts)
    shared = args.shared and args.config == 2
    router = args.router and args.config == 2
    if shared:
        w.name += "_shared1"
    if router:
        w.name += "_router"
    # the headline line: configuration 2 as the workload defines it
    primary = args.config == 2 and not shared and not router and args.experts == 512
    L = args.instances or {1: 4, 2: 10}.get(args.config, 3)
    log(f"workload {w.name}: generating {L} layer instances on the GPU")
    t0 = time.perf_counter()
    steps, inputs = [], []
    for i in range(L):
        # one workspace per instance: stages can be replayed
        ws = q.workspace(_shape_layer(q, w, shared, router), w.n)
        layer = workloads.device_layer(w, i, shared=shared, router=router)
        lg, x = synth.layer_inputs(w, i)
        inputs.append((lg, x))
        lg_d = None if router else torch.from_numpy(lg).cuda()
        x_d = torch.from_numpy(x).cuda()
        routing = q.Routing.empty(w.n, w.E, w.k)
        steps.append(Step(q, layer, lg_d, x_d, x_d.clone(), routing, ws))
    torch.cuda.synchronize()
    log(f"generated {L} x {3 * w.E * synth.expert_bytes(w.d, w.f, w.bits) // 3 / 1e9:.2f} GB "
        f"in {time.perf_counter() - t0:.1f} s")

    # routing of each instance (fixed per instance): bytes per step
    sh = torch.cuda.current_stream().cuda_stream
    for st in steps:
        st.full(sh)  # routing of each instance is fixed: bytes per step
    torch.cuda.synchronize()
    ebytes = synth.expert_bytes(w.d, w.f, w.bits)
    # the shared expert is read once per step like a touched routed expert
    touched = [touched_experts(st.routing) + (1 if shared else 0) for st in steps]
    step_bytes = [t * ebytes for t in touched]
    gu_bytes = [t * ebytes * 2 // 3 for t in touched]

    warm = [s % L for s in range(args.warmup)]
    order = [s % L for s in range(args.steps)]
    # warmup (also estimates the host enqueue time per step)
    _, _, host_s, _ = timed_region(torch, steps, warm or [0], False, 0.05)
    est = host_s / max(1, len(warm)) * len(order)
    total_ms, _, host_s, covered = timed_region(torch, steps, order, False, est)
    inst_ms, stage_ms, _, covered_i = timed_region(torch, steps, order, True, est * 2)
    # per-step times, one event pair around each step (the events add about 1 us a step)
    _, step_ms, _, _ = timed_region(torch, steps, order, "step", est * 2)
    # the dominant kernel alone: gate/up launches back to back, rotating over the instances
    # (each replays its own step's gate/up stage on that step's workspace)
    gu_ms, _, _, covered_g = timed_region(torch, steps, order, False, est, call="gate_up")
    if not (covered and covered_i and covered_g):
        log("warning: the host enqueue outlasted the spin kernel; gaps may be included")
    variants = None
    if args.config in (2, 3):
        # cache variants: a 1 GiB scratch write ahead of every step (outside its events),
        # and one instance repeated (its touched experts stay in the 256 MB memory-side
        # cache: the warm number)
        K = min(len(order), 100)
        per = est / max(1, len(order))
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fl_ms = event_steps(torch, steps, order[:K], 3.0 * per * K,
                            before=lambda sh_: scratch.fill_(1))
        del scratch
        wm_ms = event_steps(torch, steps, [0] * K, 2.0 * per * K)

        def _variant(ms, idx, how):
            p = percentiles(ms)
            p["how"] = how
            p["value_GBs_at_p50"] = round(
                float(np.mean([step_bytes[i] for i in idx])) / (p["p50"] * 1e-6) / 1e9, 1)
            return p

        variants = {
            "rotate_instances": _variant(step_ms["step"], order,
                                         f"{L} layer instances in turn (the timed value's "
                                         "workload), an event pair around each step"),
            "flush_1GiB": _variant(fl_ms, order[:K], "instances in turn, a 1 GiB scratch "
                                   "write before each step, outside its event pair"),
            "warm_one_instance": _variant(wm_ms, [0] * K, "one instance repeated: its "
                                          "touched experts stay in the memory-side cache"),
        }

    sec = total_ms * 1e-3
    tot_bytes = sum(step_bytes[i] for i in order)
    value = tot_bytes / sec / 1e9
    tok_s = len(order) * w.n / sec
    gu_sec = gu_ms * 1e-3
    gu_ach = sum(gu_bytes[i] for i in order) / gu_sec / 1e9
    stage_us = {lab: round(float(np.mean(v)) * 1e3, 2) for lab, v in stage_ms.items()}
    stage_us["instrumented_step"] = round(inst_ms / len(order) * 1e3, 2)
    stage_us["gate_up_back_to_back"] = round(gu_ms / len(order) * 1e3, 2)
    mean_touched = float(np.mean([touched[i] for i in order]))
    rec = {
        "metric": METRIC if primary else f"{METRIC} [supplementary: {w.name}]",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / len(order), 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "d_model": w.d, "d_ff": w.f, "experts": w.E,
                   "top_k": w.k, "tokens_per_step": w.n, "weight_bits": w.bits,
                   "layer_instances": L, "shared_expert": shared, "router_projection": router,
                   "step": "moe_layer_decode (routing + expert FFN: x quant, gate/up, SwiGLU, "
                           "h quant, down, combine)"},
        "tokens_per_s": round(tok_s, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "expert_bytes_per_step": round(float(np.mean([step_bytes[i] for i in order])), 1),
        "touched_experts_per_step": round(mean_touched, 2),
        "stage_us": stage_us,
        "step_us_percentiles": percentiles(step_ms["step"]),
        "cache_variants": variants,
        "roofline": {"bound": "hbm", "kernel": "k_gateup (gate/up + SwiGLU)",
                     "achieved": round(gu_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_ach / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(TRAFFIC_PROFILE) if primary else None,
                     "bytes_per_launch": round(float(np.mean([gu_bytes[i] for i in order])), 1)},
    }
    if primary and not args.no_cpu_baseline:
        log("CPU oracle baseline ...")
        rec["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    return rec


def _shape_layer(q, w, shared=False, router=False):
    """A layer description with the right sizes for workspace queries (no weights)."""
    import torch

    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    dummy16 = torch.empty(16, dtype=torch.int16, device="cuda")
    mk = lambda r, c: q.QMatrix(dummy, dummy16, r, c, w.bits)  # noqa: E731
    sh = (mk(w.f, w.d), mk(w.f, w.d), mk(w.d, w.f)) if shared else None
    rt = torch.empty((w.E, w.d), dtype=torch.int16, device="cuda") if router else None
    return q.Layer(w.d, w.f, w.E, w.k, mk(w.f, w.d), mk(w.f, w.d), mk(w.d, w.f), sh, rt)


def bench_chain(args, torch, q, synth, workloads):
    import numpy as np

    w = synth.config(4, experts=args.experts)
    shared, router = args.shared, args.router
    if shared:
        w.name += "_shared1"
    if router:
        w.name += "_router"
    log(f"workload {w.name}: generating {w.layers} layers on the GPU")
    t0 = time.perf_counter()
    ws = q.workspace(_shape_layer(q, w, shared, router), w.n)
    x0 = torch.from_numpy(synth.activations(w.seed, 0, w.n, w.d)).cuda()
    res = x0.clone()
    steps = []
    for l_ in range(w.layers):
        layer = workloads.device_layer(w, l_, shared=shared, router=router)
        lg = (None if router else
              torch.from_numpy(synth.logits(w.seed, l_, w.n, w.E, w.logits)).cuda())
        routing = q.Routing.empty(w.n, w.E, w.k)
        steps.append(Step(q, layer, lg, res, res, routing, ws))  # x is the residual stream
    torch.cuda.synchronize()
    log(f"generated in {time.perf_counter() - t0:.1f} s")
    sh = torch.cuda.current_stream().cuda_stream
    for st in steps:
        st.full(sh)
    torch.cuda.synchronize()
    ebytes = synth.expert_bytes(w.d, w.f, w.bits)
    touched = [touched_experts(st.routing) + (1 if shared else 0) for st in steps]
    chain_bytes = sum(touched) * ebytes
    order = list(range(w.layers)) * max(1, args.steps // w.layers)
    _, _, host_s, _ = timed_region(torch, steps, list(range(w.layers)), False, 0.1)
    est = host_s * len(order) / w.layers
    total_ms, _, _, covered = timed_region(torch, steps, order, False, est)
    n_chain = len(order) // w.layers
    sec = total_ms * 1e-3
    value = chain_bytes * n_chain / sec / 1e9
    per_layer = 4 if router else 3  # (router projection,) route+prep, gate/up, down+combine
    graph = (None if args.no_graph else
             chain_graph(torch, steps, n_chain, chain_bytes, w, per_layer))
    return {
        "metric": f"{METRIC} [supplementary: {w.name}]", "value": round(value, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": n_chain, "warmup": 1, "ms_per_step": round(total_ms / n_chain, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "tokens_per_step": w.n,
                   "shared_expert": shared, "router_projection": router,
                   "step": "48 x moe_layer_decode, residual chained"},
        "tokens_per_s": round(n_chain * w.n / sec, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "expert_bytes_per_step": chain_bytes,
        "expert_bytes_per_token": chain_bytes / w.n,
        "pages_bytes_per_token": 663.6e6,
        "touched_experts_per_layer": round(float(np.mean(touched)), 2),
        "enqueue_covered": covered,
        "graph": graph,
        "roofline": {"bound": "hbm", "kernel": "whole 48-layer step",
                     "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4)},
    }


def chain_graph(torch, steps, replays, chain_bytes, w, per_layer=3):
    """The 48-layer step captured once as a HIP graph (3 or 4 launches per layer) and replayed
    back to back: no host launch cost per layer and no spin kernel needed. The launches
    use no memset and no allocation, so the captured step is the eager one."""
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        sh = torch.cuda.current_stream().cuda_stream
        for st in steps:
            st.full(sh)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / replays
    return {"ms_per_step": round(ms, 4), "value_GBs": round(chain_bytes / (ms * 1e-3) / 1e9, 2),
            "tokens_per_s": round(w.n / (ms * 1e-3), 1), "replays": replays,
            "kernels_per_step": per_layer * len(steps)}


class PrefillStep:
    """Pre-built C structs of one prefill-chunk instance."""

    def __init__(self, q, layer, lg, xb, res, routing, ws):
        self.q = q
        self.layer_obj = layer  # owns the weight tensors layer_s points to
        self.layer_s = layer._struct()
        self.rout_s = routing._struct()
        self.routing = routing
        self.lg, self.xb, self.res, self.ws = lg, xb, res, ws
        self.n, self.E = lg.shape
        self.k = layer.top_k
        self.route_ws = q.route_workspace(self.n, self.E, self.k)

    def route(self, stream):
        rws = self.route_ws
        rc = self.q.lib.moe_route(self.lg.data_ptr(), self.n, self.E, self.k,
                                  ctypes.byref(self.rout_s), None if rws is None else rws.data_ptr(),
                                  0 if rws is None else rws.numel(), stream)
        assert rc == 0, rc

    def prefill(self, stream, stages):
        rc = self.q.lib.moe_expert_ffn_prefill_stages(
            ctypes.byref(self.layer_s), self.xb.data_ptr(), self.n, ctypes.byref(self.rout_s),
            self.res.data_ptr(), self.ws.data_ptr(), self.ws.numel(), stages, stream)
        assert rc == 0, rc

    def full(self, stream):
        self.route(stream)
        self.prefill(stream, self.q.PREFILL_ALL)

    def gate_up(self, stream):
        self.prefill(stream, self.q.PREFILL_GATE_UP)

    def stages(self):
        q = self.q
        return [("route", self.route),
                ("prep", lambda sh: self.prefill(sh, q.PREFILL_PREP)),
                ("gate_up", lambda sh: self.prefill(sh, q.PREFILL_GATE_UP)),
                ("down", lambda sh: self.prefill(sh, q.PREFILL_DOWN)),
                ("combine", lambda sh: self.prefill(sh, q.PREFILL_COMBINE))]


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, AMD published


def bench_prefill(args, torch, q, synth, workloads):
    """8192-token prefill chunk: route + bf16 matrix-core expert FFN per step."""
    import numpy as np

    w = synth.config(5, experts=args.experts)
    L = args.instances or 2
    log(f"workload {w.name}: generating {L} layer instances on the GPU")
    steps = []
    for i in range(L):
        # one workspace per instance, so that a stage can be replayed on its own
        ws = q.workspace(_shape_layer(q, w), w.n, prefill=True)
        layer = workloads.device_layer(w, i)
        lg, x = synth.layer_inputs(w, i)
        lg_d = torch.from_numpy(lg).cuda()
        xb = torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).cuda()
        res = torch.from_numpy(x).cuda()
        steps.append(PrefillStep(q, layer, lg_d, xb, res, q.Routing.empty(w.n, w.E, w.k), ws))
    torch.cuda.synchronize()
    P = w.n * w.k
    flop_gu = 4.0 * P * w.f * w.d  # gate and up: 2 flops per multiply-add each
    flop_dn = 2.0 * P * w.d * w.f
    warm = [s % L for s in range(args.warmup)]
    order = [s % L for s in range(args.steps)]
    for st in steps:
        st.route(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    _, _, host_s, _ = timed_region(torch, steps, warm or [0], False, 0.05)
    est = host_s / max(1, len(warm)) * len(order)
    total_ms, _, _, covered = timed_region(torch, steps, order, False, est)
    inst_ms, stage_ms, _, covered_i = timed_region(torch, steps, order, True, est * 2)
    # the dominant kernel alone, back to back over the instances (each on its own workspace)
    gu_ms, _, _, covered_g = timed_region(torch, steps, order, False, est, call="gate_up")
    stage_us = {lab: round(float(np.mean(v)) * 1e3, 2) for lab, v in stage_ms.items()}
    stage_us["instrumented_step"] = round(inst_ms / len(order) * 1e3, 2)
    stage_us["gate_up_back_to_back"] = round(gu_ms / len(order) * 1e3, 2)
    sec = total_ms * 1e-3
    gu_tflops = flop_gu / (gu_ms / len(order) * 1e-3) / 1e12
    dn_tflops = flop_dn / (stage_us["down"] * 1e-6) / 1e12
    layer_tflops = (flop_gu + flop_dn) * len(order) / sec / 1e12
    touched = [touched_experts(st.routing) for st in steps]
    ebytes = synth.expert_bytes(w.d, w.f, w.bits)
    return {
        "metric": f"{METRIC} [supplementary: {w.name}]",
        "value": round(len(order) * w.n / sec, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms / len(order), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "d_model": w.d, "d_ff": w.f, "experts": w.E,
                   "top_k": w.k, "tokens_per_step": w.n, "weight_bits": w.bits,
                   "layer_instances": L, "step": "moe_route + moe_expert_ffn_prefill"},
        "layer_tflops": round(layer_tflops, 1),
        "expert_gbs": round(float(np.mean(touched)) * ebytes * len(order) / sec / 1e9, 1),
        "stage_us": stage_us,
        "down_tflops": round(dn_tflops, 1),
        "roofline": {"bound": "mfma", "kernel": "k_pf_gateup (gate/up GEMM + SwiGLU)",
                     "achieved": round(gu_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gu_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flop_per_launch": flop_gu},
        "enqueue_covered": bool(covered and covered_i and covered_g),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the routed-expert layer on exactly one MI355X; rerun with "
              "--gpus 1.", file=sys.stderr)
        sys.exit(2)
    source = source_ids()  # before the GPU is touched (it may start git)
    import torch

    from quantized_routed_expert_router_amd import qmoe as q
    from quantized_routed_expert_router_amd import synth, workloads

    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {nbytes} bytes read, {nbytes} bytes written")
        del src, dst
    if args.config in (1, 2, 3):
        rec = bench_decode(args, torch, q, synth, workloads)
    elif args.config == 4:
        rec = bench_chain(args, torch, q, synth, workloads)
    else:
        rec = bench_prefill(args, torch, q, synth, workloads)
    rec["seed"] = 0
    rec["source"] = source
    headline = (args.config == 2 and not args.shared and not args.router
                and args.experts == 512 and not args.instances)
    if headline and not args.no_supplementary:
        rec["supplementary"] = supplementary(args, torch, q, synth, workloads)
    print(json.dumps(rec), flush=True)


def _summary(r):
    """The figures of one supplementary record that the headline line carries."""
    keep = ("value", "unit", "ms_per_step", "tokens_per_s", "pct_of_hbm_peak",
            "expert_bytes_per_step", "expert_bytes_per_token", "touched_experts_per_step",
            "layer_tflops", "stage_us", "step_us_percentiles", "cache_variants", "graph",
            "steps")
    out = {k: r[k] for k in keep if k in r}
    out["workload"] = r["config"]["workload"]
    if r.get("roofline"):
        rf = r["roofline"]
        out["roofline"] = {k: rf[k] for k in ("bound", "kernel", "achieved", "peak", "unit",
                                              "frac")}
    return out


def supplementary(args, torch, q, synth, workloads):
    """Configurations 1, 3 (T = 1 and 4), 4 (eager and one HIP graph) and 5 in the same
    run, each on its own freshly generated layers, with fewer steps than the headline."""
    import gc

    plans = [("cfg1_tiny", dict(config=1, steps=200, warmup=20)),
             ("cfg3_2bit_b64xt1", dict(config=3, T=1, steps=60, warmup=6)),
             ("cfg3_2bit_b64xt4", dict(config=3, T=4, steps=60, warmup=6)),
             ("cfg4_chain48", dict(config=4, steps=480, warmup=1)),
             ("cfg5_prefill8192", dict(config=5, steps=10, warmup=2))]
    out = {}
    for name, over in plans:
        a = argparse.Namespace(**vars(args))
        a.instances = 0
        a.no_cpu_baseline = True
        for k_, v in over.items():
            setattr(a, k_, v)
        log(f"supplementary {name}")
        if a.config in (1, 3):
            r = bench_decode(a, torch, q, synth, workloads)
        elif a.config == 4:
            r = bench_chain(a, torch, q, synth, workloads)
        else:
            r = bench_prefill(a, torch, q, synth, workloads)
        out[name] = _summary(r)
        del r
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()

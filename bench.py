#!/usr/bin/env python3
"""Throughput of the MoE layer (256 experts, top-8, gated shared expert) on one MI355X.

A step is one moe_forward call (router, top-K, dispatch, both expert GEMMs,
shared expert, combine) over one batch of seeded synthetic tokens, with the
inputs already resident in HBM.  Steps rotate over several independently drawn
layers so that weights are not served from the 256 MB Infinity Cache across
steps (8 layers at T = 1, 2 otherwise).

    python bench.py                        # the default line: every workload
    python bench.py --workload prefill4096 --steps 50 --warmup 5   # one workload

The default line's headline (`value`, `ms_per_step`, `roofline`) is the 1-token
decode, timed over exactly --steps steps after --warmup untimed ones; the
batched decode (64 tokens), the 4096-token prefill and the skewed 16384-token
prefill are measured in the same run (their own step counts) under
`workloads`, each with its roofline and a CPU-oracle baseline.  Prints one JSON
line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

# workload -> (steps, warmup, layers rotated).  The warm-up is ~0.1-0.2 s of
# steps: shorter ones leave the GPU below its working clock for part of the
# timed region (prefill4096 measured 8 % slower after 5 warm-up steps than
# after 200).
DEFAULTS = {
    "decode1": (2000, 5000, 8),
    "decode64": (200, 500, 2),
    "prefill4096": (50, 300, 2),
    "zipf16384": (20, 100, 2),
}
HEADLINE = "decode1"
SUB_WORKLOADS = ("decode64", "prefill4096", "zipf16384")
# Workloads whose dominant kernel is priced against the MFMA peak (arithmetic
# intensity above the ridge of 2.5 PFLOP/s / 8 TB/s).
MFMA_BOUND = ("zipf16384",)
REPEATS = 5
# Seconds of oracle work per timed repeat of the CPU baseline (3 repeats).
CPU_REPEAT_S = {"decode1": 5.0, "decode64": 3.0, "prefill4096": 3.0, "zipf16384": 3.0}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None, choices=sorted(DEFAULTS),
                    help="measure only this workload (default: the headline plus every other workload)")
    ap.add_argument("--layers", type=int, default=None, help="weight sets rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-major", action="store_true",
                    help="keep the routed experts row-major instead of the MFMA-tile layout")
    ap.add_argument("--cpu-scale", type=float, default=1.0, help="scales the oracle's timed sample")
    ap.add_argument("--layer-only", action="store_true",
                    help="skip the other entry points' timings (load balance, sub-block, bf16 scores, streamed "
                         "experts), so that a kernel trace holds the layer's own launches")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="only time moe_forward at batch sizes 1..64 (the full-shape layer, 8 layers rotated) and "
                         "print one JSON line per size")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Probes and host facts.
# ---------------------------------------------------------------------------

def copy_probe():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: 5 copies of {n} bytes ({n // 1024} KiB read and written per copy)")
    print(json.dumps({"copy_probe_bytes": n}))


def ceiling_probes():
    """Practical ceilings on this GPU, context for the roofline fractions: a
    plain 1 GiB device copy (bytes read + written per second) and a large
    dense bf16 matmul through torch (flops per second)."""
    import torch
    out = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        dst.copy_(src)
    s.record()
    for _ in range(10):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    out["copy_1GiB_GBps"] = round(2 * n * 10 / (s.elapsed_time(e) * 1e-3) / 1e9, 1)
    del src, dst
    m = 8192
    a = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    b = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    for _ in range(3):
        a @ b
    s.record()
    for _ in range(10):
        a @ b
    e.record()
    torch.cuda.synchronize()
    out["bf16_gemm_8192_TFLOPs"] = round(2 * m ** 3 * 10 / (s.elapsed_time(e) * 1e-3) / 1e12, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def gpu_clock():
    """Shader clock levels from rocm-smi: the highest level (MHz) and the level
    current when queried (after the runs: the idle clock).  None if the tool
    is unavailable or prints an unexpected format."""
    import re
    try:
        r = subprocess.run(["rocm-smi", "--showclkfrq", "--json"], capture_output=True, text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        text = " ".join(str(v) for k, v in card.items() if "sclk" in k.lower())
        levels = [int(m) for m in re.findall(r"(\d+)\s*Mhz", text, flags=re.I)]
        cur = re.search(r"(\d+)\s*Mhz\s*\*", text, flags=re.I)
        return {"max_level_mhz": max(levels) if levels else None,
                "current_when_queried_mhz": int(cur.group(1)) if cur else None} if levels else None
    except Exception:  # noqa: BLE001 (a missing tool or an unexpected format)
        return None


def host_facts():
    facts = {"cpu_model": None, "blas": None}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                facts["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            facts["blas"] = {"library": blas[0].get("internal_api"), "version": blas[0].get("version"),
                             "threads": blas[0].get("num_threads")}
    except Exception:  # noqa: BLE001
        pass
    return facts


# ---------------------------------------------------------------------------
# Inputs.
# ---------------------------------------------------------------------------

def device_layer(moe, mi, wl, l, base_bits):
    """Layer l of the rotation: layer 0 from the seeded CPU generator, the others
    drawn on the device (torch generator seeded layer_seed*100 + l)."""
    import torch
    d = wl.dims
    if l == 0:
        bits = dict(base_bits)
        if wl.skewed_router:
            bits["gate.weight"] = mi.make_router(d, wl.layer_seed, mi.zipf_router_gain())
        return moe.MoeLayer.from_bf16_bits(bits, d.H, d.E, d.K, d.I, d.Is, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.layer_seed * 100 + l)
    params = {}
    for name, shape in d.shapes().items():
        t = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).mul_(mi.WEIGHT_STD)
        if name == "gate.weight" and wl.skewed_router:
            t.mul_(torch.tensor(mi.zipf_router_gain(), device="cuda", dtype=torch.float32).view(-1, 1))
        params[name] = t.to(torch.bfloat16).contiguous()
        del t
    return moe.MoeLayer(d.H, d.E, d.K, d.I, d.Is, params)


def layer0_bits(mi, wl, base_bits):
    bits = dict(base_bits)
    if wl.skewed_router:
        bits["gate.weight"] = mi.make_router(wl.dims, wl.layer_seed, mi.zipf_router_gain())
    return bits


def device_x(moe, mi, wl, l):
    import torch
    if l == 0:
        return moe.bits_to_device(mi.workload_x(wl), "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.x_seed * 100 + l)
    return (torch.randn((wl.T, wl.dims.H), generator=g, device="cuda") * wl.x_std).to(torch.bfloat16)


# ---------------------------------------------------------------------------
# Work model.
# ---------------------------------------------------------------------------

def phase_work(d, T, U, phase):
    """Algorithmic (bytes, flops) of one launch of a phase.  Bytes count each
    touched expert's weights once, plus the inputs/outputs of the layer that
    the phase must read or write; intermediates are excluded."""
    H, E, K, I, Is = d.H, d.E, d.K, d.I, d.Is
    if phase == "router":
        return 2 * (E * H + T * H + H), 2 * T * H * (E + 1)
    if phase == "dispatch":
        return 0, 0
    if phase == "gate_up":
        return 2 * (U * 2 * I * H + 2 * Is * H + T * H), 2 * T * K * H * 2 * I + 2 * T * H * 2 * Is
    if phase == "down":
        return 2 * (U * H * I + H * Is), 2 * T * K * I * H + 2 * T * Is * H
    if phase == "combine":
        return 2 * T * H, 0
    raise KeyError(phase)


def step_work(d, T, U):
    """Algorithmic bytes and flops of one whole layer call."""
    per_expert = 2 * 3 * d.H * d.I
    nbytes = U * per_expert + 2 * 3 * d.H * d.Is + 2 * d.E * d.H + 2 * d.H + 2 * 2 * T * d.H
    flops = T * 2 * (d.K * 3 * d.H * d.I + 3 * d.H * d.Is + d.E * d.H + d.H)
    return nbytes, flops


def attainable_frac(nbytes, flops, sec):
    """Fraction of the attainable roofline: the roofline time is the larger of
    the memory time and the compute time at peak."""
    return max(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)) / sec


def _source_ok(rec):
    import hashlib
    csrc = os.path.join(ROOT, "sparse_mixture_experts_top8_amd", "csrc")
    h = hashlib.sha256()
    for f in (rec["source"], "common.hpp", "kernels.hpp", "lds_pipe.hpp", "handoff.hpp", "group_dispatch.hpp"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16] == rec["source_sha"]


def counter_record(workload, kernel):
    """The committed rocprofv3 counter record of `kernel` (HBM bytes per launch
    from FETCH_SIZE / WRITE_SIZE runs scaled by a plain-copy calibration; MFMA
    busy), or None when there is none or the kernel's source changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload, {}).get(kernel)
    if not rec or not _source_ok(rec):
        return None
    return rec


def measured_traffic(workload, kernel):
    rec = counter_record(workload, kernel)
    return int(rec["traffic_bytes"]) if rec and "traffic_bytes" in rec else None


def load_stats(counts):
    """Realised expert loads: max / mean and the slope of log(load) against
    log(rank) over the experts with a load (a Zipf(s) law has slope -s)."""
    import numpy as np
    c = np.sort(np.asarray(counts, dtype=np.float64))[::-1]
    nz = c[c > 0]
    r = np.arange(1, nz.size + 1, dtype=np.float64)
    slope = float(np.polyfit(np.log(r), np.log(nz), 1)[0]) if nz.size > 1 else None
    return {"max_over_mean": round(float(c.max() / c.mean()), 3), "max": int(c.max()),
            "mean": round(float(c.mean()), 2), "experts_touched": int(nz.size),
            "loglog_slope": None if slope is None else round(slope, 3),
            "sorted_loads": [int(v) for v in c]}


# ---------------------------------------------------------------------------
# Other entry points on the same batches.
# ---------------------------------------------------------------------------

def other_entry_points(moe, mi, d, wl, T, steps, warmup, nlayers, layers, xs, outs, ws, time_calls):
    """Timings of the other entry points on the same batches: the load-balance
    statistic, the sub-block form, bf16 router scores (and ranks), and routed
    experts streamed from pinned host memory."""
    import numpy as np
    import torch
    lb_steps = min(steps, 200)
    lb_out = [moe.load_balance(xs[l], layers[l], ws=ws) for l in range(nlayers)]
    load_balance = {
        "us_per_call": time_calls(lambda i: moe.load_balance(xs[i % nlayers], layers[i % nlayers], ws=ws), lb_steps),
        "lb": round(float(np.mean([float(r["lb"].item()) for r in lb_out])), 6),
        "definition": "E * sum_e f_e * P_e (slot fraction x mean full-softmax probability)"}

    norm_w = moe.bits_to_device(
        mi.f32_to_bf16_bits(np.random.default_rng(11).normal(1.0, 0.2, d.H).astype(np.float32)), "cuda")
    block = {"us_per_call": time_calls(lambda i: moe.block_forward(xs[i % nlayers], layers[i % nlayers], norm_w,
                                                                   1e-6, out=outs[i % nlayers], ws=ws),
                                       lb_steps, min(warmup, 20)),
             "definition": "out = h + layer(RMSNorm(h)), eps 1e-6"}

    layers_b = [ly.with_logits_bf16() for ly in layers]
    logits_b = moe.route(xs[0], layers_b[0], ws=ws, want_logits=True)["logits"]
    bf16_logits = {
        "us_per_call": time_calls(lambda i: moe.forward(xs[i % nlayers], layers_b[i % nlayers],
                                                        out=outs[i % nlayers], ws=ws), lb_steps, min(warmup, 20)),
        "ranks_us_per_call": time_calls(lambda i: moe.ranks(logits_b), lb_steps, 5),
        "definition": "router and shared-gate scores rounded to bf16; ranks of [T, E] fp32 scores"}

    host_params = dict(layers[0].params)
    host_params["gate_up_proj"] = host_params["gate_up_proj"].cpu().pin_memory()
    host_params["down_proj"] = host_params["down_proj"].cpu().pin_memory()
    host_layer = moe.MoeLayer(d.H, d.E, d.K, d.I, d.Is, host_params, False, layers[0].experts_tiled)
    cache = moe.expert_cache(host_layer, min(d.E, T * d.K))
    U_host = [touched_experts(moe, x, layers[0], d) for x in xs]
    st_calls = 20 if T <= 16 else 4
    st_us = time_calls(lambda i: moe.forward_streamed(xs[i % nlayers], host_layer, cache, out=outs[i % nlayers],
                                                      ws=ws), st_calls, 2)
    st_bytes = float(np.mean([U_host[i % nlayers] for i in range(st_calls)])) * 3 * d.H * d.I * 2
    streamed = {"us_per_call": st_us, "slots": min(d.E, T * d.K),
                "host_bytes_per_call": int(st_bytes),
                "host_link_GBps": round(st_bytes / (st_us * 1e-6) / 1e9, 2),
                "definition": "routed experts' weights in pinned host memory, touched ones copied per call"}
    del host_params, host_layer, cache
    torch.cuda.synchronize()
    return {"load_balance": load_balance, "block_forward": block, "bf16_logits": bf16_logits, "streamed": streamed}


def touched_experts(moe, x, layer, d, counts_out=None):
    """Experts the batch routes to, from moe_load_balance's counts (the grouped
    path's router and dispatch: no fused-kernel launches, so a kernel trace's
    fused-kernel average holds the layer's own calls only)."""
    import torch
    c = moe.load_balance(x, layer)["counts"]
    if counts_out is not None:
        counts_out.append(c.cpu().numpy())
    return int((c > 0).sum().item())


# ---------------------------------------------------------------------------
# One workload.
# ---------------------------------------------------------------------------

def measure(moe, mi, name, steps, warmup, nlayers, base_bits, args, headline=False):
    import numpy as np
    import torch
    wl = mi.WORKLOADS[name]
    d = wl.dims
    T = wl.T
    log(f"workload {name}: T={T}, {nlayers} layers rotated, steps {steps}, warmup {warmup}")
    t0 = time.time()
    layers = [device_layer(moe, mi, wl, l, base_bits) for l in range(nlayers)]
    if not args.row_major:
        # Load-time layout: the routed experts rewritten once into the
        # MFMA-tile layout (moe_tile_experts; same values, same results).
        layers = [ly.tiled() for ly in layers]
    xs = [device_x(moe, mi, wl, l) for l in range(nlayers)]
    outs = [torch.empty_like(x) for x in xs]
    ws = layers[0].workspace(T)
    torch.cuda.synchronize()
    log(f"  inputs ready in {time.time() - t0:.1f} s")

    counts0 = []
    U = [touched_experts(moe, xs[l], layers[l], d, counts0 if l == 0 else None) for l in range(nlayers)]
    U_mean = float(np.mean(U))

    for i in range(warmup):
        l = i % nlayers
        moe.forward(xs[l], layers[l], out=outs[l], ws=ws)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps back to back on the current stream,
    # bracketed by synchronisations and by events on that stream.  It is
    # repeated REPEATS times; the first repeat is the reported step time.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = []
    for rep in range(REPEATS):
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            l = i % nlayers
            moe.forward(xs[l], layers[l], out=outs[l], ws=ws)
        end.record()
        torch.cuda.synchronize()
        reps.append(start.elapsed_time(end) / steps)
    ms_per_step = reps[0]
    status, timeouts = moe.workspace_status(ws, with_count=True)

    def time_calls(call, n, warm=0):
        """Average microseconds of call(i) over n calls back to back on the
        current stream (events on that stream), after warm untimed calls."""
        for i in range(warm):
            call(i)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            call(i)
        end.record()
        torch.cuda.synchronize()
        return round(start.elapsed_time(end) / n * 1e3, 2)

    # Kernel attribution: the same steps again, right after the timed region
    # (the GPU at the same clock), each recording six events at its phase
    # boundaries on the same stream (the fused decode path records its single
    # kernel between events 0 and 1).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for e6 in ev:
        for e in e6:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        l = i % nlayers
        moe.forward_traced(xs[l], layers[l], outs[l], ws, ev[i])
    torch.cuda.synchronize()
    phase_ms = {p: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
                for j, p in enumerate(moe.PHASES)}
    fused = T <= 16 and d.H <= 2048 and d.I <= 512 and d.Is <= 512
    if fused:
        # One kernel per step: its average launch duration is the timed
        # region divided by the steps (events around each launch would add
        # their own marker overhead to a ~20 us kernel).
        phase_ms = {"decode_fused": ms_per_step}
    log("  phase us: " + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in phase_ms.items())
        + f"; step {ms_per_step * 1e3:.1f} us (repeats " + ", ".join(f"{r * 1e3:.1f}" for r in reps) + ")")

    # The other entry points after the attribution: the streamed one leaves
    # the GPU idle behind host copies for tens of milliseconds per call.
    others = {}
    if not args.layer_only:
        others = other_entry_points(moe, mi, d, wl, T, steps, warmup, nlayers, layers, xs, outs, ws, time_calls)

    step_bytes, step_flops = step_work(d, T, U_mean)
    dom = max(phase_ms, key=phase_ms.get)
    if dom == "decode_fused":
        dbytes, dflops = step_bytes, step_flops
    else:
        dbytes, dflops = phase_work(d, T, U_mean, dom)   # U: routed experts; shared added inside
    dsec = phase_ms[dom] * 1e-3
    if name in MFMA_BOUND:
        ach = dflops / dsec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = dbytes / dsec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    rec = counter_record(name, dom)
    roof.update({"kernel": dom, "kernel_us": round(phase_ms[dom] * 1e3, 2),
                 "alg_bytes_per_launch": int(dbytes), "alg_flops_per_launch": int(dflops),
                 "traffic": int(rec["traffic_bytes"]) if rec and "traffic_bytes" in rec else None,
                 "traffic_over_alg": (round(rec["traffic_bytes"] / dbytes, 3)
                                      if rec and "traffic_bytes" in rec and dbytes else None),
                 "mfma_busy": rec.get("mfma_util") if rec else None})
    sec = ms_per_step * 1e-3
    layer_stats = {
        "alg_bytes": int(step_bytes), "alg_flops": int(step_flops), "experts_touched": U_mean,
        "hbm_frac": round(step_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(step_flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "attainable_frac": round(attainable_frac(step_bytes, step_flops, sec), 4),
        "phase_us": {k: round(v * 1e3, 2) for k, v in phase_ms.items()},
    }
    srt = sorted(reps)
    res = {
        "T": T, "ms_per_step": round(ms_per_step, 5), "tokens_per_s": round(T / sec, 2),
        "steps": steps, "warmup": warmup, "layers_rotated": nlayers,
        "repeats_ms": {"n": REPEATS, "median": round(srt[REPEATS // 2], 5), "min": round(srt[0], 5),
                       "max": round(srt[-1], 5)},
        "roofline": roof, "layer": layer_stats,
        "fused_status": {"latest": status, "timed_out_calls": timeouts},
        "workload": f"{wl.name}: {wl.note}; H={d.H} E={d.E} K={d.K} I={d.I} Is={d.Is} T={T}",
    }
    if wl.skewed_router or T >= 4096:
        res["load"] = load_stats(counts0[0])
    res.update(others)
    if timeouts:
        log(f"  WARNING: {timeouts} fused-kernel calls reported a timed-out wait")

    # Layer 0's routing and output, for the parity statistics of the CPU leg.
    gpu_ref = None
    if not args.no_cpu_baseline:
        r = moe.route(xs[0], layers[0], ws=ws)
        out0 = moe.forward(xs[0], layers[0], ws=ws)
        gpu_ref = {"topk_idx": r["topk_idx"].cpu().numpy(), "perm": r["perm"].cpu().numpy(),
                   "offsets": r["offsets"].cpu().numpy(), "out": out0.float().cpu().numpy()}
    del layers, xs, outs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, gpu_ref


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, timed on the host.
# ---------------------------------------------------------------------------

def cpu_baseline(mi, wl, bits, gpu_ref, repeat_s):
    """The CPU oracle (float64 NumPy, the definition written out) on a bounded
    sample of the same workload: parameters decoded once outside the timed
    region, three timed repeats, the median reported.  Also the parity of the
    GPU's layer-0 results against the oracle: routing over the whole batch,
    output over the timed sample's tokens."""
    import numpy as np
    from oracle import moe_oracle as O
    facts = host_facts()
    threads = (facts["blas"] or {}).get("threads") or len(os.sched_getaffinity(0))
    d = wl.dims
    dec = O.decode_params(bits)               # outside the timed region
    x = mi.workload_x(wl)
    rates = []
    if wl.T == 1:
        pool = mi.make_x(d, 4096, wl.x_seed + 7000, wl.x_std)
        pos = 0
        for _ in range(3):
            n, t0 = 0, time.perf_counter()
            while n < 2 or time.perf_counter() - t0 < repeat_s:
                j = (pos + n) % pool.shape[0]
                O.forward(pool[j:j + 1], dec, d.K)
                n += 1
            rates.append(n / (time.perf_counter() - t0))
            pos += n
        sample = (f"3 repeats of ~{repeat_s:.0f} s of single-token oracle.forward calls ({pos} calls over a pool "
                  f"of {pool.shape[0]} tokens), float64, parameters decoded once beforehand")
        n_out = 1
    else:
        n = 8
        while True:
            t0 = time.perf_counter()
            O.forward(x[:n], dec, d.K)
            el = time.perf_counter() - t0
            if el > repeat_s / 2 or n >= wl.T:
                break
            n = min(wl.T, n * 2)
        for _ in range(3):
            t0 = time.perf_counter()
            O.forward(x[:n], dec, d.K)
            rates.append(n / (time.perf_counter() - t0))
        sample = (f"3 repeats of one oracle.forward call on the first {n} tokens of the {wl.T}-token batch, "
                  f"float64, parameters decoded once beforehand")
        n_out = n
    res = {"value": round(float(np.median(rates)), 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": sample, "repeats_tokens_per_s": [round(r, 3) for r in rates],
           "cpu_model": facts["cpu_model"], "blas": facts["blas"]}
    if gpu_ref is not None:
        R = O.route(x, dec, d.K)
        gi = gpu_ref["topk_idx"]
        diff = (gi != R["topk_idx"]).any(axis=1)
        cs = O.counting_sort(gi, d.E)
        ref = O.forward_with_routing(x[:n_out], dec, gi[:n_out])
        got = gpu_ref["out"][:n_out].astype(np.float64)
        res["parity"] = {
            "tokens_routed": int(wl.T), "flagged_ties": int(R["tie"].sum()),
            "index_mismatch_unflagged": int((diff & ~R["tie"]).sum()),
            "index_mismatch_flagged": int((diff & R["tie"]).sum()),
            "perm_mismatch": int((gpu_ref["perm"][:wl.T * d.K] != cs["perm"]).sum()
                                 + (gpu_ref["offsets"] != cs["offsets"]).sum()),
            "output_rows": int(n_out), "max_abs": float(np.abs(got - ref).max()),
            "rel_l2": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
        }
    return res


# ---------------------------------------------------------------------------
# Other modes.
# ---------------------------------------------------------------------------

def batch_sweep():
    """Step time of the layer at batch sizes 1..64 on either side of the
    fused-decode / grouped-path switch (T <= 16 / T > 16): 8 full-shape layers
    rotated (tiled experts), x ~ N(0, 1) seeded by T, 400 warm-up and 400 timed
    calls; bytes = touched experts once + shared expert + router + x and out."""
    import numpy as np
    import torch
    import moe_inputs as mi
    import sparse_mixture_experts_top8_amd as moe
    wl = mi.WORKLOADS["decode64"]
    d = wl.dims
    base = mi.workload_layer(wl)
    layers = [device_layer(moe, mi, wl, l, base).tiled() for l in range(8)]
    for T in [1, 2, 4, 8, 12, 16, 17, 24, 32, 48, 64]:
        g = torch.Generator(device="cuda")
        g.manual_seed(T)
        xs = [torch.randn((T, d.H), generator=g, device="cuda").to(torch.bfloat16) for _ in range(8)]
        outs = [torch.empty_like(x) for x in xs]
        ws = layers[0].workspace(T)
        for i in range(400):
            moe.forward(xs[i % 8], layers[i % 8], out=outs[i % 8], ws=ws)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(400):
            moe.forward(xs[i % 8], layers[i % 8], out=outs[i % 8], ws=ws)
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) / 400 * 1e3
        U = float(np.mean([touched_experts(moe, xs[l], layers[l], d) for l in range(8)]))
        nbytes, _ = step_work(d, T, U)
        print(json.dumps({"T": T, "path": "fused decode" if T <= 16 else "grouped", "us_per_step": round(us, 2),
                          "experts_touched": U, "alg_TBps": round(nbytes / us / 1e6, 3)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is measured on a "
              f"single MI355X and no multi-GPU path exists", file=sys.stderr)
        sys.exit(2)
    if args.batch_sweep:
        batch_sweep()
        return
    if args.copy_probe:
        return copy_probe()

    # The shader clock levels come from rocm-smi, queried before this process
    # touches the GPU (a child started after that could not run under a
    # profiler's preloaded library); only for the default line.
    clock_before_gpu_use = gpu_clock() if args.workload is None else None

    import torch

    import moe_inputs as mi
    import sparse_mixture_experts_top8_amd as moe

    prop = torch.cuda.get_device_properties(0)
    sclk = clock_before_gpu_use
    log(f"device {prop.name} ({getattr(prop, 'gcnArchName', '?')}), {prop.multi_processor_count} CUs")
    t_all = time.time()
    base_bits = mi.workload_layer(mi.WORKLOADS[HEADLINE])   # all workloads share the layer seed

    def settings(name, explicit):
        steps, warmup, nlayers = DEFAULTS[name]
        if explicit:
            steps = args.steps if args.steps is not None else steps
            warmup = args.warmup if args.warmup is not None else warmup
        return steps, warmup, args.layers if args.layers is not None else nlayers

    head = args.workload or HEADLINE
    subs = [] if args.workload else list(SUB_WORKLOADS)
    results, refs = {}, {}
    probes = None
    if subs:
        probes = ceiling_probes()
        log(f"ceiling probes: {probes}")
    # The other workloads first (their own step counts), then the headline,
    # timed over exactly --steps steps after --warmup untimed ones.
    for name in subs + [head]:
        steps, warmup, nlayers = settings(name, name == head)
        results[name], refs[name] = measure(moe, mi, name, steps, warmup, nlayers, base_bits, args,
                                            headline=name == head)
    if not args.no_cpu_baseline:
        for name in [head] + subs:
            wl = mi.WORKLOADS[name]
            log(f"timing the CPU oracle on a bounded sample of {name} ...")
            results[name]["cpu_baseline"] = cpu_baseline(mi, wl, layer0_bits(mi, wl, base_bits), refs[name],
                                                         CPU_REPEAT_S[name] * args.cpu_scale)

    h = results[head]
    wl = mi.WORKLOADS[head]
    d = wl.dims
    result = {
        "metric": "MoE-layer tokens/s + % HBM BW peak (decode) / % bf16 MFMA peak (prefill)",
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": h["warmup"],
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": h["workload"], "tokens_per_step": wl.T, "layers_rotated": h["layers_rotated"],
                   "weights": "seeded N(0,0.02) bf16",
                   "expert_layout": "row-major" if args.row_major else "mfma-tile",
                   "device": prop.name, "cus": prop.multi_processor_count, "sclk": sclk},
        "roofline": h["roofline"],
        "layer": h["layer"],
        "repeats_ms": h["repeats_ms"],
        "fused_status": h["fused_status"],
        "cpu_baseline": h.get("cpu_baseline"),
    }
    for k in ("load_balance", "block_forward", "bf16_logits", "streamed"):
        result[k] = h.get(k)
    if subs:
        result["workloads"] = {n: results[n] for n in subs}
        result["ceiling_probes"] = probes
    log(f"bench done in {time.time() - t_all:.1f} s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the MoE layer (256 experts, top-8, gated shared expert) on one MI355X.

A step is one moe_forward call (router, top-K, dispatch, both expert GEMMs,
shared expert, combine) over one batch of seeded synthetic tokens, with the
inputs already resident in HBM.  Steps rotate over several independently drawn
layers so that weights are not served from the 256 MB Infinity Cache across
steps (8 layers at T = 1, 2 otherwise).

    python bench.py                       # 1-token decode, the default workload
    python bench.py --workload prefill4096 --steps 50 --warmup 5

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode1", choices=sorted(DEFAULTS))
    ap.add_argument("--layers", type=int, default=None, help="weight sets rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-major", action="store_true",
                    help="keep the routed experts row-major instead of the MFMA-tile layout")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--layer-only", action="store_true",
                    help="skip the other entry points' timings (load balance, sub-block, bf16 scores, streamed "
                         "experts), so that a kernel trace holds the layer's own launches")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="only time moe_forward at batch sizes 1..64 (the full-shape layer, 8 layers rotated) and "
                         "print one JSON line per size")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


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
        U = float(np.mean([int((torch.bincount(moe.route(xs[l], layers[l], ws=ws)["topk_idx"].view(-1).long(),
                                               minlength=d.E) > 0).sum()) for l in range(8)]))
        nbytes, _ = step_work(d, T, U)
        print(json.dumps({"T": T, "path": "fused decode" if T <= 16 else "grouped", "us_per_step": round(us, 2),
                          "experts_touched": U, "alg_TBps": round(nbytes / us / 1e6, 3)}), flush=True)


def device_layer(moe, mi, wl, l, base_bits):
    """Layer l of the rotation: layer 0 from the seeded CPU generator, the others
    drawn on the device (torch generator seeded layer_seed*100 + l)."""
    import torch
    d = wl.dims
    if l == 0:
        bits = dict(base_bits)
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


def device_x(moe, mi, wl, l):
    import torch
    if l == 0:
        return moe.bits_to_device(mi.workload_x(wl), "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.x_seed * 100 + l)
    return (torch.randn((wl.T, wl.dims.H), generator=g, device="cuda") * wl.x_std).to(torch.bfloat16)


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


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE runs scaled by a plain-copy
    calibration), or None when there is none or the kernel's source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload, {}).get(kernel)
    if not rec:
        return None
    csrc = os.path.join(ROOT, "sparse_mixture_experts_top8_amd", "csrc")
    h = hashlib.sha256()
    for f in (rec["source"], "common.hpp", "kernels.hpp"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return int(rec["traffic_bytes"]) if h.hexdigest()[:16] == rec["source_sha"] else None


def other_entry_points(moe, mi, d, wl, T, steps, warmup, nlayers, layers, xs, outs, ws, time_calls):
    """Timings of the other entry points on the same batches: the load-balance
    statistic, the sub-block form, bf16 router scores (and ranks), and routed
    experts streamed from pinned host memory."""
    import numpy as np
    import torch
    # Load-balance statistic of the same batches (moe_load_balance: router,
    # dispatch and the statistic), timed outside the step.
    lb_steps = min(steps, 200)
    lb_out = [moe.load_balance(xs[l], layers[l], ws=ws) for l in range(nlayers)]
    load_balance = {
        "us_per_call": time_calls(lambda i: moe.load_balance(xs[i % nlayers], layers[i % nlayers], ws=ws), lb_steps),
        "lb": round(float(np.mean([float(r["lb"].item()) for r in lb_out])), 6),
        "definition": "E * sum_e f_e * P_e (slot fraction x mean full-softmax probability)"}

    # The sub-block form out = h + layer(RMSNorm(h)) on the same batches.
    norm_w = moe.bits_to_device(
        mi.f32_to_bf16_bits(np.random.default_rng(11).normal(1.0, 0.2, d.H).astype(np.float32)), "cuda")
    block = {"us_per_call": time_calls(lambda i: moe.block_forward(xs[i % nlayers], layers[i % nlayers], norm_w,
                                                                   1e-6, out=outs[i % nlayers], ws=ws),
                                       lb_steps, min(warmup, 20)),
             "definition": "out = h + layer(RMSNorm(h)), eps 1e-6"}

    # The layer with bf16 router scores (logits_bf16) on the same batches, and
    # the stable ranks of one batch's [T, E] scores.
    layers_b = [ly.with_logits_bf16() for ly in layers]
    logits_b = moe.route(xs[0], layers_b[0], ws=ws, want_logits=True)["logits"]
    bf16_logits = {
        "us_per_call": time_calls(lambda i: moe.forward(xs[i % nlayers], layers_b[i % nlayers],
                                                        out=outs[i % nlayers], ws=ws), lb_steps, min(warmup, 20)),
        "ranks_us_per_call": time_calls(lambda i: moe.ranks(logits_b), lb_steps, 5),
        "definition": "router and shared-gate scores rounded to bf16; ranks of [T, E] fp32 scores"}

    # Routed experts streamed from pinned host memory (moe_forward_streamed)
    # into a device cache big enough for one round; the bytes that cross the
    # host link per call are the touched experts' weights.
    host_params = dict(layers[0].params)
    host_params["gate_up_proj"] = host_params["gate_up_proj"].cpu().pin_memory()
    host_params["down_proj"] = host_params["down_proj"].cpu().pin_memory()
    host_layer = moe.MoeLayer(d.H, d.E, d.K, d.I, d.Is, host_params, False, layers[0].experts_tiled)
    cache = moe.expert_cache(host_layer, min(d.E, T * d.K))
    U_host = [int((torch.bincount(moe.route(x, layers[0], ws=ws)["topk_idx"].view(-1).long(),
                                  minlength=d.E) > 0).sum()) for x in xs]
    st_calls = 20 if T <= 16 else 4
    st_us = time_calls(lambda i: moe.forward_streamed(xs[i % nlayers], host_layer, cache, out=outs[i % nlayers],
                                                      ws=ws), st_calls, 2)
    st_bytes = float(np.mean([U_host[i % nlayers] for i in range(st_calls)])) * 3 * d.H * d.I * 2
    streamed = {"us_per_call": st_us, "slots": min(d.E, T * d.K),
                "host_bytes_per_call": int(st_bytes),
                "host_link_GBps": round(st_bytes / (st_us * 1e-6) / 1e9, 2),
                "definition": "routed experts' weights in pinned host memory, touched ones copied per call"}
    del host_params, host_layer, cache
    return load_balance, block, bf16_logits, streamed


def step_work(d, T, U):
    """Algorithmic bytes and flops of one whole layer call."""
    per_expert = 2 * 3 * d.H * d.I
    nbytes = U * per_expert + 2 * 3 * d.H * d.Is + 2 * d.E * d.H + 2 * d.H + 2 * 2 * T * d.H
    flops = T * 2 * (d.K * 3 * d.H * d.I + 3 * d.H * d.Is + d.E * d.H + d.H)
    return nbytes, flops


def cpu_baseline(mi, wl, bits, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    d = wl.dims
    if wl.T == 1:
        xs = mi.make_x(d, 4096, wl.x_seed + 7000, wl.x_std)
        n, t0 = 0, time.perf_counter()
        while n < 3 or (time.perf_counter() - t0 < budget_s and n < xs.shape[0]):
            O.forward(xs[n:n + 1], bits, d.K)
            n += 1
        el = time.perf_counter() - t0
        sample = f"{n} single-token calls (fresh x each), oracle.forward, float64"
        return {"value": n / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": sample, "seconds": round(el, 2)}
    x = mi.workload_x(wl)
    n = 8
    while True:
        t0 = time.perf_counter()
        O.forward(x[:n], bits, d.K)
        el = time.perf_counter() - t0
        if el > budget_s / 3 or n >= wl.T:
            break
        n = min(wl.T, n * 4)
    sample = f"first {n} tokens of the {wl.T}-token batch in one oracle.forward call, float64"
    return {"value": n / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(el, 2)}


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

    import numpy as np
    import torch

    import moe_inputs as mi
    import sparse_mixture_experts_top8_amd as moe

    wl = mi.WORKLOADS[args.workload]
    d = wl.dims
    steps, warmup, nlayers = DEFAULTS[args.workload]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    nlayers = args.layers if args.layers is not None else nlayers
    T = wl.T

    prop = torch.cuda.get_device_properties(0)
    log(f"device {prop.name} ({getattr(prop, 'gcnArchName', '?')}), {prop.multi_processor_count} CUs")
    log(f"workload {wl.name}: T={T}, {nlayers} layers rotated, steps {steps}, warmup {warmup}")
    t0 = time.time()
    base_bits = mi.workload_layer(wl)
    layers = [device_layer(moe, mi, wl, l, base_bits) for l in range(nlayers)]
    if not args.row_major:
        # Load-time layout: the routed experts rewritten once into the
        # MFMA-tile layout (moe_tile_experts; same values, same results).
        layers = [ly.tiled() for ly in layers]
    xs = [device_x(moe, mi, wl, l) for l in range(nlayers)]
    outs = [torch.empty_like(x) for x in xs]
    ws = layers[0].workspace(T)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    # Touched experts per layer (for the byte model).
    U = []
    for l in range(nlayers):
        r = moe.route(xs[l], layers[l], ws=ws)
        U.append(int((torch.bincount(r["topk_idx"].view(-1).long(), minlength=d.E) > 0).sum()))
    U_mean = float(np.mean(U))

    for i in range(warmup):
        l = i % nlayers
        moe.forward(xs[l], layers[l], out=outs[l], ws=ws)
    torch.cuda.synchronize()

    # Timed region: K steps back to back on the current stream, bracketed by
    # events on that stream.
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        l = i % nlayers
        moe.forward(xs[l], layers[l], out=outs[l], ws=ws)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps

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

    load_balance = block = bf16_logits = streamed = None
    if not args.layer_only:
        load_balance, block, bf16_logits, streamed = other_entry_points(moe, mi, d, wl, T, steps, warmup, nlayers,
                                                                        layers, xs, outs, ws, time_calls)

    # Kernel attribution: the same steps again, each recording six events at
    # its phase boundaries on the same stream (the fused decode path records
    # its single kernel between events 0 and 1).
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
        # their own marker overhead to a ~30 us kernel).
        phase_ms = {"decode_fused": ms_per_step}
    log("phase us: " + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in phase_ms.items())
        + f"; step {ms_per_step * 1e3:.1f} us")

    step_bytes, step_flops = step_work(d, T, U_mean)
    dom = max(phase_ms, key=phase_ms.get)
    if dom == "decode_fused":
        dbytes, dflops = step_work(d, T, U_mean)
    else:
        dbytes, dflops = phase_work(d, T, U_mean, dom)   # U: routed experts; shared added inside
    dsec = phase_ms[dom] * 1e-3
    mfma_bound = wl.name == "zipf16384"
    if mfma_bound:
        ach = dflops / dsec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = dbytes / dsec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": dom, "kernel_us": round(phase_ms[dom] * 1e3, 2),
                 "alg_bytes_per_launch": int(dbytes), "alg_flops_per_launch": int(dflops),
                 "traffic": measured_traffic(wl.name, dom)})

    sec = ms_per_step * 1e-3
    layer_stats = {
        "alg_bytes": int(step_bytes), "alg_flops": int(step_flops), "experts_touched": U_mean,
        "hbm_frac": round(step_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(step_flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "attainable_frac": round(min(step_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                                     step_bytes / (HBM_PEAK_GBS * 1e9)) / sec, 4),
        "phase_us": {k: round(v * 1e3, 2) for k, v in phase_ms.items()},
    }

    result = {
        "metric": "MoE-layer tokens/s + % HBM BW peak (decode) / % bf16 MFMA peak (prefill)",
        "value": round(T / sec, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}; H={d.H} E={d.E} K={d.K} I={d.I} Is={d.Is} T={T}",
                   "tokens_per_step": T, "layers_rotated": nlayers, "weights": "seeded N(0,0.02) bf16",
                   "expert_layout": "row-major" if args.row_major else "mfma-tile",
                   "device": prop.name, "cus": prop.multi_processor_count},
        "roofline": roof,
        "layer": layer_stats,
        "load_balance": load_balance,
        "block_forward": block,
        "bf16_logits": bf16_logits,
        "streamed": streamed,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(mi, wl, base_bits, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

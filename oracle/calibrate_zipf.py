"""Fit the per-expert router row gains of the skewed-load (Zipf) workload.

Writes ``moe_inputs/zipf_router_gain.txt``; run from the repository root:

    python -m oracle.calibrate_zipf

TEST INFRASTRUCTURE ONLY: routing here is the CPU oracle's (float64 logits,
stable top-K), and the only other module used is the seeded input generator.

The router of the workload has no bias and sees zero-mean inputs, so the only
lever on an expert's load is the norm of its router row: row e is
Z[e] * gain[e] with Z the ordinary N(0, 0.02) draw.  The target load profile:

1. a seeded permutation maps Zipf rank -> expert;
2. Zipf(s = 1.1) over ranks, p_k proportional to k^-s, K*T slots in total;
3. water filling: an expert can hold at most ``CAP`` of the tokens (a large row
   norm makes an expert win about half of the tokens, never more), so loads
   above the cap are clipped and the unclipped ranks are scaled up by a common
   factor until the total is again K*T.

The gains are fitted on calibration inputs (a seed of their own) with the
damped update log g += 0.2 (log target - log measured), then frozen.
"""
from __future__ import annotations

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import moe_inputs as mi  # noqa: E402
from oracle.moe_oracle import router_logits, select_topk  # noqa: E402

ZIPF_S = 1.1
CAP = 0.45
PERM_SEED = 4
ITERS = 150
DAMPING = 0.2


def zipf_targets(E: int, K: int, T: int) -> np.ndarray:
    """Water-filled Zipf(1.1) slot targets per expert, in expert order."""
    k = np.arange(1, E + 1, dtype=np.float64)
    p = k ** -ZIPF_S
    p /= p.sum()
    total = K * T
    cap = CAP * T
    target = total * p
    clipped = np.zeros(E, dtype=bool)
    for _ in range(E):
        over = (target > cap) & ~clipped
        if not over.any():
            break
        clipped |= over
        free = total - cap * clipped.sum()
        target = np.where(clipped, cap, p * free / p[~clipped].sum())
    perm = np.random.default_rng(PERM_SEED).permutation(E)   # rank r -> expert perm[r]
    out = np.empty(E)
    out[perm] = target
    return out


def loads(x_bits, router_bits, K, E):
    idx, _ = select_topk(router_logits(x_bits, router_bits), K)
    return np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)


def main():
    w = mi.WORKLOADS["zipf16384"]
    dims, T = w.dims, w.T
    E, K = dims.E, dims.K
    target = zipf_targets(E, K, T)
    x_cal = mi.make_x(dims, T, mi.ZIPF_CALIBRATION_X_SEED)
    gain = np.ones(E)
    for it in range(ITERS):
        router = mi._normal_bf16(w.layer_seed, "gate.weight", (E, dims.H), mi.WEIGHT_STD, gain=gain)
        got = loads(x_cal, router, K, E)
        big = target >= 100
        err = np.abs(got[big] / target[big] - 1).max()
        print(f"iter {it:2d}  max rel err (targets >= 100) {err:.4f}  max load {got.max():.0f}",
              flush=True)
        if err < 0.03:
            break
        gain *= np.exp(DAMPING * (np.log(target) - np.log(np.maximum(got, 0.5))))
    path = mi.ZIPF_GAIN_FILE
    with open(path, "w") as f:
        f.write("# router row gains for the Zipf(1.1) skewed-load workload, one per expert\n")
        f.write("# written by: python -m oracle.calibrate_zipf\n")
        for g in gain:
            f.write(f"{g:.9e}\n")
    router = mi._normal_bf16(w.layer_seed, "gate.weight", (E, dims.H), mi.WEIGHT_STD, gain=gain)
    got = loads(mi.workload_x(w), router, K, E)
    mean = K * T / E
    print(f"measurement x: max load {got.max():.0f} = {got.max() / mean:.1f} x mean; "
          f"min load {got.min():.0f}")


if __name__ == "__main__":
    main()

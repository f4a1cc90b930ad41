"""Seeded synthetic inputs for the sparse MoE FFN layer.

Test and benchmark infrastructure shared by the CPU oracle's tests and by the
GPU path's tests and benchmark.  This module only draws random numbers and
encodes them as bfloat16 bit patterns; it performs none of the layer's
arithmetic (no projection, softmax, selection, activation or combine).

Shapes follow the typed block signature of ``SparseMoe`` on the Linnet model
page ("Qwen3.6 35B-A3B", Blocks: SparseMoe, Linear): a ``Linear<In, Out>``
stores ``weight`` as ``[Out, In]``; the routed experts are the merged
``gate_up_proj [Experts, 2*ExpertInner, H]`` and ``down_proj
[Experts, H, ExpertInner]``; the shared expert is a ``SwiGlu<H, SharedInner>``
with separate gate, up and down Linears; the shared-expert gate is a
``Linear<H, 1>``.

Every tensor is drawn from its own PCG64 stream, keyed by (seed, tensor id),
so that any one tensor (for example only the hidden states ``x``) can be made
without drawing the others.  Values are float32 normals scaled by the
standard deviation, then rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field

import numpy as np

# Parameter names as the Linnet model page prints the SparseMoe members.
PARAM_NAMES = (
    "gate.weight",                 # router          [E, H]
    "gate_up_proj",                # routed experts  [E, 2I, H]
    "down_proj",                   # routed experts  [E, H, I]
    "shared_expert.gate.weight",   # shared SwiGlu   [Is, H]
    "shared_expert.up.weight",     # shared SwiGlu   [Is, H]
    "shared_expert.down.weight",   # shared SwiGlu   [H, Is]
    "shared_expert_gate.weight",   # scalar gate     [1, H]
)

_STREAM_ID = {name: i for i, name in enumerate(PARAM_NAMES)}
_STREAM_ID["x"] = 100

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Dims:
    """Layer dimensions: hidden H, experts E, top-K, expert inner I, shared inner Is."""
    H: int
    E: int
    K: int
    I: int
    Is: int

    def shapes(self) -> dict:
        H, E, I, Is = self.H, self.E, self.I, self.Is
        return {
            "gate.weight": (E, H),
            "gate_up_proj": (E, 2 * I, H),
            "down_proj": (E, H, I),
            "shared_expert.gate.weight": (Is, H),
            "shared_expert.up.weight": (Is, H),
            "shared_expert.down.weight": (H, Is),
            "shared_expert_gate.weight": (1, H),
        }


# Full shape bound by the model page's generics (H 2048, Experts 256, TopK 8,
# ExpertInner 512, SharedInner 512) and a toy shape for fast exact checks.
FULL = Dims(H=2048, E=256, K=8, I=512, Is=512)
TOY = Dims(H=256, E=16, K=4, I=64, Is=64)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are finite.  The low 16 bits are rounded into the high 16 bits with
    ties going to the even high half.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += u
    lsb >>= np.uint32(16)
    return lsb.astype(np.uint16)


def _rng(seed: int, name: str, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), _STREAM_ID[name], int(chunk)]))


_CHUNK_ELEMS = 1 << 22
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        n = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = ThreadPoolExecutor(max_workers=n)
    return _POOL


def _normal_bf16(seed: int, name: str, shape, std: float, gain=None) -> np.ndarray:
    """bf16 bits of std * N(0,1) float32 draws (times an optional per-row gain).

    The flattened [rows, last] view is cut into fixed row chunks; chunk c is
    drawn from the stream keyed (seed, tensor id, c), so the result does not
    depend on how many threads fill it.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1])
    rows = flat.shape[0]
    chunk_rows = max(1, _CHUNK_ELEMS // shape[-1])
    g = None if gain is None else np.asarray(gain, dtype=np.float32).reshape(-1, 1)

    def fill(c):
        r0 = c * chunk_rows
        r1 = min(rows, r0 + chunk_rows)
        v = _rng(seed, name, c).standard_normal((r1 - r0, shape[-1]), dtype=np.float32)
        v *= np.float32(std)
        if g is not None:
            v *= g[r0:r1]
        flat[r0:r1] = f32_to_bf16_bits(v)

    n_chunks = (rows + chunk_rows - 1) // chunk_rows
    if n_chunks == 1:
        fill(0)
    else:
        list(_pool().map(fill, range(n_chunks)))
    return out


def make_layer(dims: Dims, seed: int, std: float = WEIGHT_STD,
               router_row_gain: np.ndarray | None = None) -> dict:
    """All seven SparseMoe parameters as bf16 bit arrays (uint16), keyed by PARAM_NAMES.

    ``router_row_gain`` (optional, [E] float) multiplies router row e by
    gain[e] before the bf16 rounding; it is how the skewed-load workload
    biases its router (see ``zipf_router_gain``).
    """
    shapes = dims.shapes()
    layer = {}
    for name in PARAM_NAMES:
        gain = router_row_gain if name == "gate.weight" else None
        layer[name] = _normal_bf16(seed, name, shapes[name], std, gain=gain)
    return layer


def make_router(dims: Dims, seed: int, router_row_gain: np.ndarray | None = None,
                std: float = WEIGHT_STD) -> np.ndarray:
    """Only the router weight [E, H] of ``make_layer(dims, seed, ...)`` (same draw)."""
    return _normal_bf16(seed, "gate.weight", (dims.E, dims.H), std, gain=router_row_gain)


def make_x(dims: Dims, T: int, seed: int, std: float = 1.0) -> np.ndarray:
    """Hidden states x [T, H] as bf16 bits, std * N(0,1)."""
    return _normal_bf16(seed, "x", (int(T), dims.H), std)


# ---------------------------------------------------------------------------
# Workloads.  One full-shape layer (weights seed 1) is shared by the decode,
# batched-decode and prefill workloads; the skewed-load workload uses the same
# expert weights with a router whose rows are scaled by stored gains.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    T: int
    layer_seed: int
    x_seed: int
    x_std: float = 1.0
    skewed_router: bool = False
    note: str = field(default="", compare=False)


WORKLOADS = {
    "toy": Workload("toy", TOY, 8, 0, 0,
                    note="H=256, 16 experts, top-4, inner 64, 8 tokens"),
    "decode1": Workload("decode1", FULL, 1, 1, 1,
                        note="full shape, 1 token"),
    "decode64": Workload("decode64", FULL, 64, 1, 2,
                         note="full shape, 64 tokens, near-uniform routing"),
    "prefill4096": Workload("prefill4096", FULL, 4096, 1, 3,
                            note="full shape, 4096 tokens, ~128 slots per expert"),
    "zipf16384": Workload("zipf16384", FULL, 16384, 1, 4, skewed_router=True,
                          note="full shape, 16384 tokens, Zipf(1.1) expert load"),
}

ZIPF_GAIN_FILE = os.path.join(os.path.dirname(__file__), "zipf_router_gain.txt")
ZIPF_CALIBRATION_X_SEED = 1004


def zipf_router_gain() -> np.ndarray:
    """Per-expert router row gains [256] for the skewed-load workload.

    The values are data: they were fitted once by ``oracle/calibrate_zipf.py``
    (a script that routes with the CPU oracle) so that expert loads follow a
    water-filled Zipf(1.1) profile, and are read here from a text file.
    """
    return np.loadtxt(ZIPF_GAIN_FILE, dtype=np.float64).reshape(-1)


def workload_layer(w: Workload) -> dict:
    gain = zipf_router_gain() if w.skewed_router else None
    return make_layer(w.dims, w.layer_seed, router_row_gain=gain)


def workload_x(w: Workload) -> np.ndarray:
    return make_x(w.dims, w.T, w.x_seed, w.x_std)

"""Sparse MoE FFN layer (256 experts, top-8, gated shared expert) on MI355X.

Python face of the gfx950 HIP library: the layer of "Qwen3.6-35B-A3B —
Architecture Overview", section "MoE FFN: 256 Experts", with the parameter
shapes of the Linnet model page "Qwen3.6 35B-A3B" (Blocks: SparseMoe).

    layer = MoeLayer.from_bf16_bits(params_uint16, dims, device="cuda")
    out = forward(x, layer)            # x: bf16 [T, H] on the GPU
    r = route(x, layer)                # topk_idx, topk_w, offsets, perm, ...

The functions only marshal arguments to the C ABI (include/moe.h); all work
runs in the library's kernels on the caller's current HIP stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (EXPORTS, LIB_PATH, MoeError, MoeLayerT, lib, last_error,  # noqa: F401
                   strerror)

PARAM_NAMES = (
    "gate.weight",
    "gate_up_proj",
    "down_proj",
    "shared_expert.gate.weight",
    "shared_expert.up.weight",
    "shared_expert.down.weight",
    "shared_expert_gate.weight",
)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


@dataclass
class MoeLayer:
    """Device-resident parameters of one layer plus its C descriptor."""
    H: int
    E: int
    K: int
    I: int
    Is: int
    params: dict
    logits_bf16: bool = False   # router / shared-gate scores rounded to bf16
    experts_tiled: bool = False  # gate_up_proj / down_proj in the MFMA-tile layout

    def __post_init__(self):
        p = self.params
        for name in PARAM_NAMES:
            t = p[name]
            if t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
        self.desc = MoeLayerT(self.H, self.E, self.K, self.I, self.Is,
                              _ptr(p["gate.weight"]), _ptr(p["gate_up_proj"]), _ptr(p["down_proj"]),
                              _ptr(p["shared_expert.gate.weight"]), _ptr(p["shared_expert.up.weight"]),
                              _ptr(p["shared_expert.down.weight"]), _ptr(p["shared_expert_gate.weight"]),
                              int(self.logits_bf16), int(self.experts_tiled))

    @classmethod
    def from_bf16_bits(cls, bits: dict, H: int, E: int, K: int, I: int, Is: int, device="cuda",
                       logits_bf16: bool = False):
        """Upload uint16 bf16 bit arrays (numpy) to the device as bfloat16 tensors."""
        p = {n: bits_to_device(bits[n], device) for n in PARAM_NAMES}
        return cls(H, E, K, I, Is, p, logits_bf16)

    def with_logits_bf16(self, on: bool = True) -> "MoeLayer":
        """The same device parameters with the other score precision."""
        return MoeLayer(self.H, self.E, self.K, self.I, self.Is, self.params, on, self.experts_tiled)

    def tiled(self, stream=None) -> "MoeLayer":
        """A copy of the layer with its routed experts in the MFMA-tile layout
        (moe_tile_experts); the other parameters are shared."""
        p = dict(self.params)
        p["gate_up_proj"] = torch.empty_like(p["gate_up_proj"])
        p["down_proj"] = torch.empty_like(p["down_proj"])
        rc = lib.moe_tile_experts(self.desc, _ptr(p["gate_up_proj"]), _ptr(p["down_proj"]), _stream_handle(stream))
        if rc != 0:
            raise MoeError(rc, "moe_tile_experts")
        return MoeLayer(self.H, self.E, self.K, self.I, self.Is, p, self.logits_bf16, True)

    def workspace_bytes(self, T: int) -> int:
        return int(lib.moe_workspace_bytes(self.desc, int(T)))

    def workspace(self, T: int, device=None) -> torch.Tensor:
        """A new workspace for calls of up to T tokens, zero-filled as the ABI
        requires before a workspace's first use."""
        dev = device or self.params["gate.weight"].device
        return torch.zeros(max(1, self.workspace_bytes(T)), dtype=torch.uint8, device=dev)


def bits_to_device(bits, device="cuda") -> torch.Tensor:
    """uint16 numpy array of bf16 bit patterns -> contiguous bfloat16 tensor on ``device``."""
    import numpy as np
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def workspace_status(ws: torch.Tensor, stream=None, with_count: bool = False):
    """Status of the latest call made with ``ws`` (moe_workspace_status):
    0 (MOE_OK) or MOE_ERR_TIMEOUT; synchronises the stream.  With
    ``with_count`` returns (status, calls on ws whose waits timed out)."""
    import ctypes
    n = ctypes.c_uint32(0)
    rc = lib.moe_workspace_status(_ptr(ws), ws.numel(), _stream_handle(stream), ctypes.byref(n))
    if rc not in (0, _lib.MOE_ERR_TIMEOUT):
        raise MoeError(rc, "moe_workspace_status")
    return (rc, int(n.value)) if with_count else rc


def set_wait_budget_us(us: int) -> int:
    """Budget of the fused kernel's cross-workgroup waits (moe_set_wait_budget_us);
    returns the previous one."""
    prev = int(lib.moe_set_wait_budget_us(int(us)))
    if prev < 0:
        raise ValueError(f"wait budget {us} us outside [0, 60000000]")
    return prev


def _check_x(x, layer):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != layer.H or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous bfloat16 [T, {layer.H}] tensor")


def forward(x: torch.Tensor, layer: MoeLayer, out: torch.Tensor | None = None,
            ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The MoE layer on the GPU: bf16 [T, H] -> bf16 [T, H]."""
    _check_x(x, layer)
    T = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = layer.workspace(T, x.device)
    rc = lib.moe_forward(layer.desc, _ptr(x), T, _ptr(out), _ptr(ws), ws.numel(), _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_forward")
    return out


def forward_noalloc(x: torch.Tensor, layer: MoeLayer, out: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """moe_forward_noalloc: the layer with the library's static scratch in
    place of a workspace (no device allocation inside the call)."""
    _check_x(x, layer)
    if out is None:
        out = torch.empty_like(x)
    rc = lib.moe_forward_noalloc(layer.desc, _ptr(x), x.shape[0], _ptr(out), _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_forward_noalloc")
    return out


PHASES = ("router", "dispatch", "gate_up", "down", "combine")


def forward_traced(x: torch.Tensor, layer: MoeLayer, out: torch.Tensor, ws: torch.Tensor,
                   events, stream=None) -> torch.Tensor:
    """forward() recording six timing events (torch.cuda.Event, already created)
    at the phase boundaries listed in PHASES."""
    import ctypes
    arr = (ctypes.c_void_p * 6)(*[e.cuda_event for e in events])
    rc = lib.moe_forward_traced(layer.desc, _ptr(x), x.shape[0], _ptr(out), _ptr(ws), ws.numel(),
                                _stream_handle(stream), arr)
    if rc != 0:
        raise MoeError(rc, "moe_forward_traced")
    return out


def route(x: torch.Tensor, layer: MoeLayer, ws: torch.Tensor | None = None, stream=None,
          want_logits: bool = False) -> dict:
    """Routing and dispatch only; returns device tensors."""
    _check_x(x, layer)
    T, dev = x.shape[0], x.device
    r = {
        "topk_idx": torch.empty((T, layer.K), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((T, layer.K), dtype=torch.float32, device=dev),
        "offsets": torch.empty(layer.E + 1, dtype=torch.int32, device=dev),
        "perm": torch.empty(max(1, T * layer.K), dtype=torch.int32, device=dev),
        "shared_gate": torch.empty(max(1, T), dtype=torch.float32, device=dev),
    }
    r["logits"] = torch.empty((T, layer.E), dtype=torch.float32, device=dev) if want_logits else None
    if ws is None:
        ws = layer.workspace(T, dev)
    rc = lib.moe_route(layer.desc, _ptr(x), T, _ptr(r["topk_idx"]), _ptr(r["topk_w"]), _ptr(r["offsets"]),
                       _ptr(r["perm"]), _ptr(r["shared_gate"]), _ptr(r["logits"]), _ptr(ws), ws.numel(),
                       _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_route")
    return r


def load_balance(x: torch.Tensor, layer: MoeLayer, ws: torch.Tensor | None = None, stream=None) -> dict:
    """Router load-balance statistic (moe_load_balance); returns device tensors
    lb [1], mean_prob [E] and counts [E]."""
    _check_x(x, layer)
    T, dev = x.shape[0], x.device
    r = {
        "lb": torch.empty(1, dtype=torch.float32, device=dev),
        "mean_prob": torch.empty(layer.E, dtype=torch.float32, device=dev),
        "counts": torch.empty(layer.E, dtype=torch.int32, device=dev),
    }
    if ws is None:
        ws = layer.workspace(T, dev)
    rc = lib.moe_load_balance(layer.desc, _ptr(x), T, _ptr(r["lb"]), _ptr(r["mean_prob"]), _ptr(r["counts"]),
                              _ptr(ws), ws.numel(), _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_load_balance")
    return r


def block_forward(h: torch.Tensor, layer: MoeLayer, norm_w: torch.Tensor, eps: float,
                  out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The MoE sub-block out = h + layer(RMSNorm(h)) (moe_block_forward)."""
    _check_x(h, layer)
    if norm_w.dtype != torch.bfloat16 or norm_w.numel() != layer.H or not norm_w.is_contiguous():
        raise ValueError("norm_w must be a contiguous bf16 tensor of hidden elements")
    T = h.shape[0]
    if out is None:
        out = torch.empty_like(h)
    if ws is None:
        ws = layer.workspace(T, h.device)
    rc = lib.moe_block_forward(layer.desc, _ptr(norm_w), float(eps), _ptr(h), T, _ptr(out), _ptr(ws), ws.numel(),
                               _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_block_forward")
    return out


def rmsnorm(h: torch.Tensor, norm_w: torch.Tensor, eps: float, stream=None) -> torch.Tensor:
    """x = bf16(RMSNorm(h)) (moe_rmsnorm); h bf16 [T, H]."""
    if h.dtype != torch.bfloat16 or h.dim() != 2 or not h.is_contiguous():
        raise ValueError("h must be a contiguous bf16 [T, H] tensor")
    x = torch.empty_like(h)
    rc = lib.moe_rmsnorm(_ptr(norm_w), float(eps), _ptr(h), h.shape[0], h.shape[1], _ptr(x), _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_rmsnorm")
    return x


def ranks(logits: torch.Tensor, stream=None) -> torch.Tensor:
    """Stable ranks of every expert per row (moe_ranks); logits fp32 or bf16 [R, E]."""
    if logits.dim() != 2 or not logits.is_contiguous() or logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be a contiguous fp32 or bf16 [R, E] tensor")
    out = torch.empty(logits.shape, dtype=torch.int32, device=logits.device)
    rc = lib.moe_ranks(_ptr(logits), 1 if logits.dtype == torch.bfloat16 else 0, logits.shape[0], logits.shape[1],
                       _ptr(out), _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_ranks")
    return out


def expert_cache(layer: MoeLayer, capacity: int, device="cuda") -> torch.Tensor:
    """Device memory for an expert cache of ``capacity`` slots (moe_expert_cache_bytes)."""
    n = int(lib.moe_expert_cache_bytes(layer.desc, int(capacity)))
    if n == 0:
        raise ValueError("capacity must be at least 1")
    return torch.empty(n, dtype=torch.uint8, device=device)


def forward_streamed(x: torch.Tensor, layer: MoeLayer, cache: torch.Tensor, out: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The layer with gate_up_proj / down_proj in pinned host memory, the routed
    experts streamed into ``cache`` on demand (moe_forward_streamed)."""
    _check_x(x, layer)
    T = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = layer.workspace(T, x.device)
    rc = lib.moe_forward_streamed(layer.desc, _ptr(x), T, _ptr(out), _ptr(cache), cache.numel(), _ptr(ws),
                                  ws.numel(), _stream_handle(stream))
    if rc != 0:
        raise MoeError(rc, "moe_forward_streamed")
    return out

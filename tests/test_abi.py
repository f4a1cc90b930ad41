"""The C ABI without a GPU: the library loads, exports what include/moe.h
declares, and its host-side checks return the documented codes before any
HIP call (fake, never-dereferenced pointers are enough for that)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_top8_amd as moe
from sparse_mixture_experts_top8_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced by the checks


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def _layer(H=2048, E=256, K=8, I=512, Is=512, ptr=FAKE):
    return _lib.MoeLayerT(H, E, K, I, Is, *([ptr] * 7))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)\b", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(_lib.lib, name)


def test_strerror_covers_codes():
    for code in range(9):
        assert _lib.strerror(code) and _lib.strerror(code) != "unknown status code"
    assert _lib.strerror(99) == "unknown status code"


def test_workspace_bytes():
    L = _layer()
    assert _lib.lib.moe_workspace_bytes(L, 0) == 0
    assert _lib.lib.moe_workspace_bytes(L, -1) == 0
    sizes = [_lib.lib.moe_workspace_bytes(L, T) for T in (1, 64, 4096, 16384)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    # At least the per-slot bf16 expert outputs and intermediates must fit.
    T = 4096
    assert sizes[2] >= (T * 8 + T) * 2048 * 2 + T * 8 * 512 * 2
    assert _lib.lib.moe_workspace_bytes(_layer(H=100), 4) == 0


def test_workspace_bytes_never_decrease():
    # A workspace sized for T serves every batch of 1..T tokens: the size is
    # non-decreasing across every switch of the paths (fused decode at 16
    # tokens, 32-row GEMM tiles, router tile sizes and H splits).
    for dims in [(2048, 256, 8, 512, 512), (256, 16, 4, 64, 64), (2048, 256, 1, 512, 512),
                 (2048, 64, 8, 512, 512), (256, 8, 8, 64, 64)]:
        L = _layer(*dims)
        prev = 0
        for T in range(1, 20001):
            b = _lib.lib.moe_workspace_bytes(L, T)
            assert b >= prev, (dims, T, prev, b)
            prev = b


def _validate(L, x=FAKE, T=4, out=FAKE, ws=FAKE, nbytes=None):
    if nbytes is None:
        nbytes = _lib.lib.moe_workspace_bytes(L, max(T, 1))
    return _lib.lib.moe_validate(L, x, T, out, ws, nbytes)


def test_validate_accepts_good_arguments():
    assert _validate(_layer()) == _lib.MOE_OK
    assert _validate(_layer(H=256, E=16, K=4, I=64, Is=64)) == _lib.MOE_OK
    assert _validate(_layer(), x=None, out=None, ws=None, T=0, nbytes=0) == _lib.MOE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(H=2000), _lib.MOE_ERR_SHAPE), (dict(H=0), _lib.MOE_ERR_SHAPE),
    (dict(E=0), _lib.MOE_ERR_SHAPE), (dict(E=257), _lib.MOE_ERR_SHAPE),
    (dict(K=0), _lib.MOE_ERR_SHAPE), (dict(K=9), _lib.MOE_ERR_SHAPE),
    (dict(E=4, K=5), _lib.MOE_ERR_SHAPE), (dict(I=500), _lib.MOE_ERR_SHAPE),
    (dict(Is=0), _lib.MOE_ERR_SHAPE), (dict(ptr=FAKE + 8), _lib.MOE_ERR_ALIGN),
])
def test_validate_rejects_layer(kw, code):
    assert _validate(_layer(**kw)) == code
    assert _lib.last_error()


def test_validate_rejects_call_arguments():
    L = _layer()
    assert _validate(L, T=-1) == _lib.MOE_ERR_SHAPE
    assert _validate(L, T=(1 << 22) + 1, nbytes=1 << 62) == _lib.MOE_ERR_SHAPE
    assert _validate(L, x=None) == _lib.MOE_ERR_NULL
    assert _validate(L, out=None) == _lib.MOE_ERR_NULL
    assert _validate(L, ws=None) == _lib.MOE_ERR_NULL
    assert _validate(L, x=FAKE + 2) == _lib.MOE_ERR_ALIGN
    assert _validate(L, out=FAKE + 4) == _lib.MOE_ERR_ALIGN
    assert _validate(L, ws=FAKE + 8) == _lib.MOE_ERR_ALIGN
    need = _lib.lib.moe_workspace_bytes(L, 4)
    assert _validate(L, nbytes=need - 1) == _lib.MOE_ERR_WORKSPACE
    assert "needed" in _lib.last_error()
    nulled = _layer()
    nulled.down_w = None
    assert _validate(nulled) == _lib.MOE_ERR_NULL
    assert "down_w" in _lib.last_error()
    assert _lib.lib.moe_validate(None, FAKE, 4, FAKE, FAKE, 1 << 30) == _lib.MOE_ERR_NULL


def test_entry_points_fail_before_any_hip_call():
    L = _layer()
    need = _lib.lib.moe_workspace_bytes(L, 4)
    assert _lib.lib.moe_forward(L, FAKE, 4, FAKE, FAKE, need - 1, None) == _lib.MOE_ERR_WORKSPACE
    assert _lib.lib.moe_forward(L, FAKE, -3, FAKE, FAKE, need, None) == _lib.MOE_ERR_SHAPE
    assert _lib.lib.moe_forward(L, None, 0, None, None, 0, None) == _lib.MOE_OK
    assert _lib.lib.moe_route(L, FAKE, 4, None, FAKE, FAKE, FAKE, None, None, FAKE, need, None) == _lib.MOE_ERR_NULL
    assert _lib.lib.moe_route(L, FAKE, 4, FAKE + 4, FAKE, FAKE, FAKE, None, None, FAKE, need, None) == _lib.MOE_ERR_ALIGN
    assert _lib.lib.moe_route(L, FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, need - 1, None) == _lib.MOE_ERR_WORKSPACE
    assert _lib.lib.moe_route(L, None, 0, None, None, None, None, None, None, None, 0, None) == _lib.MOE_OK
    assert _lib.lib.moe_load_balance(L, FAKE, 4, None, None, None, FAKE, need, None) == _lib.MOE_ERR_NULL
    assert _lib.lib.moe_load_balance(L, FAKE + 4, 4, FAKE, None, None, FAKE, need, None) == _lib.MOE_ERR_ALIGN
    assert _lib.lib.moe_load_balance(L, FAKE, 4, FAKE + 2, None, None, FAKE, need, None) == _lib.MOE_ERR_ALIGN
    assert _lib.lib.moe_load_balance(L, FAKE, 4, FAKE, FAKE, FAKE, FAKE, need - 1, None) == _lib.MOE_ERR_WORKSPACE
    assert _lib.lib.moe_load_balance(L, FAKE, -1, FAKE, None, None, FAKE, need, None) == _lib.MOE_ERR_SHAPE
    assert _lib.lib.moe_load_balance(L, None, 0, None, None, None, None, 0, None) == _lib.MOE_OK


def test_python_wrappers_check_inputs():
    import torch
    layer_bits_shape = dict(H=256, E=16, K=4, I=64, Is=64)
    params = {n: torch.zeros(4, dtype=torch.bfloat16) for n in moe.PARAM_NAMES}
    layer = moe.MoeLayer(params=params, **layer_bits_shape)
    with pytest.raises(ValueError):
        moe.forward(torch.zeros(3, 255, dtype=torch.bfloat16), layer)
    with pytest.raises(ValueError):
        moe.forward(torch.zeros(3, 256, dtype=torch.float32), layer)
    with pytest.raises(ValueError):
        moe.MoeLayer(params={n: torch.zeros(4) for n in moe.PARAM_NAMES}, **layer_bits_shape)


def test_layer_struct_matches_header(tmp_path):
    # The ctypes mirror of moe_layer_t has the C compiler's size and offsets.
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "moe.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu\\n", sizeof(moe_layer_t), '
                   'offsetof(moe_layer_t, shared_expert_gate_w), offsetof(moe_layer_t, logits_bf16), '
                   'offsetof(moe_layer_t, experts_tiled)); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    size, gate_off, flag_off, tiled_off = map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                                                  check=True).stdout.split())
    assert ctypes.sizeof(_lib.MoeLayerT) == size
    assert _lib.MoeLayerT.shared_expert_gate_w.offset == gate_off
    assert _lib.MoeLayerT.logits_bf16.offset == flag_off
    assert _lib.MoeLayerT.experts_tiled.offset == tiled_off


def test_logits_mode_and_ranks_checks():
    L = _layer()
    assert _validate(L) == _lib.MOE_OK
    L.logits_bf16 = 1
    assert _validate(L) == _lib.MOE_OK
    L.logits_bf16 = 2
    assert _validate(L) == _lib.MOE_ERR_SHAPE and "logits_bf16" in _lib.last_error()
    assert _lib.lib.moe_workspace_bytes(L, 4) == 0
    rk = _lib.lib.moe_ranks
    assert rk(FAKE, 0, 0, 256, FAKE, None) == _lib.MOE_OK
    assert rk(FAKE, 2, 4, 256, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert rk(FAKE, 0, 4, 0, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert rk(FAKE, 0, 4, 257, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert rk(FAKE, 0, -1, 256, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert rk(None, 0, 4, 256, FAKE, None) == _lib.MOE_ERR_NULL
    assert rk(FAKE, 0, 4, 256, None, None) == _lib.MOE_ERR_NULL
    assert rk(FAKE + 2, 0, 4, 256, FAKE, None) == _lib.MOE_ERR_ALIGN
    assert rk(FAKE, 0, 4, 256, FAKE + 2, None) == _lib.MOE_ERR_ALIGN
    assert rk(FAKE + 1, 1, 4, 256, FAKE, None) == _lib.MOE_ERR_ALIGN


def test_streamed_entry_point_checks():
    L = _layer()
    per = _lib.lib.moe_expert_cache_bytes(L, 1)
    assert per == (2 * 512 * 2048 + 2048 * 512) * 2
    assert _lib.lib.moe_expert_cache_bytes(L, 8) == 8 * per
    assert _lib.lib.moe_expert_cache_bytes(L, 0) == 0
    assert _lib.lib.moe_expert_cache_bytes(_layer(H=100), 4) == 0
    need = _lib.lib.moe_workspace_bytes(L, 4)
    fs = _lib.lib.moe_forward_streamed
    assert fs(L, None, 0, None, None, 0, None, 0, None) == _lib.MOE_OK
    assert fs(L, FAKE, 4, FAKE, None, per, FAKE, need, None) == _lib.MOE_ERR_NULL
    assert fs(L, FAKE, 4, FAKE, FAKE + 8, per, FAKE, need, None) == _lib.MOE_ERR_ALIGN
    assert fs(L, FAKE, 4, FAKE, FAKE, per - 1, FAKE, need, None) == _lib.MOE_ERR_WORKSPACE
    assert fs(L, FAKE, 4, FAKE, FAKE, per, FAKE, need - 1, None) == _lib.MOE_ERR_WORKSPACE
    assert fs(L, FAKE, -2, FAKE, FAKE, per, FAKE, need, None) == _lib.MOE_ERR_SHAPE


def test_tile_experts_checks():
    L = _layer()
    te = _lib.lib.moe_tile_experts
    assert te(L, None, FAKE, None) == _lib.MOE_ERR_NULL
    assert te(L, FAKE, FAKE + 4, None) == _lib.MOE_ERR_ALIGN
    assert te(_layer(H=100), FAKE, FAKE, None) == _lib.MOE_ERR_SHAPE
    L.experts_tiled = 1
    assert te(L, FAKE, FAKE, None) == _lib.MOE_ERR_SHAPE and "already" in _lib.last_error()
    assert _validate(L) == _lib.MOE_OK
    L.experts_tiled = 3
    assert _validate(L) == _lib.MOE_ERR_SHAPE and "experts_tiled" in _lib.last_error()


def test_workspace_control_block_and_status_checks():
    # Every workspace starts with the same control block, whatever the path
    # and batch size, and the status query rejects bad arguments before any
    # HIP call.
    cb = _lib.lib.moe_workspace_control_bytes()
    assert cb > 0 and cb % 256 == 0
    for dims in [(2048, 256, 8, 512, 512), (256, 16, 4, 64, 64)]:
        for T in (1, 16, 17, 4096):
            assert _lib.lib.moe_workspace_bytes(_layer(*dims), T) > cb
    st = _lib.lib.moe_workspace_status
    assert st(None, cb, None, None) == _lib.MOE_ERR_NULL
    assert st(FAKE + 4, cb, None, None) == _lib.MOE_ERR_ALIGN
    assert st(FAKE, cb - 1, None, None) == _lib.MOE_ERR_WORKSPACE
    assert "control" in _lib.last_error()


def test_wait_budget_setter():
    sb = _lib.lib.moe_set_wait_budget_us
    prev = sb(250000)
    assert prev == 250000            # the documented default
    assert sb(0) == 250000
    assert sb(-1) == -1 and sb(60000001) == -1   # rejected, nothing changed
    assert sb(250000) == 0
    assert sb(250000) == 250000


def test_noalloc_entry_point_checks():
    # Argument checks and the scratch limit come before any HIP call.
    L = _layer()
    fn = _lib.lib.moe_forward_noalloc
    assert fn(L, None, 0, None, None) == _lib.MOE_OK
    assert fn(L, None, 4, FAKE, None) == _lib.MOE_ERR_NULL
    assert fn(L, FAKE, 4, None, None) == _lib.MOE_ERR_NULL
    assert fn(L, FAKE + 2, 4, FAKE, None) == _lib.MOE_ERR_ALIGN
    assert fn(L, FAKE, -1, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert fn(_layer(H=100), FAKE, 4, FAKE, None) == _lib.MOE_ERR_SHAPE
    # 16 MiB of scratch: 244 tokens fit at full shape, 245 do not.
    assert _lib.lib.moe_workspace_bytes(L, 244) <= 16 << 20 < _lib.lib.moe_workspace_bytes(L, 245)
    assert fn(L, FAKE, 245, FAKE, None) == _lib.MOE_ERR_WORKSPACE
    assert "static scratch" in _lib.last_error()

"""moe_forward_noalloc (static scratch in place of a workspace) against
moe_forward through the C ABI: the same kernels on the same values, so the
outputs must be identical bit for bit, call after call, including a call with a
smaller batch right after a larger one (the scratch keeps the previous call's
contents) and across the fused decode / grouped path switch.  Also checked
against the float64 oracle to the layer's tolerance."""
import sys

import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _moe():
    import sparse_mixture_experts_top8_amd as moe
    return moe


@pytest.fixture(scope="module")
def layers():
    moe = _moe()
    toy_bits = mi.workload_layer(mi.WORKLOADS["toy"])
    d = mi.TOY
    toy = moe.MoeLayer.from_bf16_bits(toy_bits, d.H, d.E, d.K, d.I, d.Is, "cuda")
    full_bits = mi.workload_layer(mi.WORKLOADS["decode1"])
    f = mi.FULL
    full = moe.MoeLayer.from_bf16_bits(full_bits, f.H, f.E, f.K, f.I, f.Is, "cuda").tiled()
    return {"toy": (d, toy_bits, toy), "full": (f, full_bits, full)}


def _pair(moe, layer, xb):
    x = moe.bits_to_device(xb, "cuda")
    got = moe.forward_noalloc(x, layer)
    ref = moe.forward(x, layer)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("shape,sizes", [("toy", (300, 40)), ("toy", (16, 3)), ("full", (200, 64)),
                                         ("full", (64, 16)), ("full", (16, 1))])
def test_noalloc_matches_forward_twice(layers, shape, sizes):
    moe = _moe()
    d, bits, layer = layers[shape]
    for i, T in enumerate(sizes):
        _say(f"case noalloc {shape} call {i} T={T}")
        xb = mi.make_x(d, T, 12000 + 10 * T + i)
        got, ref = _pair(moe, layer, xb)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (shape, T)
        if T <= 64:
            gi = moe.route(moe.bits_to_device(xb, "cuda"), layer)["topk_idx"].cpu().numpy()
            want = O.forward_with_routing(xb, bits, gi)
            g = got.float().cpu().numpy().astype(np.float64)
            assert np.abs(g - want).max() <= 2e-2
            assert np.linalg.norm(g - want) / np.linalg.norm(want) <= 1e-2


def test_noalloc_refuses_a_batch_beyond_the_scratch(layers):
    moe = _moe()
    d, _, layer = layers["full"]
    x = torch.zeros((4096, d.H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.forward_noalloc(x, layer)
    assert e.value.code == moe._lib.MOE_ERR_WORKSPACE
    # Nothing was enqueued, and the entry point still serves smaller batches.
    xb = mi.make_x(d, 5, 12999)
    got, ref = _pair(moe, layer, xb)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))

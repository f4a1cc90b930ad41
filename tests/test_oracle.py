"""Pins for the CPU oracle: facts the pages print, closed forms, special cases,
brute force on tiny inputs and library routines.  CPU only.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
sign, a transposed operand, a wrong tie order, a wrong half of the merged
gate_up tensor) makes at least one of them fail.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as mi
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(a):
    return mi.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _random_layer(dims, seed, std=0.02):
    return mi.make_layer(dims, seed, std=std)


# ---------------------------------------------------------------------------
# Figures the pages print.
# ---------------------------------------------------------------------------

def _golden_counts():
    rows = {}
    with open(os.path.join(GOLDEN, "param_counts.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, value, digits, _src = [c.strip() for c in line.split("|", 3)]
            rows[name] = (value, digits)
    return rows


def _round_sig(v, d):
    return float(f"{v:.{d - 1}e}")


def test_param_counts_match_printed_figures():
    g = _golden_counts()
    d = mi.FULL
    per_expert = O.expert_param_count(d.H, d.I)
    assert per_expert == 3 * 2048 * 512 == 3_145_728
    for key in ("expert_params_p1", "expert_params_p2"):
        value, digits = g[key]
        assert _round_sig(per_expert, int(digits)) == float(value)
    value, digits = g["active_expert_params"]
    assert _round_sig(d.K * per_expert, int(digits)) == float(value)
    # "806M total": the routed experts alone give 805.3M; with the router
    # (256 x 2048) the printed 806M is reproduced, so the figure includes it.
    value, digits = g["total_expert_params"]
    routed = d.E * per_expert
    assert _round_sig(routed, int(digits)) != float(value)
    assert _round_sig(routed + d.E * d.H, int(digits)) == float(value)
    shapes = d.shapes()
    assert shapes["gate_up_proj"] == tuple(int(v) for v in g["merged_gate_up_shape"][0].split(","))
    assert shapes["down_proj"] == tuple(int(v) for v in g["down_shape"][0].split(","))
    assert shapes["gate.weight"] == tuple(int(v) for v in g["router_shape"][0].split(","))
    assert d.K == int(g["top_k"][0])


# ---------------------------------------------------------------------------
# bf16 codec (IEEE facts).
# ---------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x4049: 3.140625, 0x3C23: 0.0099487305,
        0x0000: 0.0, 0x7F7F: 3.3895313892515355e38, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133,
    }
    got = O.bf16_to_f64(np.array(list(cases), dtype=np.uint16))
    for (bits, want), g in zip(cases.items(), got):
        assert g == pytest.approx(want, rel=1e-7, abs=0), hex(bits)
    assert math.copysign(1.0, O.bf16_to_f64(np.array([0x8000], np.uint16))[0]) == -1.0


def test_bf16_encoder_rounds_to_nearest_even():
    # 1 + 2^-8 is half way between 1 and 1 + 2^-7: ties go to the even pattern 0x3F80.
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    assert list(_bits(v)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
    r = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    back = O.bf16_to_f64(_bits(r))
    assert np.all(np.abs(back - r) <= np.abs(r) * 2.0 ** -8)


# ---------------------------------------------------------------------------
# Activations: closed forms and a library implementation.
# ---------------------------------------------------------------------------

def test_activation_closed_forms():
    assert O.sigmoid(0.0) == 0.5
    assert O.silu(0.0) == 0.0
    assert O.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    assert O.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert O.sigmoid(800.0) == 1.0 and O.sigmoid(-800.0) == 0.0
    assert O.silu(-800.0) == 0.0 and O.silu(800.0) == 800.0
    z = np.random.default_rng(1).standard_normal(4096) * 6
    t = torch.from_numpy(z)
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.sigmoid(z), torch.sigmoid(t).numpy(), rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------------------
# Router: brute-force dot products.
# ---------------------------------------------------------------------------

def test_router_logits_brute_force():
    rng = np.random.default_rng(2)
    x = _bits(rng.standard_normal((3, 8)))
    w = _bits(rng.standard_normal((5, 8)) * 0.02)
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(w)
    want = np.array([[math.fsum(xf[t, h] * wf[e, h] for h in range(8)) for e in range(5)] for t in range(3)])
    np.testing.assert_allclose(O.router_logits(x, w), want, rtol=1e-15, atol=1e-18)


# ---------------------------------------------------------------------------
# Ranks / top-K / renormalisation.
# ---------------------------------------------------------------------------

def _brute_topk(l, K):
    order = sorted(range(len(l)), key=lambda e: (-l[e], e))
    return order[:K], {e: r for r, e in enumerate(order)}


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    E, K = 12, 4
    # Integer-valued logits produce many exact ties.
    logits = rng.integers(-3, 4, size=(20, E)).astype(np.float64)
    logits[0] = 0.0
    idx, w = O.select_topk(logits, K)
    r = O.ranks(logits)
    for t in range(logits.shape[0]):
        want_idx, want_rank = _brute_topk(list(logits[t]), K)
        assert list(idx[t]) == want_idx
        assert [r[t, e] for e in range(E)] == [want_rank[e] for e in range(E)]
        # Weights: softmax over only the selected logits is the same quantity.
        sel = logits[t, want_idx]
        ref = np.exp(sel - sel.max())
        np.testing.assert_allclose(w[t], ref / ref.sum(), rtol=1e-13)
    assert list(idx[0]) == [0, 1, 2, 3]


def test_topk_invariants_on_toy_workload():
    wl = mi.WORKLOADS["toy"]
    layer = mi.workload_layer(wl)
    x = mi.workload_x(wl)
    R = O.route(x, layer, wl.dims.K)
    idx, w = R["topk_idx"], R["topk_w"]
    assert idx.shape == (wl.T, wl.dims.K) and idx.dtype == np.int32
    assert np.all((idx >= 0) & (idx < wl.dims.E))
    assert all(len(set(row)) == wl.dims.K for row in idx)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    sel_logits = np.take_along_axis(R["logits"], idx.astype(np.int64), axis=1)
    assert np.all(np.diff(sel_logits, axis=1) <= 0)
    # Everything not selected scores no higher than the K-th selected logit.
    for t in range(wl.T):
        rest = np.delete(R["logits"][t], idx[t])
        assert rest.max() <= sel_logits[t, -1]


def test_topk_special_cases():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((7, 16))
    # K = E: the renormalised weights are the plain softmax over all experts.
    idx, w = O.select_topk(logits, 16)
    full = scipy.special.softmax(logits, axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, idx.astype(np.int64), axis=1), w, rtol=1e-13)
    # K = 1: the single weight is exactly 1 and the index is the argmax.
    idx1, w1 = O.select_topk(logits, 1)
    assert np.all(w1 == 1.0) and np.array_equal(idx1[:, 0], np.argmax(logits, axis=1))
    # x = 0: all logits tie, every token is flagged, experts 0..K-1 with weight 1/K.
    d = mi.TOY
    layer = _random_layer(d, 5)
    x0 = np.zeros((4, d.H), np.uint16)
    R = O.route(x0, layer, d.K)
    assert np.all(R["topk_idx"] == np.arange(d.K)) and np.allclose(R["topk_w"], 1.0 / d.K)
    assert R["tie"].all()


def test_tie_flags_boundaries():
    K = 3
    base = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.0])
    rows = [base.copy() for _ in range(5)]
    rows[1][1] = 5.0 - 5e-7          # gap inside the top-K
    rows[2][3] = 3.0 - 5e-7          # gap across the K / K+1 boundary
    rows[3][4] = 2.0 - 5e-7          # gap below rank K+1 only: harmless
    rows[4][3] = 3.0 - 2e-6          # gap across the boundary but above 1e-6
    flags = O.tie_flags(np.array(rows)[:, ::-1].copy(), K)   # order of columns is irrelevant
    assert list(flags) == [False, True, True, False, False]


# ---------------------------------------------------------------------------
# Counting sort.
# ---------------------------------------------------------------------------

def _loop_counting_sort(topk_idx, E):
    """Textbook counting sort written out with loops: histogram, scan, cursor scatter."""
    keys = [int(v) for v in np.asarray(topk_idx).reshape(-1)]
    counts = [0] * E
    for k in keys:
        counts[k] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E]
    perm = [0] * len(keys)
    for q, k in enumerate(keys):
        perm[cursor[k]] = q
        cursor[k] += 1
    return counts, offsets, perm


@pytest.mark.parametrize("T,E,K,mode", [(8, 16, 4, "random"), (37, 16, 4, "random"),
                                        (64, 256, 8, "random"), (50, 16, 4, "same"),
                                        (0, 16, 4, "random"), (1, 256, 8, "random")])
def test_counting_sort_brute_force(T, E, K, mode):
    rng = np.random.default_rng(T * 31 + E)
    if mode == "same":
        idx = np.tile(np.array([3, 0, 15, 7], np.int32), (T, 1))
    else:
        idx = np.array([rng.permutation(E)[:K] for _ in range(T)], dtype=np.int32).reshape(T, K)
    d = O.counting_sort(idx, E)
    counts, offsets, perm = _loop_counting_sort(idx, E)
    assert list(d["counts"]) == counts and list(d["offsets"]) == offsets and list(d["perm"]) == perm
    assert d["offsets"][E] == T * K and np.all(np.diff(d["offsets"]) >= 0)
    assert np.array_equal(np.sort(d["perm"]), np.arange(T * K))
    assert np.array_equal(d["perm"][d["slot_of"]], np.arange(T * K))
    for e in range(E):
        seg = d["perm"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.all(idx.reshape(-1)[seg] == e)
        assert np.all(np.diff(seg // K) > 0)     # strictly increasing token within a segment


# ---------------------------------------------------------------------------
# The whole layer.
# ---------------------------------------------------------------------------

def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    params = {k: _bits(g[k]) for k in mi.PARAM_NAMES}
    x = _bits(g["x"])
    K = g["dims"]["K"]
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))   # noqa: E731
    closed = [4 * sig(1) * sig(2) + 2 * sig(-1) * sig(2) - 1.5 * sig(1) * sig(-1),
              -4 * sig(1) * sig(2) + 0.5 * sig(-1) * sig(2) - 3 * sig(1) * sig(-1)]
    np.testing.assert_allclose(g["out"], closed, rtol=1e-15)
    R = O.route(x, params, K)
    assert R["topk_idx"].tolist() == g["topk_idx"]
    np.testing.assert_allclose(R["topk_w"][0], [sig(1), sig(-1)], rtol=1e-15)
    np.testing.assert_allclose(O.forward(x, params, K)[0], closed, rtol=1e-14)
    np.testing.assert_allclose(O.forward_dense(x, params, K)[0], closed, rtol=1e-14)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sparse_equals_dense_brute_force(seed):
    d = mi.TOY
    layer = _random_layer(d, 10 + seed)
    x = mi.make_x(d, 8 if seed else mi.WORKLOADS["toy"].T, 20 + seed)
    sparse = O.forward(x, layer, d.K)
    dense = O.forward_dense(x, layer, d.K)
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-15)


def _torch_swiglu(X, wg, wu, wd):
    X = torch.from_numpy(X)
    return (torch.nn.functional.silu(X @ torch.from_numpy(wg).T) * (X @ torch.from_numpy(wu).T)
            @ torch.from_numpy(wd).T).numpy()


def test_identical_experts_reduce_to_one_swiglu():
    # With every routed expert equal, the weights summing to one make the routed
    # part a single dense SwiGLU whatever the routing is.
    d = mi.TOY
    layer = _random_layer(d, 30)
    layer["gate_up_proj"] = np.repeat(layer["gate_up_proj"][:1], d.E, axis=0)
    layer["down_proj"] = np.repeat(layer["down_proj"][:1], d.E, axis=0)
    x = mi.make_x(d, 11, 31)
    X = O.bf16_to_f64(x)
    gu = O.bf16_to_f64(layer["gate_up_proj"][0])
    routed = _torch_swiglu(X, gu[:d.I], gu[d.I:], O.bf16_to_f64(layer["down_proj"][0]))
    s = torch.sigmoid(torch.from_numpy(X @ O.bf16_to_f64(layer["shared_expert_gate.weight"]).T)).numpy()
    shared = _torch_swiglu(X, O.bf16_to_f64(layer["shared_expert.gate.weight"]),
                           O.bf16_to_f64(layer["shared_expert.up.weight"]),
                           O.bf16_to_f64(layer["shared_expert.down.weight"]))
    np.testing.assert_allclose(O.forward(x, layer, d.K), routed + s * shared, rtol=1e-11, atol=1e-14)
    # The merged tensor's halves are not interchangeable: swapping gate and up changes the result.
    swapped = dict(layer)
    swapped["gate_up_proj"] = np.concatenate([layer["gate_up_proj"][:, d.I:], layer["gate_up_proj"][:, :d.I]], axis=1)
    assert not np.allclose(O.forward(x, swapped, d.K), O.forward(x, layer, d.K), rtol=1e-3)


def test_zero_weight_special_cases():
    d = mi.TOY
    layer = _random_layer(d, 40)
    x = mi.make_x(d, 9, 41)
    X = O.bf16_to_f64(x)
    shared = _torch_swiglu(X, O.bf16_to_f64(layer["shared_expert.gate.weight"]),
                           O.bf16_to_f64(layer["shared_expert.up.weight"]),
                           O.bf16_to_f64(layer["shared_expert.down.weight"]))
    # Zero routed down weights leave only the gated shared expert.
    z = dict(layer, down_proj=np.zeros_like(layer["down_proj"]))
    s = 1 / (1 + np.exp(-(X @ O.bf16_to_f64(layer["shared_expert_gate.weight"]).T)))
    np.testing.assert_allclose(O.forward(x, z, d.K), s * shared, rtol=1e-12, atol=1e-15)
    # A zero shared-gate row gives a gate of exactly one half.
    z2 = dict(z, **{"shared_expert_gate.weight": np.zeros_like(layer["shared_expert_gate.weight"])})
    np.testing.assert_allclose(O.forward(x, z2, d.K), 0.5 * shared, rtol=1e-12, atol=1e-15)
    # x = 0 gives an output of exactly zero.
    assert np.all(O.forward(np.zeros_like(x), layer, d.K) == 0.0)


def test_token_permutation_and_subsets():
    d = mi.TOY
    layer = _random_layer(d, 50)
    x = mi.make_x(d, 13, 51)
    out = O.forward(x, layer, d.K)
    p = np.random.default_rng(52).permutation(13)
    np.testing.assert_allclose(O.forward(x[p], layer, d.K), out[p], rtol=1e-12, atol=1e-15)
    # Tokens do not interact: the output of a subset is the subset of the output.
    sub = np.array([0, 5, 12])
    np.testing.assert_allclose(O.forward(x[sub], layer, d.K), out[sub], rtol=1e-12, atol=1e-15)


def test_forward_with_routing_matches_own_choice():
    d = mi.TOY
    layer = _random_layer(d, 60)
    x = mi.make_x(d, 10, 61)
    R = O.route(x, layer, d.K)
    np.testing.assert_allclose(O.forward_with_routing(x, layer, R["topk_idx"]),
                               O.forward(x, layer, d.K), rtol=1e-13, atol=1e-16)
    # Order of the chosen experts does not matter to the output.
    np.testing.assert_allclose(O.forward_with_routing(x, layer, R["topk_idx"][:, ::-1].copy()),
                               O.forward(x, layer, d.K), rtol=1e-13, atol=1e-16)


def test_all_k_and_e_combinations_small():
    # Brute force over small shapes, including K = E (every expert selected).
    for E, K in itertools.product([4, 8], [1, 2, 4]):
        d = mi.Dims(H=16, E=E, K=K, I=4, Is=4)
        layer = _random_layer(d, 70 + E + K, std=0.3)
        x = mi.make_x(d, 5, 80 + E)
        np.testing.assert_allclose(O.forward(x, layer, K), O.forward_dense(x, layer, K), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Skewed-load workload: the fitted router gives the intended load profile.
# ---------------------------------------------------------------------------

def test_zipf_workload_is_skewed():
    wl = mi.WORKLOADS["zipf16384"]
    gain = mi.zipf_router_gain()
    assert gain.shape == (wl.dims.E,) and np.all(gain > 0)
    router = mi.make_layer(mi.Dims(H=wl.dims.H, E=wl.dims.E, K=wl.dims.K, I=1, Is=1), wl.layer_seed,
                           router_row_gain=gain)["gate.weight"]
    # The router tensor of the workload is the same draw with the gain applied.
    x = mi.workload_x(wl)
    idx, _ = O.select_topk(O.router_logits(x, router), wl.dims.K)
    load = np.bincount(idx.reshape(-1), minlength=wl.dims.E)
    mean = wl.T * wl.dims.K / wl.dims.E
    assert load.sum() == wl.T * wl.dims.K
    assert load.max() >= 10 * mean
    assert load.max() <= 0.5 * wl.T          # an expert cannot win more than about half the tokens


# ---------------------------------------------------------------------------
# Load-balance statistic.
# ---------------------------------------------------------------------------

def _lb_brute(x, layer, K):
    """The statistic from its definition with Python loops and the math module."""
    X = O.bf16_to_f64(x)
    W = O.bf16_to_f64(layer["gate.weight"])
    T, E = X.shape[0], W.shape[0]
    counts = [0] * E
    psum = [0.0] * E
    for t in range(T):
        l = [sum(X[t, h] * W[e, h] for h in range(X.shape[1])) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-l[e], e))
        for e in order[:K]:
            counts[e] += 1
        m = max(l)
        z = [math.exp(v - m) for v in l]
        s = sum(z)
        for e in range(E):
            psum[e] += z[e] / s
    lb = E * sum((counts[e] / (T * K)) * (psum[e] / T) for e in range(E))
    return counts, [p / T for p in psum], lb


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_load_balance_brute_force(seed):
    d = mi.Dims(H=16, E=8, K=3, I=8, Is=8)
    layer = _random_layer(d, 300 + seed, std=0.5)
    x = mi.make_x(d, 6, 310 + seed)
    r = O.load_balance(x, layer, d.K)
    counts, P, lb = _lb_brute(x, layer, d.K)
    assert list(r["counts"]) == counts
    np.testing.assert_allclose(r["mean_prob"], P, rtol=1e-12, atol=1e-15)
    assert abs(r["lb"] - lb) <= 1e-12 * lb


def test_load_balance_closed_forms():
    d = mi.TOY
    layer = _random_layer(d, 320)
    # x = 0: every logit is 0, so P_e = 1/E and experts 0..K-1 take every slot:
    # lb = E * K * (1/K) * (1/E) = 1 exactly.
    r0 = O.load_balance(np.zeros((11, d.H), np.uint16), layer, d.K)
    assert list(r0["counts"][:d.K]) == [11] * d.K and r0["counts"][d.K:].sum() == 0
    np.testing.assert_allclose(r0["mean_prob"], 1.0 / d.E, rtol=0, atol=1e-15)
    assert abs(r0["lb"] - 1.0) < 1e-14
    # Fractions and mean probabilities are distributions.
    x = mi.make_x(d, 40, 321)
    r = O.load_balance(x, layer, d.K)
    assert abs(r["fraction"].sum() - 1.0) < 1e-12 and abs(r["mean_prob"].sum() - 1.0) < 1e-12
    assert r["counts"].sum() == 40 * d.K
    # Every token sends its K slots to the same experts S: lb = (E / K) P(S),
    # P(S) the batch-mean probability mass of S.  Router rows 0..K-1 get a
    # large copy of one row, so those K experts win for inputs that align with it.
    g = O.bf16_to_f64(layer["gate.weight"]).copy()
    g[: d.K] = 8.0 * g[0] + np.arange(d.K)[:, None] * 1e-3 * np.sign(g[0])
    lay2 = dict(layer, **{"gate.weight": _bits(g)})
    xa = _bits(np.tile(np.sign(g[0]), (7, 1)) * (1.0 + 0.1 * np.arange(7))[:, None])
    r2 = O.load_balance(xa, lay2, d.K)
    assert set(np.nonzero(r2["counts"])[0]) == set(range(d.K))
    assert abs(r2["lb"] - d.E / d.K * r2["mean_prob"][: d.K].sum()) < 1e-12


def test_load_balance_token_permutation():
    d = mi.TOY
    layer = _random_layer(d, 330)
    x = mi.make_x(d, 25, 331)
    r = O.load_balance(x, layer, d.K)
    rp = O.load_balance(x[np.random.default_rng(3).permutation(25)], layer, d.K)
    assert np.array_equal(r["counts"], rp["counts"])
    np.testing.assert_allclose(rp["mean_prob"], r["mean_prob"], rtol=1e-12)
    assert abs(rp["lb"] - r["lb"]) < 1e-12 * r["lb"]


# ---------------------------------------------------------------------------
# RMSNorm and the MoE sub-block.
# ---------------------------------------------------------------------------

def test_rmsnorm_closed_forms_and_library():
    rng = np.random.default_rng(5)
    H = 64
    w = _bits(rng.normal(1.0, 0.2, H))
    wf = O.bf16_to_f64(w)
    # A constant row c gives sign(c) * w when eps = 0.
    for c in (0.75, -3.0, 2.0 ** -6):
        h = _bits(np.full((1, H), c))
        np.testing.assert_allclose(O.rmsnorm(h, w, 0.0)[0], np.sign(c) * wf, rtol=1e-15, atol=0)
    h = _bits(rng.normal(0, 1.5, (5, H)))
    # Unit weight, eps = 0: every output row has mean square exactly one.
    y = O.rmsnorm(h, _bits(np.ones(H)), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-14)
    # Positive scaling of the input leaves it unchanged (eps = 0).
    h2 = _bits(O.bf16_to_f64(h) * 4.0)
    np.testing.assert_allclose(O.rmsnorm(h2, w, 0.0), O.rmsnorm(h, w, 0.0), rtol=1e-14)
    # Brute force with loops and the math module, and torch's rms_norm in float64.
    eps = 1e-6
    got = O.rmsnorm(h, w, eps)
    H64 = O.bf16_to_f64(h)
    for t in range(H64.shape[0]):
        ms = sum(v * v for v in H64[t]) / H
        for j in range(H):
            assert abs(got[t, j] - H64[t, j] / math.sqrt(ms + eps) * wf[j]) <= 1e-14 * max(1.0, abs(got[t, j]))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(H64), (H,), torch.from_numpy(wf), eps=eps).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_block_forward_reduces_to_residual_and_layer():
    d = mi.TOY
    layer = _random_layer(d, 340)
    h = mi.make_x(d, 7, 341)
    x = _bits(O.rmsnorm(h, _bits(np.ones(d.H)), 1e-6))
    idx, _ = O.select_topk(O.router_logits(x, layer["gate.weight"]), d.K)
    # The sub-block adds the layer's output to the residual stream.
    np.testing.assert_allclose(O.block_forward_with_routing(h, x, layer, idx) - O.bf16_to_f64(h),
                               O.forward_with_routing(x, layer, idx), rtol=1e-12, atol=1e-15)
    # With every down projection zero the sub-block is the identity on h.
    z = dict(layer, down_proj=np.zeros_like(layer["down_proj"]),
             **{"shared_expert.down.weight": np.zeros_like(layer["shared_expert.down.weight"])})
    assert np.array_equal(O.block_forward_with_routing(h, x, z, idx), O.bf16_to_f64(h))


def test_decoded_params_give_identical_results():
    # Parameters decoded once (the CPU baseline's timing setup) are the same
    # values: every result is bit-identical to decoding on each use.
    d = mi.TOY
    layer = _random_layer(d, 346)
    dec = O.decode_params(layer)
    assert all(v.dtype == np.float64 for v in dec.values())
    x = mi.make_x(d, 11, 347)
    assert np.array_equal(O.forward(x, dec, d.K), O.forward(x, layer, d.K))
    assert np.array_equal(O.forward_dense(x, dec, d.K), O.forward_dense(x, layer, d.K))
    for mode in (False, True):
        a, b = O.route(x, dec, d.K, mode), O.route(x, layer, d.K, mode)
        assert all(np.array_equal(a[k], b[k]) for k in a)


def test_bf16_bits_is_the_exact_encoding():
    rng = np.random.default_rng(342)
    # Every finite bf16 pattern round-trips through its value.
    b = rng.integers(0, 1 << 16, 20000, dtype=np.uint32).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]
    assert np.array_equal(O.bf16_bits(O.bf16_to_f64(b)), b)
    # Rounded values encode as the IEEE float32 -> bf16 conversion of values
    # float32 holds exactly (no double rounding in between).
    v = rng.normal(0, 3, 5000).astype(np.float32).astype(np.float64)
    assert np.array_equal(O.bf16_bits(O.round_bf16(v)), mi.f32_to_bf16_bits(v.astype(np.float32)))
    for bad in (1.0 + 2.0 ** -9, 0.1):
        with pytest.raises(ValueError):
            O.bf16_bits(np.array([bad]))


def test_block_forward_chain_closed_form():
    # Constant rows c with eps = 0: RMSNorm gives sign(c) * w exactly, a bf16
    # value, so the chain must route and evaluate exactly those activations
    # and add h.
    d = mi.TOY
    layer = _random_layer(d, 343)
    rng = np.random.default_rng(344)
    w = _bits(rng.normal(1.0, 0.2, d.H))
    cs = np.array([0.75, -3.0, 2.0 ** -6, 1.5])
    h = _bits(np.repeat(cs[:, None], d.H, axis=1))
    out, x = O.block_forward(h, w, 0.0, layer, d.K)
    want_x = _bits(np.sign(cs)[:, None] * O.bf16_to_f64(w)[None, :])
    assert np.array_equal(x, want_x)
    assert np.array_equal(out, O.bf16_to_f64(h) + O.forward(want_x, layer, d.K))
    # Token permutation permutes the rows; h = 0 gives 0 (x = 0, layer of 0 = 0).
    hr = mi.make_x(d, 9, 345)
    o1, x1 = O.block_forward(hr, w, 1e-6, layer, d.K)
    p = rng.permutation(9)
    o2, x2 = O.block_forward(hr[p], w, 1e-6, layer, d.K)
    assert np.array_equal(x2, x1[p])
    np.testing.assert_allclose(o2, o1[p], rtol=1e-12, atol=1e-15)
    oz, xz = O.block_forward(np.zeros((3, d.H), np.uint16), w, 1e-6, layer, d.K)
    assert np.all(oz == 0.0) and np.all(O.bf16_to_f64(xz) == 0.0)


# ---------------------------------------------------------------------------
# bf16-logit routing mode: the model page types the gate projections' outputs
# as T = bf16.  Rounding pinned against IEEE conversion and exact rationals;
# routing pinned by a hand-worked case and a loop brute force.
# ---------------------------------------------------------------------------

def _fraction_round_bf16(v):
    """Nearest bf16 of a float by exact rational arithmetic (Python's round of a
    Fraction is half-to-even): v = m 2^e with m in [0.5, 1); bf16 keeps 8 bits
    of m, so round(m 2^8) 2^(e-8), with the spacing floored at 2^-133."""
    from fractions import Fraction
    if v == 0.0:
        return v
    _, e = math.frexp(v)
    shift = max(e - 8, -133)
    q = round(Fraction(v) / Fraction(2) ** shift)
    return float(q * Fraction(2) ** shift)


def test_round_bf16_matches_ieee_conversion():
    rng = np.random.default_rng(40)
    # Random float32 bit patterns over every exponent, subnormals included.
    bits = rng.integers(0, 0x7F7F0000, size=20000, dtype=np.uint32)
    bits |= rng.integers(0, 2, size=bits.size, dtype=np.uint32) << np.uint32(31)
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(f.astype(np.float64)), want)
    # Midpoints go to the even significand; just above a midpoint goes up,
    # including offsets that float32 cannot hold (no double rounding).
    cases = {1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, 1 + 2 ** -8 + 2 ** -40: 1 + 2 ** -7,
             -(1 + 2 ** -8 + 2 ** -40): -(1 + 2 ** -7), 255.5: 256.0, 2.0 ** -140: 0.0,
             3 * 2.0 ** -134: 2 * 2.0 ** -133,
             # The largest finite bf16 is (2 - 2^-7) 2^127; above (2 - 2^-8) 2^127 rounds to inf.
             3.3961e38: (2 - 2 ** -7) * 2.0 ** 127, 3.3963e38: np.inf}
    got = O.round_bf16(np.array(list(cases)))
    assert list(got) == list(cases.values())
    assert math.copysign(1.0, O.round_bf16(np.array([-0.0]))[0]) == -1.0


def test_round_bf16_matches_exact_rationals():
    rng = np.random.default_rng(41)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000)
    np.testing.assert_array_equal(O.round_bf16(v), [_fraction_round_bf16(float(a)) for a in v])
    # Every bf16 value is a fixed point.
    b = rng.integers(0, 0x7F80, size=5000).astype(np.uint16)
    vals = O.bf16_to_f64(b)
    np.testing.assert_array_equal(O.round_bf16(vals), vals)


def _tie_layer():
    """A toy layer whose router gives expert 7 the score 1 + 2^-9 and expert 2
    the score 1 (for x = e_0 + 2^-9 e_1): ahead in float64, equal in bf16.
    Expert 11 scores 1 + 2^-8 (a midpoint: rounds to 1, the even neighbour) and
    expert 5 scores 1 + 3 * 2^-8 (rounds up to 1 + 2^-6).  The shared-expert
    gate scores 2^-9 + 2^-18, which rounds to 2^-9."""
    d = mi.TOY
    layer = _random_layer(d, 42)
    r = np.zeros((d.E, d.H), np.float32)
    r[:, 0] = -1.0
    r[7, :2] = [1.0, 1.0]
    r[2, :2] = [1.0, 0.0]
    r[11, :2] = [1.0, 2.0]
    r[5, :2] = [1.0, 6.0]
    layer["gate.weight"] = _bits(r)
    g = np.zeros((1, d.H), np.float32)
    g[0, :2] = [2.0 ** -9, 2.0 ** -9]
    layer["shared_expert_gate.weight"] = _bits(g)
    x = np.zeros((1, d.H), np.float32)
    x[0, :2] = [1.0, 2.0 ** -9]
    return d, layer, _bits(x)


def test_route_bf16_hand_worked():
    d, layer, x = _tie_layer()
    e9 = 2.0 ** -9
    f64 = O.route(x, layer, 4)
    assert list(f64["topk_idx"][0]) == [5, 11, 7, 2]
    assert f64["logits"][0, 5] == 1 + 6 * e9 and f64["logits"][0, 7] == 1 + e9
    b = O.route(x, layer, 4, logits_bf16=True)
    lb = b["logits"][0]
    assert lb[5] == 1 + 2 ** -6 and lb[11] == 1.0 and lb[7] == 1.0 and lb[2] == 1.0 and lb[0] == -1.0
    # 11, 7 and 2 tie at 1.0 after rounding: lower index first.
    assert list(b["topk_idx"][0]) == [5, 2, 7, 11]
    z = math.exp(2 ** -6)
    want = np.array([z, 1.0, 1.0, 1.0]) / (z + 3.0)
    np.testing.assert_allclose(b["topk_w"][0], want, rtol=1e-15)
    assert not b["tie"].any()
    # K = 2: the bf16 choice keeps expert 2 where float64 keeps 11.
    assert list(O.route(x, layer, 2, logits_bf16=True)["topk_idx"][0]) == [5, 2]
    assert list(O.route(x, layer, 2)["topk_idx"][0]) == [5, 11]
    assert b["shared_gate"][0] == O.sigmoid(e9)
    assert f64["shared_gate"][0] == O.sigmoid(e9 + e9 * e9)


@pytest.mark.parametrize("seed", range(4))
def test_route_bf16_brute_force(seed):
    rng = np.random.default_rng(43 + seed)
    T, H, E, K = 5, 16, 10, 3
    # Coarse values: many scores collide once rounded.
    x = _bits(rng.integers(-4, 5, (T, H)) * 0.25 + rng.standard_normal((T, H)) * 1e-3)
    params = {"gate.weight": _bits(rng.integers(-3, 4, (E, H)) * 0.125 + rng.standard_normal((E, H)) * 1e-3),
              "shared_expert_gate.weight": _bits(rng.standard_normal((1, H)))}
    # Expert E - 1 copies the router row of expert 1 and expert E - 2 that of
    # expert 4 with one input's weight moved by less than a bf16 step of the
    # score: equal in bf16 more often than not.
    params["gate.weight"][E - 1] = params["gate.weight"][1]
    params["gate.weight"][E - 2] = params["gate.weight"][4]
    params["gate.weight"][E - 2, 0] ^= np.uint16(1)
    R = O.route(x, params, K, logits_bf16=True)
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(params["gate.weight"])
    gf = O.bf16_to_f64(params["shared_expert_gate.weight"])
    ties = 0
    for t in range(T):
        l = [_fraction_round_bf16(math.fsum(xf[t, h] * wf[e, h] for h in range(H))) for e in range(E)]
        ties += len(l) - len(set(l))
        order = sorted(range(E), key=lambda e: (-l[e], e))
        assert list(R["topk_idx"][t]) == order[:K]
        assert list(R["logits"][t]) == l
        ex = [math.exp(l[e] - l[order[0]]) for e in order[:K]]
        np.testing.assert_allclose(R["topk_w"][t], [v / math.fsum(ex) for v in ex], rtol=1e-14)
        zg = _fraction_round_bf16(math.fsum(xf[t, h] * gf[0, h] for h in range(H)))
        assert R["shared_gate"][t] == pytest.approx(1.0 / (1.0 + math.exp(-zg)), rel=1e-15)
    assert ties > 0


def test_route_bf16_scale_and_modes():
    d = mi.TOY
    layer = _random_layer(d, 44)
    x = mi.make_x(d, 40, 45)
    # Doubling x (exponent + 1, exact for these normal values) doubles every
    # exact score; rounding to bf16 commutes with it, so the choice and the
    # rounded scores' ratios are unchanged.
    x2 = (x + np.uint16(0x80)).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f64(x2), 2 * O.bf16_to_f64(x))
    a = O.route(x, layer, d.K, logits_bf16=True)
    b = O.route(x2, layer, d.K, logits_bf16=True)
    np.testing.assert_array_equal(b["logits"], 2 * a["logits"])
    np.testing.assert_array_equal(b["topk_idx"], a["topk_idx"])
    # The rounded scores differ from float64 by at most half a bf16 step, and
    # the sparse layer equals the dense brute force in this mode too.
    f = O.route(x, layer, d.K)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(f["logits"]))) - 7)
    assert np.all(np.abs(a["logits"] - f["logits"]) <= 0.5 * ulp)
    np.testing.assert_allclose(O.forward(x, layer, d.K, logits_bf16=True),
                               O.forward_dense(x, layer, d.K, logits_bf16=True), rtol=1e-12, atol=1e-15)
    lb = O.load_balance(x, layer, d.K, logits_bf16=True)
    np.testing.assert_array_equal(lb["topk_idx"], a["topk_idx"])

"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (per output element): expert indices bit-exact except tokens the oracle
flags as router ties (two of ranks 0..K closer than 1e-6 in float64 logits);
for those, every selected expert must score within 1e-6 of the K-th best.
Offsets and the permutation are bit-exact against the oracle's counting sort
of the GPU's indices.  The shared gate within 1e-6.
Router logits within the fp32 rounding bound of their dot products.  Routing
weights against the oracle's own weights (its float64 softmax at the chosen
experts): within 1e-6 where the scores are of moderate size (the N(0, 0.02)
router), and for every router within 1e-6 plus twice the token's largest
observed logit error (a weight's sensitivity to its logits is at most that:
dw_k/dl_j = w_k (delta_kj - w_j)); also within 1e-6 of the renormalised
softmax of the GPU's own logits.
Output max-abs <= 2e-2 and relative L2 <= 1e-2 over the whole output against
the float64 oracle evaluated with the GPU's expert choice (identical to the
oracle's own for unflagged tokens).
"""
import sys

import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 1e-2
W_TOL = 1e-6
# Roundings on the longest path to one router logit (H = 2048), for both
# router implementations: at most a 32-term MFMA dot product, then 16 or
# fewer accumulator steps, plus up to 8 chunk totals or 2 cross-wave adds.
LOGIT_CHAIN = 64


def _moe():
    import sparse_mixture_experts_top8_amd as moe
    return moe


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _np(t):
    return t.cpu().numpy()


def check_routing(xb, bits, dims, r, tag, flat_w=True):
    K, E = dims.K, dims.E
    T = xb.shape[0]
    R = O.route(xb, bits, K)
    gi = _np(r["topk_idx"])
    oi = R["topk_idx"]
    tie = R["tie"]
    diff = (gi != oi).any(axis=1)
    assert not (diff & ~tie).any(), f"{tag}: index mismatch on unflagged tokens {np.nonzero(diff & ~tie)[0][:10]}"
    # Every chosen expert is a valid choice: distinct, and within the tie gap of the K-th best.
    assert all(len(set(row)) == K for row in gi)
    kth = np.sort(R["logits"], axis=1)[:, ::-1][:, K - 1]
    chosen = np.take_along_axis(R["logits"], gi.astype(np.int64), axis=1)
    assert np.all(chosen >= kth[:, None] - O.TIE_GAP), tag
    gw = _np(r["topk_w"]).astype(np.float64)
    if r.get("logits") is not None:
        # Logits: fp32 accumulation of bf16 products; the rounding bound of a
        # dot product whose longest chain of roundings is LOGIT_CHAIN steps is
        # LOGIT_CHAIN * 2^-24 * sum_h |x_h w_h|.
        gl = _np(r["logits"]).astype(np.float64)
        S = np.abs(O.bf16_to_f64(xb)) @ np.abs(O.bf16_to_f64(bits["gate.weight"])).T
        bound = LOGIT_CHAIN * 2.0 ** -24 * S
        err_l = np.abs(gl - R["logits"])
        assert np.all(err_l <= bound), f"{tag}: logit error {err_l.max():.3e}"
        # Softmax and renormalisation of the GPU's own logits: within 1e-6.
        np.testing.assert_allclose(gw, O.renormalised_weights(gl, gi), rtol=0, atol=W_TOL)
        # Against the oracle's own weights: 1e-6 plus twice the token's largest
        # logit error at the chosen experts.
        ow = O.renormalised_weights(R["logits"], gi)
        dl = np.take_along_axis(err_l, gi.astype(np.int64), axis=1).max(axis=1)
        tol = W_TOL + 2.0 * dl
        dw = np.abs(gw - ow)
        assert np.all(dw <= tol[:, None]), f"{tag}: weight error {dw.max():.3e} vs oracle beyond its bound"
        if flat_w:
            assert dw.max() <= W_TOL, f"{tag}: weight error {dw.max():.3e} vs the oracle's own weights"
        _say(f"{tag}: max logit error {err_l.max():.3e} (max bound {bound.max():.3e}), "
             f"weight error vs oracle {dw.max():.3e} (largest per-token bound {tol.max():.3e})")
    else:
        np.testing.assert_allclose(gw, O.renormalised_weights(R["logits"], gi), rtol=0, atol=W_TOL)
    d = O.counting_sort(gi, E)
    assert np.array_equal(_np(r["offsets"]), d["offsets"]), tag
    assert np.array_equal(_np(r["perm"])[:T * K], d["perm"]), tag
    np.testing.assert_allclose(_np(r["shared_gate"])[:T], R["shared_gate"], rtol=0, atol=W_TOL)
    _say(f"{tag}: routing ok, T={T}, flagged ties {int(tie.sum())}, index diffs on flagged {int(diff.sum())}")
    return gi


def check_output(xb, bits, dims, gi, out_rows, rows, tag):
    """Rows `rows` of the GPU output against the float64 oracle with the GPU's
    expert choice (evaluated expert by expert, so the whole output of a
    16384-token batch fits in host memory)."""
    ref = O.forward_with_routing(xb[rows], bits, gi[rows])
    got = out_rows.astype(np.float64)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref ** 2))
    _say(f"{tag}: rows {len(rows)} max-abs {err.max():.3e} rel-L2 {rel:.3e} (ref rms {rms:.3e})")
    assert err.max() <= MAX_ABS, tag
    assert rel <= REL_L2, tag


def call_status(ws):
    """moe_workspace_status of the latest call made with ws: 0, or
    MOE_ERR_TIMEOUT if a wait inside the fused decode kernel or the fused
    small-batch route gave up."""
    return _moe().workspace_status(ws)


def run_layer(layer, xb, want_logits=False):
    moe = _moe()
    x = moe.bits_to_device(xb, "cuda")
    T = xb.shape[0]
    ws = layer.workspace(T)
    r = moe.route(x, layer, ws=ws, want_logits=want_logits)
    assert call_status(ws) == 0, "decode path wait timed out (route)"
    out = moe.forward(x, layer, ws=ws)
    assert call_status(ws) == 0, "decode path wait timed out (forward)"
    return r, out


# ---------------------------------------------------------------------------
# Toy shape (H=256, E=16, K=4, I=Is=64): whole-output comparison.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def toy():
    moe = _moe()
    d = mi.TOY
    bits = mi.workload_layer(mi.WORKLOADS["toy"])
    return d, bits, moe.MoeLayer.from_bf16_bits(bits, d.H, d.E, d.K, d.I, d.Is, "cuda")


# 2048 / 2049: the last batch dispatched by one workgroup and the first by the
# multi-launch dispatch (router block histograms); 6000: ~1500 slots per toy
# expert, more than eight 160-row tiles, so the groups' tiles are listed in
# blocks of eight row tiles; 9000: 128-token router tiles.
@pytest.mark.parametrize("T", [8, 1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 129, 300, 1000, 2048, 2049,
                               6000, 9000])
def test_toy_parity(toy, T):
    d, bits, layer = toy
    _say(f"case toy T={T}")
    xb = mi.workload_x(mi.WORKLOADS["toy"]) if T == 8 else mi.make_x(d, T, 1000 + T)
    r, out = run_layer(layer, xb, want_logits=True)
    gi = check_routing(xb, bits, d, r, f"toy T={T}")
    check_output(xb, bits, d, gi, _np(out.float()), np.arange(T), f"toy T={T}")


def test_toy_small_inputs_and_ties(toy):
    d, bits, layer = toy
    _say("case toy x~N(0,0.02)")
    xb = mi.make_x(d, 200, 77, std=0.02)
    r, out = run_layer(layer, xb)
    gi = check_routing(xb, bits, d, r, "toy small x")
    check_output(xb, bits, d, gi, _np(out.float()), np.arange(200), "toy small x")


def test_toy_zero_input_all_ties(toy):
    d, bits, layer = toy
    _say("case toy x=0")
    xb = np.zeros((40, d.H), np.uint16)
    r, out = run_layer(layer, xb)
    assert np.all(_np(r["topk_idx"]) == np.arange(d.K))
    np.testing.assert_allclose(_np(r["topk_w"]), 1.0 / d.K, rtol=0, atol=1e-7)
    assert np.all(_np(out.float()) == 0.0)


def test_toy_duplicate_router_rows_tie_to_lower_index():
    # Router rows 2j and 2j+1 identical: their logits are equal bit for bit on
    # both paths, so whenever expert 2j+1 is chosen, 2j must be chosen right
    # before it with the same weight (ties go to the lower expert index).
    moe = _moe()
    for E, K in [(16, 4), (256, 8)]:
        d = mi.Dims(H=256, E=E, K=K, I=64, Is=64)
        bits = mi.make_layer(d, 900 + E)
        g = bits["gate.weight"].copy()
        g[1::2] = g[0::2]
        bits["gate.weight"] = g
        layer = moe.MoeLayer.from_bf16_bits(bits, d.H, d.E, d.K, d.I, d.Is, "cuda")
        for T in (1, 5, 16, 100):
            _say(f"case toy duplicate router rows E={E} K={K} T={T}")
            xb = mi.make_x(d, T, 950 + T)
            r, _ = run_layer(layer, xb)
            gi, gw = _np(r["topk_idx"]), _np(r["topk_w"])
            for t in range(T):
                for k in range(K):
                    e = int(gi[t, k])
                    if e % 2 == 1:
                        assert k > 0 and gi[t, k - 1] == e - 1, (E, T, t, gi[t])
                        assert gw[t, k - 1] == gw[t, k], (E, T, t, gw[t])
                    elif k + 1 < K and gi[t, k + 1] == e + 1:
                        assert gw[t, k + 1] == gw[t, k]
            check_routing(xb, bits, d, r, f"dup rows E={E} T={T}")


def test_toy_other_k_and_e():
    moe = _moe()
    for (E, K) in [(8, 8), (16, 1), (32, 8), (256, 8)]:
        d = mi.Dims(H=256, E=E, K=K, I=64, Is=128)
        _say(f"case toy E={E} K={K} Is=128")
        bits = mi.make_layer(d, 500 + E + K)
        layer = moe.MoeLayer.from_bf16_bits(bits, d.H, d.E, d.K, d.I, d.Is, "cuda")
        xb = mi.make_x(d, 70, 600 + E)
        r, out = run_layer(layer, xb)
        gi = check_routing(xb, bits, d, r, f"E={E} K={K}")
        check_output(xb, bits, d, gi, _np(out.float()), np.arange(70), f"E={E} K={K}")


def test_toy_empty_and_determinism(toy):
    moe = _moe()
    d, bits, layer = toy
    _say("case toy T=0 / determinism / guard bands / permutation")
    x0 = torch.empty((0, d.H), dtype=torch.bfloat16, device="cuda")
    assert moe.forward(x0, layer).shape == (0, d.H)
    xb = mi.make_x(d, 257, 4242)
    x = moe.bits_to_device(xb, "cuda")
    # Guard bands around out and the workspace must stay untouched.
    T = xb.shape[0]
    big = torch.full((T * d.H + 2 * 4096,), 12345, dtype=torch.int16, device="cuda")
    out = big[4096:4096 + T * d.H].view(torch.bfloat16).view(T, d.H)
    need = layer.workspace_bytes(T)
    ws_big = torch.full((need + 2 * 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = ws_big[4096:4096 + need]
    moe.forward(x, layer, out=out, ws=ws)
    a = out.clone()
    moe.forward(x, layer, out=out, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out.view(torch.int16)), "not bitwise reproducible"
    assert torch.all(big[:4096] == 12345) and torch.all(big[4096 + T * d.H:] == 12345)
    assert torch.all(ws_big[:4096] == 0xA5) and torch.all(ws_big[4096 + need:] == 0xA5)
    # Permuting tokens permutes output rows bit for bit.
    p = np.random.default_rng(1).permutation(T)
    outp = moe.forward(moe.bits_to_device(xb[p], "cuda"), layer)
    torch.cuda.synchronize()
    assert torch.equal(outp.view(torch.int16).cpu(), a.view(torch.int16).cpu()[p])


def test_toy_wide_workspace_reuse(toy):
    """Large batches (T K >= 2 E 160) run gate_up persistent, each workgroup
    claiming tiles from a per-XCD counter in the workspace that the dispatch
    zeroes on every call.  One workspace, filled with 0xA5 bytes first, serves
    large batches of different sizes in turn (single- and multi-launch
    dispatch) with a smaller batch between them; every call is bit-identical
    to the same call on a fresh workspace, and one is checked against the
    oracle."""
    moe = _moe()
    d, bits, layer = toy
    Ts = [6000, 1300, 2048, 200, 6000, 2049]
    need = max(layer.workspace_bytes(T) for T in Ts)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for i, T in enumerate(Ts):
        _say(f"case toy workspace reuse call {i} T={T}")
        xb = mi.make_x(d, T, 5100 + T)
        x = moe.bits_to_device(xb, "cuda")
        a = moe.forward(x, layer, ws=ws)
        b = moe.forward(x, layer)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"T={T} (call {i}) differs from a fresh workspace"
        if i == 1:
            r, out = run_layer(layer, xb)
            gi = check_routing(xb, bits, d, r, f"toy reuse T={T}")
            check_output(xb, bits, d, gi, _np(a.float()), np.arange(T), f"toy reuse T={T}")


# ---------------------------------------------------------------------------
# Full shape (H=2048, E=256, K=8, I=Is=512).
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def full():
    moe = _moe()
    d = mi.FULL
    _say("generating the full-shape layer")
    bits = mi.workload_layer(mi.WORKLOADS["decode1"])
    layer = moe.MoeLayer.from_bf16_bits(bits, d.H, d.E, d.K, d.I, d.Is, "cuda")
    zb = dict(bits)
    zb["gate.weight"] = mi.make_router(d, mi.WORKLOADS["zipf16384"].layer_seed, mi.zipf_router_gain())
    zparams = dict(layer.params)
    zparams["gate.weight"] = moe.bits_to_device(zb["gate.weight"], "cuda")
    zlayer = moe.MoeLayer(d.H, d.E, d.K, d.I, d.Is, zparams)
    return d, bits, layer, zb, zlayer


def _sample_rows(T, gi, hot_expert=None, n=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(range(min(8, T))) | set(range(max(0, T - 8), T))
    rows |= set(rng.choice(T, size=min(n, T), replace=False).tolist())
    if hot_expert is not None:
        hot = np.nonzero((gi == hot_expert).any(axis=1))[0]
        rows |= set(hot[:8].tolist()) | set(hot[-8:].tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["decode1", "decode64", "prefill4096", "zipf16384"])
def test_full_workloads(full, name):
    d, bits, layer, zb, zlayer = full
    wl = mi.WORKLOADS[name]
    _say(f"case full {name} T={wl.T}")
    lb, ly = (zb, zlayer) if wl.skewed_router else (bits, layer)
    xb = mi.workload_x(wl)
    r, out = run_layer(ly, xb, want_logits=True)
    gi = check_routing(xb, lb, d, r, name, flat_w=not wl.skewed_router)
    counts = np.bincount(gi.reshape(-1), minlength=d.E)
    _say(f"{name}: experts touched {int((counts > 0).sum())}, max load {counts.max()}, "
         f"mean {counts.mean():.1f}")
    if wl.skewed_router:
        assert counts.max() >= 10 * counts.mean()
    # Every row of the output (4096 and 16384 rows included: the multi-launch
    # dispatch, 160-row tiles with plain weight loads and the hot experts'
    # many row tiles over all column tiles run only at these sizes).
    check_output(xb, lb, d, gi, _np(out.float()), np.arange(wl.T), name)


@pytest.mark.parametrize("T", [2049, 6000, 12000])
def test_full_past_dispatch_switch(full, T):
    # Full shape just past the one-workgroup dispatch (2048 tokens), at ~190
    # rows per expert (two 160-row tiles for most experts), and at ~375 rows
    # per expert, where the GEMM tiles go to the XCDs in units dealt in turn
    # (uniform loads: a partial last round of units), whole output.
    d, bits, layer, _, _ = full
    _say(f"case full past the dispatch switch T={T}")
    xb = mi.make_x(d, T, 9950 + T)
    r, out = run_layer(layer, xb, want_logits=True)
    gi = check_routing(xb, bits, d, r, f"full T={T}")
    check_output(xb, bits, d, gi, _np(out.float()), np.arange(T), f"full T={T}")


def test_full_decode_small_inputs(full):
    d, bits, layer, _, _ = full
    _say("case full decode x~N(0,0.02)")
    for T in (1, 5):
        xb = mi.make_x(d, T, 9000 + T, std=0.02)
        r, out = run_layer(layer, xb)
        gi = check_routing(xb, bits, d, r, f"decode small x T={T}")
        check_output(xb, bits, d, gi, _np(out.float()), np.arange(T), f"decode small x T={T}")


def test_full_decode_batches(full):
    # The fused decode path up to its largest batch (16 tokens), then the
    # first batch size past it; at 16 tokens also run-to-run bitwise
    # determinism and bitwise token-permutation equivariance.
    moe = _moe()
    d, bits, layer, _, _ = full
    for T in (2, 7, 16, 17):
        _say(f"case full decode batch T={T}")
        xb = mi.make_x(d, T, 7000 + T)
        r, out = run_layer(layer, xb, want_logits=True)
        gi = check_routing(xb, bits, d, r, f"decode batch T={T}")
        check_output(xb, bits, d, gi, _np(out.float()), np.arange(T), f"decode batch T={T}")
        if T == 16:
            x = moe.bits_to_device(xb, "cuda")
            a = moe.forward(x, layer)
            b = moe.forward(x, layer)
            p = np.random.default_rng(3).permutation(T)
            c = moe.forward(moe.bits_to_device(xb[p], "cuda"), layer)
            torch.cuda.synchronize()
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "not bitwise reproducible"
            assert torch.equal(c.view(torch.int16).cpu(), a.view(torch.int16).cpu()[p])
            assert torch.equal(a.view(torch.int16), out.view(torch.int16))


def test_full_decode_workspace_reuse(full):
    # Calls that share a workspace must not see each other's intermediate
    # values: B after A on one workspace equals B on a fresh one, bit for bit.
    moe = _moe()
    d, bits, layer, _, _ = full
    for T in (1, 16):
        _say(f"case full decode workspace reuse T={T}")
        xa = moe.bits_to_device(mi.make_x(d, T, 8100 + T), "cuda")
        xb = moe.bits_to_device(mi.make_x(d, T, 8200 + T), "cuda")
        ws = layer.workspace(T)
        fresh = moe.forward(xb, layer, ws=layer.workspace(T))
        for _ in range(3):
            moe.forward(xa, layer, ws=ws)
            got = moe.forward(xb, layer, ws=ws)
        torch.cuda.synchronize()
        assert call_status(ws) == 0
        assert torch.equal(got.view(torch.int16), fresh.view(torch.int16))


def test_decode_timeout_is_reported(full):
    # A wait budget of 0 (set from the host) makes each cross-workgroup wait
    # of the fused kernel give up at its first unsuccessful poll.  The kernel
    # still runs to completion: after a give-up it works from LDS tables
    # built from its own clamped selections and reads published data only
    # through buffer resources bounded by their arrays.  Workgroups start up
    # to ~1 us apart, so the first polls of the logit exchange miss and the
    # call must report MOE_ERR_TIMEOUT through moe_workspace_status (and count
    # in its timed-out calls); a call whose waits all succeeded at once must be
    # right.  With the budget restored the next call on the same workspace
    # reports MOE_OK and is right, and so does a grouped-path call after a
    # timed-out one.
    # The fused route of 17..64 tokens has the same bounded waits (logits to
    # selection, selections to dispatch); after a give-up its workgroups may
    # write dispatch tables from different views of the selections, which the
    # GEMMs and the combine read through clamped indices.  A batch of 65
    # tokens takes the separate router kernels, which do not wait.
    moe = _moe()
    d, bits, layer, _, _ = full
    ws = layer.workspace(65)
    timed_out = 0
    for T in (1, 16, 17, 64):
        _say(f"case full decode / fused route forced timeout T={T}")
        x = moe.bits_to_device(mi.make_x(d, T, 9990 + T), "cuda")
        good = moe.forward(x, layer, ws=ws)
        assert moe.workspace_status(ws) == 0
        prev = moe.set_wait_budget_us(0)
        try:
            for _ in range(3):
                got = moe.forward(x, layer, ws=ws)
                st = moe.workspace_status(ws)
                if st == 0:
                    assert torch.equal(got.view(torch.int16), good.view(torch.int16))
                else:
                    assert st == moe._lib.MOE_ERR_TIMEOUT
                    timed_out += 1
        finally:
            moe.set_wait_budget_us(prev)
        again = moe.forward(x, layer, ws=ws)
        st, n = moe.workspace_status(ws, with_count=True)
        assert st == 0 and n == timed_out, (st, n, timed_out)
        assert torch.equal(again.view(torch.int16), good.view(torch.int16))
    assert timed_out >= 1, "no call timed out with a zero wait budget"
    moe.set_wait_budget_us(0)
    try:
        moe.forward(moe.bits_to_device(mi.make_x(d, 16, 9995), "cuda"), layer, ws=ws)
        st16 = moe.workspace_status(ws)
        moe.forward(moe.bits_to_device(mi.make_x(d, 65, 9996), "cuda"), layer, ws=ws)
        st65 = moe.workspace_status(ws)
    finally:
        moe.set_wait_budget_us(prev)
    _say(f"forced timeouts: {timed_out} of 12 calls with waits; then fused {st16}, separate router {st65}")
    assert st65 == 0, "a call without waits reports the status of its own call"


def test_full_decode_identical_tokens(full):
    # Sixteen identical tokens: every touched expert holds all 16 pairs (a full
    # tile of columns) and all output rows must be identical.
    d, bits, layer, _, _ = full
    _say("case full decode identical tokens T=16")
    xb = np.repeat(mi.make_x(d, 1, 4711), 16, axis=0)
    r, out = run_layer(layer, xb)
    gi = check_routing(xb, bits, d, r, "identical 16")
    assert len(np.unique(gi, axis=0)) == 1
    o = out.view(torch.int16)
    assert torch.all(o == o[0:1]).item()
    check_output(xb[:1], bits, d, gi[:1], _np(out.float())[:1], np.arange(1), "identical 16")


def test_full_forced_routing_one_hot_segment(full):
    # Identical tokens: all pick the same 8 experts, so 8 segments hold every
    # token and 248 experts are empty; all output rows must be identical.
    moe = _moe()
    d, bits, layer, _, _ = full
    _say("case full forced routing T=777")
    xb = np.repeat(mi.make_x(d, 1, 31337), 777, axis=0)
    r, out = run_layer(layer, xb)
    gi = check_routing(xb, bits, d, r, "forced")
    assert len(np.unique(gi, axis=0)) == 1
    o = out.view(torch.int16)
    assert torch.all(o == o[0:1]).item()
    check_output(xb[:1], bits, d, gi[:1], _np(out.float())[:1], np.arange(1), "forced")
    del moe


# ---------------------------------------------------------------------------
# Load-balance statistic (moe_load_balance).
# ---------------------------------------------------------------------------

def _check_load_balance(moe, layer, bits, d, xb, tag):
    x = moe.bits_to_device(xb, "cuda")
    r = moe.load_balance(x, layer)
    r2 = moe.load_balance(x, layer)
    torch.cuda.synchronize()
    R = O.load_balance(xb, bits, d.K)
    counts, mp, lb = _np(r["counts"]), _np(r["mean_prob"]).astype(np.float64), float(_np(r["lb"])[0])
    assert torch.equal(r["lb"], r2["lb"]) and torch.equal(r["mean_prob"], r2["mean_prob"]), f"{tag}: not reproducible"
    if not R["tie"].any():
        assert np.array_equal(counts, R["counts"]), f"{tag}: counts differ"
    else:
        # Flagged ties may move pairs between tied experts; the total is fixed.
        assert counts.sum() == R["counts"].sum()
    # Probabilities from the GPU's fp32 logits, summed in fp32 over the batch.
    np.testing.assert_allclose(mp, R["mean_prob"], rtol=2e-4, atol=1e-7, err_msg=tag)
    assert abs(lb - R["lb"]) <= 2e-4 * R["lb"], (tag, lb, R["lb"])
    _say(f"{tag}: lb {lb:.6f} vs oracle {R['lb']:.6f}, max |dP| {np.abs(mp - R['mean_prob']).max():.2e}")
    return lb


@pytest.mark.parametrize("T", [1, 8, 33, 300, 2049])
def test_toy_load_balance(toy, T):
    d, bits, layer = toy
    moe = _moe()
    _say(f"case toy load balance T={T}")
    _check_load_balance(moe, layer, bits, d, mi.make_x(d, T, 3000 + T), f"toy lb T={T}")


def test_toy_load_balance_zero_input(toy):
    d, bits, layer = toy
    moe = _moe()
    r = moe.load_balance(torch.zeros((50, d.H), dtype=torch.bfloat16, device="cuda"), layer)
    torch.cuda.synchronize()
    assert abs(float(_np(r["lb"])[0]) - 1.0) < 1e-6
    assert np.array_equal(_np(r["counts"]), np.array([50] * d.K + [0] * (d.E - d.K)))


def test_full_load_balance(full):
    d, bits, layer, zb, zlayer = full
    moe = _moe()
    _say("case full load balance decode64 / zipf16384")
    lb64 = _check_load_balance(moe, layer, bits, d, mi.workload_x(mi.WORKLOADS["decode64"]), "decode64 lb")
    lbz = _check_load_balance(moe, zlayer, zb, d, mi.workload_x(mi.WORKLOADS["zipf16384"]), "zipf16384 lb")
    # The skewed workload is far from balanced, the near-uniform one close to it.
    assert lbz > 2.0 * lb64


# ---------------------------------------------------------------------------
# RMSNorm and the sub-block out = h + layer(RMSNorm(h)).
# ---------------------------------------------------------------------------

def _bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (2^(e - 7) for |v| in [2^e, 2^(e+1)))."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _norm_weight(d, seed):
    return mi.f32_to_bf16_bits(np.random.default_rng(seed).normal(1.0, 0.2, d.H).astype(np.float32))


@pytest.mark.parametrize("T,full_shape", [(37, False), (1000, False), (5, True), (300, True)])
def test_rmsnorm_parity(T, full_shape):
    moe = _moe()
    d = mi.FULL if full_shape else mi.TOY
    _say(f"case rmsnorm H={d.H} T={T}")
    hb = mi.make_x(d, T, 7000 + T)
    wb = _norm_weight(d, 7100 + T)
    x = moe.rmsnorm(moe.bits_to_device(hb, "cuda"), moe.bits_to_device(wb, "cuda"), 1e-6)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(_np(x.view(torch.int16)).view(np.uint16))
    ref = O.rmsnorm(hb, wb, 1e-6)
    # Rounded to bf16 from fp32: within one bf16 step of the exact value, and
    # equal to the correctly rounded value almost everywhere.
    assert np.all(np.abs(got - ref) <= _bf16_ulp(ref)), f"T={T}"
    exact = mi.f32_to_bf16_bits(ref.astype(np.float32))
    frac = np.mean(_np(x.view(torch.int16)).view(np.uint16) != exact)
    assert frac < 1e-3, frac
    _say(f"rmsnorm H={d.H} T={T}: elements off by one bf16 step {frac:.2e}")


def _check_block(moe, layer, bits, d, hb, wb, tag):
    h = moe.bits_to_device(hb, "cuda")
    w = moe.bits_to_device(wb, "cuda")
    out = moe.block_forward(h, layer, w, 1e-6)
    x = moe.rmsnorm(h, w, 1e-6)
    r = moe.route(x, layer)
    plain = moe.forward(x, layer)
    torch.cuda.synchronize()
    xb = _np(x.view(torch.int16)).view(np.uint16)
    gi = check_routing(xb, bits, d, r, tag)
    got = _np(out.float()).astype(np.float64)
    H64 = O.bf16_to_f64(hb)
    # Against the oracle with the GPU's activations and routing: beyond the
    # output's own rounding (at the magnitude of h) the layer's tolerance.
    ref = O.block_forward_with_routing(hb, xb, bits, gi)
    excess = np.abs(got - ref) - 0.5 * _bf16_ulp(ref)
    assert excess.max() <= MAX_ABS, (tag, excess.max())
    # Against the same GPU's layer output plus h: the block rounds once, the
    # two-step form first rounds the layer output (half a bf16 step at its
    # magnitude, which can exceed that of the sum when h cancels it) and then
    # the sum, so they agree within one step of the sum plus half a step of
    # the layer output.
    moe_bf16 = _np(plain.float()).astype(np.float64)
    two_step = H64 + moe_bf16
    ratio = np.abs(got - two_step) / (_bf16_ulp(two_step) + 0.5 * _bf16_ulp(moe_bf16))
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (tag, float(ratio.max()), int((ratio > 1).sum()), worst,
                                float(got[worst]), float(two_step[worst]), float(ref[worst]))
    _say(f"{tag}: max excess over rounding {excess.max():.3e}")
    _check_block_chain(moe, layer, bits, d, hb, wb, got, xb, gi, tag)


def _check_block_chain(moe, layer, bits, d, hb, wb, got, xg, gi_g, tag):
    """moe_block_forward against the oracle's own chain end to end: its float64
    RMSNorm rounded to bf16, its own routing of those activations, the layer
    and the residual (O.block_forward).

    The GPU's normalised activations (fp32 arithmetic, then bf16) can differ
    from the oracle's by one bf16 step in a few elements, where the exact value
    lies next to a rounding midpoint; that moves a logit by at most
    sum_h |dx_h| |W_r[e, h]|.  A token whose top-K+1 logits have a gap below
    1e-6 plus twice that shift may then route differently: for those tokens
    (flagged) the output is compared with the oracle evaluated on the GPU's
    activations and expert choice instead.  Every other token is compared with
    the oracle's chain."""
    ref, xo = O.block_forward(hb, wb, 1e-6, bits, d.K)
    Ro = O.route(xo, bits, d.K)
    dx = np.abs(O.bf16_to_f64(xg) - O.bf16_to_f64(xo))
    shift = (dx @ np.abs(O.bf16_to_f64(bits["gate.weight"])).T).max(axis=1)
    srt = np.sort(Ro["logits"], axis=1)[:, ::-1][:, :d.K + 1]
    flag = (np.diff(-srt, axis=1) < (O.TIE_GAP + 2.0 * shift)[:, None]).any(axis=1)
    want = ref.copy()
    if flag.any():
        f = np.nonzero(flag)[0]
        want[f] = O.block_forward_with_routing(hb[f], xg[f], bits, gi_g[f])
    assert np.array_equal(gi_g[~flag], Ro["topk_idx"][~flag]), f"{tag}: routing differs from the oracle chain's"
    excess = np.abs(got - want) - 0.5 * _bf16_ulp(want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    assert excess.max() <= MAX_ABS, (tag, excess.max())
    assert rel <= REL_L2, (tag, rel)
    _say(f"{tag}: against the oracle's own chain: max excess over rounding {excess.max():.3e}, rel-L2 {rel:.3e}, "
         f"activation rows differing {int((dx > 0).any(axis=1).sum())}, flagged {int(flag.sum())}")


@pytest.mark.parametrize("T", [1, 5, 16, 17, 100])
def test_toy_block_forward(toy, T):
    d, bits, layer = toy
    moe = _moe()
    _say(f"case toy block T={T}")
    _check_block(moe, layer, bits, d, mi.make_x(d, T, 7200 + T), _norm_weight(d, 7300 + T), f"toy block T={T}")


def test_full_block_forward(full):
    d, bits, layer, _, _ = full
    moe = _moe()
    for T in (1, 16, 64):
        _say(f"case full block T={T}")
        _check_block(moe, layer, bits, d, mi.make_x(d, T, 7400 + T), _norm_weight(d, 7500 + T), f"full block T={T}")


# ---------------------------------------------------------------------------
# bf16 scores (layer option logits_bf16) and the stable ranks entry point.
#
# The GPU rounds its fp32 scores to bf16; the oracle rounds the exact ones.
# Rounding is monotone, so the GPU's value must lie between the bf16
# roundings of (exact - bound) and (exact + bound), bound being the fp32
# error of the dot product; it equals the oracle's unless the exact score lies
# that close to a rounding midpoint.  Given the GPU's rounded scores, the
# choice of experts is an exact decision on bf16 values: it must match the
# oracle's choice from those same values bit for bit, ties included.
# ---------------------------------------------------------------------------

def _bf16_bracket(exact, bound):
    return O.round_bf16(exact - bound), O.round_bf16(exact + bound)


def check_routing_bf16(xb, bits, dims, r, tag):
    K, E = dims.K, dims.E
    T = xb.shape[0]
    R = O.route(xb, bits, K, logits_bf16=True)
    exact = O.router_logits(xb, bits["gate.weight"])
    gi = _np(r["topk_idx"])
    gl = _np(r["logits"]).astype(np.float64)
    assert np.array_equal(O.round_bf16(gl), gl), f"{tag}: returned logits are not bf16 values"
    S = np.abs(O.bf16_to_f64(xb)) @ np.abs(O.bf16_to_f64(bits["gate.weight"])).T
    lo, hi = _bf16_bracket(exact, LOGIT_CHAIN * 2.0 ** -24 * S)
    assert np.all((gl >= lo) & (gl <= hi)), f"{tag}: a rounded logit outside its bracket"
    off = gl != R["logits"]
    assert np.all(lo[off] != hi[off])
    # The decision on the GPU's own bf16 scores, bit for bit.
    want_idx, _ = O.select_topk(gl, K)
    assert np.array_equal(gi, want_idx), f"{tag}: selection differs from the oracle's on the same scores"
    same = ~off.any(axis=1)
    assert np.array_equal(gi[same], R["topk_idx"][same]), tag
    gw = _np(r["topk_w"]).astype(np.float64)
    np.testing.assert_allclose(gw, O.renormalised_weights(gl, gi), rtol=0, atol=W_TOL)
    # Against the oracle's own weights (its rounded scores at the chosen
    # experts): 1e-6 where those scores equal the GPU's, else 1e-6 plus twice
    # the largest difference of a chosen score.
    ow = O.renormalised_weights(R["logits"], gi)
    ds = np.take_along_axis(np.abs(gl - R["logits"]), gi.astype(np.int64), axis=1).max(axis=1)
    dw = np.abs(gw - ow)
    assert np.all(dw <= (W_TOL + 2.0 * ds)[:, None]), f"{tag}: weight error {dw.max():.3e} vs oracle"
    assert np.all(dw[ds == 0] <= W_TOL), f"{tag}: weights differ from the oracle's on equal scores"
    # Shared gate: the sigmoid of a bf16 value inside the gate score's bracket.
    zg = (O.bf16_to_f64(xb) @ O.bf16_to_f64(bits["shared_expert_gate.weight"]).T)[:, 0]
    Sg = np.abs(O.bf16_to_f64(xb)) @ np.abs(O.bf16_to_f64(bits["shared_expert_gate.weight"]))[0]
    glo, ghi = _bf16_bracket(zg, LOGIT_CHAIN * 2.0 ** -24 * Sg)
    gs = _np(r["shared_gate"])[:T].astype(np.float64)
    assert np.all((gs >= O.sigmoid(glo) - W_TOL) & (gs <= O.sigmoid(ghi) + W_TOL)), tag
    np.testing.assert_allclose(gs[glo == ghi], R["shared_gate"][glo == ghi], rtol=0, atol=W_TOL)
    d = O.counting_sort(gi, E)
    assert np.array_equal(_np(r["offsets"]), d["offsets"]), tag
    assert np.array_equal(_np(r["perm"])[:T * K], d["perm"]), tag
    # How often rounding made scores equal inside ranks 0..K.
    srt = np.sort(gl, axis=1)[:, ::-1][:, :K + 1]
    tied = (np.diff(srt, axis=1) == 0).any(axis=1)
    _say(f"{tag}: bf16 routing ok, T={T}, tokens with equal scores in ranks 0..K {int(tied.sum())}, "
         f"scores rounded the other way {int(off.sum())}, tokens whose choice changed with them "
         f"{int((gi != R['topk_idx']).any(axis=1).sum())}")
    return gi


def check_output_bf16(xb, bits, gi, out_rows, rows, tag):
    ref = O.forward_with_routing(xb[rows], bits, gi[rows], None, True)
    got = out_rows.astype(np.float64)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    _say(f"{tag}: rows {len(rows)} max-abs {err.max():.3e} rel-L2 {rel:.3e}")
    assert err.max() <= MAX_ABS, tag
    assert rel <= REL_L2, tag


@pytest.mark.parametrize("T", [1, 5, 16, 17, 64, 300])
def test_toy_bf16_logits(toy, T):
    d, bits, layer = toy
    lb = layer.with_logits_bf16()
    _say(f"case toy bf16 logits T={T}")
    xb = mi.make_x(d, T, 9100 + T)
    r, out = run_layer(lb, xb, want_logits=True)
    gi = check_routing_bf16(xb, bits, d, r, f"toy bf16 T={T}")
    check_output_bf16(xb, bits, gi, _np(out.float()), np.arange(T), f"toy bf16 T={T}")
    # The fp32 mode on the same layer descriptor's tensors is unaffected.
    r32, _ = run_layer(layer, xb, want_logits=True)
    check_routing(xb, bits, d, r32, f"toy fp32 after bf16 T={T}")


def test_toy_bf16_zero_input(toy):
    d, bits, layer = toy
    for T in (3, 40):
        r, out = run_layer(layer.with_logits_bf16(), np.zeros((T, d.H), np.uint16), want_logits=True)
        assert np.all(_np(r["topk_idx"]) == np.arange(d.K))
        np.testing.assert_allclose(_np(r["topk_w"]), 1.0 / d.K, rtol=0, atol=W_TOL)
        assert np.all(_np(out.float()) == 0.0)


@pytest.mark.parametrize("T", [1, 16, 64, 4096])
def test_full_bf16_logits(full, T):
    d, bits, layer, _, _ = full
    _say(f"case full bf16 logits T={T}")
    xb = mi.workload_x(mi.WORKLOADS["prefill4096"]) if T == 4096 else mi.make_x(d, T, 9200 + T)
    r, out = run_layer(layer.with_logits_bf16(), xb, want_logits=True)
    gi = check_routing_bf16(xb, bits, d, r, f"full bf16 T={T}")
    check_output_bf16(xb, bits, gi, _np(out.float()), np.arange(T), f"full bf16 T={T}")


@pytest.mark.parametrize("T", [64, 2048])
def test_full_bf16_logits_skewed(full, T):
    # Scores of size ~50 have a bf16 spacing of 0.25: ties are frequent.  64
    # tokens take the fused route, 2048 the separate router kernels.
    d, _, _, zb, zlayer = full
    wl = mi.WORKLOADS["zipf16384"]
    xb = mi.workload_x(wl)[:T]
    _say(f"case full bf16 logits, skewed router, T={T}")
    r, out = run_layer(zlayer.with_logits_bf16(), xb, want_logits=True)
    gi = check_routing_bf16(xb, zb, d, r, f"skewed bf16 T={T}")
    check_output_bf16(xb, zb, gi, _np(out.float()), np.arange(T), f"skewed bf16 T={T}")


@pytest.mark.parametrize("E,R", [(1, 3), (7, 5), (16, 1000), (64, 9), (255, 33), (256, 4096)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ranks_parity(E, R, dtype):
    moe = _moe()
    rng = np.random.default_rng(E * 7 + R)
    # Few distinct values: many exact ties; plus signed zeros and infinities.
    v = (rng.integers(-6, 7, (R, E)) * 0.375).astype(np.float32)
    v[rng.random((R, E)) < 0.05] = -0.0
    v[rng.random((R, E)) < 0.02] = np.inf
    v[rng.random((R, E)) < 0.02] = -np.inf
    t = torch.from_numpy(v).to("cuda")
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    got = _np(moe.ranks(t))
    np.testing.assert_array_equal(got, O.ranks(v.astype(np.float64)))
    assert np.all(np.sort(got, axis=1) == np.arange(E))


def test_ranks_agree_with_route(full):
    moe = _moe()
    d, bits, layer, _, _ = full
    xb = mi.make_x(d, 300, 9300)
    for ly in (layer, layer.with_logits_bf16()):
        r = moe.route(moe.bits_to_device(xb, "cuda"), ly, want_logits=True)
        rk = _np(moe.ranks(r["logits"]))
        gi = _np(r["topk_idx"])
        np.testing.assert_array_equal(np.take_along_axis(rk, gi.astype(np.int64), axis=1),
                                      np.broadcast_to(np.arange(d.K), gi.shape))
        np.testing.assert_array_equal(rk, O.ranks(_np(r["logits"]).astype(np.float64)))


# ---------------------------------------------------------------------------
# Routed experts streamed from pinned host memory (moe_forward_streamed).
# The GEMMs are the same kernels reading the same values from cache slots, so
# against moe_forward's grouped path (T > 16) the output is bit for bit the
# same, whatever the number of rounds; at every T it is checked against the
# oracle too.
# ---------------------------------------------------------------------------

def _host_layer(layer):
    moe = _moe()
    p = dict(layer.params)
    p["gate_up_proj"] = p["gate_up_proj"].cpu().pin_memory()
    p["down_proj"] = p["down_proj"].cpu().pin_memory()
    return moe.MoeLayer(layer.H, layer.E, layer.K, layer.I, layer.Is, p, layer.logits_bf16, layer.experts_tiled)


@pytest.fixture(scope="module")
def toy_host(toy):
    d, bits, layer = toy
    return _host_layer(layer)


@pytest.mark.parametrize("T", [1, 5, 17, 64, 300])
@pytest.mark.parametrize("cap", [16, 3, 1])
def test_toy_streamed(toy, toy_host, T, cap):
    moe = _moe()
    d, bits, layer = toy
    _say(f"case toy streamed T={T} slots={cap}")
    xb = mi.make_x(d, T, 9400 + T)
    x = moe.bits_to_device(xb, "cuda")
    cache = moe.expert_cache(toy_host, cap)
    got = moe.forward_streamed(x, toy_host, cache)
    ref = moe.forward(x, layer)
    r = moe.route(x, layer, want_logits=True)
    torch.cuda.synchronize()
    gi = check_routing(xb, bits, d, r, f"toy streamed T={T}")
    check_output(xb, bits, d, gi, _np(got.float()), np.arange(T), f"toy streamed T={T} slots={cap}")
    # The streamed path routes with the separate router kernels, the resident
    # path of 17..64 tokens with the fused route: equal bits also check that
    # both compute the same routing.
    if T > 16:
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "streamed != resident"


def test_toy_streamed_cache_reuse(toy, toy_host):
    # A cache that served other batches (and more rounds) gives the same bits.
    moe = _moe()
    d, bits, layer = toy
    xa = moe.bits_to_device(mi.make_x(d, 300, 9500), "cuda")
    xb = moe.bits_to_device(mi.make_x(d, 40, 9501), "cuda")
    fresh = moe.forward_streamed(xb, toy_host, moe.expert_cache(toy_host, 2))
    cache = moe.expert_cache(toy_host, 2)
    for _ in range(2):
        moe.forward_streamed(xa, toy_host, cache)
        again = moe.forward_streamed(xb, toy_host, cache)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), fresh.view(torch.int16))
    assert torch.equal(again.view(torch.int16), moe.forward(xb, layer).view(torch.int16))


def test_streamed_rejects_wrong_memory(toy, toy_host):
    moe = _moe()
    d, bits, layer = toy
    x = moe.bits_to_device(mi.make_x(d, 20, 9600), "cuda")
    cache = moe.expert_cache(toy_host, 4)
    # Experts in device memory, in pageable host memory, or in a pinned
    # allocation holding half of them (torch's pinned allocator rounds sizes
    # up to a power of two, so a buffer only slightly short would be padded
    # to the full size): refused before anything is launched.
    p = dict(toy_host.params)
    bad = {"device": dict(p, gate_up_proj=layer.params["gate_up_proj"]),
           "pageable": dict(p, down_proj=p["down_proj"].clone()),
           "short": dict(p, down_proj=torch.empty((d.E // 2) * d.H * d.I, dtype=torch.bfloat16).pin_memory())}
    for name, params in bad.items():
        try:
            moe.forward_streamed(x, moe.MoeLayer(d.H, d.E, d.K, d.I, d.Is, params), cache)
        except moe.MoeError as e:
            assert e.code == moe._lib.MOE_ERR_MEMORY, (name, str(e))
            _say(f"{name}: {e}")
        else:
            pytest.fail(f"{name}: not refused")


@pytest.mark.parametrize("T,cap", [(1, 8), (16, 256), (64, 40), (4096, 256)])
def test_full_streamed(full, T, cap):
    moe = _moe()
    d, bits, layer, _, _ = full
    host = _host_layer(layer)
    _say(f"case full streamed T={T} slots={cap}")
    xb = mi.workload_x(mi.WORKLOADS["prefill4096"]) if T == 4096 else mi.make_x(d, T, 9700 + T)
    x = moe.bits_to_device(xb, "cuda")
    got = moe.forward_streamed(x, host, moe.expert_cache(host, cap))
    ref = moe.forward(x, layer)
    r = moe.route(x, layer, want_logits=True)
    torch.cuda.synchronize()
    gi = check_routing(xb, bits, d, r, f"full streamed T={T}")
    # At 4096 tokens the streamed output must equal the resident path's bit for
    # bit (below), and test_full_workloads checks that output whole against the
    # oracle; here a sample of rows is enough.
    rows = np.arange(T) if T <= 64 else _sample_rows(T, gi)
    check_output(xb, bits, d, gi, _np(got.float())[rows], rows, f"full streamed T={T} slots={cap}")
    if T > 16:
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "streamed != resident"


# ---------------------------------------------------------------------------
# Routed experts in the MFMA-tile layout (moe_tile_experts): same values in
# other places, so the grouped path's output is the same bit for bit.
# ---------------------------------------------------------------------------

def _tile_by_definition(a):
    """The documented tile layout, written with numpy from its definition:
    [E, R, Kd] -> [E, R/16, Kd/64, 2, 64, 8], lane l = 16 q + r16 holding
    row 16 b + r16 and k-step elements 16 q + 8 h .. + 7."""
    E, R, Kd = a.shape
    v = a.reshape(E, R // 16, 16, Kd // 64, 4, 2, 8)          # e, b, r16, ks, q, h, j
    return np.ascontiguousarray(v.transpose(0, 1, 3, 5, 4, 2, 6)).reshape(-1)


def test_tiled_layout_bytes(toy):
    moe = _moe()
    d, bits, layer = toy
    t = layer.tiled()
    torch.cuda.synchronize()
    for name in ("gate_up_proj", "down_proj"):
        got = _np(t.params[name].view(torch.int16)).view(np.uint16).reshape(-1)
        assert np.array_equal(got, _tile_by_definition(bits[name])), name


@pytest.mark.parametrize("T", [1, 5, 16, 17, 300])
def test_toy_tiled_matches_row_major(toy, T):
    moe = _moe()
    d, bits, layer = toy
    t = layer.tiled()
    xb = mi.make_x(d, T, 9800 + T)
    x = moe.bits_to_device(xb, "cuda")
    got = moe.forward(x, t)
    r = moe.route(x, layer)
    torch.cuda.synchronize()
    gi = _np(r["topk_idx"])
    check_output(xb, bits, d, gi, _np(got.float()), np.arange(T), f"toy tiled T={T}")
    # Both paths (fused decode for T <= 16, grouped above) give the same bits
    # with either layout.
    assert torch.equal(got.view(torch.int16), moe.forward(x, layer).view(torch.int16))
    # The streamed path runs the grouped kernels at every T: the same bits as
    # forward wherever forward takes the grouped path too.
    host = _host_layer(t)
    st = moe.forward_streamed(x, host, moe.expert_cache(host, 3))
    torch.cuda.synchronize()
    check_output(xb, bits, d, gi, _np(st.float()), np.arange(T), f"toy tiled streamed T={T}")
    if T > 16:
        assert torch.equal(st.view(torch.int16), got.view(torch.int16))


def test_full_gemm_tile_regimes(full):
    # Both sides of each switch of the grouped GEMMs at full shape: 32-row
    # tiles up to 8 slots per expert on average (256 tokens), 160-row tiles
    # with streamed weight loads up to 16 (512 tokens), then plain loads.
    # 256 tokens (2048 pairs) is also the last batch dispatched by one
    # workgroup per group, 257 the first by a single workgroup.
    # Every row against the oracle, and the tiled expert layout bitwise equal
    # to the row-major one.
    moe = _moe()
    d, bits, layer, _, _ = full
    t = layer.tiled()
    for T in (256, 257, 512, 513):
        _say(f"case full GEMM tile regime T={T}")
        xb = mi.make_x(d, T, 9700 + T)
        r, out = run_layer(layer, xb, want_logits=True)
        gi = check_routing(xb, bits, d, r, f"tile regime T={T}")
        check_output(xb, bits, d, gi, _np(out.float()), np.arange(T), f"tile regime T={T}")
        got = moe.forward(moe.bits_to_device(xb, "cuda"), t)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), out.view(torch.int16)), f"T={T}"


def test_full_workspace_sized_for_largest_batch(full):
    # One workspace sized for 600 tokens serves batches of every path below
    # it (fused decode, 32-row and 160-row GEMM tiles) with the same bits as
    # a workspace of each batch's own size.
    moe = _moe()
    d, bits, layer, _, _ = full
    big = layer.workspace(600)
    for T in (1, 16, 17, 256, 257, 600):
        _say(f"case full shared workspace T={T}")
        x = moe.bits_to_device(mi.make_x(d, T, 9600 + T), "cuda")
        a = moe.forward(x, layer, ws=big)
        torch.cuda.synchronize()
        if T <= 64:
            assert call_status(big) == 0, "fused path wait timed out"
        b = moe.forward(x, layer)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"T={T}"


def test_full_tiled_matches_row_major(full):
    moe = _moe()
    d, bits, layer, _, _ = full
    t = layer.tiled()
    for T in (1, 7, 16, 64, 4096):
        xb = mi.workload_x(mi.WORKLOADS["prefill4096"]) if T == 4096 else mi.make_x(d, T, 9900 + T)
        x = moe.bits_to_device(xb, "cuda")
        a = moe.forward(x, t)
        b = moe.forward(x, layer)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"T={T}"
        _say(f"full tiled T={T}: identical to row-major")

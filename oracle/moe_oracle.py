"""CPU oracle for the sparse MoE FFN layer (256 experts, top-8, gated shared expert).

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow reference that the
HIP path is checked against.  Only the test suite, the package's smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
calls it and shares no code with it.

What it computes is the definition written out, in float64 throughout:

* "Qwen3.6-35B-A3B — Architecture Overview" (Hugging Face blog),
  section "MoE FFN: 256 Experts":
  - Router: a learned Linear 2048 -> 256 scores every expert for each token;
    softmax over all scores; the 8 best are kept and their weights rescaled so
    that they sum to one.
  - Experts: expert_e(x) = SiLU(x W_gate_e) * (x W_up_e) W_down_e, gate and up
    stored merged as one [256, 1024, 2048] tensor, inner size 512.
  - Shared expert: the same SwiGLU, always active, scaled by
    sigmoid(Linear(x, 1)).
* "Qwen3.6 35B-A3B" model page for Linnet (nest.franknoh.dev), section
  Blocks: ``Linear`` stores ``weight [Out, In]`` (so y = x W^T), ``SparseMoe``
  lists ``gate``, ``gate_up_proj [E, 2I, H]``, ``down_proj [E, H, I]``,
  ``shared_expert: SwiGlu``, ``shared_expert_gate: Linear<H, 1>``, and a
  private ``ranks`` that gives every expert an integer rank per row.

Readings where the pages leave a step open (each also listed with the design
notes of this repository):

* rows [0, I) of gate_up_proj[e] are the gate projection, rows [I, 2I) the up
  projection (merged in name order);
* no biases (none appear in the formulas);
* router logits are kept in float64, not rounded to bf16; the second routing
  mode (``logits_bf16=True``) follows the model page's types instead: the
  outputs of both gate projections (``gate: Linear<H, Experts, T>`` and
  ``shared_expert_gate: Linear<H, 1, T>``, T = bf16) are the exact dot
  products rounded to the nearest bf16 (ties to even), and ranking, softmax
  and the sigmoid gate all act on those rounded values; equal rounded logits
  are ordered by expert index like any other tie;
* rank: higher logit first, equal logits ordered by lower expert index;
  ``topk_idx[t, k]`` lists the selected experts in rank order;
* SiLU(z) = z * sigmoid(z), sigmoid(z) = 1 / (1 + exp(-z));
* the shared-expert gate scales only the shared expert's output;
* no capacity limit: every (token, expert) pair is computed;
* the layer output excludes the residual and any norm;
* the load-balance statistic is E * sum_e f_e * P_e (slot fraction times
  mean full-softmax probability), the page giving no formula;
* the MoE sub-block is out = h + MoE(bf16(RMSNorm(h))), RMSNorm the textbook
  h / sqrt(mean(h^2) + eps) * w.

Inputs are bf16 bit patterns (uint16 arrays); parameters are passed as a
mapping of bf16 bit patterns, or of their float64 values decoded once with
``decode_params``, keyed by the model page's member names: ``gate.weight``,
``gate_up_proj``, ``down_proj``, ``shared_expert.gate.weight``,
``shared_expert.up.weight``, ``shared_expert.down.weight``,
``shared_expert_gate.weight``.

Parity status: every function here is pinned by tests/test_oracle.py (closed
forms, special cases, brute force, a hand-worked example).  The absolute
output values at full size have no printed counterpart on the pages; they
rest on the definition plus those pins.
"""
from __future__ import annotations

import numpy as np

TIE_GAP = 1e-6


# ---------------------------------------------------------------------------
# bf16 decoding: a bf16 value is the top half of an IEEE float32.
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns: shift into the high half of a float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def param_values(a: np.ndarray) -> np.ndarray:
    """Values of a parameter: bf16 bit patterns (uint16) are decoded exactly;
    an array of float64 values (``decode_params``) is taken as it is."""
    a = np.asarray(a)
    return a if a.dtype == np.float64 else bf16_to_f64(a)


def decode_params(params: dict) -> dict:
    """Every parameter decoded once to float64 (the same values the functions
    below decode on each use), so that repeated calls skip the decoding."""
    return {name: bf16_to_f64(v) for name, v in params.items()}


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each float64, ties to the even significand.

    bfloat16 keeps 8 significant bits: in the binade [2^e, 2^(e+1)) its values
    are spaced 2^(e-7) apart, and below 2^-126 (subnormals) 2^-133 apart.  The
    value is divided by that spacing, rounded to an integer half-to-even
    (``np.round``) and scaled back; both steps are exact in float64.
    Magnitudes that round past the largest finite bf16 become infinite; zeros
    keep their sign.  Finite inputs assumed.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = 2.0 ** (np.maximum(e, -126.0) - 7.0)
    r = np.round(v / step) * step
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    return np.where(a == 0, v, r)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are bf16 numbers already (for example
    the output of ``round_bf16``): the value is exact in float32, whose top
    half is its bf16 pattern.  Raises if a value is not a bf16 number."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)) or np.any(f.astype(np.float64) != np.asarray(v, dtype=np.float64)):
        raise ValueError("not a bf16 value")
    return (u >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Elementwise activations (textbook definitions; the pages name them only).
# ---------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


# ---------------------------------------------------------------------------
# Router (section "MoE FFN: 256 Experts", Router; model page ``gate: Linear``).
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[e, h], float64 ([T, H] x [E, H] -> [T, E])."""
    return bf16_to_f64(x) @ param_values(router_w).T


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Softmax over the expert axis, max subtracted first."""
    l = np.asarray(logits, dtype=np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def ranks(logits: np.ndarray) -> np.ndarray:
    """Integer rank of every expert per row (model page: ``SparseMoe.ranks``).

    rank[t, e] = #{j : l[t, j] > l[t, e]} + #{j < e : l[t, j] == l[t, e]},
    i.e. the position of e when experts are sorted by descending logit with
    ties broken by lower index.  Uses a stable sort of the negated logits.
    """
    l = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-l, axis=1, kind="stable")
    r = np.empty_like(order)
    rows = np.arange(l.shape[0])[:, None]
    r[rows, order] = np.arange(l.shape[1])[None, :]
    return r.astype(np.int32)


def select_topk(logits: np.ndarray, K: int):
    """Top-K experts in rank order and their renormalised softmax weights.

    Returns ``topk_idx [T, K] int32`` and ``topk_w [T, K] float64`` where
    topk_w[t, k] = p[t, e_k] / sum_j p[t, e_j] with p the softmax over all E.
    """
    l = np.asarray(logits, dtype=np.float64)
    r = ranks(l)
    T, E = l.shape
    topk_idx = np.empty((T, K), dtype=np.int32)
    for k in range(K):
        topk_idx[:, k] = np.argmax(r == k, axis=1)
    p = softmax_rows(l)
    sel = np.take_along_axis(p, topk_idx.astype(np.int64), axis=1)
    topk_w = sel / sel.sum(axis=1, keepdims=True)
    return topk_idx, topk_w


def renormalised_weights(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """Renormalised softmax weights for a given choice of experts (any order)."""
    p = softmax_rows(logits)
    sel = np.take_along_axis(p, np.asarray(topk_idx, dtype=np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def tie_flags(logits: np.ndarray, K: int, gap: float = TIE_GAP) -> np.ndarray:
    """True for tokens whose ranks 0..K contain two neighbours closer than ``gap``.

    Sorted descending, the gaps between rank r and r+1 for r = 0..K-1 are
    checked: a gap below ``gap`` inside the top K can reorder ``topk_idx``, one
    at the K/K+1 boundary can change which experts are selected.
    """
    l = np.sort(np.asarray(logits, dtype=np.float64), axis=1)[:, ::-1]
    m = min(K + 1, l.shape[1])
    gaps = l[:, : m - 1] - l[:, 1:m]
    return (gaps < gap).any(axis=1)


def route_logits(x: np.ndarray, params: dict, logits_bf16: bool = False) -> np.ndarray:
    """The router's scores in the chosen mode: float64, or rounded to bf16."""
    logits = router_logits(x, params["gate.weight"])
    return round_bf16(logits) if logits_bf16 else logits


def route(x: np.ndarray, params: dict, K: int, logits_bf16: bool = False) -> dict:
    """Router + softmax + top-K + renormalise + shared-expert gate scalar.

    With ``logits_bf16`` the scores are rounded to bf16 first; equal scores are
    then common and are ordered by expert index, so no token is flagged as a
    tie ("tie" is all False): the choice is fully determined by the rounded
    scores.
    """
    logits = route_logits(x, params, logits_bf16)
    topk_idx, topk_w = select_topk(logits, K)
    s = shared_gate(x, params, logits_bf16)
    tie = np.zeros(logits.shape[0], dtype=bool) if logits_bf16 else tie_flags(logits, K)
    return {"logits": logits, "topk_idx": topk_idx, "topk_w": topk_w,
            "shared_gate": s, "tie": tie}


def shared_gate(x: np.ndarray, params: dict, logits_bf16: bool = False) -> np.ndarray:
    """s[t] = sigmoid(x[t] . w_sg) for the [1, H] shared_expert_gate Linear
    (its output rounded to bf16 first with ``logits_bf16``)."""
    z = (bf16_to_f64(x) @ param_values(params["shared_expert_gate.weight"]).T)[:, 0]
    return sigmoid(round_bf16(z) if logits_bf16 else z)


# ---------------------------------------------------------------------------
# Dispatch: group the (token, slot) pairs by expert.
# ---------------------------------------------------------------------------

def counting_sort(topk_idx: np.ndarray, E: int) -> dict:
    """Stable grouping of pair ids q = t*K + k by expert key topk_idx[t, k].

    counts[e]   number of pairs routed to e
    offsets     exclusive prefix sum of counts, length E+1, offsets[E] = T*K
    perm[s]     pair id at slot s; slots of expert e are offsets[e]..offsets[e+1]-1,
                in increasing pair id (so increasing token)
    slot_of[q]  inverse of perm
    """
    key = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(key, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(key, kind="stable")
    slot_of = np.empty_like(perm)
    slot_of[perm] = np.arange(perm.size)
    return {"counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
            "perm": perm.astype(np.int32), "slot_of": slot_of.astype(np.int32)}


# ---------------------------------------------------------------------------
# Experts (section "MoE FFN: 256 Experts", Experts and Shared Expert).
# ---------------------------------------------------------------------------

def swiglu(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """(SiLU(X Wg^T) * (X Wu^T)) Wd^T with weights stored [Out, In], float64 in/out."""
    return (silu(X @ w_gate.T) * (X @ w_up.T)) @ w_down.T


def routed_expert(X: np.ndarray, params: dict, e: int, I: int) -> np.ndarray:
    """expert_e applied to float64 rows X: gate = gate_up_proj[e, :I], up = gate_up_proj[e, I:]."""
    gu = param_values(params["gate_up_proj"][e])
    wd = param_values(params["down_proj"][e])
    return swiglu(X, gu[:I], gu[I:], wd)


def shared_expert(X: np.ndarray, params: dict) -> np.ndarray:
    return swiglu(X, param_values(params["shared_expert.gate.weight"]),
                  param_values(params["shared_expert.up.weight"]),
                  param_values(params["shared_expert.down.weight"]))


def _dims(params: dict):
    E, two_i, H = params["gate_up_proj"].shape
    return H, E, two_i // 2


def forward_with_routing(x: np.ndarray, params: dict, topk_idx: np.ndarray,
                         topk_w: np.ndarray | None = None,
                         logits_bf16: bool = False) -> np.ndarray:
    """Layer output [T, H] float64 for a given expert choice.

    Weights default to the renormalised softmax of the oracle's own logits
    (in the routing mode ``logits_bf16`` selects) restricted to ``topk_idx``;
    the shared-expert gate follows the same mode.  Dispatch goes through ``counting_sort``:
    each expert is evaluated once on the rows routed to it, and each row's
    result is added to its token, scaled by the routing weight.
    """
    H, E, I = _dims(params)
    X = bf16_to_f64(x)
    T, K = np.asarray(topk_idx).shape
    if topk_w is None:
        topk_w = renormalised_weights(route_logits(x, params, logits_bf16), topk_idx)
    w_flat = np.asarray(topk_w, dtype=np.float64).reshape(-1)
    d = counting_sort(topk_idx, E)
    acc = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        lo, hi = int(d["offsets"][e]), int(d["offsets"][e + 1])
        if lo == hi:
            continue
        q = d["perm"][lo:hi].astype(np.int64)
        tok = q // K
        Y = routed_expert(X[tok], params, e, I)
        acc[tok] += w_flat[q, None] * Y          # tokens within one segment are distinct
    s = shared_gate(x, params, logits_bf16)
    return acc + s[:, None] * shared_expert(X, params)


def forward(x: np.ndarray, params: dict, K: int, logits_bf16: bool = False) -> np.ndarray:
    """The layer: route, dispatch to the top-K experts, combine, add the gated shared expert."""
    logits = route_logits(x, params, logits_bf16)
    topk_idx, topk_w = select_topk(logits, K)
    return forward_with_routing(x, params, topk_idx, topk_w, logits_bf16)


def forward_dense(x: np.ndarray, params: dict, K: int, logits_bf16: bool = False) -> np.ndarray:
    """Brute force for tiny inputs: run all E experts on every token, mask to the top-K.

    out[t] = sum_e mask[t, e] * w[t, e] * expert_e(x_t) + s_t * shared(x_t),
    with w = renormalised softmax over the experts whose rank is below K.
    """
    H, E, I = _dims(params)
    X = bf16_to_f64(x)
    logits = route_logits(x, params, logits_bf16)
    r = ranks(logits)
    p = softmax_rows(logits)
    mask = (r < K).astype(np.float64)
    w = p * mask
    w = w / w.sum(axis=1, keepdims=True)
    out = np.zeros((X.shape[0], H), dtype=np.float64)
    for e in range(E):
        out += w[:, e:e + 1] * routed_expert(X, params, e, I)
    return out + shared_gate(x, params, logits_bf16)[:, None] * shared_expert(X, params)


# ---------------------------------------------------------------------------
# Load-balance statistic (section "MoE FFN: 256 Experts", Load Balancing).
# ---------------------------------------------------------------------------

def load_balance(x: np.ndarray, params: dict, K: int, logits_bf16: bool = False) -> dict:
    """Forward-only load-balance statistic of one batch.

    The page names an auxiliary loss (coefficient 0.001) that penalises uneven
    use of the experts, without a formula.  Reading taken here: the fraction
    of the T*K routing slots that go to expert e, f_e = counts[e] / (T K),
    times the batch mean of its full-softmax router probability,
    P_e = (1/T) sum_t p[t, e], summed over the experts and scaled by E:

        lb = E * sum_e f_e * P_e

    which is 1 when both are uniform and grows as routing concentrates (the
    training loss would be 0.001 * lb; no gradient is formed here).
    """
    logits = route_logits(x, params, logits_bf16)
    topk_idx, _ = select_topk(logits, K)
    T, E = logits.shape
    counts = np.bincount(topk_idx.reshape(-1).astype(np.int64), minlength=E)
    f = counts / float(T * K)
    P = softmax_rows(logits).mean(axis=0)
    return {"counts": counts.astype(np.int32), "fraction": f, "mean_prob": P,
            "lb": float(E * np.sum(f * P)), "logits": logits, "topk_idx": topk_idx,
            "tie": np.zeros(T, dtype=bool) if logits_bf16 else tie_flags(logits, K)}


# ---------------------------------------------------------------------------
# The MoE sub-block around the layer ("Qwen3.6-35B-A3B — Architecture
# Overview", Stage 2: Transform Blocks: RMSNorm -> MoE FFN -> +residual; model
# page, AttentionLayer / DeltaLayer: post_attention_layernorm: RmsNorm<H, T>
# with param weight [H]).
# ---------------------------------------------------------------------------

def rmsnorm(h: np.ndarray, norm_w: np.ndarray, eps: float) -> np.ndarray:
    """y[t] = h[t] / sqrt(mean_j h[t, j]^2 + eps) * w, float64 (bf16 bit inputs).

    The pages give the module and its weight but no formula: the textbook
    RMSNorm is taken, the weight multiplying directly and eps from the caller.
    """
    H = bf16_to_f64(h)
    w = bf16_to_f64(norm_w).reshape(-1)
    return H / np.sqrt(np.mean(H * H, axis=1, keepdims=True) + eps) * w[None, :]


def block_forward(h: np.ndarray, norm_w: np.ndarray, eps: float, params: dict, K: int,
                  logits_bf16: bool = False):
    """The MoE sub-block end to end: x = bf16(RMSNorm(h)), routed by the
    oracle's own router, out = h + MoE(x).  Returns (out [T, H] float64,
    x as bf16 bits [T, H])."""
    x_bits = bf16_bits(round_bf16(rmsnorm(h, norm_w, eps)))
    return bf16_to_f64(h) + forward(x_bits, params, K, logits_bf16), x_bits


def block_forward_with_routing(h: np.ndarray, x_bits: np.ndarray, params: dict,
                               topk_idx: np.ndarray, logits_bf16: bool = False) -> np.ndarray:
    """h + MoE(x) for given bf16 activations x (the normalised h rounded to
    bf16, the type the model page gives every activation) and routing."""
    return bf16_to_f64(h) + forward_with_routing(x_bits, params, topk_idx, None, logits_bf16)


def expert_param_count(H: int, I: int) -> int:
    """Parameters of one SwiGLU expert: gate [I, H] + up [I, H] + down [H, I]."""
    return 3 * H * I


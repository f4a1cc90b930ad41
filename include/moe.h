/*
 * moe.h — C ABI of the sparse mixture-of-experts FFN layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (Qwen3.6-35B-A3B MoE FFN), as defined by "Qwen3.6-35B-A3B —
 * Architecture Overview" (Hugging Face blog), section "MoE FFN: 256 Experts",
 * with the tensor shapes of the Linnet model page "Qwen3.6 35B-A3B",
 * Blocks: SparseMoe, SwiGlu, Linear:
 *
 *   logits[t, e] = x[t] . router_w[e]                              (router)
 *                  (rounded to bf16 when the layer asks for bf16 scores)
 *   top-K experts per token by logit (ties: lower expert index first),
 *   w[t, k]      = softmax(logits[t])[e_k] / sum_j softmax(logits[t])[e_j]
 *   expert_e(v)  = (SiLU(v Wg_e^T) * (v Wu_e^T)) Wd_e^T,
 *                  Wg_e = gate_up_w[e, 0:I, :], Wu_e = gate_up_w[e, I:2I, :],
 *                  Wd_e = down_w[e]
 *   out[t]       = sum_k w[t, k] expert_{e_k}(x[t])
 *                + sigmoid(x[t] . shared_expert_gate_w) * shared(x[t])
 *
 * with shared(v) the same SwiGLU over shared_gate_w / shared_up_w /
 * shared_down_w (inner size Is).  No biases, no residual, no norm: out is the
 * MoE block's output alone.  Every (token, expert) pair is computed (no
 * capacity limit).
 *
 * Conventions for every entry point:
 *  - Tensors are dense row-major bf16 (uint16 bit patterns of bfloat16) unless
 *    stated; a Linear weight is stored [Out, In].  Device pointers are owned
 *    by the caller; the library keeps none of them after a call returns and
 *    allocates no device memory.
 *  - Every device pointer must be 16-byte aligned.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  The caller must keep x, out, the weights and the workspace
 *    alive and unmodified until the stream work has completed.  Calls that
 *    share a workspace must be ordered on one stream.
 *  - Results are bitwise reproducible from run to run on the same device.
 *  - Return value: MOE_OK or one of the MOE_ERR_* codes below.  All argument
 *    checks run before any HIP call; then nothing has been enqueued.
 *    moe_last_error() gives a per-thread text for the last failure.
 *  - Inputs are assumed finite; NaN/Inf in x or the weights give unspecified
 *    routing.
 *  - Workspace: device memory of moe_workspace_bytes(L, T) bytes, 16-byte
 *    aligned, owned by the caller.  A new workspace must be zero-filled once
 *    before its first call (hipMemset, or allocate it zeroed); the library
 *    keeps it valid after that, whatever the calls' sizes and paths.  Its
 *    first moe_workspace_control_bytes() bytes are a control block that
 *    records each call (see moe_workspace_status).
 *
 * Supported dimensions: H % 256 == 0, I % 64 == 0, Is % 64 == 0,
 * 1 <= K <= 8, K <= E <= 256, 0 <= T <= 2^22.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL                          */
  MOE_ERR_SHAPE = 2,     /* T < 0, K/E/H/I/Is outside the supported set         */
  MOE_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned             */
  MOE_ERR_WORKSPACE = 4, /* ws_bytes < moe_workspace_bytes(L, T)                */
  MOE_ERR_DEVICE = 5,    /* the current HIP device is not a gfx950              */
  MOE_ERR_LAUNCH = 6,    /* a HIP call failed; moe_last_error() has its text    */
  MOE_ERR_MEMORY = 7,    /* memory of the wrong kind or too small an allocation */
  MOE_ERR_TIMEOUT = 8    /* moe_workspace_status: a wait inside the latest call's
                            fused kernel timed out, so that call's outputs are
                            invalid                                             */
};

/* One MoE layer: dimensions and device pointers to its seven parameters
 * (Linnet page, Blocks: SparseMoe members gate, gate_up_proj, down_proj,
 * shared_expert {gate, up, down}, shared_expert_gate). */
typedef struct moe_layer {
  int32_t hidden;        /* H                                                    */
  int32_t num_experts;   /* E                                                    */
  int32_t top_k;         /* K                                                    */
  int32_t expert_inner;  /* I                                                    */
  int32_t shared_inner;  /* Is                                                   */
  const void *router_w;             /* bf16 [E, H]      gate.weight                */
  const void *gate_up_w;            /* bf16 [E, 2I, H]  rows [0,I) gate, [I,2I) up */
  const void *down_w;               /* bf16 [E, H, I]   down_proj                  */
  const void *shared_gate_w;        /* bf16 [Is, H]     shared_expert.gate.weight  */
  const void *shared_up_w;          /* bf16 [Is, H]     shared_expert.up.weight    */
  const void *shared_down_w;        /* bf16 [H, Is]     shared_expert.down.weight  */
  const void *shared_expert_gate_w; /* bf16 [1, H]      shared_expert_gate.weight  */
  /* Score precision (Linnet page, Blocks: SparseMoe, whose gate and
   * shared_expert_gate are Linear<..., T> and whose ranks takes scores of type
   * T = bf16):
   *   0  router and shared-gate scores kept in fp32 (accumulation precision);
   *   1  each score rounded to the nearest bf16 (ties to even) before anything
   *      uses it: ranking (equal rounded scores order by expert index), the
   *      softmax weights, the sigmoid gate, and the logits moe_route returns.
   * Any other value is rejected with MOE_ERR_SHAPE. */
  int32_t logits_bf16;
  /* Layout of gate_up_w and down_w: 0 row-major as above; 1 the MFMA-tile
   * layout moe_tile_experts writes (same values in other places; every path
   * gives the same bits with either layout). */
  int32_t experts_tiled;
} moe_layer_t;

/* Bytes of device workspace that moe_route / moe_forward need for T tokens
 * (0 for T <= 0 or unsupported dimensions).  Non-decreasing in T: a workspace
 * of moe_workspace_bytes(L, T) bytes serves every call of 1..T tokens.
 * Host-only; no HIP call. */
size_t moe_workspace_bytes(const moe_layer_t *L, int64_t T);

/* Check the arguments of a moe_forward call without touching the GPU.
 * Returns the code moe_forward would return before its first HIP call. */
int moe_validate(const moe_layer_t *L, const void *x, int64_t T, const void *out,
                 const void *ws, size_t ws_bytes);

/* Routing and dispatch only (router, softmax, top-K, renormalise, the
 * shared-expert gate scalar, and the stable grouping of (token, k) pairs by
 * expert).  Same kernels and results as inside moe_forward.
 *   x         bf16 [T, H]
 *   topk_idx  int32 [T, K]  selected experts in rank order (descending logit,
 *                           ties to the lower expert index)
 *   topk_w    fp32 [T, K]   renormalised routing weights (sum to 1 per token)
 *   offsets   int32 [E+1]   segment starts: pairs of expert e occupy slots
 *                           offsets[e] .. offsets[e+1]-1; offsets[E] = T*K
 *   perm      int32 [T*K]   pair id q = t*K + k held by each slot, ascending
 *                           t within a segment
 *   shared_gate fp32 [T] or NULL   sigmoid(x[t] . shared_expert_gate_w)
 *   logits    fp32 [T, E] or NULL  router logits (fp32 accumulation; the
 *                                  rounded bf16 values when L->logits_bf16)
 * T = 0 is a successful no-op. */
int moe_route(const moe_layer_t *L, const void *x, int64_t T,
              int32_t *topk_idx, float *topk_w, int32_t *offsets, int32_t *perm,
              float *shared_gate, float *logits,
              void *ws, size_t ws_bytes, void *stream);

/* Forward-only router load-balance statistic of a batch ("Qwen3.6-35B-A3B —
 * Architecture Overview", section "MoE FFN: 256 Experts", Load Balancing:
 * an auxiliary loss penalises uneven expert use; the page gives no formula).
 * With f_e = counts[e] / (T K), the share of the T*K routing slots that expert
 * e receives, and P_e = (1/T) sum_t softmax(logits[t])[e], the batch-mean
 * full-softmax probability:
 *   lb        fp32 [1]   E * sum_e f_e * P_e  (1 when both are uniform; the
 *                        training loss would be 0.001 * lb)
 *   mean_prob fp32 [E] or NULL   P_e
 *   counts    int32 [E] or NULL  pairs routed to each expert
 * Device pointers, 4-byte aligned; x bf16 [T, H] and the workspace (size from
 * moe_workspace_bytes) 16-byte aligned.  Routes with moe_forward's logits
 * kernel for T > 16 (at any T), the same top-K rule and summation order
 * (identical indices and weights) and the same dispatch kernels; sums are in
 * a fixed order, so repeated calls give identical results.  T = 0 is a
 * successful no-op.  Errors as moe_route. */
int moe_load_balance(const moe_layer_t *L, const void *x, int64_t T, float *lb, float *mean_prob,
                     int32_t *counts, void *ws, size_t ws_bytes, void *stream);

/* The whole layer: out bf16 [T, H] (round to nearest even from an fp32
 * accumulation).  x and out must not overlap.  T = 0 is a successful no-op. */
int moe_forward(const moe_layer_t *L, const void *x, int64_t T, void *out,
                void *ws, size_t ws_bytes, void *stream);

/* The MoE sub-block of a transformer block: out = h + MoE(RMSNorm(h))
 * ("Qwen3.6-35B-A3B — Architecture Overview", Stage 2: Transform Blocks:
 * RMSNorm -> MoE FFN -> +residual; Linnet model page, AttentionLayer /
 * DeltaLayer: post_attention_layernorm RmsNorm<H> with weight [H]).
 *   h       bf16 [T, H]  residual stream entering the sub-block
 *   norm_w  bf16 [H]     RMSNorm weight; x = bf16(h / sqrt(mean(h^2) + eps) * norm_w)
 *                        (the textbook RMSNorm: the pages give no formula)
 *   eps     finite, >= 0
 *   out     bf16 [T, H]  bf16(h + layer(x)), the residual added to the fp32
 *                        accumulation before its one rounding
 * The norm is applied in the fused decode kernel's LDS copy of x (T <= 16) or
 * by a norm kernel feeding the grouped path; the residual is added where the
 * output is written (no extra pass over out).  Workspace, alignment, errors
 * and h/out overlap as moe_forward (h plays the role of x). */
int moe_block_forward(const moe_layer_t *L, const void *norm_w, float eps, const void *h, int64_t T,
                      void *out, void *ws, size_t ws_bytes, void *stream);

/* RMSNorm alone (the norm moe_block_forward applies): x = bf16(h[t] /
 * sqrt(mean_j h[t, j]^2 + eps) * norm_w), fp32 arithmetic, the sum of squares
 * in a fixed order.  h, x bf16 [T, H], norm_w bf16 [H], 16-byte aligned, H a
 * positive multiple of 256 (at most 65536), no workspace.  T = 0 is a
 * successful no-op. */
int moe_rmsnorm(const void *norm_w, float eps, const void *h, int64_t T, int64_t H, void *x, void *stream);

/* Rank of every expert in each row of scores (Linnet page, Blocks: SparseMoe,
 * ranks: integer ranks [R, Experts] of a score tensor [R, Experts]):
 *   ranks[r, e] = #{j : l[r, j] > l[r, e]} + #{j < e : l[r, j] == l[r, e]}
 * i.e. 0 for the best score, equal scores ordered by lower expert index, the
 * same order moe_route selects in (its topk_idx[r, k] is the expert of rank
 * k).  -0 equals +0; NaN counts as -inf.
 *   logits  [R, E] device, fp32 (dtype 0, 4-byte aligned) or bf16 (dtype 1,
 *           2-byte aligned)
 *   ranks   int32 [R, E] device, 4-byte aligned
 * 1 <= E <= 256, 0 <= R <= 2^22; R = 0 is a successful no-op.  Asynchronous
 * on stream; errors as moe_route. */
int moe_ranks(const void *logits, int32_t dtype, int64_t R, int64_t E, int32_t *ranks, void *stream);

/* Rewrite the routed experts' weights of L (row-major, device memory) into
 * the MFMA-tile layout: for each expert, each block of 16 consecutive rows and
 * each 64-wide k-step, 2 KB ordered half h (0, 1), lane l (0..63), 8 elements,
 * lane l holding row 16 * block + l % 16 and k-step elements
 * 16 (l / 16) + 8 h .. + 7.  Each load instruction of the grouped GEMMs then
 * reads 1 KB of consecutive bytes.
 *   gate_up_tiled  device, E * 2I * H bf16, 16-byte aligned, not overlapping
 *   down_tiled     device, E * H * I bf16, 16-byte aligned, not overlapping
 * A layer descriptor with these pointers and experts_tiled = 1 gives results
 * bit-identical to the row-major layer's grouped path.  Asynchronous on
 * stream; errors as moe_forward (MOE_ERR_SHAPE if L is already tiled). */
int moe_tile_experts(const moe_layer_t *L, void *gate_up_tiled, void *down_tiled, void *stream);

/* Device bytes of an expert cache with `capacity` slots for moe_forward_streamed:
 * each slot holds one routed expert's gate_up [2I, H] and down [H, I] bf16
 * weights (6 MiB at H = 2048, I = 512).  0 if capacity < 1 or the dimensions
 * are unsupported.  Host-only; no HIP call. */
size_t moe_expert_cache_bytes(const moe_layer_t *L, int32_t capacity);

/* The layer with its routed experts' weights in host memory, streamed into a
 * device cache on demand ("One Token Through Qwen3.6" (InferedThoughts),
 * Where the Weights Live: weights pass from system RAM into GPU memory, the
 * hierarchy made explicit; One Complete Decode Step: routing decides which
 * expert weights a layer needs).
 *   L->gate_up_w, L->down_w  pinned host memory (hipHostMalloc), [E, 2I, H]
 *                            and [E, H, I] bf16, 16-byte aligned; every other
 *                            weight in device memory as for moe_forward
 *   cache, cache_bytes       device memory, 16-byte aligned; its slot count
 *                            C = min(E, cache_bytes / moe_expert_cache_bytes(L, 1))
 *                            must be at least 1
 * The router and dispatch run on the device as in moe_forward; then the
 * touched experts (ascending index) are processed in rounds of C: each round
 * copies its experts' weights from host memory into the cache (a device
 * kernel reading the host mapping: no host synchronisation, the whole call
 * stays asynchronous on `stream`) and runs the grouped GEMMs on them.  Only
 * touched experts cross the host link (U * 6 MiB for U touched experts).
 * Results equal moe_forward's grouped path for the same inputs bit for bit
 * (T > 16; smaller batches use the grouped path here, not the fused decode
 * kernel).  The cache holds no state between calls; calls sharing a cache
 * must be ordered on one stream.  MOE_ERR_MEMORY if gate_up_w or down_w is not
 * pinned host memory or its allocation is smaller than E experts.  Other
 * arguments, workspace and errors as moe_forward. */
int moe_forward_streamed(const moe_layer_t *L, const void *x, int64_t T, void *out, void *cache,
                         size_t cache_bytes, void *ws, size_t ws_bytes, void *stream);

/* moe_forward that also records caller-created HIP events (hipEvent_t) on
 * `stream` at its phase boundaries, for timing the kernels:
 *   events[0] before the router, [1] after the router (top-K, weights, shared
 *   gate), [2] after dispatch (counting sort), [3] after the gate_up GEMM,
 *   [4] after the down GEMM, [5] after the combine.
 * A path that fuses phases records the boundaries it does not separate back
 * to back.  events == NULL is exactly moe_forward.  Same arguments, errors
 * and results as moe_forward. */
int moe_forward_traced(const moe_layer_t *L, const void *x, int64_t T, void *out,
                       void *ws, size_t ws_bytes, void *stream, void *const *events);

/* Bytes of the control block at the start of every workspace (a constant;
 * part of moe_workspace_bytes).  Host-only. */
size_t moe_workspace_control_bytes(void);

/* Status of the latest moe_route / moe_forward / moe_block_forward /
 * moe_forward_traced / moe_load_balance / moe_forward_streamed call made with
 * this workspace, once it has run: synchronises `stream` (the stream those
 * calls were made on), stores in *timed_out_calls (if not NULL) how many
 * calls on this workspace since it was zero-filled had a wait time out, then
 * returns
 *   MOE_OK           the call completed normally (or no call has used ws yet);
 *   MOE_ERR_TIMEOUT  the call took the fused small-batch path (T <= 16) and one
 *                    of that kernel's cross-workgroup waits gave up after its
 *                    time budget: the kernel ran to completion, but the call's
 *                    outputs are invalid.  The kernel runs one workgroup per
 *                    compute unit and its waits need all of them resident at
 *                    once, which holds when no other work occupies the
 *                    device's compute units for the whole budget (0.25 s);
 *                    a budget of 0 forces this status;
 *   MOE_ERR_NULL / MOE_ERR_ALIGN / MOE_ERR_WORKSPACE for a bad ws pointer or
 *                    ws_bytes < moe_workspace_control_bytes();
 *   MOE_ERR_LAUNCH   if the copy of the status words or the
 *                    synchronisation fails.
 * The grouped path (T > 16) has no such waits and always reports MOE_OK. */
int moe_workspace_status(const void *ws, size_t ws_bytes, void *stream, uint32_t *timed_out_calls);

/* Diagnostic, process-wide: the time each cross-workgroup wait of the fused
 * kernel may take before it gives up (default 250000 us), for calls made
 * after this one.  0 makes a wait give up at its first unsuccessful poll (it
 * forces the MOE_ERR_TIMEOUT path; every kernel still runs to completion and
 * touches only its own arrays).  Returns the previous budget, or -1 (nothing
 * changed) if us is outside [0, 60000000].  Host-only; no HIP call. */
int64_t moe_set_wait_budget_us(int64_t us);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and the same results, bit for bit, with the workspace replaced
 * by a static scratch array of 16 MiB that the library holds on each device it
 * runs on until the process ends (enough for T up to 244 at H 2048, E 256,
 * K 8, I = Is = 512; moe_workspace_bytes(L, T) must be at most 16 MiB, else
 * MOE_ERR_WORKSPACE and nothing is enqueued).  No hipMalloc, hipFree or other
 * allocating call.  The first call on a device also enqueues, on `stream`, a
 * kernel that zero-fills the scratch's control block.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (other streams, or
 * other host threads) race and must be serialised by the caller.  Other
 * arguments and errors as moe_forward; a fused-kernel timeout (see
 * moe_workspace_status) is not reported through this entry point. */
int moe_forward_noalloc(const moe_layer_t *L, const void *x, int64_t T, void *out, void *stream);

/* Static text for a status code. */
const char *moe_strerror(int code);

/* Text describing the last failure on the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

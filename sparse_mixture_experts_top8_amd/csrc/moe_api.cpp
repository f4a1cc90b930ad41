// C ABI of the MoE layer: argument checks, workspace carving and the launch
// sequence.  Declared in include/moe.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <unistd.h>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <algorithm>

#include "moe.h"
#include "kernels.hpp"

using moe::bf16_t;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

constexpr int64_t kMaxTokens = int64_t(1) << 22;

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
constexpr size_t align256_c(size_t v) { return (v + 255) & ~size_t(255); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const moe_layer_t* L, int64_t T) {
  if (!L) return fail(MOE_ERR_NULL, "layer descriptor is NULL");
  const int64_t H = L->hidden, E = L->num_experts, K = L->top_k, I = L->expert_inner, Is = L->shared_inner;
  if (T < 0) return fail(MOE_ERR_SHAPE, "T = %lld is negative", (long long)T);
  if (T > kMaxTokens) return fail(MOE_ERR_SHAPE, "T = %lld exceeds the supported maximum %lld", (long long)T, (long long)kMaxTokens);
  if (H <= 0 || H % 256) return fail(MOE_ERR_SHAPE, "hidden = %lld must be a positive multiple of 256", (long long)H);
  if (E < 1 || E > 256) return fail(MOE_ERR_SHAPE, "num_experts = %lld must be in [1, 256]", (long long)E);
  if (K < 1 || K > 8 || K > E) return fail(MOE_ERR_SHAPE, "top_k = %lld must be in [1, min(8, num_experts)]", (long long)K);
  if (I <= 0 || I % 64) return fail(MOE_ERR_SHAPE, "expert_inner = %lld must be a positive multiple of 64", (long long)I);
  if (Is <= 0 || Is % 64) return fail(MOE_ERR_SHAPE, "shared_inner = %lld must be a positive multiple of 64", (long long)Is);
  if (L->logits_bf16 != 0 && L->logits_bf16 != 1)
    return fail(MOE_ERR_SHAPE, "logits_bf16 = %d must be 0 or 1", (int)L->logits_bf16);
  if (L->experts_tiled != 0 && L->experts_tiled != 1)
    return fail(MOE_ERR_SHAPE, "experts_tiled = %d must be 0 or 1", (int)L->experts_tiled);
  return MOE_OK;
}

struct Carve {
  moe::Work w;
  size_t bytes;
};

// Both workspace layouts start with the same two regions: the control block
// (error word, latest-call word, the fused path's arrival flags) and the fused
// path's tagged logits sized for its largest batch.  Nothing else writes
// them, so a word keeps its meaning whichever path ran last.
constexpr size_t kCtlBytes = align256_c((size_t)moe::kDecodeCtlWords * 4);
constexpr size_t kLogitTagBytes =
    align256_c((size_t)moe::kDecodeReplicas * (size_t)(moe::kDecodeMaxT * 256 + 64) * 8);
constexpr size_t kControlRegionBytes = kCtlBytes + kLogitTagBytes;
static_assert(kLogitTagBytes >= ((size_t)moe::kRouteMaxT * 256 + (size_t)moe::kDecodeReplicas * moe::kRouteSelStride) * 8,
              "the tagged region holds the fused route's logits and selection copies");
static_assert(moe::kDecodeMaxT * 256 + 64 == 16 * 256 + 64, "tagged-logit region sized for the largest fused batch");

// Workspace layout, each region 256-byte aligned.  With base == nullptr only
// the size is computed.
Carve carve(const moe_layer_t* L, int64_t T, char* base) {
  const size_t H = L->hidden, E = L->num_experts, K = L->top_k, I = L->expert_inner, Is = L->shared_inner;
  const size_t t = (size_t)T, tk = t * K, nblk = (size_t)moe::router_blocks(T);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  Carve c{};
  c.w.ctl = (uint32_t*)take(kCtlBytes);
  c.w.lt = (uint64_t*)take(kLogitTagBytes);
  c.w.topk_idx = (int32_t*)take(tk * 4);
  c.w.topk_w = (float*)take(tk * 4);
  c.w.gate_s = (float*)take(t * 4);
  c.w.rlog = (float*)take((size_t)moe::router_partial_rows(T, (int)H) * moe::router_cols((int)E) * 4);
  c.w.blk_counts = (int32_t*)take(nblk * E * 4);
  c.w.offsets = (int32_t*)take((E + 1) * 4);
  c.w.tiles_gu = (int32_t*)take((E + 2) * 4);
  c.w.tiles_dn = (int32_t*)take((E + 2) * 4);
  c.w.claims = (int32_t*)take(2 * 8 * 128);
  c.w.tdesc_gu = (int4*)take((size_t)moe::gemm_tile_bound(T, (int)K, (int)E, 2 * (int)I, 2 * (int)Is) * 16);
  c.w.tdesc_dn = (int4*)take((size_t)moe::gemm_tile_bound(T, (int)K, (int)E, (int)H, (int)H) * 16);
  c.w.perm = (int32_t*)take(tk * 4);
  c.w.slot_of = (int32_t*)take(tk * 4);
  c.w.slot_tok = (int32_t*)take(tk * 4);
  c.w.h = (bf16_t*)take(tk * I * 2);
  c.w.h_sh = (bf16_t*)take(t * Is * 2);
  c.w.y = (bf16_t*)take((tk + t) * H * 2);
  c.w.psum = (float*)take(nblk * E * 4);
  c.w.xn = (bf16_t*)take(t * H * 2);
  c.w.st_list = (int32_t*)take((E + 1) * 4);
  c.w.st_slot = (int32_t*)take(E * 4);
  c.w.st_win_gu = (int32_t*)take(E * 16);
  c.w.st_win_dn = (int32_t*)take(E * 16);
  c.bytes = off;
  return c;
}

// The fused decode path serves small batches of the supported shapes
// (T <= kDecodeMaxT); whether the device's grid can hold the layer's
// per-workgroup shares is decided at launch (decode_fits), so the workspace of
// such a call is sized for either path.
bool decode_shape(const moe_layer_t* L, int64_t T) {
  return T >= 1 && T <= moe::kDecodeMaxT && L->hidden <= 2048 && L->expert_inner <= 512 &&
         L->shared_inner <= 512;
}
bool use_decode(const moe_layer_t* L, int64_t T, int grid) {
  return decode_shape(L, T) && moe::decode_fits(L->hidden, L->num_experts, L->shared_inner, grid);
}

struct DecodeCarve {
  uint32_t* ctl;
  uint64_t* logits_t;
  int32_t* topk_idx;
  float* topk_w;
  float* gate_s;
  bf16_t* h;
  bf16_t* h_sh;
  size_t bytes;
};

DecodeCarve carve_decode(const moe_layer_t* L, int64_t T, char* base) {
  const size_t E = L->num_experts, K = L->top_k, I = L->expert_inner, Is = L->shared_inner;
  const size_t t = (size_t)T, tk = t * K;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  DecodeCarve c{};
  c.ctl = (uint32_t*)take(kCtlBytes);
  c.logits_t = (uint64_t*)take(kLogitTagBytes);   // copies at stride decode_logit_stride(T) <= that of kDecodeMaxT
  c.topk_idx = (int32_t*)take(tk * 4);
  c.topk_w = (float*)take(tk * 4);
  c.gate_s = (float*)take(t * 4);
  c.h = (bf16_t*)take(tk * I * 2);
  c.h_sh = (bf16_t*)take(t * Is * 2);
  c.bytes = off;
  return c;
}

// Non-decreasing in T, so that a workspace sized for T serves every call of
// 1..T tokens: every region of carve() grows with T (the router partials and
// tile descriptors through their bounds), and past the fused decode path's
// largest batch its workspace for that batch is still covered.
size_t workspace_need(const moe_layer_t* L, int64_t T) {
  const size_t grouped = carve(L, T, nullptr).bytes;
  const int64_t td = std::min<int64_t>(T, moe::kDecodeMaxT);
  return decode_shape(L, td) ? std::max(grouped, carve_decode(L, td, nullptr).bytes) : grouped;
}

// Call-unique epochs for the decode path's start protocol: a per-process
// sequence started from the clock and the process id.
std::atomic<unsigned long long> g_epoch{0};
std::once_flag g_epoch_once;
unsigned long long next_epoch() {
  std::call_once(g_epoch_once, [] {
    const unsigned long long t = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    g_epoch.store((t << 16) ^ ((unsigned long long)getpid() << 44) ^ 0x9E3779B97F4A7C15ull);
  });
  // The low 32 bits tag the decode path's published logits; 0 is never used.
  unsigned long long e = ++g_epoch;
  while ((uint32_t)e == 0u) e = ++g_epoch;
  return e;
}

// Budget of each bounded wait of the fused path, in ticks of the 100 MHz
// wall clock (moe_set_wait_budget_us).
std::atomic<unsigned long long> g_wait_ticks{moe::kDefaultWaitTicks};

moe::LayerArgs layer_args(const moe_layer_t* L) {
  moe::LayerArgs a;
  a.H = L->hidden;
  a.E = L->num_experts;
  a.K = L->top_k;
  a.I = L->expert_inner;
  a.Is = L->shared_inner;
  a.router_w = (const bf16_t*)L->router_w;
  a.gate_up_w = (const bf16_t*)L->gate_up_w;
  a.down_w = (const bf16_t*)L->down_w;
  a.sh_gate_w = (const bf16_t*)L->shared_gate_w;
  a.sh_up_w = (const bf16_t*)L->shared_up_w;
  a.sh_down_w = (const bf16_t*)L->shared_down_w;
  a.sh_expert_gate = (const bf16_t*)L->shared_expert_gate_w;
  a.logits_bf16 = L->logits_bf16;
  a.tiled = L->experts_tiled;
  return a;
}

int check_weights(const moe_layer_t* L) {
  const void* p[7] = {L->router_w, L->gate_up_w, L->down_w, L->shared_gate_w,
                      L->shared_up_w, L->shared_down_w, L->shared_expert_gate_w};
  static const char* names[7] = {"router_w", "gate_up_w", "down_w", "shared_gate_w",
                                 "shared_up_w", "shared_down_w", "shared_expert_gate_w"};
  for (int i = 0; i < 7; ++i) {
    if (!p[i]) return fail(MOE_ERR_NULL, "%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  return MOE_OK;
}

// Per-device facts, looked up once: is it a gfx950, how many CUs.
struct DeviceInfo {
  std::once_flag once;
  bool ok = false;
  int cus = 0;
  int decode_grid = 0;
  char arch[64] = {0};
};
DeviceInfo g_dev[64];

int device_check(int* cus, int* decode_grid = nullptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "device index %d out of range", dev);
  DeviceInfo& d = g_dev[dev];
  std::call_once(d.once, [&] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      std::strncpy(d.arch, prop.gcnArchName, sizeof d.arch - 1);
      d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      d.cus = prop.multiProcessorCount;
      if (d.ok) d.decode_grid = std::min(d.cus, moe::decode_max_grid(d.cus));
    }
  });
  if (!d.ok) return fail(MOE_ERR_DEVICE, "device %d is '%s', not gfx950", dev, d.arch);
  *cus = d.cus;
  if (decode_grid) *decode_grid = d.decode_grid;
  return MOE_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

moe::DecodeArgs decode_args(const moe_layer_t* L, const void* x, int64_t T, const DecodeCarve& c) {
  moe::DecodeArgs a{};
  a.L = layer_args(L);
  a.x = (const bf16_t*)x;
  a.T = (int)T;
  a.ctl = c.ctl;
  a.logits_t = c.logits_t;
  a.topk_idx = c.topk_idx;
  a.topk_w = c.topk_w;
  a.gate_s = c.gate_s;
  a.h = c.h;
  a.h_sh = c.h_sh;
  a.epoch = next_epoch();
  a.wait_ticks = g_wait_ticks.load(std::memory_order_relaxed);
  return a;
}

// The grouped path's workspace view for one call (its tag in the control block).
moe::Work grouped_work(const moe_layer_t* L, int64_t T, void* ws) {
  moe::Work w = carve(L, T, (char*)ws).w;
  w.call_tag = (uint32_t)next_epoch();
  return w;
}

// Router and dispatch of the grouped path: one fused launch for small
// batches (its bounded waits report through the control block like the
// fused decode path's), else the router kernels, then the dispatch kernels.
// between() runs after the router (a phase mark of the traced forward).
template <typename Between>
int route_dispatch(const moe::LayerArgs& a, const bf16_t* x, int t, const moe::Work& w, float* logits,
                   hipStream_t s, Between between) {
  int rc;
  if (moe::route_fused_fits(t, a.H, a.K)) {
    if ((rc = launch_status(moe::launch_route_fused(a, x, t, w, logits, g_wait_ticks.load(std::memory_order_relaxed), s),
                            "route")) != MOE_OK)
      return rc;
    return between();
  }
  if ((rc = launch_status(moe::launch_router(a, x, t, w, logits, s), "router")) != MOE_OK) return rc;
  if ((rc = between()) != MOE_OK) return rc;
  return launch_status(moe::launch_dispatch(a, t, w, s), "dispatch");
}
int no_mark() { return MOE_OK; }

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_layer_t* L, int64_t T) {
  if (check_dims(L, T) != MOE_OK || T <= 0) return 0;
  return workspace_need(L, T);
}

int moe_validate(const moe_layer_t* L, const void* x, int64_t T, const void* out, const void* ws,
                 size_t ws_bytes) {
  int rc = check_dims(L, T);
  if (rc != MOE_OK) return rc;
  if ((rc = check_weights(L)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x) return fail(MOE_ERR_NULL, "x is NULL");
  if (!out) return fail(MOE_ERR_NULL, "out is NULL");
  if (!ws) return fail(MOE_ERR_NULL, "workspace is NULL");
  if (!aligned16(x)) return fail(MOE_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned16(out)) return fail(MOE_ERR_ALIGN, "out is not 16-byte aligned");
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  const size_t need = workspace_need(L, T);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for T = %lld", ws_bytes, need, (long long)T);
  return MOE_OK;
}

int moe_route(const moe_layer_t* L, const void* x, int64_t T, int32_t* topk_idx, float* topk_w,
              int32_t* offsets, int32_t* perm, float* shared_gate, float* logits, void* ws,
              size_t ws_bytes, void* stream) {
  int rc = check_dims(L, T);
  if (rc != MOE_OK) return rc;
  if ((rc = check_weights(L)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !topk_w || !offsets || !perm || !ws)
    return fail(MOE_ERR_NULL, "x, topk_idx, topk_w, offsets, perm and workspace are required");
  const void* ptrs[8] = {x, topk_idx, topk_w, offsets, perm, ws, shared_gate, logits};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(MOE_ERR_ALIGN, "a pointer argument is not 16-byte aligned");
  const size_t need = workspace_need(L, T);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for T = %lld", ws_bytes, need, (long long)T);
  int cus = 0, dgrid = 0;
  if ((rc = device_check(&cus, &dgrid)) != MOE_OK) return rc;
  if (use_decode(L, T, dgrid)) {
    moe::DecodeArgs a = decode_args(L, x, T, carve_decode(L, T, (char*)ws));
    a.route_only = 1;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    if (shared_gate) a.gate_s = shared_gate;
    a.logits_out = logits;
    a.offsets_out = offsets;
    a.perm_out = perm;
    return launch_status(moe::launch_decode(a, dgrid, (hipStream_t)stream), "decode (route)");
  }
  moe::Work w = grouped_work(L, T, ws);
  w.topk_idx = topk_idx;
  w.topk_w = topk_w;
  w.offsets = offsets;
  w.perm = perm;
  if (shared_gate) w.gate_s = shared_gate;
  const moe::LayerArgs a = layer_args(L);
  hipStream_t s = (hipStream_t)stream;
  return route_dispatch(a, (const bf16_t*)x, (int)T, w, logits, s, no_mark);
}

int moe_load_balance(const moe_layer_t* L, const void* x, int64_t T, float* lb, float* mean_prob,
                     int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(L, T);
  if (rc != MOE_OK) return rc;
  if ((rc = check_weights(L)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !lb || !ws) return fail(MOE_ERR_NULL, "x, lb and workspace are required");
  const void* ptrs[5] = {x, ws, lb, mean_prob, counts};
  for (int i = 0; i < 2; ++i)
    if (!aligned16(ptrs[i])) return fail(MOE_ERR_ALIGN, "x or the workspace is not 16-byte aligned");
  for (int i = 2; i < 5; ++i)
    if (ptrs[i] && ((uintptr_t)ptrs[i] & 3u)) return fail(MOE_ERR_ALIGN, "lb, mean_prob and counts need 4-byte alignment");
  const size_t need = workspace_need(L, T);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for T = %lld", ws_bytes, need, (long long)T);
  int cus = 0, dgrid = 0;
  if ((rc = device_check(&cus, &dgrid)) != MOE_OK) return rc;
  // Always the grouped path's router and dispatch (any T).
  const moe::Work w = grouped_work(L, T, ws);
  const moe::LayerArgs a = layer_args(L);
  hipStream_t s = (hipStream_t)stream;
  const int t = (int)T;
  if ((rc = launch_status(moe::launch_router(a, (const bf16_t*)x, t, w, nullptr, s, w.psum), "router")) != MOE_OK)
    return rc;
  if ((rc = launch_status(moe::launch_dispatch(a, t, w, s), "dispatch")) != MOE_OK) return rc;
  return launch_status(moe::launch_load_balance(a, t, w, lb, mean_prob, counts, s), "load balance");
}

namespace {

// The layer (norm_w == nullptr) or the sub-block out = x + layer(RMSNorm(x)).
int forward_impl(const moe_layer_t* L, const void* x, int64_t T, void* out, void* ws, size_t ws_bytes,
                 void* stream, void* const* events, const void* norm_w, float eps) {
  int rc = moe_validate(L, x, T, out, ws, ws_bytes);
  if (rc != MOE_OK || T == 0) return rc;
  int cus = 0, dgrid = 0;
  if ((rc = device_check(&cus, &dgrid)) != MOE_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int i) -> int {
    if (!events) return MOE_OK;
    return launch_status(hipEventRecord((hipEvent_t)events[i], s), "hipEventRecord");
  };
  if ((rc = mark(0)) != MOE_OK) return rc;
  if (use_decode(L, T, dgrid)) {
    moe::DecodeArgs da = decode_args(L, x, T, carve_decode(L, T, (char*)ws));
    da.out = (bf16_t*)out;
    if (norm_w) {
      da.norm_w = (const bf16_t*)norm_w;
      da.eps = eps;
      da.residual = (const bf16_t*)x;
    }
    if ((rc = launch_status(moe::launch_decode(da, dgrid, s), "decode")) != MOE_OK) return rc;
    for (int i = 1; i <= 5; ++i)
      if ((rc = mark(i)) != MOE_OK) return rc;
    return MOE_OK;
  }
  const moe::Work w = grouped_work(L, T, ws);
  const moe::LayerArgs a = layer_args(L);
  const int t = (int)T;
  const bf16_t* xin = (const bf16_t*)x;
  if (norm_w) {
    if ((rc = launch_status(moe::launch_rmsnorm(xin, (const bf16_t*)norm_w, eps, t, a.H, w.xn, s), "rmsnorm")) !=
        MOE_OK)
      return rc;
    xin = w.xn;
  }
  if ((rc = route_dispatch(a, xin, t, w, nullptr, s, [&] { return mark(1); })) != MOE_OK) return rc;
  if ((rc = mark(2)) != MOE_OK) return rc;
  if ((rc = launch_status(moe::launch_gate_up(a, xin, t, w, cus, s), "gate_up")) != MOE_OK) return rc;
  if ((rc = mark(3)) != MOE_OK) return rc;
  if ((rc = launch_status(moe::launch_down(a, t, w, cus, s), "down")) != MOE_OK) return rc;
  if ((rc = mark(4)) != MOE_OK) return rc;
  if ((rc = launch_status(moe::launch_combine(a, t, w, (bf16_t*)out, s, norm_w ? (const bf16_t*)x : nullptr),
                          "combine")) != MOE_OK)
    return rc;
  return mark(5);
}

}  // namespace

int moe_forward_traced(const moe_layer_t* L, const void* x, int64_t T, void* out, void* ws,
                       size_t ws_bytes, void* stream, void* const* events) {
  return forward_impl(L, x, T, out, ws, ws_bytes, stream, events, nullptr, 0.f);
}

int moe_forward(const moe_layer_t* L, const void* x, int64_t T, void* out, void* ws, size_t ws_bytes,
                void* stream) {
  return forward_impl(L, x, T, out, ws, ws_bytes, stream, nullptr, nullptr, 0.f);
}

int moe_block_forward(const moe_layer_t* L, const void* norm_w, float eps, const void* h, int64_t T, void* out,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!norm_w) return fail(MOE_ERR_NULL, "norm_w is NULL");
  if (!aligned16(norm_w)) return fail(MOE_ERR_ALIGN, "norm_w is not 16-byte aligned");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MOE_ERR_SHAPE, "eps must be finite and >= 0");
  return forward_impl(L, h, T, out, ws, ws_bytes, stream, nullptr, norm_w, eps);
}

int moe_rmsnorm(const void* norm_w, float eps, const void* h, int64_t T, int64_t H, void* x, void* stream) {
  if (T < 0 || T > (int64_t(1) << 22)) return fail(MOE_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (H <= 0 || H % 256 || H > (int64_t(1) << 16))
    return fail(MOE_ERR_SHAPE, "hidden = %lld must be a positive multiple of 256", (long long)H);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MOE_ERR_SHAPE, "eps must be finite and >= 0");
  if (T == 0) return MOE_OK;
  if (!norm_w || !h || !x) return fail(MOE_ERR_NULL, "norm_w, h and x are required");
  if (!aligned16(norm_w) || !aligned16(h) || !aligned16(x)) return fail(MOE_ERR_ALIGN, "a pointer is not 16-byte aligned");
  int cus = 0, dgrid = 0;
  int rc = device_check(&cus, &dgrid);
  if (rc != MOE_OK) return rc;
  return launch_status(moe::launch_rmsnorm((const bf16_t*)h, (const bf16_t*)norm_w, eps, (int)T, (int)H, (bf16_t*)x,
                                           (hipStream_t)stream),
                       "rmsnorm");
}

int moe_ranks(const void* logits, int32_t dtype, int64_t R, int64_t E, int32_t* ranks, void* stream) {
  if (dtype != 0 && dtype != 1) return fail(MOE_ERR_SHAPE, "dtype = %d must be 0 (fp32) or 1 (bf16)", (int)dtype);
  if (E < 1 || E > 256) return fail(MOE_ERR_SHAPE, "E = %lld must be in [1, 256]", (long long)E);
  if (R < 0 || R > kMaxTokens) return fail(MOE_ERR_SHAPE, "R = %lld out of range", (long long)R);
  if (R == 0) return MOE_OK;
  if (!logits || !ranks) return fail(MOE_ERR_NULL, "logits and ranks are required");
  if (((uintptr_t)logits & (dtype ? 1u : 3u)) || ((uintptr_t)ranks & 3u))
    return fail(MOE_ERR_ALIGN, "logits and ranks need their element alignment");
  int cus = 0, dgrid = 0;
  int rc = device_check(&cus, &dgrid);
  if (rc != MOE_OK) return rc;
  return launch_status(moe::launch_ranks(logits, (int)dtype, (int)R, (int)E, ranks, (hipStream_t)stream), "ranks");
}

}  // extern "C"

namespace {

// Bytes of one expert's gate_up and down weights.
size_t expert_gu_bytes(const moe_layer_t* L) { return (size_t)2 * L->expert_inner * L->hidden * 2; }
size_t expert_dn_bytes(const moe_layer_t* L) { return (size_t)L->hidden * L->expert_inner * 2; }

// p must lie in pinned host memory whose allocation holds [p, p + need);
// *dev receives the device address of p.
int host_span(const void* p, size_t need, const char* name, const void** dev) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess || at.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(MOE_ERR_MEMORY, "%s is not pinned host memory (allocate it with hipHostMalloc)", name);
  }
  void* base = nullptr;
  size_t size = 0;
  if (hipPointerGetAttribute(&base, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR, (hipDeviceptr_t)p) != hipSuccess ||
      hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE, (hipDeviceptr_t)p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_MEMORY, "%s: the extent of its allocation cannot be queried", name);
  }
  const size_t at_off = (size_t)((const char*)p - (const char*)base);
  if ((const char*)p < (const char*)base || at_off > size || size - at_off < need)
    return fail(MOE_ERR_MEMORY, "%s: its allocation holds %zu bytes from it, %zu needed", name,
                at_off <= size ? size - at_off : (size_t)0, need);
  void* dbase = nullptr;
  if (hipHostGetDevicePointer(&dbase, base, 0) != hipSuccess || !dbase) {
    (void)hipGetLastError();
    return fail(MOE_ERR_MEMORY, "%s: no device mapping for its host allocation", name);
  }
  *dev = (const char*)dbase + at_off;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_tile_experts(const moe_layer_t* L, void* gate_up_tiled, void* down_tiled, void* stream) {
  int rc = check_dims(L, 1);
  if (rc != MOE_OK) return rc;
  if ((rc = check_weights(L)) != MOE_OK) return rc;
  if (L->experts_tiled) return fail(MOE_ERR_SHAPE, "the layer's experts are already tiled");
  if (!gate_up_tiled || !down_tiled) return fail(MOE_ERR_NULL, "gate_up_tiled and down_tiled are required");
  if (!aligned16(gate_up_tiled) || !aligned16(down_tiled)) return fail(MOE_ERR_ALIGN, "an output is not 16-byte aligned");
  int cus = 0, dgrid = 0;
  if ((rc = device_check(&cus, &dgrid)) != MOE_OK) return rc;
  const int E = L->num_experts, H = L->hidden, I = L->expert_inner;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = launch_status(moe::launch_pack_tiles((const bf16_t*)L->gate_up_w, (bf16_t*)gate_up_tiled, E, 2 * I, H, s),
                          "tile gate_up")) != MOE_OK)
    return rc;
  return launch_status(moe::launch_pack_tiles((const bf16_t*)L->down_w, (bf16_t*)down_tiled, E, H, I, s),
                       "tile down");
}

size_t moe_expert_cache_bytes(const moe_layer_t* L, int32_t capacity) {
  if (check_dims(L, 1) != MOE_OK || capacity < 1) return 0;
  return (size_t)capacity * (expert_gu_bytes(L) + expert_dn_bytes(L));
}

int moe_forward_streamed(const moe_layer_t* L, const void* x, int64_t T, void* out, void* cache,
                         size_t cache_bytes, void* ws, size_t ws_bytes, void* stream) {
  int rc = moe_validate(L, x, T, out, ws, ws_bytes);
  if (rc != MOE_OK || T == 0) return rc;
  if (!cache) return fail(MOE_ERR_NULL, "the expert cache is NULL");
  if (!aligned16(cache)) return fail(MOE_ERR_ALIGN, "the expert cache is not 16-byte aligned");
  const size_t gu = expert_gu_bytes(L), dn = expert_dn_bytes(L);
  const int64_t E = L->num_experts;
  const int64_t C = std::min<int64_t>((int64_t)(cache_bytes / (gu + dn)), E);
  if (C < 1) return fail(MOE_ERR_WORKSPACE, "the expert cache has %zu bytes, one slot needs %zu", cache_bytes, gu + dn);
  int cus = 0, dgrid = 0;
  if ((rc = device_check(&cus, &dgrid)) != MOE_OK) return rc;
  const void *host_gu = nullptr, *host_dn = nullptr;
  if ((rc = host_span(L->gate_up_w, (size_t)E * gu, "gate_up_w", &host_gu)) != MOE_OK) return rc;
  if ((rc = host_span(L->down_w, (size_t)E * dn, "down_w", &host_dn)) != MOE_OK) return rc;
  const int64_t R = (std::min<int64_t>(E, T * L->top_k) + C - 1) / C;
  const moe::Work w = grouped_work(L, T, ws);
  moe::LayerArgs a = layer_args(L);
  char* slot_gu = (char*)cache;
  char* slot_dn = slot_gu + (size_t)C * gu;
  hipStream_t s = (hipStream_t)stream;
  const int t = (int)T;
  // The separate router kernels (no cross-workgroup waits), whose routing the
  // fused route reproduces bit for bit: the stream plan and the slot map
  // trust the dispatch tables.
  if ((rc = launch_status(moe::launch_router(a, (const bf16_t*)x, t, w, nullptr, s), "router")) != MOE_OK) return rc;
  if ((rc = launch_status(moe::launch_dispatch(a, t, w, s), "dispatch")) != MOE_OK) return rc;
  if ((rc = launch_status(moe::launch_stream_plan(a, w, (int)C, (int)R, s), "stream plan")) != MOE_OK) return rc;
  // The GEMMs read routed weights from the slots, indexed by slot.
  a.gate_up_w = (const bf16_t*)slot_gu;
  a.down_w = (const bf16_t*)slot_dn;
  for (int64_t r = 0; r < R; ++r) {
    if ((rc = launch_status(moe::launch_stream_copy(a, host_gu, host_dn, slot_gu, slot_dn, w, (int)C, (int)r, s),
                            "stream copy")) != MOE_OK)
      return rc;
    if ((rc = launch_status(moe::launch_gate_up(a, (const bf16_t*)x, t, w, cus, s, w.st_win_gu + 4 * r, w.st_slot),
                            "gate_up")) != MOE_OK)
      return rc;
    if ((rc = launch_status(moe::launch_down(a, t, w, cus, s, w.st_win_dn + 4 * r, w.st_slot), "down")) != MOE_OK)
      return rc;
  }
  return launch_status(moe::launch_combine(a, t, w, (bf16_t*)out, s), "combine");
}

size_t moe_workspace_control_bytes(void) { return kControlRegionBytes; }

}  // extern "C"

// ---- moe_forward without a caller workspace ----
// Scratch of the no-allocation entry point: one array per device (each GPU the
// library runs on holds its own copy until the process ends).  Host code uses
// only the device address hipGetSymbolAddress gives for the current device,
// never the array's name.
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void scratch_clear_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[64];

// The scratch's device address on the current device, set up on the first
// call made on that device: its control block is zero-filled once by a kernel
// on `s` (the fused path's words must start holding no call's tag; nothing
// else in it needs clearing, every call writes what it later reads).
int scratch_for_device(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "device index %d out of range", dev);
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&] {
    void* p = nullptr;
    sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (sl.err == hipSuccess && p) {
      hipLaunchKernelGGL(scratch_clear_kernel, dim3(64), dim3(256), 0, s, (uint32_t*)p, kControlRegionBytes / 4);
      sl.err = hipGetLastError();
    }
    if (sl.err == hipSuccess) sl.ptr = p;
  });
  if (sl.err != hipSuccess || !sl.ptr)
    return fail(MOE_ERR_LAUNCH, "static scratch on device %d: %s", dev, hipGetErrorString(sl.err));
  *out = sl.ptr;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_layer_t* L, const void* x, int64_t T, void* out, void* stream) {
  int rc = check_dims(L, T);
  if (rc != MOE_OK) return rc;
  if ((rc = check_weights(L)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x) return fail(MOE_ERR_NULL, "x is NULL");
  if (!out) return fail(MOE_ERR_NULL, "out is NULL");
  if (!aligned16(x)) return fail(MOE_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned16(out)) return fail(MOE_ERR_ALIGN, "out is not 16-byte aligned");
  const size_t need = workspace_need(L, T);
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "T = %lld needs %zu bytes of scratch; the static scratch holds %zu",
                (long long)T, need, kScratchBytes);
  int cus = 0;
  if ((rc = device_check(&cus)) != MOE_OK) return rc;
  void* ws = nullptr;
  if ((rc = scratch_for_device((hipStream_t)stream, &ws)) != MOE_OK) return rc;
  return forward_impl(L, x, T, out, ws, kScratchBytes, stream, nullptr, nullptr, 0.f);
}

int moe_workspace_status(const void* ws, size_t ws_bytes, void* stream, uint32_t* timed_out_calls) {
  if (!ws) return fail(MOE_ERR_NULL, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < kControlRegionBytes)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, fewer than its %zu-byte control region", ws_bytes,
                kControlRegionBytes);
  uint32_t w[3] = {0u, 0u, 0u};
  hipStream_t s = (hipStream_t)stream;
  int rc = launch_status(hipMemcpyAsync(w, ws, sizeof w, hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
  if (rc != MOE_OK) return rc;
  if ((rc = launch_status(hipStreamSynchronize(s), "hipStreamSynchronize")) != MOE_OK) return rc;
  static_assert(moe::kCtlError == 0 && moe::kCtlLast == 1 && moe::kCtlTimeouts == 2, "status words");
  if (timed_out_calls) *timed_out_calls = w[2];
  if (w[1] != 0u && w[0] == w[1])
    return fail(MOE_ERR_TIMEOUT, "a cross-workgroup wait of the latest call on this workspace timed out; "
                                 "its outputs are invalid");
  return MOE_OK;
}

int64_t moe_set_wait_budget_us(int64_t us) {
  const unsigned long long prev = g_wait_ticks.load();
  if (us < 0 || us > 60000000) return -1;
  g_wait_ticks.store((unsigned long long)us * 100ull);
  return (int64_t)(prev / 100ull);
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "unsupported or invalid dimensions";
    case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_DEVICE: return "current device is not a gfx950";
    case MOE_ERR_LAUNCH: return "a HIP call failed";
    case MOE_ERR_MEMORY: return "memory of the wrong kind or extent";
    case MOE_ERR_TIMEOUT: return "a wait inside the fused kernel timed out; that call's outputs are invalid";
    default: return "unknown status code";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

// Grouped expert GEMMs on gfx950 MFMA (v_mfma_f32_16x16x32_bf16), one group
// per routed expert plus one for the shared expert (group E, all T tokens).
//
//  gate_up:  for the rows of group g (gathered x rows of its tokens)
//            G = A Wg^T, U = A Wu^T,  h = SiLU(G) * U  -> bf16
//  down:     Y = h Wd^T -> bf16 per row (routing weights and the shared gate
//            are applied when the rows are combined)
//
// Definition: "Qwen3.6-35B-A3B — Architecture Overview", section "MoE FFN: 256
// Experts" (expert_e(x) = SiLU(x W_gate_e) * (x W_up_e) W_down_e, gate and up
// merged as [256, 1024, 2048]; shared expert of the same form, scaled by
// sigmoid(Linear(x, 1))); Linnet model page, Blocks: SparseMoe
// (gate_up_proj [E, 2I, H], down_proj [E, H, I]) and SwiGlu.
//
// One workgroup per tile of 160 rows x 128 weight rows (160 rows hold a
// typical expert of a 4096-token batch, about 128 +- 11 rows, in one tile, so
// its weights stream once); two workgroups share a CU, so one's start-up
// overlaps the other's streaming.  Batches of a few rows per expert use
// 32-row tiles, four workgroups per CU; batches of many (two 160-row tiles
// per expert on average) run gate_up in 192 x 256 tiles of eight waves, one
// persistent workgroup per CU that claims its XCD's tiles in turn (the down
// projection keeps 160 x 128, one workgroup per tile).  Wave w owns weight
// rows 32w .. 32w + 31 of the tile as two 16-column MFMA blocks: for gate_up
// the gate rows and the up rows of the same 16 inner rows (SiLU(g) * u is
// formed in registers, both blocks having the same layout), for down 32 output
// columns.  Each wave covers all rows of the tile.
//
// k advances in steps of 64 through a four-deep ring, three steps in flight:
// the weight fragments of a wave are needed by that wave alone and go straight
// into registers in MFMA operand layout; the activation tile (gathered x rows
// or h rows) is shared by the tile's waves and goes to LDS by the direct-to-LDS
// loads (global_load_lds_dwordx4).  Within a k-step, lane quarter q (lane / 16)
// covers k 16q .. 16q + 15, eight per MFMA k-step; activations and weights
// use the same order, so the products are unchanged and each lane reads 32
// contiguous bytes of a weight row per step.  The LDS operands of a step are
// read in groups, each group's reads issued before the MFMAs of the group
// ahead of it.
//
// LDS rows of the activation tile are 128 bytes; the 16-byte chunk c of row r
// is stored at chunk c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1).  A
// ds_read_b128 of an MFMA operand reads rows 0 .. 15 of a block, one chunk
// column each: with 64 four-byte banks two consecutive rows share the bank
// space, and the term from bit 3 gives rows r and r + 8 different chunks (a
// plain r & 7 serves them from the same banks: MI355X counted bank conflicts
// on half of the GEMM's LDS cycles).  LDS is read with inline ds_read_b128 and the
// load counter waited for explicitly: the compiler would otherwise drain every
// outstanding direct-to-LDS load before any LDS access.  For the same reason
// every load in the loop is issued unconditionally, so the counts the
// explicit waits rely on are exact (rows past a group repeat its last row,
// k-steps past the contraction read zeros through the weight resource).
//
// Scheduling: workgroups are handed to the eight XCDs round-robin (workgroup i
// on XCD i % 8); the tile list is cut into eight contiguous ranges and XCD x
// takes range x in order, or for large batches dealt to the XCDs in units
// (see the kernel).  Within a group, tiles come in blocks of row tiles,
// column tile major inside a block (gemm_tile_order; eight row tiles per
// block, one for the 160- and 32-row gate_up tiles): a block's row tiles of
// one weight slab, and its column tiles of one activation block, run side by
// side in one XCD and share them through its L2.
#include "kernels.hpp"
#include "lds_pipe.hpp"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace moe {

namespace {

using namespace pipe;

constexpr int BK = 64;
constexpr int NS = 4;            // ring depth (activation LDS stages = weight register slots)
// Shape of a tile of BM rows and NW waves, each wave owning 32 weight rows
// (160 x 128 with four waves; 32 x 128 for small batches; 192 x 256 with
// eight waves for large ones).
template <int BM, int NW>
struct TileShape {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kBN = 32 * NW;                // weight rows per tile
  static constexpr int kATile = BM * BK * 2;        // activation stage: 20 KB (160 rows), 4 KB (32), 24 KB (192)
  static constexpr int kMBlocks = BM / 16;          // 16-row MFMA blocks
  static constexpr int kGroup = kMBlocks <= 6 ? kMBlocks : kMBlocks / 2;   // blocks read from LDS together
  static constexpr int kADma = BM * 8 / kThreads;   // direct-to-LDS instructions per wave per step (16-byte units / threads)
  static constexpr int kVmPerStep = kADma + 4;      // per wave: activation loads + 4 weight loads
  static constexpr int kPerCU = NW == 8 ? 1 : (BM > 64 ? 2 : 4);   // workgroups per CU (LDS: NS stages each)
  static constexpr int kLds = NS * kATile > NW * BM * 64 ? NS * kATile : NW * BM * 64;   // ring, or the epilogue tiles
  static_assert((BM * 8) % kThreads == 0 && (kMBlocks == kGroup || kMBlocks == 2 * kGroup),
                "rows are read in one or two groups of blocks");
};

constexpr int kNonTemporal = 2;   // buffer-load cache policy bit: non-temporal (streamed once)

// WAUX: cache policy of the weight loads (0, or kNonTemporal for batches so
// small that each weight fragment feeds one tile of a few rows).  BM: rows
// per tile; NW: waves (4, or 8 for the 192 x 256 tiles of large batches,
// which read 56 KB per k-step for 192 x 256 outputs where two 160 x 128
// workgroups read 72 KB for 2 x 160 x 128).
template <bool GATE_UP, int WAUX, int BM, int NW, bool PERSIST = false>
__global__ __launch_bounds__((TileShape<BM, NW>::kThreads), (TileShape<BM, NW>::kPerCU)) void grouped_gemm_kernel(LayerArgs L, const bf16_t* __restrict__ x, int T,
                                                             Work w, const int* __restrict__ prefix,
                                                             const int4* __restrict__ tdesc,
                                                             const int* __restrict__ slot_tok,
                                                             const int* __restrict__ window,
                                                             const int* __restrict__ slot_map, int unit,
                                                             int tile_bound) {
  using S = TileShape<BM, NW>;
  constexpr int kATile = S::kATile, kMBlocks = S::kMBlocks, kGroup = S::kGroup, kADma = S::kADma;
  constexpr int kVmPerStep = S::kVmPerStep, BN = S::kBN;
  __shared__ __attribute__((aligned(1024))) char lds[S::kLds];

  const int E = L.E, K = L.K, H = L.H;
  // Tile of this workgroup: XCD x = blockIdx % 8 takes the x-th contiguous
  // eighth of the tile list, in order.  With a window (streamed experts) the
  // list is two ranges of the dispatch list: {first, count} of one round's
  // routed tiles, then {first, count} of shared tiles.
  int ntiles, lo0 = 0, n0, lo1 = 0;
  if (window) {
    lo0 = uni(window[0]);
    n0 = uni(window[1]);
    lo1 = uni(window[2]);
    ntiles = n0 + uni(window[3]);
  } else {
    // Clamped to the tile bound, as every table field below is clamped to
    // its range: when a fused route's bounded wait gives up (the call then
    // reports MOE_ERR_TIMEOUT), its workgroups may have written tables from
    // different views of the selections; results are wrong, but no access
    // leaves its array.  With consistent tables the clamps change nothing.
    ntiles = min(max(uni(prefix[E + 1]), 0), tile_bound);   // tile_bound: gemm_tile_bound of this GEMM
    n0 = ntiles;
  }
  // unit == 0: XCD x takes the x-th contiguous eighth of the tile list, in
  // order.  Otherwise units of `unit` consecutive tiles (the workgroups one
  // XCD holds at once) are dealt to the XCDs in turn, unit u to XCD u % 8, for as many
  // whole rounds of eight units as the list holds; the rest is cut into eight
  // equal parts, one per XCD.  Workgroup j of XCD x (blockIdx = 8 j + x) takes
  // tile j % unit of unit (j / unit) * 8 + x in the whole rounds, so an XCD
  // works through its units in order with each unit's tiles side by side, and
  // every XCD gets a share of hot and cold groups alike and the same number
  // of tiles, +-1 (with eight contiguous ranges, the range holding the hot
  // experts' or the shared group's tiles ran on alone at the end: MI355X,
  // Zipf(1.1) loads over 16384 tokens, one XCD for the last ~50 us of
  // gate_up).  The grid holds at least one round more than the whole rounds,
  // so every tile has its workgroup.
  //
  // PERSIST: one workgroup per CU instead, each taking the tiles its XCD would
  // have run, in the same order, through a per-XCD counter (j = the number of
  // tiles that XCD's workgroups took before); the next claim is requested
  // during each tile.  With one eight-wave workgroup per CU a new
  // workgroup started ~2.2 us after the last one ended, plus ~0.8 us for the
  // tile count and descriptor (MI355X, Zipf(1.1) over 16384 tokens, ~14 tiles
  // per CU).
  const int j8 = blockIdx.x >> 3, xcd = (int)(blockIdx.x & 7);
  const int rounds = unit ? ntiles / (8 * unit) : 0, full = rounds * unit;
  auto tile_of = [&](int j, int& t) -> bool {
    if (!unit) {
      const int chunk = (ntiles + 7) >> 3;
      if (j >= chunk) return false;
      t = xcd * chunk + j;
    } else if (j < full) {
      t = ((j / unit) * 8 + xcd) * unit + j % unit;
    } else {
      const int rest = ntiles - 8 * full, part = (rest + 7) >> 3, jj = j - full;
      if (jj >= part) return false;
      t = 8 * full + xcd * part + jj;
    }
    return t < ntiles;
  };
  // Each counter sits on a 128-byte line of its own and is used by one XCD's
  // workgroups.  The claim is an atomic add with return of device scope (no
  // sc1 bit, as the compiler emits its own agent-scope atomics on gfx950), so
  // a count is right whichever XCD a workgroup runs on.  Every lane issues
  // it; only thread 0's offset lies inside the 4-byte resource, so the count
  // rises by one per tile and no branch holds the result (a divergent one
  // made the compiler wait for the atomic at once).
  __shared__ int s_claim;
  const rsrc_t claim_rs = make_rsrc(w.claims + 32 * (8 * (GATE_UP ? 0 : 1) + xcd), 4u);
  const int claim_off = threadIdx.x == 0 ? 0 : 4;
  auto claim = [&]() { return __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, claim_rs, claim_off, 0, 0); };
  int next_claim = 0;   // thread 0: the claim requested during the current tile

  auto body = [&](const int t) {
  // (PERSIST runs without a window or slot map.)
  const int4 d = PERSIST ? tdesc[t] : tdesc[t < n0 ? lo0 + t : lo1 + (t - n0)];
  const int g = min(max(uni(d.x), 0), E);
  const bool shared = g == E;
  const int nrows = min(max(uni(d.z), 1), shared ? T : T * K);
  const int seg0 = shared ? 0 : min(max(uni(d.y), 0), T * K - nrows);
  const int m0 = min(uni(d.w & 0xFFFF), (nrows - 1) / BM) * BM;
  const int nt = min(max(uni(d.w >> 16), 0),
                     (GATE_UP ? (2 * (shared ? L.Is : L.I) + BN - 1) / BN : H / BN) - 1);
  // Weight block of the group: its expert index, or its cache slot.
  const int gw = (!PERSIST && slot_map && !shared) ? uni(slot_map[g]) : g;
  const int kdim = GATE_UP ? H : (shared ? L.Is : L.I);
  const int inner_n = shared ? L.Is : L.I;           // gate_up: inner rows of the group
  const int nreal = kdim / BK;                       // real k-steps
  const int nsteps = ((nreal + NS - 1) / NS) * NS;   // padded to the ring depth (padding: zero weights)
  const int rows_here = min(BM, nrows - m0);         // rows of this tile inside the group (>= 1)

  // The thread index is made opaque once per tile so that the persistent
  // loop recomputes the lane-dependent offsets below instead of holding them
  // across tiles (where they were spilled).
  int tid_ = (int)threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid_));
  const int tid = tid_;
  const int wave = tid >> 6, lane = tid & 63;
  const int wv = uni(wave);
  const int l16 = lane & 15, q = lane >> 4;
  const uint32_t lds_base = (uint32_t)(size_t)(lds_ptr_t)lds;

  // ---- activation sources: direct-to-LDS instruction j (0..kADma-1) of
  // wave w writes 16-byte unit p = 64 (NW j + w) + lane, i.e. row
  // r = 8 (NW j + w) + lane / 8, stored chunk lane % 8, holding the global
  // chunk (lane % 8) ^ swz(r).
  const bf16_t* a_src[kADma];
#pragma unroll
  for (int j = 0; j < kADma; ++j) {
    const int r = 8 * (NW * j + wv) + (lane >> 3);
    const int gch = ((lane & 7) ^ lds_swizzle(r)) * 8;
    const int row = m0 + min(r, rows_here - 1);         // rows past the group repeat its last row
    if (GATE_UP) {
      const int tok = shared ? row : min(max(slot_tok[seg0 + row], 0), T - 1);
      a_src[j] = x + (size_t)tok * H + gch;
    } else {
      a_src[j] = shared ? w.h_sh + (size_t)row * L.Is + gch : w.h + (size_t)(seg0 + row) * L.I + gch;
    }
  }
  // ---- weight sources: block b (0, 1) of wave w is weight row (of the tile)
  // 32 w + 16 b + lane % 16; lane quarter q reads elements 16q .. 16q + 15 of
  // each k-step (two 16-byte loads), through a buffer resource.
  rsrc_t b_rs[2];
  uint32_t b_off[2];
  // Byte steps between k-steps and between the two halves of a k-step: row
  // major, or the MFMA-tile layout of routed experts (16-row block, k-step,
  // half, lane: one contiguous 1 KB per load instruction).
  const bool tiled = L.tiled && !shared;
  const uint32_t k_stride = tiled ? 2048u : 2u * BK, h_stride = tiled ? 1024u : 16u;
  if (tiled) {
    const int nk = kdim / BK;
    if (GATE_UP) {
      b_rs[0] = b_rs[1] = make_rsrc(L.gate_up_w + (size_t)gw * 2 * L.I * H, (uint32_t)(2 * L.I * H * 2));
      b_off[0] = 2048u * (uint32_t)((nt * NW + wv) * nk) + 16u * lane;
      b_off[1] = 2048u * (uint32_t)((L.I / 16 + nt * NW + wv) * nk) + 16u * lane;
    } else {
      b_rs[0] = b_rs[1] = make_rsrc(L.down_w + (size_t)gw * H * L.I, (uint32_t)(H * kdim * 2));
#pragma unroll
      for (int b = 0; b < 2; ++b) b_off[b] = 2048u * (uint32_t)((nt * 2 * NW + 2 * wv + b) * nk) + 16u * lane;
    }
  } else if (GATE_UP) {
    const int inner = min(nt * 16 * NW + 16 * wv + l16, inner_n - 1);   // past the inner size: repeated, dropped
    if (shared) {
      b_rs[0] = make_rsrc(L.sh_gate_w, (uint32_t)(L.Is * H * 2));
      b_rs[1] = make_rsrc(L.sh_up_w, (uint32_t)(L.Is * H * 2));
      b_off[0] = b_off[1] = 2u * (uint32_t)(inner * H + 16 * q);
    } else {
      b_rs[0] = b_rs[1] = make_rsrc(L.gate_up_w + (size_t)gw * 2 * L.I * H, (uint32_t)(2 * L.I * H * 2));
      b_off[0] = 2u * (uint32_t)(inner * H + 16 * q);
      b_off[1] = 2u * (uint32_t)((L.I + inner) * H + 16 * q);
    }
  } else {
    const bf16_t* base = shared ? L.sh_down_w : L.down_w + (size_t)gw * H * L.I;
    b_rs[0] = b_rs[1] = make_rsrc(base, (uint32_t)(H * kdim * 2));
#pragma unroll
    for (int b = 0; b < 2; ++b) b_off[b] = 2u * (uint32_t)((nt * BN + 32 * wv + 16 * b + l16) * kdim + 16 * q);
  }

  u32x4 wb[NS][2][2];     // weight fragments: [slot][block][k-step of 32]
  auto issue = [&](u32x4 (&wbs)[2][2], int st, int ks) {
    char* sbase = lds + st * kATile;
    const int kv = min(ks, nreal - 1);          // padding steps re-read the last real step
#pragma unroll
    for (int j = 0; j < kADma; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[j] + kv * BK), (lds_ptr_t)(sbase + 1024 * (NW * j + wv)),
                                       16, 0, 0);
    const bool real = ks < nreal;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wbs[b][h] = __builtin_amdgcn_raw_buffer_load_b128(
            b_rs[b], real ? b_off[b] + k_stride * (uint32_t)ks + h_stride * h : kOutside, 0, WAUX);
  };

  f32x4 acc[kMBlocks][2];
#pragma unroll
  for (int i = 0; i < kMBlocks; ++i)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int mblocks = (rows_here + 15) >> 4;    // 16-row blocks holding rows of the group

  issue(wb[0], 0, 0);
  issue(wb[1], 1, 1);
  issue(wb[2], 2, 2);
  // The next claim, behind the first three steps' loads: a wait for the token
  // indices above would otherwise wait for the atomic too (the counter
  // retires loads in order); by step 2 it has returned.
  if constexpr (PERSIST) next_claim = claim();
  // One k-step.  YOUNGER: loads of later steps already issued when this one
  // starts (two, except in the last two steps), kVmPerStep per step and wave;
  // ISSUE: whether this step requests step ks + 3.  Both are compile-time
  // constants so that the compiler's own wait insertion sees straight-line
  // counts (with a run-time condition it adds a wait for zero outstanding
  // loads before the first use of a weight register in every iteration).
  auto step = [&](auto younger_c, auto issue_c, u32x4 (&wcur)[2][2], u32x4 (&wnext)[2][2], int st, int ks) {
    constexpr int YOUNGER = decltype(younger_c)::value;
    wait_vm<YOUNGER * kVmPerStep>();   // this step's loads have landed
    barrier();   // every wave's part of the stage is in LDS; the stage read last step is free
    // Step ks + 3 is requested here, or for eight-wave tiles ahead of the
    // last group's MFMAs (see below).
    constexpr bool kLateIssue = NW == 8;
    if constexpr (decltype(issue_c)::value && !kLateIssue) issue(wnext, (st + 3) % NS, ks + 3);
    const uint32_t sa0 = lds_base + st * kATile + l16 * 128 + (((2 * q) ^ lds_swizzle(l16)) << 4);
    const uint32_t sa1 = lds_base + st * kATile + l16 * 128 + (((2 * q + 1) ^ lds_swizzle(l16)) << 4);
    using seq = std::make_integer_sequence<int, kGroup>;
    auto mma = [&](int i0, int h, u32x4 (&av)[kGroup]) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        acc[i0 + i][0] = mfma16(av[i], wcur[0][h], acc[i0 + i][0]);
        acc[i0 + i][1] = mfma16(av[i], wcur[1][h], acc[i0 + i][1]);
      }
    };
    // The operand groups of the step (k half 0, then 1; with two groups of
    // 16-row blocks, rows of the first group, then the second) are read one
    // group ahead of their MFMAs, so that the two waves of a SIMD, which
    // leave the barrier together, do not wait for LDS at the same time.  The
    // second group's MFMAs are skipped when the tile's rows end before it
    // (uniform branch); its reads are not.  Eight-wave tiles request step
    // ks + 3 ahead of the last group's MFMAs, not ahead of the first: a wave
    // whose load stalls on a full address queue then has MFMAs in flight, and
    // the loads still have two steps to land (MI355X, Zipf(1.1) over 16384
    // tokens, gate_up averaged over three repeats on one box: 622 us after
    // the first group, 614 after the second, 608 after the third, 630 at the
    // end of the step; ahead of the first group was 21 us slower than after
    // it).  The four-wave tiles measured 1-4 us slower with any late request.
    u32x4 X[kGroup], Y[kGroup];
    if constexpr (kMBlocks > kGroup) {
      lds_read_group<0>(X, sa0, seq{});
      lds_read_group<kGroup>(Y, sa0, seq{});
      wait_lds_keep<kGroup>(X);
      mma(0, 0, X);
      lds_read_group<0>(X, sa1, seq{});
      wait_lds_keep<kGroup>(Y);
      if (mblocks > kGroup) mma(kGroup, 0, Y);
      lds_read_group<kGroup>(Y, sa1, seq{});
      wait_lds_keep<kGroup>(X);
      mma(0, 1, X);
      if constexpr (decltype(issue_c)::value && kLateIssue) issue(wnext, (st + 3) % NS, ks + 3);
      wait_lds_keep<0>(Y);
      if (mblocks > kGroup) mma(kGroup, 1, Y);
    } else {
      lds_read_group<0>(X, sa0, seq{});
      lds_read_group<0>(Y, sa1, seq{});
      wait_lds_keep<kGroup>(X);
      mma(0, 0, X);
      if constexpr (decltype(issue_c)::value && kLateIssue) issue(wnext, (st + 3) % NS, ks + 3);
      wait_lds_keep<0>(Y);
      mma(0, 1, Y);
    }
  };
  static_assert(NS == 4, "the loop below is unrolled for four slots");
  using c0 = std::integral_constant<int, 0>;
  using c1 = std::integral_constant<int, 1>;
  using c2 = std::integral_constant<int, 2>;
  using yes = std::true_type;
  using no = std::false_type;
  int k4 = 0;
  for (; k4 + NS < nsteps; k4 += NS) {
    step(c2{}, yes{}, wb[0], wb[3], 0, k4);
    step(c2{}, yes{}, wb[1], wb[0], 1, k4 + 1);
    step(c2{}, yes{}, wb[2], wb[1], 2, k4 + 2);
    step(c2{}, yes{}, wb[3], wb[2], 3, k4 + 3);
  }
  // The last four steps (nsteps is a multiple of four): only the first
  // requests a later step.
  step(c2{}, yes{}, wb[0], wb[3], 0, k4);
  step(c2{}, no{}, wb[1], wb[0], 1, k4 + 1);
  step(c1{}, no{}, wb[2], wb[1], 2, k4 + 2);
  step(c0{}, no{}, wb[3], wb[2], 3, k4 + 3);

  // ---- epilogue: D[4 (lane / 16) + i][lane % 16] of each 16 x 16 block ----
  // All loads have landed (the last step waited for zero outstanding); every
  // wave has passed the last step's barrier only after the others finished
  // reading the stage before it, so a barrier here frees the whole LDS.
  // Each wave writes its part as bf16 into its own LDS tile (row-major), then
  // stores 16-byte row chunks; rows past the group fall outside the store
  // resource and are dropped.
  barrier();
  bf16_t* ep = reinterpret_cast<bf16_t*>(lds + wv * (BM * 32 * 2));    // BM rows x 32 columns per wave
  static_assert(NW * BM * 32 * 2 <= S::kLds, "the epilogue tiles fit in LDS");
  constexpr int kCols = GATE_UP ? 16 : 32;
#pragma unroll
  for (int i = 0; i < kMBlocks; ++i)
#pragma unroll
    for (int b = 0; b < (GATE_UP ? 1 : 2); ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = GATE_UP ? siluf_(acc[i][0][r]) * acc[i][1][r] : acc[i][b][r];
        ep[(16 * i + 4 * q + r) * kCols + 16 * b + l16] = (bf16_t)f32_to_bf16(v);
      }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  bf16_t* obase;
  uint32_t ostride, ocol;
  bool wave_ok = true;
  if (GATE_UP) {
    ocol = nt * 16 * NW + 16 * wv;
    wave_ok = (int)ocol < inner_n;
    ostride = inner_n * 2;
    obase = (shared ? w.h_sh : w.h) + (size_t)(seg0 + m0) * inner_n;
  } else {
    ocol = nt * BN + 32 * wv;
    ostride = H * 2;
    obase = w.y + ((shared ? (size_t)T * K : (size_t)seg0) + m0) * H;
  }
  const rsrc_t ors = make_rsrc(obase, wave_ok ? (uint32_t)rows_here * ostride : 0u);
  constexpr int kChunks = kCols / 8;                 // 16-byte chunks per row
#pragma unroll
  for (int c0 = 0; c0 < BM * kChunks; c0 += 64) {
    const int c = c0 + lane, row = c / kChunks, cc = c % kChunks;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ep + row * kCols + 8 * cc);
    __builtin_amdgcn_raw_buffer_store_b128(v, ors, (uint32_t)row * ostride + 2u * ocol + 16u * cc, 0, 0);
  }
  };

  if constexpr (!PERSIST) {
    int t;
    if (!tile_of(j8, t)) return;
    body(t);
  } else {
    // Every wave has read s_claim before it passes the first barrier of the
    // tile, and thread 0 rewrites it only after the tile's last one.  The
    // barrier after the rewrite also keeps the next tile's loads into the
    // ring off the epilogue tiles until every wave has stored its part.
    // (lgkmcnt(0): thread 0's LDS write has completed before the barrier.)
    const int first = claim();
    if (threadIdx.x == 0) s_claim = first;
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier();
    int t;
    for (int j = uni(s_claim); tile_of(j, t);) {
      body(t);
      if (threadIdx.x == 0) s_claim = next_claim;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      barrier();
      j = uni(s_claim);
    }
  }
}

// out[t] = bf16( sum_k w[t, k] y[slot_of(t, k)] + gate[t] y[T*K + t] ), k in
// order, fp32 sum.  The K + 1 row indices and scales are requested first,
// then all K + 1 rows, so the loads overlap instead of forming a chain.
constexpr int kMaxK = 8;
template <int NT>
__global__ __launch_bounds__(NT) void combine_kernel(int T, int H, int K, Work w, bf16_t* __restrict__ out,
                                                      const bf16_t* __restrict__ residual) {
  const int per_tok = H >> 3;
  const size_t idx = (size_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= (size_t)T * per_tok) return;
  const int t = (int)(idx / per_tok), c = (int)(idx % per_tok) * 8;
  size_t row[kMaxK + 1];
  float sc[kMaxK + 1];
#pragma unroll
  for (int k = 0; k <= kMaxK; ++k) {
    if (k < K) {
      row[k] = (size_t)min(max(w.slot_of[(size_t)t * K + k], 0), T * K - 1);   // (clamped: see the GEMMs)
      sc[k] = w.topk_w[(size_t)t * K + k];
    } else {
      row[k] = (size_t)T * K + t;
      sc[k] = k == K ? w.gate_s[t] : 0.f;
    }
  }
  // y rows are read once and out is written once: non-temporal accesses keep
  // them from displacing other data in the caches (zipf16384: 137 -> 109 us).
  u32x4 v[kMaxK + 1];
#pragma unroll
  for (int k = 0; k <= kMaxK; ++k)
    if (k <= K) v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w.y + row[k] * H + c));
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
  for (int k = 0; k <= kMaxK; ++k) {
    if (k <= K) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += sc[k] * bf16_to_f32(v[k][j] & 0xFFFFu);
        acc[2 * j + 1] += sc[k] * bf16_to_f32(v[k][j] >> 16);
      }
    }
  }
  if (residual) {
    // The sub-block's residual add, after the sum: one rounding to bf16.
    const u32x4 r = ld16(residual + (size_t)t * H + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = bf16_to_f32(r[j] & 0xFFFFu) + acc[2 * j];
      acc[2 * j + 1] = bf16_to_f32(r[j] >> 16) + acc[2 * j + 1];
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + (size_t)t * H + c));
}

// Tiles an XCD holds at once (workgroups per CU times its CUs), and the
// grid: the whole rounds of eight units below the tile bound and one more
// (unit 0, contiguous ranges: the bound rounded up to a multiple of eight).
int gemm_unit(int per_cu, int num_cus) { return std::max(1, per_cu * (num_cus > 0 ? num_cus : 256) / 8); }
unsigned gemm_grid(int64_t bound, int unit) {
  if (!unit) return (unsigned)(8 * ((bound + 7) / 8));
  const int64_t r = 8 * (int64_t)unit;
  return (unsigned)(r * (bound / r + 1));
}
// Units dealt in turn for batches of at least two 160-row tiles per expert
// on average (gemm_wide), where expert loads may be skewed enough for
// contiguous ranges to end unevenly (MI355X, Zipf(1.1) over 16384 tokens:
// gate_up 713 -> 660 us); contiguous ranges below (4096 tokens, 128 rows per
// expert, measured 437 us per layer with contiguous ranges against 443 us
// with units).
static bool gemm_units(const LayerArgs& L, int T) { return gemm_wide(T, L.K, L.E); }

}  // namespace

// Weight loads are non-temporal when a batch averages at most one 16-row
// block of slots per expert: each weight fragment then feeds a single nearly
// empty tile and is never read again (MI355X decode64: 270 -> 260 us).  With
// more rows per expert the same hint measured slower (prefill4096 +8 %,
// zipf16384 +19 %, where hot experts' weights are reused across row tiles).
static bool stream_weights(const LayerArgs& L, int T) { return (int64_t)T * L.K <= 16 * (int64_t)L.E; }

// Kernel of a batch: the tile shape by gemm_bm / gemm_bn (32 x 128 for the
// smallest batches, 192 x 256 with eight waves for the largest, else
// 160 x 128), weight cache policy by stream_weights.
template <bool GATE_UP>
static auto gemm_kernel_for(const LayerArgs& L, int T, bool persist) {
  if (gemm_small_rows(T, L.K, L.E)) return grouped_gemm_kernel<GATE_UP, kNonTemporal, kGemmBMSmall, 4>;
  if constexpr (GATE_UP) {
    if (gemm_wide(T, L.K, L.E))
      return persist ? grouped_gemm_kernel<true, 0, kGemmBMWide, 8, true> : grouped_gemm_kernel<true, 0, kGemmBMWide, 8>;
  }
  return stream_weights(L, T) ? grouped_gemm_kernel<GATE_UP, kNonTemporal, kGemmBM, 4>
                              : grouped_gemm_kernel<GATE_UP, 0, kGemmBM, 4>;
}
static_assert(TileShape<kGemmBMWide, 8>::kBN == kGemmBNWide && TileShape<kGemmBM, 4>::kBN == kGemmBNW &&
                  TileShape<kGemmBMSmall, 4>::kBN == kGemmBNW,
              "the dispatch's column tiles match the kernels'");

static int gemm_per_cu(const LayerArgs& L, int T, bool gate_up) {
  if (gemm_small_rows(T, L.K, L.E)) return TileShape<kGemmBMSmall, 4>::kPerCU;
  return gate_up && gemm_wide(T, L.K, L.E) ? TileShape<kGemmBMWide, 8>::kPerCU : TileShape<kGemmBM, 4>::kPerCU;
}
static int gemm_threads(const LayerArgs& L, int T, bool gate_up) { return gate_up && gemm_wide(T, L.K, L.E) ? 512 : 256; }

hipError_t launch_gate_up(const LayerArgs& L, const bf16_t* x, int T, const Work& w, int num_cus,
                          hipStream_t s, const int* window, const int* slot_map) {
  // The dispatch tables go in as separate read-only arguments: uniform reads of
  // them then compile to scalar loads.
  const int64_t bound = gemm_tile_bound(T, L.K, L.E, 2 * L.I, 2 * L.Is);
  const int unit = gemm_units(L, T) ? gemm_unit(gemm_per_cu(L, T, true), num_cus) : 0;
  // The large-batch tiles run persistent (one workgroup per CU claiming its
  // XCD's tiles), except over a window of the streamed path, whose rounds
  // would need their own counters.
  const bool persist = !window && !slot_map && gemm_wide(T, L.K, L.E);
  auto k = gemm_kernel_for<true>(L, T, persist);
  const unsigned grid = persist ? (unsigned)(8 * ((std::max(num_cus, 8) + 7) / 8)) : gemm_grid(bound, unit);
  hipLaunchKernelGGL(k, dim3(grid), dim3(gemm_threads(L, T, true)), 0, s, L, x, T, w, (const int*)w.tiles_gu,
                     (const int4*)w.tdesc_gu, (const int*)w.slot_tok, window, slot_map, unit, (int)bound);
  return hipGetLastError();
}

hipError_t launch_down(const LayerArgs& L, int T, const Work& w, int num_cus, hipStream_t s, const int* window,
                       const int* slot_map) {
  const int64_t bound = gemm_tile_bound(T, L.K, L.E, L.H, L.H);
  // Units in the ratio of a group's down tiles to its gate_up tiles (row and
  // column tiles of either shape) deal every group to about the XCD that ran
  // its gate_up tiles, whose L2 may still hold its h rows.
  int unit = 0;
  if (gemm_units(L, T)) {
    const int bmg = gemm_bm(T, L.K, L.E, true), bng = gemm_bn(T, L.K, L.E, true);
    const int bmd = gemm_bm(T, L.K, L.E, false), bnd = gemm_bn(T, L.K, L.E, false);
    const int64_t ngu = (2 * L.I + bng - 1) / bng, ndn = L.H / bnd;
    const int64_t ug = gemm_unit(gemm_per_cu(L, T, true), num_cus);
    unit = (int)std::max<int64_t>(1, ug * ndn * bmg / (ngu * bmd));
  }
  auto k = gemm_kernel_for<false>(L, T, false);
  hipLaunchKernelGGL(k, dim3(gemm_grid(bound, unit)), dim3(gemm_threads(L, T, false)), 0, s, L, (const bf16_t*)nullptr, T, w,
                     (const int*)w.tiles_dn, (const int4*)w.tdesc_dn, (const int*)w.slot_tok, window, slot_map, unit,
                     (int)bound);
  return hipGetLastError();
}

hipError_t launch_combine(const LayerArgs& L, int T, const Work& w, bf16_t* out, hipStream_t s,
                          const bf16_t* residual) {
  const size_t n = (size_t)T * (L.H / 8);
  // Under 256 workgroups of 256 threads, 64-thread workgroups spread the
  // rows over more CUs (decode64 combine 6.7 -> 6.3 us).
  if (n < 256 * 256) {
    hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, s, T, L.H, L.K, w, out,
                       residual);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(combine_kernel<256>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, L.H, L.K, w, out,
                     residual);
  return hipGetLastError();
}

}  // namespace moe

// Host-side internal interfaces of the BEAM library: workspace layout, the
// device plan record, and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/beam_moe.h"

namespace beam {

// Tokens per routing block (selection, block-local ranks, per-block counts).
constexpr int kSelBlock = 64;
// Largest E the selection and scan kernels handle.
constexpr int kMaxExperts = 1024;

// Written by the scan kernel, read by the expert kernels.  Tiles are listed
// routed first (expert-major, ascending expert id), then the shared tiles.
struct Plan {
  int32_t pairs;            // P = surviving (token, expert) pairs
  int32_t n_tiles_routed;   // tiles of routed experts
  int32_t n_tiles_shared;   // tiles of the fused shared expert
  int32_t active_experts;
  // work counters of the dynamically scheduled prefill gate/up and down
  // kernels (zeroed with the plan, taken with atomics by the kernels)
  int32_t gate_up_next;
  int32_t down_next;
};

// One tile of rows of a (virtual) expert: rows [row0, row0 + rows) of the
// compacted pair order (routed) or of the token order (shared, expert == E).
struct Tile {
  int32_t expert;
  int32_t row0;
  int32_t rows;
  int32_t pad;
};

// Expert-stationary prefill: tiles of this many token rows (12 blocks of 32)
// for layers with packed weights and no shared experts whose batches give an
// expert at least kEsMinPerExpert top-K candidates on average.
constexpr int kEsTileRows = 384;
constexpr int kEsMinPerExpert = 256;
// Packed layers with shared experts: from this many tokens the fused shared
// expert (every token) runs on the expert-stationary kernels, on tiles of
// kEsTileRows consecutive tokens, and the routed tiles on the 128-row ones
// (DeepSeek-V2-Lite prefill shapes on MI355X, us per step with / without:
// T = 1536 289 / 285, T = 2048 309 / 324, T = 4096 388 / 410).
constexpr int kEsSharedMinT = 2048;

struct WsLayout {
  size_t plan, logits, idx, gates, mask, counts, rank, block_counts, expert_off, tiles, perm_token,
      slot_pos, h, h_shared, o, o_shared, o_part, zsel, dz, lreg_tok, es_x, es_h, total;
  size_t o_part_bytes;   // 0 when the layer's down product never splits
  int32_t max_tiles;
};

// Number of k slices of the router logits (partial sums added by selection).
int router_ksplit(const beam_moe_layer& L, int32_t T);
// Rows of partial logits the workspace reserves (>= router_ksplit(L, T') * T'
// for every T' <= T; non-decreasing in T).
long router_logit_rows(const beam_moe_layer& L, int32_t T);
// Row-tile height of the expert kernels (multiple of 16).
int expert_tile_rows(const beam_moe_layer& L, int32_t T);
// True when the shared experts of a batch run on the expert-stationary
// kernels (see kEsSharedMinT); the routed down product then never splits k.
bool es_shared_experts(const beam_moe_layer& L, int32_t T);
WsLayout workspace_layout(const beam_moe_layer& L, int32_t T);

struct Ptrs {
  // routing
  float* logits;
  int32_t* idx;
  float* gates;
  uint32_t* mask;
  int32_t* counts;
  int32_t* rank;
  int32_t* block_counts;
  int32_t* expert_off;
  Plan* plan;
  Tile* tiles;
  int32_t* perm_token;
  int32_t* slot_pos;
  // experts
  void* h;
  void* h_shared;
  void* o;          // [P][D] expert outputs: fp32 for fp32 layers, bf16 otherwise
  void* o_shared;   // [T][D] shared-expert outputs, same type
  // k-split down products (prefill tiles): fp32 partial outputs
  // [kMaxDownSplit][T K][D], then the shared ones [kMaxDownSplit][T][D]
  float* o_part;
  // expert-stationary prefill: packed tokens and packed h of every tile
  // (routed tiles, or the shared experts' tiles of consecutive tokens)
  void* es_x;   // [tiles][12 x D/64 blocks of 32 x 64] bf16
  void* es_h;   // [tiles][12 x I/64 blocks] (shared: S Is / 64 blocks)
  // mask-router backward
  float* zsel;       // [T][K] mask logit of each candidate
  float* dz;         // [P] dL/dz of each pair (pair order)
  float* lreg_tok;   // [T] sum of m_hat over the token's candidates
};

// k split of the prefill down product: chosen on the device, identically by
// the down and combine kernels, from the plan's tile count.  A launch whose
// items (tiles x output blocks) leave the resident workgroups badly used --
// fewer items than workgroups, or a last round mostly empty -- idles CUs;
// splitting the k range s ways multiplies the items by s and divides their
// length by s.  s (1 to kMaxDownSplit) minimises ceil(items s / slots) / s,
// the time in units of one unsplit item, and is taken only when it saves at
// least a third of that time: the fp32 partials cost HBM traffic (written
// here, read by the combine), and the estimate takes every item to be as
// long as a full tile's.
constexpr int kMaxDownSplit = 4;
__host__ __device__ inline int down_split(long items, long slots) {
  if (slots <= 0 || items <= 0) return 1;
  const long cost1 = (items + slots - 1) / slots * 12;   // rounds x 12 / s, 12 = lcm(1..4)
  int best = 1;
  long best_cost = cost1;
  for (int s = 2; s <= kMaxDownSplit; ++s) {
    const long cost = (items * s + slots - 1) / slots * (12 / s);
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return 3 * best_cost <= 2 * cost1 ? best : 1;
}

// ---- launchers (return hipSuccess or the launch error) ----
hipError_t launch_router_logits(const beam_moe_layer& L, const void* x, int32_t T, const Ptrs& p,
                                hipStream_t s);
// True when the plan comes from per-expert token bitmaps in one workgroup
// (they and the batch's selections fit in its LDS); otherwise the scan and
// scatter kernels follow the selection.
bool select_builds_plan(const beam_moe_layer& L, int32_t T);
// all_pairs: every top-K candidate is kept (masks written as all ones, gates
// unmasked, no shared tiles in the plan) and each candidate's mask logit is
// written to p.zsel -- the routing of the mask-router backward.
hipError_t launch_select(const beam_moe_layer& L, int32_t T, int tile_rows, const Ptrs& p,
                         hipStream_t s, bool all_pairs = false);
hipError_t launch_scan(const beam_moe_layer& L, int32_t T, int tile_rows, const Ptrs& p,
                       hipStream_t s, bool all_pairs = false);
hipError_t launch_scatter(const beam_moe_layer& L, int32_t T, const Ptrs& p, hipStream_t s);
hipError_t launch_gate_up(const beam_moe_layer& L, const void* x, int32_t T, int tile_rows,
                          const WsLayout& w, const Ptrs& p, hipStream_t s);
// allow_split: the prefill down product may split k (fp32 partials in
// p.o_part, added by the combine); the mask-router backward reads O itself
// and passes false.
hipError_t launch_down(const beam_moe_layer& L, int32_t T, int tile_rows, const WsLayout& w,
                       const Ptrs& p, hipStream_t s, bool allow_split = false);
// Single-token batches of bf16 layers with intermediate sizes up to 2048
// (4096 with FP8 expert weights): the down product and the combine in one
// launch (y written directly).
bool down_combine_fused(const beam_moe_layer& L, int32_t T);
hipError_t launch_down_combine_t1(const beam_moe_layer& L, const Ptrs& p, void* y, hipStream_t s);
// Single-token batches whose down product takes that launch and whose d_model
// is at most 2048 (4096 with FP8 expert weights): gate/up and SwiGLU as
// matrix-vector products.
bool gate_up_t1(const beam_moe_layer& L, int32_t T);
hipError_t launch_gate_up_t1(const beam_moe_layer& L, const void* x, const Ptrs& p, hipStream_t s);
hipError_t launch_combine(const beam_moe_layer& L, int32_t T, int tile_rows, const Ptrs& p,
                          void* y, hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_mfma_loop(float* out, int blocks, int iters, hipStream_t s);
// Packed operand layout of `mats` bf16 matrices [rows][cols] (see the header).
hipError_t launch_pack_weights(const void* w, int mats, int rows, int cols, void* packed,
                               hipStream_t s);
// Mask-router backward from the all-pairs expert outputs O: per-pair dL/dz and
// per-token sums of m_hat, then dL/dWm, dL/db_m and L_reg.
hipError_t launch_mask_grad(const beam_moe_layer& L, const void* x, const void* dy, int32_t T,
                            float beta, float* dwm, float* dbm, float* lreg, const Ptrs& p,
                            hipStream_t s);

// Workgroups of `block` threads of `kernel` that fit on the device at once
// (occupancy x CUs), cached per device and kernel.
int resident_blocks(const void* kernel, int block);

// Profiler hooks around each launch (no-ops unless the profiler is on).
void prof_before(const char* name, hipStream_t s);
void prof_after(hipStream_t s);

}  // namespace beam

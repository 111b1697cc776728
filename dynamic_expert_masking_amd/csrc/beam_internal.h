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
};

// One tile of rows of a (virtual) expert: rows [row0, row0 + rows) of the
// compacted pair order (routed) or of the token order (shared, expert == E).
struct Tile {
  int32_t expert;
  int32_t row0;
  int32_t rows;
  int32_t pad;
};

struct WsLayout {
  size_t plan, logits, idx, gates, mask, counts, rank, block_counts, expert_off, tiles, perm_token,
      slot_pos, h, h_shared, o, o_shared, zsel, dz, lreg_tok, total;
  int32_t max_tiles;
};

// Number of k slices of the router logits (partial sums added by selection).
int router_ksplit(const beam_moe_layer& L, int32_t T);
// Row-tile height of the expert kernels (multiple of 16).
int expert_tile_rows(const beam_moe_layer& L, int32_t T);
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
  // mask-router backward
  float* zsel;       // [T][K] mask logit of each candidate
  float* dz;         // [P] dL/dz of each pair (pair order)
  float* lreg_tok;   // [T] sum of m_hat over the token's candidates
};

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
hipError_t launch_down(const beam_moe_layer& L, int32_t T, int tile_rows, const WsLayout& w,
                       const Ptrs& p, hipStream_t s);
hipError_t launch_combine(const beam_moe_layer& L, int32_t T, const Ptrs& p, void* y,
                          hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
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

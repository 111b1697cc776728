// C ABI of the BEAM masked-MoE layer: argument validation, workspace
// carving, launch sequence, work accounting and the launch profiler.
#include <string.h>

#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "beam_internal.h"

namespace beam {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int expert_tile_rows(const beam_moe_layer& L, int32_t T) {
  if (L.dtype == BEAM_F32) return 16;
  // Expected tokens per routed expert if every top-K candidate were kept.
  const long per_expert = (long(T) * L.K + L.E - 1) / L.E;
  // FP8 weights only have the streaming kernels (tiles of up to 64 rows)
  if (per_expert <= 96 || L.expert_format == BEAM_WEIGHTS_FP8_E4M3) {
    // Layers without shared experts size these tiles by the surviving pairs
    // expected from the layer's Avg-K (fine-grained layer, T = 512: 16-row
    // tiles for about 6 pairs per expert instead of 64-row ones, 126 -> 122
    // us per step on MI355X).  With shared experts, whose tiles span the
    // whole batch at the same height, smaller tiles re-read the shared
    // weights more often than they save (DeepSeek-V2-Lite T = 256: 236 ->
    // 254 us), so those keep the top-K estimate.
    long pe = per_expert;
    if (L.n_shared == 0 && L.expected_avg_k > 0.f)
      pe = long(std::ceil(double(T) * L.expected_avg_k / L.E));
    if (pe <= 16) return 16;
    if (pe <= 32) return 32;
    return 64;
  }
  // packed weights: the expert-stationary kernels (no shared experts, at
  // least kEsMinPerExpert candidates per expert), else tiles of 128 rows
  if (L.wp_gate && L.n_shared == 0 && L.D % 128 == 0) {
    // surviving pairs per expert expected from the layer's Avg-K (K if unknown)
    const float avg_k = L.expected_avg_k > 0.f ? L.expected_avg_k : float(L.K);
    if (double(T) * avg_k >= double(kEsMinPerExpert) * L.E) return kEsTileRows;
  }
  if (per_expert < 512 || L.wp_gate) return 128;
  return 256;
}

bool es_shared_experts(const beam_moe_layer& L, int32_t T) {
  return L.wsp_gate && L.n_shared > 0 && L.dtype == BEAM_BF16 && L.expert_format == BEAM_WEIGHTS_DTYPE &&
         T >= kEsSharedMinT && L.D % 128 == 0 && L.I_shared % 64 == 0 &&
         expert_tile_rows(L, T) == 128;
}

// Rows of router partial logits ([KS][T] of them) that the workspace holds
// for a batch of T tokens: an upper bound on KS(T') * T' over every T' <= T,
// so that a workspace sized for T_max serves every smaller batch (KS rises as
// T falls).  The router splits k at most 4 ways, and only while its grid of
// blocks x KS workgroups stays within 512 (from 256 tokens; below, while
// blocks x (KS - 1) < 256, which is the weaker bound).  With at least
// ceil(T / 64) token blocks that needs T <= 16384 for a 2-way split,
// T <= 10880 for 3 and T <= 8192 for 4.  A maximum of non-decreasing terms,
// so the bound (and the whole workspace size) is non-decreasing in T.
long router_logit_rows(const beam_moe_layer& L, int32_t T) {
  if (L.dtype == BEAM_F32) return T;
  const long t = T;
  return std::max({t, 2 * std::min<long>(t, 16384), 3 * std::min<long>(t, 10880),
                   4 * std::min<long>(t, 8192)});
}

WsLayout workspace_layout(const beam_moe_layer& L, int32_t T) {
  WsLayout w;
  const size_t TK = size_t(T) * L.K;
  const size_t elt = L.dtype == BEAM_F32 ? 4 : 2;
  const size_t nblk = (size_t(T) + kSelBlock - 1) / kSelBlock;
  const size_t IS = size_t(L.n_shared) * L.I_shared;
  // Smallest tile height is 16 rows: bound on the tile count (any height).
  w.max_tiles = int32_t((TK + 15) / 16 + std::min<size_t>(L.E, TK) + (size_t(T) + 15) / 16 + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  w.plan = take(sizeof(Plan));
  w.logits = take(size_t(router_logit_rows(L, T)) * 2 * L.E * 4);
  w.idx = take(TK * 4);
  w.gates = take(TK * 4);
  w.mask = take(size_t(T) * 4);
  w.counts = take(size_t(L.E) * 4);
  w.rank = take(TK * 4);
  w.block_counts = take(nblk * L.E * 4);
  w.expert_off = take(size_t(L.E + 1) * 4);
  w.tiles = take(size_t(w.max_tiles) * sizeof(Tile));
  w.perm_token = take((TK + 64) * 4);   // + 64: whole 16-row groups are read
  w.slot_pos = take(TK * 4);
  w.h = take(TK * L.I * elt);
  w.h_shared = take(size_t(T) * IS * elt);
  w.o = take(TK * L.D * elt);
  w.o_shared = take(IS ? size_t(T) * L.D * elt : 0);
  // fp32 partials of a k-split prefill down product (tiles over 64 rows,
  // bf16 weights): kMaxDownSplit x ([T K][D] + [T][D]).  The tile height, and
  // so this size, is non-decreasing in T.
  const bool split_down = L.dtype != BEAM_F32 && L.expert_format != BEAM_WEIGHTS_FP8_E4M3 &&
                          expert_tile_rows(L, T) > 64;
  w.o_part_bytes = split_down ? size_t(kMaxDownSplit) * (TK + (IS ? T : 0)) * L.D * 4 : 0;
  w.o_part = take(w.o_part_bytes);
  // expert-stationary prefill: packed tokens and h of every tile (routed
  // tiles without shared experts; the shared experts' tiles with them)
  const bool es = expert_tile_rows(L, T) == kEsTileRows;
  const size_t es_tiles = es ? size_t((TK + kEsTileRows - 1) / kEsTileRows + std::min<size_t>(L.E, TK)) : 0;
  const size_t ess_tiles = es_shared_experts(L, T) ? (size_t(T) + kEsTileRows - 1) / kEsTileRows : 0;
  w.es_x = take(std::max(es_tiles, ess_tiles) * kEsTileRows * L.D * 2);
  w.es_h = take(std::max(es_tiles * L.I, ess_tiles * IS) * kEsTileRows * 2);
  w.zsel = take(TK * 4);
  w.dz = take(TK * 4);
  w.lreg_tok = take(size_t(T) * 4);
  w.total = off;
  return w;
}

int resident_blocks(const void* kernel, int block) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(dev, kernel);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 1, cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int n = per_cu * cus;
  cache[key] = n;
  return n;
}

// ---------------------------------------------------------------------------
// Profiler
// ---------------------------------------------------------------------------

namespace {
struct ProfState {
  bool on = false;
  int max = 0;
  int n = 0;
  bool pending = false;
  std::vector<hipEvent_t> ev0, ev1;
  std::vector<const char*> names;
};
ProfState g_prof;
}  // namespace

void prof_before(const char* name, hipStream_t s) {
  g_prof.pending = false;
  if (!g_prof.on || g_prof.n >= g_prof.max) return;
  if (hipEventRecord(g_prof.ev0[g_prof.n], s) != hipSuccess) return;
  g_prof.names[g_prof.n] = name;
  g_prof.pending = true;
}

void prof_after(hipStream_t s) {
  if (!g_prof.pending) return;
  g_prof.pending = false;
  if (hipEventRecord(g_prof.ev1[g_prof.n], s) == hipSuccess) ++g_prof.n;
}

}  // namespace beam

using namespace beam;

// ---------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------

// Largest element count that 32-bit row offsets reach (x [T][D], one expert's
// weight matrix, the shared experts' stacked matrices).
constexpr long kMaxOffsetElems = 0x7FFFFFFFL;

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int check_layer(const beam_moe_layer* L) {
  if (!L) return BEAM_ERR_INVALID_ARG;
  if (L->dtype != BEAM_F32 && L->dtype != BEAM_BF16) return BEAM_ERR_INVALID_ARG;
  if (L->D <= 0 || L->E <= 0 || L->K <= 0 || L->I <= 0 || L->n_shared < 0)
    return BEAM_ERR_INVALID_ARG;
  if (L->K > L->E) return BEAM_ERR_INVALID_ARG;
  if (L->gating & ~(BEAM_GATE_SOFTMAX_ALL | BEAM_GATE_RENORM | BEAM_GATE_BINARY))
    return BEAM_ERR_INVALID_ARG;
  if ((L->gating & BEAM_GATE_BINARY) && (L->gating & BEAM_GATE_SOFTMAX_ALL))
    return BEAM_ERR_INVALID_ARG;
  if (L->segment_len < 0) return BEAM_ERR_INVALID_ARG;
  if (!(L->expected_avg_k >= 0.f && L->expected_avg_k <= float(L->K))) return BEAM_ERR_INVALID_ARG;
  if (L->n_shared > 0 && L->I_shared <= 0) return BEAM_ERR_INVALID_ARG;
  const void* req[] = {L->w_router, L->w_mask, L->w_gate, L->w_up, L->w_down};
  for (const void* p : req)
    if (!p || !aligned16(p)) return BEAM_ERR_INVALID_ARG;
  if (L->n_shared > 0) {
    const void* sh[] = {L->ws_gate, L->ws_up, L->ws_down};
    for (const void* p : sh)
      if (!p || !aligned16(p)) return BEAM_ERR_INVALID_ARG;
  }
  if ((L->b_router && (reinterpret_cast<uintptr_t>(L->b_router) & 3u)) ||
      (L->b_mask && (reinterpret_cast<uintptr_t>(L->b_mask) & 3u)))
    return BEAM_ERR_INVALID_ARG;
  if (L->K > 32 || L->E > kMaxExperts) return BEAM_ERR_UNSUPPORTED;
  if (L->D % 64 || L->I % 64 || L->D > 16384 || L->I > (1 << 20)) return BEAM_ERR_UNSUPPORTED;
  if (L->n_shared > 0 && (L->I_shared % 64 || long(L->n_shared) * L->I_shared > (1 << 20)))
    return BEAM_ERR_UNSUPPORTED;
  // The tiled kernels address weight rows with 32-bit element offsets.
  if (long(L->I) * L->D > kMaxOffsetElems ||
      long(L->n_shared) * L->I_shared * L->D > kMaxOffsetElems)
    return BEAM_ERR_UNSUPPORTED;
  if (L->expert_format != BEAM_WEIGHTS_DTYPE && L->expert_format != BEAM_WEIGHTS_FP8_E4M3)
    return BEAM_ERR_INVALID_ARG;
  // packed copies: all that the layer uses, or none (bf16 weights only)
  {
    const void* pk[] = {L->wp_gate, L->wp_up, L->wp_down};
    const void* pks[] = {L->wsp_gate, L->wsp_up, L->wsp_down};
    int given = 0, bad = 0;
    for (const void* q : pk) {
      given += q != nullptr;
      bad += q && !aligned16(q);
    }
    for (const void* q : pks) {
      given += q != nullptr;
      bad += q && !aligned16(q);
    }
    const int need = L->n_shared > 0 ? 6 : 3;
    if (given > 0) {
      if (bad || L->dtype != BEAM_BF16 || L->expert_format != BEAM_WEIGHTS_DTYPE) return BEAM_ERR_INVALID_ARG;
      if (!L->wp_gate || !L->wp_up || !L->wp_down) return BEAM_ERR_INVALID_ARG;
      if (L->n_shared > 0 && (!L->wsp_gate || !L->wsp_up || !L->wsp_down)) return BEAM_ERR_INVALID_ARG;
      if (given != need) return BEAM_ERR_INVALID_ARG;   // shared copies without shared experts
    }
  }
  if (L->expert_format == BEAM_WEIGHTS_FP8_E4M3) {
    const float* sc[] = {L->scale_gate, L->scale_up, L->scale_down};
    for (const float* p : sc)
      if (!p || !aligned16(p)) return BEAM_ERR_INVALID_ARG;
    if (L->n_shared > 0) {
      const float* ss[] = {L->scale_shared_gate, L->scale_shared_up, L->scale_shared_down};
      for (const float* p : ss)
        if (!p || !aligned16(p)) return BEAM_ERR_INVALID_ARG;
    }
    // E4M3 weights go with bf16 activations; weight rows stream in 128-byte chunks
    if (L->dtype != BEAM_BF16 || L->D % 128 || L->I % 128 ||
        (L->n_shared > 0 && L->I_shared % 128))
      return BEAM_ERR_UNSUPPORTED;
  }
  return BEAM_OK;
}

static int check_call(const beam_moe_layer* L, const void* x, int32_t T, void* ws, size_t ws_bytes,
                      WsLayout* lay) {
  int st = check_layer(L);
  if (st != BEAM_OK) return st;
  if (T < 0) return BEAM_ERR_INVALID_ARG;
  if (long(T) * L->K > (1L << 30) || long(T) * L->D > kMaxOffsetElems) return BEAM_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_OK;
  if (!x || !aligned16(x)) return BEAM_ERR_INVALID_ARG;
  *lay = workspace_layout(*L, T);
  if (!ws || !aligned16(ws) || ws_bytes < lay->total) return BEAM_ERR_WORKSPACE;
  return BEAM_OK;
}

static int check_route_out(const beam_route_out* out) {
  if (!out || !out->topk_idx || !out->gates || !out->mask || !out->expert_count)
    return BEAM_ERR_INVALID_ARG;
  const uintptr_t a = reinterpret_cast<uintptr_t>(out->topk_idx) |
                      reinterpret_cast<uintptr_t>(out->gates) |
                      reinterpret_cast<uintptr_t>(out->mask) |
                      reinterpret_cast<uintptr_t>(out->expert_count);
  return (a & 3u) ? BEAM_ERR_INVALID_ARG : BEAM_OK;
}

static Ptrs carve(const WsLayout& w, void* ws, const beam_route_out* out) {
  char* b = static_cast<char*>(ws);
  Ptrs p;
  p.logits = reinterpret_cast<float*>(b + w.logits);
  p.idx = out ? out->topk_idx : reinterpret_cast<int32_t*>(b + w.idx);
  p.gates = out ? out->gates : reinterpret_cast<float*>(b + w.gates);
  p.mask = out ? out->mask : reinterpret_cast<uint32_t*>(b + w.mask);
  p.counts = out ? out->expert_count : reinterpret_cast<int32_t*>(b + w.counts);
  p.rank = reinterpret_cast<int32_t*>(b + w.rank);
  p.block_counts = reinterpret_cast<int32_t*>(b + w.block_counts);
  p.expert_off = reinterpret_cast<int32_t*>(b + w.expert_off);
  p.plan = reinterpret_cast<Plan*>(b + w.plan);
  p.tiles = reinterpret_cast<Tile*>(b + w.tiles);
  p.perm_token = reinterpret_cast<int32_t*>(b + w.perm_token);
  p.slot_pos = reinterpret_cast<int32_t*>(b + w.slot_pos);
  p.h = b + w.h;
  p.h_shared = b + w.h_shared;
  p.o = b + w.o;
  p.o_shared = b + w.o_shared;
  p.o_part = w.o_part_bytes ? reinterpret_cast<float*>(b + w.o_part) : nullptr;
  p.es_x = b + w.es_x;
  p.es_h = b + w.es_h;
  p.zsel = reinterpret_cast<float*>(b + w.zsel);
  p.dz = reinterpret_cast<float*>(b + w.dz);
  p.lreg_tok = reinterpret_cast<float*>(b + w.lreg_tok);
  return p;
}

#define BEAM_TRY(expr)                         \
  do {                                         \
    if ((expr) != hipSuccess) return BEAM_ERR_HIP; \
  } while (0)

static int run_routing(const beam_moe_layer& L, const void* x, int32_t T, int tile_rows,
                       const Ptrs& p, hipStream_t s) {
  BEAM_TRY(launch_router_logits(L, x, T, p, s));
  BEAM_TRY(launch_select(L, T, tile_rows, p, s));
  if (!select_builds_plan(L, T)) BEAM_TRY(launch_scan(L, T, tile_rows, p, s));
  return BEAM_OK;
}

extern "C" {

size_t beam_moe_workspace_size(const beam_moe_layer* layer, int32_t T_max) {
  if (check_layer(layer) != BEAM_OK || T_max < 0) return 0;
  if (long(T_max) * layer->K > (1L << 30) || long(T_max) * layer->D > kMaxOffsetElems) return 0;
  return workspace_layout(*layer, T_max).total;
}

int beam_moe_route(const beam_moe_layer* layer, const void* x, int32_t T,
                   const beam_route_out* out, void* ws, size_t ws_bytes, void* stream) {
  WsLayout lay;
  int st = check_call(layer, x, T, ws, ws_bytes, &lay);
  if (st != BEAM_OK) return st;
  if ((st = check_route_out(out)) != BEAM_OK) return st;
  if (T == 0) return BEAM_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Ptrs p = carve(lay, ws, out);
  return run_routing(*layer, x, T, expert_tile_rows(*layer, T), p, s);
}

int beam_moe_forward(const beam_moe_layer* layer, const void* x, int32_t T, void* y,
                     const beam_route_out* out, void* ws, size_t ws_bytes, void* stream) {
  WsLayout lay;
  int st = check_call(layer, x, T, ws, ws_bytes, &lay);
  if (st != BEAM_OK) return st;
  if (out && (st = check_route_out(out)) != BEAM_OK) return st;
  if (T == 0) return BEAM_OK;
  if (!y || !aligned16(y) || y == x) return BEAM_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Ptrs p = carve(lay, ws, out);
  const int tile_rows = expert_tile_rows(*layer, T);
  if ((st = run_routing(*layer, x, T, tile_rows, p, s)) != BEAM_OK) return st;
  if (!select_builds_plan(*layer, T)) BEAM_TRY(launch_scatter(*layer, T, p, s));
  if (gate_up_t1(*layer, T)) BEAM_TRY(launch_gate_up_t1(*layer, x, p, s));
  else BEAM_TRY(launch_gate_up(*layer, x, T, tile_rows, lay, p, s));
  if (down_combine_fused(*layer, T)) {
    BEAM_TRY(launch_down_combine_t1(*layer, p, y, s));
    return BEAM_OK;
  }
  BEAM_TRY(launch_down(*layer, T, tile_rows, lay, p, s, /*allow_split=*/true));
  BEAM_TRY(launch_combine(*layer, T, tile_rows, p, y, s));
  return BEAM_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is a static device array.
// ---------------------------------------------------------------------------

// Every GPU the library runs on holds its own copy of this array from the
// first call of beam_moe_forward_static on it until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address on each GPU comes from hipGetSymbolAddress, once per device,
// and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[BEAM_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int beam_moe_forward_static(const beam_moe_layer* layer, const void* x, int32_t T, void* y,
                            const beam_route_out* out, void* stream) {
  // Sizes are checked before any HIP call: a batch whose workspace exceeds
  // the array is rejected with nothing launched.
  int st = check_layer(layer);
  if (st != BEAM_OK) return st;
  if (T < 0) return BEAM_ERR_INVALID_ARG;
  if (long(T) * layer->K > (1L << 30) || long(T) * layer->D > kMaxOffsetElems) return BEAM_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_OK;
  if (workspace_layout(*layer, T).total > size_t(BEAM_STATIC_WORKSPACE_BYTES)) return BEAM_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return BEAM_ERR_HIP;
  return beam_moe_forward(layer, x, T, y, out, ws, size_t(BEAM_STATIC_WORKSPACE_BYTES), stream);
}

int beam_moe_mask_backward(const beam_moe_layer* layer, const void* x, const void* dy, int32_t T,
                           float beta, float* dwm, float* dbm, float* lreg, void* ws,
                           size_t ws_bytes, void* stream) {
  WsLayout lay;
  int st = check_call(layer, x, T, ws, ws_bytes, &lay);
  if (st != BEAM_OK) return st;
  if (layer->gating != 0 || layer->segment_len > 1) return BEAM_ERR_UNSUPPORTED;
  if (!dwm || !lreg || (reinterpret_cast<uintptr_t>(dwm) & 15u) ||
      (reinterpret_cast<uintptr_t>(lreg) & 3u) || (dbm && (reinterpret_cast<uintptr_t>(dbm) & 3u)))
    return BEAM_ERR_INVALID_ARG;
  if (T == 0) return BEAM_OK;
  if (!dy || !aligned16(dy)) return BEAM_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const beam_moe_layer& L = *layer;
  const Ptrs p = carve(lay, ws, nullptr);
  const int tile_rows = expert_tile_rows(L, T);
  // routing with every candidate kept, then every candidate's expert output
  BEAM_TRY(launch_router_logits(L, x, T, p, s));
  BEAM_TRY(launch_select(L, T, tile_rows, p, s, true));
  if (!select_builds_plan(L, T)) {
    BEAM_TRY(launch_scan(L, T, tile_rows, p, s, true));
    BEAM_TRY(launch_scatter(L, T, p, s));
  }
  BEAM_TRY(launch_gate_up(L, x, T, tile_rows, lay, p, s));
  BEAM_TRY(launch_down(L, T, tile_rows, lay, p, s));
  BEAM_TRY(launch_mask_grad(L, x, dy, T, beta, dwm, dbm, lreg, p, s));
  return BEAM_OK;
}

int beam_moe_stats_host(const beam_moe_layer* layer, const int32_t* counts, int32_t T,
                        beam_stats* out) {
  int st = check_layer(layer);
  if (st != BEAM_OK) return st;
  if (!out || T < 0 || (!counts && T > 0)) return BEAM_ERR_INVALID_ARG;
  const beam_moe_layer& L = *layer;
  beam_stats s;
  memset(&s, 0, sizeof(s));
  s.T = T;
  s.E = L.E;
  s.K = L.K;
  int64_t P = 0;
  int act = 0;
  for (int e = 0; e < L.E && T > 0; ++e) {
    if (counts[e] < 0) return BEAM_ERR_INVALID_ARG;
    P += counts[e];
    act += counts[e] > 0;
  }
  const double elt = L.dtype == BEAM_F32 ? 4.0 : 2.0;
  const double D = L.D, I = L.I, Is = L.I_shared, S = L.n_shared;
  s.active_pairs = P;
  s.active_experts = act;
  s.avg_k = T > 0 ? double(P) / T : 0.0;
  s.flops_routed = 6.0 * D * I * double(P);
  s.flops_topk_routed = 6.0 * D * I * double(T) * L.K;
  s.flops_shared = 6.0 * D * Is * S * T;
  s.flops_router = 4.0 * double(L.E) * D * T;
  s.flops_reduction = T > 0 ? 1.0 - s.flops_routed / s.flops_topk_routed : 0.0;
  const bool fp8 = L.expert_format == BEAM_WEIGHTS_FP8_E4M3;
  // bytes of one expert's three matrices (FP8: codes plus one fp32 per row)
  const double per_routed = fp8 ? 3.0 * D * I + 4.0 * (2.0 * I + D) : 3.0 * D * I * elt;
  const double per_shared = fp8 ? 3.0 * D * Is + 4.0 * (2.0 * Is + D) : 3.0 * D * Is * elt;
  s.bytes_active_expert_weights = per_routed * act + per_shared * S;
  s.bytes_total_min = s.bytes_active_expert_weights + 2.0 * L.E * D * elt + 2.0 * double(T) * D * elt;
  *out = s;
  return BEAM_OK;
}

int beam_moe_stats(const beam_moe_layer* layer, const int32_t* expert_count, int32_t T,
                   beam_stats* host_out, void* stream) {
  int st = check_layer(layer);
  if (st != BEAM_OK) return st;
  if (!host_out || T < 0 || (!expert_count && T > 0)) return BEAM_ERR_INVALID_ARG;
  std::vector<int32_t> h(layer->E, 0);
  if (T > 0) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(h.data(), expert_count, sizeof(int32_t) * layer->E, hipMemcpyDeviceToHost,
                       s) != hipSuccess)
      return BEAM_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return BEAM_ERR_HIP;
  }
  return beam_moe_stats_host(layer, h.data(), T, host_out);
}

const char* beam_status_str(int status) {
  switch (status) {
    case BEAM_OK: return "BEAM_OK";
    case BEAM_ERR_INVALID_ARG: return "BEAM_ERR_INVALID_ARG: invalid argument";
    case BEAM_ERR_UNSUPPORTED: return "BEAM_ERR_UNSUPPORTED: shape or option not supported";
    case BEAM_ERR_WORKSPACE: return "BEAM_ERR_WORKSPACE: workspace missing or too small";
    case BEAM_ERR_HIP: return "BEAM_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown beam_status";
  }
}

int beam_profile_begin(int32_t max_launches) {
  if (max_launches <= 0 || g_prof.on) return BEAM_ERR_INVALID_ARG;
  if (int(g_prof.ev0.size()) < max_launches) {
    while (int(g_prof.ev0.size()) < max_launches) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return BEAM_ERR_HIP;
      if (hipEventCreate(&b) != hipSuccess) return BEAM_ERR_HIP;
      g_prof.ev0.push_back(a);
      g_prof.ev1.push_back(b);
    }
  }
  g_prof.names.assign(max_launches, nullptr);
  g_prof.max = max_launches;
  g_prof.n = 0;
  g_prof.pending = false;
  g_prof.on = true;
  return BEAM_OK;
}

int beam_profile_end(const char** names, int32_t* launches, double* total_ms, int32_t max_out) {
  if (!g_prof.on) return BEAM_ERR_INVALID_ARG;
  g_prof.on = false;
  std::vector<std::string> order;
  std::map<std::string, std::pair<int, double>> agg;
  std::map<std::string, const char*> keep;
  for (int i = 0; i < g_prof.n; ++i) {
    if (hipEventSynchronize(g_prof.ev1[i]) != hipSuccess) return BEAM_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_prof.ev0[i], g_prof.ev1[i]) != hipSuccess) return BEAM_ERR_HIP;
    const std::string k(g_prof.names[i]);
    if (!agg.count(k)) {
      order.push_back(k);
      keep[k] = g_prof.names[i];
    }
    agg[k].first += 1;
    agg[k].second += ms;
  }
  int n = 0;
  for (const auto& k : order) {
    if (n >= max_out) break;
    if (names) names[n] = keep[k];
    if (launches) launches[n] = agg[k].first;
    if (total_ms) total_ms[n] = agg[k].second;
    ++n;
  }
  return n;
}

int beam_moe_pack_weights(const void* w, int32_t mats, int32_t rows, int32_t cols, void* packed,
                          void* stream) {
  if (!w || !packed || !aligned16(w) || !aligned16(packed) || mats < 0 || rows <= 0 || cols <= 0 ||
      rows % 32 || cols % 64 || long(rows) * cols > kMaxOffsetElems)
    return BEAM_ERR_INVALID_ARG;
  const size_t bytes = size_t(mats) * rows * cols * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(packed);
  if (mats > 0 && a < b + bytes && b < a + bytes) return BEAM_ERR_INVALID_ARG;   // overlap
  if (mats == 0) return BEAM_OK;
  return launch_pack_weights(w, mats, rows, cols, packed, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? BEAM_OK
             : BEAM_ERR_HIP;
}

int beam_mfma_loop(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u) || blocks <= 0 || iters <= 0 ||
      blocks > (1 << 20))
    return BEAM_ERR_INVALID_ARG;
  return launch_mfma_loop(out, blocks, iters, static_cast<hipStream_t>(stream)) == hipSuccess
             ? BEAM_OK
             : BEAM_ERR_HIP;
}

int beam_copy_kernel(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes % 16 || !aligned16(dst) || !aligned16(src)) return BEAM_ERR_INVALID_ARG;
  if (bytes == 0) return BEAM_OK;
  return launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK
                                                                                      : BEAM_ERR_HIP;
}

}  // extern "C"

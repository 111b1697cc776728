// Expert kernels of the BEAM layer: grouped SwiGLU gate/up products, grouped
// down products, and the gated combine.
//
// Method: BEAM page on aitrends.kr ("BEAM: Dynamic MoE 라우팅을 위한 Binary
// Expert Activation Masking"), method paragraph Step 4: y = sum_i g_hat_i
// E_i(x) with g_hat = g * m; only pairs with m = 1 are evaluated (ai-feeds.com
// summary, section on inference), and shared experts are added with gate 1
// (aitrends.kr page, limitation C).  Experts are SwiGLU FFNs,
// E(x) = Wd (silu(Wg x) * (Wu x)).
//
// Work is listed as (tile, n-block) items: tiles come from the scan kernel
// (routed tiles expert-major, then the shared tiles); the fused shared expert
// is virtual expert E whose intermediate rows are the n_shared experts'
// rows back to back.  Grids are persistent: workgroup b takes items b,
// b + gridDim.x, ... up to the device-side item count, so no host readback of
// the counts is needed.
#include <cmath>
#include <map>
#include <mutex>

#include "beam_internal.h"
#include "gemm_engines.h"
#include "prefill_engine.h"
#include "stream_engine.h"

namespace beam {

struct ExpertArgs {
  const void* x;
  const void* wg;
  const void* wu;
  const void* wd;
  const void* sg;
  const void* su;
  const void* sd;
  // FP8 E4M3 expert weights: float32 scale of each output row (else null)
  const float* qg;    // [E][I]
  const float* qu;    // [E][I]
  const float* qd;    // [E][D]
  const float* qsg;   // [S*Is] (the fused shared expert's intermediate rows)
  const float* qsu;   // [S*Is]
  const float* qsd;   // [S][D]
  // the same weights in the packed operand layout (prefill kernels), or null
  const u16* pg;    // [E] x packed [I][D]
  const u16* pu;
  const u16* pd;    // [E] x packed [D][I]
  const u16* psg;   // packed [S*Is][D]
  const u16* psu;
  const u16* psd;   // [S] x packed [D][Is]
  int T, D, E, I, S, Is;
  const Plan* plan;
  const Tile* tiles;
  const int32_t* perm_token;
  const int32_t* expert_off;   // [E + 1] first pair of each expert (prefill item order)
  int tile_rows;               // rows per routed tile (the last of an expert may be shorter)
  // expert-stationary prefill (tiles of kEsTileRows rows): packed tokens of
  // each tile ([tile][12 x D/64 blocks of 32 x 64]) and packed h ([tile][12 x I/64])
  u16* xpk;
  u16* hpk;
  void* h;         // [P][I]
  void* h_sh;      // [T][S*Is]
  void* o;         // [P][D] expert outputs: fp32 (fp32 layers) or bf16
  void* o_sh;      // [T][D] shared-expert outputs, same type
  // k-split prefill down: fp32 partials [split][T K][D] and [split][T][D]
  float* op;
  float* op_sh;
  long op_stride, op_sh_stride;   // elements per split
  int down_slots;                 // resident workgroups of the down kernel (0: never split)
  int es_ntiles;                  // > 0: the expert-stationary kernels take the shared
                                  // experts, tiles of kEsTileRows consecutive tokens
};

// Order of the shared items.  Every shared tile reads the same weights, so
// the items are taken in groups of 8 weight blocks x nts tiles, weight block
// fastest: item w and w + 8 read the same block, and the streaming kernels run
// item w on XCD w % 8, so the tiles of one block meet in one L2.
__device__ __forceinline__ void shared_item(long w2, int nts, int nbs, int& t, int& nb) {
  constexpr int kX = 8;
  const long g = w2 / (long(kX) * nts);
  const int q = int(w2 - g * kX * nts);
  const int r = min(kX, nbs - int(g) * kX);   // blocks in this group
  t = q / r;
  nb = int(g) * kX + q % r;
}

// Tile record via scalar loads (see ld_const).
__device__ __forceinline__ Tile ld_tile(const Tile* p) {
  const i32x4 v = ld_const(reinterpret_cast<const i32x4*>(p));
  Tile t;
  t.expert = v[0];
  t.row0 = v[1];
  t.rows = v[2];
  t.pad = v[3];
  return t;
}

// Decodes work item w into (tile index, n-block, shared?): routed items
// tile-major, then the shared items.
__device__ __forceinline__ bool work_item(long w, int ntr, int nts, int nbr, int nbs, int& ti,
                                          int& nb, bool& shared) {
  const long wr = long(ntr) * nbr;
  if (w < wr) {
    ti = int(w / nbr);
    nb = int(w % nbr);
    shared = false;
    return true;
  }
  const long w2 = w - wr;
  if (w2 < long(nts) * nbs) {
    int t;
    shared_item(w2, nts, nbs, t, nb);
    ti = ntr + t;
    shared = true;
    return true;
  }
  return false;
}

// Down items: routed (tile, d-block) tile-major, then the shared items.
__device__ __forceinline__ void down_item(long w, int ntr, int nts, int nb_all, int& ti, int& nb) {
  const long wr = long(ntr) * nb_all;
  if (w < wr) {
    ti = int(w / nb_all);
    nb = int(w % nb_all);
  } else {
    int t;
    shared_item(w - wr, nts, nb_all, t, nb);
    ti = ntr + t;
  }
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU (bf16)
// ---------------------------------------------------------------------------

// Cooperative shared items (bf16 launches with a 4-way k split) pay off once
// a shared weight block would otherwise be streamed for this many tiles:
// with fewer, their per-step barriers cost more than the re-reads they save
// (timed on MI355X at T = 1 .. 256, DeepSeek-V2-Lite shapes).
constexpr int kCoopGateUpTiles = 4;
constexpr int kCoopDownTiles = 8;

// Streaming (decode) gate/up: items are (tile, n-block of 16*NB intermediate
// rows); the 2*NB streamed matrices are the gate and up rows of each 16-row
// group, which share the token operand (see stream_engine.h).  F8: the
// weights are E4M3 codes with row scales.
template <int MT, int NB, bool F8>
struct GateUpStream {
  static constexpr int NMAT = 2 * NB;
  static constexpr bool kMultiSeg = false;
  static constexpr long EB = F8 ? 1 : 2;   // bytes per weight
  const ExpertArgs* a;
  int ntr, nts, nbr, nbs;
  long total;
  __device__ long total_items() const { return total; }
  __device__ void decode(long item, int lane, StreamItem<NMAT, MT>& it) const {
    it.valid = item >= 0;
    it.nseg = 1;
    it.w_seg = 0;
    it.x_seg = 0;
    it.cps = a->D / chunk_k<F8>();
    it.w_row = a->D * EB;
    if (!it.valid) {
      it.cps = 1;
      it.w_row = 0;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) it.w[m] = (const unsigned char*)a->wg;
#pragma unroll
      for (int b = 0; b < MT; ++b) it.x[b] = (const u16*)a->x;
      return;
    }
    int ti, nb;
    bool shared;
    work_item(item, ntr, nts, nbr, nbs, ti, nb, shared);
    const Tile tl = ld_tile(a->tiles + ti);
    const size_t eoff = shared ? 0 : size_t(tl.expert) * a->I * a->D * EB;
    const unsigned char* wg = (const unsigned char*)(shared ? a->sg : a->wg) + eoff;
    const unsigned char* wu = (const unsigned char*)(shared ? a->su : a->wu) + eoff;
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const size_t off = size_t(nb * NB + g) * 16 * a->D * EB;
      it.w[2 * g] = wg + off;
      it.w[2 * g + 1] = wu + off;
    }
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const int r = 16 * b + (lane & 15);
      int t = tl.row0 + r;
      if (!shared) {
        // the 16 rows' tokens by scalar loads, each lane picking its own (the
        // perm_token region is padded so that reading 16 past a tile's start
        // stays inside it)
        const int32_t* pt = a->perm_token + tl.row0 + 16 * b;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int32_t v = ld_const(pt + j);
          t = (lane & 15) == j ? v : t;
        }
      }
      if (r >= tl.rows) t = 0;   // absent rows read token 0
      it.x[b] = (const u16*)a->x + size_t(t) * a->D;
    }
  }
  // Cooperative items (bf16, k split 4): (block of NB shared row groups, four
  // consecutive shared tiles), block fastest; the w-th wave takes tile 4g + w.
  long n_coop = 0;
  __device__ long coop_items() const { return n_coop; }
  __device__ bool decode_coop(long item, int w, int lane, StreamItem<NMAT, MT>& it) const {
    const int nb = int(item % nbs), g = int(item / nbs);
    const int t = 4 * g + w;
    const bool mine = t < nts;
    it.valid = true;
    it.nseg = 1;
    it.w_seg = 0;
    it.x_seg = 0;
    it.cps = a->D / chunk_k<F8>();
    it.w_row = a->D * EB;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const size_t off = size_t(nb * NB + q) * 16 * a->D * EB;
      it.w[2 * q] = (const unsigned char*)a->sg + off;
      it.w[2 * q + 1] = (const unsigned char*)a->su + off;
    }
    const Tile tl = ld_tile(a->tiles + ntr + (mine ? t : 0));
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const int r = 16 * b + (lane & 15);
      const int tok = mine && r < tl.rows ? tl.row0 + r : 0;   // absent rows read token 0
      it.x[b] = (const u16*)a->x + size_t(tok) * a->D;
    }
    return mine;
  }
  __device__ void epilogue_coop(long item, int w, const f32x4 (&acc)[NMAT][MT], int lane) const {
    const int nb = int(item % nbs), g = int(item / nbs);
    store_h(ld_tile(a->tiles + ntr + 4 * g + w), nb, true, acc, lane);
  }
  __device__ void scales(long item, int, int lane, f32x4 (&sc)[NMAT]) const {
    int ti, nb;
    bool shared;
    work_item(item, ntr, nts, nbr, nbs, ti, nb, shared);
    const Tile tl = ld_tile(a->tiles + ti);
    const size_t base = shared ? 0 : size_t(tl.expert) * a->I;
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const size_t n0 = base + size_t(nb * NB + g) * 16;
      sc[2 * g] = row_scales16((shared ? a->qsg : a->qg) + n0, lane);
      sc[2 * g + 1] = row_scales16((shared ? a->qsu : a->qu) + n0, lane);
    }
  }
  __device__ void epilogue(long item, const f32x4 (&acc)[NMAT][MT], int lane) const {
    int ti, nb;
    bool shared;
    work_item(item, ntr, nts, nbr, nbs, ti, nb, shared);
    store_h(ld_tile(a->tiles + ti), nb, shared, acc, lane);
  }
  __device__ void store_h(const Tile tl, int nb, bool shared, const f32x4 (&acc)[NMAT][MT],
                          int lane) const {
    const int Iv = shared ? a->S * a->Is : a->I;
    u16* hb = shared ? (u16*)a->h_sh : (u16*)a->h;
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const int r = 16 * b + (lane & 15);
      if (r < tl.rows) {
#pragma unroll
        for (int g = 0; g < NB; ++g) {
          const f32x4 gv = acc[2 * g][b], uv = acc[2 * g + 1][b];
          const int n = (nb * NB + g) * 16 + 4 * (lane >> 4);
          ushort4 hv;
          hv.x = f32_to_bf16(silu_f32(gv[0]) * uv[0]);
          hv.y = f32_to_bf16(silu_f32(gv[1]) * uv[1]);
          hv.z = f32_to_bf16(silu_f32(gv[2]) * uv[2]);
          hv.w = f32_to_bf16(silu_f32(gv[3]) * uv[3]);
          *reinterpret_cast<ushort4*>(hb + size_t(tl.row0 + r) * Iv + n) = hv;
        }
      }
    }
  }
};

template <int MT, int NB, int U, int KSPLIT, bool F8>
__global__ __launch_bounds__(kStreamWaves * 64) void k_gate_up_stream(ExpertArgs a) {
  constexpr int NMAT = 2 * NB;
  __shared__ __align__(16) unsigned char lds[StreamLds<NMAT, MT, U, KSPLIT>::kBytes];
  GateUpStream<MT, NB, F8> pb;
  pb.a = &a;
  pb.ntr = ld_const(&a.plan->n_tiles_routed);
  pb.nts = ld_const(&a.plan->n_tiles_shared);
  pb.nbr = a.I / (16 * NB);
  pb.nbs = a.S > 0 ? (a.S * a.Is) / (16 * NB) : 1;
  pb.total = long(pb.ntr) * pb.nbr + long(pb.nts) * pb.nbs;
  if constexpr (KSPLIT == 4 && !F8) {
    if (pb.nts >= kCoopGateUpTiles) {
      // shared tiles as cooperative items, ahead of the routed items
      pb.n_coop = long((pb.nts + 3) / 4) * pb.nbs;
      pb.total = long(pb.ntr) * pb.nbr;
      stream_coop_run<NMAT, MT>(pb, lds, StreamLds<NMAT, MT, U, KSPLIT>::kWaveBytes);
    }
  }
  stream_run<NMAT, MT, U, KSPLIT, F8>(pb, lds, pb.n_coop);
}

// Streaming (decode) down: items are (tile, d-block of 16*NB output rows),
// the NB 16-row groups streamed as NB matrices that share the h operand; the
// fused shared expert has one k segment per shared expert.
template <int MT, int NB, bool F8>
struct DownStream {
  static constexpr bool kMultiSeg = true;
  static constexpr long EB = F8 ? 1 : 2;   // bytes per weight
  const ExpertArgs* a;
  int ntr, nts, nb_all;
  long total;
  __device__ long total_items() const { return total; }
  __device__ void decode(long item, int lane, StreamItem<NB, MT>& it) const {
    it.valid = item >= 0;
    if (!it.valid) {
      it.nseg = 1;
      it.cps = 1;
#pragma unroll
      for (int g = 0; g < NB; ++g) it.w[g] = (const unsigned char*)a->wd;
      it.w_row = it.w_seg = it.x_seg = 0;
#pragma unroll
      for (int b = 0; b < MT; ++b) it.x[b] = (const u16*)a->h;
      return;
    }
    int ti, nb;
    down_item(item, ntr, nts, nb_all, ti, nb);
    const bool shared = ti >= ntr;
    const Tile tl = ld_tile(a->tiles + ti);
    const int d0 = nb * 16 * NB;
    const unsigned char* w0;
    if (shared) {
      it.nseg = a->S;
      it.cps = a->Is / chunk_k<F8>();
      w0 = (const unsigned char*)a->sd + size_t(d0) * a->Is * EB;
      it.w_row = a->Is * EB;
      it.w_seg = long(a->D) * a->Is * EB;
      it.x_seg = a->Is;
    } else {
      it.nseg = 1;
      it.cps = a->I / chunk_k<F8>();
      w0 = (const unsigned char*)a->wd + (size_t(tl.expert) * a->D + d0) * a->I * EB;
      it.w_row = a->I * EB;
      it.w_seg = 0;
      it.x_seg = 0;
    }
#pragma unroll
    for (int g = 0; g < NB; ++g) it.w[g] = w0 + size_t(16 * g) * it.w_row;
    const long hs = shared ? long(a->S) * a->Is : a->I;
    const u16* hb = shared ? (const u16*)a->h_sh : (const u16*)a->h;
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const int r = 16 * b + (lane & 15);
      // absent rows read the tile's first row
      it.x[b] = hb + size_t(tl.row0 + (r < tl.rows ? r : 0)) * hs;
    }
  }
  __device__ void scales(long item, int seg, int lane, f32x4 (&sc)[NB]) const {
    int ti, nb;
    down_item(item, ntr, nts, nb_all, ti, nb);
    const bool shared = ti >= ntr;
    const float* q = shared ? a->qsd + size_t(seg) * a->D
                            : a->qd + size_t(ld_tile(a->tiles + ti).expert) * a->D;
#pragma unroll
    for (int g = 0; g < NB; ++g) sc[g] = row_scales16(q + (nb * NB + g) * 16, lane);
  }
  // Cooperative items (bf16, k split 4): (d-block, four consecutive shared
  // tiles), d-block fastest; the w-th wave takes tile 4g + w.
  long n_coop = 0;
  __device__ long coop_items() const { return n_coop; }
  __device__ bool decode_coop(long item, int w, int lane, StreamItem<NB, MT>& it) const {
    const int nb = int(item % nb_all), g = int(item / nb_all);
    const int t = 4 * g + w;
    const bool mine = t < nts;
    it.valid = true;
    it.nseg = a->S;
    it.cps = a->Is / chunk_k<F8>();
    it.w_row = a->Is * EB;
    it.w_seg = long(a->D) * a->Is * EB;
    it.x_seg = a->Is;
    const unsigned char* w0 = (const unsigned char*)a->sd + size_t(nb * 16 * NB) * a->Is * EB;
#pragma unroll
    for (int q = 0; q < NB; ++q) it.w[q] = w0 + size_t(16 * q) * it.w_row;
    const Tile tl = ld_tile(a->tiles + ntr + (mine ? t : 0));
    const long hs = long(a->S) * a->Is;
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const int r = 16 * b + (lane & 15);
      it.x[b] = (const u16*)a->h_sh + size_t(tl.row0 + (mine && r < tl.rows ? r : 0)) * hs;
    }
    return mine;
  }
  __device__ void epilogue_coop(long item, int w, const f32x4 (&acc)[NB][MT], int lane) const {
    const int nb = int(item % nb_all), g = int(item / nb_all);
    store_o(ld_tile(a->tiles + ntr + 4 * g + w), nb, true, acc, lane);
  }
  __device__ void epilogue(long item, const f32x4 (&acc)[NB][MT], int lane) const {
    int ti, nb;
    down_item(item, ntr, nts, nb_all, ti, nb);
    const bool shared = ti >= ntr;
    store_o(ld_tile(a->tiles + ti), nb, shared, acc, lane);
  }
  __device__ void store_o(const Tile tl, int nb, bool shared, const f32x4 (&acc)[NB][MT],
                          int lane) const {
    u16* ob = static_cast<u16*>(shared ? a->o_sh : a->o);
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const int r = 16 * b + (lane & 15);
      if (r < tl.rows) {
#pragma unroll
        for (int g = 0; g < NB; ++g) {
          const int d = (nb * NB + g) * 16 + 4 * (lane >> 4);
          const f32x4 v = acc[g][b];
          st4_bf16(ob, size_t(tl.row0 + r) * a->D + d, v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
};

template <int MT, int NB, int U, int KSPLIT, bool F8>
__global__ __launch_bounds__(kStreamWaves * 64) void k_down_stream(ExpertArgs a) {
  __shared__ __align__(16) unsigned char lds[StreamLds<NB, MT, U, KSPLIT>::kBytes];
  DownStream<MT, NB, F8> pb;
  pb.a = &a;
  pb.ntr = ld_const(&a.plan->n_tiles_routed);
  pb.nts = ld_const(&a.plan->n_tiles_shared);
  pb.nb_all = a.D / (16 * NB);
  pb.total = long(pb.ntr + pb.nts) * pb.nb_all;
  if constexpr (KSPLIT == 4 && !F8) {
    if (pb.nts >= kCoopDownTiles) {
      // shared tiles as cooperative items, ahead of the routed items
      pb.n_coop = long((pb.nts + 3) / 4) * pb.nb_all;
      pb.total = long(pb.ntr) * pb.nb_all;
      stream_coop_run<NB, MT>(pb, lds, StreamLds<NB, MT, U, KSPLIT>::kWaveBytes);
    }
  }
  stream_run<NB, MT, U, KSPLIT, F8>(pb, lds, pb.n_coop);
}

// Tiled (prefill): the BN weight rows of an n-block are BN/2 intermediate
// rows of Wg and the same rows of Wu, interleaved in 32-row groups (gate, up,
// gate, up, ...) so that a lane holds gate and up of the same element.
struct GateUpTiledProv {
  const u16* wg;
  const u16* wu;
  const u16* xb;
  const int32_t* perm;
  int D, Iv, i0, row0, rows;
  __device__ int nseg() const { return 1; }
  __device__ int seg_chunks() const { return D / 64; }
  __device__ const u16* wbase(int g, int) const { return (g & 1) ? wu : wg; }
  __device__ uint32_t woff(int r) const {
    int irow = i0 + (r >> 6) * 32 + (r & 31);
    if (irow >= Iv) irow = 0;
    return uint32_t(long(irow) * D);
  }
  __device__ const u16* xbase(int) const { return xb; }
  __device__ uint32_t xoff(int r) const {
    const int rr = r < rows ? r : 0;   // absent rows read the tile's first token
    const int t = perm ? perm[row0 + rr] : row0 + rr;
    return uint32_t(long(t) * D);
  }
};

template <int BN, int BM>
__global__ __launch_bounds__(256, 2) void k_gate_up_tiled(ExpertArgs a) {
  __shared__ TiledSmem<BN, BM> sm;
  constexpr int JN = BN / 64, JM = BM / 64, IB = BN / 2;   // IB: intermediate rows per tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int ntr = a.plan->n_tiles_routed, nts = a.plan->n_tiles_shared;
  const int nbr = (a.I + IB - 1) / IB, nbs = a.S > 0 ? (a.S * a.Is + IB - 1) / IB : 1;
  const long total = long(ntr) * nbr + long(nts) * nbs;
  for (XcdRange it = xcd_range(total); it.next < it.end; it.next += it.step) {
    int ti, nb;
    bool shared;
    work_item(it.next, ntr, nts, nbr, nbs, ti, nb, shared);
    const Tile tl = a.tiles[ti];
    const int Iv = shared ? a.S * a.Is : a.I;
    GateUpTiledProv pv;
    pv.wg = shared ? (const u16*)a.sg : (const u16*)a.wg + size_t(tl.expert) * a.I * a.D;
    pv.wu = shared ? (const u16*)a.su : (const u16*)a.wu + size_t(tl.expert) * a.I * a.D;
    pv.perm = shared ? nullptr : a.perm_token;
    pv.xb = (const u16*)a.x;
    pv.D = a.D;
    pv.Iv = Iv;
    pv.i0 = nb * IB;
    pv.row0 = tl.row0;
    pv.rows = tl.rows;
    f32x16 acc[JN][JM];
    tiled_accumulate<BN, BM>(pv, sm, acc, tl.rows);
    u16* hb = shared ? (u16*)a.h_sh : (u16*)a.h;
#pragma unroll
    for (int p = 0; p < JN / 2; ++p)
#pragma unroll
      for (int jm = 0; jm < JM; ++jm) {
        const int r = wm * (BM / 2) + jm * 32 + (lane & 31);
        if (r < tl.rows) {
          const f32x16 g = acc[2 * p][jm], u = acc[2 * p + 1][jm];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = nb * IB + (wn * (JN / 2) + p) * 32 + 8 * q + 4 * (lane >> 5);
            if (n < Iv) {
              ushort4 hv;
              hv.x = f32_to_bf16(silu_f32(g[4 * q + 0]) * u[4 * q + 0]);
              hv.y = f32_to_bf16(silu_f32(g[4 * q + 1]) * u[4 * q + 1]);
              hv.z = f32_to_bf16(silu_f32(g[4 * q + 2]) * u[4 * q + 2]);
              hv.w = f32_to_bf16(silu_f32(g[4 * q + 3]) * u[4 * q + 3]);
              *reinterpret_cast<ushort4*>(hb + size_t(tl.row0 + r) * Iv + n) = hv;
            }
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// down (bf16): O[row][d] = sum_i h[row][i] Wd[d][i]
// ---------------------------------------------------------------------------

struct DownProvBase {
  const u16* wd;     // expert's [D][I] or shared [S][D][Is]
  const u16* h;      // rows of h for this tile, row stride hs
  int D, Iv, Is, S, hs, d0, rows;
  bool shared;
  __device__ int nseg() const { return shared ? S : 1; }
  __device__ int seg_chunks() const { return (shared ? Is : Iv) / 64; }
  __device__ const u16* wbase(int, int seg) const { return shared ? wd + size_t(seg) * D * Is : wd; }
  __device__ uint32_t woff(int r) const {
    int d = d0 + r;
    if (d >= D) d = 0;
    return uint32_t(long(d) * (shared ? Is : Iv));
  }
  __device__ const u16* xbase(int seg) const { return h + (shared ? seg * Is : 0); }
  __device__ uint32_t xoff(int r) const { return uint32_t(long(r < rows ? r : 0) * hs); }
};

template <class P>
__device__ __forceinline__ void down_setup(const ExpertArgs& a, const Tile& tl, bool shared, P& pv) {
  pv.D = a.D;
  pv.S = a.S;
  pv.Is = a.Is;
  pv.shared = shared;
  pv.rows = tl.rows;
  if (shared) {
    pv.wd = (const u16*)a.sd;
    pv.Iv = a.S * a.Is;
    pv.hs = a.S * a.Is;
    pv.h = (const u16*)a.h_sh + size_t(tl.row0) * pv.hs;
  } else {
    pv.wd = (const u16*)a.wd + size_t(tl.expert) * a.D * a.I;
    pv.Iv = a.I;
    pv.hs = a.I;
    pv.h = (const u16*)a.h + size_t(tl.row0) * pv.hs;
  }
}

// With a k split (down_split: too few items to fill the GPU), item w is
// split w % ks of (tile, d-block) w / ks: the adjacent items of one output
// block read disjoint k ranges of the same weight rows, and each writes its
// fp32 partial sums to its own slice of the partial buffer; the combine adds
// the slices in split order.
template <int BN, int BM>
__global__ __launch_bounds__(256, 2) void k_down_tiled(ExpertArgs a) {
  __shared__ TiledSmem<BN, BM> sm;
  constexpr int JN = BN / 64, JM = BM / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int ntr = a.plan->n_tiles_routed, nts = a.plan->n_tiles_shared;
  const int nb_all = (a.D + BN - 1) / BN;
  const long items = long(ntr + nts) * nb_all;
  const int ks = down_split(items, a.down_slots);
  for (XcdRange it = xcd_range(items * ks); it.next < it.end; it.next += it.step) {
    int ti, nb;
    const long wi = it.next / ks;
    const int split = int(it.next - wi * ks);
    down_item(wi, ntr, nts, nb_all, ti, nb);
    const bool shared = ti >= ntr;
    const Tile tl = a.tiles[ti];
    DownProvBase pv;
    down_setup(a, tl, shared, pv);
    pv.d0 = nb * BN;
    const int C = pv.nseg() * pv.seg_chunks();
    f32x16 acc[JN][JM];
    tiled_accumulate<BN, BM>(pv, sm, acc, tl.rows, C * split / ks, C * (split + 1) / ks);
    u16* ob = static_cast<u16*>(shared ? a.o_sh : a.o);
    float* pb = shared ? a.op_sh + split * a.op_sh_stride : a.op + split * a.op_stride;
#pragma unroll
    for (int jn = 0; jn < JN; ++jn)
#pragma unroll
      for (int jm = 0; jm < JM; ++jm) {
        const int r = wm * (BM / 2) + jm * 32 + (lane & 31);
        if (r < tl.rows) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = nb * BN + wn * (BN / 2) + jn * 32 + 8 * q + 4 * (lane >> 5);
            if (d < a.D) {
              const f32x16& v = acc[jn][jm];
              const size_t e = size_t(tl.row0 + r) * a.D + d;
              if (ks == 1)
                st4_bf16(ob, e, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
              else
                *reinterpret_cast<float4*>(pb + e) =
                    make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            }
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Prefill kernels on packed weights (tiles of 128 token rows; prefill_engine.h)
// ---------------------------------------------------------------------------

// Routed items of the packed kernels, expert by expert and n-block-major
// within an expert: the tiles of one expert that read the same weight block
// are adjacent items, so they run at about the same time on one XCD (the
// item space is cut into one contiguous part per XCD) and the block comes
// from HBM once; these kernels stream their weights at close to the HBM rate,
// and with tile-major items an expert's two or three 128-row tiles each
// fetched its weights from HBM again.  Item w lies in the range of the
// expert of tile w / nb_per_tile (the tile-major order covers each expert's
// tiles contiguously too), whose first tile and tile count follow from its
// pair offsets.
__device__ __forceinline__ void packed_routed_item(const ExpertArgs& a, long w, int nb_per_tile,
                                                   int& ti, int& nb) {
  const int ti0 = int(w / nb_per_tile);
  const Tile t0 = ld_tile(a.tiles + ti0);
  const int off = ld_const(a.expert_off + t0.expert);
  const int cnt = ld_const(a.expert_off + t0.expert + 1) - off;
  const int base = ti0 - (t0.row0 - off) / a.tile_rows;
  const int nt = (cnt + a.tile_rows - 1) / a.tile_rows;
  const long q = w - long(base) * nb_per_tile;
  nb = int(q / nt);
  ti = base + int(q - long(nb) * nt);
}

// Gate/up: a workgroup's 256 weight rows are 128 intermediate rows of Wg and
// Wu; wave w takes intermediate rows 32 w .. 32 w + 31 as its gate block
// (j = 0) and up block (j = 1), so a lane holds gate and up of the same
// elements and SwiGLU is applied in registers.
struct GateUpPackedProv {
  const u16* wg;     // packed [Iv][D] of the (virtual) expert
  const u16* wu;
  const u16* xb;
  int D, Iv, i0, wave;
  const int32_t* perm;
  int row0, rows;
  __device__ int nseg() const { return 1; }
  __device__ int seg_chunks() const { return D / kPK; }
  __device__ const u16* wbase(int j, int) const { return j ? wu : wg; }
  __device__ uint32_t wblk(int) const {
    int rb = (i0 >> 5) + wave;
    if (rb >= (Iv >> 5)) rb = 0;   // absent rows: results never stored
    return uint32_t(rb) * uint32_t(D / kPK) * kPackBlock;
  }
  __device__ const u16* xbase(int) const { return xb; }
  __device__ uint32_t xoff(int R) const {
    const int rr = R < rows ? R : 0;   // absent rows read the tile's first token
    const int t = perm ? perm[row0 + rr] : row0 + rr;
    return uint32_t(t) * uint32_t(D);
  }
};

constexpr int kPackedIB = 128;   // intermediate rows per packed gate/up item

// One item of the packed gate/up kernel (item < ntr nbr + nts nbs).
__device__ __forceinline__ void packed_gate_up_item(const ExpertArgs& a, PrefillSmem<128>& sm, long item,
                                                    int ntr, int nts, int nbr, int nbs) {
  constexpr int BM = 128, JM = BM / 32, IB = kPackedIB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  {
    int ti, nb;
    bool shared;
    work_item(item, ntr, nts, nbr, nbs, ti, nb, shared);
    if (!shared) packed_routed_item(a, item, nbr, ti, nb);
    const Tile tl = ld_tile(a.tiles + ti);
    const int Iv = shared ? a.S * a.Is : a.I;
    GateUpPackedProv pv;
    pv.wg = shared ? a.psg : a.pg + size_t(tl.expert) * a.I * a.D;
    pv.wu = shared ? a.psu : a.pu + size_t(tl.expert) * a.I * a.D;
    pv.perm = shared ? nullptr : a.perm_token;
    pv.xb = (const u16*)a.x;
    pv.D = a.D;
    pv.Iv = Iv;
    pv.i0 = nb * IB;
    pv.wave = wave;
    pv.row0 = tl.row0;
    pv.rows = tl.rows;
    f32x16 acc[2][JM];
    prefill_accumulate<BM>(pv, sm, acc, tl.rows);
    u16* hb = shared ? (u16*)a.h_sh : (u16*)a.h;
#pragma unroll
    for (int b = 0; b < JM; ++b) {
      const int r = b * 32 + (lane & 31);
      if (r < tl.rows) {
        const f32x16 g = acc[0][b], u = acc[1][b];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb * IB + 32 * wave + 8 * q + 4 * (lane >> 5);
          if (n < Iv) {
            ushort4 hv;
            hv.x = f32_to_bf16(silu_f32(g[4 * q + 0]) * u[4 * q + 0]);
            hv.y = f32_to_bf16(silu_f32(g[4 * q + 1]) * u[4 * q + 1]);
            hv.z = f32_to_bf16(silu_f32(g[4 * q + 2]) * u[4 * q + 2]);
            hv.w = f32_to_bf16(silu_f32(g[4 * q + 3]) * u[4 * q + 3]);
            *reinterpret_cast<ushort4*>(hb + size_t(tl.row0 + r) * Iv + n) = hv;
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_gate_up_packed(ExpertArgs a) {
  __shared__ PrefillSmem<128> sm;
  const int ntr = ld_const(&a.plan->n_tiles_routed), nts = ld_const(&a.plan->n_tiles_shared);
  const int nbr = (a.I + kPackedIB - 1) / kPackedIB;
  const int nbs = a.S > 0 ? (a.S * a.Is + kPackedIB - 1) / kPackedIB : 1;
  const long total = long(ntr) * nbr + long(nts) * nbs;
  for (XcdRange it = xcd_range(total); it.next < it.end; it.next += it.step)
    packed_gate_up_item(a, sm, it.next, ntr, nts, nbr, nbs);
}

// Down: a workgroup's 256 weight rows are output features d0 .. d0 + 255;
// wave w takes d0 + 64 w .. + 63 as two 32-row blocks.  The fused shared
// expert has one k segment (one packed matrix) per shared expert.  With a k
// split (down_split) the items are split as in k_down_tiled, and each split
// writes fp32 partials.  With shared experts the items are handed out in
// order by a work counter (ItemQueue): the shared tiles (full, 128 rows)
// come after the routed ones (often a few rows), so a static split left the
// XCDs with routed parts idle early (DeepSeek-V2-Lite prefill T = 4096 on
// MI355X: 158 -> 135 us).  Routed-only layers keep the static split (the
// fine-grained T = 8192 layer: 66.5 us static, 69.5 with the counter), and
// so does the gate/up kernel, where the counter cost more in L2 reuse than
// it gained (206 -> 215 us on the DeepSeek-V2-Lite layer).
struct DownPackedProv {
  const u16* wd;     // packed [D][I] of the expert, or the shared experts' first [D][Is]
  const u16* h;      // rows of h for this tile, row stride hs
  int D, Iv, Is, S, hs, d0, wave, rows;
  bool shared;
  __device__ int nseg() const { return shared ? S : 1; }
  __device__ int seg_chunks() const { return (shared ? Is : Iv) / kPK; }
  __device__ const u16* wbase(int, int seg) const { return shared ? wd + size_t(seg) * D * Is : wd; }
  __device__ uint32_t wblk(int j) const {
    int rb = (d0 >> 5) + 2 * wave + j;
    if (rb >= (D >> 5)) rb = 0;
    return uint32_t(rb) * uint32_t(seg_chunks()) * kPackBlock;
  }
  __device__ const u16* xbase(int seg) const { return h + (shared ? seg * Is : 0); }
  __device__ uint32_t xoff(int R) const { return uint32_t(R < rows ? R : 0) * uint32_t(hs); }
};

constexpr int kPackedDB = 256;   // output features per packed down item

// One item of the packed down kernel (item < (ntr + nts) nb_all ks).
__device__ __forceinline__ void packed_down_item(const ExpertArgs& a, PrefillSmem<128>& sm, long item,
                                                 int ntr, int nts, int nb_all, int ks) {
  constexpr int BM = 128, JM = BM / 32, DB = kPackedDB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  {
    int ti, nb;
    const long wi = item / ks;
    const int split = int(item - wi * ks);
    down_item(wi, ntr, nts, nb_all, ti, nb);
    const bool shared = ti >= ntr;
    if (!shared) packed_routed_item(a, wi, nb_all, ti, nb);
    const Tile tl = ld_tile(a.tiles + ti);
    DownPackedProv pv;
    pv.D = a.D;
    pv.S = a.S;
    pv.Is = a.Is;
    pv.shared = shared;
    pv.rows = tl.rows;
    pv.wave = wave;
    pv.d0 = nb * DB;
    if (shared) {
      pv.wd = a.psd;
      pv.Iv = a.S * a.Is;
      pv.hs = a.S * a.Is;
      pv.h = (const u16*)a.h_sh + size_t(tl.row0) * pv.hs;
    } else {
      pv.wd = a.pd + size_t(tl.expert) * a.D * a.I;
      pv.Iv = a.I;
      pv.hs = a.I;
      pv.h = (const u16*)a.h + size_t(tl.row0) * pv.hs;
    }
    const int C = pv.nseg() * pv.seg_chunks();
    f32x16 acc[2][JM];
    prefill_accumulate<BM>(pv, sm, acc, tl.rows, C * split / ks, C * (split + 1) / ks);
    u16* ob = static_cast<u16*>(shared ? a.o_sh : a.o);
    float* pb = shared ? a.op_sh + split * a.op_sh_stride : a.op + split * a.op_stride;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int b = 0; b < JM; ++b) {
        const int r = b * 32 + (lane & 31);
        if (r < tl.rows) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = pv.d0 + 64 * wave + 32 * j + 8 * q + 4 * (lane >> 5);
            if (d < a.D) {
              const f32x16& v = acc[j][b];
              const size_t e = size_t(tl.row0 + r) * a.D + d;
              if (ks == 1)
                st4_bf16(ob, e, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
              else
                *reinterpret_cast<float4*>(pb + e) =
                    make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            }
          }
        }
      }
  }
}

__global__ __launch_bounds__(256, 1) void k_down_packed(ExpertArgs a) {
  __shared__ PrefillSmem<128> sm;
  const int ntr = ld_const(&a.plan->n_tiles_routed), nts = ld_const(&a.plan->n_tiles_shared);
  const int nb_all = (a.D + kPackedDB - 1) / kPackedDB;
  const long items = long(ntr + nts) * nb_all;
  const int ks = down_split(items, a.down_slots);
  // shared tiles present: the work counter; otherwise the static split
  const bool dyn = nts > 0;
  const XcdRange xr = xcd_range(items * ks);
  __shared__ int qslot[2];
  ItemQueue q(const_cast<int32_t*>(&a.plan->down_next), qslot);
  for (long item = dyn ? long(blockIdx.x) : xr.next; item < (dyn ? items * ks : xr.end);
       item = dyn ? q.next() : item + xr.step) {
    if (dyn) q.claim();
    packed_down_item(a, sm, item, ntr, nts, nb_all, ks);
  }
}

// Packed operand layout (see beam_moe_pack_weights): one thread per 16-byte
// chunk of the output, i.e. per (matrix, row block, k block, k-step, lane).
__global__ __launch_bounds__(256) void k_pack_weights(const u16* __restrict__ w, long chunks,
                                                      int rows, int cols, u16* __restrict__ out) {
  const long per_mat = long(rows) * cols / 8;
  for (long q = long(blockIdx.x) * blockDim.x + threadIdx.x; q < chunks; q += long(gridDim.x) * blockDim.x) {
    const long m = q / per_mat;
    const long r = q - m * per_mat;        // chunk within the matrix
    const long blk = r >> 8;               // 256 chunks per 32 x 64 block
    const int within = int(r & 255);
    const int s = within >> 6, l = within & 63;
    const long kbs = cols / 64;
    const long rb = blk / kbs, kb = blk - rb * kbs;
    const long row = 32 * rb + (l & 31);
    const long col = 64 * kb + 16 * s + 8 * (l >> 5);
    const u16* src = w + m * long(rows) * cols + row * cols + col;
    *reinterpret_cast<u32x4*>(out + q * 8) = *reinterpret_cast<const u32x4*>(src);
  }
}

hipError_t launch_pack_weights(const void* w, int mats, int rows, int cols, void* packed,
                               hipStream_t s) {
  const long chunks = long(mats) * rows * cols / 8;
  const long blocks = std::min<long>((chunks + 255) / 256, 8192);
  prof_before("pack_weights", s);
  hipLaunchKernelGGL(k_pack_weights, dim3(unsigned(std::max<long>(blocks, 1))), dim3(256), 0, s,
                     (const u16*)w, chunks, rows, cols, (u16*)packed);
  prof_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Expert-stationary prefill (tiles of kEsTileRows rows): the tokens of each
// tile are packed into the MFMA operand layout once (k_pack_tokens_es),
// gate/up writes h in the same packed layout, and both products run the
// expert-stationary engine, so that an expert's weight blocks stream from
// HBM once per tile.  The tiles are the routed tiles of the plan (layers
// without shared experts), or, with es_ntiles > 0, the fused shared expert's
// tiles of consecutive tokens (the routed tiles then run on the 128-row
// kernels).
// ---------------------------------------------------------------------------

__device__ __forceinline__ size_t es_tile_elems(int K) { return size_t(kEsTokBlocks) * K * 32; }

// Tiles of the expert-stationary kernels: their count, and tile t.
__device__ __forceinline__ int es_tile_count(const ExpertArgs& a) {
  return a.es_ntiles > 0 ? a.es_ntiles : ld_const(&a.plan->n_tiles_routed);
}
__device__ __forceinline__ Tile es_tile(const ExpertArgs& a, int t) {
  if (a.es_ntiles > 0) {
    Tile tl;
    tl.expert = a.E;
    tl.row0 = t * kEsTileRows;
    tl.rows = min(kEsTileRows, a.T - tl.row0);
    tl.pad = 0;
    return tl;
  }
  return ld_tile(a.tiles + t);
}

// Packed tokens of every routed tile: 16-byte chunk (tile t, token block tb,
// k block kb, k-step s, lane l) = x[token of row 32 tb + l % 32][64 kb + 16 s
// + 8 (l / 32) .. + 7]; rows past the tile's end take its first token (their
// results are never stored).  Blocks with no token of the tile are skipped.
__global__ __launch_bounds__(256) void k_pack_tokens_es(ExpertArgs a) {
  const int ntr = es_tile_count(a);
  const bool sh = a.es_ntiles > 0;
  const int C = a.D / kPK;
  const long per_tile = long(kEsTokBlocks) * C * 256;
  const long total = long(ntr) * per_tile;
  for (long q = long(blockIdx.x) * blockDim.x + threadIdx.x; q < total; q += long(gridDim.x) * blockDim.x) {
    const int t = int(q / per_tile);
    const long rem = q - long(t) * per_tile;
    const int tb = int(rem / (long(C) * 256));
    const int kb = int((rem >> 8) % C);
    const int w = int(rem & 255), s = w >> 6, l = w & 63;
    const Tile tl = es_tile(a, t);
    if (32 * tb >= tl.rows) continue;
    const int r = 32 * tb + (l & 31);
    const int row = tl.row0 + (r < tl.rows ? r : 0);
    const int tok = sh ? row : a.perm_token[row];
    const u16* src = static_cast<const u16*>(a.x) + size_t(tok) * a.D + 64 * kb + 16 * s + 8 * (l >> 5);
    u16* dst = a.xpk + size_t(t) * es_tile_elems(a.D) + (size_t(tb) * C + kb) * kPackBlock + 512 * s + 8 * l;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

struct EsGateUpProv {
  const u16* wg;   // packed gate matrix of the expert, at row block 2 nb
  const u16* wu;
  const u16* xt;   // packed tokens of the tile
  int C;
  __device__ int chunks() const { return C; }
  __device__ const u16* wbase(int bb) const {
    return (bb < 2 ? wg : wu) + size_t(bb & 1) * C * kPackBlock;
  }
  __device__ uint32_t wslice(int c) const { return uint32_t(c) * kPackBlock; }
  __device__ const u16* xbase() const { return xt; }
};

// Items: (tile, block of 64 intermediate rows), tile-major, handed out in
// order by a work counter (ItemQueue).  A static split gives each XCD one
// expert's tile, and tiles differ in height (a 290-row tile puts three
// 32-token blocks on some waves, a 256-row one two), so the XCDs with the
// tallest tiles finished last (Mixtral-shaped T = 2048 on MI355X: 551 -> 515
// us with the counter, 550 with per-XCD counters that steal once their
// part is done).  Weight blocks 0, 1 are
// gate rows 64 nb .. 64 nb + 63, blocks 2, 3 the same up rows: a lane holds
// gate and up of the same element, and SwiGLU is applied in registers.  h is
// written in the packed layout of the down product's token operand.
// Rows of the expert-stationary products: the routed experts' I, or the
// fused shared experts' S Is.
__device__ __forceinline__ int es_rows(const ExpertArgs& a) { return a.es_ntiles > 0 ? a.S * a.Is : a.I; }

// One item of the expert-stationary gate/up (item < tiles x es_rows / 64).
__device__ __forceinline__ void es_gate_up_item(const ExpertArgs& a, EsSmem& sm, long item) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool sh = a.es_ntiles > 0;
  const int Iv = es_rows(a);
  const int nbk = Iv / 64;
  const int C = a.D / kPK, CI = Iv / kPK;
  {
    const int t = int(item / nbk), nb = int(item - long(t) * nbk);
    const Tile tl = es_tile(a, t);
    EsGateUpProv pv;
    pv.C = C;
    const size_t ebase = sh ? 0 : size_t(tl.expert) * a.I * a.D;
    pv.wg = (sh ? a.psg : a.pg) + ebase + size_t(2 * nb) * C * kPackBlock;
    pv.wu = (sh ? a.psu : a.pu) + ebase + size_t(2 * nb) * C * kPackBlock;
    pv.xt = a.xpk + size_t(t) * es_tile_elems(a.D);
    const int nbt = (tl.rows + 31) / 32;
    f32x16 acc[kEsWBlocks][kEsWaveBlocks];
    es_accumulate(pv, sm, acc, nbt);
    u16* ht = a.hpk + size_t(t) * es_tile_elems(Iv);
#pragma unroll
    for (int j = 0; j < kEsWaveBlocks; ++j) {
      const int tb = es_token_block(wave, j, nbt);
      if (tb >= nbt) continue;   // wave-uniform
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (j == 2 && !es_block_valid(wave, b, nbt)) continue;   // (up block b + 2: same parity)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& g = acc[b][j];
          const f32x16& u = acc[b + 2][j];
          ushort4 hv;
          hv.x = f32_to_bf16(silu_f32(g[4 * q + 0]) * u[4 * q + 0]);
          hv.y = f32_to_bf16(silu_f32(g[4 * q + 1]) * u[4 * q + 1]);
          hv.z = f32_to_bf16(silu_f32(g[4 * q + 2]) * u[4 * q + 2]);
          hv.w = f32_to_bf16(silu_f32(g[4 * q + 3]) * u[4 * q + 3]);
          // element (token 32 tb + lane % 32, k = 64 nb + 32 b + 8 q + 4 (lane / 32) .. + 3)
          const int s2 = 2 * b + (q >> 1), l2 = (lane & 31) + 32 * (q & 1);
          *reinterpret_cast<ushort4*>(ht + (size_t(tb) * CI + nb) * kPackBlock + 512 * s2 + 8 * l2 +
                                      4 * (lane >> 5)) = hv;
        }
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_gate_up_es(ExpertArgs a) {
  __shared__ EsSmem sm;
  const long total = long(es_tile_count(a)) * (es_rows(a) / 64);
  __shared__ int qslot[2];
  ItemQueue q(const_cast<int32_t*>(&a.plan->gate_up_next), qslot);
  for (long item = blockIdx.x; item < total; item = q.next()) {
    q.claim();
    es_gate_up_item(a, sm, item);
  }
}

struct EsDownProv {
  const u16* wd;   // packed down matrix of the expert (of the first shared expert), at row
                   // block 4 db (D % 128 == 0)
  const u16* ht;
  int CI;          // k slices
  int cps;         // k slices per packed matrix: CI, or Is / 64 for the shared experts,
                   // whose k range runs through one packed [D][Is] matrix per expert
  size_t seg;      // elements per packed matrix
  __device__ int chunks() const { return CI; }
  __device__ const u16* wbase(int bb) const { return wd + size_t(bb) * cps * kPackBlock; }
  __device__ uint32_t wslice(int c) const {
    const int sg = c / cps;
    return uint32_t(size_t(sg) * seg + size_t(c - sg * cps) * kPackBlock);
  }
  __device__ const u16* xbase() const { return ht; }
};

// Items: (tile, block of 128 output rows), tile-major.  O rows are written
// in pair order for the combine (shared experts: O_shared rows in token
// order).
// One item of the expert-stationary down product (item < tiles x D / 128).
__device__ __forceinline__ void es_down_item(const ExpertArgs& a, EsSmem& sm, long item) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool sh = a.es_ntiles > 0;
  const int Iv = es_rows(a);
  const int ndb = a.D / 128;
  const int CI = Iv / kPK;
  {
    const int t = int(item / ndb), db = int(item - long(t) * ndb);
    const Tile tl = es_tile(a, t);
    EsDownProv pv;
    pv.CI = CI;
    pv.cps = sh ? a.Is / kPK : CI;
    pv.seg = size_t(a.D) * (sh ? a.Is : a.I);
    pv.wd = sh ? a.psd + size_t(4 * db) * pv.cps * kPackBlock
               : a.pd + size_t(tl.expert) * a.D * a.I + size_t(4 * db) * CI * kPackBlock;
    pv.ht = a.hpk + size_t(t) * es_tile_elems(Iv);
    const int nbt = (tl.rows + 31) / 32;
    f32x16 acc[kEsWBlocks][kEsWaveBlocks];
    es_accumulate(pv, sm, acc, nbt);
    u16* ob = static_cast<u16*>(sh ? a.o_sh : a.o);
#pragma unroll
    for (int j = 0; j < kEsWaveBlocks; ++j) {
      const int m = 32 * es_token_block(wave, j, nbt) + (lane & 31);
      if (m >= tl.rows) continue;
#pragma unroll
      for (int b = 0; b < kEsWBlocks; ++b) {
        if (j == 2 && !es_block_valid(wave, b, nbt)) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = 128 * db + 32 * b + 8 * q + 4 * (lane >> 5);
          const f32x16& v = acc[b][j];
          st4_bf16(ob, size_t(tl.row0 + m) * a.D + d, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_down_es(ExpertArgs a) {
  __shared__ EsSmem sm;
  const long total = long(es_tile_count(a)) * (a.D / 128);
  for (XcdRange it = xcd_range(total); it.next < it.end; it.next += it.step) es_down_item(a, sm, it.next);
}

// Layers whose shared experts run expert-stationary (es_ntiles > 0): one
// launch per product takes the fused shared expert's items (expert-stationary
// engine: MFMA- and L2-heavy) and the routed tiles' items (128-row packed
// engine: a few tokens per expert, weight streaming) from one work counter,
// so that the two kinds run side by side.  Run as two launches, the routed
// gate/up alone took 136 us and the shared one 102 us on the
// DeepSeek-V2-Lite prefill layer at T = 4096, against 208 us for the launch
// that took both on the packed engine.  Item order, measured on that layer
// (gate/up / down us): the kinds alternating 206 / 132, shared first 224 /
// 109, routed first 220 / 159; the gate/up kernel alternates, the down
// kernel (176 long shared items for 256 CUs) takes the shared ones first.
union MixedSmem {
  EsSmem es;
  PrefillSmem<128> pk;
};

// Item i: *shared = is a shared item; returns its index among its kind (ns
// shared items, nr routed ones), the kinds alternating while both last, or
// the shared ones first.
__device__ __forceinline__ long mixed_item(long i, long ns, long nr, bool alternate, bool* shared) {
  if (!alternate) {
    *shared = i < ns;
    return i < ns ? i : i - ns;
  }
  const long m = min(ns, nr);
  if (i < 2 * m) {
    *shared = (i & 1) == 0;
    return i >> 1;
  }
  *shared = ns > nr;
  return m + (i - 2 * m);
}

__global__ __launch_bounds__(256, 1) void k_gate_up_mixed(ExpertArgs a) {
  __shared__ MixedSmem sm;
  const long ns = long(a.es_ntiles) * (a.S * a.Is / 64);
  const int ntr = ld_const(&a.plan->n_tiles_routed);
  const int nbr = (a.I + kPackedIB - 1) / kPackedIB;
  const long nr = long(ntr) * nbr;
  __shared__ int qslot[2];
  ItemQueue q(const_cast<int32_t*>(&a.plan->gate_up_next), qslot);
  for (long item = blockIdx.x; item < ns + nr; item = q.next()) {
    q.claim();
    bool shared;
    const long j = mixed_item(item, ns, nr, true, &shared);
    if (shared) es_gate_up_item(a, sm.es, j);   // workgroup-uniform
    else packed_gate_up_item(a, sm.pk, j, ntr, 0, nbr, 1);
  }
}

__global__ __launch_bounds__(256, 1) void k_down_mixed(ExpertArgs a) {
  __shared__ MixedSmem sm;
  const long ns = long(a.es_ntiles) * (a.D / 128);
  const int ntr = ld_const(&a.plan->n_tiles_routed);
  const int nb_all = (a.D + kPackedDB - 1) / kPackedDB;
  const long nr = long(ntr) * nb_all;
  __shared__ int qslot[2];
  ItemQueue q(const_cast<int32_t*>(&a.plan->down_next), qslot);
  for (long item = blockIdx.x; item < ns + nr; item = q.next()) {
    q.claim();
    bool shared;
    const long j = mixed_item(item, ns, nr, false, &shared);
    if (shared) es_down_item(a, sm.es, j);
    else packed_down_item(a, sm.pk, j, ntr, 0, nb_all, 1);
  }
}

// ---------------------------------------------------------------------------
// fp32 layers: plain SIMT products over the same tiles (16 rows per tile).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_gate_up_f32(ExpertArgs a) {
  const int ntr = a.plan->n_tiles_routed, nts = a.plan->n_tiles_shared;
  const int nbr = a.I / 16, nbs = a.S > 0 ? (a.S * a.Is) / 16 : 1;
  const long total = long(ntr) * nbr + long(nts) * nbs;
  const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    int ti, nb;
    bool shared;
    work_item(w, ntr, nts, nbr, nbs, ti, nb, shared);
    const Tile tl = a.tiles[ti];
    if (r >= tl.rows) continue;
    const int Iv = shared ? a.S * a.Is : a.I;
    const float* wg = shared ? (const float*)a.sg : (const float*)a.wg + size_t(tl.expert) * a.I * a.D;
    const float* wu = shared ? (const float*)a.su : (const float*)a.wu + size_t(tl.expert) * a.I * a.D;
    const int t = shared ? tl.row0 + r : a.perm_token[tl.row0 + r];
    const float* xr = (const float*)a.x + size_t(t) * a.D;
    const int n = nb * 16 + c;
    const float* g_row = wg + size_t(n) * a.D;
    const float* u_row = wu + size_t(n) * a.D;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < a.D; ++k) {
      g = fmaf(xr[k], g_row[k], g);
      u = fmaf(xr[k], u_row[k], u);
    }
    float* hb = shared ? (float*)a.h_sh : (float*)a.h;
    hb[size_t(tl.row0 + r) * Iv + n] = silu_f32(g) * u;
  }
}

__global__ __launch_bounds__(256) void k_down_f32(ExpertArgs a) {
  const int ntr = a.plan->n_tiles_routed, nts = a.plan->n_tiles_shared;
  const int nb_all = (a.D + 15) / 16;
  const long total = long(ntr + nts) * nb_all;
  const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    int ti, nb;
    down_item(w, ntr, nts, nb_all, ti, nb);
    const bool shared = ti >= ntr;
    const Tile tl = a.tiles[ti];
    const int d = nb * 16 + c;
    if (r >= tl.rows || d >= a.D) continue;
    float s = 0.f;
    if (shared) {
      const int hs = a.S * a.Is;
      const float* hr = (const float*)a.h_sh + size_t(tl.row0 + r) * hs;
      for (int sx = 0; sx < a.S; ++sx) {
        const float* wrow = (const float*)a.sd + size_t(sx) * a.D * a.Is + size_t(d) * a.Is;
        for (int i = 0; i < a.Is; ++i) s = fmaf(hr[sx * a.Is + i], wrow[i], s);
      }
      static_cast<float*>(a.o_sh)[size_t(tl.row0 + r) * a.D + d] = s;
    } else {
      const float* hr = (const float*)a.h + size_t(tl.row0 + r) * a.I;
      const float* wrow = (const float*)a.wd + size_t(tl.expert) * a.D * a.I + size_t(d) * a.I;
      for (int i = 0; i < a.I; ++i) s = fmaf(hr[i], wrow[i], s);
      static_cast<float*>(a.o)[size_t(tl.row0 + r) * a.D + d] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_{k=0}^{K-1} g_hat[t][k] O[slot_pos[t][k]] + O_shared[t],
// accumulated in fp32 in slot order, rounded once.  O is stored in the
// layer's dtype (bf16 layers: each expert output rounded to bf16 once, which
// halves its write and read traffic).  A token with no surviving
// pair and no shared expert gets exactly 0.
// ---------------------------------------------------------------------------

// The slots of a token are walked in chunks of KC: the O rows of a chunk are
// loaded together (absent entries read row 0, a valid address), then added in
// slot order; a select, not a product with 0, drops the absent ones, so the
// sums are those of the plain slot loop.  With COMPACT the kept slots
// (slot_pos >= 0) are first gathered, in slot order, at the front of the LDS
// list and only those are walked; without it all K slots are.  Small batches
// take KC > 1 (one load per slot in turn would wait out a memory latency per
// kept slot): all K slots in one chunk when K <= 8, else the kept ones four at
// a time.  Large batches take the kept slots one at a time (many resident
// workgroups hide the latency, and padded loads would cost bandwidth).
// Split down products (plan-dependent, see down_split): each O row is the
// sum of the fp32 partials of the splits, added in split order.
struct CombineSplit {
  const Plan* plan;        // null: the down product is never split
  int slots, nb_all;       // as passed to the down kernel
  const float* op;
  const float* op_sh;
  long op_stride, op_sh_stride;
};

__device__ __forceinline__ float4 split_row4(const float* base, long stride, int ks, size_t e) {
  float4 v = *reinterpret_cast<const float4*>(base + e);
  for (int q = 1; q < ks; ++q) {
    const float4 w = *reinterpret_cast<const float4*>(base + q * stride + e);
    v.x += w.x;
    v.y += w.y;
    v.z += w.z;
    v.w += w.w;
  }
  return v;
}

template <bool BF16, int KC, bool COMPACT>
__global__ __launch_bounds__(256) void k_combine(int T, int D, int K, const float* __restrict__ gates,
                                                 const int32_t* __restrict__ slot_pos,
                                                 const void* __restrict__ o,
                                                 const void* __restrict__ o_sh, void* __restrict__ y,
                                                 CombineSplit cs) {
  __shared__ float s_g[32];
  __shared__ int32_t s_p[32];
  __shared__ int s_n;
  const int t = blockIdx.x;
  int ks = 1;
  if (cs.plan) {
    const int ntr = ld_const(&cs.plan->n_tiles_routed), nts = ld_const(&cs.plan->n_tiles_shared);
    ks = down_split(long(ntr + nts) * cs.nb_all, cs.slots);
  }
  if (threadIdx.x < 32) {   // wave 0
    const int l = threadIdx.x;
    const bool in = l < K;
    const int32_t pl = in ? slot_pos[size_t(t) * K + l] : -1;
    const float gl = in ? gates[size_t(t) * K + l] : 0.f;
    if (COMPACT) {
      const uint64_t kept = __ballot(pl >= 0);
      s_p[l] = -1;
      if (pl >= 0) {
        const int r = __popcll(kept & ((1ull << l) - 1ull));
        s_p[r] = pl;
        s_g[r] = gl;
      }
      if (l == 0) s_n = __popcll(kept);
    } else {
      s_p[l] = pl;
      s_g[l] = gl;
    }
  }
  __syncthreads();
  const int nk = COMPACT ? s_n : K;
  if (ks > 1) {   // fp32 partial sums of a split down product, slot by slot
    for (int d = threadIdx.x * 4; d < D; d += blockDim.x * 4) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < nk; ++k) {
        const int pk = s_p[k];
        if (pk < 0) continue;
        const float g = s_g[k];
        const float4 v = split_row4(cs.op, cs.op_stride, ks, size_t(pk) * D + d);
        acc.x += g * v.x;
        acc.y += g * v.y;
        acc.z += g * v.z;
        acc.w += g * v.w;
      }
      if (o_sh) {
        const float4 sh = split_row4(cs.op_sh, cs.op_sh_stride, ks, size_t(t) * D + d);
        acc.x += sh.x;
        acc.y += sh.y;
        acc.z += sh.z;
        acc.w += sh.w;
      }
      if (BF16) st4_bf16(static_cast<u16*>(y), size_t(t) * D + d, acc.x, acc.y, acc.z, acc.w);
      else *reinterpret_cast<float4*>((float*)y + size_t(t) * D + d) = acc;
    }
    return;
  }
  for (int d = threadIdx.x * 4; d < D; d += blockDim.x * 4) {
    float4 sh = make_float4(0.f, 0.f, 0.f, 0.f);
    if (o_sh) sh = ld4_f32<BF16>(o_sh, size_t(t) * D + d);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < nk; k0 += KC) {
      float4 v[KC];
      int pk[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        pk[j] = s_p[k0 + j];
        v[j] = ld4_f32<BF16>(o, size_t(pk[j] < 0 ? 0 : pk[j]) * D + d);
      }
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const float g = s_g[k0 + j];
        const bool on = pk[j] >= 0;
        acc.x = on ? acc.x + g * v[j].x : acc.x;
        acc.y = on ? acc.y + g * v[j].y : acc.y;
        acc.z = on ? acc.z + g * v[j].z : acc.z;
        acc.w = on ? acc.w + g * v[j].w : acc.w;
      }
    }
    if (o_sh) {
      acc.x += sh.x;
      acc.y += sh.y;
      acc.z += sh.z;
      acc.w += sh.w;
    }
    if (BF16) {
      st4_bf16(static_cast<u16*>(y), size_t(t) * D + d, acc.x, acc.y, acc.z, acc.w);
    } else {
      *reinterpret_cast<float4*>((float*)y + size_t(t) * D + d) = acc;
    }
  }
}

// Large bf16 batches: one wave per token
// (each workgroup's four waves take tokens 4 b + w, then a grid stride),
// lane l holding outputs 8 l .. 8 l + 7 of each 512-wide pass, so that every
// kept slot's row is read with one 16-byte load per pass, all P passes in
// flight at once (SPLIT: the down product may have split k; then the fp32
// partials of the splits, added in split order).  The sum is the same as
// k_combine's: fp32, kept slots in slot order, the shared output last, one
// rounding.  Against k_combine (one workgroup per token) on MI355X: 14.5 ->
// 12.0 us on the DeepSeek-V2-Lite prefill batch (T = 4096), 24.7 -> 22.0 on
// the fine-grained T = 8192 one, 10.3 -> 9.9 on the Mixtral-shaped T = 2048
// one.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int P, bool SPLIT>
__global__ __launch_bounds__(256) void k_combine_tok(int T, int D, int K, const float* __restrict__ gates,
                                                     const int32_t* __restrict__ slot_pos,
                                                     const u16* __restrict__ o, const u16* __restrict__ o_sh,
                                                     u16* __restrict__ y, CombineSplit cs) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int ks = 1;
  if constexpr (SPLIT) {   // the down product may have split k
    const int ntr = ld_const(&cs.plan->n_tiles_routed), nts = ld_const(&cs.plan->n_tiles_shared);
    ks = down_split(long(ntr + nts) * cs.nb_all, cs.slots);
  }
  for (int t = blockIdx.x * 4 + wave; t < T; t += gridDim.x * 4) {
    int32_t pl = -1;
    float gl = 0.f;
    if (lane < K) {
      pl = slot_pos[size_t(t) * K + lane];
      gl = gates[size_t(t) * K + lane];
    }
    uint64_t kept = __ballot(pl >= 0);
    float acc[P][8];
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[q][i] = 0.f;
    while (kept) {   // wave-uniform
      const int k = __ffsll(static_cast<unsigned long long>(kept)) - 1;
      kept &= kept - 1;
      const int p = __shfl(pl, k);
      const float g = __shfl(gl, k);
      if (SPLIT && ks > 1) {   // wave-uniform
#pragma unroll
        for (int q = 0; q < P; ++q) {
          const int d = 512 * q + 8 * lane;
          if (d < D) {
            const float4 a = split_row4(cs.op, cs.op_stride, ks, size_t(p) * D + d);
            const float4 b = split_row4(cs.op, cs.op_stride, ks, size_t(p) * D + d + 4);
            acc[q][0] += g * a.x;
            acc[q][1] += g * a.y;
            acc[q][2] += g * a.z;
            acc[q][3] += g * a.w;
            acc[q][4] += g * b.x;
            acc[q][5] += g * b.y;
            acc[q][6] += g * b.z;
            acc[q][7] += g * b.w;
          }
        }
        continue;
      }
      u32x4 v[P];
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int d = 512 * q + 8 * lane;
        v[q] = d < D ? ld16(o + size_t(p) * D + d) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < P; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[q][2 * i] += g * bf16_lo(v[q][i]);
          acc[q][2 * i + 1] += g * bf16_hi(v[q][i]);
        }
    }
    if (SPLIT && o_sh && ks > 1) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int d = 512 * q + 8 * lane;
        if (d < D) {
          const float4 a = split_row4(cs.op_sh, cs.op_sh_stride, ks, size_t(t) * D + d);
          const float4 b = split_row4(cs.op_sh, cs.op_sh_stride, ks, size_t(t) * D + d + 4);
          acc[q][0] += a.x;
          acc[q][1] += a.y;
          acc[q][2] += a.z;
          acc[q][3] += a.w;
          acc[q][4] += b.x;
          acc[q][5] += b.y;
          acc[q][6] += b.z;
          acc[q][7] += b.w;
        }
      }
    } else if (o_sh) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int d = 512 * q + 8 * lane;
        if (d < D) {
          const u32x4 v = ld16(o_sh + size_t(t) * D + d);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[q][2 * i] += bf16_lo(v[i]);
            acc[q][2 * i + 1] += bf16_hi(v[i]);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int d = 512 * q + 8 * lane;
      if (d < D) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r[i] = uint32_t(f32_to_bf16(acc[q][2 * i])) | (uint32_t(f32_to_bf16(acc[q][2 * i + 1])) << 16);
        *reinterpret_cast<u32x4*>(y + size_t(t) * D + d) = r;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Single-token batches: the down product and the combine in one launch.
//
// With one token every expert's down product is a matrix-vector product, so
// a workgroup takes kDcRows output rows and every segment of the token --
// its kept slots in slot order, then the shared experts -- one segment per
// wave: the wave streams the segment's kDcRows weight rows and its h row
// with all loads in flight at once, and takes the kDcRows dot products with
// fp32 sums and fixed-order wave reductions.  The dots meet in LDS, and one
// wave adds them per row in segment order, each kept slot times its gate
// (y = sum_k g_k (W_k h_k) + sum_s Ws_s h_s), rounding y once.  Against the
// streaming down kernel and the combine (O stored in bf16 between them) the
// result differs only by that rounding.  Segments of at most kDcMaxChunks
// 16-byte chunks per lane (intermediate sizes up to 2048 for bf16 weights,
// 4096 for FP8 ones).
// ---------------------------------------------------------------------------

constexpr int kDcRows = 4;         // output rows per workgroup (DeepSeek-V2-Lite shapes, step
                                   // us on MI355X: 2 rows 31.9, 4 rows 30.6, 8 rows 31.5, 16 rows 37.3)
constexpr int kDcWaves = 8;        // waves per workgroup: segments taken per round
constexpr int kDcMaxChunks = 4;    // 16-byte chunks of a segment row per lane
constexpr int kDcMaxShared = 8;
constexpr int kDcMaxSeg = 32 + kDcMaxShared;

struct DownCombineArgs {
  const void* wd;      // [E][D][I]: bf16, or E4M3 codes
  const void* sd;      // [S][D][Is]
  const float* qd;     // FP8: scale of each output row [E][D] (else null)
  const float* qsd;    // FP8: [S][D]
  const u16* h;        // [P][I], pair order
  const u16* h_sh;     // [1][S Is]
  const int32_t* slot_pos;
  const float* gates;
  const int32_t* idx;
  u16* y;
  int D, I, Is, S, K;
};

// Weight elements per 16-byte chunk.
template <bool F8>
constexpr int dc_chunk() { return F8 ? 16 : 8; }

bool down_combine_fused(const beam_moe_layer& L, int32_t T) {
  const bool f8 = L.expert_format == BEAM_WEIGHTS_FP8_E4M3;
  const long rows_max = long(kWave) * kDcMaxChunks * (f8 ? 16 : 8);
  return T == 1 && L.dtype == BEAM_BF16 && L.I <= rows_max && L.n_shared <= kDcMaxShared &&
         (L.n_shared == 0 || L.I_shared <= rows_max) && L.K <= 32 && L.D % kDcRows == 0;
}

// FP8: a chunk holds 16 codes, widened exactly to bf16 in registers; each
// weight row's dot is multiplied by the row's scale before it leaves the wave.
template <bool F8, int NJ>   // NJ: 16-byte chunks per lane of the longest segment row
__global__ __launch_bounds__(kDcWaves * 64) void k_down_combine_t1(DownCombineArgs a) {
  constexpr int CK = dc_chunk<F8>();
  constexpr int HL = F8 ? 2 : 1;   // 16-byte loads of h per chunk
  __shared__ float s_dot[kDcMaxSeg][kDcRows];
  __shared__ float s_gate[kDcMaxSeg];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d0 = blockIdx.x * kDcRows;
  // the token's slots, lane k < K: pair position (-1: masked), gate, expert
  int pos = -1, ex = 0;
  float gt = 0.f;
  if (lane < a.K) {
    pos = a.slot_pos[lane];
    gt = a.gates[lane];
    ex = a.idx[lane];
  }
  const unsigned long long kept = __ballot(pos >= 0);
  const int nk = __popcll(kept);
  const int nseg = nk + a.S;
  const int rank = __popcll(kept & ((1ull << lane) - 1ull));
  for (int q = wave; q < nseg; q += kDcWaves) {   // wave-uniform
    const unsigned char* w;
    const u16* hr;
    const float* sc = nullptr;   // FP8: scales of this segment's rows d0 ..
    int len;
    float gq = 1.f;
    if (q < nk) {   // the q-th kept slot
      const unsigned long long sel = __ballot(((kept >> lane) & 1ull) && rank == q);
      const int k = __ffsll(static_cast<unsigned long long>(sel)) - 1;
      const int ek = __builtin_amdgcn_readlane(ex, k);
      const int pk = __builtin_amdgcn_readlane(pos, k);
      gq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gt), k));
      w = static_cast<const unsigned char*>(a.wd) + (size_t(ek) * a.D + d0) * a.I * (F8 ? 1 : 2);
      hr = a.h + size_t(pk) * a.I;
      if (F8) sc = a.qd + size_t(ek) * a.D + d0;
      len = a.I;
    } else {        // shared expert q - nk
      const int sx = q - nk;
      w = static_cast<const unsigned char*>(a.sd) + (size_t(sx) * a.D + d0) * a.Is * (F8 ? 1 : 2);
      hr = a.h_sh + size_t(sx) * a.Is;
      if (F8) sc = a.qsd + size_t(sx) * a.D + d0;
      len = a.Is;
    }
    const size_t row_bytes = size_t(len) * (F8 ? 1 : 2);
    const int nch = len / CK;
    u32x4 hv[NJ][HL], wv[kDcRows][NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {   // every load issued before any use
      const int c = lane + kWave * j;
      const int cc = c < nch ? c : 0;
#pragma unroll
      for (int u = 0; u < HL; ++u) hv[j][u] = ld16(hr + size_t(cc) * CK + 8 * u);
#pragma unroll
      for (int r = 0; r < kDcRows; ++r) wv[r][j] = ld16_stream(w + r * row_bytes + size_t(cc) * 16);
    }
    float dot[kDcRows];
#pragma unroll
    for (int r = 0; r < kDcRows; ++r) dot[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (lane + kWave * j >= nch) continue;   // chunk past the row: no contribution
#pragma unroll
      for (int u = 0; u < HL; ++u)
#pragma unroll
        for (int r = 0; r < kDcRows; ++r) {
          // this chunk's 8 weights that meet h values 8u .. 8u + 7, as bf16
          const u32x4 wb = F8 ? e4m3x8_to_bf16(wv[r][j][2 * u], wv[r][j][2 * u + 1]) : wv[r][j];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float h0 = __uint_as_float(hv[j][u][i] << 16);
            const float h1 = __uint_as_float(hv[j][u][i] & 0xffff0000u);
            dot[r] = fmaf(__uint_as_float(wb[i] << 16), h0, dot[r]);
            dot[r] = fmaf(__uint_as_float(wb[i] & 0xffff0000u), h1, dot[r]);
          }
        }
    }
#pragma unroll
    for (int r = 0; r < kDcRows; ++r) {
      float v = wave_sum_f32(dot[r]);
      if (F8) v *= sc[r];
      if (lane == 0) s_dot[q][r] = v;
    }
    if (lane == 0) s_gate[q] = gq;
  }
  __syncthreads();
  if (wave == 0 && lane < kDcRows) {
    float acc = 0.f;
    for (int q = 0; q < nk; ++q) acc += s_gate[q] * s_dot[q][lane];   // slot order
    float sh = 0.f;
    for (int q = nk; q < nseg; ++q) sh += s_dot[q][lane];
    a.y[d0 + lane] = f32_to_bf16(acc + sh);
  }
}

// Single-token batches, gate/up and SwiGLU (d_model up to 2048 with bf16
// weights, 4096 with FP8): each expert's gate and up products are
// matrix-vector products too. A workgroup takes one intermediate row of
// every segment -- the kept slots, then each shared expert -- one segment per
// wave: the wave issues the segment's gate and up rows and the token's x row
// at once (NJ 16-byte chunks per lane, no more than the row has), forms both
// dots in fp32 with fixed-order wave reductions, and writes h = silu(g) * u
// (rounded to bf16 once) where the down product reads it (pair order; the
// shared experts' [S Is] row). One row per workgroup measured fastest: at
// four rows a workgroup's registers left one workgroup resident per compute
// unit and the grid ran in two uneven waves; staging x in LDS once per
// workgroup did not help. FP8: a chunk holds 16 codes, widened exactly to
// bf16 in registers, and each dot is multiplied by its row's scale before
// SwiGLU.
struct GateUpT1Args {
  const void* wg;       // [E][I][D]: bf16, or E4M3 codes
  const void* wu;
  const void* sg;       // [S Is][D]
  const void* su;
  const float* qg;      // FP8: row scales [E][I] (else null)
  const float* qu;
  const float* qsg;     // FP8: [S Is]
  const float* qsu;
  const u16* x;
  const int32_t* slot_pos;
  const int32_t* idx;
  u16* h;               // [P][I]
  u16* h_sh;            // [1][S Is]
  int D, I, Is, S, K;
};

bool gate_up_t1(const beam_moe_layer& L, int32_t T) {
  const int ck = L.expert_format == BEAM_WEIGHTS_FP8_E4M3 ? 16 : 8;   // elements per chunk
  return down_combine_fused(L, T) && L.D % ck == 0 && L.D <= kWave * kDcMaxChunks * ck;
}

template <bool F8, int NJ>   // NJ: 16-byte chunks per lane of a row
__global__ __launch_bounds__(kDcWaves * 64) void k_gate_up_t1(GateUpT1Args a) {
  constexpr int CK = dc_chunk<F8>();
  constexpr int HL = F8 ? 2 : 1;   // 16-byte loads of x per chunk
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x;
  int pos = -1, ex = 0;
  if (lane < a.K) {
    pos = a.slot_pos[lane];
    ex = a.idx[lane];
  }
  const unsigned long long kept = __ballot(pos >= 0);
  const int nk = __popcll(kept);
  const int nseg = nk + a.S;
  const int rank = __popcll(kept & ((1ull << lane) - 1ull));
  const int nch = a.D / CK;
  const size_t row_bytes = size_t(a.D) * (F8 ? 1 : 2);
  for (int q = wave; q < nseg; q += kDcWaves) {   // wave-uniform
    size_t wrow;   // row of the segment's matrices
    const void* gm;
    const void* um;
    const float* qg;
    const float* qu;
    u16* hr;
    if (q < nk) {   // the q-th kept slot
      if (row >= a.I) continue;
      const unsigned long long sel = __ballot(((kept >> lane) & 1ull) && rank == q);
      const int k = __ffsll(static_cast<unsigned long long>(sel)) - 1;
      const int ek = __builtin_amdgcn_readlane(ex, k);
      const int pk = __builtin_amdgcn_readlane(pos, k);
      wrow = size_t(ek) * a.I + row;
      gm = a.wg;
      um = a.wu;
      qg = a.qg;
      qu = a.qu;
      hr = a.h + size_t(pk) * a.I + row;
    } else {        // shared expert q - nk: row sx Is + row of the fused matrices
      if (row >= a.Is) continue;
      wrow = size_t(q - nk) * a.Is + row;
      gm = a.sg;
      um = a.su;
      qg = a.qsg;
      qu = a.qsu;
      hr = a.h_sh + wrow;
    }
    const unsigned char* g = static_cast<const unsigned char*>(gm) + wrow * row_bytes;
    const unsigned char* u = static_cast<const unsigned char*>(um) + wrow * row_bytes;
    u32x4 xv[NJ][HL], gv[NJ], uv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {   // every load issued before any use
      const int c = lane + kWave * j;
      const size_t cc = size_t(c < nch ? c : 0);
#pragma unroll
      for (int v = 0; v < HL; ++v) xv[j][v] = ld16(a.x + cc * CK + 8 * v);
      gv[j] = ld16_stream(g + cc * 16);
      uv[j] = ld16_stream(u + cc * 16);
    }
    float dg = 0.f, du = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (lane + kWave * j >= nch) continue;   // chunk past the row: no contribution
#pragma unroll
      for (int v = 0; v < HL; ++v) {
        // this chunk's 8 weights that meet x values 8v .. 8v + 7, as bf16
        const u32x4 gb = F8 ? e4m3x8_to_bf16(gv[j][2 * v], gv[j][2 * v + 1]) : gv[j];
        const u32x4 ub = F8 ? e4m3x8_to_bf16(uv[j][2 * v], uv[j][2 * v + 1]) : uv[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = __uint_as_float(xv[j][v][i] << 16), x1 = __uint_as_float(xv[j][v][i] & 0xffff0000u);
          dg = fmaf(__uint_as_float(gb[i] << 16), x0, dg);
          dg = fmaf(__uint_as_float(gb[i] & 0xffff0000u), x1, dg);
          du = fmaf(__uint_as_float(ub[i] << 16), x0, du);
          du = fmaf(__uint_as_float(ub[i] & 0xffff0000u), x1, du);
        }
      }
    }
    float gs = wave_sum_f32(dg), us = wave_sum_f32(du);
    if (F8) {
      gs *= qg[wrow];
      us *= qu[wrow];
    }
    if (lane == 0) *hr = f32_to_bf16(silu_f32(gs) * us);
  }
}

hipError_t launch_gate_up_t1(const beam_moe_layer& L, const void* x, const Ptrs& p, hipStream_t s) {
  GateUpT1Args a;
  a.wg = L.w_gate;
  a.wu = L.w_up;
  a.sg = L.ws_gate;
  a.su = L.ws_up;
  a.qg = L.scale_gate;
  a.qu = L.scale_up;
  a.qsg = L.scale_shared_gate;
  a.qsu = L.scale_shared_up;
  a.x = static_cast<const u16*>(x);
  a.slot_pos = p.slot_pos;
  a.idx = p.idx;
  a.h = static_cast<u16*>(p.h);
  a.h_sh = static_cast<u16*>(p.h_shared);
  a.D = L.D;
  a.I = L.I;
  a.Is = L.I_shared;
  a.S = L.n_shared;
  a.K = L.K;
  const bool f8 = L.expert_format == BEAM_WEIGHTS_FP8_E4M3;
  const int nj = (L.D / (f8 ? 16 : 8) + kWave - 1) / kWave;   // 1 .. kDcMaxChunks
  const dim3 grid(unsigned(std::max(L.I, L.n_shared > 0 ? L.I_shared : 0))), block(kDcWaves * 64);
  auto go = [&](auto k1, auto k2, auto k3, auto k4) {
    if (nj <= 1) hipLaunchKernelGGL(k1, grid, block, 0, s, a);
    else if (nj == 2) hipLaunchKernelGGL(k2, grid, block, 0, s, a);
    else if (nj == 3) hipLaunchKernelGGL(k3, grid, block, 0, s, a);
    else hipLaunchKernelGGL(k4, grid, block, 0, s, a);
  };
  if (f8) {
    prof_before("gate_up_swiglu_t1_fp8", s);
    go(k_gate_up_t1<true, 1>, k_gate_up_t1<true, 2>, k_gate_up_t1<true, 3>, k_gate_up_t1<true, 4>);
  } else {
    prof_before("gate_up_swiglu_t1", s);
    go(k_gate_up_t1<false, 1>, k_gate_up_t1<false, 2>, k_gate_up_t1<false, 3>, k_gate_up_t1<false, 4>);
  }
  prof_after(s);
  return hipGetLastError();
}

hipError_t launch_down_combine_t1(const beam_moe_layer& L, const Ptrs& p, void* y, hipStream_t s) {
  DownCombineArgs a;
  a.wd = L.w_down;
  a.sd = L.ws_down;
  a.qd = L.scale_down;
  a.qsd = L.scale_shared_down;
  a.h = static_cast<const u16*>(p.h);
  a.h_sh = static_cast<const u16*>(p.h_shared);
  a.slot_pos = p.slot_pos;
  a.gates = p.gates;
  a.idx = p.idx;
  a.y = static_cast<u16*>(y);
  a.D = L.D;
  a.I = L.I;
  a.Is = L.I_shared;
  a.S = L.n_shared;
  a.K = L.K;
  const dim3 grid(unsigned(L.D / kDcRows)), block(kDcWaves * 64);
  const bool f8 = L.expert_format == BEAM_WEIGHTS_FP8_E4M3;
  const int len = std::max(L.I, L.n_shared > 0 ? L.I_shared : 0);
  const int nj = (len / (f8 ? 16 : 8) + kWave - 1) / kWave;   // 1 .. kDcMaxChunks
  auto go = [&](auto k1, auto k2, auto k3, auto k4) {
    if (nj <= 1) hipLaunchKernelGGL(k1, grid, block, 0, s, a);
    else if (nj == 2) hipLaunchKernelGGL(k2, grid, block, 0, s, a);
    else if (nj == 3) hipLaunchKernelGGL(k3, grid, block, 0, s, a);
    else hipLaunchKernelGGL(k4, grid, block, 0, s, a);
  };
  if (f8) {
    prof_before("down_combine_fp8", s);
    go(k_down_combine_t1<true, 1>, k_down_combine_t1<true, 2>, k_down_combine_t1<true, 3>,
       k_down_combine_t1<true, 4>);
  } else {
    prof_before("down_combine", s);
    go(k_down_combine_t1<false, 1>, k_down_combine_t1<false, 2>, k_down_combine_t1<false, 3>,
       k_down_combine_t1<false, 4>);
  }
  prof_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static ExpertArgs expert_args(const beam_moe_layer& L, const void* x, int32_t T, const Ptrs& p) {
  ExpertArgs a;
  a.x = x;
  a.wg = L.w_gate;
  a.wu = L.w_up;
  a.wd = L.w_down;
  a.sg = L.ws_gate;
  a.su = L.ws_up;
  a.sd = L.ws_down;
  a.qg = L.scale_gate;
  a.qu = L.scale_up;
  a.qd = L.scale_down;
  a.qsg = L.scale_shared_gate;
  a.qsu = L.scale_shared_up;
  a.qsd = L.scale_shared_down;
  a.pg = (const u16*)L.wp_gate;
  a.pu = (const u16*)L.wp_up;
  a.pd = (const u16*)L.wp_down;
  a.psg = (const u16*)L.wsp_gate;
  a.psu = (const u16*)L.wsp_up;
  a.psd = (const u16*)L.wsp_down;
  a.T = T;
  a.D = L.D;
  a.E = L.E;
  a.I = L.I;
  a.S = L.n_shared;
  a.Is = L.I_shared;
  a.plan = p.plan;
  a.tiles = p.tiles;
  a.perm_token = p.perm_token;
  a.expert_off = p.expert_off;
  a.tile_rows = 0;
  a.es_ntiles = 0;
  a.xpk = reinterpret_cast<u16*>(p.es_x);
  a.hpk = reinterpret_cast<u16*>(p.es_h);
  a.h = p.h;
  a.h_sh = p.h_shared;
  a.o = p.o;
  a.o_sh = p.o_shared;
  a.op = p.o_part;
  a.op_stride = long(T) * L.K * L.D;
  a.op_sh = p.o_part ? p.o_part + kMaxDownSplit * a.op_stride : nullptr;
  a.op_sh_stride = long(T) * L.D;
  a.down_slots = 0;
  return a;
}

// Persistent grid of the streaming kernels: as many workgroups as can be
// resident at once (occupancy x CUs, queried once per kernel and device).
constexpr long kStreamGrid = 512;   // a typical resident grid, for sizing choices only

// The variants below were chosen by timing on MI355X over the decode batch
// sizes of three layer shapes (d_model 1536 to 4096, d_ff 256 to 14336).
// Multi-tile problems stream two 16-row groups per item; k is split four ways
// only for d_model >= 4096 (gate/up) and two ways for d_ff >= 1024 (down).
// Single-tile (16-row) problems: the k split follows the chunks per item, so
// that each wave's share still holds several 64-wide chunks, and items carry
// two 16-row groups when that leaves at least two shares per wave of a full
// grid (fewer, longer items cost less per byte; too few would idle CUs).
static int stream_ksplit_chunks(int chunks) { return chunks >= 16 ? 4 : chunks >= 8 ? 2 : 1; }
constexpr long kWideShares = 2 * kStreamGrid * kStreamWaves;

// A multiple of 8, so that item i of the round-robin deal runs on XCD i % 8.
static unsigned stream_grid(const void* kernel, long items_bound, int ksplit) {
  const long groups = kStreamWaves / ksplit;
  const long cap = std::max<long>(8, resident_blocks(kernel, kStreamWaves * 64) / 8 * 8);
  const long want = ((items_bound + groups - 1) / groups + 7) / 8 * 8;
  return unsigned(std::max<long>(8, std::min<long>(cap, want)));
}

// Upper bound on the number of tiles the scan can produce.
static long tile_bound(const beam_moe_layer& L, int32_t T, int tile_rows, long* shared_tiles) {
  const long pairs = long(T) * L.K;
  const long routed = (pairs + tile_rows - 1) / tile_rows + std::min<long>(L.E, pairs);
  *shared_tiles = L.n_shared > 0 ? (T + tile_rows - 1) / tile_rows : 0;
  return routed;
}

// Persistent grid of the tiled kernels: resident workgroups, a multiple of 8.
static unsigned tiled_grid(const void* kernel, long items) {
  long cap = resident_blocks(kernel, 256);
  cap = std::max<long>(8, cap / 8 * 8);
  return unsigned(std::max<long>(1, std::min<long>(cap, items)));
}

static unsigned persistent_grid(long items, long cap) {
  long g = std::min(items, cap);
  return unsigned(std::max<long>(g, 1));
}

// Launches the streaming gate/up variant <MT token blocks, NB row groups,
// U-chunk stages, k split KS, FP8 weights?>.
template <int MT, int NB, int U, int KS, bool F8>
static void gate_up_stream_k(const ExpertArgs& a, long ntr, long nts, int I, int Is_all,
                             hipStream_t s) {
  const long items = ntr * (I / (16 * NB)) + nts * (Is_all / (16 * NB));
  hipLaunchKernelGGL((k_gate_up_stream<MT, NB, U, KS, F8>),
                     dim3(stream_grid((const void*)&k_gate_up_stream<MT, NB, U, KS, F8>, items, KS)),
                     dim3(kStreamWaves * 64), 0, s, a);
}

// The same with the k split ks (1, 2 or 4) chosen at run time.
template <int MT, int NB, int U, bool F8>
static void gate_up_stream(const ExpertArgs& a, long ntr, long nts, int I, int Is_all, int ks,
                           hipStream_t s) {
  if (ks == 1) gate_up_stream_k<MT, NB, U, 1, F8>(a, ntr, nts, I, Is_all, s);
  else if (ks == 2) gate_up_stream_k<MT, NB, U, 2, F8>(a, ntr, nts, I, Is_all, s);
  else gate_up_stream_k<MT, NB, U, 4, F8>(a, ntr, nts, I, Is_all, s);
}

template <int MT, int NB, int U, int KS, bool F8>
static void down_stream_k(const ExpertArgs& a, long tiles, int D, hipStream_t s) {
  const long items = tiles * (D / (16 * NB));
  hipLaunchKernelGGL((k_down_stream<MT, NB, U, KS, F8>),
                     dim3(stream_grid((const void*)&k_down_stream<MT, NB, U, KS, F8>, items, KS)),
                     dim3(kStreamWaves * 64), 0, s, a);
}

template <int MT, int NB, int U, bool F8>
static void down_stream(const ExpertArgs& a, long tiles, int D, int ks, hipStream_t s) {
  if (ks == 1) down_stream_k<MT, NB, U, 1, F8>(a, tiles, D, s);
  else if (ks == 2) down_stream_k<MT, NB, U, 2, F8>(a, tiles, D, s);
  else down_stream_k<MT, NB, U, 4, F8>(a, tiles, D, s);
}

// Routed 16-row tiles a batch of T tokens is expected to give, for choosing
// the streaming variant: the distinct experts that T x Avg-K pairs hit
// (E (1 - e^(-T Avg-K / E)), Avg-K from the descriptor's hint, K when
// unknown) plus one tile per 16 pairs, at most the bound ntr the grid is
// sized for.  The bound (one tile per expert up to T x K) overstates small
// batches of many experts: the fine-grained layer at T = 16 has about 37
// active experts against a bound of 228 tiles.
static long expected_routed_tiles(const beam_moe_layer& L, int T, long ntr) {
  const double pairs = double(T) * (L.expected_avg_k > 0.f ? L.expected_avg_k : float(L.K));
  const double expect = double(L.E) * (1.0 - std::exp(-pairs / L.E)) + std::floor(pairs / 16.0);
  return std::min<long>(ntr, long(std::ceil(expect)));
}

// Streaming launches for tiles of 16, 32 or 64 rows.  Weight chunks are 128
// bytes of a row in both formats, so the k split follows the chunk count.
template <bool F8>
static void gate_up_streaming(const beam_moe_layer& L, const ExpertArgs& a, long ntr, long nts,
                              int tile_rows, hipStream_t s) {
  const int Is_all = L.n_shared ? L.n_shared * L.I_shared : 0;
  const int chunks = L.D / chunk_k<F8>();
  if constexpr (F8) {
    // FP8 (half the bytes per item): 16-row tiles stream one row group per
    // item with the smallest k split that still gives about 3/4 of a share
    // per wave of a full grid; 32-row tiles four row groups on short rows,
    // else two with a 2-way split; 64-row tiles as bf16.
    if (tile_rows == 16) {
      // (expected tiles: T = 1, 12.6 -> 12.0 us with the 4-way split the
      // bound's 2-way choice missed)
      const long items1 = expected_routed_tiles(L, a.T, ntr) * (L.I / 16) + nts * (Is_all / 16);
      const long want = kStreamGrid * kStreamWaves * 3 / 4;
      const int ks = items1 >= want ? 1 : 2 * items1 >= want ? 2 : 4;
      gate_up_stream<1, 1, 1, F8>(a, ntr, nts, L.I, Is_all, ks, s);
      return;
    }
    if (tile_rows == 32) {
      // rows of fewer than 32 chunks: four row groups per item (DeepSeek-V2-Lite
      // shapes, T = 256: 91.5 -> 85.8 us on MI355X against two)
      if (chunks < 32) gate_up_stream_k<2, 4, 1, 1, F8>(a, ntr, nts, L.I, Is_all, s);
      else gate_up_stream<2, 2, 1, F8>(a, ntr, nts, L.I, Is_all, 2, s);
      return;
    }
  }
  if (tile_rows == 16) {
    const int ks = stream_ksplit_chunks(chunks);
    // Two row groups per item when the expected tiles give enough shares
    // (fine-grained layer, T = 16: one group 40.4 us per step on MI355X
    // against 42.3 with two, which the bound alone would pick), or when the
    // shares are long, at least 16 chunks per wave (Mixtral-shaped, T = 1:
    // 84.7 us against 85.3 with one).
    const long items2 = expected_routed_tiles(L, a.T, ntr) * (L.I / 32) + nts * (Is_all / 32);
    if (items2 * ks >= kWideShares || chunks / ks >= 16)
      gate_up_stream<1, 2, 1, F8>(a, ntr, nts, L.I, Is_all, ks, s);
    else gate_up_stream<1, 1, 1, F8>(a, ntr, nts, L.I, Is_all, ks, s);
  } else if (tile_rows == 32) {
    // rows of fewer than 64 chunks: four row groups per item and no k split,
    // as for the 64-row tiles below (DeepSeek-V2-Lite shapes, T = 256: gate/up
    // 144.7 -> 137.6 us on MI355X against two row groups and a 2-way split;
    // two row groups with no split 152.0, four with a 2-way split 142.7)
    if constexpr (!F8) {
      if (chunks < 64) {
        gate_up_stream_k<2, 4, 1, 1, F8>(a, ntr, nts, L.I, Is_all, s);
        return;
      }
    }
    gate_up_stream<2, 2, 1, F8>(a, ntr, nts, L.I, Is_all, chunks >= 64 ? 4 : 2, s);
  } else {
    if constexpr (!F8) {
      // 64-row tiles, rows of fewer than 64 chunks (no k split): four row
      // groups per item, so the tile's token rows are re-read once per 64
      // weight rows instead of once per 32 (DeepSeek-V2-Lite shapes, T = 512:
      // 168 -> 147 us on MI355X).  With the 4-way split of longer rows that
      // variant would spill; with short intermediate rows (fine-grained,
      // I = 256: 4 items per tile) it leaves too few items (60 -> 64 us).
      if (chunks < 64 && L.I >= 1024) {
        gate_up_stream_k<4, 4, 1, 1, F8>(a, ntr, nts, L.I, Is_all, s);
        return;
      }
    }
    gate_up_stream<4, 2, 1, F8>(a, ntr, nts, L.I, Is_all, chunks >= 64 ? 4 : 1, s);
  }
}

template <bool F8>
static void down_streaming(const beam_moe_layer& L, const ExpertArgs& a, long tiles,
                           int tile_rows, hipStream_t s) {
  const int chunks = L.I / chunk_k<F8>();
  if (tile_rows == 16) {
    const int ks = stream_ksplit_chunks(chunks);
    if (tiles * (L.D / 32) * ks >= kWideShares) down_stream<1, 2, 1, F8>(a, tiles, L.D, ks, s);
    else down_stream<1, 1, 2, F8>(a, tiles, L.D, ks, s);
  } else if constexpr (!F8) {
    // 32- and 64-row tiles: four row groups per item (fewer re-reads of the
    // tile's h rows per weight byte; T = 256: 84 -> 76 us, T = 512:
    // 113 -> 92 us on MI355X, DeepSeek-V2-Lite shapes)
    if (tile_rows == 32) down_stream_k<2, 4, 1, 2, F8>(a, tiles, L.D, s);
    else down_stream<4, 4, 1, F8>(a, tiles, L.D, chunks >= 16 ? 2 : 1, s);
  } else if (tile_rows == 32) {
    down_stream_k<2, 2, 1, 2, F8>(a, tiles, L.D, s);
  } else {
    down_stream<4, 2, 1, F8>(a, tiles, L.D, chunks >= 16 ? 2 : 1, s);
  }
}

hipError_t launch_gate_up(const beam_moe_layer& L, const void* x, int32_t T, int tile_rows,
                          const WsLayout&, const Ptrs& p, hipStream_t s) {
  ExpertArgs a = expert_args(L, x, T, p);
  long nts;
  const long ntr = tile_bound(L, T, tile_rows, &nts);
  if (L.dtype == BEAM_F32) {
    const long items = ntr * (L.I / 16) + nts * (L.n_shared ? (L.n_shared * L.I_shared) / 16 : 0);
    prof_before("gate_up_f32", s);
    hipLaunchKernelGGL(k_gate_up_f32, dim3(persistent_grid(items, 2048)), dim3(256), 0, s, a);
    prof_after(s);
    return hipGetLastError();
  }
  if (L.expert_format == BEAM_WEIGHTS_FP8_E4M3) {   // tiles of at most 64 rows
    prof_before("gate_up_swiglu_stream_fp8", s);
    gate_up_streaming<true>(L, a, ntr, nts, tile_rows, s);
    prof_after(s);
  } else if (tile_rows <= 64) {
    prof_before("gate_up_swiglu_stream", s);
    gate_up_streaming<false>(L, a, ntr, nts, tile_rows, s);
    prof_after(s);
  } else if (tile_rows == kEsTileRows) {   // expert-stationary (packed weights)
    prof_before("pack_tokens_es", s);
    const long chunks = ntr * kEsTokBlocks * long(L.D / kPK) * 256;
    hipLaunchKernelGGL(k_pack_tokens_es, dim3(unsigned(std::min<long>((chunks + 255) / 256, 4096))),
                       dim3(256), 0, s, a);
    prof_after(s);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    prof_before("gate_up_swiglu_es", s);
    hipLaunchKernelGGL(k_gate_up_es, dim3(tiled_grid((const void*)&k_gate_up_es, ntr * (L.I / 64))),
                       dim3(256), 0, s, a);
    prof_after(s);
  } else if (L.wp_gate && es_shared_experts(L, T)) {
    // routed tiles on the 128-row kernel, the shared experts' tiles of
    // consecutive tokens on the expert-stationary ones
    a.tile_rows = tile_rows;
    a.es_ntiles = (T + kEsTileRows - 1) / kEsTileRows;
    prof_before("shared_pack_tokens_es", s);
    const long chunks = long(a.es_ntiles) * kEsTokBlocks * long(L.D / kPK) * 256;
    hipLaunchKernelGGL(k_pack_tokens_es, dim3(unsigned(std::min<long>((chunks + 255) / 256, 4096))),
                       dim3(256), 0, s, a);
    prof_after(s);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    prof_before("gate_up_swiglu_mixed", s);
    const long items = long(a.es_ntiles) * (L.n_shared * L.I_shared / 64) + ntr * ((L.I + 127) / 128);
    hipLaunchKernelGGL(k_gate_up_mixed, dim3(tiled_grid((const void*)&k_gate_up_mixed, items)), dim3(256), 0,
                       s, a);
    prof_after(s);
  } else if (L.wp_gate) {   // packed weights: tiles of 128 token rows
    a.tile_rows = tile_rows;
    const long items = ntr * ((L.I + 127) / 128) +
                       nts * (L.n_shared ? (L.n_shared * L.I_shared + 127) / 128 : 0);
    prof_before("gate_up_swiglu_packed", s);
    hipLaunchKernelGGL(k_gate_up_packed, dim3(tiled_grid((const void*)&k_gate_up_packed, items)),
                       dim3(256), 0, s, a);
    prof_after(s);
  } else {
    const int ib = tile_rows == 256 ? 64 : 128;   // intermediate rows per tile
    const long items = ntr * ((L.I + ib - 1) / ib) +
                       nts * (L.n_shared ? (L.n_shared * L.I_shared + ib - 1) / ib : 0);
    prof_before("gate_up_swiglu_tiled", s);
    if (tile_rows == 256)
      hipLaunchKernelGGL((k_gate_up_tiled<128, 256>),
                         dim3(tiled_grid((const void*)&k_gate_up_tiled<128, 256>, items)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_gate_up_tiled<256, 128>),
                         dim3(tiled_grid((const void*)&k_gate_up_tiled<256, 128>, items)), dim3(256), 0, s, a);
    prof_after(s);
  }
  return hipGetLastError();
}

// Resident workgroups of the tiled down kernel for a tile height (0: the
// launch streams, no split).
static int down_tiled_slots(const beam_moe_layer& L, int tile_rows) {
  if (L.wp_gate) return resident_blocks((const void*)&k_down_packed, 256);
  if (tile_rows == 256) return resident_blocks((const void*)&k_down_tiled<128, 256>, 256);
  if (tile_rows == 128) return resident_blocks((const void*)&k_down_tiled<256, 128>, 256);
  return 0;
}
static int down_tiled_nb(const beam_moe_layer& L, int tile_rows) {
  const int bn = L.wp_gate ? 256 : tile_rows == 256 ? 128 : 256;
  return (L.D + bn - 1) / bn;
}
static bool down_may_split(const beam_moe_layer& L, int tile_rows) {
  return L.dtype != BEAM_F32 && L.expert_format != BEAM_WEIGHTS_FP8_E4M3 && tile_rows > 64 &&
         tile_rows != kEsTileRows;
}

hipError_t launch_down(const beam_moe_layer& L, int32_t T, int tile_rows, const WsLayout&,
                       const Ptrs& p, hipStream_t s, bool allow_split) {
  ExpertArgs a = expert_args(L, nullptr, T, p);
  const bool ess = L.wp_gate && es_shared_experts(L, T);
  if (allow_split && p.o_part && down_may_split(L, tile_rows) && !ess)
    a.down_slots = down_tiled_slots(L, tile_rows);
  long nts;
  const long ntr = tile_bound(L, T, tile_rows, &nts);
  if (L.dtype == BEAM_F32) {
    const long items = (ntr + nts) * ((L.D + 15) / 16);
    prof_before("down_f32", s);
    hipLaunchKernelGGL(k_down_f32, dim3(persistent_grid(items, 2048)), dim3(256), 0, s, a);
    prof_after(s);
    return hipGetLastError();
  }
  if (L.expert_format == BEAM_WEIGHTS_FP8_E4M3) {   // tiles of at most 64 rows
    prof_before("down_stream_fp8", s);
    down_streaming<true>(L, a, ntr + nts, tile_rows, s);
    prof_after(s);
  } else if (tile_rows <= 64) {
    prof_before("down_stream", s);
    down_streaming<false>(L, a, ntr + nts, tile_rows, s);
    prof_after(s);
  } else if (tile_rows == kEsTileRows) {   // expert-stationary (packed weights)
    prof_before("down_es", s);
    hipLaunchKernelGGL(k_down_es, dim3(tiled_grid((const void*)&k_down_es, ntr * (L.D / 128))),
                       dim3(256), 0, s, a);
    prof_after(s);
  } else if (ess) {
    // routed tiles on the 128-row kernel (no k split), the shared experts'
    // tiles on the expert-stationary one (output O_shared)
    a.tile_rows = tile_rows;
    a.es_ntiles = (T + kEsTileRows - 1) / kEsTileRows;
    prof_before("down_mixed", s);
    const long items = long(a.es_ntiles) * (L.D / 128) + ntr * ((L.D + 255) / 256);
    hipLaunchKernelGGL(k_down_mixed, dim3(tiled_grid((const void*)&k_down_mixed, items)), dim3(256), 0, s, a);
    prof_after(s);
  } else if (L.wp_gate) {   // packed weights: tiles of 128 token rows
    a.tile_rows = tile_rows;
    const long items = (ntr + nts) * ((L.D + 255) / 256);
    const long gi = a.down_slots > 0 ? items * kMaxDownSplit : items;
    prof_before("down_packed", s);
    hipLaunchKernelGGL(k_down_packed, dim3(tiled_grid((const void*)&k_down_packed, gi)), dim3(256),
                       0, s, a);
    prof_after(s);
  } else {
    const int bn = tile_rows == 256 ? 128 : 256;
    const long items = (ntr + nts) * ((L.D + bn - 1) / bn);
    // room for the items of a k split (the device decides from the plan)
    const long gi = a.down_slots > 0 ? items * kMaxDownSplit : items;
    prof_before("down_tiled", s);
    if (tile_rows == 256)
      hipLaunchKernelGGL((k_down_tiled<128, 256>),
                         dim3(tiled_grid((const void*)&k_down_tiled<128, 256>, gi)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_down_tiled<256, 128>),
                         dim3(tiled_grid((const void*)&k_down_tiled<256, 128>, gi)), dim3(256), 0, s, a);
    prof_after(s);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const beam_moe_layer& L, int32_t T, int tile_rows, const Ptrs& p,
                          void* y, hipStream_t s) {
  const void* osh = L.n_shared > 0 ? p.o_shared : nullptr;
  CombineSplit cs{nullptr, 0, 0, nullptr, nullptr, 0, 0};
  if (p.o_part && down_may_split(L, tile_rows) && !(L.wp_gate && es_shared_experts(L, T))) {
    const ExpertArgs a = expert_args(L, nullptr, T, p);
    cs = CombineSplit{p.plan, down_tiled_slots(L, tile_rows), down_tiled_nb(L, tile_rows), a.op, a.op_sh,
                      a.op_stride, a.op_sh_stride};
  }
  prof_before("combine", s);
  const bool bf = L.dtype != BEAM_F32;
  if (bf && T >= 1024 && L.D <= 4096 && L.D % 8 == 0) {
    const unsigned grid = unsigned(std::min<long>((T + 3) / 4, 2048));
    auto tok = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, T, L.D, L.K, p.gates, p.slot_pos,
                         (const u16*)p.o, (const u16*)osh, (u16*)y, cs);
    };
    const int P = (L.D + 511) / 512;
    if (cs.plan) {
      if (P <= 1) tok(k_combine_tok<1, true>);
      else if (P <= 2) tok(k_combine_tok<2, true>);
      else if (P <= 3) tok(k_combine_tok<3, true>);
      else if (P <= 4) tok(k_combine_tok<4, true>);
      else tok(k_combine_tok<8, true>);
    } else {
      if (P <= 1) tok(k_combine_tok<1, false>);
      else if (P <= 2) tok(k_combine_tok<2, false>);
      else if (P <= 3) tok(k_combine_tok<3, false>);
      else if (P <= 4) tok(k_combine_tok<4, false>);
      else tok(k_combine_tok<8, false>);
    }
    prof_after(s);
    return hipGetLastError();
  }
  // Below 1024 tokens: all K slots in one chunk when K <= 8, else the kept
  // slots four at a time; from 1024 tokens: the kept slots one at a time.
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(unsigned(T)), dim3(256), 0, s, T, L.D, L.K, p.gates, p.slot_pos,
                       p.o, osh, y, cs);
  };
  if (T >= 1024) bf ? go(k_combine<true, 1, true>) : go(k_combine<false, 1, true>);
  else if (L.K <= 2) bf ? go(k_combine<true, 2, false>) : go(k_combine<false, 2, false>);
  else if (L.K <= 4) bf ? go(k_combine<true, 4, false>) : go(k_combine<false, 4, false>);
  else if (L.K <= 8) bf ? go(k_combine<true, 8, false>) : go(k_combine<false, 8, false>);
  else bf ? go(k_combine<true, 4, true>) : go(k_combine<false, 4, true>);
  prof_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plain copy (counter calibration)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_copy16(uint4* __restrict__ dst,
                                                const uint4* __restrict__ src, long n) {
  for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += long(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

// MFMA throughput probe: every wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 accumulation chains on register operands (the
// chains keep the matrix unit busy across their latency), then stores the
// sum of its accumulators so the work is kept.  FLOPs per launch:
// blocks * 4 waves * iters * 4 * (2 * 32 * 32 * 16).
__global__ __launch_bounds__(256) void k_mfma_loop(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  // bf16 values 2^-8 .. (lane-dependent), so that sums stay small and finite
  const uint32_t va = 0x3B803B80u + (uint32_t(lane & 7) << 16);
  const u32x4 a = u32x4{va, va, va, va}, b = u32x4{0x3B803B80u, 0x3B803B80u, 0x3B803B80u, 0x3B803B80u};
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32_bf16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_mfma_loop(float* out, int blocks, int iters, hipStream_t s) {
  prof_before("mfma_loop", s);
  hipLaunchKernelGGL(k_mfma_loop, dim3(unsigned(blocks)), dim3(256), 0, s, out, iters);
  prof_after(s);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const long n = long(bytes / 16);
  const long blocks = std::min<long>((n + 255) / 256, 4096);
  prof_before("copy16", s);
  hipLaunchKernelGGL(k_copy16, dim3(unsigned(std::max<long>(blocks, 1))), dim3(256), 0, s,
                     (uint4*)dst, (const uint4*)src, n);
  prof_after(s);
  return hipGetLastError();
}

}  // namespace beam

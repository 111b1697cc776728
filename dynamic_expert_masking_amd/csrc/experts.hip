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
#include <map>
#include <mutex>

#include "beam_internal.h"
#include "gemm_engines.h"
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
  int T, D, E, I, S, Is;
  const Plan* plan;
  const Tile* tiles;
  const int32_t* perm_token;
  void* h;         // [P][I]
  void* h_sh;      // [T][S*Is]
  void* o;         // [P][D] expert outputs: fp32 (fp32 layers) or bf16
  void* o_sh;      // [T][D] shared-expert outputs, same type
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

template <int BN, int BM>
__global__ __launch_bounds__(256, 2) void k_down_tiled(ExpertArgs a) {
  __shared__ TiledSmem<BN, BM> sm;
  constexpr int JN = BN / 64, JM = BM / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int ntr = a.plan->n_tiles_routed, nts = a.plan->n_tiles_shared;
  const int nb_all = (a.D + BN - 1) / BN;
  const long total = long(ntr + nts) * nb_all;
  for (XcdRange it = xcd_range(total); it.next < it.end; it.next += it.step) {
    int ti, nb;
    down_item(it.next, ntr, nts, nb_all, ti, nb);
    const bool shared = ti >= ntr;
    const Tile tl = a.tiles[ti];
    DownProvBase pv;
    down_setup(a, tl, shared, pv);
    pv.d0 = nb * BN;
    f32x16 acc[JN][JM];
    tiled_accumulate<BN, BM>(pv, sm, acc, tl.rows);
    u16* ob = static_cast<u16*>(shared ? a.o_sh : a.o);
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
              st4_bf16(ob, size_t(tl.row0 + r) * a.D + d, v[4 * q], v[4 * q + 1], v[4 * q + 2],
                       v[4 * q + 3]);
            }
          }
        }
      }
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
template <bool BF16, int KC, bool COMPACT>
__global__ __launch_bounds__(256) void k_combine(int T, int D, int K, const float* __restrict__ gates,
                                                 const int32_t* __restrict__ slot_pos,
                                                 const void* __restrict__ o,
                                                 const void* __restrict__ o_sh, void* __restrict__ y) {
  __shared__ float s_g[32];
  __shared__ int32_t s_p[32];
  __shared__ int s_n;
  const int t = blockIdx.x;
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
  a.T = T;
  a.D = L.D;
  a.E = L.E;
  a.I = L.I;
  a.S = L.n_shared;
  a.Is = L.I_shared;
  a.plan = p.plan;
  a.tiles = p.tiles;
  a.perm_token = p.perm_token;
  a.h = p.h;
  a.h_sh = p.h_shared;
  a.o = p.o;
  a.o_sh = p.o_shared;
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
    // per wave of a full grid; 32-row tiles two row groups, split only for
    // long rows; 64-row tiles as bf16.
    if (tile_rows == 16) {
      const long items1 = ntr * (L.I / 16) + nts * (Is_all / 16);
      const long want = kStreamGrid * kStreamWaves * 3 / 4;
      const int ks = items1 >= want ? 1 : 2 * items1 >= want ? 2 : 4;
      gate_up_stream<1, 1, 1, F8>(a, ntr, nts, L.I, Is_all, ks, s);
      return;
    }
    if (tile_rows == 32) {
      gate_up_stream<2, 2, 1, F8>(a, ntr, nts, L.I, Is_all, chunks >= 32 ? 2 : 1, s);
      return;
    }
  }
  if (tile_rows == 16) {
    const int ks = stream_ksplit_chunks(chunks);
    const long items2 = ntr * (L.I / 32) + nts * (Is_all / 32);
    if (items2 * ks >= kWideShares) gate_up_stream<1, 2, 1, F8>(a, ntr, nts, L.I, Is_all, ks, s);
    else gate_up_stream<1, 1, 1, F8>(a, ntr, nts, L.I, Is_all, ks, s);
  } else if (tile_rows == 32) {
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
  const ExpertArgs a = expert_args(L, x, T, p);
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

hipError_t launch_down(const beam_moe_layer& L, int32_t T, int tile_rows, const WsLayout&,
                       const Ptrs& p, hipStream_t s) {
  const ExpertArgs a = expert_args(L, nullptr, T, p);
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
  } else {
    const int bn = tile_rows == 256 ? 128 : 256;
    const long items = (ntr + nts) * ((L.D + bn - 1) / bn);
    prof_before("down_tiled", s);
    if (tile_rows == 256)
      hipLaunchKernelGGL((k_down_tiled<128, 256>),
                         dim3(tiled_grid((const void*)&k_down_tiled<128, 256>, items)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_down_tiled<256, 128>),
                         dim3(tiled_grid((const void*)&k_down_tiled<256, 128>, items)), dim3(256), 0, s, a);
    prof_after(s);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const beam_moe_layer& L, int32_t T, const Ptrs& p, void* y,
                          hipStream_t s) {
  const void* osh = L.n_shared > 0 ? p.o_shared : nullptr;
  prof_before("combine", s);
  // Below 1024 tokens: all K slots in one chunk when K <= 8, else the kept
  // slots four at a time; from 1024 tokens: the kept slots one at a time.
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(unsigned(T)), dim3(256), 0, s, T, L.D, L.K, p.gates, p.slot_pos,
                       p.o, osh, y);
  };
  const bool bf = L.dtype != BEAM_F32;
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

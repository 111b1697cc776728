// Routing kernels of the BEAM layer: router and mask-router logits, top-K
// selection with softmax and the binary mask, per-expert counts, and the
// compaction of surviving (token, expert) pairs into expert-major order.
//
// Method: BEAM page on aitrends.kr ("BEAM: Dynamic MoE 라우팅을 위한 Binary
// Expert Activation Masking"), method paragraph Steps 1-3 and the gate
// product of Step 4; skipping masked experts follows the ai-feeds.com
// summary's section on inference (only experts whose mask is 1 run).
#include "beam_internal.h"
#include "gemm_engines.h"

namespace beam {

// ---------------------------------------------------------------------------
// Router + mask-router logits (no bias): part[ks][t][j], j < E -> Wr row j,
// j >= E -> Wm row j-E.  For small batches the k range is split over KS
// workgroups (ks) so that the router's weight rows stream through many CUs;
// the selection kernel adds the KS partial sums in ks order, then the bias.
// ---------------------------------------------------------------------------

struct RouterArgs {
  const u16* x;
  const u16* wr;
  const u16* wm;
  float* part;
  int T, D, E, KS;
};

__device__ __forceinline__ const u16* router_row(const RouterArgs& a, int j) {
  if (j < a.E) return a.wr + size_t(j) * a.D;
  if (j < 2 * a.E) return a.wm + size_t(j - a.E) * a.D;
  return nullptr;
}

__device__ __forceinline__ void router_store(const RouterArgs& a, int ks, int t, int j, float v) {
  if (t >= a.T || j >= 2 * a.E) return;
  a.part[(size_t(ks) * a.T + t) * 2 * a.E + j] = v;
}

// NM groups of 16 router rows (rows j0 .. j0 + 16 NM) x 16*MT token rows.
template <int NM, int MT>
struct RouterSkinnyProv {
  const RouterArgs* a;
  int j0, t0, k0;   // k0: first element of this k slice
  __device__ int nseg() const { return 1; }
  __device__ int seg_chunks() const { return a->D / 64 / a->KS; }
  __device__ const u16* w(int g, int r, int) const {
    const u16* p = router_row(*a, j0 + 16 * g + r);
    return p ? p + k0 : nullptr;
  }
  __device__ const u16* x(int r, int) const {
    const int t = t0 + r;
    return t < a->T ? a->x + size_t(t) * a->D + k0 : nullptr;
  }
};

// The skinny router handles small batches and layers with few experts (whose
// 2E router rows would waste most of a tiled weight block).  A workgroup
// takes NM groups of 16 router rows x 16*MT tokens x one k slice.  Small
// batches use one row group and split k so that the router's weight rows
// stream through many CUs; from 2048 tokens on, four row groups share each
// token-row load (the token rows, not the weights, are then the traffic:
// T = 4096, E = 64: 26.8 -> 21.8 us on MI355X; at 256 tokens the smaller grid
// costs more than the re-reads).  Layers of at least 128 experts have enough
// row groups to keep the grid full with four per workgroup from 256 tokens
// on (E = 212, T = 512: 15.9 -> 14.8 us).
constexpr int kRouterSkinnyMaxT = 1024;
__host__ __device__ inline bool router_use_skinny(int T, int E) { return T <= kRouterSkinnyMaxT || E <= 64; }
__host__ __device__ inline int router_nm(int T, int E) { return (T >= 2048 && 2 * E >= 64) || (T >= 256 && E >= 128) ? 4 : 1; }
// From kRouterWideT tokens the token blocks are tall (32 tokens, 64 with
// four row groups from 2048 tokens) and the k split fills the grid instead
// (router_ksplit): each weight row is then loaded for more tokens.  MI355X,
// us for (row groups, token blocks of 16, k split), against the earlier
// choice: DeepSeek-V2-Lite shapes T = 4096 (4, 4, 4) 18.1 against (4, 2, 1)
// 20.0; fine-grained T = 512 (4, 2, 4) 11.6 against (4, 1, 2) 14.6;
// Mixtral-shaped T = 2048 (1, 2, 4) 9.0 against (1, 1, 2) 10.1.
constexpr int kRouterWideT = 256;
__host__ __device__ inline int router_mt(int T, int E) {
  const int nrb = (2 * E + 16 * router_nm(T, E) - 1) / (16 * router_nm(T, E));
  if (T >= kRouterWideT) return router_nm(T, E) == 4 && T >= 2048 ? 4 : 2;
  if (T <= 16) return 1;
  if (T <= 32) return 2;
  if (long(nrb) * ((T + 63) / 64) >= 256) return 4;
  if (long(nrb) * ((T + 31) / 32) >= 256) return 2;
  return 1;
}

// red: 4 * NM * MT * 64 f32x4 of LDS.
template <int NM, int MT>
__device__ __forceinline__ void router_skinny_block(const RouterArgs& a, int blk, f32x4* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrb = (2 * a.E + 16 * NM - 1) / (16 * NM);
  const int ks = blk % a.KS;
  const int rest = blk / a.KS;
  const int j0 = (rest % nrb) * 16 * NM;
  const int t0 = (rest / nrb) * 16 * MT;
  RouterSkinnyProv<NM, MT> pv{&a, j0, t0, ks * (a.D / a.KS)};
  f32x4 acc[NM][MT];
  skinny_accumulate<NM, MT, (NM * MT >= 4 ? 1 : 4 / (NM * MT))>(pv, lane, wave, 4, acc);
  skinny_reduce<NM, MT>(acc, red, lane, wave, 4);
  // wave w stores the (row group, token block) pairs q with q % 4 == w
  for (int q = wave; q < NM * MT; q += 4) {
    f32x4 v = acc[0][0];
#pragma unroll
    for (int g = 0; g < NM; ++g)
#pragma unroll
      for (int b = 0; b < MT; ++b)
        if (g * MT + b == q) v = acc[g][b];
    const int t = t0 + 16 * (q % MT) + (lane & 15);
    const int j = j0 + 16 * (q / MT) + 4 * (lane >> 4);
    // v holds router rows j .. j + 3 of token t: one 16-byte store when E is
    // even (rows of 2E floats, j a multiple of 4: the four exist or none does)
    if ((a.E & 1) == 0) {
      if (t < a.T && j < 2 * a.E)
        *reinterpret_cast<f32x4*>(a.part + (size_t(ks) * a.T + t) * 2 * a.E + j) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) router_store(a, ks, t, j + i, v[i]);
    }
  }
}

template <int NM, int MT>
__global__ __launch_bounds__(256) void k_router_skinny(RouterArgs a) {
  __shared__ f32x4 red[4 * NM * MT * kWave];
  router_skinny_block<NM, MT>(a, blockIdx.x, red);
}

// Tiled router (large batches with many experts): tiles of 64 rows of one
// router matrix x 128 tokens, both operands double-buffered in LDS
// (tiled_accumulate_db).  At T = 8192 and 212 experts that is 512 items,
// two workgroups per CU, which hide each other's load latency (256-token
// tiles, one workgroup per CU: 39.3 -> 35.7 us on MI355X).  Tiles of 64 x
// 64 (four workgroups per CU) or 128 x 128 and 256 x 64 (fewer operand
// re-reads) were slower: 41.6, 36.2 and 40.6 us against 34.1.
constexpr int kRouterBN = 64, kRouterBM = 128;

// A tile covers rows [jb, jb + 64) of one of the two weight matrices
// (which = 0: Wr, 1: Wm), so that its rows share one base address.
struct RouterTiledProv {
  const RouterArgs* a;
  int which, jb, t0;
  __device__ int nseg() const { return 1; }
  __device__ int seg_chunks() const { return a->D / 64; }
  __device__ const u16* wbase(int, int) const { return which ? a->wm : a->wr; }
  __device__ uint32_t woff(int r) const {
    const int j = jb + r;
    return uint32_t((j < a->E ? j : 0) * a->D);
  }
  __device__ const u16* xbase(int) const { return a->x; }
  __device__ uint32_t xoff(int r) const {
    const int t = t0 + r;
    return uint32_t((t < a->T ? t : 0) * a->D);
  }
};

// Persistent: items are (token tile, matrix, 64-row block).
__global__ __launch_bounds__(256, 2) void k_router_tiled(RouterArgs a) {
  __shared__ TiledSmem2<kRouterBN, kRouterBM> sm;
  constexpr int JN = kRouterBN / 64, JM = kRouterBM / 64;
  const int nrb = (a.E + kRouterBN - 1) / kRouterBN;   // blocks per matrix
  const long total = long((a.T + kRouterBM - 1) / kRouterBM) * 2 * nrb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  for (XcdRange it = xcd_range(total); it.next < it.end; it.next += it.step) {
    const int rb = int(it.next % (2 * nrb));
    const int t0 = int(it.next / (2 * nrb)) * kRouterBM;
    RouterTiledProv pv{&a, rb / nrb, (rb % nrb) * kRouterBN, t0};
    f32x16 acc[JN][JM];
    tiled_accumulate_db<kRouterBN, kRouterBM>(pv, sm, acc, a.T - t0);
#pragma unroll
    for (int jn = 0; jn < JN; ++jn)
#pragma unroll
      for (int jm = 0; jm < JM; ++jm) {
        const int t = t0 + wm * (kRouterBM / 2) + jm * 32 + (lane & 31);
        // Entries 4q .. 4q + 3 of a lane are four consecutive router rows of
        // one token: one 16-byte store when E is a multiple of 4 (then the
        // four exist or none does).  Scalar stores of single logits, 32
        // tokens' rows per instruction, took 49 us instead of 39 at T = 8192.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jr = pv.jb + wn * (kRouterBN / 2) + jn * 32 + 8 * q + 4 * (lane >> 5);
          const f32x16& v = acc[jn][jm];
          if ((a.E & 3) == 0) {
            if (t < a.T && jr < a.E)
              *reinterpret_cast<float4*>(a.part + size_t(t) * 2 * a.E + pv.which * a.E + jr) =
                  make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (jr + i < a.E) router_store(a, 0, t, pv.which * a.E + jr + i, v[4 * q + i]);
          }
        }
      }
  }
}

// fp32 layers: one thread per (token, router row), k in float4 steps.
struct RouterArgsF32 {
  const float* x;
  const float* wr;
  const float* wm;
  float* part;
  int T, D, E;
};

__global__ __launch_bounds__(256) void k_router_f32(RouterArgsF32 a) {
  const long q = long(blockIdx.x) * blockDim.x + threadIdx.x;
  const int R = 2 * a.E;
  if (q >= long(a.T) * R) return;
  const int t = int(q / R), j = int(q % R);
  const float* w = j < a.E ? a.wr + size_t(j) * a.D : a.wm + size_t(j - a.E) * a.D;
  const float* xr = a.x + size_t(t) * a.D;
  float s = 0.f;
  for (int k = 0; k < a.D; k += 4) {
    const float4 xv = *reinterpret_cast<const float4*>(xr + k);
    const float4 wv = *reinterpret_cast<const float4*>(w + k);
    s = fmaf(xv.x, wv.x, s);
    s = fmaf(xv.y, wv.y, s);
    s = fmaf(xv.z, wv.z, s);
    s = fmaf(xv.w, wv.w, s);
  }
  a.part[size_t(t) * R + j] = s;
}

// One token, bf16, d_model up to 4096 (a multiple of 8): the 2E logits are
// matrix-vector products. One wave per router row: it issues every 16-byte
// chunk of its row and of x at once, sums in fp32 and reduces over the wave
// in a fixed order; the logits land unsplit (KS = 1).
bool router_t1(const beam_moe_layer& L, int32_t T) {
  return T == 1 && L.dtype == BEAM_BF16 && L.D % 8 == 0 && L.D <= kWave * 8 * 8;
}

template <int NJ>   // 16-byte chunks per lane: D <= 512 NJ
__global__ __launch_bounds__(256) void k_router_t1(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= 2 * a.E) return;   // wave-uniform
  const u16* w = router_row(a, j);
  const int nch = a.D / 8;
  u32x4 xv[NJ], wv[NJ];
#pragma unroll
  for (int q = 0; q < NJ; ++q) {
    const int c = lane + kWave * q;
    const size_t cc = size_t(c < nch ? c : 0) * 8;
    xv[q] = ld16(a.x + cc);
    wv[q] = ld16_stream(w + cc);
  }
  float d = 0.f;
#pragma unroll
  for (int q = 0; q < NJ; ++q) {
    if (lane + kWave * q >= nch) continue;   // chunk past the row: no contribution
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d = fmaf(__uint_as_float(wv[q][i] << 16), __uint_as_float(xv[q][i] << 16), d);
      d = fmaf(__uint_as_float(wv[q][i] & 0xffff0000u), __uint_as_float(xv[q][i] & 0xffff0000u), d);
    }
  }
  d = wave_sum_f32(d);
  if (lane == 0) a.part[j] = d;
}

int router_ksplit(const beam_moe_layer& L, int32_t T) {
  if (L.dtype == BEAM_F32 || router_t1(L, T) || !router_use_skinny(T, L.E)) return 1;
  // Split k (at most 4 ways, so that selection reads at most 4 partial sums
  // per logit) when the (row block x token block) grid is small.
  const int chunks = L.D / 64;
  const int nm = router_nm(T, L.E), mt = router_mt(T, L.E);
  const long blocks = long((2 * L.E + 16 * nm - 1) / (16 * nm)) * ((T + 16 * mt - 1) / (16 * mt));
  int best = 1;
  for (int ks = 2; ks <= 4; ++ks) {
    const bool fills = T >= kRouterWideT ? blocks * ks <= 512 : blocks * (ks - 1) < 256;
    if (chunks % ks == 0 && chunks / ks >= 4 && fills) best = ks;
  }
  return best;
}

hipError_t launch_router_logits(const beam_moe_layer& L, const void* x, int32_t T, const Ptrs& p,
                                hipStream_t s) {
  float* part = p.logits;
  if (L.dtype == BEAM_F32) {
    RouterArgsF32 a{(const float*)x, (const float*)L.w_router, (const float*)L.w_mask, part,
                    T, L.D, L.E};
    const long n = long(T) * 2 * L.E;
    prof_before("router_logits_f32", s);
    hipLaunchKernelGGL(k_router_f32, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, a);
    prof_after(s);
    return hipGetLastError();
  }
  const int KS = router_ksplit(L, T);
  if (long(KS) * T > router_logit_rows(L, T)) return hipErrorInvalidValue;   // workspace bound
  RouterArgs a{(const u16*)x, (const u16*)L.w_router, (const u16*)L.w_mask, part, T, L.D, L.E, KS};
  if (router_t1(L, T)) {
    const dim3 grid(unsigned((2 * L.E + 3) / 4));
    // chunks per lane sized to the row, so no lane re-reads a chunk for nothing
    const int nj = (L.D / 8 + kWave - 1) / kWave;
    const dim3 block(256);
    prof_before("router_logits_t1", s);
    switch (nj) {
      case 1: hipLaunchKernelGGL(k_router_t1<1>, grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL(k_router_t1<2>, grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL(k_router_t1<3>, grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL(k_router_t1<4>, grid, block, 0, s, a); break;
      case 5: hipLaunchKernelGGL(k_router_t1<5>, grid, block, 0, s, a); break;
      case 6: hipLaunchKernelGGL(k_router_t1<6>, grid, block, 0, s, a); break;
      case 7: hipLaunchKernelGGL(k_router_t1<7>, grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(k_router_t1<8>, grid, block, 0, s, a); break;
    }
    prof_after(s);
  } else if (router_use_skinny(T, L.E)) {
    const int nm = router_nm(T, L.E), mt = router_mt(T, L.E);
    const int nrb = (2 * L.E + 16 * nm - 1) / (16 * nm);
    const int ntb = (T + 16 * mt - 1) / (16 * mt);
    const dim3 grid(unsigned(nrb * ntb * KS));
    prof_before("router_logits_skinny", s);
    if (nm == 4) {
      if (mt == 1) hipLaunchKernelGGL((k_router_skinny<4, 1>), grid, dim3(256), 0, s, a);
      else if (mt == 2) hipLaunchKernelGGL((k_router_skinny<4, 2>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_router_skinny<4, 4>), grid, dim3(256), 0, s, a);
    } else {
      if (mt == 1) hipLaunchKernelGGL((k_router_skinny<1, 1>), grid, dim3(256), 0, s, a);
      else if (mt == 2) hipLaunchKernelGGL((k_router_skinny<1, 2>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_router_skinny<1, 4>), grid, dim3(256), 0, s, a);
    }
    prof_after(s);
  } else {
    const int nrb = (L.E + kRouterBN - 1) / kRouterBN;
    const long items = long((T + kRouterBM - 1) / kRouterBM) * 2 * nrb;
    long cap = resident_blocks((const void*)&k_router_tiled, 256);
    cap = std::max<long>(8, cap / 8 * 8);
    const unsigned grid = unsigned(std::max<long>(1, std::min<long>(items, cap)));
    prof_before("router_logits_tiled", s);
    hipLaunchKernelGGL(k_router_tiled, dim3(grid), dim3(256), 0, s, a);
    prof_after(s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan: from per-expert pair counts (in LDS), the expert offsets of the
// compacted pair order and the tile list.  Experts with no surviving pair
// get no tile, so their weights are never read.  Runs in one workgroup of NT
// threads.  On return sm.off holds the exclusive offsets.
// ---------------------------------------------------------------------------

// In-place exclusive prefix sums of two arrays of n entries at once, in
// passes of NT entries: wave-level scans, then the wave totals.
template <int NT>
__device__ void block_exclusive_scan2(int32_t* v1, int32_t* v2, int n,
                                      int32_t* tmp /* >= 4 * NT / 64 + 2 entries */) {
  constexpr int NW = NT / kWave;
  static_assert(NW <= kWave, "one wave scans the wave totals");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t c1 = 0, c2 = 0;   // totals of the earlier passes
  for (int base = 0; base < n; base += NT) {
    const int i = base + tid;
    const int32_t a = i < n ? v1[i] : 0;
    const int32_t b = i < n ? v2[i] : 0;
    const int32_t ia = wave_inclusive_scan_i32(a, lane);
    const int32_t ib = wave_inclusive_scan_i32(b, lane);
    if (lane == 63) {
      tmp[wave] = ia;
      tmp[NW + wave] = ib;
    }
    __syncthreads();
    // wave 0 turns the wave totals into exclusive wave offsets and the pass
    // totals, so that every wave then reads one entry per array
    if (wave == 0) {
      const int32_t ta = lane < NW ? tmp[lane] : 0;
      const int32_t tb = lane < NW ? tmp[NW + lane] : 0;
      const int32_t sa = wave_inclusive_scan_i32(ta, lane);
      const int32_t sb = wave_inclusive_scan_i32(tb, lane);
      if (lane < NW) {
        tmp[2 * NW + lane] = sa - ta;
        tmp[3 * NW + lane] = sb - tb;
      }
      if (lane == NW - 1) {
        tmp[4 * NW] = sa;
        tmp[4 * NW + 1] = sb;
      }
    }
    __syncthreads();
    if (i < n) {
      v1[i] = c1 + tmp[2 * NW + wave] + ia - a;
      v2[i] = c2 + tmp[3 * NW + wave] + ib - b;
    }
    c1 += tmp[4 * NW];
    c2 += tmp[4 * NW + 1];
    __syncthreads();
  }
}

struct PlanSmem {
  int32_t cnt[kMaxExperts];
  int32_t off[kMaxExperts];
  int32_t toff[kMaxExperts];
  int32_t tmp[4 * 1024 / kWave + 2];   // block_exclusive_scan2 scratch for 1024 threads
  int32_t act;
};

// write_out = false: only sm.off / sm.toff (every workgroup of a multi-
// workgroup kernel computes them; one stores the plan).
template <int NT>
__device__ void build_plan(PlanSmem& sm, int T, int E, int tile_rows, int has_shared,
                           int32_t* __restrict__ counts, int32_t* __restrict__ expert_off,
                           Plan* __restrict__ plan, Tile* __restrict__ tiles, bool write_out = true) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) sm.act = 0;
  for (int e = tid; e < E; e += NT) {
    const int32_t c = sm.cnt[e];
    sm.off[e] = c;
    sm.toff[e] = (c + tile_rows - 1) / tile_rows;
  }
  __syncthreads();
  const int32_t last_cnt = sm.cnt[E - 1];
  const int32_t last_tiles = sm.toff[E - 1];
  block_exclusive_scan2<NT>(sm.off, sm.toff, E, sm.tmp);
  for (int e0 = 0; e0 < E; e0 += NT) {   // whole waves, for the ballot
    const int e = e0 + tid;
    const unsigned long long act = __ballot(e < E && sm.cnt[e] > 0);
    if (lane == 0 && act) atomicAdd(&sm.act, int32_t(__popcll(act)));
  }
  __syncthreads();
  // The global outputs are stored after the last barrier.
  if (!write_out) return;
  const int32_t P = sm.off[E - 1] + last_cnt;
  const int32_t ntr = sm.toff[E - 1] + last_tiles;
  const int32_t nts = has_shared ? (T + tile_rows - 1) / tile_rows : 0;
  for (int e = tid; e < E; e += NT) {
    const int32_t c = sm.cnt[e];
    counts[e] = c;
    expert_off[e] = sm.off[e];
    const int nt = (c + tile_rows - 1) / tile_rows;
    for (int j = 0; j < nt; ++j) {
      Tile tl;
      tl.expert = e;
      tl.row0 = sm.off[e] + j * tile_rows;
      tl.rows = min(tile_rows, c - j * tile_rows);
      tl.pad = 0;
      tiles[sm.toff[e] + j] = tl;
    }
  }
  for (int j = tid; j < nts; j += NT) {
    Tile tl;
    tl.expert = E;
    tl.row0 = j * tile_rows;
    tl.rows = min(tile_rows, T - j * tile_rows);
    tl.pad = 0;
    tiles[ntr + j] = tl;
  }
  if (tid == 0) {
    expert_off[E] = P;
    Plan pl;
    pl.pairs = P;
    pl.n_tiles_routed = ntr;
    pl.n_tiles_shared = nts;
    pl.active_experts = sm.act;
    pl.gate_up_next = 0;
    pl.down_next = 0;
    *plan = pl;
  }
}

// ---------------------------------------------------------------------------
// Selection: top-K by descending router logit (equal logits: lower expert
// index first), softmax over the K kept logits, mask bit m_k = [z >= 0] on
// the candidates, g_hat = g * m.
//
// Three forms.  Up to 16 tokens, one workgroup selects and plans
// (k_select_plan).  Otherwise one wave selects each token (k_select_tokens);
// then, when the batch's per-expert token bitmaps (E x ceil(T/64) words) and
// its selections fit in one workgroup's LDS, a one-workgroup kernel builds the
// plan and places every pair (k_plan_bitmap), and else one workgroup per
// 64-token block records block-local ranks and counts (k_block_ranks) and the
// scan and scatter kernels follow.
// ---------------------------------------------------------------------------

constexpr int kSelWaves = 16;   // waves of the one-workgroup selection
constexpr int kSelMergedMax = 16;   // largest batch whose selection builds the plan itself
// Limits of the bitmap plan (LDS of its one workgroup).
constexpr int kPlanWords = 4096;    // E * ceil(T / 64) bitmap words
constexpr int kPlanPairs = 8192;    // T * K selections (above, the block-rank kernels are faster)
constexpr int kPlanTokens = 4096;   // T
constexpr int kPlanThreads = 1024;  // plan kernel workgroup
constexpr int kSelThreads = 256;    // selection: four tokens per workgroup, one wave per SIMD

bool select_builds_plan(const beam_moe_layer& L, int32_t T) {
  return long(L.E) * ((T + kSelBlock - 1) / kSelBlock) <= kPlanWords &&
         long(T) * L.K <= kPlanPairs && T <= kPlanTokens;
}

struct SelectArgs {
  const float* part;   // [KS][T][2E] router / mask-router partial logits
  int KS;
  const float* br;
  const float* bm;
  int T, E, K;
  int gating;   // beam_gate_flag bits
  int seg;      // segment routing: > 1 = token t routes as token t - t % seg
  int32_t* idx;
  float* gates;
  uint32_t* mask;
  int32_t* rank;
  int32_t* block_counts;
  // mask-router backward: keep every candidate, record the mask logits
  int all_pairs;
  float* zsel;
  // plan
  int tile_rows, has_shared;
  int32_t* counts;
  int32_t* expert_off;
  Plan* plan;
  Tile* tiles;
  int32_t* perm_token;
  int32_t* slot_pos;
};

// Row of the router logits that token t's routing is decided on: its own,
// or with segment routing the first token of its segment.
__device__ __forceinline__ int route_row(const SelectArgs& a, int t) {
  return a.seg > 1 ? t - t % a.seg : t;
}

// Gates of one token from its K selected logits: lane k < K holds slot k's
// logit r_k and its mask bit; r_0 (the largest) sits in lane 0.  Without
// options, g = softmax over the K logits; BEAM_GATE_SOFTMAX_ALL divides by the
// sum over all E experts instead (lane l's NPER logits in r_all, -inf for
// absent experts); BEAM_GATE_BINARY sets g = 1 on every slot;
// BEAM_GATE_RENORM renormalises g * m over the kept slots.
template <int NPER>
__device__ __forceinline__ float token_gate(int gating, bool slot, bool keep, float r_k,
                                            const float (&r_all)[NPER]) {
  const float r_0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r_k), 0));
  const float ex = slot ? ((gating & BEAM_GATE_BINARY) ? 1.f : expf(r_k - r_0)) : 0.f;
  float den;
  if (gating & BEAM_GATE_BINARY) {
    den = 1.f;
  } else if (gating & BEAM_GATE_SOFTMAX_ALL) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < NPER; ++i) part += expf(r_all[i] - r_0);   // exp(-inf) = 0
    den = wave_sum_f32(part);
  } else {
    den = wave_sum_f32(ex);
  }
  float gh = keep ? ex / den : 0.f;
  if (gating & BEAM_GATE_RENORM) {
    const float s = wave_sum_f32(gh);
    gh = s > 0.f ? gh / s : 0.f;
  }
  return gh;
}

constexpr int kTopKBufWords = 96;   // per-wave LDS scratch of select_topk

// Top-K of one token by one wave.  Expert e = 64 i + lane has logit vals[i];
// experts e >= E are absent.  On return lane k < K holds the k-th selected
// expert and its logit, in descending logit order, equal logits by ascending
// expert index (1 <= K <= min(E, 32)).  buf: kTopKBufWords words of LDS
// owned by this wave.
//
// The K-th largest order key is found bit by bit from the top: a candidate
// prefix is kept when at least K keys are at or above it, counted with one
// compare per register slot and scalar popcounts of the ballots; the search
// ends early once exactly K keys are at or above the prefix.  The selection
// is every key above the threshold plus, among the keys equal to it, those
// of the lowest expert indices.  The winners are compacted in expert order,
// each one's rank is counted against the others, and they are placed by rank.
template <int NPER>
__device__ __forceinline__ void select_topk(const float (&vals)[NPER], int E, int K, int lane,
                                            uint32_t* buf, int& my_e, float& my_r) {
  uint32_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) key[i] = (lane + kWave * i < E) ? float_key(vals[i]) : 0u;
  // Present keys are at least float_key(-inf) > 0, and K <= E of them exist,
  // so the threshold p ends above 0 and absent experts are never selected.
  uint32_t p = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = p | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) cnt += __popcll(__ballot(key[i] >= c));
    if (cnt >= K) {
      p = c;
      if (cnt == K) break;
    }
  }
  unsigned long long sel[NPER];
  int need = K;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    sel[i] = __ballot(key[i] > p);
    need -= __popcll(sel[i]);
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    unsigned long long eq = __ballot(key[i] == p);
    while (need > 0 && eq) {   // equal keys: lowest expert index first
      const unsigned long long lo = eq & (~eq + 1ull);
      sel[i] |= lo;
      eq ^= lo;
      --need;
    }
  }
  // compaction in expert order: positions 0..K-1
  uint32_t* ck = buf;
  uint32_t* ce = buf + 32;
  uint32_t* sk = buf + 64;
  int base = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if ((sel[i] >> lane) & 1ull) {
      const int pos = base + __popcll(sel[i] & ((1ull << lane) - 1ull));
      ck[pos] = key[i];
      ce[pos] = uint32_t(kWave * i + lane);
    }
    base += __popcll(sel[i]);
  }
  __builtin_amdgcn_wave_barrier();
  const bool slot = lane < K;
  const uint32_t mk = slot ? ck[lane] : 0u;
  const uint32_t me = slot ? ce[lane] : 0u;
  // rank among the K: larger keys, and equal keys earlier in expert order
  int r = 0;
  for (int j = 0; j < K; ++j) {
    const uint32_t kj = uint32_t(__builtin_amdgcn_readlane(int(mk), j));
    r += (kj > mk || (kj == mk && j < lane)) ? 1 : 0;
  }
  __builtin_amdgcn_wave_barrier();
  if (slot) {
    sk[r] = mk;
    ck[r] = me;   // expert of rank r (ck is free once every lane read its entry)
  }
  __builtin_amdgcn_wave_barrier();
  my_e = slot ? int(ck[lane]) : 0;
  my_r = slot ? key_float(sk[lane]) : 0.f;
}

// r and z of token t for this lane's experts (e = lane + 64 i): the KS
// partial sums added in ks order, then the biases; experts past E give 0.
// Every load is issued unconditionally (absent experts read expert 0 and are
// dropped by a select) so that they are in flight together: a branch around
// each load compiles to a wait for it.  With NPER >= 16 the partial sums are
// read one ks slice per round, to bound the registers.
template <int NPER, int KS>
__device__ __forceinline__ void token_logits_k(const SelectArgs& a, int t, int lane,
                                               float (&rv)[NPER], float (&zv)[NPER]) {
  const int E = a.E;
  const float* row = a.part + size_t(route_row(a, t)) * 2 * E;
  const size_t kstride = size_t(a.T) * 2 * E;
  const float* brp = a.br ? a.br : a.part;   // a valid address either way
  const float* bmp = a.bm ? a.bm : a.part;
  // with NPER >= 16 the biases are read after the partial sums (registers)
  constexpr bool kBiasFirst = NPER < 16;
  auto ee = [&](int i) {   // expert of register slot i, or 0 past E
    const int e = lane + kWave * i;
    return e < E ? e : 0;
  };
  float bb[NPER], bz[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if (kBiasFirst) {
      bb[i] = brp[ee(i)];
      bz[i] = bmp[ee(i)];
    }
    rv[i] = zv[i] = 0.f;
  }
  constexpr int KB = NPER >= 16 ? 1 : KS;   // ks slices per round
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += KB) {
    float pr[KB][NPER], pz[KB][NPER];
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        pr[u][i] = row[size_t(k0 + u) * kstride + ee(i)];
        pz[u][i] = row[size_t(k0 + u) * kstride + E + ee(i)];
      }
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        rv[i] += pr[u][i];
        zv[i] += pz[u][i];
      }
  }
  if (!kBiasFirst) {
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      bb[i] = brp[ee(i)];
      bz[i] = bmp[ee(i)];
    }
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const bool ok = lane + kWave * i < E;
    rv[i] = ok ? rv[i] + (a.br ? bb[i] : 0.f) : 0.f;
    zv[i] = ok ? zv[i] + (a.bm ? bz[i] : 0.f) : 0.f;
  }
}

template <int NPER>
__device__ __forceinline__ void token_logits(const SelectArgs& a, int t, int lane,
                                             float (&rv)[NPER], float (&zv)[NPER]) {
  switch (a.KS) {   // uniform
    case 1: token_logits_k<NPER, 1>(a, t, lane, rv, zv); break;
    case 2: token_logits_k<NPER, 2>(a, t, lane, rv, zv); break;
    case 3: token_logits_k<NPER, 3>(a, t, lane, rv, zv); break;
    default: token_logits_k<NPER, 4>(a, t, lane, rv, zv); break;
  }
}

// Token t's selection by one wave.  Expert e's logits are held by lane
// e % 64 in register e / 64; the KS partial sums are added in ks order, then
// the biases; select_topk picks the K.  buf: the wave's select_topk scratch.
template <int NPER>
__device__ __forceinline__ void select_token(const SelectArgs& a, int t, int lane, uint32_t* buf) {
  const int E = a.E, K = a.K;
  float rv[NPER], vals[NPER], zv[NPER];
  token_logits<NPER>(a, t, lane, rv, zv);
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + kWave * i;
    vals[i] = e < E ? rv[i] + 0.0f : -__builtin_inff();   // + 0: -0 and +0 compare alike
  }
  float r_all[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) r_all[i] = vals[i];
  int my_e;
  float my_r;
  select_topk<NPER>(vals, E, K, lane, buf, my_e, my_r);
  const bool slot = lane < K;
  const int e_k = slot ? my_e : 0;
  const float r_k = slot ? my_r : 0.f;
  float z_k = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const float c = __shfl(zv[i], e_k & 63, kWave);
    if (i == (e_k >> 6)) z_k = c;
  }
  const bool keep = slot && (a.all_pairs || z_k >= 0.f);
  const unsigned long long bal = __ballot(keep);
  const float gh = token_gate<NPER>(a.gating, slot, keep, r_k, r_all);
  if (slot) {
    a.idx[size_t(t) * K + lane] = e_k;
    a.gates[size_t(t) * K + lane] = gh;
    if (a.all_pairs) a.zsel[size_t(t) * K + lane] = z_k;
  }
  if (lane == 0) a.mask[t] = uint32_t(bal);
}

struct BitmapPlanSmem {
  unsigned long long bits[kPlanWords];   // [E][W]: bit t%64 of word t/64: token t keeps e
  int32_t pre[kPlanWords];               // [E][W]: pairs of expert e in earlier words
  uint16_t idx[kPlanPairs];              // selections of the batch, [T][K]
  uint32_t mask[kPlanTokens];            // mask bits of the batch
  PlanSmem plan;
};

// One wave per token, NT / 64 tokens per workgroup.
template <int NPER, int NT>
__global__ __launch_bounds__(NT) void k_select_tokens(SelectArgs a) {
  __shared__ uint32_t sbuf[NT / kWave][kTopKBufWords];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * (NT / kWave) + wave;
  if (t < a.T) select_token<NPER>(a, t, lane, sbuf[wave]);
}

// The plan from all tokens' selections, in one workgroup: every token's mask
// and indices are copied into LDS with independent loads, per-expert token
// bitmaps give the counts, and a pair's position is off[e] + (kept tokens of
// e before t): expert-major, tokens ascending within an expert.
template <int NT>
__global__ __launch_bounds__(NT) void k_plan_bitmap(SelectArgs a) {
  __shared__ BitmapPlanSmem sm;
  const int tid = threadIdx.x;
  const int T = a.T, E = a.E, K = a.K;
  const int W = (T + kSelBlock - 1) / kSelBlock;
  const int TK = T * K;
  // masks and indices copied together: both arrays' loads in flight at once
  for (int i0 = 0; i0 < max(T, TK); i0 += 4 * NT) {
    uint32_t vm[4];
    int32_t vi[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT + tid;
      vm[u] = a.mask[i < T ? i : 0];
      vi[u] = a.idx[i < TK ? i : 0];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT + tid;
      if (i < T) sm.mask[i] = vm[u];
      if (i < TK) sm.idx[i] = uint16_t(vi[u]);
    }
  }
  for (int i = tid; i < E * W; i += NT) sm.bits[i] = 0ull;
  __syncthreads();
  for (int q = tid; q < TK; q += NT) {
    const int tt = q / K, k = q - tt * K;
    if ((sm.mask[tt] >> k) & 1u) atomicOr(&sm.bits[sm.idx[q] * W + (tt >> 6)], 1ull << (tt & 63));
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int32_t run = 0;
    for (int w = 0; w < W; ++w) {
      sm.pre[e * W + w] = run;
      run += __popcll(sm.bits[e * W + w]);
    }
    sm.plan.cnt[e] = run;
  }
  __syncthreads();
  build_plan<NT>(sm.plan, T, E, a.tile_rows, a.has_shared, a.counts, a.expert_off, a.plan, a.tiles);
  for (int q = tid; q < TK; q += NT) {
    const int tt = q / K, k = q - tt * K;
    int pos = -1;
    if ((sm.mask[tt] >> k) & 1u) {
      const int e = sm.idx[q], w = tt >> 6;
      const unsigned long long before = sm.bits[e * W + w] & ((1ull << (tt & 63)) - 1ull);
      pos = sm.plan.off[e] + sm.pre[e * W + w] + __popcll(before);
      a.perm_token[pos] = tt;
    }
    a.slot_pos[q] = pos;
  }
}

// Batches of at most kSelWaves tokens, one workgroup: wave w selects token w
// (its partial logit slices loaded in one round), then the same workgroup
// builds the plan from the batch's per-expert token bitmaps in LDS, as
// k_plan_bitmap does: one launch instead of two.
template <int NPER, int NT>
__global__ __launch_bounds__(NT) void k_select_plan(SelectArgs a) {
  __shared__ unsigned long long bits[kMaxExperts];
  __shared__ int32_t s_idx[kSelWaves * 32];
  __shared__ uint32_t s_mask[kSelWaves];
  __shared__ PlanSmem s_plan;
  __shared__ uint32_t sbuf[kSelWaves][kTopKBufWords];
  static_assert(kSelMergedMax <= kSelWaves, "one token per wave");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, K = a.K;
  for (int e = tid; e < E; e += blockDim.x) bits[e] = 0ull;
  __syncthreads();   // bits[] cleared

  const int t = wave;
  // this wave's token outputs, stored at the end
  int out_e = 0;
  float out_g = 0.f, out_z = 0.f;
  uint32_t out_mask = 0;
  if (t < T) {
    // r and z of token t: partial sums added in ks order, then the biases
    float rv[NPER], zv[NPER];
    token_logits<NPER>(a, t, lane, rv, zv);
    float vals[NPER], r_all[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = lane + kWave * i;
      vals[i] = e < E ? rv[i] + 0.0f : -__builtin_inff();   // + 0: -0 == +0
      r_all[i] = e < E ? rv[i] : -__builtin_inff();
    }
    int my_e;
    float my_r;
    select_topk<NPER>(vals, E, K, lane, sbuf[wave], my_e, my_r);
    const bool slot = lane < K;
    const int e_k = slot ? my_e : 0;
    const float r_k = slot ? my_r : 0.f;
    // mask logit of expert e_k lives in lane e_k % 64, register e_k / 64
    float z_k = 0.f;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const float c = __shfl(zv[i], e_k & 63, kWave);
      if (i == (e_k >> 6)) z_k = c;
    }
    const bool keep = slot && (a.all_pairs || z_k >= 0.f);
    const unsigned long long bal = __ballot(keep);
    const float gh = token_gate<NPER>(a.gating, slot, keep, r_k, r_all);
    if (slot) s_idx[t * 32 + lane] = e_k;
    if (lane == 0) s_mask[t] = uint32_t(bal);
    if (keep) atomicOr(&bits[e_k], 1ull << t);
    out_e = e_k;
    out_g = gh;
    out_z = z_k;
    out_mask = uint32_t(bal);
  }
  __syncthreads();

  PlanSmem& pl = s_plan;
  for (int e = tid; e < E; e += blockDim.x) pl.cnt[e] = __popcll(bits[e]);
  __syncthreads();
  build_plan<NT>(pl, T, E, a.tile_rows, a.has_shared, a.counts, a.expert_off, a.plan, a.tiles);
  for (int q = tid; q < T * K; q += blockDim.x) {
    const int tl = q / K, k = q - tl * K;
    int pos = -1;
    if ((s_mask[tl] >> k) & 1u) {
      const int e = s_idx[tl * 32 + k];
      pos = pl.off[e] + __popcll(bits[e] & ((1ull << tl) - 1ull));
      a.perm_token[pos] = tl;
    }
    a.slot_pos[q] = pos;
  }
  if (t < T) {
    if (lane < K) {
      a.idx[size_t(t) * K + lane] = out_e;
      a.gates[size_t(t) * K + lane] = out_g;
      if (a.all_pairs) a.zsel[size_t(t) * K + lane] = out_z;
    }
    if (lane == 0) a.mask[t] = out_mask;
  }
}

// Block ranks from the selections already written (idx, mask): one
// workgroup per 64-token block builds the block's per-expert token bitmaps
// and records each surviving pair's rank among the block's pairs of its
// expert (token order) and the block's per-expert counts.  The selection
// itself ran before with one wave per token across the whole GPU; selecting
// inside these workgroups (four tokens per wave, one 64-token block per
// workgroup) kept half the CUs idle at T = 8192 (fine-grained layer: 23.2 us
// for selection and ranks together, now 14.1 + 7.2 us).
__global__ __launch_bounds__(256) void k_block_ranks(SelectArgs a) {
  __shared__ unsigned long long bits[kMaxExperts];
  __shared__ uint32_t s_mask[kSelBlock];
  const int tid = threadIdx.x, blk = blockIdx.x;
  const int t0 = blk * kSelBlock;
  const int T = a.T, E = a.E, K = a.K;
  const int nt = min(kSelBlock, T - t0);
  for (int e = tid; e < E; e += blockDim.x) bits[e] = 0ull;
  if (tid < nt) s_mask[tid] = a.mask[t0 + tid];
  __syncthreads();
  for (int q = tid; q < nt * K; q += blockDim.x) {
    const int tl = q / K, k = q - tl * K;
    if ((s_mask[tl] >> k) & 1u) atomicOr(&bits[a.idx[size_t(t0) * K + q]], 1ull << tl);
  }
  __syncthreads();
  for (int q = tid; q < nt * K; q += blockDim.x) {
    const int tl = q / K, k = q - tl * K;
    int rk = -1;
    if ((s_mask[tl] >> k) & 1u)
      rk = __popcll(bits[a.idx[size_t(t0) * K + q]] & ((1ull << tl) - 1ull));
    a.rank[size_t(t0) * K + q] = rk;
  }
  for (int e = tid; e < E; e += blockDim.x)
    a.block_counts[size_t(blk) * E + e] = __popcll(bits[e]);
}

hipError_t launch_select(const beam_moe_layer& L, int32_t T, int tile_rows, const Ptrs& p,
                         hipStream_t s, bool all_pairs) {
  SelectArgs a;
  a.part = p.logits;
  a.KS = router_ksplit(L, T);
  a.br = L.b_router;
  a.bm = L.b_mask;
  a.T = T;
  a.E = L.E;
  a.K = L.K;
  a.gating = L.gating;
  a.seg = L.segment_len;
  a.idx = p.idx;
  a.gates = p.gates;
  a.mask = p.mask;
  a.rank = p.rank;
  a.block_counts = p.block_counts;
  a.tile_rows = tile_rows;
  a.has_shared = (L.n_shared > 0 && !all_pairs) ? 1 : 0;
  a.all_pairs = all_pairs ? 1 : 0;
  a.zsel = p.zsel;
  a.counts = p.counts;
  a.expert_off = p.expert_off;
  a.plan = p.plan;
  a.tiles = p.tiles;
  a.perm_token = p.perm_token;
  a.slot_pos = p.slot_pos;
  // Up to 16 tokens one workgroup selects and plans: one launch fewer (T = 1:
  // 13.4 -> 9.6 us for both steps on MI355X).  From 32 tokens on, selecting
  // in one workgroup costs more than the second launch saves.
  if (T <= kSelMergedMax) {
    prof_before("select_plan", s);
    // one wave per token: a single wave for one token, 4 waves for up to 4
    // tokens, 8 for up to 8 (fewer waves at each barrier), else 16 (T = 1,
    // DeepSeek-V2-Lite shapes: select+plan 7.35 -> 6.74 us, step 35.8 -> 35.3
    // us on MI355X with one wave instead of four; T = 8: 8.2 -> 7.9 us with
    // 8 waves instead of 16)
    auto go = [&](auto k1, auto k4, auto k8, auto k16) {
      if (T == 1) hipLaunchKernelGGL(k1, dim3(1), dim3(64), 0, s, a);
      else if (T <= 4) hipLaunchKernelGGL(k4, dim3(1), dim3(256), 0, s, a);
      else if (T <= 8) hipLaunchKernelGGL(k8, dim3(1), dim3(512), 0, s, a);
      else hipLaunchKernelGGL(k16, dim3(1), dim3(1024), 0, s, a);
    };
    if (L.E <= 64)
      go(k_select_plan<1, 64>, k_select_plan<1, 256>, k_select_plan<1, 512>, k_select_plan<1, 1024>);
    else if (L.E <= 128)
      go(k_select_plan<2, 64>, k_select_plan<2, 256>, k_select_plan<2, 512>, k_select_plan<2, 1024>);
    else if (L.E <= 256)
      go(k_select_plan<4, 64>, k_select_plan<4, 256>, k_select_plan<4, 512>, k_select_plan<4, 1024>);
    else
      go(k_select_plan<16, 64>, k_select_plan<16, 256>, k_select_plan<16, 512>, k_select_plan<16, 1024>);
    prof_after(s);
    return hipGetLastError();
  }
  if (select_builds_plan(L, T)) {
    constexpr int nt = kSelThreads;
    const dim3 g{unsigned((T + nt / kWave - 1) / (nt / kWave)), 1, 1}, b{unsigned(nt), 1, 1};
    prof_before("select_topk_mask", s);
    if (L.E <= 64) hipLaunchKernelGGL((k_select_tokens<1, nt>), g, b, 0, s, a);
    else if (L.E <= 128) hipLaunchKernelGGL((k_select_tokens<2, nt>), g, b, 0, s, a);
    else if (L.E <= 256) hipLaunchKernelGGL((k_select_tokens<4, nt>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_select_tokens<16, nt>), g, b, 0, s, a);
    prof_after(s);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    prof_before("plan_bitmap", s);
    // small batches: 4 waves reach each barrier sooner than 16 (T=64: 7.45 -> 7.2 us)
    if (long(T) * L.K <= 2048)
      hipLaunchKernelGGL((k_plan_bitmap<256>), dim3(1), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_plan_bitmap<kPlanThreads>), dim3(1), dim3(kPlanThreads), 0, s, a);
    prof_after(s);
    return hipGetLastError();
  }
  // Larger batches: one wave per token across the GPU, then the block ranks.
  {
    constexpr int nt = kSelThreads;
    const dim3 g{unsigned((T + nt / kWave - 1) / (nt / kWave)), 1, 1}, b{unsigned(nt), 1, 1};
    prof_before("select_topk_mask", s);
    if (L.E <= 64) hipLaunchKernelGGL((k_select_tokens<1, nt>), g, b, 0, s, a);
    else if (L.E <= 128) hipLaunchKernelGGL((k_select_tokens<2, nt>), g, b, 0, s, a);
    else if (L.E <= 256) hipLaunchKernelGGL((k_select_tokens<4, nt>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_select_tokens<16, nt>), g, b, 0, s, a);
    prof_after(s);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  const int nblk = (T + kSelBlock - 1) / kSelBlock;
  prof_before("block_ranks", s);
  hipLaunchKernelGGL(k_block_ranks, dim3(unsigned(nblk)), dim3(256), 0, s, a);
  prof_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scan (one workgroup, multi-block batches): per-expert totals and per-block
// exclusive offsets, then the plan.
// ---------------------------------------------------------------------------

constexpr int kScanVals = 32;   // block counts per thread held in registers by k_scan

__global__ __launch_bounds__(1024) void k_scan(int T, int E, int nblk, int tile_rows,
                                               int has_shared, int32_t* __restrict__ block_counts,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ expert_off,
                                               Plan* __restrict__ plan, Tile* __restrict__ tiles) {
  __shared__ PlanSmem psm;
  __shared__ int32_t s_part[1024];
  const int tid = threadIdx.x;
  // G threads per expert (the largest power of two with G * E <= 1024, at
  // most 64), each holding up to kScanVals consecutive block counts of its
  // expert in registers: thread (part, e) = (tid / E, tid % E) owns blocks
  // [part * per, part * per + per).  Its sum goes to LDS, and the sums of the
  // earlier parts give its running offset.  A thread's loads are independent,
  // so it waits for memory about once.
  int G = 1;
  while (2 * G * E <= 1024 && G < 64) G *= 2;
  const int per = (nblk + G - 1) / G;
  if (per <= kScanVals) {
    const int part = tid / E, e = tid - part * E;
    const bool act = part < G;
    const int b0 = part * per;
    int32_t c[kScanVals];
    int32_t sum = 0;
#pragma unroll
    for (int u = 0; u < kScanVals; ++u) {
      const int b = b0 + u;
      c[u] = (act && u < per && b < nblk) ? block_counts[size_t(b) * E + e] : 0;
      sum += c[u];
    }
    if (act) s_part[part * E + e] = sum;
    __syncthreads();
    if (act) {
      int32_t run = 0;
      for (int q = 0; q < part; ++q) run += s_part[q * E + e];
#pragma unroll
      for (int u = 0; u < kScanVals; ++u) {
        const int b = b0 + u;
        if (u < per && b < nblk) {
          block_counts[size_t(b) * E + e] = run;
          run += c[u];
        }
      }
      if (part == G - 1) psm.cnt[e] = run;
    }
  } else {
    for (int e = tid; e < E; e += 1024) {
      // exclusive running sum over blocks, 8 independent loads at a time
      int32_t run = 0;
      for (int bb = 0; bb < nblk; bb += 8) {
        int32_t c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = bb + u < nblk ? block_counts[size_t(bb + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (bb + u < nblk) {
            block_counts[size_t(bb + u) * E + e] = run;
            run += c[u];
          }
      }
      psm.cnt[e] = run;
    }
  }
  __syncthreads();
  build_plan<1024>(psm, T, E, tile_rows, has_shared, counts, expert_off, plan, tiles);
}

// Scan and scatter in one launch, for batches of at most G * kScanVals
// blocks (G as in k_scan): one workgroup per 64-token block.  Each recomputes,
// from the block counts (L2-resident), every expert's total and its own
// block's offset within the expert (the sum over earlier blocks), scans the
// totals into the expert offsets (workgroup 0 stores the plan and tiles), and
// places its block's pairs.  One launch instead of a one-workgroup scan
// followed by the scatter.
__global__ __launch_bounds__(1024) void k_scan_scatter(int T, int E, int K, int nblk, int tile_rows,
                                                       int has_shared,
                                                       const int32_t* __restrict__ block_counts,
                                                       const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ rank,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ expert_off,
                                                       Plan* __restrict__ plan, Tile* __restrict__ tiles,
                                                       int32_t* __restrict__ perm_token,
                                                       int32_t* __restrict__ slot_pos) {
  __shared__ PlanSmem psm;
  __shared__ int32_t s_all[1024], s_below[1024];
  __shared__ int32_t s_pre[kMaxExperts];
  const int tid = threadIdx.x, blk = blockIdx.x;
  int G = 1;
  while (2 * G * E <= 1024 && G < 64) G *= 2;
  const int per = (nblk + G - 1) / G;   // <= kScanVals (host check)
  const int part = tid / E, e0 = tid - part * E;
  const bool act = part < G;
  const int b0 = part * per;
  int32_t all = 0, below = 0;
#pragma unroll
  for (int u = 0; u < kScanVals; ++u) {
    const int b = b0 + u;
    const int32_t c = (act && u < per && b < nblk) ? block_counts[size_t(b) * E + e0] : 0;
    all += c;
    below += b < blk ? c : 0;
  }
  if (act) {
    s_all[part * E + e0] = all;
    s_below[part * E + e0] = below;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int32_t a = 0, bl = 0;
    for (int q = 0; q < G; ++q) {
      a += s_all[q * E + e];
      bl += s_below[q * E + e];
    }
    psm.cnt[e] = a;
    s_pre[e] = bl;
  }
  __syncthreads();
  build_plan<1024>(psm, T, E, tile_rows, has_shared, counts, expert_off, plan, tiles, blk == 0);
  const int t0 = blk * kSelBlock;
  for (int q = tid; q < kSelBlock * K; q += 1024) {
    const int tl = q / K, k = q - tl * K;
    const int t = t0 + tl;
    if (t >= T) continue;
    const size_t sk = size_t(t) * K + k;
    const int rk = rank[sk];
    int pos = -1;
    if (rk >= 0) {
      const int e = idx[sk];
      pos = psm.off[e] + s_pre[e] + rk;
      perm_token[pos] = t;
    }
    slot_pos[sk] = pos;
  }
}

// Whether the scan kernel also scatters (k_scan_scatter); the scatter launch
// is then empty.
static bool scan_scatters(const beam_moe_layer& L, int32_t T) {
  const int nblk = (T + kSelBlock - 1) / kSelBlock;
  int G = 1;
  while (2 * G * L.E <= 1024 && G < 64) G *= 2;
  return nblk <= long(G) * kScanVals;
}

hipError_t launch_scan(const beam_moe_layer& L, int32_t T, int tile_rows, const Ptrs& p,
                       hipStream_t s, bool all_pairs) {
  const int nblk = (T + kSelBlock - 1) / kSelBlock;
  if (scan_scatters(L, T)) {
    prof_before("scan_scatter", s);
    hipLaunchKernelGGL(k_scan_scatter, dim3(unsigned(nblk)), dim3(1024), 0, s, T, L.E, L.K, nblk,
                       tile_rows, (L.n_shared > 0 && !all_pairs) ? 1 : 0, p.block_counts, p.idx,
                       p.rank, p.counts, p.expert_off, p.plan, p.tiles, p.perm_token, p.slot_pos);
    prof_after(s);
    return hipGetLastError();
  }
  prof_before("scan_tiles", s);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, T, L.E, nblk, tile_rows,
                     (L.n_shared > 0 && !all_pairs) ? 1 : 0, p.block_counts, p.counts,
                     p.expert_off, p.plan, p.tiles);
  prof_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scatter (multi-block batches): position of every surviving pair in the
// expert-major compacted order (ascending expert, then ascending token), its
// token, and the per-slot position used by the combine (-1 for masked slots).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_scatter(int T, int E, int K, const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ rank,
                                                 const int32_t* __restrict__ block_off,
                                                 const int32_t* __restrict__ expert_off,
                                                 int32_t* __restrict__ perm_token,
                                                 int32_t* __restrict__ slot_pos) {
  const int blk = blockIdx.x;
  const int t0 = blk * kSelBlock;
  for (int q = threadIdx.x; q < kSelBlock * K; q += blockDim.x) {
    const int tl = q / K, k = q % K;
    const int t = t0 + tl;
    if (t >= T) continue;
    const size_t sk = size_t(t) * K + k;
    const int rk = rank[sk];
    int pos = -1;
    if (rk >= 0) {
      const int e = idx[sk];
      pos = expert_off[e] + block_off[size_t(blk) * E + e] + rk;
      perm_token[pos] = t;
    }
    slot_pos[sk] = pos;
  }
}

hipError_t launch_scatter(const beam_moe_layer& L, int32_t T, const Ptrs& p, hipStream_t s) {
  if (scan_scatters(L, T)) return hipSuccess;   // placed by the scan kernel
  const int nblk = (T + kSelBlock - 1) / kSelBlock;
  prof_before("scatter_pairs", s);
  hipLaunchKernelGGL(k_scatter, dim3(unsigned(nblk)), dim3(256), 0, s, T, L.E, L.K, p.idx, p.rank,
                     p.block_counts, p.expert_off, p.perm_token, p.slot_pos);
  prof_after(s);
  return hipGetLastError();
}

}  // namespace beam

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
// Router + mask-router logits: logits[t][j], j < E -> r_j, j >= E -> z_{j-E}
// (fp32, bias added).  Weight rows 0..2E-1 are Wr's rows then Wm's rows.
// ---------------------------------------------------------------------------

struct RouterArgs {
  const u16* x;
  const u16* wr;
  const u16* wm;
  const float* br;
  const float* bm;
  float* logits;
  int T, D, E;
};

__device__ __forceinline__ const u16* router_row(const RouterArgs& a, int j) {
  if (j < a.E) return a.wr + size_t(j) * a.D;
  if (j < 2 * a.E) return a.wm + size_t(j - a.E) * a.D;
  return nullptr;
}

__device__ __forceinline__ void router_store(const RouterArgs& a, int t, int j, float v) {
  if (t >= a.T || j >= 2 * a.E) return;
  float b = 0.f;
  if (j < a.E) {
    if (a.br) b = a.br[j];
  } else if (a.bm) {
    b = a.bm[j - a.E];
  }
  a.logits[size_t(t) * 2 * a.E + j] = v + b;
}

template <int MT>
struct RouterSkinnyProv {
  const RouterArgs* a;
  int j0, t0;
  __device__ int nseg() const { return 1; }
  __device__ int seg_chunks() const { return a->D / 64; }
  __device__ const u16* w(int, int r, int) const { return router_row(*a, j0 + r); }
  __device__ const u16* x(int r, int) const {
    const int t = t0 + r;
    return t < a->T ? a->x + size_t(t) * a->D : nullptr;
  }
};

// One workgroup per (16*MT tokens) x (16 router rows); 4 waves split k.
template <int MT>
__global__ __launch_bounds__(256) void k_router_skinny(RouterArgs a) {
  __shared__ f32x4 red[4 * MT * kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrb = (2 * a.E + 15) / 16;
  const int j0 = (blockIdx.x % nrb) * 16;
  const int t0 = (blockIdx.x / nrb) * 16 * MT;
  RouterSkinnyProv<MT> pv{&a, j0, t0};
  f32x4 acc[1][MT];
  skinny_accumulate<1, MT, (MT >= 4 ? 1 : 4 / MT)>(pv, lane, wave, 4, acc);
  skinny_reduce<1, MT>(acc, red, lane, wave, 4);
  // wave w stores the M tiles mt with mt % 4 == w
  for (int mt = wave; mt < MT; mt += 4) {
    f32x4 v = acc[0][0];
#pragma unroll
    for (int b = 0; b < MT; ++b)
      if (b == mt) v = acc[0][b];
    const int t = t0 + 16 * mt + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) router_store(a, t, j0 + 4 * (lane >> 4) + i, v[i]);
  }
}

template <int BM>
struct RouterTiledProv {
  const RouterArgs* a;
  int j0, t0;
  __device__ int nseg() const { return 1; }
  __device__ int seg_chunks() const { return a->D / 64; }
  __device__ const u16* w(int r, int) const { return router_row(*a, j0 + r); }
  __device__ const u16* x(int r, int) const {
    const int t = t0 + r;
    return t < a->T ? a->x + size_t(t) * a->D : nullptr;
  }
};

// One workgroup per (BM tokens) x (128 router rows).
template <int BM>
__global__ __launch_bounds__(256) void k_router_tiled(RouterArgs a) {
  __shared__ TiledSmem<BM> sm;
  const int nrb = (2 * a.E + kTBN - 1) / kTBN;
  const int j0 = (blockIdx.x % nrb) * kTBN;
  const int t0 = (blockIdx.x / nrb) * BM;
  RouterTiledProv<BM> pv{&a, j0, t0};
  f32x4 acc[4][BM / 32];
  tiled_accumulate<BM>(pv, sm, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
#pragma unroll
  for (int jn = 0; jn < 4; ++jn)
#pragma unroll
    for (int jm = 0; jm < BM / 32; ++jm) {
      const int t = t0 + wm * (BM / 2) + jm * 16 + (lane & 15);
      const int j = j0 + wn * 64 + jn * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) router_store(a, t, j + i, acc[jn][jm][i]);
    }
}

// fp32 layers: one thread per (token, router row), k in float4 steps.
struct RouterArgsF32 {
  const float* x;
  const float* wr;
  const float* wm;
  const float* br;
  const float* bm;
  float* logits;
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
  float b = 0.f;
  if (j < a.E) {
    if (a.br) b = a.br[j];
  } else if (a.bm) {
    b = a.bm[j - a.E];
  }
  a.logits[size_t(t) * R + j] = s + b;
}

hipError_t launch_router_logits(const beam_moe_layer& L, const void* x, int32_t T, float* logits,
                                hipStream_t s) {
  if (L.dtype == BEAM_F32) {
    RouterArgsF32 a{(const float*)x, (const float*)L.w_router, (const float*)L.w_mask, L.b_router,
                    L.b_mask, logits, T, L.D, L.E};
    const long n = long(T) * 2 * L.E;
    prof_before("router_logits_f32", s);
    hipLaunchKernelGGL(k_router_f32, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, a);
    prof_after(s);
    return hipGetLastError();
  }
  RouterArgs a{(const u16*)x, (const u16*)L.w_router, (const u16*)L.w_mask, L.b_router, L.b_mask,
               logits, T, L.D, L.E};
  if (T <= 64) {
    const int nrb = (2 * L.E + 15) / 16;
    const int mt = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
    const int ntb = (T + 16 * mt - 1) / (16 * mt);
    const dim3 grid(unsigned(nrb * ntb));
    prof_before("router_logits_skinny", s);
    if (mt == 1) hipLaunchKernelGGL(k_router_skinny<1>, grid, dim3(256), 0, s, a);
    else if (mt == 2) hipLaunchKernelGGL(k_router_skinny<2>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_router_skinny<4>, grid, dim3(256), 0, s, a);
    prof_after(s);
  } else {
    const int nrb = (2 * L.E + kTBN - 1) / kTBN;
    const int ntb = (T + 63) / 64;
    prof_before("router_logits_tiled", s);
    hipLaunchKernelGGL(k_router_tiled<64>, dim3(unsigned(nrb * ntb)), dim3(256), 0, s, a);
    prof_after(s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection: top-K by descending router logit (equal logits: lower expert
// index first), softmax over the K kept logits, mask bit m_k = [z >= 0] on
// the candidates, g_hat = g * m.  One workgroup per 64-token block; each wave
// handles 16 tokens.  Also computes, per block, the block-local rank of every
// surviving pair among the block's pairs of the same expert (token order) and
// the per-expert pair count of the block.
// ---------------------------------------------------------------------------

constexpr int kKeysPerLane = kMaxExperts / kWave;   // 16

__global__ __launch_bounds__(256) void k_select(const float* __restrict__ logits, int T, int E,
                                                int K, int32_t* __restrict__ idx,
                                                float* __restrict__ gates,
                                                uint32_t* __restrict__ mask,
                                                int32_t* __restrict__ rank,
                                                int32_t* __restrict__ block_counts) {
  __shared__ unsigned long long bits[kMaxExperts];
  __shared__ int32_t s_idx[kSelBlock * 32];
  __shared__ uint32_t s_mask[kSelBlock];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x;
  const int t0 = blk * kSelBlock;
  for (int e = tid; e < E; e += blockDim.x) bits[e] = 0ull;
  __syncthreads();

  const int nper = (E + kWave - 1) / kWave;
  for (int tl = wave; tl < kSelBlock; tl += 4) {
    const int t = t0 + tl;
    if (t >= T) break;
    const float* row = logits + size_t(t) * 2 * E;
    unsigned long long key[kKeysPerLane];
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
      const int e = lane + kWave * i;
      key[i] = 0ull;
      if (i < nper && e < E)
        key[i] = (static_cast<unsigned long long>(float_key(row[e])) << 32) |
                 static_cast<unsigned long long>(0xFFFFFFFFu - uint32_t(e));
    }
    // K rounds of a wave-wide maximum; round k only considers keys below the
    // previous winner (keys are distinct because they embed the index).
    unsigned long long mine = 0ull, prev = ~0ull;
    for (int k = 0; k < K; ++k) {
      unsigned long long lm = 0ull;
#pragma unroll
      for (int i = 0; i < kKeysPerLane; ++i)
        if (key[i] < prev && key[i] > lm) lm = key[i];
      const unsigned long long wmx = wave_max_u64(lm);
      if (lane == k) mine = wmx;
      prev = wmx;
    }
    const bool slot = lane < K;
    const int e_k = slot ? int(0xFFFFFFFFu - uint32_t(mine & 0xFFFFFFFFull)) : 0;
    const float r_k = slot ? row[e_k] : 0.f;
    const float r_0 = __shfl(r_k, 0, kWave);
    const float ex = slot ? expf(r_k - r_0) : 0.f;
    const float sum = wave_sum_f32(ex);
    const bool keep = slot && row[E + e_k] >= 0.f;
    const unsigned long long bal = __ballot(keep);
    if (slot) {
      idx[size_t(t) * K + lane] = e_k;
      gates[size_t(t) * K + lane] = keep ? ex / sum : 0.f;
      s_idx[tl * 32 + lane] = e_k;
    }
    if (lane == 0) {
      mask[t] = uint32_t(bal);
      s_mask[tl] = uint32_t(bal);
    }
    if (keep) atomicOr(&bits[e_k], 1ull << tl);
  }
  __syncthreads();

  for (int q = tid; q < kSelBlock * K; q += blockDim.x) {
    const int tl = q / K, k = q % K;
    const int t = t0 + tl;
    if (t >= T) continue;
    int rk = -1;
    if ((s_mask[tl] >> k) & 1u) {
      const int e = s_idx[tl * 32 + k];
      rk = __popcll(bits[e] & ((1ull << tl) - 1ull));
    }
    rank[size_t(t) * K + k] = rk;
  }
  for (int e = tid; e < E; e += blockDim.x)
    block_counts[size_t(blk) * E + e] = __popcll(bits[e]);
}

hipError_t launch_select(const beam_moe_layer& L, int32_t T, const Ptrs& p, hipStream_t s) {
  const int nblk = (T + kSelBlock - 1) / kSelBlock;
  prof_before("select_topk_mask", s);
  hipLaunchKernelGGL(k_select, dim3(unsigned(nblk)), dim3(256), 0, s, p.logits, T, L.E, L.K,
                     p.idx, p.gates, p.mask, p.rank, p.block_counts);
  prof_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scan (one workgroup): per-expert totals and per-block exclusive offsets,
// expert offsets in the compacted order, and the tile list.  Experts with no
// surviving pair get no tile, so their weights are never read.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void block_exclusive_scan(int32_t* v, int n, int32_t* tmp) {
  // Hillis-Steele over n <= 1024 entries with blockDim.x == 1024.
  const int tid = threadIdx.x;
  int32_t own = tid < n ? v[tid] : 0;
  tmp[tid] = own;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  if (tid < n) v[tid] = tmp[tid] - own;
  __syncthreads();
}

__global__ __launch_bounds__(1024) void k_scan(int T, int E, int nblk, int tile_rows,
                                               int has_shared, int32_t* __restrict__ block_counts,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ expert_off,
                                               Plan* __restrict__ plan, Tile* __restrict__ tiles) {
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts];
  __shared__ int32_t s_toff[kMaxExperts];
  __shared__ int32_t s_tmp[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    int32_t run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int32_t c = block_counts[size_t(b) * E + e];
      block_counts[size_t(b) * E + e] = run;
      run += c;
    }
    s_cnt[e] = run;
    counts[e] = run;
    s_off[e] = run;
    s_toff[e] = (run + tile_rows - 1) / tile_rows;
  }
  __syncthreads();
  const int32_t last_cnt = E > 0 ? s_cnt[E - 1] : 0;
  const int32_t last_tiles = E > 0 ? s_toff[E - 1] : 0;
  block_exclusive_scan(s_off, E, s_tmp);
  block_exclusive_scan(s_toff, E, s_tmp);
  const int32_t P = s_off[E - 1] + last_cnt;
  const int32_t ntr = s_toff[E - 1] + last_tiles;
  const int32_t nts = has_shared ? (T + tile_rows - 1) / tile_rows : 0;
  for (int e = tid; e < E; e += 1024) {
    expert_off[e] = s_off[e];
    const int c = s_cnt[e];
    const int nt = (c + tile_rows - 1) / tile_rows;
    for (int j = 0; j < nt; ++j) {
      Tile tl;
      tl.expert = e;
      tl.row0 = s_off[e] + j * tile_rows;
      tl.rows = min(tile_rows, c - j * tile_rows);
      tl.pad = 0;
      tiles[s_toff[e] + j] = tl;
    }
  }
  for (int j = tid; j < nts; j += 1024) {
    Tile tl;
    tl.expert = E;
    tl.row0 = j * tile_rows;
    tl.rows = min(tile_rows, T - j * tile_rows);
    tl.pad = 0;
    tiles[ntr + j] = tl;
  }
  // active experts
  int act = 0;
  for (int e = tid; e < E; e += 1024) act += s_cnt[e] > 0;
  s_tmp[tid] = act;
  __syncthreads();
  for (int off = 512; off >= 1; off >>= 1) {
    if (tid < off) s_tmp[tid] += s_tmp[tid + off];
    __syncthreads();
  }
  if (tid == 0) {
    expert_off[E] = P;
    Plan pl;
    pl.pairs = P;
    pl.n_tiles_routed = ntr;
    pl.n_tiles_shared = nts;
    pl.active_experts = s_tmp[0];
    *plan = pl;
  }
}

hipError_t launch_scan(const beam_moe_layer& L, int32_t T, int tile_rows, const Ptrs& p,
                       hipStream_t s) {
  const int nblk = (T + kSelBlock - 1) / kSelBlock;
  prof_before("scan_tiles", s);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, T, L.E, nblk, tile_rows,
                     L.n_shared > 0 ? 1 : 0, p.block_counts, p.counts, p.expert_off, p.plan,
                     p.tiles);
  prof_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scatter: position of every surviving pair in the expert-major compacted
// order (ascending expert, then ascending token), its token, and the
// per-slot position used by the combine (-1 for masked slots).
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
  const int nblk = (T + kSelBlock - 1) / kSelBlock;
  prof_before("scatter_pairs", s);
  hipLaunchKernelGGL(k_scatter, dim3(unsigned(nblk)), dim3(256), 0, s, T, L.E, L.K, p.idx, p.rank,
                     p.block_counts, p.expert_off, p.perm_token, p.slot_pos);
  prof_after(s);
  return hipGetLastError();
}

}  // namespace beam

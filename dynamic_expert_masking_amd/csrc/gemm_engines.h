// Two bf16 MFMA matrix-product engines for the BEAM kernels.
//
// Both compute, for one output tile, acc = W_rows . X_rows^T, where W rows
// are weight rows (the "n" dimension: expert intermediate rows, output
// features or router rows) and X rows are token rows (the "m" dimension),
// both contiguous along k.  Operands come from a provider object:
//
//   int nseg()            number of k segments (a shared-expert group is one
//                         segment per shared expert; otherwise 1)
//   int seg_chunks()      64-wide k chunks per segment
//   const u16* w(r, seg)  start of weight row r of the tile in segment seg,
//                         or nullptr (row absent: reads as zeros)
//   const u16* x(r, seg)  start of token row r of the tile, or nullptr
//
// Skinny engine (decode-shaped tiles): 16 weight rows per matrix (NMAT
// matrices, e.g. gate and up) x 16*MT token rows.  Weights stream from HBM
// straight into MFMA operand registers (each weight element is used by at
// most MT MFMAs, so staging through LDS buys nothing); the k range is split
// across the workgroup's waves and the partial sums are added through LDS in
// a fixed wave order, so results do not depend on timing.
//
// Tiled engine (prefill-shaped tiles): BN = 128 weight rows x BM token rows,
// both staged through LDS in 64-wide k slices with double buffering; 4 waves
// in a 2 x 2 layout each own a 64 x BM/2 sub-tile of 16 x 16 MFMA blocks.
#pragma once
#include <type_traits>

#include "device_common.h"

namespace beam {

// ---------------------------------------------------------------------------
// Skinny engine
// ---------------------------------------------------------------------------

// acc[mat][mt][i] = sum_k W_mat[row 4*(lane/16)+i][k] * X[row 16*mt + lane%16][k]
// over this wave's share of the k chunks.
template <int NMAT, int MT, int U, class Prov>
__device__ __forceinline__ void skinny_accumulate(const Prov& pv, int lane, int wave, int nwaves,
                                                  f32x4 (&acc)[NMAT][MT]) {
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int b = 0; b < MT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nseg = pv.nseg();
  const int cps = pv.seg_chunks();
  const int C = nseg * cps;
  const int c_begin = (C * wave) / nwaves;
  const int c_end = (C * (wave + 1)) / nwaves;
  // Lane l covers k = 16*(l/16) .. +15 of each 64-wide chunk: two MFMAs per
  // chunk, the first on elements 0..7, the second on 8..15 (same mapping for
  // both operands).
  const int koff = (lane >> 4) * 16;
  const int r = lane & 15;

  for (int seg = c_begin / cps; seg < nseg && seg * cps < c_end; ++seg) {
    const int lo = max(c_begin, seg * cps) - seg * cps;
    const int hi = min(c_end, (seg + 1) * cps) - seg * cps;
    const u16* wp[NMAT];
    const u16* xp[MT];
#pragma unroll
    for (int a = 0; a < NMAT; ++a) {
      const u16* p = pv.w(a, r, seg);
      wp[a] = p ? p + koff : nullptr;
    }
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const u16* p = pv.x(16 * b + r, seg);
      xp[b] = p ? p + koff : nullptr;
    }
    for (int c = lo; c < hi; c += U) {
      u32x4 wv[U][NMAT][2];
      u32x4 xv[U][MT][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = (c + u) * 64;
        const bool ok = (c + u) < hi;
#pragma unroll
        for (int a = 0; a < NMAT; ++a) {
          wv[u][a][0] = zero16();
          wv[u][a][1] = zero16();
          if (ok && wp[a]) {
            wv[u][a][0] = ld16_stream(wp[a] + k);
            wv[u][a][1] = ld16_stream(wp[a] + k + 8);
          }
        }
#pragma unroll
        for (int b = 0; b < MT; ++b) {
          xv[u][b][0] = zero16();
          xv[u][b][1] = zero16();
          if (ok && xp[b]) {
            xv[u][b][0] = ld16(xp[b] + k);
            xv[u][b][1] = ld16(xp[b] + k + 8);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if ((c + u) < hi) {
#pragma unroll
          for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int b = 0; b < MT; ++b) {
              acc[a][b] = mfma_bf16(wv[u][a][0], xv[u][b][0], acc[a][b]);
              acc[a][b] = mfma_bf16(wv[u][a][1], xv[u][b][1], acc[a][b]);
            }
        }
      }
    }
  }
}

// Adds the waves' partial sums in wave order 0, 1, ..., nwaves-1.  red is an
// LDS array of nwaves * NMAT * MT * 64 f32x4.  On return every wave holds
// the full sums in acc (only the entries it later uses matter).  Ends with a
// barrier so red may be reused.
template <int NMAT, int MT>
__device__ __forceinline__ void skinny_reduce(f32x4 (&acc)[NMAT][MT], f32x4* red, int lane,
                                              int wave, int nwaves) {
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int b = 0; b < MT; ++b) red[((wave * NMAT + a) * MT + b) * kWave + lane] = acc[a][b];
  __syncthreads();
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      f32x4 s = red[((0 * NMAT + a) * MT + b) * kWave + lane];
      for (int w = 1; w < nwaves; ++w) s += red[((w * NMAT + a) * MT + b) * kWave + lane];
      acc[a][b] = s;
    }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Tiled engine (prefill-shaped tiles)
//
// One workgroup of 4 waves computes a tile of BN weight rows x BM token rows
// (BN x BM = 256 x 128 or 128 x 256); waves sit in a 2 x 2 layout and each
// owns BN/2 weight rows x BM/2 token rows as blocks of 32 x 32 MFMAs
// (v_mfma_f32_32x32x16_bf16, fp32 accumulators; 8 blocks per wave, so two
// workgroups fit on a CU and cover each other's barrier waits).  The k range
// is walked in 64-wide slices: the next slice of both operands is loaded from
// global memory into registers (coalesced 16-byte loads, 8 lanes per 128-byte
// row segment, 32-bit offsets from a uniform base) while the current slice is
// multiplied out of a padded LDS tile (row stride 144 bytes, so the 16 rows
// read by 16 consecutive lanes hit distinct banks).  Loads are branch-free:
// absent rows read row 0 of their operand and the slice past the end reads
// the first element of its bases, so the compiler's load counters stay exact;
// absent rows only feed accumulator rows or columns that the epilogues never
// store.  The MFMA loop is branch-free too: the number of a wave's 32-token
// blocks that hold valid rows is decided once per tile (a wave-uniform
// value), and the slice loop is instantiated for each count.
// ---------------------------------------------------------------------------

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16_at(const u16* base, uint32_t elem_off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + size_t(elem_off) * 2);
}
__device__ __forceinline__ u32x4 ld16_at_stream(const u16* base, uint32_t elem_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + size_t(elem_off) * 2));
}

constexpr int kTBK = 64;            // k slice
constexpr int kTLD = kTBK + 8;      // padded LDS row (bf16 elements)

template <int BN, int BM>
struct TiledSmem {
  u16 w[BN * kTLD];
  u16 x[BM * kTLD];
};

// Calls f(std::integral_constant<int, n>) for the runtime n in 0..J.
template <int J, class F>
__device__ __forceinline__ void tiled_dispatch(int n, F&& f) {
  if constexpr (J == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (n >= J) f(std::integral_constant<int, J>{});
    else tiled_dispatch<J - 1>(n, f);
  }
}

// Provider interface (per tile):
//   int nseg(), seg_chunks()
//   const u16* wbase(g, seg)    uniform base of weight rows [32g, 32g+32) in segment seg
//   uint32_t   woff(r)          element offset of weight row r (0..BN-1) from its base
//   const u16* xbase(seg)       uniform base of the token rows in segment seg
//   uint32_t   xoff(r)          element offset of token row r (0..BM-1) from xbase
// acc[jn][jm][i] = C[n = (BN/2)*(wave&1) + 32*jn + 8*(i/4) + 4*(lane/32) + i%4]
//                   [m = (BM/2)*(wave>>1) + 32*jm + lane%32]
// MFMAs of 32-row token blocks at or past rows_valid are skipped.
// k chunks [c_lo, c_hi) of the provider's nseg * seg_chunks (c_hi < 0: to
// the end), for a k split of the product.
template <int BN, int BM, class Prov>
__device__ __forceinline__ void tiled_accumulate(const Prov& pv, TiledSmem<BN, BM>& sm,
                                                 f32x16 (&acc)[BN / 64][BM / 64], int rows_valid,
                                                 int c_lo = 0, int c_hi = -1) {
  constexpr int JN = BN / 64, JM = BM / 64;
  constexpr int WL = BN / 32;   // weight chunks per thread per slice
  constexpr int XL = BM / 32;   // token chunks per thread per slice
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is uniform across the wave; readfirstlane lets the compiler
  // know it, so per-wave decisions below are scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
#pragma unroll
  for (int a = 0; a < JN; ++a)
#pragma unroll
    for (int b = 0; b < JM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int nseg = pv.nseg();
  const int cps = pv.seg_chunks();
  const int C = c_hi < 0 ? nseg * cps : c_hi;
  const int lrow = tid >> 3;          // 0..31
  const int lcol = (tid & 7) * 8;     // element offset of this thread's 16 bytes
  uint32_t wo[WL], xo[XL];
#pragma unroll
  for (int i = 0; i < WL; ++i) wo[i] = pv.woff(lrow + 32 * i) + lcol;
#pragma unroll
  for (int i = 0; i < XL; ++i) xo[i] = pv.xoff(lrow + 32 * i) + lcol;

  struct Stage {
    u32x4 w[WL];
    u32x4 x[XL];
  };
  // The slice past the end reads the first element of the last segment's
  // bases (all lanes the same line), so that every call issues the same
  // loads.  Its offsets are masked to zero with integer arithmetic: a select
  // between two base pointers can become a branch around each load, and the
  // join of such branches makes the compiler wait for every load in flight.
  auto load = [&](Stage& st, int c) {
    const uint32_t msk = c < C ? ~0u : 0u;
    const int cc = max(min(c, C - 1), 0);   // an empty range reads chunk 0
    const int seg = cc / cps;
    const uint32_t km = uint32_t(cc - seg * cps) * kTBK;
    const u16* xb = pv.xbase(seg);
#pragma unroll
    for (int i = 0; i < WL; ++i)   // this thread's row lrow + 32 i lies in row group i
      st.w[i] = ld16_at_stream(pv.wbase(i, seg), (wo[i] + km) & msk);
#pragma unroll
    for (int i = 0; i < XL; ++i) st.x[i] = ld16_at(xb, (xo[i] + km) & msk);
  };
  auto store = [&](const Stage& st) {
#pragma unroll
    for (int i = 0; i < WL; ++i)
      *reinterpret_cast<u32x4*>(&sm.w[(lrow + 32 * i) * kTLD + lcol]) = st.w[i];
#pragma unroll
    for (int i = 0; i < XL; ++i)
      *reinterpret_cast<u32x4*>(&sm.x[(lrow + 32 * i) * kTLD + lcol]) = st.x[i];
  };
  const int fr = lane & 31;
  const int fk = (lane >> 5) * 8;
  // The first NJ of this wave's 32-token blocks, straight-line code.
  auto compute = [&](auto nj_const) {
    constexpr int NJ = decltype(nj_const)::value;
#pragma unroll
    for (int ks = 0; ks < kTBK / 16; ++ks) {
      u32x4 wf[JN], xf[NJ > 0 ? NJ : 1];
#pragma unroll
      for (int jn = 0; jn < JN; ++jn)
        wf[jn] = *reinterpret_cast<const u32x4*>(
            &sm.w[(wn * (BN / 2) + jn * 32 + fr) * kTLD + ks * 16 + fk]);
#pragma unroll
      for (int jm = 0; jm < NJ; ++jm)
        xf[jm] = *reinterpret_cast<const u32x4*>(
            &sm.x[(wm * (BM / 2) + jm * 32 + fr) * kTLD + ks * 16 + fk]);
#pragma unroll
      for (int jm = 0; jm < NJ; ++jm)
#pragma unroll
        for (int jn = 0; jn < JN; ++jn) acc[jn][jm] = mfma32_bf16(wf[jn], xf[jm], acc[jn][jm]);
    }
  };
  auto run = [&](auto nj_const) {
    Stage st;
    load(st, c_lo);
    for (int c = c_lo; c < C; ++c) {
      store(st);          // slice c
      __syncthreads();
      load(st, c + 1);    // in flight while slice c is multiplied
      // Issue all of the next slice's loads before the MFMAs (the scheduler
      // otherwise sinks some of them below the first MFMAs).
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(nj_const)::value > 0) compute(nj_const);
      __syncthreads();
    }
  };
  // Token blocks of this wave that hold valid rows (a wave-uniform count),
  // chosen once per tile so the slice loop has no branches around its MFMAs.
  const int nj = min(JM, max(0, (rows_valid - wm * (BM / 2) + 31) / 32));
  tiled_dispatch<JM>(nj, run);
}

// The tiled engine with both operands double-buffered in LDS, for tiles
// whose MFMAs per slice are few (the router's 64 x 128 tiles: 8 per wave):
// tiled_accumulate's slice loop (store, barrier, load, multiply, barrier)
// leaves each slice's load latency and LDS round trip exposed, and took
// 27 us for the fine-grained T = 8192 router even with every load an L2 hit.
// Here iteration c issues the loads of slice c + 2, multiplies slice c out
// of buffer c % 2 (all of its fragment reads issued first), stores slice
// c + 1 (loaded during iteration c - 1) into the other buffer, whose slice
// c - 1 was read before the last barrier, and ends with the one barrier
// (that router on MI355X: 34.2 -> 30.0 us).  Full k range only; same
// provider and accumulator layout.
template <int BN, int BM>
struct TiledSmem2 {
  u16 w[2][BN * kTLD];
  u16 x[2][BM * kTLD];
};

template <int BN, int BM, class Prov>
__device__ __forceinline__ void tiled_accumulate_db(const Prov& pv, TiledSmem2<BN, BM>& sm,
                                                    f32x16 (&acc)[BN / 64][BM / 64], int rows_valid) {
  constexpr int JN = BN / 64, JM = BM / 64;
  constexpr int WL = BN / 32;
  constexpr int XL = BM / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
#pragma unroll
  for (int a = 0; a < JN; ++a)
#pragma unroll
    for (int b = 0; b < JM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  const int cps = pv.seg_chunks();
  const int C = pv.nseg() * cps;
  const int lrow = tid >> 3;
  const int lcol = (tid & 7) * 8;
  uint32_t wo[WL], xo[XL];
#pragma unroll
  for (int i = 0; i < WL; ++i) wo[i] = pv.woff(lrow + 32 * i) + lcol;
#pragma unroll
  for (int i = 0; i < XL; ++i) xo[i] = pv.xoff(lrow + 32 * i) + lcol;
  struct Stage {
    u32x4 w[WL];
    u32x4 x[XL];
  };
  // past the end: offset 0 of the last segment's bases (masked, no branch)
  auto load = [&](Stage& st, int c) {
    const uint32_t msk = c < C ? ~0u : 0u;
    const int cc = max(min(c, C - 1), 0);
    const int seg = cc / cps;
    const uint32_t km = uint32_t(cc - seg * cps) * kTBK;
    const u16* xb = pv.xbase(seg);
#pragma unroll
    for (int i = 0; i < WL; ++i) st.w[i] = ld16_at(pv.wbase(i, seg), (wo[i] + km) & msk);
#pragma unroll
    for (int i = 0; i < XL; ++i) st.x[i] = ld16_at(xb, (xo[i] + km) & msk);
  };
  auto store = [&](const Stage& st, int buf) {
#pragma unroll
    for (int i = 0; i < WL; ++i)
      *reinterpret_cast<u32x4*>(&sm.w[buf][(lrow + 32 * i) * kTLD + lcol]) = st.w[i];
#pragma unroll
    for (int i = 0; i < XL; ++i)
      *reinterpret_cast<u32x4*>(&sm.x[buf][(lrow + 32 * i) * kTLD + lcol]) = st.x[i];
  };
  const int fr = lane & 31;
  const int fk = (lane >> 5) * 8;
  auto run = [&](auto nj_const) {
    constexpr int NJ = decltype(nj_const)::value;
    auto compute = [&](int buf) {
      u32x4 wf[4][JN], xf[4][NJ > 0 ? NJ : 1];
#pragma unroll
      for (int ks = 0; ks < kTBK / 16; ++ks) {
#pragma unroll
        for (int jn = 0; jn < JN; ++jn)
          wf[ks][jn] = *reinterpret_cast<const u32x4*>(
              &sm.w[buf][(wn * (BN / 2) + jn * 32 + fr) * kTLD + ks * 16 + fk]);
#pragma unroll
        for (int jm = 0; jm < NJ; ++jm)
          xf[ks][jm] = *reinterpret_cast<const u32x4*>(
              &sm.x[buf][(wm * (BM / 2) + jm * 32 + fr) * kTLD + ks * 16 + fk]);
      }
#pragma unroll
      for (int ks = 0; ks < kTBK / 16; ++ks)
#pragma unroll
        for (int jm = 0; jm < NJ; ++jm)
#pragma unroll
          for (int jn = 0; jn < JN; ++jn) acc[jn][jm] = mfma32_bf16(wf[ks][jn], xf[ks][jm], acc[jn][jm]);
    };
    Stage st[2];
    load(st[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load(st[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    store(st[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    auto step = [&](int c, Stage& nxt_load, const Stage& to_store, int buf) {
      load(nxt_load, c + 2);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NJ > 0) compute(buf);
      __builtin_amdgcn_sched_barrier(0);
      store(to_store, buf ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };
    int c = 0;
    for (; c + 2 <= C; c += 2) {
      step(c, st[0], st[1], 0);
      step(c + 1, st[1], st[0], 1);
    }
    if (c < C) step(c, st[0], st[1], 0);
  };
  const int nj = min(JM, max(0, (rows_valid - wm * (BM / 2) + 31) / 32));
  tiled_dispatch<JM>(nj, run);
}

// Persistent, XCD-aware work split: workgroups are dispatched round-robin over
// the 8 XCDs (b % 8), so the item space is cut into 8 contiguous parts and the
// workgroups of one XCD stride through its part.  Items that share operands
// and are adjacent in the item order then meet in the same L2.
constexpr int kXcds = 8;

struct XcdRange {
  long next, step, end;
};

__device__ __forceinline__ XcdRange xcd_range(long total) {
  const long G = gridDim.x;
  const long groups = G >= kXcds ? kXcds : 1;
  const long x = blockIdx.x % groups;
  const long per = G / groups;                  // workgroups per XCD part
  const long li = blockIdx.x / groups;
  XcdRange r;
  const long p0 = total * x / groups, p1 = total * (x + 1) / groups;
  r.next = li < per ? p0 + li : p1;             // leftover workgroups idle
  r.step = per;
  r.end = p1;
  return r;
}

// Dynamic item order for persistent kernels whose items differ in length
// (tiles of different heights, shared and routed items): a workgroup starts
// with item blockIdx.x, then takes the next value of a device counter (zeroed
// before the launch by the kernel that writes the plan) plus the grid size.
// Items are handed out in order over the whole chip, so the items that run
// at once are neighbours in the item order, as xcd_range's parts are, but on
// every XCD.  Thread 0 claims the following item when an item starts, so the
// atomic's latency overlaps the item's first loads, and hands it to the other
// threads through LDS when the item ends.  slot is a __shared__ int[2]: the
// two alternate, so one barrier per item suffices.
struct ItemQueue {
  int* counter;
  int* slot;
  int par = 0;
  int nxt = 0;
  __device__ ItemQueue(int* c, int* s) : counter(c), slot(s) {}
  __device__ void claim() {
    if (threadIdx.x == 0) nxt = atomicAdd(counter, 1) + int(gridDim.x);
  }
  __device__ long next() {
    if (threadIdx.x == 0) slot[par] = nxt;
    __syncthreads();
    const long v = slot[par];
    par ^= 1;
    return v;
  }
};

}  // namespace beam

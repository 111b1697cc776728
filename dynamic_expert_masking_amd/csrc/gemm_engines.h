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
// Tiled engine
// ---------------------------------------------------------------------------

constexpr int kTBN = 128;           // weight rows per tile
constexpr int kTBK = 64;            // k slice
constexpr int kTLD = kTBK + 8;      // padded LDS row (bf16 elements)

template <int BM>
struct TiledSmem {
  u16 w[2][kTBN * kTLD];
  u16 x[2][BM * kTLD];
};

// acc[jn][jm][i] = C[n = 64*(wave&1) + 16*jn + 4*(lane/16) + i]
//                   [m = (BM/2)*(wave>>1) + 16*jm + lane%16]
template <int BM, class Prov>
__device__ __forceinline__ void tiled_accumulate(const Prov& pv, TiledSmem<BM>& sm,
                                                 f32x4 (&acc)[4][BM / 32]) {
  constexpr int JM = BM / 32;
  constexpr int XL = BM / 32;   // X chunks per thread per slice (BM*8/256)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < JM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nseg = pv.nseg();
  const int cps = pv.seg_chunks();
  const int C = nseg * cps;
  const int lrow = tid >> 3;          // 0..31
  const int lcol = (tid & 7) * 8;     // element offset of this thread's 16 bytes

  const u16* wr[4];
  const u16* xr[XL];
  auto set_rows = [&](int seg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u16* p = pv.w(lrow + 32 * i, seg);
      wr[i] = p ? p + lcol : nullptr;
    }
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const u16* p = pv.x(lrow + 32 * i, seg);
      xr[i] = p ? p + lcol : nullptr;
    }
  };
  u32x4 wreg[4], xreg[XL];
  auto load = [&](int cc) {
    const int k = cc * kTBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) wreg[i] = wr[i] ? ld16_stream(wr[i] + k) : zero16();
#pragma unroll
    for (int i = 0; i < XL; ++i) xreg[i] = xr[i] ? ld16(xr[i] + k) : zero16();
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&sm.w[buf][(lrow + 32 * i) * kTLD + lcol]) = wreg[i];
#pragma unroll
    for (int i = 0; i < XL; ++i)
      *reinterpret_cast<u32x4*>(&sm.x[buf][(lrow + 32 * i) * kTLD + lcol]) = xreg[i];
  };

  int seg = 0, cc = 0;
  set_rows(0);
  load(0);
  store(0);
  __syncthreads();
  const int fr = lane & 15;
  const int fk = (lane >> 4) * 8;
  for (int c = 0; c < C; ++c) {
    const int buf = c & 1;
    const bool more = (c + 1) < C;
    if (more) {
      if (++cc == cps) {
        cc = 0;
        ++seg;
        set_rows(seg);
      }
      load(cc);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 wf[4], xf[JM];
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        wf[jn] = *reinterpret_cast<const u32x4*>(
            &sm.w[buf][(wn * 64 + jn * 16 + fr) * kTLD + ks * 32 + fk]);
#pragma unroll
      for (int jm = 0; jm < JM; ++jm)
        xf[jm] = *reinterpret_cast<const u32x4*>(
            &sm.x[buf][(wm * (BM / 2) + jm * 16 + fr) * kTLD + ks * 32 + fk]);
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
#pragma unroll
        for (int jm = 0; jm < JM; ++jm) acc[jn][jm] = mfma_bf16(wf[jn], xf[jm], acc[jn][jm]);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }
}

}  // namespace beam

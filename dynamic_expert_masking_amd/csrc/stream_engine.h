// Streaming engine for decode-shaped expert products (bf16 MFMA).
//
// Each work item is one 16-row block of NMAT weight matrices (e.g. gate and
// up) applied to one tile of 16*MT token rows over the whole k range.
// Persistent workgroups of 4 waves take the items round-robin (workgroup b:
// items b, b + G, b + 2G, ...); within a workgroup, groups of KSPLIT waves
// share an item and split its k chunks (KSPLIT = 1: every wave streams whole
// items on its own).
//
// Memory access: weights are read with coalesced, non-temporal 16-byte loads
// in which 8 consecutive lanes cover one 128-byte line of a row, so every load
// instruction touches 8 whole lines (2 instructions per 16 rows x 64 k chunk).
// A wave-private LDS tile then turns each chunk into the MFMA operand layout
// (lane l: row l % 16, k = 8*(l/16) .. +7 and 32 + 8*(l/16) .. +7).  Token
// rows are small and cache-resident and are loaded straight in operand layout.
// Stages of U chunks are double-buffered in registers, so the next stage's
// loads are in flight while the current one is multiplied; the next item's
// first stage is issued before the current item's epilogue.
#pragma once
#include "device_common.h"

namespace beam {

constexpr int kStreamWaves = 4;
constexpr int kLdsRow = 72;   // 64 k values + 8 pad (bf16) per LDS tile row

// Per-item operand addresses, filled by the problem's decode().
template <int NMAT, int MT>
struct StreamItem {
  const u16* w[NMAT];    // first element (k = 0, segment 0) of row 0 of the block
  long w_row;            // elements between consecutive weight rows
  long w_seg;            // elements between segments
  const u16* x[MT];      // this lane's token row (row lane%16 of M tile mt) at k = 0;
                         // absent rows point at a safe dummy row
  long x_seg;            // elements between segments of a token row
  int nseg, cps;         // segments, 64-wide chunks per segment
  bool valid;            // false: no item; pointers are safe dummies (w_row = w_seg = 0)
};

template <int NMAT, int MT, int U>
struct StreamStage {
  u32x4 w[U][NMAT][2];
  u32x4 x[U][MT][2];
};

// Issues the loads of chunks c_begin .. c_begin+U-1 of an item.  Every call
// issues the same number of loads (chunks past c_end re-read the item's last
// chunk; absent items and token rows read a safe dummy address), so the
// compiler can count outstanding loads exactly and wait only for the stage it
// consumes.  consume() skips chunks past c_end and absent items, and an absent
// token row only feeds MFMA output columns that are never stored.
template <int NMAT, int MT, int U>
__device__ __forceinline__ void stream_issue(StreamStage<NMAT, MT, U>& st,
                                             const StreamItem<NMAT, MT>& it, int c_begin,
                                             int c_end, int lane) {
  const int wr = lane >> 3;            // coalesced: rows wr and wr + 8
  const int wc = (lane & 7) * 8;       // column (elements) within the chunk
  const int xk = (lane >> 4) * 8;      // operand layout k offset
  const int c_last = max(c_end - 1, 0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = min(c_begin + u, c_last);
    const int seg = c / it.cps;
    const int j = c - seg * it.cps;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const u16* p = it.w[m] + seg * it.w_seg + long(wr) * it.w_row + j * 64 + wc;
      st.w[u][m][0] = ld16_stream(p);
      st.w[u][m][1] = ld16_stream(p + 8 * it.w_row);
    }
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const u16* q = it.x[b] + seg * it.x_seg + j * 64 + xk;
      st.x[u][b][0] = ld16(q);
      st.x[u][b][1] = ld16(q + 32);
    }
  }
}

// LDS of one workgroup.  Each wave owns a region holding its transpose tiles:
// NMAT tiles of 16 x kLdsRow bf16, twice when a stage has several chunks (so
// consecutive chunks of a stage use alternate tiles).  With a k split, the
// partial sums of the wave are exchanged through the same region once the
// wave has consumed its share (a wave's LDS accesses complete in order).
template <int NMAT, int MT, int U, int KSPLIT>
struct StreamLds {
  static constexpr int kBufs = U > 1 ? 2 : 1;
  static constexpr int kTileBytes = kBufs * NMAT * 16 * kLdsRow * 2;
  static constexpr int kRedBytes = KSPLIT > 1 ? NMAT * MT * kWave * 16 : 0;
  static constexpr int kWaveBytes = kTileBytes > kRedBytes ? kTileBytes : kRedBytes;
  static constexpr int kBytes = kStreamWaves * kWaveBytes;
  static_assert(kWaveBytes % 16 == 0, "regions must stay 16-byte aligned");
};

// lds: this wave's transpose tiles (alternating per chunk when U > 1).
template <int NMAT, int MT, int U>
__device__ __forceinline__ void stream_consume(const StreamStage<NMAT, MT, U>& st, bool valid,
                                               int c_begin, int c_end, u16* lds, int lane,
                                               f32x4 (&acc)[NMAT][MT]) {
  const int wr = lane >> 3, wc = (lane & 7) * 8;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!valid || c_begin + u >= c_end) continue;
    u16* buf = lds + (U > 1 ? (u & 1) : 0) * NMAT * 16 * kLdsRow;
    u32x4 f[NMAT][2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      u16* t = buf + m * 16 * kLdsRow;
      *reinterpret_cast<u32x4*>(t + wr * kLdsRow + wc) = st.w[u][m][0];
      *reinterpret_cast<u32x4*>(t + (wr + 8) * kLdsRow + wc) = st.w[u][m][1];
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const u16* t = buf + m * 16 * kLdsRow;
      f[m][0] = *reinterpret_cast<const u32x4*>(t + fr * kLdsRow + fk);
      f[m][1] = *reinterpret_cast<const u32x4*>(t + fr * kLdsRow + 32 + fk);
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int b = 0; b < MT; ++b) {
        acc[m][b] = mfma_bf16(f[m][0], st.x[u][b][0], acc[m][b]);
        acc[m][b] = mfma_bf16(f[m][1], st.x[u][b][1], acc[m][b]);
      }
  }
}

// Runs the stream for one workgroup.  Problem P provides:
//   long total_items() const
//   void decode(long item, int lane, StreamItem<NMAT, MT>& it)   (sets it.valid)
//   void epilogue(long item, const f32x4 (&acc)[NMAT][MT], int lane)
// acc[m][b][i] = sum_k W_m[row 4*(lane/16)+i][k] * X[row 16*b + lane%16][k].
// lds_all: StreamLds<NMAT, MT, U, KSPLIT>::kBytes bytes, 16-byte aligned.
template <int NMAT, int MT, int U, int KSPLIT, class P>
__device__ __forceinline__ void stream_run(P& prob, unsigned char* lds_all) {
  using Lds = StreamLds<NMAT, MT, U, KSPLIT>;
  constexpr int GROUPS = kStreamWaves / KSPLIT;
  const int lane = threadIdx.x & 63;
  // wave-uniform, and known to be so: item decoding then stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave / KSPLIT, kw = wave % KSPLIT;
  u16* lds = reinterpret_cast<u16*>(lds_all + wave * Lds::kWaveBytes);
  auto red = [&](int w) { return reinterpret_cast<f32x4*>(lds_all + w * Lds::kWaveBytes); };

  // Items are dealt round-robin: the k-th item of workgroup b is b + G*k
  // (G = gridDim.x), taken by group k % GROUPS in round k / GROUPS.  The whole
  // grid thus sweeps the item list front to back, so the weight blocks in
  // flight at any time are neighbours and spread evenly over the HBM
  // channels; with G a multiple of 8, item i always runs on XCD i % 8.
  const long total = prob.total_items();
  const long G = gridDim.x;
  const long mine_n = total > long(blockIdx.x) ? (total - blockIdx.x + G - 1) / G : 0;
  const long rounds = (mine_n + GROUPS - 1) / GROUPS;
  if (rounds <= 0) return;   // uniform across the workgroup
  auto item_of = [&](long k) { return k < mine_n ? long(blockIdx.x) + G * k : -1L; };

  // this wave's chunk share [cb, ce) of an item with C chunks
  auto share = [&](const StreamItem<NMAT, MT>& it, int& cb, int& ce) {
    const int C = it.nseg * it.cps;
    cb = C * kw / KSPLIT;
    ce = C * (kw + 1) / KSPLIT;
  };

  StreamItem<NMAT, MT> cur, nxt;
  long item = item_of(group);
  prob.decode(item, lane, cur);
  int cb, ce;
  share(cur, cb, ce);
  StreamStage<NMAT, MT, U> A, B;
  stream_issue<NMAT, MT, U>(A, cur, cb, ce, lane);

  for (long r = 0; r < rounds; ++r) {
    const long nitem = item_of((r + 1) * GROUPS + group);
    prob.decode(nitem, lane, nxt);
    int nb, ne;
    share(nxt, nb, ne);
    f32x4 acc[NMAT][MT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int b = 0; b < MT; ++b) acc[m][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stages of this round: c = cb, cb + U, ...; A holds the first.  Pairs
    // (A, B) keep buffer roles static.  The next round's first stage is issued
    // as soon as this round's last stage is in flight; it lands in A, or in B
    // when the round has an odd number of stages (then moved to A after the
    // epilogue, by which time its loads have had the epilogue to complete).
    bool next_in_b = false;
    for (int c = cb; c < ce; c += 2 * U) {
      const int c2 = c + U;
      if (c2 < ce) {
        stream_issue<NMAT, MT, U>(B, cur, c2, ce, lane);
      } else {
        stream_issue<NMAT, MT, U>(B, nxt, nb, ne, lane);
        next_in_b = true;
      }
      stream_consume<NMAT, MT, U>(A, cur.valid, c, ce, lds, lane, acc);
      if (c2 < ce) {
        const int c3 = c2 + U;
        if (c3 < ce) stream_issue<NMAT, MT, U>(A, cur, c3, ce, lane);
        else stream_issue<NMAT, MT, U>(A, nxt, nb, ne, lane);
        stream_consume<NMAT, MT, U>(B, cur.valid, c2, ce, lds, lane, acc);
      }
    }
    if (ce <= cb) stream_issue<NMAT, MT, U>(A, nxt, nb, ne, lane);   // empty share
    // combine the group's partial sums (fixed wave order) and finish the item
    if (KSPLIT > 1) {
      f32x4* mine = red(wave);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int b = 0; b < MT; ++b) mine[(m * MT + b) * kWave + lane] = acc[m][b];
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int b = 0; b < MT; ++b) {
            f32x4 s = acc[m][b];
            for (int w = 1; w < KSPLIT; ++w) s += red(wave + w)[(m * MT + b) * kWave + lane];
            acc[m][b] = s;
          }
        if (cur.valid) prob.epilogue(item, acc, lane);
      }
      __syncthreads();
    } else if (cur.valid) {
      prob.epilogue(item, acc, lane);
    }
    if (next_in_b) A = B;
    cur = nxt;
    cb = nb;
    ce = ne;
    item = nitem;
  }
}

}  // namespace beam

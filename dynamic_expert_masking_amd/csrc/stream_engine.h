// Streaming engine for decode-shaped expert products (bf16 MFMA).
//
// Each work item is one 16-row block of NMAT weight matrices (e.g. gate and
// up) applied to one tile of 16*MT token rows over the whole k range.
// Persistent workgroups of 4 waves take the items round-robin (workgroup b:
// items b, b + G, b + 2G, ...); within a workgroup, groups of KSPLIT waves
// share an item and split its k chunks (KSPLIT = 1: every wave streams whole
// items on its own).
//
// Memory access: weights are read in chunks of 128 bytes of each of the 16
// rows (64 k values of bf16, or 128 of FP8 E4M3), with coalesced,
// non-temporal 16-byte loads in which 8 consecutive lanes cover one 128-byte
// line of a row, so every load instruction touches 8 whole lines (2
// instructions per chunk).  A wave-private LDS tile then turns each chunk
// into the MFMA operand layout (lane l: row l % 16 and 8 consecutive k
// values).  FP8 codes go through the tile as they are and are widened to
// bf16, exactly, in registers after the fragment reads (one round trip per
// chunk; widening first and sending the two halves through the tile took
// two: DeepSeek-V2-Lite FP8 shapes on MI355X, see stream_consume).  Token rows are small and cache-resident
// and are loaded straight in operand layout.  Stages of U chunks are
// double-buffered in registers, so the next stage's loads are in flight while
// the current one is multiplied; the next item's first stage is issued before
// the current item's epilogue.
//
// FP8 weights carry one float32 scale per row: products are accumulated
// unscaled and multiplied by the row scales at the end of each k segment
// (segments are separate matrices, e.g. the fused shared experts' down
// projections, each with its own scales).
#pragma once
#include "device_common.h"

namespace beam {

constexpr int kStreamWaves = 4;
constexpr int kLdsRow = 72;   // 64 bf16 values + 8 pad per LDS tile row

// k values per 128-byte chunk of a weight row.
template <bool F8>
constexpr int chunk_k() { return F8 ? 128 : 64; }

// Per-item operand addresses, filled by the problem's decode().
template <int NMAT, int MT>
struct StreamItem {
  const unsigned char* w[NMAT];  // first byte (k = 0, segment 0) of row 0 of the block
  long w_row;            // bytes between consecutive weight rows
  long w_seg;            // bytes between segments
  const u16* x[MT];      // this lane's token row (row lane%16 of M tile mt) at k = 0;
                         // absent rows point at a safe dummy row
  long x_seg;            // elements between segments of a token row
  int nseg, cps;         // segments, 128-byte chunks per segment row
  bool valid;            // false: no item; pointers are safe dummies (w_row = w_seg = 0)
};

// Token operands per chunk and M tile: bf16 chunks hold two MFMA k-steps,
// FP8 chunks four.
template <int NMAT, int MT, int U, bool F8>
struct StreamStage {
  static constexpr int kX = chunk_k<F8>() / 32;
  u32x4 w[U][NMAT][2];
  u32x4 x[U][MT][kX];
};

// Issues the loads of chunks c_begin .. c_begin+U-1 of an item.  Every call
// issues the same number of loads (chunks past c_end re-read the item's last
// chunk; absent items and token rows read a safe dummy address), so the
// compiler can count outstanding loads exactly and wait only for the stage it
// consumes.  consume() skips chunks past c_end and absent items, and an absent
// token row only feeds MFMA output columns that are never stored.
//
// k order inside a chunk (applied to weights and tokens alike, which leaves
// the products unchanged): bf16 k-step q of lane group s = lane/16 covers
// k = 32q + 8s .. +7; FP8 steps 0..3 cover k = 16s, 64 + 16s, 16s + 8 and
// 64 + 16s + 8 (.. +7): the low and then the high 8 codes of the two 16-code
// fragments a lane reads from the LDS tile.
template <int NMAT, int MT, int U, bool F8>
__device__ __forceinline__ void stream_issue(StreamStage<NMAT, MT, U, F8>& st,
                                             const StreamItem<NMAT, MT>& it, int c_begin,
                                             int c_end, int lane) {
  constexpr int KC = chunk_k<F8>();
  const int wr = lane >> 3;            // coalesced: rows wr and wr + 8
  const int wb = (lane & 7) * 16;      // byte column within the chunk
  const int xk = (lane >> 4) * (F8 ? 16 : 8);   // operand layout k offset
  const int c_last = max(c_end - 1, 0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = min(c_begin + u, c_last);
    const int seg = c / it.cps;
    const int j = c - seg * it.cps;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const unsigned char* p = it.w[m] + seg * it.w_seg + long(wr) * it.w_row + j * 128 + wb;
      st.w[u][m][0] = ld16_stream(p);
      st.w[u][m][1] = ld16_stream(p + 8 * it.w_row);
    }
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const u16* q = it.x[b] + seg * it.x_seg + j * KC + xk;
      if constexpr (F8) {
        st.x[u][b][0] = ld16(q);
        st.x[u][b][1] = ld16(q + 64);
        st.x[u][b][2] = ld16(q + 8);
        st.x[u][b][3] = ld16(q + 72);
      } else {
        st.x[u][b][0] = ld16(q);
        st.x[u][b][1] = ld16(q + 32);
      }
    }
  }
}

// LDS of one workgroup.  Each wave owns a region holding its transpose tiles:
// NMAT tiles of 16 x kLdsRow bf16, twice when a stage has several chunks (so
// consecutive chunks of a stage use alternate tiles).  With a k split, the
// partial sums of the wave are exchanged through the same region once the
// wave has consumed its share (a wave's LDS accesses complete in order).
template <int NMAT, int MT, int U, int KSPLIT>
struct StreamLds {   // (the same for bf16 and FP8 weights)
  static constexpr int kBufs = U > 1 ? 2 : 1;
  static constexpr int kTileBytes = kBufs * NMAT * 16 * kLdsRow * 2;
  static constexpr int kRedBytes = KSPLIT > 1 ? NMAT * MT * kWave * 16 : 0;
  static constexpr int kWaveBytes = kTileBytes > kRedBytes ? kTileBytes : kRedBytes;
  static constexpr int kBytes = kStreamWaves * kWaveBytes;
  static_assert(kWaveBytes % 16 == 0, "regions must stay 16-byte aligned");
};

// lds: this wave's transpose tiles (alternating per chunk when U > 1).
// chunk_end(c) runs after the MFMAs of chunk c (FP8 segment scaling).
template <int NMAT, int MT, int U, bool F8, class CE>
__device__ __forceinline__ void stream_consume(const StreamStage<NMAT, MT, U, F8>& st, bool valid,
                                               int c_begin, int c_end, u16* lds, int lane,
                                               f32x4 (&acc)[NMAT][MT], CE&& chunk_end) {
  const int wr = lane >> 3, wc = (lane & 7) * 8;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!valid || c_begin + u >= c_end) continue;
    u16* buf = lds + (U > 1 ? (u & 1) : 0) * NMAT * 16 * kLdsRow;
    if constexpr (F8) {
      // The raw codes go through the tile (each lane's 16 bytes at the place
      // its 8 widened bf16 values would take) and are widened after the
      // fragment reads: one LDS round trip per chunk instead of one per half.
      // Lane l reads codes k = 16 (l/16) .. +15 and 64 + 16 (l/16) .. +15 of
      // row l % 16; their low 8 codes are k-steps 0 and 1, their high 8
      // steps 2 and 3 (the order of the token operands), and the MFMAs run
      // in the same order as when each half went through the tile.
      u32x4 r[NMAT][2];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        u16* t = buf + m * 16 * kLdsRow;
        *reinterpret_cast<u32x4*>(t + wr * kLdsRow + wc) = st.w[u][m][0];
        *reinterpret_cast<u32x4*>(t + (wr + 8) * kLdsRow + wc) = st.w[u][m][1];
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const u16* t = buf + m * 16 * kLdsRow;
        r[m][0] = *reinterpret_cast<const u32x4*>(t + fr * kLdsRow + fk);
        r[m][1] = *reinterpret_cast<const u32x4*>(t + fr * kLdsRow + 32 + fk);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const u32x4 f0 = e4m3x8_to_bf16(r[m][0][2 * hf], r[m][0][2 * hf + 1]);
          const u32x4 f1 = e4m3x8_to_bf16(r[m][1][2 * hf], r[m][1][2 * hf + 1]);
#pragma unroll
          for (int b = 0; b < MT; ++b) {
            acc[m][b] = mfma_bf16(f0, st.x[u][b][2 * hf], acc[m][b]);
            acc[m][b] = mfma_bf16(f1, st.x[u][b][2 * hf + 1], acc[m][b]);
          }
        }
    } else {
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
      // x steps 0, 1
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int b = 0; b < MT; ++b) {
          acc[m][b] = mfma_bf16(f[m][0], st.x[u][b][0], acc[m][b]);
          acc[m][b] = mfma_bf16(f[m][1], st.x[u][b][1], acc[m][b]);
        }
    }
    chunk_end(c_begin + u);
  }
}

// Runs the stream for one workgroup.  Problem P provides:
//   long total_items() const
//   void decode(long item, int lane, StreamItem<NMAT, MT>& it)   (sets it.valid)
//   void epilogue(long item, const f32x4 (&acc)[NMAT][MT], int lane)
// and, for FP8 weights (F8 = true):
//   void scales(long item, int seg, int lane, f32x4 (&sc)[NMAT])
//     (scales of this lane's accumulator rows of each matrix in segment seg)
//   static constexpr bool kMultiSeg   (items may have several segments)
// acc[m][b][i] = sum_k W_m[row 4*(lane/16)+i][k] * X[row 16*b + lane%16][k],
// with W_m the scaled weights for FP8.
// lds_all: StreamLds<NMAT, MT, U, KSPLIT>::kBytes bytes, 16-byte aligned.
template <int NMAT, int MT, int U, int KSPLIT, bool F8, class P>
__device__ __forceinline__ void stream_run(P& prob, unsigned char* lds_all, long n0 = 0) {
  using Lds = StreamLds<NMAT, MT, U, KSPLIT>;
  using Stage = StreamStage<NMAT, MT, U, F8>;
  constexpr int GROUPS = kStreamWaves / KSPLIT;
  const int lane = threadIdx.x & 63;
  // wave-uniform, and known to be so: item decoding then stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave / KSPLIT, kw = wave % KSPLIT;
  u16* lds = reinterpret_cast<u16*>(lds_all + wave * Lds::kWaveBytes);
  auto red = [&](int w) { return reinterpret_cast<f32x4*>(lds_all + w * Lds::kWaveBytes); };

  // Items are dealt round-robin: the k-th item of workgroup b is b + G*k
  // (G = gridDim.x; less n0, see below), taken by group k % GROUPS in round
  // k / GROUPS.  The whole
  // grid thus sweeps the item list front to back, so the weight blocks in
  // flight at any time are neighbours and spread evenly over the HBM
  // channels; with G a multiple of 8, item i always runs on XCD i % 8.
  // n0 leading slots of the deal belong to cooperative items (run before by
  // stream_coop_run); this workgroup's k-th slot is blockIdx.x + G*k.
  const long total = prob.total_items();
  const long G = gridDim.x, b = blockIdx.x;
  const long k0 = n0 > b ? (n0 - b + G - 1) / G : 0;
  const long kend = n0 + total > b ? (n0 + total - b + G - 1) / G : 0;
  const long mine_n = kend - k0;
  const long rounds = (mine_n + GROUPS - 1) / GROUPS;
  if (rounds <= 0) return;   // uniform across the workgroup
  auto item_of = [&](long k) { return k < mine_n ? b + G * (k0 + k) - n0 : -1L; };

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
  Stage A, B;
  stream_issue<NMAT, MT, U, F8>(A, cur, cb, ce, lane);

  for (long r = 0; r < rounds; ++r) {
    const long nitem = item_of((r + 1) * GROUPS + group);
    prob.decode(nitem, lane, nxt);
    int nb, ne;
    share(nxt, nb, ne);
    f32x4 acc[NMAT][MT], tot[NMAT][MT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int b = 0; b < MT; ++b) acc[m][b] = tot[m][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // FP8: at the end of each segment (or of the share), tot += scales * acc;
    // single-segment items scale acc in place at the end of the share
    auto chunk_end = [&](int c) {
      if constexpr (F8) {
        if constexpr (P::kMultiSeg) {
          if ((c + 1) % cur.cps == 0 || c + 1 == ce) {
            f32x4 sc[NMAT];
            prob.scales(item, c / cur.cps, lane, sc);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int b = 0; b < MT; ++b) {
                tot[m][b] += sc[m] * acc[m][b];
                acc[m][b] = f32x4{0.f, 0.f, 0.f, 0.f};
              }
          }
        } else if (c + 1 == ce) {
          f32x4 sc[NMAT];
          prob.scales(item, 0, lane, sc);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int b = 0; b < MT; ++b) acc[m][b] *= sc[m];
        }
      }
    };
    // stages of this round: c = cb, cb + U, ...; A holds the first.  Pairs
    // (A, B) keep buffer roles static.  The next round's first stage is issued
    // as soon as this round's last stage is in flight; it lands in A, or in B
    // when the round has an odd number of stages (then moved to A after the
    // epilogue, by which time its loads have had the epilogue to complete).
    bool next_in_b = false;
    for (int c = cb; c < ce; c += 2 * U) {
      const int c2 = c + U;
      if (c2 < ce) {
        stream_issue<NMAT, MT, U, F8>(B, cur, c2, ce, lane);
      } else {
        stream_issue<NMAT, MT, U, F8>(B, nxt, nb, ne, lane);
        next_in_b = true;
      }
      stream_consume<NMAT, MT, U, F8>(A, cur.valid, c, ce, lds, lane, acc, chunk_end);
      if (c2 < ce) {
        const int c3 = c2 + U;
        if (c3 < ce) stream_issue<NMAT, MT, U, F8>(A, cur, c3, ce, lane);
        else stream_issue<NMAT, MT, U, F8>(A, nxt, nb, ne, lane);
        stream_consume<NMAT, MT, U, F8>(B, cur.valid, c2, ce, lds, lane, acc, chunk_end);
      }
    }
    if (ce <= cb) stream_issue<NMAT, MT, U, F8>(A, nxt, nb, ne, lane);   // empty share
    if constexpr (F8 && P::kMultiSeg) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int b = 0; b < MT; ++b) acc[m][b] = tot[m][b];
    }
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

// ---------------------------------------------------------------------------
// Cooperative items (bf16, 4 waves): several token tiles that read the same
// weight block -- the shared experts' tiles -- are taken by one workgroup,
// one tile per wave, so that the block is streamed once instead of once per
// tile.  Each wave loads a quarter of the k chunks (the k split of
// stream_run) and turns its chunk into the operand layout in its own LDS
// region; after a barrier every wave multiplies the four regions' chunks
// with its own token tile, and a second barrier frees the regions.  Every
// wave thus accumulates its tile over the whole k range, with no reduction.
//
// Problem P provides, besides what stream_run needs:
//   long coop_items() const
//   bool decode_coop(long item, int w, int lane, StreamItem<NMAT, MT>& it)
//        (weights of the item's block; token rows of the item's w-th tile;
//         returns false when the item has no w-th tile: its rows are dummies)
//   void epilogue_coop(long item, int w, const f32x4 (&acc)[NMAT][MT], int lane)
// Cooperative items take the first coop_items() slots of the round-robin deal
// (workgroup b: slots b, b + G, ...); stream_run then continues the deal.
// ---------------------------------------------------------------------------

template <int NMAT, int MT>
struct CoopStage {
  u32x4 w[NMAT][2];      // this wave's chunk of the block
  u32x4 x[4][MT][2];     // own tile's token operands for the four waves' chunks
};

// Chunk range [cb, ce) of wave w's quarter of C chunks.
__device__ __forceinline__ void coop_share(int C, int w, int& cb, int& ce) {
  cb = C * w / 4;
  ce = C * (w + 1) / 4;
}

// Chunk c of the item (segment-aware), clamped into [0, C).
template <int NMAT, int MT>
__device__ __forceinline__ void coop_load_w(CoopStage<NMAT, MT>& st, const StreamItem<NMAT, MT>& it,
                                            int c, int lane) {
  const int seg = c / it.cps, j = c - seg * it.cps;
  const int wr = lane >> 3, wb = (lane & 7) * 16;
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const unsigned char* p = it.w[m] + seg * it.w_seg + long(wr) * it.w_row + j * 128 + wb;
    st.w[m][0] = ld16_stream(p);
    st.w[m][1] = ld16_stream(p + 8 * it.w_row);
  }
}

// Loads of step s: this wave's chunk cb_w + s, and the token operands of
// every wave's chunk cb_r + s (clamped to the last chunk of each quarter;
// quarters that ran out are skipped in consume).
template <int NMAT, int MT>
__device__ __forceinline__ void coop_issue(CoopStage<NMAT, MT>& st, const StreamItem<NMAT, MT>& it,
                                           int C, int kw, int s, int lane) {
  const int xk = (lane >> 4) * 8;
  int cb, ce;
  coop_share(C, kw, cb, ce);
  coop_load_w(st, it, min(cb + s, max(ce - 1, 0)), lane);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int rb, re;
    coop_share(C, r, rb, re);
    const int c = min(rb + s, max(re - 1, 0));
    const int seg = c / it.cps, j = c - seg * it.cps;
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      const u16* q = it.x[b] + seg * it.x_seg + j * 64 + xk;
      st.x[r][b][0] = ld16(q);
      st.x[r][b][1] = ld16(q + 32);
    }
  }
}

template <int NMAT, int MT>
__device__ __forceinline__ void coop_consume(const CoopStage<NMAT, MT>& st, int C, int kw, int s,
                                             bool mine, unsigned char* lds_all, int wave_bytes,
                                             int lane, f32x4 (&acc)[NMAT][MT]) {
  const int wr = lane >> 3, wc = (lane & 7) * 8;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  int cb, ce;
  coop_share(C, kw, cb, ce);
  if (cb + s < ce) {
    u16* own = reinterpret_cast<u16*>(lds_all + kw * wave_bytes);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      u16* t = own + m * 16 * kLdsRow;
      *reinterpret_cast<u32x4*>(t + wr * kLdsRow + wc) = st.w[m][0];
      *reinterpret_cast<u32x4*>(t + (wr + 8) * kLdsRow + wc) = st.w[m][1];
    }
  }
  __syncthreads();
  if (mine) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int rb, re;
      coop_share(C, r, rb, re);
      if (rb + s >= re) continue;
      const u16* reg = reinterpret_cast<const u16*>(lds_all + r * wave_bytes);
      u32x4 f[NMAT][2];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const u16* t = reg + m * 16 * kLdsRow;
        f[m][0] = *reinterpret_cast<const u32x4*>(t + fr * kLdsRow + fk);
        f[m][1] = *reinterpret_cast<const u32x4*>(t + fr * kLdsRow + 32 + fk);
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int b = 0; b < MT; ++b) {
          acc[m][b] = mfma_bf16(f[m][0], st.x[r][b][0], acc[m][b]);
          acc[m][b] = mfma_bf16(f[m][1], st.x[r][b][1], acc[m][b]);
        }
    }
  }
  __syncthreads();
}

// Runs this workgroup's cooperative items (KSPLIT = 4 launches, bf16).
// lds_all: StreamLds<NMAT, MT, U, 4>::kBytes; wave_bytes: its kWaveBytes.
template <int NMAT, int MT, class P>
__device__ __forceinline__ void stream_coop_run(P& prob, unsigned char* lds_all, int wave_bytes) {
  const int lane = threadIdx.x & 63;
  const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long n = prob.coop_items();
  const long G = gridDim.x;
  for (long item = blockIdx.x; item < n; item += G) {
    StreamItem<NMAT, MT> it;
    const bool mine = prob.decode_coop(item, kw, lane, it);
    const int C = it.nseg * it.cps;
    int steps, e0;
    coop_share(C, 3, e0, steps);
    steps -= e0;   // the last quarter is the longest
    f32x4 acc[NMAT][MT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int b = 0; b < MT; ++b) acc[m][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    CoopStage<NMAT, MT> A, B;
    coop_issue(A, it, C, kw, 0, lane);
    for (int s = 0; s < steps; s += 2) {
      coop_issue(B, it, C, kw, s + 1, lane);
      coop_consume(A, C, kw, s, mine, lds_all, wave_bytes, lane, acc);
      if (s + 1 < steps) {
        coop_issue(A, it, C, kw, s + 2, lane);
        coop_consume(B, C, kw, s + 1, mine, lds_all, wave_bytes, lane, acc);
      }
    }
    if (mine) prob.epilogue_coop(item, kw, acc, lane);
  }
}

}  // namespace beam

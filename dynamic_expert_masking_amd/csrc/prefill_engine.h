// Prefill matrix-product engine for expert weights in the packed operand
// layout (gfx950).
//
// Packed layout of a weight matrix W [R][K] (R and K multiples of 32 and 64):
// blocks of 32 rows x 64 k, block (rb, kb) at element (rb * K/64 + kb) * 2048;
// inside a block, k-step s (16 k values) then lane l, 8 elements each:
//   packed[(rb * K/64 + kb) * 2048 + s * 512 + l * 8 + j]
//     = W[32 rb + l % 32][64 kb + 16 s + 8 (l / 32) + j],
// which is the A operand of v_mfma_f32_32x32x16_bf16 for lane l.  One wave's
// 16-byte loads of a k-step then read 1 KB of contiguous memory -- eight
// whole 128-byte lines -- straight into operand registers.  (Loads in the
// operand layout from row-major weights touch 32 lines per instruction and
// run at about a third of the rate, even from L2.)
//
// One workgroup of 4 waves computes an output tile of 256 weight rows x BM
// token rows (BM = 128) with fp32 accumulators.  Wave w owns weight rows
// [64 w, 64 w + 64) (two 32-row blocks) against all BM token rows, so every
// weight element is loaded by exactly one wave, kStages - 1 k slices ahead of
// its use.  Token rows are shared by the 4 waves through a ring of three LDS
// slice buffers: each 64-wide slice is loaded with coalesced 16-byte loads
// (8 lanes per 128-byte row segment) one slice ahead, and stored with the
// 16-byte chunks of each 128-byte row XOR-swizzled by (row / 2) % 8, so that
// the 16 lanes of an LDS phase hit distinct bank groups both when storing and
// when reading MFMA fragments.  One barrier per slice.  Loads are branch-free
// (absent rows read a valid row whose results are never stored; the slices
// past the end read offset 0 of their bases), and the MFMA loop is
// instantiated per count of valid 32-token blocks.
#pragma once
#include "beam_internal.h"
#include "device_common.h"
#include "gemm_engines.h"

namespace beam {

constexpr int kPK = 64;        // k slice (elements)
constexpr int kPStages = 3;   // weight slices held in registers per wave

template <int BM>
struct PrefillSmem {
  u16 x[3][BM * kPK];   // a ring of three token slices
};

constexpr int kPackBlock = 32 * kPK;   // elements of one packed 32 x 64 block

// Element offset, in a slice buffer, of the 16-byte chunk c (k = 8c .. 8c+7)
// of token row R.
__device__ __forceinline__ int prefill_x_off(int R, int c) {
  return R * kPK + 8 * (c ^ ((R >> 1) & 7));
}

// Provider interface (per tile):
//   int nseg(), seg_chunks()        k segments and 64-wide slices per segment
//   const u16* wbase(j, seg)        packed matrix of this wave's weight block j
//                                   (0 or 1) in segment seg
//   uint32_t wblk(j)                element offset of that block's row of
//                                   packed blocks (32 rb * seg_chunks * 64)
//   const u16* xbase(seg)           uniform base of the token rows
//   uint32_t xoff(R)                element offset of token row R (0..BM-1)
// On return acc[j][b][i] = C[n = 64 wave + 32 j + 8 (i / 4) + 4 (lane / 32) + i % 4]
//                          [m = 32 b + lane % 32]
// for the first NJ = ceil(rows_valid / 32) token blocks (the others are
// left at zero).
// k chunks [c_lo, c_hi) of the provider's nseg * seg_chunks (c_hi < 0: to the
// end), for a k split of the product.
template <int BM, class Prov>
__device__ __forceinline__ void prefill_accumulate(const Prov& pv, PrefillSmem<BM>& sm,
                                                   f32x16 (&acc)[2][BM / 32], int rows_valid,
                                                   int c_lo = 0, int c_hi = -1) {
  constexpr int JM = BM / 32;      // token blocks
  constexpr int XL = BM / 32;      // token chunks per thread per slice
  const int tid = threadIdx.x;
  const int lane = tid & 63;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < JM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][b][i] = 0.f;

  const int nseg = pv.nseg();
  const int cps = pv.seg_chunks();
  const int C = c_hi < 0 ? nseg * cps : c_hi;
  // weight operand offsets: this lane's 16 bytes of each packed k-step
  uint32_t wo[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wo[j] = pv.wblk(j) + 8 * lane;
  // token slice loads: rows tid / 8 + 32 i, chunk tid % 8
  const int trow = tid >> 3, tch = tid & 7;
  uint32_t xo[XL];
  int xl[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    xo[i] = pv.xoff(trow + 32 * i) + 8 * tch;
    xl[i] = prefill_x_off(trow + 32 * i, tch);
  }
  // fragment reads: row lane % 32 of each 32-token block, chunk 2 s + lane / 32
  int fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = prefill_x_off(lane & 31, 2 * s + (lane >> 5));

  struct WStage {
    u32x4 v[2][4];
  };
  struct XStage {
    u32x4 v[XL];
  };
  // Slice c of this wave's weights; past the end, offset 0 of the last
  // segment's bases (masked with integer arithmetic, so no branch).
  auto load_w = [&](WStage& st, int c) {
    const uint32_t msk = c < C ? ~0u : 0u;
    const int cc = max(min(c, C - 1), 0);   // an empty range reads chunk 0
    const int seg = cc / cps;
    const uint32_t kb = uint32_t(cc - seg * cps) * kPackBlock;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u16* b = pv.wbase(j, seg);
#pragma unroll
      for (int s = 0; s < 4; ++s) st.v[j][s] = ld16_at(b, (wo[j] + kb + 512 * s) & msk);
    }
  };
  auto load_x = [&](XStage& st, int c) {
    const uint32_t msk = c < C ? ~0u : 0u;
    const int cc = max(min(c, C - 1), 0);   // an empty range reads chunk 0
    const int seg = cc / cps;
    const uint32_t km = uint32_t(cc - seg * cps) * kPK;
    const u16* xb = pv.xbase(seg);
#pragma unroll
    for (int i = 0; i < XL; ++i) st.v[i] = ld16_at(xb, (xo[i] + km) & msk);
  };
  // store a token slice at LDS element offset buf (0, BM*64 or 2*BM*64)
  auto store_x_at = [&](const XStage& st, int buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) *reinterpret_cast<u32x4*>(&sm.x[0][buf + xl[i]]) = st.v[i];
  };
  auto store_x = [&](const XStage& st, int) { store_x_at(st, 0); };

  auto run = [&](auto nj_const) {
    constexpr int NJ = decltype(nj_const)::value;
    typedef u32x4 Frag[NJ];
    // fragments of k-step s of the slice at LDS element offset buf
    auto frag = [&](Frag& xf, int buf, int s) {
#pragma unroll
      for (int b = 0; b < NJ; ++b)
        xf[b] = *reinterpret_cast<const u32x4*>(&sm.x[0][buf + b * 32 * kPK + fo[s]]);
    };
    auto mma = [&](const WStage& w, const Frag& xf, int s) {
#pragma unroll
      for (int b = 0; b < NJ; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][b] = mfma32_bf16(w.v[j][s], xf[b], acc[j][b]);
    };
    // One k-step's MFMAs with the next k-step's fragment reads threaded
    // between them (one LDS read per two MFMAs), so that the reads are in
    // flight while the matrix unit is busy.
    auto overlap = [&](const WStage& w, const Frag& cur, int s, Frag& nxt, int nbuf, int ns) {
      frag(nxt, nbuf, ns);
      mma(w, cur, s);
#pragma unroll
      for (int b = 0; b < NJ; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two MFMAs
      }
    };
    // The same with the step's global loads threaded in as well, ceil(loads /
    // 2 NJ) after each pair of MFMAs of the first two k-steps, so that the
    // wave issues them while the matrix unit works through queued MFMAs
    // (DeepSeek-V2-Lite prefill T = 4096 on MI355X: gate/up 216 -> 208 us,
    // down 163 -> 159 us).
    auto overlap_v = [&](const WStage& w, const Frag& cur, int s, Frag& nxt, int nbuf, int ns) {
      frag(nxt, nbuf, ns);
      mma(w, cur, s);
      constexpr int VM = (XL + 8 + 2 * NJ - 1) / (2 * NJ);
#pragma unroll
      for (int b = 0; b < NJ; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two MFMAs
        __builtin_amdgcn_sched_group_barrier(0x020, VM, 0);  // global loads
      }
    };
    constexpr int SL = BM * kPK;   // elements per slice buffer
    WStage ws[kPStages];
    XStage xs;
    Frag fa, fb;
    // The prologue issues loads in the loop's pattern (token slice, then
    // weight slice), so that the compiler's wait counts agree at the loop
    // header with those inside the loop.
    load_x(xs, c_lo);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ws[0], c_lo);
    __builtin_amdgcn_sched_barrier(0);
    store_x(xs, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_x(xs, c_lo + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 1; q < kPStages - 1; ++q) load_w(ws[q], c_lo + q);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    frag(fa, 0, 0);
    int bcur = 0, bnxt = SL;   // LDS buffers of slices c and c + 1 (a ring of three)
    // Iteration c: store token slice c + 1 (loaded during iteration c - 1)
    // into the next buffer, issue the loads of token slice c + 2 and weight
    // slice c + kStages - 1, then multiply slice c.  The one barrier sits
    // after k-step 1: past it, slice c + 1 is in LDS (every wave stored its
    // part before the barrier), so k-step 0 of slice c + 1 is read during
    // k-step 3 of slice c; and the buffer written at iteration c + 1 (that
    // of slice c - 1) was last read before this barrier.
    // The token stores come first (a scheduling barrier), then the token
    // loads ahead of the weight loads, threaded among the MFMAs of the first
    // two k-steps: loads complete in issue order, so waiting for the token
    // slice before storing it must not also wait for weight loads issued
    // after it.
    auto step = [&](int c, const WStage& cur, WStage& nxt) {
      store_x_at(xs, bnxt);
      __builtin_amdgcn_sched_barrier(0);
      load_x(xs, c + 2);
      load_w(nxt, c + kPStages - 1);
      overlap_v(cur, fa, 0, fb, bcur, 1);
      overlap_v(cur, fb, 1, fa, bcur, 2);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      overlap(cur, fa, 2, fb, bcur, 3);
      __builtin_amdgcn_sched_barrier(0);
      overlap(cur, fb, 3, fa, bnxt, 0);
      __builtin_amdgcn_sched_barrier(0);
      const int bn = bnxt + SL;
      bcur = bnxt;
      bnxt = bn == 3 * SL ? 0 : bn;
    };
    // whole rounds of kStages slices (static stage indices), then the rest
    int c = c_lo;
    static_assert(kPStages == 3, "the loop is unrolled for three stages");
    for (; c + 3 <= C; c += 3) {
      step(c, ws[0], ws[2]);
      step(c + 1, ws[1], ws[0]);
      step(c + 2, ws[2], ws[1]);
    }
    if (c < C) step(c, ws[0], ws[2]);
    if (c + 1 < C) step(c + 1, ws[1], ws[0]);
    // the last fragment reads (of the slice past the end) are discarded;
    // the next tile's stores wait at its first barrier
    __syncthreads();
  };
  static_assert(BM == 128, "tiles of 128 token rows");
  const int nj = min(JM, max(1, (rows_valid + 31) / 32));
  tiled_dispatch<JM>(nj, [&](auto nj_const) {
    if constexpr (decltype(nj_const)::value > 0) run(nj_const);
  });
}

// ---------------------------------------------------------------------------
// Expert-stationary engine: one workgroup multiplies a 128-row block of
// weights (four packed 32-row blocks) with every token of one tile of up to
// kEsTileRows rows, so each weight block of an expert is read from HBM once
// per tile instead of once per 128-token tile.  The roles of the packed
// engine above are swapped: the weight slice (16 KB per 64-wide k slice)
// goes through a ring of three LDS buffers and is shared by the 4 waves;
// each wave takes the tile's 32-token blocks w, w + 4, w + 8 and loads them
// straight into MFMA operand registers from a packed copy of the tokens (the
// same block layout as the packed weights: block (tb, kb) of a tile at
// element (tb * C + kb) * 2048, lane l's 16 bytes of k-step s at s * 512 +
// l * 8).  Weight and token slices are both held in three rotating register
// stages; one barrier per slice, after its third k-step, so that the
// fragments of the next slice's first k-step are read during its fourth.
// ---------------------------------------------------------------------------

constexpr int kEsTokBlocks = kEsTileRows / 32;   // tokens of one tile: 12 blocks of 32
constexpr int kEsWaveBlocks = kEsTokBlocks / 4;   // token blocks per wave
constexpr int kEsWBlocks = 4;               // 32-row weight blocks per workgroup

struct EsSmem {
  u16 w[3][kEsWBlocks * kPackBlock];   // three weight slice buffers (a ring)
};

// Provider interface (per item):
//   int chunks()                   64-wide k slices of the product
//   const u16* wbase(bb)           packed matrix of weight block bb (0..3), at
//                                  its row of packed blocks
//   uint32_t wslice(c)             element offset of k slice c from wbase (c *
//                                  kPackBlock within one packed matrix)
//   const u16* xbase()             packed tokens of the tile (block row 0)
// On return acc[bb][j][i] = C[n = 32 bb + 8 (i / 4) + 4 (lane / 32) + i % 4]
//                            [m = 32 tb_j + lane % 32]
// for the token blocks tb_j = es_token_block(wave, j, nbt) < nbt (the others
// are left at zero); for j = 2 only the weight blocks bb that
// es_block_valid(wave, bb, nbt) accepts.
//
// Token blocks of a wave: w, w + 4, w + 8, except in tiles of 9 or 10
// blocks.  There the third block would fall to one or two waves, which
// would then take half as long again as the others at every barrier;
// instead blocks 8 and 9 are split by weight-block parity: waves 0 and 1
// take block 8, waves 2 and 3 block 9, each with the weight blocks of its
// own parity (w % 2 and w % 2 + 2 -- a gate block and the up block of the
// same rows).  The busiest wave then issues 40 MFMAs per slice instead of
// 48.
__device__ __forceinline__ bool es_split_tile(int nbt) { return nbt == 9 || nbt == 10; }
__device__ __forceinline__ int es_token_block(int wave, int j, int nbt) {
  if (j < 2 || !es_split_tile(nbt)) return wave + 4 * j;
  return 8 + wave / 2;
}
__device__ __forceinline__ bool es_block_valid(int wave, int bb, int nbt) {
  return !es_split_tile(nbt) || ((bb ^ wave) & 1) == 0;
}
template <class Prov>
__device__ __forceinline__ void es_accumulate(const Prov& pv, EsSmem& sm,
                                              f32x16 (&acc)[kEsWBlocks][kEsWaveBlocks], int nbt) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int b = 0; b < kEsWBlocks; ++b)
#pragma unroll
    for (int j = 0; j < kEsWaveBlocks; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][j][i] = 0.f;
  const int C = pv.chunks();
  // weight slice loads: thread tid takes block tid / 64, its lane's 16 bytes
  // of the four k-steps
  const int wbb = tid >> 6;
  const u16* wb = pv.wbase(wbb) + 8 * lane;
  const u16* xb = pv.xbase() + 8 * lane;
  // this wave's token blocks w + 4 j (wave-uniform count), and the block
  // it shares in a tile of 9 or 10 blocks (-1: none)
  const bool split = es_split_tile(nbt);
  const int nj = split ? 2 : min(kEsWaveBlocks, max(0, (nbt - wave + 3) / 4));
  const int xblk = split && es_token_block(wave, 2, nbt) < nbt ? es_token_block(wave, 2, nbt) : -1;

  struct WStage {
    u32x4 v[4];
  };
  struct XStage {
    u32x4 v[kEsWaveBlocks][4];
  };
  auto load_w = [&](WStage& st, int c) {
    const uint32_t off = pv.wslice(min(c, C - 1));   // past the end: the last slice
#pragma unroll
    for (int s = 0; s < 4; ++s) st.v[s] = ld16_at_stream(wb, off + 512 * s);
  };
  auto store_w = [&](const WStage& st, int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      *reinterpret_cast<u32x4*>(&sm.w[buf][wbb * kPackBlock + 512 * s + 8 * lane]) = st.v[s];
  };

  // NJ own token blocks; XP = 0, or 1 + p: block xblk too, with the weight
  // blocks of parity p
  auto run = [&](auto nj_const, auto xp_const) {
    constexpr int NJ = decltype(nj_const)::value;
    constexpr int XP = decltype(xp_const)::value;
    constexpr int NT = NJ + (XP ? 1 : 0);   // token blocks loaded
    auto load_x = [&](XStage& st, int c) {
      const int cc = min(c, C - 1);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int tb = j < NJ ? wave + 4 * j : xblk;
        const uint32_t off = uint32_t(tb * C + cc) * kPackBlock;
#pragma unroll
        for (int s = 0; s < 4; ++s) st.v[j][s] = ld16_at(xb, off + 512 * s);
      }
    };
    WStage ws[3];
    XStage xs[3];
    u32x4 wf[kEsWBlocks];   // block b's fragment of the next k-step to multiply
    auto wl = [&](int buf) { return &sm.w[buf][8 * lane]; };
    // K-steps S0 .. S1 - 1 of slice c (LDS buffer buf) in groups of (weight
    // block b, k-step s): the group's NJ MFMAs, then VM of the step's global
    // loads (while any remain, k-steps 0-2), one store of the next weight
    // slice into LDS (the groups of k-step 2), and the read of block b's
    // fragment of the following k-step -- k-step 0 of slice c + 1 (buffer
    // nbuf) after k-step 3 -- into the register the MFMAs just consumed.
    // A fragment read then has three groups of MFMAs to arrive, and the wave
    // issues its loads and stores while the matrix unit works through queued
    // MFMAs instead of ahead of them; the grouping is pinned with
    // scheduling-group barriers (left alone, the compiler sinks every read
    // to just before its MFMAs).  Mixtral-shaped T = 2048 on MI355X, gate/up
    // / down: 583 / 283 us with loads, stores and reads in blocks, 551 / 265
    // with the loads threaded, 572 / 273 with the stores too (two buffers,
    // stores after the last read), 557 / 265 with this ring of three.
    auto ksteps = [&](const XStage& xs, int buf, int nbuf, auto s0c, auto s1c) {
      constexpr int S0 = decltype(s0c)::value, S1 = decltype(s1c)::value;
      constexpr int NL = 4 * NT + 4;
      constexpr int VM = (NL + 11) / 12;
#pragma unroll
      for (int s = S0; s < S1; ++s) {
#pragma unroll
        for (int b = 0; b < kEsWBlocks; ++b) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[b][j] = mfma32_bf16(wf[b], xs.v[j][s], acc[b][j]);
          const bool X = XP != 0 && (b & 1) == XP - 1;   // a constant after unrolling
          if (X) acc[b][NJ] = mfma32_bf16(wf[b], xs.v[NJ][s], acc[b][NJ]);
          if (NJ > 0) __builtin_amdgcn_sched_group_barrier(0x008, NJ, 0);   // MFMAs
          if (X) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (s < 3 && VM * (4 * s + b) < NL) __builtin_amdgcn_sched_group_barrier(0x020, VM, 0);
          if (s == 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS store
          wf[b] = *reinterpret_cast<const u32x4*>(s < 3 ? wl(buf) + b * kPackBlock + 512 * (s + 1)
                                                        : wl(nbuf) + b * kPackBlock);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
      }
    };
    // Stage k % 3 holds slice k, LDS buffer k % 3 too.  Loads complete in
    // issue order, so each iteration issues its token slice before its
    // weight slice: waiting for a token slice then never waits for a weight
    // slice issued later.  The prologue issues x0, w0, w1, x1, w2, as the
    // loop would have.
    load_x(xs[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ws[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ws[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    load_x(xs[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ws[2], 2);
    __builtin_amdgcn_sched_barrier(0);
    store_w(ws[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kEsWBlocks; ++b) wf[b] = *reinterpret_cast<const u32x4*>(wl(0) + b * kPackBlock);
    // Iteration c: issue token slice c + 2 and weight slice c + 3, multiply
    // k-steps 0-2 of slice c while storing weight slice c + 1 into its
    // buffer (that of slice c - 2, last read before the previous barrier),
    // barrier, then k-step 3 while reading k-step 0 of slice c + 1.  A weight
    // slice has two iterations to arrive, a token slice two.
    auto step = [&](int c, WStage& wstore, XStage& xcur, XStage& xnext, WStage& wnext, int buf,
                    int nbuf) {
      load_x(xnext, c + 2);
      load_w(wnext, c + 3);
      ksteps(xcur, buf, nbuf, std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
      store_w(wstore, nbuf);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      ksteps(xcur, buf, nbuf, std::integral_constant<int, 3>{}, std::integral_constant<int, 4>{});
      __builtin_amdgcn_sched_barrier(0);
    };
    int c = 0;
    for (; c + 3 <= C; c += 3) {
      step(c, ws[1], xs[0], xs[2], ws[0], 0, 1);
      step(c + 1, ws[2], xs[1], xs[0], ws[1], 1, 2);
      step(c + 2, ws[0], xs[2], xs[1], ws[2], 2, 0);
    }
    if (c < C) step(c, ws[1], xs[0], xs[2], ws[0], 0, 1);
    if (c + 1 < C) step(c + 1, ws[2], xs[1], xs[0], ws[1], 1, 2);
    // the last fragment reads (of the slice past the end) are discarded;
    // the next item's stores wait at its first barrier
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  if (xblk >= 0) {
    if (wave & 1) run(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
  } else {
    tiled_dispatch<kEsWaveBlocks>(nj, [&](auto nj_const) { run(nj_const, I0{}); });
  }
}

}  // namespace beam

// Indexer score (page "GLM5 TensorCast 适配设计", section "DSA Indexer fused
// semantic op": cache scoring, head-weight mixing and head reduction;
// section "Performance model design", buckets "q-k index score MMA" and
// "head weight multiply, head reduce, relu / q-scale / k-scale shaping"):
//
//     score[t, s] = kscale[s] * sum_h w[t, h] * max(q[t, h, :] . k[s, :], 0)
//
// for every causal key s <= pos(t), written as fp32 into a [N, row_stride]
// scratch matrix that the top-k kernel reads.  kscale is 1 except for an
// FP8 cache, whose key value is code * scale; the scale is positive, so it is
// applied after the head sum.
//
// Matrix-core path (bf16 query, bf16 or e4m3 keys, n_heads % 32 == 0,
// d_idx == 128): one v_mfma_f32_32x32x16_bf16 tile has the 32 heads of one
// query token on M and 32 keys on N, contracting 16 of the 128 dims per
// instruction.  The 32x32 accumulator leaves each lane with one key column
// and 16 of the 32 head rows, so ReLU * w and 16 of the 32 head terms are
// summed in-lane and one cross-half exchange finishes the head reduction.
// A workgroup is 4 waves sharing one query block (1 or 2 tokens of a
// request) and one key chunk; each wave streams 32-key tiles of the paged
// cache straight from HBM into a private LDS ring (DMA, non-temporal) and
// reads them back as MFMA operands.  Keys of an e4m3 cache are widened
// exactly to bf16 with the hardware conversion.
//
// Vector path: any dtype / shape within the documented limits, one thread
// per (query token, key), fp32 arithmetic.
#include <utility>

#include "common.h"

namespace dsa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));   // 32 e4m3 codes

constexpr int kTile = 32;      // keys per MFMA tile
constexpr int kWaves = 4;      // waves per workgroup
// Dim mapping of the MFMA operands.  Lane half hf = lane / 32 and K-step s
// (0..7) hold 8 consecutive dims starting at:
//   bf16 keys: 16 s + 8 hf   (one 16-byte load per step, natural order)
//   fp8 keys:  64 hf + 8 s   (each lane half reads 64 contiguous bytes)
// The query operand uses the same mapping, so every product pairs q[d]
// with k[d].
template <bool FP8>
__device__ __forceinline__ int dim_of(int hf, int s) {
  return FP8 ? (64 * hf + 8 * s) : (16 * s + 8 * hf);
}

// ------------------------------------------------- keys through LDS
// Same contraction, but the keys reach LDS by DMA (global_load_lds_dwordx4)
// in whole 1 KB lines: one wave instruction carries 4 consecutive 256-byte
// bf16 rows (or 8 128-byte e4m3 rows).  Each wave streams its own tiles
// through a private ring of kRing buffers, each refilled as soon as its
// tile has been read into registers (kRing tiles in flight while the wave
// multiplies), so no barrier is ever needed; the MFMA key operand is read back with
// ds_read_b128 (e4m3 bytes widened to bf16 in registers).  Lane l of DMA
// instruction m lands at byte 16 l of block m; piece p (16 bytes) of row r
// sits at slot p ^ (r % P) of the row (P pieces per row), which spreads
// the 32 rows of one operand load over distinct banks.  An e4m3 tile's 32
// scales follow its rows (one 4-byte DMA per lane, two copies).
constexpr int kRing = 2;       // bf16 tiles (8 KiB) in flight per wave
constexpr int kRingF8 = 2;     // e4m3 tiles (4.25 KiB) in flight per wave (3 or 4 measured slower)
static_assert(kRing >= 2 && kRing <= 4 && kRingF8 >= 2 && kRingF8 <= 4,
              "tile waits cover rings of 2 to 4 tiles");
constexpr int kMaxTpw = 64;                      // tiles per wave (one block id per lane)
template <bool F8>
struct DmaTile {
  static constexpr int kRowBytes = F8 ? 128 : 256;
  static constexpr int kPieces = kRowBytes / 16;            // 16-byte pieces per row
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;
  static constexpr int kKeyInstr = kTile / kRowsPerInstr;   // 4 or 8
  static constexpr int kInstr = kKeyInstr + (F8 ? 1 : 0);   // + the scales
  static constexpr int kScaleOff = kTile * kRowBytes;       // scales after the rows
  static constexpr int kBytes = kScaleOff + (F8 ? 256 : 0);
};

// f(integral_constant<int, I>) for I = 0 .. N-1 (indices usable as
// constants, e.g. for register arrays)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int OFF>
__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ float lds_f32(uint32_t addr) {
  float r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int N, typename T>
__device__ __forceinline__ void lgkm_keep(T& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "n"(N));
}
// s_waitcnt on the vector-memory count only (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// s_waitcnt vmcnt(I later): a tile is I DMA instructions, so the tile
// issued `later` tiles before the newest one has landed
template <int I>
__device__ __forceinline__ void wait_tile(int later) {
  switch (later) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<I>(); break;
    case 2: wait_vm<2 * I>(); break;
    default: wait_vm<3 * I>(); break;
  }
}

// MAXT: tiles per wave the LDS score buffer holds.  With 16 (launches of
// several rounds) two workgroups share a CU, so one's start overlaps the
// other's stream.
// QF8: e4m3 queries (rotated, quantised per head, q_scale per token and
// head) against an e4m3 cache, contracted on the fp8 matrix cores.
// SPAN: launches of several rounds over requests of one query token each
// (long varlen rows).  A fixed grid of workgroups (two per CU) splits the
// batch's key tiles evenly: the requests' tiles, each request's rounded up
// to whole 128-key range chunks, are laid end to end and workgroup g takes
// the g-th equal share, in pieces of up to 4 MAXT tiles.  No workgroup is
// launched without work and they all finish together; the score ranges
// (for the top-k's long rows) are then recorded per 32-key tile.
template <int TQ, int MT, bool F8, int MAXT, bool QF8 = false, bool SPAN = false>
__global__ __launch_bounds__(256, MAXT <= 32 ? 2 : 1) void k_score_dma(
    const uint16_t* __restrict__ q, const float* __restrict__ qscale,
    const float* __restrict__ w,
    const uint8_t* __restrict__ kc, const float* __restrict__ kscale,
    const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ block_table,
    int32_t max_blocks, int32_t block_size, int64_t num_slots,
    int32_t max_seq_len, int32_t qblocks_per_req, int32_t nchunks,
    int32_t tiles_per_wave_arg, float* __restrict__ scores, int64_t row_stride,
    float2* __restrict__ crange, int32_t range_stride, int32_t B, int32_t win_lo,
    int32_t win_hi) {
  constexpr int H = 32 * MT;
  static_assert(!QF8 || F8, "e4m3 queries go with an e4m3 cache");
  using DT = DmaTile<F8>;
  static_assert(kWaves == kRangeParts, "one range entry per wave and chunk");
  constexpr int RING = F8 ? kRingF8 : kRing;
  __shared__ __align__(16) uint8_t ring[kWaves][RING][DT::kBytes];
  // the workgroup's scores, [token][key within chunk], written out at the
  // end: score stores interleaved with the key stream slow the reads down
  __shared__ __align__(16) float sc[TQ][kWaves * MAXT * kTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;
  const int col = lane & 31;

  static_assert(!SPAN || TQ == 1, "spans cover requests of one query token");
  // One chunk: the tiles from key_beg up to key_lim (and the query block's
  // last position) of request b, query block qb, tiles_per_wave per wave.
  // chunk: its index among the request's range chunks (non-SPAN).
  auto run = [&](const int b, const int qb, const int32_t key_beg, const int tiles_per_wave,
                 const int32_t key_lim, const int chunk) {
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;

  // The wave's tiles are first_tile + kWaves i, i < ntiles (<= 64).  A
  // 32-key tile never spans two cache blocks, so one block-table entry
  // gives the whole tile.  Lane i fetches tile i's entry once, with a vector
  // load; each tile then takes it with v_readlane, so the tile loop issues
  // no scalar memory loads (a scalar load could only be waited for together
  // with every outstanding LDS read).  The tiles' places depend only on the
  // chunk, so the load is issued first, beside the request's length and
  // query range, rather than behind them: the first tile's address then
  // waits for one memory round trip instead of two.
  const int first_tile = key_beg / kTile + wave;
  int32_t bid_lane = -1;
  {
    const int32_t blk = (first_tile + kWaves * lane) * kTile / block_size;
    if (lane < tiles_per_wave && blk < max_blocks) bid_lane = bt_row[blk];
  }

  const int32_t L = min(seq_lens[b], max_seq_len);
  const int32_t tbeg = cu_q[b];
  const int32_t qlen = min(cu_q[b + 1] - tbeg, L);
  const int32_t t0 = qb * TQ;
  if (t0 >= qlen) return;
  const int nt = min(TQ, qlen - t0);
  // the block's tokens tbeg + t0 .. + nt - 1: nothing to do outside the window
  if (tbeg + t0 + nt <= win_lo || tbeg + t0 >= win_hi) return;
  const int32_t pos0 = L - qlen + t0;
  const int32_t key_end = min(pos0 + nt, key_lim);
  if (key_beg >= key_end) return;
  const int end_tile = (key_end + kTile - 1) / kTile;
  const int ntiles = end_tile > first_tile
                         ? min(tiles_per_wave, (end_tile - first_tile + kWaves - 1) / kWaves)
                         : 0;
  // query operand (head 32 mt + col, dims 16 s + 8 hf) and head weights
  // (accumulator register r of a 32x32 tile holds head 8 (r / 4) + 4 hf +
  // r % 4 of column col: four runs of 4 consecutive heads).  Issued after
  // the block-id load, so the first tile's address waits only for that,
  // and before any tile DMA, so waiting for them never waits for a tile.
  // The loads are unconditional (a block with one token loads that token
  // twice): the second token's scores are then never written out, and
  // branch-free loads leave the compiler's wait counting exact.
  // bf16 queries: qa[.][.][s] = dims dim_of(hf, s); e4m3 queries: qa8[.][.][s]
  // = the 32 code bytes of dims 64 s + 32 hf .. + 31 (the key operand takes
  // the same bytes of its row, so each product pairs equal dims)
  constexpr int QS = QF8 ? 1 : 8;
  constexpr int QS8 = QF8 ? 2 : 1;
  bf16x8 qa[TQ][MT][QS];
  i32x8 qa8[TQ][MT][QS8];
  float wr[TQ][MT][16];
#pragma unroll
  for (int tt = 0; tt < TQ; ++tt) {
    const int64_t tok = tbeg + t0 + (tt < nt ? tt : 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (QF8) {
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q) + (tok * H + mt * 32 + col) * 128;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * s + 32 * hf);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * s + 32 * hf + 16);
          qa8[tt][mt][s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
      } else {
        const uint16_t* qrow = q + (tok * H + mt * 32 + col) * 128;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          qa[tt][mt][s] = *reinterpret_cast<const bf16x8*>(qrow + dim_of<F8>(hf, s));
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t hw = tok * H + mt * 32 + 8 * g + 4 * hf;
        const float4 w4 = *reinterpret_cast<const float4*>(w + hw);
        float4 s4 = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        if constexpr (QF8) s4 = *reinterpret_cast<const float4*>(qscale + hw);
        // the query's scale joins its head weight (both multiply the head's
        // ReLU term; the scale is positive)
        wr[tt][mt][4 * g + 0] = w4.x * s4.x;
        wr[tt][mt][4 * g + 1] = w4.y * s4.y;
        wr[tt][mt][4 * g + 2] = w4.z * s4.z;
        wr[tt][mt][4 * g + 3] = w4.w * s4.w;
      }
    }
  }
  asm volatile("" ::: "memory");

  auto tile_row0 = [&](int i) -> int64_t {     // slot of the tile's first key, or -1
    if (i >= ntiles) return -1;
    const int32_t s0 = (first_tile + kWaves * i) * kTile;
    const int32_t bid = __builtin_amdgcn_readlane(bid_lane, i);
    const int64_t slot0 = static_cast<int64_t>(bid) * block_size + s0 % block_size;
    return (bid >= 0 && s0 / block_size < max_blocks && slot0 + kTile <= num_slots) ? slot0 : -1;
  };

  // DMA geometry of this lane: row R m + lane / P, slot lane % P (R rows
  // per instruction, P pieces per row)
  const int drow = lane / DT::kPieces;
  const int dslot = lane % DT::kPieces;
  // Each key is read once per call (all query tokens of a block share the
  // workgroup), so the DMA carries the non-temporal cache policy: streaming
  // reads then leave L2 and the last-level cache alone.
  constexpr int kStream = 2;   // cache-policy bits: nt
  auto dma = [&](int slot, int64_t row0) {
    uint8_t* buf = &ring[wave][slot][0];
    const int64_t base = row0 < 0 ? 0 : row0;
#pragma unroll
    for (int m = 0; m < DT::kKeyInstr; ++m) {
      const int row = DT::kRowsPerInstr * m + drow;
      const int piece = dslot ^ (row % DT::kPieces);
      const uint8_t* src = kc + (base + row) * DT::kRowBytes + 16 * piece;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(buf + 1024 * m), 16, 0, kStream);
    }
    if constexpr (F8) {
      // the tile's 32 scales, lanes 32 .. 63 a second copy
      __builtin_amdgcn_global_load_lds(
          kscale + base + (lane & 31),
          (__attribute__((address_space(3))) void*)(buf + DT::kScaleOff), 4, 0, kStream);
    }
  };
  // r0[j]: first slot of the tile that ring slot j holds or is loading
  // (tile j, then j + RING, ...)
  int64_t r0[RING];
  static_for<RING>([&](auto jc) { r0[decltype(jc)::value] = tile_row0(decltype(jc)::value); });
  static_for<RING>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if (j < ntiles) dma(j, r0[j]);
  });

  // The query and weight registers are re-defined by an empty asm once
  // their loads are in: the compiler's wait tracking then no longer ties
  // the MFMAs of every tile to outstanding vector-memory operations (it
  // would otherwise wait for all tile DMAs in flight before each tile).
#pragma unroll
  for (int tt = 0; tt < TQ; ++tt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (QF8) {
#pragma unroll
        for (int st = 0; st < 2; ++st) asm volatile("" : "+v"(qa8[tt][mt][st]));
      } else {
#pragma unroll
        for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(qa[tt][mt][st]));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(wr[tt][mt][r]));
    }
  asm volatile("" : "+v"(bid_lane));

  // key operand of this lane: row col; bf16: piece 2 s + hf at slot
  // (2 s + hf) ^ (col % 16); e4m3: pieces 4 hf + j (dims 64 hf + 16 j ..)
  // at slot (4 hf + j) ^ (col % 8)
  const uint32_t rbase = static_cast<uint32_t>(col) * DT::kRowBytes;
  const int csw = col % DT::kPieces;
  // range of token hf's causal scores among this wave's keys
  float rmin = INFINITY, rmax = -INFINITY;
  const int32_t my_pos = hf < nt ? pos0 + hf : -1;
  for (int i0 = 0; i0 < ntiles; i0 += RING) {
    static_for<RING>([&](auto jc) {
      constexpr int j = decltype(jc)::value;   // ring slot of tile i
      const int i = i0 + j;
      if (i >= ntiles) return;
      const int64_t my_r0 = r0[j];
      r0[j] = tile_row0(i + RING);
      // tile i landed when at most the later tiles' DMAs are pending (tiles
      // up to i + RING - 1 are issued at this point)
      const int later = min(ntiles - 1 - i, RING - 1);
      wait_tile<DT::kInstr>(later);
      const uint32_t tb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (__attribute__((address_space(3))) uint8_t*)(&ring[wave][j][0]))) + rbase;
      // Slot j is refilled with tile i + RING as soon as every LDS read of
      // tile i has returned (the tile then lives in registers): RING tiles
      // are in flight while the wave multiplies.  The memory clobber keeps
      // the DMA behind the reads' waits.
      auto refill = [&]() {
        asm volatile("" ::: "memory");
        if (i + RING < ntiles) dma(j, r0[j]);
      };
      bf16x8 kv[QF8 ? 1 : 8];
      i32x8 kv8[QF8 ? 2 : 1];
      float kscl = 1.0f;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (!F8) {
        static_for<8>([&](auto sc) {
          constexpr int st = decltype(sc)::value;
          kv[st] = lds_b128<0>(tb + 16u * static_cast<uint32_t>((2 * st + hf) ^ csw));
        });
        static_for<8>([&](auto sc) {
          constexpr int st = decltype(sc)::value;
          lgkm_keep<7 - st>(kv[st]);
        });
        refill();
      } else {
        // the key's scale first, then its four 16-byte pieces
        kscl = lds_f32<0>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                   (__attribute__((address_space(3))) uint8_t*)(&ring[wave][j][0]))) +
               DT::kScaleOff + 4u * static_cast<uint32_t>(col));
        u32x4 raw[4];
        // bf16 queries: pieces 4 hf + jj (dims 64 hf + 16 jj ..), widened;
        // e4m3 queries: pieces 4 (jj / 2) + 2 hf + jj % 2 (dims 64 s + 32 hf
        // .. for K-step s = jj / 2), kept as codes
        static_for<4>([&](auto jc2) {
          constexpr int jj = decltype(jc2)::value;
          const int piece = QF8 ? 4 * (jj >> 1) + 2 * hf + (jj & 1) : 4 * hf + jj;
          raw[jj] = __builtin_bit_cast(
              u32x4, lds_b128<0>(tb + 16u * static_cast<uint32_t>(piece ^ csw)));
        });
        static_for<4>([&](auto jc2) {
          constexpr int jj = decltype(jc2)::value;
          lgkm_keep<3 - jj>(raw[jj]);
          if constexpr (jj == 0) asm volatile("" : "+v"(kscl));
          if constexpr (!QF8) {
            kv[2 * jj] = fp8x8_to_bf16x8(raw[jj][0], raw[jj][1]);
            kv[2 * jj + 1] = fp8x8_to_bf16x8(raw[jj][2], raw[jj][3]);
          }
        });
        if constexpr (QF8) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const u32x4 lo = raw[2 * st], hi = raw[2 * st + 1];
            kv8[st] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          }
        }
        refill();
      }
      float part[TQ];
#pragma unroll
      for (int tt = 0; tt < TQ; ++tt) part[tt] = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x16 acc[TQ];
#pragma unroll
        for (int tt = 0; tt < TQ; ++tt) acc[tt] = f32x16{};
        if constexpr (QF8) {
          // e4m3 x e4m3, 64 dims per instruction (format code 0 = e4m3 for
          // both operands; block scales 127 = 2^0)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int tt = 0; tt < TQ; ++tt)
              acc[tt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  qa8[tt][mt][st], kv8[st], acc[tt], 0, 0, 0, 127, 0, 127);
        } else
        static_for<8>([&](auto sc) {
          constexpr int st = decltype(sc)::value;
#pragma unroll
          for (int tt = 0; tt < TQ; ++tt)
            acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[tt][mt][st], kv[st],
                                                              acc[tt], 0, 0, 0);
        });
#pragma unroll
        for (int tt = 0; tt < TQ; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            part[tt] = fmaf(wr[tt][mt][r], fmaxf(acc[tt][r], 0.0f), part[tt]);
      }
#pragma unroll
      for (int tt = 0; tt < TQ; ++tt) part[tt] = lane_sum_x32(part[tt]);
      // lane half hf keeps token hf's score for key
      // (first_tile + kWaves i) * kTile + col (0 when the tile has no row)
      float v = part[0];
      if constexpr (TQ > 1) v = hf ? part[1] : part[0];
      v *= kscl;
      if (my_r0 < 0) v = 0.0f;
      if (crange) {   // uniform: recorded only for batches of long rows
        const bool causal = (first_tile + kWaves * i) * kTile + col <= my_pos;
        if constexpr (SPAN) {
          // one entry per tile: range chunks of 128 keys, one part per tile
          float lo = causal ? v : INFINITY, hi = causal ? v : -INFINITY;
          half_minmax(lo, hi);
          if (col == 0 && hf < nt && tbeg + t0 + hf >= win_lo && tbeg + t0 + hf < win_hi)
            crange[(tbeg + t0 + hf - win_lo) * static_cast<int64_t>(range_stride) + first_tile +
                   kWaves * i] = make_float2(lo, hi);
        } else {
          rmin = fminf(rmin, causal ? v : INFINITY);
          rmax = fmaxf(rmax, causal ? v : -INFINITY);
        }
      }
      if (hf < TQ) sc[hf < TQ ? hf : 0][(kWaves * i + wave) * kTile + col] = v;
    });
  }

  // ---- the wave's range entries: one per token of the block
  if constexpr (!SPAN) {
    if (crange) half_minmax(rmin, rmax);
    if (crange && col == 0 && hf < nt && tbeg + t0 + hf >= win_lo && tbeg + t0 + hf < win_hi)
      crange[(tbeg + t0 + hf - win_lo) * static_cast<int64_t>(range_stride) +
             chunk * kRangeParts + wave] = make_float2(rmin, rmax);
  }

  // ---- write the chunk's scores: token tt, keys key_beg .. key_end - 1
  // (up to the next multiple of 4, inside the padded row), 16 bytes per
  // thread and instruction
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const int n4 = (key_end - key_beg + 3) / 4;
#pragma unroll
  for (int tt = 0; tt < TQ; ++tt) {
    if (tt >= nt) break;
    const int64_t tok = tbeg + t0 + tt;
    if (tok < win_lo || tok >= win_hi) continue;
    float* row = scores + (tok - win_lo) * row_stride + key_beg;
    for (int c = threadIdx.x; c < n4; c += 256)
      reinterpret_cast<float4*>(row)[c] = reinterpret_cast<const float4*>(&sc[tt][0])[c];
  }
  };   // run

  if constexpr (SPAN) {
    // tiles of request bb: its keys rounded up to whole 128-key chunks, or
    // none without a query token
    auto tiles_of = [&](int bb) -> uint32_t {
      if (bb >= B) return 0u;
      const int32_t L = min(seq_lens[bb], max_seq_len);
      const int32_t c = cu_q[bb];
      const int32_t ql = cu_q[bb + 1] - c;
      return (ql > 0 && L > 0 && c >= win_lo && c < win_hi)
                 ? static_cast<uint32_t>((L + 127) / 128 * 4) : 0u;
    };
    uint32_t total = 0;
    for (int b0 = 0; b0 < B; b0 += 64)
      total += __builtin_amdgcn_readlane(wave_scan_incl(tiles_of(b0 + lane)), 63);
    const uint32_t beg = static_cast<uint32_t>(
        static_cast<uint64_t>(blockIdx.x) * total / gridDim.x);
    const uint32_t end = static_cast<uint32_t>(
        static_cast<uint64_t>(blockIdx.x + 1) * total / gridDim.x);
    uint32_t base = 0;           // tiles of the requests before b0
    for (int b0 = 0; b0 < B && base < end; b0 += 64) {
      const uint32_t n = tiles_of(b0 + lane);
      const uint32_t incl = wave_scan_incl(n);
      const uint32_t st = base + incl - n;
      uint64_t m = __ballot(n > 0 && st < end && st + n > beg);
      while (m) {
        const int i = __builtin_ctzll(m);
        m &= m - 1;
        const uint32_t s_b = __builtin_amdgcn_readlane(st, i);
        const uint32_t n_b = __builtin_amdgcn_readlane(n, i);
        const uint32_t lt1 = min(end, s_b + n_b) - s_b;
        for (uint32_t lt = max(beg, s_b) - s_b; lt < lt1; lt += kWaves * MAXT) {
          const int cnt = static_cast<int>(min(lt1 - lt, static_cast<uint32_t>(kWaves * MAXT)));
          run(b0 + i, 0, static_cast<int32_t>(lt) * kTile, (cnt + kWaves - 1) / kWaves,
              static_cast<int32_t>(lt + cnt) * kTile, 0);
          if (crange) {
            // the piece's tiles past the row (up to its last 128-key chunk):
            // empty ranges, so the top-k reads no stale entry
            const int bb = b0 + i;
            const uint32_t first_pad =
                static_cast<uint32_t>((min(seq_lens[bb], max_seq_len) + kTile - 1) / kTile);
            const int64_t rrow = static_cast<int64_t>(cu_q[bb] - win_lo) * range_stride;
            for (uint32_t tt = max(lt, first_pad) + threadIdx.x; tt < lt + cnt; tt += 256)
              crange[rrow + tt] = make_float2(INFINITY, -INFINITY);
          }
          lds_barrier();           // the scores' LDS is free for the next piece
        }
      }
      base += __builtin_amdgcn_readlane(incl, 63);
    }
  } else {
    const int chunk = blockIdx.x % nchunks;
    const int qbg = blockIdx.x / nchunks;
    const int32_t chunk_keys = kTile * kWaves * tiles_per_wave_arg;
    run(qbg / qblocks_per_req, qbg % qblocks_per_req, chunk * chunk_keys, tiles_per_wave_arg,
        (chunk + 1) * chunk_keys, chunk);
  }
}

template <int TQ, int MT, bool F8, int MAXT, bool QF8, bool SPAN = false>
hipError_t launch_dma_t(IndexerArgs& a, int qbpr, int nchunks, int64_t tpw,
                        hipStream_t stream) {
  const dsa_batch& b = a.b;
  int64_t grid;
  if constexpr (SPAN) {
    // per-tile range entries: chunks of 128 keys, one part per 32-key tile
    a.chunk_keys = 4 * kTile;
    a.range_stride = (b.max_seq_len + 4 * kTile - 1) / (4 * kTile) * kRangeParts;
    grid = 2 * static_cast<int64_t>(device_cus());
  } else {
    // the range layout the top-k reads: kRangeParts entries per chunk
    a.chunk_keys = static_cast<int32_t>(kTile * kWaves * tpw);
    a.range_stride = nchunks * kRangeParts;
    grid = static_cast<int64_t>(b.num_reqs) * qbpr * nchunks;
  }
  if (grid == 0) return hipSuccess;
  k_score_dma<TQ, MT, F8, MAXT, QF8, SPAN><<<static_cast<unsigned>(grid), 256, 0, stream>>>(
      static_cast<const uint16_t*>(a.q), a.q_scale, a.w,
      static_cast<const uint8_t*>(a.k_cache), a.k_scale, b.seq_lens, b.cu_q,
      b.block_table, b.max_blocks, b.block_size, b.num_slots, b.max_seq_len,
      qbpr, nchunks, static_cast<int32_t>(tpw), a.scores, a.row_stride, a.chunk_range,
      a.range_stride, b.num_reqs, a.win_lo, a.win_hi);
  return hipGetLastError();
}

template <int TQ, int MT, bool F8, bool QF8 = false>
hipError_t launch_dma(IndexerArgs& a, hipStream_t stream) {
  const dsa_batch& b = a.b;
  const int qbpr = (b.max_q_len + TQ - 1) / TQ;
  // one round of workgroups: about 256 of them (one per CU) share the
  // longest request
  const int64_t groups = static_cast<int64_t>(b.num_reqs) * qbpr;
  const int64_t tiles_total = (b.max_seq_len + kTile - 1) / kTile;
  int64_t want = groups >= 256 ? 1 : (256 + groups - 1) / groups;     // chunks per request
  int64_t tpw = (tiles_total + want * kWaves - 1) / (want * kWaves);  // tiles per wave
  if (tpw < 1) tpw = 1;
  if (tpw > kMaxTpw) tpw = kMaxTpw;        // one block id per lane
  int nchunks = static_cast<int>((tiles_total + tpw * kWaves - 1) / (tpw * kWaves));
  // several rounds of single-token requests (long varlen rows, e4m3 keys):
  // an even split of the batch's tiles over two workgroups per CU
  if constexpr (TQ == 1 && MT == 1 && F8) {
    if (groups * nchunks > 256 && tpw > 16)
      return launch_dma_t<TQ, MT, F8, 32, QF8, true>(a, qbpr, nchunks, tpw, stream);
  }
  return launch_dma_t<TQ, MT, F8, kMaxTpw, QF8>(a, qbpr, nchunks, tpw, stream);
}

// ---------------------------------------------------------------- vector path
__device__ __forceinline__ float ld(const void* p, int64_t i, int dt) {
  if (dt == DSA_F32) return static_cast<const float*>(p)[i];
  if (dt == DSA_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  return fp8_to_f32(static_cast<const uint8_t*>(p)[i]);
}

// one thread per (token, key); the token's query and weights sit in LDS
__global__ __launch_bounds__(256) void k_score_vector(
    const void* __restrict__ q, int q_dtype, const float* __restrict__ qscale,
    const float* __restrict__ w,
    const void* __restrict__ kc, const float* __restrict__ kscale,
    int cache_dtype, int H, int D, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, int32_t B,
    const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t block_size, int64_t num_slots, int32_t max_seq_len,
    int32_t key_blocks, float* __restrict__ scores, int64_t row_stride, int32_t win_lo) {
  __shared__ float sq[8192];
  __shared__ float sw[64];
  const int t = win_lo + static_cast<int>(blockIdx.x / key_blocks);
  const int kb = blockIdx.x % key_blocks;
  const int b = request_of(cu_q, B, t);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  if (kb * 256 > pos) return;
  for (int i = threadIdx.x; i < H * D; i += 256)
    sq[i] = ld(q, static_cast<int64_t>(t) * H * D + i, q_dtype);
  for (int i = threadIdx.x; i < H; i += 256)   // e4m3 queries: times their scale
    sw[i] = w[static_cast<int64_t>(t) * H + i] *
            (qscale ? qscale[static_cast<int64_t>(t) * H + i] : 1.0f);
  __syncthreads();
  const int32_t s = kb * 256 + threadIdx.x;
  if (s > pos) return;
  const int64_t slot = slot_of(block_table + static_cast<int64_t>(b) * max_blocks,
                               s, block_size, max_blocks, num_slots);
  float score = 0.0f;
  if (slot >= 0) {
    for (int h = 0; h < H; ++h) {
      float dot = 0.0f;
      for (int d = 0; d < D; ++d)
        dot = fmaf(sq[h * D + d], ld(kc, slot * D + d, cache_dtype), dot);
      score = fmaf(sw[h], fmaxf(dot, 0.0f), score);
    }
    if (cache_dtype == DSA_FP8_E4M3) score *= kscale[slot];
  }
  scores[static_cast<int64_t>(t - win_lo) * row_stride + s] = score;
}

}  // namespace

bool indexer_mfma_ok(const IndexerArgs& a) {
  const bool qf8 = a.q_dtype == DSA_FP8_E4M3 && a.cache_dtype == DSA_FP8_E4M3;
  return (a.q_dtype == DSA_BF16 || qf8) &&
         (a.cache_dtype == DSA_BF16 || a.cache_dtype == DSA_FP8_E4M3) &&
         a.d_idx == 128 && (a.n_heads == 32 || a.n_heads == 64) &&
         a.b.block_size % kTile == 0;
}

hipError_t launch_indexer_score(IndexerArgs& a, hipStream_t stream) {
  const dsa_batch& b = a.b;
  if (b.num_q_tokens == 0) return hipSuccess;
  if (b.max_seq_len <= kTopkRegCap) a.chunk_range = nullptr;   // see kTopkRegCap
  if (prefill_score_ok(a)) return launch_score_prefill(a, stream);
  if (indexer_mfma_ok(a)) {
    const bool fp8 = a.cache_dtype == DSA_FP8_E4M3;
    const bool one = b.max_q_len == 1;
    const bool mt2 = a.n_heads == 64;
    if (!fp8) {
      if (one) return mt2 ? launch_dma<1, 2, false>(a, stream) : launch_dma<1, 1, false>(a, stream);
      return mt2 ? launch_dma<2, 2, false>(a, stream) : launch_dma<2, 1, false>(a, stream);
    }
    if (a.q_dtype == DSA_FP8_E4M3) {
      if (one) return mt2 ? launch_dma<1, 2, true, true>(a, stream)
                          : launch_dma<1, 1, true, true>(a, stream);
      return mt2 ? launch_dma<2, 2, true, true>(a, stream) : launch_dma<2, 1, true, true>(a, stream);
    }
    if (one) return mt2 ? launch_dma<1, 2, true>(a, stream) : launch_dma<1, 1, true>(a, stream);
    return mt2 ? launch_dma<2, 2, true>(a, stream) : launch_dma<2, 1, true>(a, stream);
  }
  a.chunk_range = nullptr;   // the top-k finds the range itself (vector path)
  const int key_blocks = (b.max_seq_len + 255) / 256;
  const int64_t grid = static_cast<int64_t>(a.win_hi - a.win_lo) * key_blocks;
  if (grid <= 0) return hipSuccess;
  k_score_vector<<<static_cast<unsigned>(grid), 256, 0, stream>>>(
      a.q, a.q_dtype, a.q_scale, a.w, a.k_cache, a.k_scale, a.cache_dtype, a.n_heads,
      a.d_idx, b.seq_lens, b.cu_q, b.num_reqs, b.block_table, b.max_blocks,
      b.block_size, b.num_slots, b.max_seq_len, key_blocks, a.scores,
      a.row_stride, a.win_lo);
  return hipGetLastError();
}

}  // namespace dsa

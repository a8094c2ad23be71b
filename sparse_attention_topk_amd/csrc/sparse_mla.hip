// Absorbed sparse MLA over the selected latent rows.
//
// Page "GLM5 TensorCast 适配设计", section "DSA Indexer fused semantic op":
// topk_limit and topk_indices reach the MLA backend, which attends only to
// the selected positions; section "Performance model design": the sparse
// attention length is the top-k width.  Page "GLM5 full-stack LoRA",
// section 2.2: absorbed MLA - queries live in the latent space, so attention
// runs directly over the cached latent rows.  For a query token t, head h
// and its valid indices J:
//     z[h, j] = scale * q[t, h, :] . kv[j, :]          (R + P dims)
//     out[t, h, :] = sum_j softmax_j(z[h, :]) * kv[j, 0:R]
//     lse[t, h] = log sum_j exp z[h, j]
//
// Matrix-core paths (bf16, R = 512, P = 64, 64 heads): one workgroup per
// (query token, key split) covers all 64 heads, so every selected latent row
// crosses HBM once per token.  Rows are gathered into LDS straight from
// memory (global_load_lds_dwordx4, whole 128-byte lines per instruction).
//   k_mla_ws: splits of up to 1,024 indices (decode: a few tokens, many
//     splits).  32-row tiles in a ring of four; eight waves, warp
//     specialised: four logit waves on tile k, four P.V waves on tile k - 1.
//   k_mla_prefill: up to 2,048 indices per workgroup (many tokens, one split,
//     or long splits).  64-row tiles, two in LDS; four waves, each doing its
//     share of the logits, softmax and P.V on v_mfma_f32_32x32x16_bf16.
// Both keep a per-head reference maximum that a later key may exceed by a
// fixed slack before it moves; a move rescales the running sums and
// accumulators in place, so each tile is processed once.  With more than
// one key split, each split writes its normalised partial output and
// log-sum-exp, and the token's splits merge them by LSE weights, a part of
// the heads each, once every split has arrived (see mla_store_or_merge;
// splits of a token are placed on one XCD).
//
// Vector path (fp32 or other shapes): one workgroup per (token, head),
// fp32 arithmetic, logits in LDS.
#include <cstdlib>
#include <type_traits>
#include <utility>

#include "common.h"

namespace dsa {
namespace {

constexpr int kR = 512, kP = 64, kD = kR + kP;
constexpr int kH = 64;                  // heads per workgroup (all of them)
constexpr int kT = 32;                  // keys per tile
constexpr int kHT = 1;                  // 16-head tiles per wave
constexpr int kHG = kH / (16 * kHT);    // head groups (4)
constexpr int kWavesM = 2 * kHG;        // waves: head group x key half (8, two per SIMD)
constexpr int kThreads = 64 * kWavesM;  // 512
constexpr int kPvNT = kR / 4 / 16;      // 16-dim tiles per wave in P.V (128 dims)
constexpr int kDmaWaves = 4;            // waves that issue the tile DMAs
constexpr int kPieces = kD / 8;         // 16-byte pieces per latent row (72)
constexpr int kTilePieces = kT * kPieces;             // 2304
constexpr int kDmaInstr = kTilePieces / 64;           // 36 wave loads per tile
constexpr int kDmaPerWave = kDmaInstr / kDmaWaves;    // 9
constexpr int kBufs = 4;                // tiles resident: current + 3 in flight
constexpr int kMaxSplitLen = 2048;      // indices per workgroup
constexpr int kMaxSplits = 32;          // merge weights fit behind the staged block
constexpr int kQSteps = kD / 32;        // 18 K-steps of the logits
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Probabilities are 2^(z - m) against a per-head reference m fixed by the
// head's first key; a later key may exceed m by up to this much (in log2
// units), so p <= 2^64 and the fp32 sums stay far from overflow.
constexpr float kMoveSlack = 64.0f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// fp32 -> bf16, round to nearest even, with gfx950's conversion
// instruction (v_cvt_pk_bf16_f32: two values per instruction)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// a -> bits 0..15, b -> bits 16..31
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// slot of index j of token t, or -1 when j is outside [jbeg, jend), the
// entry is negative, beyond the token's position, or off the cache
__device__ __forceinline__ int64_t sel_slot(const int32_t* __restrict__ idx_row,
                                            int j, int jend, int32_t pos,
                                            const int32_t* bt_row,
                                            int32_t block_size,
                                            int32_t max_blocks,
                                            int64_t num_slots) {
  if (j >= jend) return -1;
  const int32_t p = idx_row[j];
  if (p < 0 || p > pos) return -1;
  return slot_of(bt_row, p, block_size, max_blocks, num_slots);
}

// LDS operand loads issued as inline asm: as builtins the compiler puts an
// s_waitcnt vmcnt(0) in front of a transpose load (it assumes the load may
// read LDS still being written by a tile DMA), which would wait for the
// tiles in flight.  The caller waits for the results with lgkm_keep<N>(),
// which takes the consumed register as an operand so the compiler cannot
// read it earlier.  Every sequence starts with lgkm_drain(), so the
// compiler's own LDS operations are retired before the counting starts.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(p)));
}
// 4 consecutive bf16 of LDS read with the gfx950 transpose load: within each
// 16-lane group, lane j supplies 4 elements that become A[4j .. 4j+3] and
// lane i receives A[i], A[16+i], A[32+i], A[48+i].
template <int OFF>
__device__ __forceinline__ v4i16 tr_load(uint32_t addr) {
  v4i16 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ uint32_t b32_load(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 u128_load(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ bf16x8 b128_load(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// f(integral_constant<int, I>) for I = 0 .. N-1, so that loop indices can
// feed immediates
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// Waits until at most N LDS operations are outstanding; `r` is the register
// the next instruction consumes, tied so the compiler cannot read it earlier.
template <int N, typename T>
__device__ __forceinline__ void lgkm_keep(T& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "n"(N));
}
__device__ __forceinline__ void lgkm_drain() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
// s_waitcnt with only the vector-memory count (gfx9 encoding: low four bits
// in [3:0], high two in [15:14]; lgkmcnt / expcnt fields at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// cross-lane reductions over lanes l ^ 16 and l ^ 32 (gfx950 permlane swaps:
// each returns the values of the two lanes of the pair)
// max of logits (never NaN; -inf for keys without a row).  These take the
// compiler's own max instruction, never inline asm: the first inputs come
// straight from MFMA accumulators, and the compiler inserts the wait states
// that a VALU read of an MFMA result needs only for instructions it can see
// (an asm max read the accumulators before the last MFMA had written them).
__device__ __forceinline__ float max_nn(float a, float b) { return __builtin_fmaxf(a, b); }
__device__ __forceinline__ float max3_nn(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}
__device__ __forceinline__ float max_x16_x32(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nn(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float sum_x16_x32(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// A token's splits meet at one 64-bit word in the workspace, alone on its
// 128-byte line (kWordStride words apart), so that polls and counts of
// different tokens never queue on one line: the tag of the call (upper 48
// bits), the merge parts given up by their owners (bits 8..11) and the
// splits arrived (bits 0..7).  A word with another tag, whatever the
// workspace held before, counts as no arrival, and so does a finished word
// of this call (every split arrived): that is what a replay of the same
// launch (same tag) finds.  A compare-and-swap fails only when another
// split changed the word after it was read; before the last arrival each
// split changes it at most twice (its arrival, and giving up its part), so
// the loop ends within 2 n_split + 1 rounds.  The first compare-and-swap
// guesses the word the last arrival finds (`guess`), so the split that
// arrives last, which merges and is on the kernel's critical path, usually
// needs a single round trip.  A split that is not the last adds
// `give_up` (its parts, merged by the last split instead); returns the
// low 16 bits of the word it left, 0 if the loop ran out.
constexpr int kWordStride = 16;
constexpr int kParts = 4;                 // merge parts of 16 heads (three or more splits)
static_assert(kMaxSplits < 256, "arrival count fits in 8 bits");
__device__ uint32_t arrive(unsigned long long* word, unsigned long long tag, int n_split,
                           uint32_t guess, uint32_t give_up) {
  unsigned long long cur = (tag << 16) | (static_cast<unsigned long long>(guess) << 8) |
                           static_cast<unsigned long long>(n_split - 1);
  for (int round = 0; round <= 2 * n_split + 1; ++round) {
    const bool counting = (cur >> 16) == tag && (cur & 0xFFu) < static_cast<uint32_t>(n_split);
    unsigned long long next = (counting ? cur : tag << 16) + 1;
    if ((next & 0xFFu) != static_cast<uint32_t>(n_split))
      next |= static_cast<unsigned long long>(give_up) << 8;
    const unsigned long long prev = atomicCAS(word, cur, next);
    if (prev == cur) return static_cast<uint32_t>(next & 0xFFFFull);
    cur = prev;
  }
  return 0;
}

// LDS layout of a 32-row tile (36 KB): rows in four groups h of 8, the 72
// 16-byte pieces of a row in nine groups g of 8.  Block (h, g) is 1 KB at
// 9216 h + 1024 g and is filled by one DMA instruction: lane l lands at
// 16 l and carries row 8 h + rho, piece 8 g + pi with
//     l = 8 (pi ^ (h & 1)) + (rho ^ 4 (pi & 1)),
// so every DMA instruction fetches whole 128-byte lines (8 rows x 128 B) and
// a lane's nine instructions of a tile differ only in an immediate offset.
// The lane map makes both LDS read patterns conflict-free for 32 and for 64
// banks: the logit loads (16 consecutive rows, one piece, 16 bytes per lane)
// and the value transpose loads (16 consecutive rows, two adjacent pieces,
// 8 bytes per lane).
__device__ __forceinline__ uint32_t tile_byte(int row, int piece) {
  const int h = row >> 3, rho = row & 7, pi = piece & 7;
  const int l = 8 * (pi ^ (h & 1)) + (rho ^ (4 * (pi & 1)));
  return 9216u * h + 1024u * (piece >> 3) + 16u * l;
}

// Barrier for the tile loop: LDS operations of this wave complete, then all
// waves meet.  Unlike an LDS release fence it does not wait for the tile DMA
// in flight (a DMA write to LDS counts as an LDS write for the fence); the
// loop waits for each tile's own DMA explicitly with s_waitcnt vmcnt before
// its first use.  The memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}



// The merge's pieces.  A word holds 4 bf16 dims of a head row.
__device__ __forceinline__ void unpack_bf16x4(unsigned long long v, float (&x)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    x[e] = __uint_as_float(static_cast<uint32_t>((v >> (16 * e)) & 0xFFFFu) << 16);
}
__device__ __forceinline__ unsigned long long pack_bf16x4(const float (&x)[4], float inv) {
  return static_cast<unsigned long long>(pack2_bf16(x[0] * inv, x[1] * inv)) |
         (static_cast<unsigned long long>(pack2_bf16(x[2] * inv, x[3] * inv)) << 32);
}
// Head h's split weights exp(lse_s - max) in place of its log-sum-exps
// wt[s * kH + h], 1 / their sum into wt[n_split * kH + h], and the merged
// log-sum-exp into lse (when given).
__device__ __forceinline__ void merge_weights(float* wt, int h, int n_split, int t,
                                              float* __restrict__ lse) {
  float mx = -INFINITY;
  for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, wt[s * kH + h]);
  float sum = 0.0f;
  for (int s = 0; s < n_split; ++s) {
    const float wgt = mx == -INFINITY ? 0.0f : expf(wt[s * kH + h] - mx);
    wt[s * kH + h] = wgt;
    sum += wgt;
  }
  wt[n_split * kH + h] = sum > 0.0f ? 1.0f / sum : 0.0f;
  if (lse) lse[static_cast<int64_t>(t) * kH + h] = sum > 0.0f ? mx + logf(sum) : -INFINITY;
}

// Merges heads PH p .. PH p + PH - 1 of token t over all its splits: the
// weights of those heads, then every split's bf16 partial row summed in
// split order (0, 1, ...) whichever split merges, with this split's own
// rows taken from the staged block, rounded exactly as the others read
// theirs; so the result does not depend on which split merges.  Thread tid
// takes dims 4 wq .. 4 wq + 3 (wq = tid % 128) of heads PH p + tid / 128 +
// (NT / 128) i, as the partials were written.  The words of kSr splits
// are requested before any is used, the first kSr splits' while the
// weights are made.
constexpr int kRowB = kR * 2 + 16;
constexpr int kWords = kR / 4;            // 8-byte words (4 dims) of a head row
template <int NT, int PH>
__device__ void merge_part(const uint8_t* stage, int p, int t, int split, int n_split,
                           uint16_t* __restrict__ out, float* __restrict__ lse,
                           const uint16_t* __restrict__ part_o,
                           const float* __restrict__ part_lse) {
  constexpr int kRowsPer = NT / kWords;
  constexpr int kPass = PH / kRowsPer;
  const int tid = threadIdx.x;
  const int wq = tid % kWords;
  const int hr = PH * p + tid / kWords;
  float* wt = reinterpret_cast<float*>(const_cast<uint8_t*>(stage) + kH * kRowB);
  const unsigned long long* po = reinterpret_cast<const unsigned long long*>(
      part_o + static_cast<int64_t>(t) * n_split * kH * kR) + wq;
  constexpr int kSr = PH > 16 ? 2 : 4;      // splits per round of loads
  unsigned long long wv[kSr][kPass];
  auto load4 = [&](int s0) {
#pragma unroll
    for (int g = 0; g < kSr; ++g) {
      const int sg = s0 + g;
      if (sg < n_split && sg != split) {
#pragma unroll
        for (int i = 0; i < kPass; ++i)
          wv[g][i] = __hip_atomic_load(
              const_cast<unsigned long long*>(po + (sg * kH + hr + kRowsPer * i) * kWords),
              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
#pragma unroll
        for (int i = 0; i < kPass; ++i) wv[g][i] = 0;
      }
    }
  };
  load4(0);
  for (int c = tid; c < n_split * PH; c += NT) {
    const int s = c / PH, h = PH * p + c % PH;
    wt[s * kH + h] = __hip_atomic_load(
        const_cast<float*>(part_lse) + (static_cast<int64_t>(t) * n_split + s) * kH + h,
        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid < PH) merge_weights(wt, PH * p + tid, n_split, t, lse);
  __syncthreads();
  float acc[kPass][4];
#pragma unroll
  for (int i = 0; i < kPass; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.0f;
  for (int s0 = 0;;) {
#pragma unroll
    for (int g = 0; g < kSr; ++g) {
      const int sg = s0 + g;
      if (sg < n_split) {
#pragma unroll
        for (int i = 0; i < kPass; ++i) {
          const int h = hr + kRowsPer * i;
          float x[4];
          unpack_bf16x4(sg == split ? *reinterpret_cast<const unsigned long long*>(
                                          stage + h * kRowB + 8 * wq)
                                    : wv[g][i],
                        x);
          const float wgt = wt[sg * kH + h];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wgt, x[e], acc[i][e]);
        }
      }
    }
    s0 += kSr;
    if (s0 >= n_split) break;
    load4(s0);
  }
  unsigned long long* ob = reinterpret_cast<unsigned long long*>(
      out + static_cast<int64_t>(t) * kH * kR) + wq;
#pragma unroll
  for (int i = 0; i < kPass; ++i) {
    const int h = hr + kRowsPer * i;
    ob[h * kWords] = pack_bf16x4(acc[i], wt[n_split * kH + h]);
  }
}

// A bound on the polls of an owner waiting for its token's other splits
// (the wait is bounded in time too: wait_ticks).
constexpr int kSpinPolls = 4096;

// The workgroup's staged result leaves it.  stage holds the normalised
// bf16 rows of its 64 heads (head h at byte h * kRowB, kRowB = 2 R + 16),
// and every lse is stored already (into lse, or as a partial).  With one
// split the rows are copied to out; with several, this split's rows are
// stored as its partial and the token's splits merge them (see below).
// Every thread of the workgroup calls it; stage must have room behind the
// rows for the merge weights.
template <int NT>
__device__ __forceinline__ void mla_store_or_merge(
    uint8_t* stage, uint32_t* counter, int t, int split, int n_split, bool partial,
    int32_t wait_ticks,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_lse, unsigned long long* __restrict__ arrivals,
    unsigned long long call_tag) {
  const int tid = threadIdx.x;
  constexpr int row_b = kRowB;
  tile_barrier();
  // Copy the staged block out.  The output: 16-byte pieces of a contiguous
  // region.
  if (!partial) {
    constexpr int row_pieces = kR * 2 / 16;
    constexpr int total = kH * row_pieces;
    u32x4* dst = reinterpret_cast<u32x4*>(out + static_cast<int64_t>(t) * kH * kR);
    for (int c = tid; c < total; c += NT) {
      const int h = c / row_pieces, pc = c % row_pieces;
      dst[c] = *reinterpret_cast<const u32x4*>(stage + h * row_b + 16 * pc);
    }
    return;
  }
  // Partials (bf16, normalised) are read back by other workgroups of this
  // launch, maybe on another XCD: they are stored as relaxed device-scope
  // atomics, which the hardware keeps coherent across XCDs by themselves,
  // so no cache-wide write-back or invalidation is needed to hand them
  // over.  8-byte words (4 dims), consecutive lanes on consecutive words,
  // so every store instruction writes four whole 128-byte lines: thread tid
  // takes word tid % 128 of head rows tid / 128 + (NT / 128) i.
  //
  // The heads are merged in parts: with two splits two halves of 32 heads,
  // split s owning half s; with more, kParts parts of 16, split p (p <
  // kParts) owning part p, and parts without an owner (fewer splits than
  // parts) falling to the last split.  With wait_ticks > 0 (the host sets
  // it when every workgroup of the launch is resident at once) an owner
  // waits, for at most wait_ticks s_memrealtime ticks (10 ns), until every
  // split has arrived and merges its own parts, so a split stores only the
  // rows of parts it does not own.  Otherwise, or once an owner stops
  // waiting, the owner stores its own rows too
  // and gives its parts up in the token's word, and the last split merges
  // every part given up.  Every thread waits until its partial stores have
  // completed (reached the device-coherent level) before the workgroup
  // counts its arrival or gives a part up, and partials are loaded
  // (device-scope atomic loads) only by a split that has seen every
  // arrival, so each part is merged exactly once, from complete rows.
  const int n_parts = n_split == 2 ? 2 : kParts;
  const int ph = kH / n_parts;                     // heads per part
  const uint32_t all_parts = (1u << n_parts) - 1u;
  const uint32_t mine = split < n_parts ? 1u << split : 0u;
  const uint32_t unowned = n_split < n_parts ? all_parts & ~((1u << n_split) - 1u) : 0u;
  constexpr int kRowsPer = NT / kWords;            // head rows per pass
  constexpr uint32_t kGiveUp = 0x100u;
  const bool coop = wait_ticks > 0;
  const int wq = tid % kWords;
  const int h0 = tid / kWords;
  unsigned long long* dst = reinterpret_cast<unsigned long long*>(
      part_o + (static_cast<int64_t>(t) * n_split + split) * kH * kR);
  auto store_rows = [&](uint32_t parts_mask) {
#pragma unroll 8
    for (int i = 0; i < kH / kRowsPer; ++i) {
      const int h = h0 + kRowsPer * i;
      if ((parts_mask >> (h / ph)) & 1u) {         // uniform: h / ph = i / (ph / kRowsPer)
        const unsigned long long v =
            *reinterpret_cast<const unsigned long long*>(stage + h * row_b + 8 * wq);
        __hip_atomic_store(dst + h * kWords + wq, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  store_rows(coop ? all_parts & ~mine : all_parts);
  wait_vm<0>();
  __syncthreads();
  unsigned long long* wp = arrivals + kWordStride * t;
  if (tid == 0) {
    // without coop every other owner gives its parts up on arrival
    const uint32_t guess = coop ? 0u : all_parts & ~unowned & ~mine;
    const uint32_t w = arrive(wp, call_tag, n_split, guess, coop ? 0u : mine);
    uint32_t todo = 0;
    if ((w & 0xFFu) == static_cast<uint32_t>(n_split)) {
      todo = mine | unowned | ((w >> 8) & all_parts);
    } else if (coop && mine) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      todo = kGiveUp;
      for (int poll = 0; poll < kSpinPolls; ++poll) {
        __builtin_amdgcn_s_sleep(2);
        const unsigned long long cur =
            __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((cur & 0xFFu) == static_cast<uint32_t>(n_split)) {
          todo = mine;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > static_cast<uint64_t>(wait_ticks)) break;
      }
    }
    *counter = todo;
  }
  __syncthreads();
  uint32_t todo = *counter;
  if (todo == kGiveUp) {
    // stop waiting: store this split's own rows, then give its parts up
    // unless the last split has arrived meanwhile (after the last arrival
    // the word no longer changes)
    store_rows(mine);
    wait_vm<0>();
    __syncthreads();
    if (tid == 0) {
      uint32_t res = mine;
      unsigned long long cur = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int round = 0; round <= 2 * n_split + 1; ++round) {
        if ((cur & 0xFFu) == static_cast<uint32_t>(n_split)) break;
        const unsigned long long prev =
            atomicCAS(wp, cur, cur | (static_cast<unsigned long long>(mine) << 8));
        if (prev == cur) {
          res = 0;
          break;
        }
        cur = prev;
      }
      *counter = res;
    }
    __syncthreads();
    todo = *counter;
  }
  if (todo == 0) return;
  asm volatile("" ::: "memory");
#pragma unroll 1
  for (int p = 0; p < n_parts; ++p) {
    if (!((todo >> p) & 1u)) continue;
    if (n_parts == 2)
      merge_part<NT, kH / 2>(stage, p, t, split, n_split, out, lse, part_o, part_lse);
    else
      merge_part<NT, kH / kParts>(stage, p, t, split, n_split, out, lse, part_o, part_lse);
  }
}

// ------------------------------------------------- warp-specialised pipeline
// The same contraction with the work of a tile split by role instead of by
// phase.  Waves 0..3 (one per SIMD) are logit waves: wave hg holds the
// queries of heads 16 hg .. 16 hg + 15 in registers and computes their
// logits for all 32 keys of a tile (two 16-key blocks per K-step, the query
// operand shared), the per-head tile maxima in-lane plus two permlane swaps,
// and the bf16 probabilities; it also issues its 8-row group of the tile
// DMAs.  Waves 4..7 are P.V waves: wave 4 + pq accumulates all 64 heads
// over value dims 128 pq .. 128 pq + 127, so each value element is read from
// LDS once and feeds four MFMAs (one per head group).  Iteration k: logit
// waves work on tile k while P.V waves work on tile k - 1 with the
// probabilities the logit waves published one iteration earlier (a double
// buffer in LDS); one barrier per iteration.  Ring of four tiles: k - 1
// (P.V), k (logits), k + 1 and k + 2 in flight (tile k + 2 is issued at the
// start of iteration k, into the slot tile k - 2 left).
// Reference maxima: a head's reference is fixed by its
// first key and may be exceeded by kMoveSlack before it moves; when it moves,
// the logit wave rescales its sums and publishes the factor 2^(m_old -
// m_new), and the P.V waves rescale that head group's accumulators in place
// before adding the tile (no restart: each tile is processed once).
constexpr int kWsSplitCap = 1024;       // indices per workgroup (slot table)
struct MlaSharedWs {
  uint16_t k[kBufs][kT * kD];           // row-major tiles, 4 x 36864 B
  int32_t slots[kWsSplitCap];           // physical row of each index, or -1
  uint32_t vbits[kWsSplitCap / kT];     // per tile: bit k = key k has a row
  u32x4 xp[2][kHG][64];                 // probabilities [buffer][head group][lane]
  float xf[2][kH];                      // per-head rescale factors
  alignas(16) uint32_t xflag[2][kHG];   // per head group: its factors apply
  float xl[kH];                         // per-head 1 / sum (epilogue)
  uint32_t counter;
};
static_assert(sizeof(MlaSharedWs) <= 160 * 1024, "LDS budget");
static_assert(kH * kRowB + (kMaxSplits + 1) * kH * 4 <= sizeof(MlaSharedWs::k),
              "staged partials and merge weights fit in the tile buffers");

__global__ __launch_bounds__(kThreads, 1) void k_mla_ws(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t n_tokens,
    int32_t n_split, int32_t split_len, float scale_log2,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
    int32_t B, const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t block_size, int64_t num_slots, int32_t max_seq_len,
    uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
    unsigned long long* __restrict__ arrivals, unsigned long long call_tag, int32_t wait_ticks) {
  __shared__ MlaSharedWs sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g16 = lane >> 4;
  const bool logit = wave < kHG;        // waves 0..3; waves 4..7 are P.V waves
  const int hg = wave & 3;              // logit wave: heads 16 hg ..; P.V wave: dims 128 hg ..

  int vb = blockIdx.x;
  if (n_split > 1 && (gridDim.x & 7) == 0)
    vb = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int t = vb / n_split;
  const int split = vb % n_split;
  if (t >= n_tokens) return;

  const int32_t* idx_row = topk_idx + static_cast<int64_t>(t) * topk;
  const int jbeg = split * split_len;
  const int jend = min(topk, jbeg + split_len);
  const int ntiles = jend > jbeg ? (jend - jbeg + kT - 1) / kT : 0;
  const int jpad = jbeg + ntiles * kT;

  // The split's physical rows and per-tile validity masks, in two memory
  // round trips: the indices beside the request's place (cu_q and seq_lens
  // read whole), then the block-table entries.  The logit waves' queries
  // are requested only behind those (loads return in order: ahead of them
  // the 72 KiB of queries would delay both trips).
  constexpr int kIdxPer = kWsSplitCap / kThreads;    // 2
  int32_t p[kIdxPer];
#pragma unroll
  for (int i = 0; i < kIdxPer; ++i) {
    const int j = jbeg + kThreads * i + tid;
    p[i] = j < jend ? idx_row[j] : -1;
  }
  int b;
  int32_t pos;
  token_place(cu_q, seq_lens, B, t, max_seq_len, b, pos);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  int32_t bid[kIdxPer];
#pragma unroll
  for (int i = 0; i < kIdxPer; ++i) {
    const bool ok = p[i] >= 0 && p[i] <= pos && p[i] / block_size < max_blocks;
    bid[i] = ok ? bt_row[p[i] / block_size] : -1;
    if (!ok) p[i] = -1;
  }
  asm volatile("" ::: "memory");
  // logit waves' queries: heads 16 hg + l16, dims 32 st + 8 g16 .. + 7 of
  // K-step st
  bf16x8 qb[kQSteps];
  if (logit) {
    const int64_t qbase = (static_cast<int64_t>(t) * kH + 16 * hg + l16) * kD;
#pragma unroll
    for (int st = 0; st < kQSteps; ++st)
      qb[st] = *reinterpret_cast<const bf16x8*>(q + qbase + 32 * st + 8 * g16);
  }
#pragma unroll
  for (int i = 0; i < kIdxPer; ++i) {
    const int j = jbeg + kThreads * i + tid;
    int32_t slot = -1;
    if (p[i] >= 0) {
      const int64_t s = static_cast<int64_t>(bid[i]) * block_size + p[i] % block_size;
      slot = (s >= 0 && s < num_slots) ? static_cast<int32_t>(s) : -1;
    }
    if (j < jpad) sh.slots[j - jbeg] = slot;
    const uint64_t m = __ballot(j < jpad && slot >= 0);
    const int tw = (kThreads * i + 64 * wave) / kT;
    if (lane == 0 && tw < ntiles) sh.vbits[tw] = static_cast<uint32_t>(m);
    if (lane == 0 && tw + 1 < ntiles) sh.vbits[tw + 1] = static_cast<uint32_t>(m >> 32);
  }
  tile_barrier();

  // DMA geometry (logit wave w fills row group w of a tile: nine
  // instructions, one per 128-byte piece group; keys without a row load row
  // 0 and are masked)
  const int dpi = (lane >> 3) ^ (wave & 1);
  const int drow = 8 * wave + ((lane & 7) ^ (4 * (dpi & 1)));
  const uint32_t dcol = 16u * static_cast<uint32_t>(dpi);
  auto dma_piece = [&](const uint8_t* src, uint8_t* dst, auto gc) {
    constexpr int G = decltype(gc)::value;
    __builtin_amdgcn_global_load_lds(
        src + 128 * G, (__attribute__((address_space(3))) void*)(dst + 1024 * G), 16, 0, 0);
  };
  auto tile_src = [&](int tile) {
    const int32_t sl = sh.slots[tile * kT + drow];
    return reinterpret_cast<const uint8_t*>(kv) + static_cast<uint64_t>(max(sl, 0)) * (2 * kD) + dcol;
  };

  if (logit) {
    // ================================================== logit waves
    const uint8_t* s0 = ntiles > 0 ? tile_src(0) : nullptr;
    const uint8_t* s1 = ntiles > 1 ? tile_src(1) : nullptr;
    if (s0) static_for<kDmaPerWave>([&](auto g) {
      dma_piece(s0, reinterpret_cast<uint8_t*>(sh.k[0]) + 9216 * wave, g); });
    if (s1) static_for<kDmaPerWave>([&](auto g) {
      dma_piece(s1, reinterpret_cast<uint8_t*>(sh.k[1]) + 9216 * wave, g); });
    // the queries and tile 0 are in when at most tile 1's loads are pending
    if (ntiles > 1) wait_vm<kDmaPerWave>(); else wait_vm<0>();
#pragma unroll
    for (int st = 0; st < kQSteps; ++st) asm volatile("" : "+v"(qb[st]));
    // K-operand rows of this lane: keys l16 (block 0) and 16 + l16 (block 1);
    // K-step st reads piece 4 st + g16: group st >> 1 (an immediate) and one
    // of two offsets per block
    const uint32_t ko[2][2] = {{tile_byte(l16, g16), tile_byte(l16, 4 + g16)},
                               {tile_byte(16 + l16, g16), tile_byte(16 + l16, 4 + g16)}};
    float m_ref = -INFINITY;            // head 16 hg + l16
    float l_part = 0.0f;
    for (int k = 0; k <= ntiles; ++k) {
      tile_barrier();                   // tile k landed; P(k - 1) read by the P.V waves
      if (k >= ntiles) continue;
      // refill: tile k + 2 into the slot tile k - 2 left, one DMA instruction
      // after every second K-step
      const bool refill = k + 2 < ntiles;
      const uint8_t* rsrc = refill ? tile_src(k + 2) : nullptr;
      uint8_t* rdst = reinterpret_cast<uint8_t*>(sh.k[(k + 2) % kBufs]) + 9216 * wave;
      if (refill) asm volatile("" : "+v"(rsrc));
      const uint32_t kb = lds_addr(sh.k[k % kBufs]);
      const uint32_t vb32 = sh.vbits[k];
      f32x4 part[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
      {
        constexpr int kAhead = 3;       // K-steps of operands in flight
        bf16x8 kr[kAhead][2];
        lgkm_drain();
        static_for<kAhead>([&](auto sc) {
          constexpr int S = decltype(sc)::value;
          kr[S][0] = b128_load<1024 * (S >> 1)>(kb + ko[0][S & 1]);
          kr[S][1] = b128_load<1024 * (S >> 1)>(kb + ko[1][S & 1]);
        });
        static_for<kQSteps>([&](auto sc) {
          constexpr int S = decltype(sc)::value;
          constexpr int R = S % kAhead;
          constexpr int kAfter = 2 * ((kQSteps - 1 - S) < (kAhead - 1) ? (kQSteps - 1 - S) : (kAhead - 1));
          lgkm_keep<kAfter + 1>(kr[R][0]);
          part[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[R][0], qb[S], part[0], 0, 0, 0);
          lgkm_keep<kAfter>(kr[R][1]);
          part[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[R][1], qb[S], part[1], 0, 0, 0);
          if constexpr (S + kAhead < kQSteps) {
            kr[R][0] = b128_load<1024 * ((S + kAhead) >> 1)>(kb + ko[0][(S + kAhead) & 1]);
            kr[R][1] = b128_load<1024 * ((S + kAhead) >> 1)>(kb + ko[1][(S + kAhead) & 1]);
          }
          if constexpr (S % 2 == 1 && S / 2 < kDmaPerWave) {
            if (refill) {
              asm volatile("" ::: "memory");
              dma_piece(rsrc, rdst, std::integral_constant<int, S / 2>{});
            }
          }
        });
      }
      // ---- softmax: lane (l16, g16) holds head 16 hg + l16's logits of keys
      // 4 g16 + i (block 0) and 16 + 4 g16 + i (block 1)
      float zr[8];
      if (__builtin_amdgcn_readfirstlane(vb32) == 0xFFFFFFFFu) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zr[i] = part[0][i];
          zr[4 + i] = part[1][i];
        }
      } else {
        const uint32_t v0 = vb32 >> (4 * g16), v1 = vb32 >> (16 + 4 * g16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zr[i] = ((v0 >> i) & 1u) ? part[0][i] : -INFINITY;
          zr[4 + i] = ((v1 >> i) & 1u) ? part[1][i] : -INFINITY;
        }
      }
      float mx = max_nn(max3_nn(zr[0], zr[1], zr[2]), max3_nn(zr[3], zr[4], zr[5]));
      mx = max_x16_x32(max3_nn(mx, zr[6], zr[7])) * scale_log2;
      // the reference moves on the head's first key, or when the tile beats
      // it by more than the slack; a move of a live reference rescales
      float factor = 1.0f;
      bool moved = false;
      if (m_ref == -INFINITY) {
        m_ref = mx;                      // stays -inf while no key has a row
      } else if (mx > m_ref + kMoveSlack) {
        factor = __builtin_amdgcn_exp2f(m_ref - mx);
        m_ref = mx;
        moved = true;
      }
      const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(zr[i], scale_log2, -mu));
      l_part *= factor;
#pragma unroll
      for (int i = 0; i < 8; ++i) l_part += pr[i];
      const int pb = k & 1;
      u32x4 pk;
      pk[0] = pack2_bf16(pr[0], pr[1]);
      pk[1] = pack2_bf16(pr[2], pr[3]);
      pk[2] = pack2_bf16(pr[4], pr[5]);
      pk[3] = pack2_bf16(pr[6], pr[7]);
      sh.xp[pb][hg][lane] = pk;
      const bool any = __ballot(moved) != 0;
      if (any && g16 == 0) sh.xf[pb][16 * hg + l16] = factor;
      if (lane == 0) sh.xflag[pb][hg] = any ? 1u : 0u;
      // tile k + 1 is in when at most tile k + 2's loads are pending
      if (k + 1 < ntiles) {
        if (refill) wait_vm<kDmaPerWave>(); else wait_vm<0>();
      }
    }
    tile_barrier();                      // every P.V wave is done with the tiles
    const float l = sum_x16_x32(l_part);
    if (g16 == 0) {
      sh.xl[16 * hg + l16] = l > 0.0f ? 1.0f / l : 0.0f;      // the P.V waves scale by it
      const float lh = l > 0.0f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
      const int h = 16 * hg + l16;
      if (n_split > 1)
        __hip_atomic_store(part_lse + (static_cast<int64_t>(t) * n_split + split) * kH + h,
                           lh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (lse)
        lse[static_cast<int64_t>(t) * kH + h] = lh;
    }
    tile_barrier();                      // sums published
    tile_barrier();                      // rows staged
  } else {
    // ================================================== P.V waves
    // O[n][nt]: heads 16 n + 4 g16 + i (i = 0..3), dims 128 pq + 16 nt + l16
    const int pq = hg;
    f32x4 o[kHG][kPvNT];
#pragma unroll
    for (int n = 0; n < kHG; ++n)
#pragma unroll
      for (int nt = 0; nt < kPvNT; ++nt) o[n][nt] = f32x4{0, 0, 0, 0};
    // transpose-load offsets: rows 4 g16 + l16 / 4 (keys 0..15) and 16 + that
    // (keys 16..31), dims 128 pq + 16 nt + 4 (l16 & 3)
    const int vrow_a = 4 * g16 + (l16 >> 2);
    const int vrow_b = 16 + vrow_a;
    const int vb_lo = (l16 & 3) >> 1;
    uint32_t voff_a[4], voff_b[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t half = 8u * static_cast<uint32_t>(l16 & 1);
      voff_a[m] = tile_byte(vrow_a, 16 * pq + 2 * m + vb_lo) + half;
      voff_b[m] = tile_byte(vrow_b, 16 * pq + 2 * m + vb_lo) + half;
    }
    for (int k = 0; k <= ntiles; ++k) {
      tile_barrier();                   // P(k - 1) published
      if (k == 0) continue;
      const int j = k - 1;
      const int pb = j & 1;
      // a head group whose references moved: rescale its rows first
      const u32x4 fl = *reinterpret_cast<const u32x4*>(&sh.xflag[pb][0]);
      if ((fl[0] | fl[1] | fl[2] | fl[3]) != 0u) {
#pragma unroll
        for (int n = 0; n < kHG; ++n) {
          if (!fl[n]) continue;
          float f[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) f[i] = sh.xf[pb][16 * n + 4 * g16 + i];
#pragma unroll
          for (int nt = 0; nt < kPvNT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[n][nt][i] *= f[i];
        }
      }
      const uint32_t tb = lds_addr(sh.k[j % kBufs]);
      uint32_t va[4], vb[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        va[m] = tb + voff_a[m];
        vb[m] = tb + voff_b[m];
      }
      bf16x8 pa[kHG];
      lgkm_drain();
#pragma unroll
      for (int n = 0; n < kHG; ++n)
        pa[n] = __builtin_bit_cast(bf16x8, sh.xp[pb][n][lane]);
      lgkm_drain();
      constexpr int kLoads = 2 * kPvNT;               // 16
      constexpr int kAhead = 8;
      v4i16 vr[kAhead];
      auto vload = [&](auto ld) -> v4i16 {
        constexpr int L = decltype(ld)::value;
        constexpr int NT = L >> 1;
        return (L & 1) ? tr_load<1024 * (NT >> 2)>(vb[NT & 3])
                       : tr_load<1024 * (NT >> 2)>(va[NT & 3]);
      };
      static_for<kAhead>([&](auto ld) { vr[decltype(ld)::value] = vload(ld); });
      static_for<kPvNT>([&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        v4i16& a0 = vr[(2 * NT) % kAhead];
        v4i16& a1 = vr[(2 * NT + 1) % kAhead];
        constexpr int kAfter = (kLoads - 2 - 2 * NT) < (kAhead - 2) ? (kLoads - 2 - 2 * NT) : (kAhead - 2);
        lgkm_keep<kAfter>(a0);
        lgkm_keep<kAfter>(a1);
        const v8i16 v01 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, v01);
#pragma unroll
        for (int n = 0; n < kHG; ++n)
          o[n][NT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[n], vop, o[n][NT], 0, 0, 0);
        if constexpr (2 * NT + kAhead < kLoads) {
          a0 = vload(std::integral_constant<int, 2 * NT + kAhead>{});
          a1 = vload(std::integral_constant<int, 2 * NT + kAhead + 1>{});
        }
      });
    }
    tile_barrier();                      // every wave is done with the tiles
    tile_barrier();                      // sums published
    // normalised bf16 rows into the staging block (over the ring)
    uint8_t* stage = reinterpret_cast<uint8_t*>(&sh.k[0][0]);
#pragma unroll
    for (int n = 0; n < kHG; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * n + 4 * g16 + i;
        const float inv = sh.xl[h];
#pragma unroll
        for (int nt = 0; nt < kPvNT; ++nt) {
          const int d = 128 * pq + 16 * nt + l16;
          *reinterpret_cast<uint16_t*>(stage + h * kRowB + 2 * d) = f32_to_bf16_rne(o[n][nt][i] * inv);
        }
      }
    }
    tile_barrier();                      // rows staged
  }
  mla_store_or_merge<kThreads>(reinterpret_cast<uint8_t*>(&sh.k[0][0]), &sh.counter, t, split,
                               n_split, n_split > 1, wait_ticks, out, lse, part_o, part_lse,
                               arrivals, call_tag);
}

// ------------------------------------------------------- one token per workgroup
// The same contraction for batches of many tokens without key splits
// (prefill), and for key splits longer than k_mla_ws takes: one workgroup
// per (token, split) of up to 2,048 indices, 4 waves (one per SIMD), 64-key tiles
// and v_mfma_f32_32x32x16_bf16, which one wave issues at the matrix cores'
// full rate (the 16x16x32 shape reaches about two thirds of it).
//  * Logits: wave w = (head group g = w & 1, key block kb = w >> 1) holds the
//    queries of heads 32 g .. 32 g + 31 in accumulator registers (read by the
//    MFMA directly) and computes their logits over keys 32 kb .. 32 kb + 31
//    of the tile, keys on M and heads on N: a lane holds one head and 16 keys
//    (8 j + 4 (l / 32) + i), so the per-head maxima and sums are in-lane
//    plus one permlane swap.
//  * Probabilities go to LDS as bf16 MFMA A operands: K-step u of key block
//    kb covers keys 16 u + 4 (l / 32) + i and 16 u + 8 + 4 (l / 32) + i, which
//    are exactly the lane's own keys j = 2 u, 2 u + 1.  They are taken
//    against the head's current reference before the other key block's
//    maximum is known; only when some maximum of the head group passes the
//    reference by more than the slack (the first tile with a row, then
//    rarely) does the group exchange maxima, move the reference, rescale
//    and take them again (one barrier per tile besides the tile barrier).
//  * P.V: wave w accumulates all 64 heads over value dims 128 w .. + 127
//    (O in registers), each value fragment read once with the transpose
//    load and feeding both head groups; operands three MFMA pairs ahead.
// Two tiles in LDS: the current one and the next one's DMA.  Each wave's 18
// DMA instructions of tile k + 1 are spread over tile k's MFMAs (issued all
// at once, they hold the wave at the issue until the memory queue has room,
// with no other wave on its SIMD).  The slot table holds half of the
// indices at a time (the second half replaces the first at tile 14, once
// the rows of tile 15 are read; rows are read one tile ahead of their DMA).
constexpr int kPfT = 64;                 // keys per tile
constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfHalf = 1024;            // slot-table entries resident at once
constexpr int kPfQSteps = kD / 16;       // 36 K-steps of the logits
struct MlaSharedPf {
  uint16_t k[2][kPfT * kD];              // two tiles in the layout of tile_byte (8 row groups)
  int32_t slots[kPfHalf];                // physical rows of one half of the indices, or -1
  uint32_t vbits[kMaxSplitLen / 32];     // per 32-key block: bit i = key i has a row
  u32x4 xp[2][2][2][64];                 // P: [head group][key block][K-step][lane]
  float xm[2][2][32];                    // per-head maxima of a key block (sums at the end)
  float xf[2][32];                       // per-head rescale factors (1 / sums at the end)
  alignas(16) uint32_t xflag[2];         // per head group: its factors apply
  alignas(16) uint32_t xneed[4];         // per wave: a maximum passed the reference
  uint32_t counter;                      // split merge: this workgroup merges
};
// LDS operations of P.V pairs i + 1 .. i + lead (four with a K-step's first
// pair, two otherwise), the count allowed outstanding when pair i's own
// operands must have arrived
constexpr int pv_ops_after(int i, int lead) {
  int n = 0;
  for (int j = i + 1; j <= i + lead && j < 16; ++j) n += (j % 4 == 0) ? 4 : 2;
  return n;
}
static_assert(sizeof(MlaSharedPf) <= 160 * 1024, "LDS budget");
static_assert(kH * kRowB + (kMaxSplits + 1) * kH * 4 <= sizeof(MlaSharedPf::k),
              "staged rows and merge weights fit in the tile buffers");

__global__ __launch_bounds__(kPfThreads, 1) void k_mla_prefill(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t n_tokens,
    int32_t n_split, int32_t split_len, float scale_log2,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q, int32_t B,
    const int32_t* __restrict__ block_table, int32_t max_blocks, int32_t block_size,
    int64_t num_slots, int32_t max_seq_len, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
    unsigned long long* __restrict__ arrivals, unsigned long long call_tag, int32_t wait_ticks) {
  __shared__ MlaSharedPf sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave & 1;               // logits: head group
  const int kb = wave >> 1;             // logits: key block of the tile
  const int n32 = lane & 31;            // logits: head 32 g + n32; P.V: dim column
  const int hh = lane >> 5;             // lane half
  // workgroup = (token, key split); the splits of a token on one XCD
  int vb = blockIdx.x;
  if (n_split > 1 && (gridDim.x & 7) == 0)
    vb = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int t = vb / n_split;
  const int split = vb % n_split;
  if (t >= n_tokens) return;
  // the split's indices: topk_idx[t][jbeg + j] for j < cnt (cnt <= 2048)
  const int jbeg = split * split_len;
  const int cnt = max(0, min(topk, jbeg + split_len) - jbeg);
  const int32_t* idx_row = topk_idx + static_cast<int64_t>(t) * topk + jbeg;
  const int ntiles = (cnt + kPfT - 1) / kPfT;             // <= 32 tiles

  // ---- the token's physical rows (8 indices per thread, j = tid + 256 i):
  // indices beside the request's place, then the block-table entries; the
  // queries are requested behind those
  constexpr int kPer = kMaxSplitLen / kPfThreads;          // 8
  int32_t p[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tid + kPfThreads * i;
    p[i] = j < cnt ? idx_row[j] : -1;
  }
  int b;
  int32_t pos;
  token_place(cu_q, seq_lens, B, t, max_seq_len, b, pos);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  int32_t sl[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool ok = p[i] >= 0 && p[i] <= pos && p[i] / block_size < max_blocks;
    const int32_t bid = ok ? bt_row[p[i] / block_size] : -1;
    const int64_t s0 = static_cast<int64_t>(bid) * block_size + (ok ? p[i] % block_size : 0);
    sl[i] = (bid >= 0 && s0 < num_slots) ? static_cast<int32_t>(s0) : -1;
  }
  asm volatile("" ::: "memory");
  // queries, the B operand of head group g: head 32 g + n32, dims 16 s + 8 hh
  bf16x8 qb[kPfQSteps];
  {
    const int64_t qbase = (static_cast<int64_t>(t) * kH + 32 * g + n32) * kD + 8 * hh;
#pragma unroll
    for (int st = 0; st < kPfQSteps; ++st)
      qb[st] = *reinterpret_cast<const bf16x8*>(q + qbase + 16 * st);
  }
  // slot table (first half) and validity masks of every 32-key block
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tid + kPfThreads * i;
    if (i < kPer / 2) sh.slots[j] = sl[i];
    const uint64_t m = __ballot(j < cnt && sl[i] >= 0);
    if (lane == 0) {
      sh.vbits[(kPfThreads * i + 64 * wave) / 32] = static_cast<uint32_t>(m);
      sh.vbits[(kPfThreads * i + 64 * wave) / 32 + 1] = static_cast<uint32_t>(m >> 32);
    }
  }
  tile_barrier();

  // DMA of a tile: wave w fills row groups 2 w and 2 w + 1 (nine 1 KB blocks
  // each, the lane map of tile_byte); rows without a physical row read row 0
  // A wave's 18 DMA instructions of a tile are issued one at a time, spread
  // over the previous tile's MFMAs: a wave that issues many at once waits
  // at the issue until the memory pipeline has room, with nothing else to
  // run on its SIMD.  src[hr] is the lane's row of group 2 w + hr.
  const uint8_t* src[2];
  // LDS address of the slot-table entry of the lane's row in group 2 w + hr
  // of a tile (entry 0 for a tile past the end)
  auto slot_addr = [&](int tile, bool real, int hr) {
    const int h = 2 * wave + hr;
    const int pi = (lane >> 3) ^ (h & 1);
    const int row = 8 * h + ((lane & 7) ^ (4 * (pi & 1)));
    const int j = real ? tile * kPfT + row : 0;
    return lds_addr(&sh.slots[j >= kPfHalf ? j - kPfHalf : j]);
  };
  auto set_src = [&](int hr, int32_t slot) {
    const int h = 2 * wave + hr;
    const int pi = (lane >> 3) ^ (h & 1);
    src[hr] = reinterpret_cast<const uint8_t*>(kv) +
              static_cast<uint64_t>(max(slot, 0)) * (2 * kD) + 16u * pi;
  };
  auto dma_rows = [&](int tile, bool real) {
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) {
      const int h = 2 * wave + hr;
      const int pi = (lane >> 3) ^ (h & 1);
      const int row = 8 * h + ((lane & 7) ^ (4 * (pi & 1)));
      const int j = real ? tile * kPfT + row : 0;
      set_src(hr, real ? sh.slots[j >= kPfHalf ? j - kPfHalf : j] : -1);
    }
  };
  // instruction d = 9 hr + G9 of the wave's share of a tile into buffer buf
  auto dma_one = [&](int buf, int d) {
    const int hr = d / 9, G9 = d % 9;
    uint8_t* dst = reinterpret_cast<uint8_t*>(sh.k[buf]) + 9216 * (2 * wave + hr) + 1024 * G9;
    __builtin_amdgcn_global_load_lds(src[hr] + 128 * G9,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  if (ntiles > 0) {
    dma_rows(0, true);
#pragma unroll
    for (int d = 0; d < 18; ++d) dma_one(0, d);
  }

  // logit operand offsets: row 32 kb + n32, piece 2 s + hh (group s / 4, an
  // immediate; four in-group offsets for s % 4)
  uint32_t ko[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const uint32_t full = tile_byte(32 * kb + n32, 2 * s4 + hh);
    ko[s4] = full;
  }
  // value operand offsets (transpose loads): within each 16-lane group G,
  // lane j supplies row 4 hh + j / 4 (+ 8 x) of a 16-key step and dims
  // 128 w + 32 d + 16 (G & 1) + 4 (j & 3) .. + 3; vo[x][d & 1] holds the
  // lane-dependent part, the rest is immediate
  const int j16 = lane & 15;
  const int G = lane >> 4;
  uint32_t vo[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int d1 = 0; d1 < 2; ++d1) {
      const int row = 8 * x + 4 * hh + (j16 >> 2);
      const int piece = 16 * wave + 4 * d1 + 2 * (G & 1) + ((j16 & 3) >> 1);
      vo[x][d1] = tile_byte(row, piece) + 8u * static_cast<uint32_t>(j16 & 1);
    }

  float m_ref = -INFINITY;              // head 32 g + n32
  float l_part = 0.0f;
  // O[g'][d]: heads 32 g' + 8 (r / 4) + 4 hh + r % 4, dims 128 w + 32 d + n32
  f32x16 o[2][4];
#pragma unroll
  for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
    for (int d = 0; d < 4; ++d) o[g2][d] = f32x16{};

  // the queries were requested before tile 0's DMA (18 loads per wave)
  wait_vm<18>();
#pragma unroll
  for (int st = 0; st < kPfQSteps; ++st) asm volatile("" : "+a"(qb[st]));

  // rows of tile 1, whose DMA is issued during tile 0
  dma_rows(1, 1 < ntiles);

  for (int k = 0; k < ntiles; ++k) {
    wait_vm<0>();                       // this wave's DMAs of tile k
    tile_barrier();                     // tile k landed; every wave is done with tile k - 1
    if (k == kPfHalf / kPfT - 2 && ntiles > kPfHalf / kPfT) {
      // the second half of the slot table: the rows of tile 15 were read at
      // the end of tile 13, those of tile 16 are read at the end of this one
#pragma unroll
      for (int i = 0; i < kPer / 2; ++i) sh.slots[tid + kPfThreads * i] = sl[kPer / 2 + i];
      tile_barrier();
    }
    const int nbuf = (k + 1) & 1;
    const uint32_t tb = lds_addr(sh.k[k & 1]);
    uint32_t vbw;

    // ---- logits of key block kb, head group g: 36 MFMAs, operands 3 ahead,
    // DMA instructions 0 .. 11 of tile k + 1 after every third
    f32x16 sacc = f32x16{};
    {
      constexpr int kAhead = 3;
      bf16x8 kr[kAhead];
      lgkm_drain();
      vbw = b32_load<0>(lds_addr(&sh.vbits[2 * k + kb]));   // completes before kr[0]
      static_for<kAhead>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        kr[S] = b128_load<1024 * (S >> 2)>(tb + ko[S & 3]);
      });
      static_for<kPfQSteps>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        constexpr int R = S % kAhead;
        constexpr int kAfter = (kPfQSteps - 1 - S) < (kAhead - 1) ? (kPfQSteps - 1 - S) : (kAhead - 1);
        lgkm_keep<kAfter>(kr[R]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[R], qb[S], sacc, 0, 0, 0);
        if constexpr (S % 3 == 0) dma_one(nbuf, S / 3);
        if constexpr (S + kAhead < kPfQSteps)
          kr[R] = b128_load<1024 * ((S + kAhead) >> 2)>(tb + ko[(S + kAhead) & 3]);
      });
    }
    // ---- softmax: lane (n32, hh) holds keys 8 j + 4 hh + i (register 4 j + i).
    // The probabilities are first taken against the current reference,
    // without waiting for the other key block's maximum: that is exact
    // unless a maximum of the group passes the reference by more than the
    // slack, which every wave of the group learns at the barrier, and then
    // the group takes them again against the common new reference (the
    // first tile with a row always does).
    lgkm_keep<0>(vbw);
    const uint32_t vbk = vbw >> (4 * hh);
    float z[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      z[r] = ((vbk >> (8 * (r >> 2) + (r & 3))) & 1u) ? sacc[r] : -INFINITY;
    float mx = z[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = max_nn(mx, z[r]);
    {
      const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
      mx = max_nn(__uint_as_float(c[0]), __uint_as_float(c[1])) * scale_log2;
    }
    if (hh == 0) sh.xm[g][kb][n32] = mx;
    const bool need = mx > m_ref + kMoveSlack;          // -inf reference: any row
    float psum;                         // the lane's share of the tile's sum
    auto probs = [&]() {
      const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(z[r], scale_log2, -mu));
      psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) psum += pr[r];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 pk;
        pk[0] = pack2_bf16(pr[8 * u + 0], pr[8 * u + 1]);
        pk[1] = pack2_bf16(pr[8 * u + 2], pr[8 * u + 3]);
        pk[2] = pack2_bf16(pr[8 * u + 4], pr[8 * u + 5]);
        pk[3] = pack2_bf16(pr[8 * u + 6], pr[8 * u + 7]);
        sh.xp[g][kb][u][lane] = pk;
      }
    };
    probs();
    {
      const bool any_need = __ballot(need) != 0;
      if (lane == 0) sh.xneed[wave] = any_need ? 1u : 0u;
    }
    tile_barrier();                     // probabilities and the groups' flags published

    // ---- P.V over the tile: 16 MFMA pairs (K-step st = i / 4, dim block
    // d = i % 4; both head groups share the value operand).  Operands are
    // requested three pairs ahead: the probabilities of both head groups
    // with the first pair of a K-step, two value fragments with each pair.
    // DMA instructions 12 .. 17 of tile k + 1 follow pairs 0 .. 5.
    // The groups' flags and the slot-table entries of tile k + 2 are
    // requested ahead of the first operands; the first three pairs'
    // operands are requested again if a group takes its probabilities anew.
    const uint32_t pb = lds_addr(&sh.xp[0][0][0][lane]);
    {
      constexpr int kLead = 3;
      bf16x8 pa[2][2];
      v4i16 vv[4][2];
      auto issue = [&](auto ic) {
        constexpr int I = decltype(ic)::value;
        constexpr int ST = I >> 2, D = I & 3, KB2 = ST >> 1, U = ST & 1;
        if constexpr (D == 0) {
          pa[ST & 1][0] = b128_load<1024 * (0 * 4 + KB2 * 2 + U)>(pb);
          pa[ST & 1][1] = b128_load<1024 * (1 * 4 + KB2 * 2 + U)>(pb);
        }
        constexpr int kVImm = 9216 * (4 * KB2 + 2 * U) + 1024 * (D >> 1);
        vv[D][0] = tr_load<kVImm>(tb + vo[0][D & 1]);
        vv[D][1] = tr_load<kVImm>(tb + vo[1][D & 1]);
      };
      const bool next_real = k + 2 < ntiles;
      u32x4 nd = u128_load<0>(lds_addr(sh.xneed));
      uint32_t sv0 = b32_load<0>(slot_addr(k + 2, next_real, 0));
      uint32_t sv1 = b32_load<0>(slot_addr(k + 2, next_real, 1));
      static_for<kLead>([&](auto ic) { issue(ic); });
      lgkm_keep<2 + pv_ops_after(-1, kLead)>(nd);
      if ((nd[0] | nd[1] | nd[2] | nd[3]) != 0) {
        lgkm_drain();
        // waves g and g + 2 hold head group g
        if ((nd[g] | nd[g + 2]) != 0) {
          const float mxa = max_nn(mx, sh.xm[g][kb ^ 1][n32]);
          float factor = 1.0f;
          bool moved = false;
          if (m_ref == -INFINITY) {
            m_ref = mxa;                // stays -inf while no key has a row
          } else if (mxa > m_ref + kMoveSlack) {
            factor = __builtin_amdgcn_exp2f(m_ref - mxa);
            m_ref = mxa;
            moved = true;
          }
          l_part *= factor;
          probs();
          const bool any = __ballot(moved) != 0;
          if (kb == 0) {
            if (any && hh == 0) sh.xf[g][n32] = factor;
            if (lane == 0) sh.xflag[g] = any ? 1u : 0u;
          }
        } else if (kb == 0 && lane == 0) {
          sh.xflag[g] = 0u;
        }
        tile_barrier();                 // probabilities and factors published
        // a head group whose references moved is rescaled before P.V
        const uint32_t f0 = sh.xflag[0], f1 = sh.xflag[1];
        if (f0 | f1) {
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            if (!(g2 ? f1 : f0)) continue;
            float fr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) fr[r] = sh.xf[g2][8 * (r >> 2) + 4 * hh + (r & 3)];
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[g2][d][r] *= fr[r];
          }
        }
        lgkm_drain();
        static_for<kLead>([&](auto ic) { issue(ic); });
      }
      l_part += psum;
      static_for<16>([&](auto ic) {
        constexpr int I = decltype(ic)::value;
        constexpr int ST = I >> 2, D = I & 3;
        if constexpr (I + kLead < 16) issue(std::integral_constant<int, I + kLead>{});
        // operations issued after pair I's: those of pairs I + 1 .. I + kLead
        constexpr int kAfter = pv_ops_after(I, kLead);
        if constexpr (D == 0) {
          lgkm_keep<kAfter + 2>(pa[ST & 1][0]);
          lgkm_keep<kAfter + 2>(pa[ST & 1][1]);
        }
        lgkm_keep<kAfter>(vv[D][0]);
        lgkm_keep<kAfter>(vv[D][1]);
        const v8i16 v01 = __builtin_shufflevector(vv[D][0], vv[D][1], 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, v01);
        o[0][D] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ST & 1][0], vop, o[0][D], 0, 0, 0);
        o[1][D] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ST & 1][1], vop, o[1][D], 0, 0, 0);
        if constexpr (I < 6) dma_one(nbuf, 12 + I);
      });
      // rows of tile k + 2 for the DMA issued during tile k + 1 (row 0
      // after the last tile)
      lgkm_keep<0>(sv0);
      lgkm_keep<0>(sv1);
      set_src(0, next_real ? static_cast<int32_t>(sv0) : -1);
      set_src(1, next_real ? static_cast<int32_t>(sv1) : -1);
    }
  }
  wait_vm<0>();                          // the DMA issued during the last tile
  tile_barrier();                        // every wave is done with the tiles

  // ---- per-head sums, lse, 1 / sum
  {
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part),
                                                    false, false);
    const float lw = __uint_as_float(c[0]) + __uint_as_float(c[1]);
    if (hh == 0) sh.xm[g][kb][n32] = lw;
  }
  tile_barrier();
  if (kb == 0 && hh == 0) {
    const float l = sh.xm[g][0][n32] + sh.xm[g][1][n32];
    sh.xf[g][n32] = l > 0.0f ? 1.0f / l : 0.0f;
    const float lh = l > 0.0f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
    const int h = 32 * g + n32;
    if (n_split > 1)
      __hip_atomic_store(part_lse + (static_cast<int64_t>(t) * n_split + split) * kH + h,
                         lh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else if (lse)
      lse[static_cast<int64_t>(t) * kH + h] = lh;
  }
  tile_barrier();
  // ---- normalised bf16 rows into the staging block (over the tiles), then
  // out (or stored as this split's partial, the last split merging)
  uint8_t* stage = reinterpret_cast<uint8_t*>(&sh.k[0][0]);
#pragma unroll
  for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hl = 8 * (r >> 2) + 4 * hh + (r & 3);
      const float inv = sh.xf[g2][hl];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int dim = 128 * wave + 32 * d + n32;
        *reinterpret_cast<uint16_t*>(stage + (32 * g2 + hl) * kRowB + 2 * dim) =
            f32_to_bf16_rne(o[g2][d][r] * inv);
      }
    }
  mla_store_or_merge<kPfThreads>(stage, &sh.counter, t, split, n_split, n_split > 1, wait_ticks,
                                 out, lse, part_o, part_lse, arrivals, call_tag);
}

// ---------------------------------------------------------------- vector path
constexpr int kVecMaxD = 1024;

__device__ __forceinline__ float ldv(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i])
              : static_cast<const float*>(p)[i];
}

__global__ __launch_bounds__(256) void k_mla_vector(
    const void* __restrict__ q, const void* __restrict__ kv, bool bf16,
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t n_heads,
    int32_t R, int32_t D, float scale, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, int32_t B,
    const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t block_size, int64_t num_slots, int32_t max_seq_len,
    void* __restrict__ out, float* __restrict__ lse) {
  __shared__ float sq[kVecMaxD];
  __shared__ float sz[DSA_MAX_TOPK];
  __shared__ int64_t sslot[DSA_MAX_TOPK];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int t = blockIdx.x / n_heads;
  const int h = blockIdx.x % n_heads;
  const int b = request_of(cu_q, B, t);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  const int32_t* idx_row = topk_idx + static_cast<int64_t>(t) * topk;
  const int64_t qb = (static_cast<int64_t>(t) * n_heads + h) * D;
  for (int d = tid; d < D; d += 256) sq[d] = ldv(q, qb + d, bf16);
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < topk; j += 256) {
    const int64_t slot = sel_slot(idx_row, j, topk, pos, bt_row, block_size,
                                  max_blocks, num_slots);
    sslot[j] = slot;
    float zj = -INFINITY;
    if (slot >= 0) {
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(sq[d], ldv(kv, slot * D + d, bf16), dot);
      zj = dot * scale;
    }
    sz[j] = zj;
    mx = fmaxf(mx, zj);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.0f;
  for (int j = tid; j < topk; j += 256) {
    const float e = sslot[j] >= 0 ? expf(sz[j] - mx) : 0.0f;
    sz[j] = e;
    sum += e;
  }
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  sum = red[0] + red[1] + red[2] + red[3];
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  const int64_t ob = (static_cast<int64_t>(t) * n_heads + h) * R;
  for (int r = tid; r < R; r += 256) {
    float acc = 0.0f;
    for (int j = 0; j < topk; ++j) {
      const int64_t slot = sslot[j];
      if (slot >= 0) acc = fmaf(sz[j], ldv(kv, slot * D + r, bf16), acc);
    }
    const float v = acc * inv;
    if (bf16)
      static_cast<uint16_t*>(out)[ob + r] = f32_to_bf16_rne(v);
    else
      static_cast<float*>(out)[ob + r] = v;
  }
  if (tid == 0 && lse)
    lse[static_cast<int64_t>(t) * n_heads + h] = sum > 0.0f ? mx + logf(sum) : -INFINITY;
}

}  // namespace

bool mla_mfma_ok(const dsa_batch& b, int dtype, int n_heads, int R, int P) {
  // slots are kept as 32-bit row numbers on this path
  return dtype == DSA_BF16 && R == kR && P == kP && n_heads == kH &&
         b.num_slots <= INT32_MAX;
}

int mla_choose_split(const dsa_batch* b, int dtype, int n_heads, int R, int P,
                     int topk) {
  if (!mla_mfma_ok(*b, dtype, n_heads, R, P)) return 1;
  // at most kMaxSplitLen indices per workgroup; beyond that, one workgroup
  // per CU at least: split the keys of each token until there are >= 256
  // workgroups, keeping >= 4 tiles per split
  const int min_split = max(1, (topk + kMaxSplitLen - 1) / kMaxSplitLen);
  const int64_t wgs = static_cast<int64_t>(b->num_q_tokens);
  if (wgs <= 0 || wgs >= 256) return min_split;
  int split = static_cast<int>((256 + wgs - 1) / wgs);
  const int max_split = min(kMaxSplits, max(1, topk / (4 * kT)));
  return max(min_split, min(split, max_split));
}

// How long (s_memrealtime ticks of 10 ns) a split waits for its token's
// other splits before it leaves its part of the merge to the last split:
// 20 us, or DSA_MERGE_WAIT_TICKS from the environment (0: never waits).
static int32_t merge_wait_ticks() {
  const char* e = getenv("DSA_MERGE_WAIT_TICKS");
  if (!e || !*e) return 2000;
  const long v = strtol(e, nullptr, 10);
  return v < 0 ? 0 : (v > 1000000 ? 1000000 : static_cast<int32_t>(v));
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
  const dsa_batch& b = a.b;
  if (b.num_q_tokens == 0) return hipSuccess;
  if (mla_mfma_ok(b, a.dtype, a.n_heads, a.R, a.P)) {
    const int n_split = a.n_split;
    int split_len = (a.topk + n_split - 1) / n_split;
    split_len = (split_len + kT - 1) / kT * kT;
    if (split_len > kMaxSplitLen || n_split > kMaxSplits) return hipErrorInvalidValue;
    if (n_split > 1 && (!a.part_o || !a.part_lse || !a.arrivals || !a.call_tag))
      return hipErrorInvalidValue;
    const int64_t grid = static_cast<int64_t>(b.num_q_tokens) * n_split;
    // one workgroup per CU (both kernels take most of the LDS): when the
    // grid fits the device every split of a token is resident at once, and
    // the owners of the merge parts wait for the last split (at most
    // merge_wait_ticks()) and merge their parts in parallel
    const int32_t wait_ticks = grid <= device_cus() ? merge_wait_ticks() : 0;
    if (n_split > 1 && split_len <= kWsSplitCap) {
      // key splits short enough for the warp-specialised pipeline's slot table
      k_mla_ws<<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(
          static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv),
          a.idx, a.topk, b.num_q_tokens, n_split, split_len, a.scale * kLog2e,
          b.seq_lens, b.cu_q, b.num_reqs, b.block_table, b.max_blocks,
          b.block_size, b.num_slots, b.max_seq_len,
          static_cast<uint16_t*>(a.out), a.lse, a.part_o, a.part_lse, a.arrivals,
          a.call_tag, wait_ticks);
      return hipGetLastError();
    }
    // longer splits (up to kMaxSplitLen indices), or one per token
    k_mla_prefill<<<static_cast<unsigned>(grid), kPfThreads, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv),
        a.idx, a.topk, b.num_q_tokens, n_split, split_len, a.scale * kLog2e,
        b.seq_lens, b.cu_q, b.num_reqs, b.block_table, b.max_blocks,
        b.block_size, b.num_slots, b.max_seq_len,
        static_cast<uint16_t*>(a.out), a.lse, a.part_o, a.part_lse, a.arrivals,
        a.call_tag, wait_ticks);
    return hipGetLastError();
  }
  const int64_t grid = static_cast<int64_t>(b.num_q_tokens) * a.n_heads;
  k_mla_vector<<<static_cast<unsigned>(grid), 256, 0, stream>>>(
      a.q, a.kv, a.dtype == DSA_BF16, a.idx, a.topk, a.n_heads, a.R, a.R + a.P,
      a.scale, b.seq_lens, b.cu_q, b.num_reqs, b.block_table, b.max_blocks,
      b.block_size, b.num_slots, b.max_seq_len, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa

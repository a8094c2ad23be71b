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
// Matrix-core path (bf16, R = 512, P = 64, 64 heads): one workgroup per
// (query token, key split) covers all 64 heads, so every selected latent row
// crosses HBM once per token.  Rows are gathered in 32-row tiles straight
// from HBM into LDS (global_load_lds_dwordx4) through a ring of four tile
// buffers (whole 128-byte lines per DMA instruction): three tiles are in
// flight while one is multiplied.  Eight waves, two per SIMD; the first
// four also issue the tile DMAs, so when one of them waits for room in the
// memory queue the other wave on its SIMD keeps the matrix core busy:
//   logits: wave w = 2 hg + kh: the 16 keys 16 kh .. 16 kh + 15 of the tile
//           against the 16 heads of head group hg over all 576 dims
//           (v_mfma_f32_16x16x32_bf16, queries in registers), so each tile
//           row is read from LDS by four waves;
//   softmax: the two waves of a head group swap their per-head maxima and
//           publish their bf16 probabilities in LDS; the reference maximum
//           moves rarely (only when a tile beats it by more than 64 in
//           base-2 log units), so the common tile needs no rescale of the
//           accumulators;
//   P.V:    wave w = 4 php + pq: the 32 heads of head groups 2 php and
//           2 php + 1 over value dims 128 pq .. 128 pq + 127 and all 32
//           keys; each value fragment, read with the gfx950 LDS transpose
//           load straight from the row-major tile, feeds two MFMAs (one per
//           head group), so each value element is read by two waves instead
//           of four.
// With more than one key split, each split writes its normalised partial
// output and log-sum-exp, and the split that finishes last merges them by
// LSE weights (splits of a token are placed on one XCD, so the partials it
// reads back are still in that XCD's L2).
//
// Vector path (fp32 or other shapes): one workgroup per (token, head),
// fp32 arithmetic, logits in LDS.
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
constexpr int kPvHT = 2;                // 16-head tiles per wave in P.V
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

struct MlaShared {
  uint16_t k[kBufs][kT * kD];           // row-major tiles, 4 x 36864 B
  int32_t slots[kMaxSplitLen];          // physical row of each index, or -1
  uint32_t vbits[kMaxSplitLen / kT];    // per tile: bit k = key k has a row
  u32x2 xp[kWavesM][kHT][64];           // bf16 probabilities, per wave / head tile / lane
  float xm[kWavesM][kHT][64];           // per-head tile maxima (sums at the end)
  alignas(16) uint32_t xf[kWavesM];     // per wave: a reference maximum moves
  alignas(16) uint32_t xr[kWavesM];     // per wave: the split must restart
  uint32_t counter;
};
static_assert(sizeof(MlaShared) <= 160 * 1024, "LDS budget");
static_assert(kH * (kR * 2 + 16) + (kMaxSplits + 1) * kH * 4 <= sizeof(MlaShared::k),
              "staged partials and merge weights fit in the tile buffers");

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

// Arrival count of a split at its token's word.  The word holds the tag of
// the call that last counted there (upper 48 bits) and that call's
// arrivals (lower 16): a word with another tag, whatever the workspace held
// before, counts as no arrival.  A compare-and-swap fails only when another
// split of the token changed the word after it was read, which each of them
// does once, so the loop ends within n_split + 1 rounds (the first may
// fail on the guess below).
__device__ __forceinline__ float lo_f(unsigned long long u) {
  return __uint_as_float(static_cast<uint32_t>(u));
}
__device__ __forceinline__ float hi_f(unsigned long long u) {
  return __uint_as_float(static_cast<uint32_t>(u >> 32));
}

// The first compare-and-swap guesses that every other split has already
// counted, so the split that arrives last (the one that merges, on the
// kernel's critical path) usually needs a single round trip; a wrong guess
// costs the others one more.
__device__ uint32_t arrive(unsigned long long* word, unsigned long long tag, int n_split) {
  unsigned long long cur = (tag << 16) | static_cast<unsigned long long>(n_split - 1);
  for (int round = 0; round <= n_split + 1; ++round) {
    const unsigned long long next = (cur >> 16) == tag ? cur + 1 : (tag << 16) | 1ull;
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

// whether any wave's flag word is set (kWavesM words, 16-byte aligned)
__device__ __forceinline__ bool any_word(const uint32_t* w) {
  static_assert(kWavesM % 4 == 0, "flag words are read four at a time");
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < kWavesM; i += 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + i);
    o |= v[0] | v[1] | v[2] | v[3];
  }
  return o != 0;
}

__device__ __forceinline__ u32x2 pack_bf16x4(const float* p) {
  u32x2 r;
  r[0] = pack2_bf16(p[0], p[1]);
  r[1] = pack2_bf16(p[2], p[3]);
  return r;
}

// The workgroup's staged result leaves it.  stage holds the normalised
// bf16 rows of its 64 heads (head h at byte h * kRowB, kRowB = 2 R + 16),
// and every lse is stored already (into lse, or as a partial).  With one
// split the rows are copied to out; with several, this split's rows are
// stored as its partial, and the split that arrives last at the token's
// word merges all of them.  Every thread of the workgroup calls it; stage
// must have room behind the rows for the merge weights.
constexpr int kRowB = kR * 2 + 16;
__device__ __forceinline__ void mla_store_or_merge(
    uint8_t* stage, uint32_t* counter, int t, int split, int n_split, bool partial,
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
    for (int c = tid; c < total; c += kThreads) {
      const int h = c / row_pieces, pc = c % row_pieces;
      dst[c] = *reinterpret_cast<const u32x4*>(stage + h * row_b + 16 * pc);
    }
    return;
  }
  // Partials (bf16, normalised) are read back by another workgroup of this
  // launch, maybe on another XCD: they are stored as relaxed device-scope
  // atomics, which the hardware keeps coherent across XCDs by themselves,
  // so no cache-wide write-back or invalidation is needed to hand them
  // over.  8-byte words (4 dims), consecutive lanes on consecutive words,
  // so every store instruction writes four whole 128-byte lines: thread tid
  // takes word tid % 128 of head rows tid / 128 + 2 i.
  constexpr int kWords = kR / 4;                   // 8-byte words per head row
  constexpr int kRowsPer = kThreads / kWords;      // head rows per pass (4)
  const int wq = tid % kWords;
  const int h0 = tid / kWords;
  unsigned long long* dst = reinterpret_cast<unsigned long long*>(
      part_o + (static_cast<int64_t>(t) * n_split + split) * kH * kR);
#pragma unroll 8
  for (int i = 0; i < kH / kRowsPer; ++i) {
    const int h = h0 + kRowsPer * i;
    const unsigned long long v =
        *reinterpret_cast<const unsigned long long*>(stage + h * row_b + 8 * wq);
    __hip_atomic_store(dst + h * kWords + wq, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- the split that arrives last merges the token's partials.  Every
  // thread waits until its partial stores have completed (reached the
  // device-coherent level) before the workgroup counts its arrival; the
  // merging workgroup loads the others' partials only after its own count
  // came back, with device-scope atomic loads.
  wait_vm<0>();
  __syncthreads();
  if (tid == 0) *counter = arrive(arrivals + t, call_tag, n_split) == static_cast<uint32_t>(n_split);
  __syncthreads();
  if (!*counter) return;
  asm volatile("" ::: "memory");
  // Thread tid merges dims 4 wq .. 4 wq + 3 of heads h0 + 2 i (as the
  // partials were written: whole lines per instruction).  Splits are
  // summed in split order (0, 1, ...) whichever finished last, so the
  // result does not depend on the arrival order; this split's own partial
  // comes from the staged block, rounded exactly as the others read theirs.
  const unsigned long long* po = reinterpret_cast<const unsigned long long*>(
      part_o + static_cast<int64_t>(t) * n_split * kH * kR) + wq;
  auto word = [&](int s, int h) -> unsigned long long {
    return __hip_atomic_load(const_cast<unsigned long long*>(po + (s * kH + h) * kWords),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto own = [&](int h) -> unsigned long long {
    return *reinterpret_cast<const unsigned long long*>(stage + h * row_b + 8 * wq);
  };
  auto unpack = [](unsigned long long v, float (&x)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = __uint_as_float(static_cast<uint32_t>((v >> (16 * e)) & 0xFFFFu) << 16);
  };
  unsigned long long* ob = reinterpret_cast<unsigned long long*>(
      out + static_cast<int64_t>(t) * kH * kR) + wq;
  auto put = [&](int h, const float (&x)[4], float inv) {
    const unsigned long long v =
        static_cast<unsigned long long>(pack2_bf16(x[0] * inv, x[1] * inv)) |
        (static_cast<unsigned long long>(pack2_bf16(x[2] * inv, x[3] * inv)) << 32);
    ob[h * kWords] = v;
  };
  // with two splits, the other split's rows are in flight while the
  // weights are made
  unsigned long long u[kH / kRowsPer];
  if (n_split == 2) {
#pragma unroll
    for (int i = 0; i < kH / kRowsPer; ++i) u[i] = word(1 - split, h0 + kRowsPer * i);
  }
  // split weights exp(lse_s - max) per head in place of the log-sum-exps,
  // then 1 / their sum, behind the staged block
  float* wt = reinterpret_cast<float*>(stage + kH * row_b);
  for (int c = tid; c < n_split * kH; c += kThreads)
    wt[c] = __hip_atomic_load(part_lse + static_cast<int64_t>(t) * n_split * kH + c,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tid < kH) {
    float mx = -INFINITY;
    for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, wt[s * kH + tid]);
    float sum = 0.0f;
    for (int s = 0; s < n_split; ++s) {
      const float wgt = mx == -INFINITY ? 0.0f : expf(wt[s * kH + tid] - mx);
      wt[s * kH + tid] = wgt;
      sum += wgt;
    }
    wt[n_split * kH + tid] = sum > 0.0f ? 1.0f / sum : 0.0f;
    if (lse) lse[static_cast<int64_t>(t) * kH + tid] = sum > 0.0f ? mx + logf(sum) : -INFINITY;
  }
  __syncthreads();
  if (n_split == 2) {
#pragma unroll
    for (int i = 0; i < kH / kRowsPer; ++i) {
      const int h = h0 + kRowsPer * i;
      float m[4], o4[4], x[4];
      unpack(own(h), m);
      unpack(u[i], o4);
      const float w0 = wt[h], w1 = wt[kH + h];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = split == 0 ? m[e] : o4[e];
        const float p1 = split == 0 ? o4[e] : m[e];
        x[e] = fmaf(w1, p1, w0 * p0);
      }
      put(h, x, wt[2 * kH + h]);
    }
  } else {
    // Eight head rows at a time, splits in groups of four: the group's
    // words (the eight rows of each of its splits) are requested before any
    // is used, so a group costs one memory round trip rather than one per
    // split.  The loads are unconditional (a split past the last re-reads
    // the last, and this split's own words are read but taken from the
    // staged block), so the compiler issues them back to back.  Splits are
    // summed in split order.
    for (int i0 = 0; i0 < kH / kRowsPer; i0 += 8) {
      float acc[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = 0.0f;
      for (int s0 = 0; s0 < n_split; s0 += 4) {
        unsigned long long wv[4][8];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            wv[g][i] = word(min(s0 + g, n_split - 1), h0 + kRowsPer * (i0 + i));
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int sg = s0 + g;
          if (sg < n_split) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int h = h0 + kRowsPer * (i0 + i);
              float p[4];
              unpack(sg == split ? own(h) : wv[g][i], p);
              const float wgt = wt[sg * kH + h];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wgt, p[e], acc[i][e]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int h = h0 + kRowsPer * (i0 + i);
        put(h, acc[i], wt[n_split * kH + h]);
      }
    }
  }
  // every split of this call has arrived: clear the word, so that a replay
  // of the same launch (same tag) counts from zero again
  if (tid == 0) __hip_atomic_store(arrivals + t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup = (query token, key split), all 64 heads, kWavesM waves (two
// per SIMD).  Logits and softmax: wave w = 2 hg + kh, heads 16 kHT hg .. in
// kHT 16-head tiles n (head 16 kHT hg + 16 n + lane % 16 in the query
// operand).  P.V: wave w = 4 php + pq, heads 32 php .. 32 php + 31.
//   logits:  S^T[16 keys, 16 heads] = K . Q^T per head tile over 18 K-steps,
//            keys 16 kh + 4 g16 + i on the rows (lane group g16 = lane / 16),
//            so lane (l16, g16) holds head l16's logits of 4 keys;
//   softmax: max over the wave's 16 keys in-lane plus two permlane swaps,
//            then the partner wave's (2 hg + 1 - kh) maxima through LDS;
//   P.V:     O[16 heads, 16 dims] += P[16 heads, 32 keys] . V[32 keys, 16 dims]
//            for each of the wave's two head tiles, with K-index 8 g16 + e =
//            key 4 g16 + e (e < 4) or key 16 + 4 g16 + e - 4: lane (l16, g16)
//            of the P operand takes the 4 probabilities that lane holds in
//            the head group's kh = 0 wave, then those of its kh = 1 wave
//            (both from LDS), and two transpose loads of rows 4 g16 + c and
//            16 + 4 g16 + c give the value operand in the same key order.
__global__ __launch_bounds__(kThreads, 1) void k_mla_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t n_tokens,
    int32_t n_split, int32_t split_len, float scale_log2,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
    int32_t B, const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t block_size, int64_t num_slots, int32_t max_seq_len,
    uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
    unsigned long long* __restrict__ arrivals, unsigned long long call_tag) {
  __shared__ MlaShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g16 = lane >> 4;
  const int hg = wave >> 1;             // heads 16 kHT hg .. 16 kHT hg + 16 kHT - 1
  const int kh = wave & 1;
  const int partner = wave ^ 1;

  // Workgroups are dealt to the eight XCDs in turn (workgroup i to XCD
  // i % 8); with a grid that divides by 8, the splits of a token take
  // consecutive places in one XCD's share.
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
  const int jpad = jbeg + ntiles * kT;           // tile-aligned end

  // Index loads first: they depend only on t.
  constexpr int kIdxPer = kMaxSplitLen / kThreads;   // 4
  int32_t p[kIdxPer];
#pragma unroll
  for (int i = 0; i < kIdxPer; ++i) {
    const int j = jbeg + kThreads * i + tid;
    p[i] = j < jend ? idx_row[j] : -1;
  }
  const int b = request_of_wave(cu_q, B, t);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  int32_t bid[kIdxPer];
#pragma unroll
  for (int i = 0; i < kIdxPer; ++i) {
    const bool ok = p[i] >= 0 && p[i] <= pos && p[i] / block_size < max_blocks;
    bid[i] = ok ? bt_row[p[i] / block_size] : -1;
    if (!ok) p[i] = -1;
  }

  // Physical row of every index of this split (padded with -1 to whole
  // tiles) and a 32-bit validity mask per tile, in LDS.
#pragma unroll
  for (int i = 0; i < kIdxPer; ++i) {
    const int j = jbeg + kThreads * i + tid;      // a wave covers 64 aligned j
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

  static_assert(kQSteps / 4 == 4 && kPvNT == 8 && kDmaPerWave == 9 && kHT == 1,
                "the refill pieces 0..3 follow logit K-steps, 4..8 P.V dim tiles");
  // DMA of local tile `tile` into buffer `buf`: wave w < kDmaWaves fills
  // row group h = w, one instruction per piece group g (the other waves
  // issue none).  Keys without a row load row 0 (finite cache data) and are
  // masked out of the softmax.
  const int dpi = (lane >> 3) ^ (wave & 1);
  const int drow = 8 * wave + ((lane & 7) ^ (4 * (dpi & 1)));
  const uint32_t dcol = 16u * static_cast<uint32_t>(dpi);
  auto dma = [&](int tile, uint16_t* buf) {
    if (wave >= kDmaWaves) return;
    const int32_t sl = sh.slots[tile * kT + drow];
    const uint8_t* src = reinterpret_cast<const uint8_t*>(kv) +
                         static_cast<uint64_t>(max(sl, 0)) * (2 * kD) + dcol;
    uint8_t* dst = reinterpret_cast<uint8_t*>(buf) + 9216 * wave;
    static_for<kDmaPerWave>([&](auto g) {
      constexpr int G = decltype(g)::value;
      __builtin_amdgcn_global_load_lds(
          src + 128 * G, (__attribute__((address_space(3))) void*)(dst + 1024 * G), 16, 0, 0);
    });
  };

  // Per-lane LDS byte offsets inside a tile buffer.  Logits: the lane's key
  // row 16 kh + l16, even / odd K-steps.  Values: transpose-load rows
  // 4 g16 + l16 / 4 (keys 0..15, a) and 16 + 4 g16 + l16 / 4 (keys 16..31,
  // b) at dims 128 pq + 16 nt + 4 (l16 & 3), for nt & 3 = m.
  const int krow = 16 * kh + l16;
  const uint32_t kodd[2] = {tile_byte(krow, g16), tile_byte(krow, 4 + g16)};
  const int php = wave >> 2;            // P.V: head groups 2 php, 2 php + 1
  const int pq = wave & 3;              // P.V: value dims 128 pq .. 128 pq + 127
  const int vrow_a = 4 * g16 + (l16 >> 2);
  const int vrow_b = 16 + vrow_a;
  const int vb_lo = (l16 & 3) >> 1;
  uint32_t voff_a[4], voff_b[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    // piece 16 pq + 2 m + vb_lo (+ 8 (nt >> 2) as an immediate), half l16 & 1
    const uint32_t half = 8u * static_cast<uint32_t>(l16 & 1);
    voff_a[m] = tile_byte(vrow_a, 16 * pq + 2 * m + vb_lo) + half;
    voff_b[m] = tile_byte(vrow_b, 16 * pq + 2 * m + vb_lo) + half;
  }

  f32x4 o[kPvHT][kPvNT];                  // heads 32 php + 16 n + 4 g16 + i, dims 128 pq + 16 nt + l16
#pragma unroll
  for (int n = 0; n < kPvHT; ++n)
#pragma unroll
    for (int nt = 0; nt < kPvNT; ++nt) o[n][nt] = f32x4{0, 0, 0, 0};
  float m_ref[kHT], l_part[kHT];   // head 16 kHT hg + 16 n + l16: reference, this lane's sum
#pragma unroll
  for (int n = 0; n < kHT; ++n) {
    m_ref[n] = -INFINITY;
    l_part[n] = 0.0f;
  }

#pragma unroll
  for (int i = 0; i < kBufs - 1; ++i)
    if (i < ntiles) dma(i, sh.k[i]);

  // The query rows (logit B operand: head 16 kHT hg + 16 n + l16, dims
  // 32 st + 8 g16 .. +8) are loaded behind the first tiles' DMAs, so their
  // 72 KB overlap the tiles' latency instead of delaying the slot table and
  // the first DMAs.  The wait for them also covers those tiles (the count
  // is in issue order), which land at about the same time; the registers
  // are then re-defined by an empty asm, so the compiler's wait tracking
  // no longer ties the logits of every tile to outstanding loads.
  bf16x8 qb[kHT][kQSteps];
#pragma unroll
  for (int n = 0; n < kHT; ++n) {
    const int64_t qbase = (static_cast<int64_t>(t) * kH + 16 * kHT * hg + 16 * n + l16) * kD;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s)
      qb[n][s] = *reinterpret_cast<const bf16x8*>(q + qbase + 32 * s + 8 * g16);
  }
  wait_vm<0>();
#pragma unroll
  for (int n = 0; n < kHT; ++n)
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) asm volatile("" : "+v"(qb[n][s]));

  for (int it = 0; it < ntiles; ++it) {
    // this wave's part of tile `it` is in when at most the later tiles'
    // loads are pending
    const int later = min(ntiles - 1 - it, kBufs - 2);
    if (later >= 2) wait_vm<2 * kDmaPerWave>();
    else if (later == 1) wait_vm<kDmaPerWave>();
    else wait_vm<0>();
    tile_barrier();              // (A) tile `it` complete, tile it-1 released
    const uint16_t* kt = sh.k[it % kBufs];
    const uint32_t vb32 = sh.vbits[it];
    // The ring's refill (tile it + kBufs - 1 into the buffer tile it - 1
    // left) is issued one DMA instruction at a time, spread over the tile's
    // MFMAs (after every fourth logit K-step: pieces 0..3; after P.V dim
    // tiles 0, 2, 3, 5, 6: pieces 4..8) rather than all at once: with the memory
    // queue full an issue waits for room, and spread out those waits
    // overlap the MFMAs in flight.
    // This lane's source row is read here, before the logits' LDS counting
    // starts, and the value is tied so the read has returned by then.
    const bool refill = wave < kDmaWaves && it + kBufs - 1 < ntiles;
    int32_t rsl = wave < kDmaWaves ? sh.slots[min(it + kBufs - 1, ntiles - 1) * kT + drow] : 0;
    asm volatile("" : "+v"(rsl));
    const uint8_t* rsrc = reinterpret_cast<const uint8_t*>(kv) +
                          static_cast<uint64_t>(max(rsl, 0)) * (2 * kD) + dcol;
    uint8_t* rdst = reinterpret_cast<uint8_t*>(sh.k[(it + kBufs - 1) % kBufs]) + 9216 * wave;

    // ---- logits: part[n][i] = head 16 kHT hg + 16 n + l16, key 16 kh + 4 g16 + i
    // K-step st reads piece 4 st + g16 of the lane's row: group st >> 1 (an
    // immediate 1024 (st >> 1)) and one of two per-lane offsets.
    f32x4 part[kHT];
#pragma unroll
    for (int n = 0; n < kHT; ++n) part[n] = f32x4{0, 0, 0, 0};
    {
      const uint32_t kb = lds_addr(kt);
      const uint32_t kbase[2] = {kb + kodd[0], kb + kodd[1]};
      constexpr int kAhead = 4;
      bf16x8 kr[kAhead];
      lgkm_drain();
      static_for<kAhead>([&](auto st) {
        constexpr int S = decltype(st)::value;
        kr[S] = b128_load<1024 * (S >> 1)>(kbase[S & 1]);
      });
      static_for<kQSteps>([&](auto st) {
        constexpr int S = decltype(st)::value;
        bf16x8& cur = kr[S % kAhead];
        constexpr int kAfter = (kQSteps - 1 - S) < (kAhead - 1) ? (kQSteps - 1 - S) : (kAhead - 1);
        lgkm_keep<kAfter>(cur);
#pragma unroll
        for (int n = 0; n < kHT; ++n)
          part[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qb[n][S], part[n], 0, 0, 0);
        if constexpr (S + kAhead < kQSteps)
          cur = b128_load<1024 * ((S + kAhead) >> 1)>(kbase[(S + kAhead) & 1]);
        if constexpr (S % 4 == 3) {               // pieces 0 .. 3
          constexpr int G = S / 4;
          if (refill) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_global_load_lds(
                rsrc + 128 * G, (__attribute__((address_space(3))) void*)(rdst + 1024 * G), 16, 0, 0);
          }
        }
      });
      
    }

    // ---- softmax.  The scale is positive, so the raw logits order as the
    // scaled ones: maxima are taken raw and scaled once, and each
    // probability is exp2(fma(raw, scale, -reference)).  Keys without a row
    // take -inf (skipped when the whole tile has rows, the usual case).
    float zr[kHT][4], mx[kHT];
    if (__builtin_amdgcn_readfirstlane(vb32) == 0xFFFFFFFFu) {
#pragma unroll
      for (int n = 0; n < kHT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) zr[n][i] = part[n][i];
    } else {
      const uint32_t vbl = vb32 >> (16 * kh + 4 * g16);
#pragma unroll
      for (int n = 0; n < kHT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) zr[n][i] = ((vbl >> i) & 1u) ? part[n][i] : -INFINITY;
    }
    bool need = false;
#pragma unroll
    for (int n = 0; n < kHT; ++n) {
      const float r = max_nn(max3_nn(zr[n][0], zr[n][1], zr[n][2]), zr[n][3]);
      mx[n] = max_x16_x32(r) * scale_log2;
      need |= mx[n] > m_ref[n] + kMoveSlack;
    }
    // speculative probabilities against the current reference maxima
    float pr[kHT][4];
#pragma unroll
    for (int n = 0; n < kHT; ++n) {
      const float mu = m_ref[n] == -INFINITY ? 0.0f : m_ref[n];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pr[n][i] = __builtin_amdgcn_exp2f(fmaf(zr[n][i], scale_log2, -mu));
    }
    const bool wave_need = __ballot(need) != 0;
#pragma unroll
    for (int n = 0; n < kHT; ++n) {
      sh.xp[wave][n][lane] = pack_bf16x4(pr[n]);
      sh.xm[wave][n][lane] = mx[n];
    }
    if (lane == 0) sh.xf[wave] = wave_need ? 1u : 0u;
    tile_barrier();              // (B) maxima, flags and probabilities published
    if (any_word(sh.xf)) {
      // Some reference maximum of the workgroup moves; every wave takes this
      // branch.  A head's first key sets its reference (its sums are still
      // zero, nothing to rescale).  A head whose tile maximum beats its
      // reference by more than kMoveSlack would overflow: then the new maxima
      // become the references and the workgroup restarts its split from the
      // first tile with zero sums (later restarts can only come from later
      // tiles, so there are at most ntiles of them).  The accumulators are
      // never rescaled in place.
      bool restart = false;
#pragma unroll
      for (int n = 0; n < kHT; ++n) {
        const float mfull = fmaxf(mx[n], sh.xm[partner][n][lane]);
        const bool first = m_ref[n] == -INFINITY && mfull != -INFINITY;
        const bool over = m_ref[n] != -INFINITY && mfull > m_ref[n] + kMoveSlack;
        restart |= over;
        if (first || over) m_ref[n] = mfull;
        const float mu = m_ref[n] == -INFINITY ? 0.0f : m_ref[n];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pr[n][i] = __builtin_amdgcn_exp2f(fmaf(zr[n][i], scale_log2, -mu));
      }
#pragma unroll
      for (int n = 0; n < kHT; ++n) sh.xp[wave][n][lane] = pack_bf16x4(pr[n]);
      const bool wave_restart = __ballot(restart) != 0;   // all lanes vote
      if (lane == 0) sh.xr[wave] = wave_restart ? 1u : 0u;
      tile_barrier();            // (C) probabilities against the new maxima
      if (any_word(sh.xr)) {
#pragma unroll
        for (int n = 0; n < kHT; ++n) l_part[n] = 0.0f;
#pragma unroll
        for (int n = 0; n < kPvHT; ++n)
#pragma unroll
          for (int nt = 0; nt < kPvNT; ++nt) o[n][nt] = f32x4{0, 0, 0, 0};
        wait_vm<0>();
        tile_barrier();          // every wave is done with the ring
#pragma unroll
        for (int i = 0; i < kBufs - 1; ++i)
          if (i < ntiles) dma(i, sh.k[i]);
        it = -1;
        continue;
      }
    }
#pragma unroll
    for (int n = 0; n < kHT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) l_part[n] += pr[n][i];
    // P operands of head groups 2 php + n: keys 0..15 from wave 2 (2 php + n),
    // keys 16..31 from wave 2 (2 php + n) + 1, as published in LDS
    bf16x8 pa[kPvHT];
#pragma unroll
    for (int n = 0; n < kPvHT; ++n) {
      const u32x2 p0 = sh.xp[4 * php + 2 * n][0][lane];
      const u32x2 p1 = sh.xp[4 * php + 2 * n + 1][0][lane];
      const u32x4 v = {p0[0], p0[1], p1[0], p1[1]};
      pa[n] = __builtin_bit_cast(bf16x8, v);
    }

    // ---- O += P . V: 8 dim tiles of both head tiles, two transpose loads
    // per dim tile, 8 loads in flight.  Dim tile nt reads piece
    // 16 pq + 2 nt + b of its rows: group 2 pq + (nt >> 2) (an immediate
    // 1024 (nt >> 2)) and one of four per-lane offsets per row set.
    {
      const uint32_t tb = lds_addr(kt);
      uint32_t va[4], vb[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        va[m] = tb + voff_a[m];
        vb[m] = tb + voff_b[m];
      }
      constexpr int kLoads = 2 * kPvNT;               // 16
      constexpr int kAhead = 8;
      v4i16 vr[kAhead];
      auto vload = [&](auto ld) -> v4i16 {
        constexpr int L = decltype(ld)::value;
        constexpr int NT = L >> 1;
        return (L & 1) ? tr_load<1024 * (NT >> 2)>(vb[NT & 3])
                       : tr_load<1024 * (NT >> 2)>(va[NT & 3]);
      };
      lgkm_drain();
      static_for<kAhead>([&](auto ld) { vr[decltype(ld)::value] = vload(ld); });
      static_for<kPvNT>([&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        v4i16& a0 = vr[(2 * NT) % kAhead];
        v4i16& a1 = vr[(2 * NT + 1) % kAhead];
        // loads issued after load 2 NT + 1
        constexpr int kAfter = (kLoads - 2 - 2 * NT) < (kAhead - 2) ? (kLoads - 2 - 2 * NT) : (kAhead - 2);
        lgkm_keep<kAfter>(a0);
        lgkm_keep<kAfter>(a1);
        const v8i16 v01 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, v01);
#pragma unroll
        for (int n = 0; n < kPvHT; ++n)
          o[n][NT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[n], vop, o[n][NT], 0, 0, 0);
        if constexpr (2 * NT + kAhead < kLoads) {
          a0 = vload(std::integral_constant<int, 2 * NT + kAhead>{});
          a1 = vload(std::integral_constant<int, 2 * NT + kAhead + 1>{});
        }
        // pieces 4 .. 8 after dim tiles 0, 2, 3, 5, 6
        constexpr int G = NT == 0 ? 4 : NT == 2 ? 5 : NT == 3 ? 6 : NT == 5 ? 7 : NT == 6 ? 8 : -1;
        if constexpr (G >= 0) {
          if (refill) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_global_load_lds(
                rsrc + 128 * G, (__attribute__((address_space(3))) void*)(rdst + 1024 * G), 16, 0, 0);
          }
        }
      });
    }
  }

  // ---- epilogue: per-head sums, normalisation, staged coalesced stores
#pragma unroll
  for (int n = 0; n < kHT; ++n) l_part[n] = sum_x16_x32(l_part[n]);
  tile_barrier();                // every wave is done with the tiles and xm
#pragma unroll
  for (int n = 0; n < kHT; ++n) sh.xm[wave][n][lane] = l_part[n];
  tile_barrier();
  float lse_h[kHT];                // head 16 kHT hg + 16 n + l16
#pragma unroll
  for (int n = 0; n < kHT; ++n) {
    const float l = l_part[n] + sh.xm[partner][n][lane];
    lse_h[n] = l > 0.0f ? (m_ref[n] + log2f(l)) * kLn2 : -INFINITY;
  }
  float inv_l[kPvHT];              // head 32 php + 16 n + l16
#pragma unroll
  for (int n = 0; n < kPvHT; ++n) {
    const float l = sh.xm[4 * php + 2 * n][0][lane] + sh.xm[4 * php + 2 * n + 1][0][lane];
    inv_l[n] = l > 0.0f ? 1.0f / l : 0.0f;
  }
  const bool partial = n_split > 1;
  // rows of the staged block (bf16, the output's or the partial's values):
  // head h (0..63) at byte h * row_b of the tile buffers (free now); 16
  // bytes of padding per row spread the banks
  constexpr int row_b = kR * 2 + 16;
  uint8_t* stage = reinterpret_cast<uint8_t*>(&sh.k[0][0]);
  // heads i and i + 1 of a lane are converted together
#pragma unroll
  for (int n = 0; n < kPvHT; ++n) {
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const int hl = 4 * g16 + i;
      const float il0 = __shfl(inv_l[n], hl);
      const float il1 = __shfl(inv_l[n], hl + 1);
      const int h = 32 * php + 16 * n + hl;
#pragma unroll
      for (int nt = 0; nt < kPvNT; ++nt) {
        const int d = 128 * pq + 16 * nt + l16;
        const uint32_t pk = pack2_bf16(o[n][nt][i] * il0, o[n][nt][i + 1] * il1);
        *reinterpret_cast<uint16_t*>(stage + h * row_b + 2 * d) = static_cast<uint16_t>(pk);
        *reinterpret_cast<uint16_t*>(stage + (h + 1) * row_b + 2 * d) =
            static_cast<uint16_t>(pk >> 16);
      }
    }
  }
  if (kh == 0 && g16 == 0) {
#pragma unroll
    for (int n = 0; n < kHT; ++n) {
      const int h = 16 * kHT * hg + 16 * n + l16;
      if (partial)
        __hip_atomic_store(part_lse + (static_cast<int64_t>(t) * n_split + split) * kH + h,
                           lse_h[n], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (lse)
        lse[static_cast<int64_t>(t) * kH + h] = lse_h[n];
    }
  }
  mla_store_or_merge(stage, &sh.counter, t, split, n_split, partial, out, lse, part_o,
                     part_lse, arrivals, call_tag);
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
// Reference maxima: as in k_mla_mfma, a head's reference is fixed by its
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
    unsigned long long* __restrict__ arrivals, unsigned long long call_tag) {
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
  mla_store_or_merge(reinterpret_cast<uint8_t*>(&sh.k[0][0]), &sh.counter, t, split, n_split,
                     n_split > 1, out, lse, part_o, part_lse, arrivals, call_tag);
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
    if (n_split > 1 && split_len <= kWsSplitCap) {
      // key splits short enough for the warp-specialised pipeline's slot table
      k_mla_ws<<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(
          static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv),
          a.idx, a.topk, b.num_q_tokens, n_split, split_len, a.scale * kLog2e,
          b.seq_lens, b.cu_q, b.num_reqs, b.block_table, b.max_blocks,
          b.block_size, b.num_slots, b.max_seq_len,
          static_cast<uint16_t*>(a.out), a.lse, a.part_o, a.part_lse, a.arrivals,
          a.call_tag);
      return hipGetLastError();
    }
    k_mla_mfma<<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv),
        a.idx, a.topk, b.num_q_tokens, n_split, split_len, a.scale * kLog2e,
        b.seq_lens, b.cu_q, b.num_reqs, b.block_table, b.max_blocks,
        b.block_size, b.num_slots, b.max_seq_len,
        static_cast<uint16_t*>(a.out), a.lse, a.part_o, a.part_lse, a.arrivals,
        a.call_tag);
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

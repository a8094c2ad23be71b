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
// Matrix-core path (bf16, R = 512, P = 64, heads in groups of 32):
// a workgroup = (query token, group of 32 heads, key split), 4 waves.  Each
// 32-key tile of selected rows is gathered from HBM as 16-byte pieces of the
// 1152-byte rows (one row is 72 pieces; the 256 threads issue them
// back-to-back, so every row is fetched as whole 128-byte lines), and the
// next two tiles are in flight while the current one is multiplied.
// The tile is staged in LDS twice: row-major (the key operand of the logits,
// 8 consecutive dims per lane) and transposed for the first R dims (the
// value operand of P.V needs 8 consecutive keys per lane).
//   logits: v_mfma_f32_16x16x32_bf16, wave (mh, nk) computes 16 heads x 16
//           keys over 576 dims; its 16 query rows stay in registers;
//   softmax: online (running max / sum per head, base-2 exponentials);
//   P.V:    wave w accumulates O[32 heads, dims 128w .. 128w+127] in fp32.
// With more than one key split, each split writes its normalised partial
// output and log-sum-exp, and a combine kernel merges them by LSE weights.
//
// Vector path (fp32 or other shapes): one workgroup per (token, head),
// fp32 arithmetic, logits in LDS.
#include <type_traits>

#include "common.h"

namespace dsa {
namespace {

constexpr int kR = 512, kP = 64, kD = kR + kP;
constexpr int kH = 64;                  // heads per workgroup (all of them)
constexpr int kT = 32;                  // keys per tile
constexpr int kThreads = 256;           // 4 waves, one per SIMD
constexpr int kPS = kT + 8;             // P stride (elements)
constexpr int kPieces = kD / 8;         // 16-byte pieces per latent row (72)
constexpr int kTilePieces = kT * kPieces;             // 2304
constexpr int kDmaInstr = kTilePieces / 64;           // 36 wave loads per tile
constexpr int kDmaPerWave = kDmaInstr / 4;            // 9
constexpr int kBufs = 3;                // tiles resident: current + 2 in flight
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max used for the exponentials only moves when a tile's max
// exceeds it by more than this (in log2 units), so O is rarely rescaled;
// p = 2^(z - m) then stays below 2^8.
constexpr float kRescaleSlack = 8.0f;

typedef short v4i16 __attribute__((ext_vector_type(4)));

struct MlaShared {
  uint16_t k[kBufs][kT * kD];           // row-major tiles, 3 x 36864 B
  int64_t slots[DSA_MAX_TOPK];          // physical row of each index, or -1
  uint32_t vbits[DSA_MAX_TOPK / kT];    // per tile: bit k = key k has a row
  uint32_t counter;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
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

// 4 consecutive bf16 of LDS read with the gfx950 transpose load: within each
// 16-lane group, lane j supplies 4 elements that become A[4j .. 4j+3] and
// lane i receives A[i], A[16+i], A[32+i], A[48+i].
__device__ __forceinline__ v4i16 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
}

// Transpose loads issued as inline asm: as a builtin the compiler puts an
// s_waitcnt vmcnt(0) in front of each one (it assumes the load may read LDS
// still being written by a tile DMA), which would wait for the prefetch of
// the tile after next.  The caller waits for the results itself with
// lds_wait*() below, which take the result registers as operands so the
// compiler cannot use them earlier.  All LDS operations issued this way are
// retired with lgkmcnt(0) before the compiler issues LDS operations of its
// own again.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const uint16_t*)(p)));
}
__device__ __forceinline__ v4i16 tr_load(uint32_t addr) {
  v4i16 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ bf16x8 b128_load(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
// Waits until at most N LDS operations are outstanding; `r` is the register
// the next instruction consumes, tied so the compiler cannot read it earlier.
template <int N, typename T>
__device__ __forceinline__ void lgkm_keep(T& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "n"(N));
}
// cross-lane reductions over lanes l ^ 16 and l ^ 32 (gfx950 permlane swaps:
// each returns the values of the two lanes of the pair)
__device__ __forceinline__ float max_x16_x32(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float sum_x16_x32(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
// retire every outstanding LDS / scalar-memory operation of the compiler
// before an asm-counted sequence starts
__device__ __forceinline__ void lgkm_drain() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// A tile row is 72 16-byte pieces; piece c of row r is stored at piece
// position c ^ swz(r) of that row.  Rows are 1152 bytes (a multiple of the
// LDS bank width), so without the swizzle the 16 rows read by one MFMA
// operand load would hit the same banks.  swz < 8 keeps every position
// inside the row (0..63 and 64..71 map onto themselves).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int tile_elem(int row, int dim) {
  return row * kD + 8 * ((dim >> 3) ^ swz(row)) + (dim & 7);
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

// One workgroup = (query token, key split), all 64 heads, 4 waves (one per
// SIMD); wave w owns heads 16 w .. 16 w + 15 end to end.
//   logits:  S^T = K . Q^T over the tile's 32 keys (two
//            v_mfma_f32_16x16x32_bf16 tiles with keys on M): lane
//            (l16, g16) holds head l16's logits for keys 4 g16 + i and
//            16 + 4 g16 + i (i < 4), so the online-softmax max / sum are
//            in-lane plus two permlane-swap reductions;
//   P.V:     those 8 probabilities are, unchanged, the lane's A operand of
//            O[16 heads, 16 dims] += P[16 heads, 32 keys] . V[32 keys, 16 dims]
//            provided the value operand uses the same key order: the gfx950
//            transpose load of rows 4 g16 + c and 16 + 4 g16 + c gives lane
//            (l16, g16) exactly those keys for dim l16.  Probabilities never
//            leave registers, and the wave covers all 512 value dims.
// Tiles go straight from HBM into one of three LDS buffers
// (global_load_lds_dwordx4, 1 KB of LDS per wave instruction), so two tiles
// are in flight while the third is multiplied; LDS operand loads are
// software-pipelined (8 key loads, 16 transpose loads in flight).  One
// barrier per tile.
__global__ __launch_bounds__(kThreads, 1) void k_mla_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t n_tokens,
    int32_t n_split, int32_t split_len, float scale_log2,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
    int32_t B, const int32_t* __restrict__ block_table, int32_t max_blocks,
    int32_t block_size, int64_t num_slots, int32_t max_seq_len,
    uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ MlaShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g16 = lane >> 4;

  const int t = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  if (t >= n_tokens) return;

  // query rows of this wave's 16 heads (logit B operand): head 16 w + l16,
  // dims 32 s + 8 g16 .. +8; issued first, they only depend on t
  constexpr int kQS = kD / 32;                       // 18
  const int64_t qbase = (static_cast<int64_t>(t) * kH + 16 * wave + l16) * kD;
  bf16x8 qb[kQS];
#pragma unroll
  for (int s = 0; s < kQS; ++s)
    qb[s] = *reinterpret_cast<const bf16x8*>(q + qbase + 32 * s + 8 * g16);

  const int b = request_of_block(cu_q, B, t, &sh.counter);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  const int32_t* idx_row = topk_idx + static_cast<int64_t>(t) * topk;
  const int jbeg = split * split_len;
  const int jend = min(topk, jbeg + split_len);
  const int ntiles = jend > jbeg ? (jend - jbeg + kT - 1) / kT : 0;
  const int jpad = jbeg + ntiles * kT;           // tile-aligned end

  // Resolve the physical row of every index of this split once, into LDS
  // (padded with -1 to whole tiles), plus a 32-bit validity mask per tile:
  // index loads first, then block-table loads, each batch issued together.
  for (int j0 = jbeg; j0 < jpad; j0 += 8 * kThreads) {
    int32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + kThreads * i + tid;
      p[i] = j < jend ? idx_row[j] : -1;
    }
    int32_t bid[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = p[i] >= 0 && p[i] <= pos && p[i] / block_size < max_blocks;
      bid[i] = ok ? bt_row[p[i] / block_size] : -1;
      if (!ok) p[i] = -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + kThreads * i + tid;    // a wave covers 64 aligned j
      int64_t slot = -1;
      if (p[i] >= 0) {
        slot = static_cast<int64_t>(bid[i]) * block_size + p[i] % block_size;
        if (slot < 0 || slot >= num_slots) slot = -1;
      }
      if (j < jpad) sh.slots[j - jbeg] = slot;
      const uint64_t m = __ballot(j < jpad && slot >= 0);
      const int tw = (j0 + kThreads * i + 64 * wave - jbeg) / kT;
      if (lane == 0 && tw < ntiles) sh.vbits[tw] = static_cast<uint32_t>(m);
      if (lane == 0 && tw + 1 < ntiles) sh.vbits[tw + 1] = static_cast<uint32_t>(m >> 32);
    }
  }
  lds_barrier();

  f32x4 o[kR / 16];                     // dims 16 nt + l16, heads 4 g16 + i
#pragma unroll
  for (int nt = 0; nt < kR / 16; ++nt) o[nt] = f32x4{0, 0, 0, 0};
  float m_ref = -INFINITY, l_run = 0.0f;   // head 16 w + l16 (all g16 alike)

  // DMA of one tile into LDS buffer `kt`: wave instruction q (q = wave + 4 i)
  // fills LDS pieces 64 q .. 64 q + 63; lane l loads the global piece that
  // belongs at LDS piece 64 q + l.  Keys without a row load row 0 (finite
  // cache data) and are masked out of the softmax.
  auto dma = [&](int tile_beg, uint16_t* kt) {
    int64_t sl[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i)
      sl[i] = sh.slots[tile_beg - jbeg + (64 * (wave + 4 * i) + lane) / kPieces];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int qi = wave + 4 * i;
      const int pc = 64 * qi + lane;
      const int row = pc / kPieces;
      const int col = (pc % kPieces) ^ swz(row);
      const uint16_t* src = kv + (sl[i] < 0 ? 0 : sl[i]) * kD + col * 8;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(kt + 512 * qi), 16, 0, 0);
    }
  };

  // operand rows: keys l16 and 16 + l16 (logits), transpose loads of keys
  // 4 g16 + c and 16 + 4 g16 + c at dims 16 nt + vd (values)
  const int ksw0 = swz(l16), ksw1 = swz(16 + l16);
  const int vr0 = 4 * g16 + (l16 >> 2);
  const int vd = 4 * (l16 & 3);
  const int vsw0 = swz(vr0), vsw1 = swz(vr0 + 16);

  auto tile_step = [&](int it) {
    uint16_t* kt = sh.k[it % kBufs];
    // this tile's loads are done when at most the next tile's are pending
    if (it + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kDmaPerWave);   // vmcnt(9)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0)
    tile_barrier();
    // every wave is past step it-1, so buffer (it + 2) % 3 is free
    if (it + 2 < ntiles) dma(jbeg + (it + 2) * kT, sh.k[(it + 2) % kBufs]);
    const uint32_t vb32 = sh.vbits[it];

    // ---- logits S^T: part[c] holds keys 16 c + 4 g16 + i, head 16 w + l16.
    // 36 operand loads (load ld: step ld / 2, key half ld % 2), 8 in flight
    f32x4 part[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    {
      const uint32_t kb0 = lds_addr(&kt[l16 * kD]), kb1 = lds_addr(&kt[(16 + l16) * kD]);
      auto kaddr = [&](int ld) -> uint32_t {
        const int c = ld & 1, st = ld >> 1;
        return (c ? kb1 : kb0) + 16u * static_cast<uint32_t>((4 * st + g16) ^ (c ? ksw1 : ksw0));
      };
      constexpr int kLoads = 2 * kQS;
      bf16x8 kr[8];
      lgkm_drain();
#pragma unroll
      for (int ld = 0; ld < 8; ++ld) kr[ld] = b128_load(kaddr(ld));
#pragma unroll
      for (int ld = 0; ld < kLoads; ++ld) {
        bf16x8& cur = kr[ld & 7];
        constexpr int kAhead = 7;
        // loads issued after load ld: min(7, kLoads - 1 - ld)
        if (ld + kAhead <= kLoads - 1) lgkm_keep<7>(cur);
        else if (kLoads - 1 - ld == 6) lgkm_keep<6>(cur);
        else if (kLoads - 1 - ld == 5) lgkm_keep<5>(cur);
        else if (kLoads - 1 - ld == 4) lgkm_keep<4>(cur);
        else if (kLoads - 1 - ld == 3) lgkm_keep<3>(cur);
        else if (kLoads - 1 - ld == 2) lgkm_keep<2>(cur);
        else if (kLoads - 1 - ld == 1) lgkm_keep<1>(cur);
        else lgkm_keep<0>(cur);
        part[ld & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qb[ld >> 1], part[ld & 1], 0, 0, 0);
        if (ld + 8 < kLoads) kr[ld & 7] = b128_load(kaddr(ld + 8));
      }
    }

    // ---- online softmax over the tile (lane = head l16, keys of its g16)
    const uint32_t vbl = vb32 >> (4 * g16);
    float z[8];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[4 * c + i] = ((vbl >> (16 * c + i)) & 1u) ? part[c][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[4 * c + i]);
      }
    mx = max_x16_x32(mx);
    const bool move = mx > m_ref + kRescaleSlack || (m_ref == -INFINITY && mx != -INFINITY);
    const float m_new = move ? mx : m_ref;
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    float p[8];
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(z[e] - m_use);     // 0 for masked keys
      ps += p[e];
    }
    ps = sum_x16_x32(ps);
    if (__ballot(move)) {
      // rescale the rows of heads whose reference max moved (rare)
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g16 + i);
#pragma unroll
      for (int nt = 0; nt < kR / 16; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= a4[i];
      l_run *= alpha;
    }
    l_run += ps;
    m_ref = m_new;
    bf16x8 pa;
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[e] = static_cast<__bf16>(p[e]);

    // ---- O[16 heads, 512 dims] += P . V: 64 transpose loads (load 2 nt + c:
    // key half c of dim tile nt), 16 in flight
    {
      const uint32_t vb0 = lds_addr(&kt[vr0 * kD]), vb1 = lds_addr(&kt[(vr0 + 16) * kD]);
      auto vaddr = [&](int ld) -> uint32_t {
        const int c = ld & 1, nt = ld >> 1;
        const int dim = 16 * nt + vd;
        return (c ? vb1 : vb0) + 16u * static_cast<uint32_t>((dim >> 3) ^ (c ? vsw1 : vsw0)) +
               2u * static_cast<uint32_t>(dim & 7);
      };
      constexpr int kLoads = 2 * (kR / 16);           // 64
      v4i16 vr[16];
      lgkm_drain();
#pragma unroll
      for (int ld = 0; ld < 16; ++ld) vr[ld] = tr_load(vaddr(ld));
#pragma unroll
      for (int nt = 0; nt < kR / 16; ++nt) {
        v4i16& a0 = vr[(2 * nt) & 15];
        v4i16& a1 = vr[(2 * nt + 1) & 15];
        // loads issued after load 2 nt + 1: min(14, kLoads - 2 - 2 nt)
        if (2 * nt + 16 <= kLoads) { lgkm_keep<14>(a0); lgkm_keep<14>(a1); }
        else if (kLoads - 2 - 2 * nt == 12) { lgkm_keep<12>(a0); lgkm_keep<12>(a1); }
        else if (kLoads - 2 - 2 * nt == 10) { lgkm_keep<10>(a0); lgkm_keep<10>(a1); }
        else if (kLoads - 2 - 2 * nt == 8) { lgkm_keep<8>(a0); lgkm_keep<8>(a1); }
        else if (kLoads - 2 - 2 * nt == 6) { lgkm_keep<6>(a0); lgkm_keep<6>(a1); }
        else if (kLoads - 2 - 2 * nt == 4) { lgkm_keep<4>(a0); lgkm_keep<4>(a1); }
        else if (kLoads - 2 - 2 * nt == 2) { lgkm_keep<2>(a0); lgkm_keep<2>(a1); }
        else { lgkm_keep<0>(a0); lgkm_keep<0>(a1); }
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 v01 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, v01),
                                                        o[nt], 0, 0, 0);
        if (2 * nt + 16 < kLoads) {
          vr[(2 * nt) & 15] = tr_load(vaddr(2 * nt + 16));
          vr[(2 * nt + 1) & 15] = tr_load(vaddr(2 * nt + 17));
        }
      }
    }
  };

  if (ntiles > 0) dma(jbeg, sh.k[0]);
  if (ntiles > 1) dma(jbeg + kT, sh.k[1]);
  for (int it = 0; it < ntiles; ++it) tile_step(it);

  // ---- epilogue: rows of o are heads 16 w + 4 g16 + i
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  const float lse_h = l_run > 0.0f ? (m_ref + log2f(l_run)) * kLn2 : -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * g16 + i;
    const float il = __shfl(inv_l, hl);
    const int h = 16 * wave + hl;
#pragma unroll
    for (int nt = 0; nt < kR / 16; ++nt) {
      const int r = 16 * nt + l16;
      const float v = o[nt][i] * il;
      if (n_split == 1)
        out[(static_cast<int64_t>(t) * kH + h) * kR + r] = f32_to_bf16_rne(v);
      else
        part_o[((static_cast<int64_t>(t) * n_split + split) * kH + h) * kR + r] = v;
    }
  }
  if (g16 == 0) {
    const int h = 16 * wave + l16;
    if (n_split == 1) {
      if (lse) lse[static_cast<int64_t>(t) * kH + h] = lse_h;
    } else {
      part_lse[(static_cast<int64_t>(t) * n_split + split) * kH + h] = lse_h;
    }
  }
}

// merge split partials: one thread per (token, head, 8 dims); the split
// weights exp(lse_s - lse) are computed once per thread
__global__ __launch_bounds__(256) void k_mla_combine(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    int32_t N, int32_t n_heads, int32_t R, int32_t n_split,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int chunks = R / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(N) * n_heads * chunks) return;
  const int c = static_cast<int>(i % chunks);
  const int64_t th = i / chunks;                 // t * n_heads + h
  const int h = static_cast<int>(th % n_heads);
  const int64_t t = th / n_heads;
  float mx = -INFINITY;
  for (int s = 0; s < n_split; ++s)
    mx = fmaxf(mx, part_lse[(t * n_split + s) * n_heads + h]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float wsum = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const float wgt = expf(part_lse[(t * n_split + s) * n_heads + h] - mx);
      wsum += wgt;
      const f32x4* src = reinterpret_cast<const f32x4*>(
          part_o + ((t * n_split + s) * n_heads + h) * R + 8 * c);
      const f32x4 a = src[0], b = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += wgt * a[e];
        acc[4 + e] += wgt * b[e];
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  u32x4 packed;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    packed[e] = static_cast<uint32_t>(f32_to_bf16_rne(acc[2 * e] * inv)) |
                (static_cast<uint32_t>(f32_to_bf16_rne(acc[2 * e + 1] * inv)) << 16);
  *reinterpret_cast<u32x4*>(out + th * R + 8 * c) = packed;
  if (c == 0 && lse) lse[th] = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
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

bool mla_mfma_ok(int dtype, int n_heads, int R, int P) {
  return dtype == DSA_BF16 && R == kR && P == kP && n_heads == kH;
}

int mla_choose_split(const dsa_batch* b, int dtype, int n_heads, int R, int P,
                     int topk) {
  if (!mla_mfma_ok(dtype, n_heads, R, P)) return 1;
  // one workgroup per CU at least: split the keys of each token until there
  // are >= 256 workgroups, keeping >= 4 tiles per split
  const int64_t wgs = static_cast<int64_t>(b->num_q_tokens);
  if (wgs <= 0 || wgs >= 256) return 1;
  int split = static_cast<int>((256 + wgs - 1) / wgs);
  const int max_split = max(1, topk / (4 * kT));
  return min(split, max_split);
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
  const dsa_batch& b = a.b;
  if (b.num_q_tokens == 0) return hipSuccess;
  if (mla_mfma_ok(a.dtype, a.n_heads, a.R, a.P)) {
    const int n_split = a.n_split;
    int split_len = (a.topk + n_split - 1) / n_split;
    split_len = (split_len + kT - 1) / kT * kT;
    const int64_t grid = static_cast<int64_t>(b.num_q_tokens) * n_split;
    k_mla_mfma<<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv),
        a.idx, a.topk, b.num_q_tokens, n_split, split_len, a.scale * kLog2e,
        b.seq_lens, b.cu_q, b.num_reqs, b.block_table, b.max_blocks,
        b.block_size, b.num_slots, b.max_seq_len,
        static_cast<uint16_t*>(a.out), a.lse, a.part_o, a.part_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split == 1) return e;
    const int64_t total = static_cast<int64_t>(b.num_q_tokens) * a.n_heads * (kR / 8);
    k_mla_combine<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(
        a.part_o, a.part_lse, b.num_q_tokens, a.n_heads, kR, n_split,
        static_cast<uint16_t*>(a.out), a.lse);
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

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
constexpr int kDmaPerWave = kTilePieces / 64 / 4;     // 9 loads per wave per tile
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
  uint16_t p[kH * kPS];                 // probabilities (bf16), 5120 B
  float alpha[kH];                      // per-head O rescale of this tile
  float fin_l[kH];
  float fin_m[kH];
  int64_t slots[DSA_MAX_TOPK];          // physical row of each index, or -1
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

// One workgroup = (query token, key split), all 64 heads, 4 waves.
//   logits:  wave w computes S^T = K . Q^T for its 16 heads (16 w .. +16)
//            and the tile's 32 keys (two v_mfma_f32_16x16x32_bf16 tiles with
//            keys on M); each lane then holds 8 keys of one head, so the
//            online-softmax max / sum are in-lane plus two exchanges, and
//            the wave owns its heads' running statistics;
//   P.V:     wave w accumulates O[64 heads, dims 128 w .. +128] from the
//            probabilities of all heads (LDS) and the value rows read
//            straight from the row-major tile with transpose loads: a
//            16-lane group reads a 4-key x 16-dim block and each lane gets
//            4 keys of one dim, the MFMA operand layout.
// Gathered tiles go straight from HBM into one of three LDS tile buffers
// (global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS), so two
// tiles are in flight while the third is multiplied, with no register cost.
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
  const int b = request_of_block(cu_q, B, t, &sh.counter);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  const int32_t* idx_row = topk_idx + static_cast<int64_t>(t) * topk;
  const int jbeg = split * split_len;
  const int jend = min(topk, jbeg + split_len);

  // Resolve the physical row of every index of this split once, into LDS:
  // index loads first, then block-table loads, each batch issued together.
  // The gathers below then wait on no dependent global load.
  for (int j0 = jbeg; j0 < jend; j0 += 8 * kThreads) {
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
      const int j = j0 + kThreads * i + tid;
      if (j < jend) {
        int64_t slot = -1;
        if (p[i] >= 0) {
          slot = static_cast<int64_t>(bid[i]) * block_size + p[i] % block_size;
          if (slot < 0 || slot >= num_slots) slot = -1;
        }
        sh.slots[j - jbeg] = slot;
      }
    }
  }
  lds_barrier();

  // query rows of this wave's 16 heads (logit B operand): head 16 w + l16,
  // dims 32 s + 8 g16 .. +8
  const int64_t qbase = (static_cast<int64_t>(t) * kH + 16 * wave + l16) * kD;
  bf16x8 qb[kD / 32];
#pragma unroll
  for (int s = 0; s < kD / 32; ++s)
    qb[s] = *reinterpret_cast<const bf16x8*>(q + qbase + 32 * s + 8 * g16);

  f32x4 o[4][8];                        // [head tile][dim tile]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[mt][nt] = f32x4{0, 0, 0, 0};
  float m_ref = -INFINITY, l_run = 0.0f;   // head 16 w + l16 (all g16 alike)

  // DMA of one tile into LDS buffer `kt`: wave instruction q (q = wave + 4 i)
  // fills LDS pieces 64 q .. 64 q + 63; lane l loads the global piece that
  // belongs at LDS piece 64 q + l.  Keys without a row load row 0 (finite
  // cache data) and are masked out of the softmax.
  auto dma = [&](int tile_beg, uint16_t* kt) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int qi = wave + 4 * i;
      const int pc = 64 * qi + lane;
      const int row = pc / kPieces;
      const int col = (pc % kPieces) ^ swz(row);
      const int j = tile_beg + row;
      const int64_t slot = j < jend ? sh.slots[j - jbeg] : -1;
      const uint16_t* src = kv + (slot < 0 ? 0 : slot) * kD + col * 8;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(kt + 512 * qi), 16, 0, 0);
    }
  };

  const int ntiles = (jend - jbeg + kT - 1) / kT;
  auto tile_step = [&](int it) {
    const int tb = jbeg + it * kT;
    uint16_t* kt = sh.k[it % kBufs];
    // this tile's loads are done when at most the next tile's are pending
    if (it + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kDmaPerWave);   // vmcnt(9)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0)
    tile_barrier();
    // every wave is past step it-1, so buffer (it + 2) % 3 is free
    if (it + 2 < ntiles) dma(jbeg + (it + 2) * kT, sh.k[(it + 2) % kBufs]);

    // ---- logits S^T: key 16 kh + 4 g16 + i, head 16 w + l16
    f32x4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const bf16x8 kk = *reinterpret_cast<const bf16x8*>(
            &kt[tile_elem(16 * kh + l16, 32 * s + 8 * g16)]);
        acc[kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qb[s], acc[kh], 0, 0, 0);
      }
    }
    float z[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tb + 16 * kh + 4 * g16 + i;
        const bool ok = j < jend && sh.slots[j - jbeg] >= 0;
        z[4 * kh + i] = ok ? acc[kh][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[4 * kh + i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool move = mx > m_ref + kRescaleSlack || (m_ref == -INFINITY && mx != -INFINITY);
    const float m_new = move ? mx : m_ref;
    const float alpha = move ? exp2f(m_ref - m_new) : 1.0f;   // 0 from -inf
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    float ps = 0.0f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      uint32_t pk[2];
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float p0 = exp2f(z[4 * kh + i] - m_use);
        const float p1 = exp2f(z[4 * kh + i + 1] - m_use);
        ps += p0 + p1;
        pk[i / 2] = static_cast<uint32_t>(f32_to_bf16_rne(p0)) |
                    (static_cast<uint32_t>(f32_to_bf16_rne(p1)) << 16);
      }
      *reinterpret_cast<u32x2*>(&sh.p[(16 * wave + l16) * kPS + 16 * kh + 4 * g16]) =
          u32x2{pk[0], pk[1]};
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_ref = m_new;
    if (g16 == 0) sh.alpha[16 * wave + l16] = alpha;
    tile_barrier();

    // ---- O = alpha * O + P V for this wave's 128 dims
    float a16[4][4];
    bool any = false;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a16[mt][i] = sh.alpha[16 * mt + 4 * g16 + i];
        any |= a16[mt][i] != 1.0f;
      }
    if (__ballot(any)) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[mt][nt][i] *= a16[mt][i];
    }
    bf16x8 pa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      pa[mt] = *reinterpret_cast<const bf16x8*>(&sh.p[(16 * mt + l16) * kPS + 8 * g16]);
    // transpose-load rows 8 g16 + l16 / 4 (and +4) at dims 4 (l16 % 4) .. +4
    const int vr = 8 * g16 + (l16 >> 2);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int dim = 128 * wave + 16 * nt + 4 * (l16 & 3);
      const v4i16 v0 = lds_read_tr(&kt[tile_elem(vr, dim)]);
      const v4i16 v1 = lds_read_tr(&kt[tile_elem(vr + 4, dim)]);
      // whole-vector shuffle + bit cast (element-wise __bf16 inserts of the
      // transpose-load results were lowered into a broadcast of element 0)
      typedef short v8i16 __attribute__((ext_vector_type(8)));
      const v8i16 v01 = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, v01);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mt], vb, o[mt][nt], 0, 0, 0);
    }
  };

  if (ntiles > 0) dma(jbeg, sh.k[0]);
  if (ntiles > 1) dma(jbeg + kT, sh.k[1]);
  for (int it = 0; it < ntiles; ++it) tile_step(it);

  // ---- epilogue: every wave needs l / m of all 64 heads
  if (g16 == 0) {
    sh.fin_l[16 * wave + l16] = l_run;
    sh.fin_m[16 * wave + l16] = m_ref;
  }
  lds_barrier();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * mt + 4 * g16 + i;
      const float lh = sh.fin_l[h];
      const float il = lh > 0.0f ? 1.0f / lh : 0.0f;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int r = 128 * wave + 16 * nt + l16;
        const float v = o[mt][nt][i] * il;
        if (n_split == 1)
          out[(static_cast<int64_t>(t) * kH + h) * kR + r] = f32_to_bf16_rne(v);
        else
          part_o[((static_cast<int64_t>(t) * n_split + split) * kH + h) * kR + r] = v;
      }
    }
  }
  if (wave == 0) {
    const float lh = sh.fin_l[lane];
    const float lse_h = lh > 0.0f ? (sh.fin_m[lane] + log2f(lh)) * kLn2 : -INFINITY;
    if (n_split == 1) {
      if (lse) lse[static_cast<int64_t>(t) * kH + lane] = lse_h;
    } else {
      part_lse[(static_cast<int64_t>(t) * n_split + split) * kH + lane] = lse_h;
    }
  }
}

// merge split partials: one thread per (token, head, dim)
template <typename OutT>
__global__ __launch_bounds__(256) void k_mla_combine(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    int32_t N, int32_t n_heads, int32_t R, int32_t n_split,
    OutT* __restrict__ out, float* __restrict__ lse) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(N) * n_heads * R;
  if (i >= total) return;
  const int r = static_cast<int>(i % R);
  const int64_t th = i / R;                 // t * n_heads + h
  const int h = static_cast<int>(th % n_heads);
  const int64_t t = th / n_heads;
  float mx = -INFINITY;
  for (int s = 0; s < n_split; ++s)
    mx = fmaxf(mx, part_lse[(t * n_split + s) * n_heads + h]);
  float acc = 0.0f, wsum = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const float ls = part_lse[(t * n_split + s) * n_heads + h];
      const float wgt = expf(ls - mx);
      wsum += wgt;
      acc += wgt * part_o[((t * n_split + s) * n_heads + h) * R + r];
    }
  }
  const float v = wsum > 0.0f ? acc / wsum : 0.0f;
  if constexpr (sizeof(OutT) == 2)
    out[i] = f32_to_bf16_rne(v);
  else
    out[i] = v;
  if (r == 0 && lse) lse[th] = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
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
    const int64_t total = static_cast<int64_t>(b.num_q_tokens) * a.n_heads * kR;
    k_mla_combine<uint16_t><<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(
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

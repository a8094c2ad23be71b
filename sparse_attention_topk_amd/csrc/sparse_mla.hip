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
constexpr int kHG = 32;                 // heads per workgroup
constexpr int kT = 32;                  // keys per tile
constexpr int kKS = kD + 8;             // row-major key stride (elements)
constexpr int kVS = kT + 8;             // transposed value stride (elements)
constexpr int kPS = kT + 8;             // P stride (elements)
constexpr int kPieces = kD / 8;         // 16-byte pieces per latent row (72)
constexpr int kPerThread = kT * kPieces / 256;   // 9
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct MlaShared {
  uint16_t k[kT * kKS];                 // 37376 B
  uint16_t vt[kR * kVS];                // 40960 B
  float s[kHG][kT + 1];                 // logits exchange
  uint16_t p[4][kHG * kPS];             // per-wave probabilities (bf16)
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

__global__ __launch_bounds__(256, 1) void k_mla_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t n_tokens,
    int32_t n_heads, int32_t n_split, int32_t split_len, float scale_log2,
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
  const int mh = wave & 1;
  const int nk = wave >> 1;

  // Workgroup order: consecutive ids go round-robin over the 8 XCDs, so the
  // head groups of one (token, split) unit are given ids 8 apart; they land
  // on the same XCD and the second read of each gathered row hits its L2.
  const int n_hg = n_heads / kHG;
  const int lo8 = blockIdx.x & 7;
  const int hi = blockIdx.x >> 3;
  const int hg = hi % n_hg;
  const int unit = (hi / n_hg) * 8 + lo8;
  if (unit >= n_tokens * n_split) return;
  const int t = unit / n_split;
  const int split = unit % n_split;

  const int b = request_of_block(cu_q, B, t, &sh.counter);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  const int32_t* idx_row = topk_idx + static_cast<int64_t>(t) * topk;
  const int jbeg = split * split_len;
  const int jend = min(topk, jbeg + split_len);

  // Resolve the physical row of every index of this split once, into LDS:
  // index loads first, then block-table loads, each batch issued together.
  // The gathers below then wait on no dependent global load.
  for (int j0 = jbeg; j0 < jend; j0 += 8 * 256) {
    int32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + 256 * i + tid;
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
      const int j = j0 + 256 * i + tid;
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

  // query rows of this wave's 16 heads (logit A operand): head 16 mh + l16,
  // dims 32 s + 8 g16 .. +8
  const int64_t qbase = (static_cast<int64_t>(t) * n_heads + hg * kHG + mh * 16 + l16) * kD;
  bf16x8 qa[kD / 32];
#pragma unroll
  for (int s = 0; s < kD / 32; ++s)
    qa[s] = *reinterpret_cast<const bf16x8*>(q + qbase + 32 * s + 8 * g16);

  f32x4 o[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[mt][nt] = f32x4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;   // for head (lane & 31)

  // gather registers: piece c = tid + 256 i of the tile -> key c / 72,
  // 16-byte piece c % 72 of that key's row; consecutive threads read
  // consecutive pieces, so each row arrives as whole 128-byte lines
  auto gather = [&](u32x4 (&g)[kPerThread], int tile_beg) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + 256 * i;
      const int key = c / kPieces;
      const int pc = c % kPieces;
      const int j = tile_beg + key;
      const int64_t slot = j < jend ? sh.slots[j - jbeg] : -1;
      g[i] = slot >= 0 ? *reinterpret_cast<const u32x4*>(kv + slot * kD + pc * 8)
                       : u32x4{0, 0, 0, 0};
    }
  };
  // registers -> row-major LDS copy of the tile
  auto stage = [&](const u32x4 (&g)[kPerThread], int tile_beg) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + 256 * i;
      const int key = c / kPieces;
      const int pc = c % kPieces;
      *reinterpret_cast<u32x4*>(&sh.k[key * kKS + pc * 8]) = g[i];
    }
  };
  // row-major latent dims -> transposed value tile: unit u = (dim chunk
  // u / 16, key pair u % 16) reads 8 dims of two keys and writes 8 dwords,
  // each holding one dim of both keys
  auto transpose = [&]() {
#pragma unroll
    for (int i = 0; i < (kR / 8) * (kT / 2) / 256; ++i) {
      const int u = tid + 256 * i;
      const int kp = u & 15;
      const int dc = u >> 4;
      const u32x4 a = *reinterpret_cast<const u32x4*>(&sh.k[(2 * kp) * kKS + dc * 8]);
      const u32x4 c = *reinterpret_cast<const u32x4*>(&sh.k[(2 * kp + 1) * kKS + dc * 8]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t even = (a[m] & 0xFFFFu) | (c[m] << 16);
        const uint32_t odd = (a[m] >> 16) | (c[m] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(&sh.vt[(dc * 8 + 2 * m) * kVS + 2 * kp]) = even;
        *reinterpret_cast<uint32_t*>(&sh.vt[(dc * 8 + 2 * m + 1) * kVS + 2 * kp]) = odd;
      }
    }
  };

  auto tile_step = [&](u32x4 (&g)[kPerThread], int tb) {
    stage(g, tb);
    if (tb + 2 * kT < jend) gather(g, tb + 2 * kT);     // two tiles ahead
    lds_barrier();
    transpose();

    // ---- logits: 16 heads (mh) x 16 keys (nk)
    f32x4 acc = {0, 0, 0, 0};
    const uint16_t* kb = &sh.k[(16 * nk + l16) * kKS + 8 * g16];
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) {
      const bf16x8 kk = *reinterpret_cast<const bf16x8*>(kb + 32 * s);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], kk, acc, 0, 0, 0);
    }
    {
      const int j = tb + 16 * nk + l16;
      const bool ok = j < jend && sh.slots[j - jbeg] >= 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sh.s[16 * mh + 4 * g16 + i][16 * nk + l16] = ok ? acc[i] * scale_log2 : -INFINITY;
    }
    lds_barrier();

    // ---- online softmax: lane handles head (lane & 31), keys 16*(lane>>5)..+16
    const int hh = lane & 31;
    const int kh = (lane >> 5) * 16;
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      z[j] = sh.s[hh][kh + j];
      mx = fmaxf(mx, z[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ps = 0.0f;
    uint16_t* pw = &sh.p[wave][hh * kPS + kh];
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const float p0 = exp2f(z[j] - m_use);
      const float p1 = exp2f(z[j + 1] - m_use);
      ps += p0 + p1;
      *reinterpret_cast<uint32_t*>(pw + j) =
          static_cast<uint32_t>(f32_to_bf16_rne(p0)) |
          (static_cast<uint32_t>(f32_to_bf16_rne(p1)) << 16);
    }
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // the P tile is wave-private: order its LDS writes before the reads below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

    // ---- O = alpha * O + P V for this wave's 128 dims
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 16 * mt + 4 * g16 + i);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[mt][nt][i] *= a4[i];
    }
    bf16x8 pa[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      pa[mt] = *reinterpret_cast<const bf16x8*>(&sh.p[wave][(16 * mt + l16) * kPS + 8 * g16]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int dim = 128 * wave + 16 * nt + l16;
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(&sh.vt[dim * kVS + 8 * g16]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mt], vb, o[mt][nt], 0, 0, 0);
    }
    lds_barrier();
  };

  u32x4 ga[kPerThread], gb[kPerThread];
  if (jbeg < jend) gather(ga, jbeg);
  if (jbeg + kT < jend) gather(gb, jbeg + kT);
  for (int tb = jbeg; tb < jend; tb += 2 * kT) {
    tile_step(ga, tb);
    if (tb + kT < jend) tile_step(gb, tb + kT);
  }

  // ---- epilogue
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  const float lse_h = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  const int head0 = hg * kHG;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = 16 * mt + 4 * g16 + i;
      const float il = __shfl(inv_l, hl);
      const int h = head0 + hl;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int r = 128 * wave + 16 * nt + l16;
        const float v = o[mt][nt][i] * il;
        if (n_split == 1)
          out[(static_cast<int64_t>(t) * n_heads + h) * kR + r] = f32_to_bf16_rne(v);
        else
          part_o[((static_cast<int64_t>(t) * n_split + split) * n_heads + h) * kR + r] = v;
      }
    }
  }
  if (wave == 0 && lane < 32) {
    const int h = head0 + lane;
    if (n_split == 1) {
      if (lse) lse[static_cast<int64_t>(t) * n_heads + h] = lse_h;
    } else {
      part_lse[(static_cast<int64_t>(t) * n_split + split) * n_heads + h] = lse_h;
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
  return dtype == DSA_BF16 && R == kR && P == kP && n_heads % kHG == 0 &&
         n_heads > 0;
}

int mla_choose_split(const dsa_batch* b, int dtype, int n_heads, int R, int P,
                     int topk) {
  if (!mla_mfma_ok(dtype, n_heads, R, P)) return 1;
  const int64_t wgs = static_cast<int64_t>(b->num_q_tokens) * (n_heads / kHG);
  if (wgs <= 0 || wgs >= 256) return 1;
  int split = static_cast<int>((256 + wgs - 1) / wgs);
  const int max_split = max(1, topk / (4 * kT));    // >= 4 tiles per split
  return min(split, max_split);
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
  const dsa_batch& b = a.b;
  if (b.num_q_tokens == 0) return hipSuccess;
  if (mla_mfma_ok(a.dtype, a.n_heads, a.R, a.P)) {
    const int n_split = a.n_split;
    int split_len = (a.topk + n_split - 1) / n_split;
    split_len = (split_len + kT - 1) / kT * kT;
    const int64_t units = static_cast<int64_t>(b.num_q_tokens) * n_split;
    const int64_t grid = (units + 7) / 8 * 8 * (a.n_heads / kHG);
    k_mla_mfma<<<static_cast<unsigned>(grid), 256, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv),
        a.idx, a.topk, b.num_q_tokens, a.n_heads, n_split, split_len,
        a.scale * kLog2e,
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

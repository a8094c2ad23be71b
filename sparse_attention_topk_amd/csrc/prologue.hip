// Indexer prologue (page "GLM5 TensorCast 适配设计", section "DSA Indexer
// fused semantic op": the op's inputs hidden_states, qa_normed, RoPE cos /
// sin, wq_b, wk, weights_proj, k_norm weight, head_dim, qk_rope_head_dim,
// and the indexer cache it writes; section "Performance model design",
// buckets 1-4: the q, k and head-weight projections and RoPE):
//
//     q = RoPE(qa_normed wq_b^T)             [N, H, D] bf16
//     k = RoPE(RMSNorm(hidden wk^T) * k_norm) [N, D]    bf16, into the cache
//     w = hidden weights_proj^T              [N, H]    fp32
//
// Weights are linear-layer weights [out, in], so both operands of every
// product run along the reduction dim in memory.  RoPE turns the pairs
// (j, j + R/2), j < R/2, of the first R dims by the token's angle j
// (rotate-half); the key's cache write is a bf16 copy, or on the FP8 path
// the activation rotation and quantisation of dsa_rotate_quantize applied to
// the bf16 key.
//
// Two launches.  k_proj_gemm: a split-K bf16 GEMM on 32x32x16 matrix-core
// tiles; a workgroup computes 64 tokens x 64 output columns over one K
// range, operands staged through LDS (double buffered), and writes fp32
// partial sums.  The q columns (H * D of them, K = q_lora_rank) and the k|w
// columns (D + H, K = hidden) are one grid.  k_proj_epilogue: one wave per
// (token, head) sums the q partials in split order and applies RoPE; one
// wave per token sums the k|w partials, normalises k, applies RoPE, writes
// k, the cache row and w.  The split order is fixed, so results are
// deterministic.
#include <algorithm>
#include <cmath>
#include <utility>

#include "common.h"

namespace dsa {
namespace {

constexpr int kBM = 64;            // tokens per GEMM tile
constexpr int kBN = 64;            // output columns per GEMM tile
constexpr int kBK = 32;            // reduction dims per stage
constexpr int kRowB = kBK * 2 + 16;   // LDS row bytes (16 bytes of padding)
constexpr int kPF = 4;             // stages in flight per workgroup

// f(integral_constant<int, I>) for I = 0 .. N-1
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

struct GemmPart {
  const uint16_t* a;      // [M, K] bf16 activations
  const uint16_t* w0;     // [n0, K] bf16 weights (columns 0 .. n0 - 1)
  const uint16_t* w1;     // [n1, K] bf16 weights (columns n0 .. n0 + n1 - 1) or null
  int32_t n0, n1, K;
  int32_t splits;         // K ranges (each a multiple of kBK)
  int32_t col_tiles;      // ceil((n0 + n1) / kBN)
  float* part;            // [splits, M, n0 + n1] fp32
};

// grid: [q tiles][kw tiles]; a tile = (token tile, column tile, split)
__global__ __launch_bounds__(256) void k_proj_gemm(GemmPart pq, GemmPart pk, int32_t M,
                                                   int32_t q_tiles) {
  __shared__ __align__(16) uint8_t sa[2][kBM * kRowB];
  __shared__ __align__(16) uint8_t sb[2][kBN * kRowB];
  const bool is_q = static_cast<int>(blockIdx.x) < q_tiles;
  const GemmPart& p = is_q ? pq : pk;
  int tile = is_q ? blockIdx.x : blockIdx.x - q_tiles;
  const int split = tile % p.splits;
  tile /= p.splits;
  const int ct = tile % p.col_tiles;
  const int mt = tile / p.col_tiles;
  const int n_tot = p.n0 + p.n1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ksteps = p.K / kBK;
  const int s_beg = static_cast<int>(static_cast<int64_t>(ksteps) * split / p.splits);
  const int s_end = static_cast<int>(static_cast<int64_t>(ksteps) * (split + 1) / p.splits);

  // staging: thread tid carries 16 bytes of row tid / 4 (piece tid % 4) of
  // both tiles; rows past the matrix load zeros
  const int lrow = tid >> 2, lpc = tid & 3;
  const int arow = mt * kBM + lrow;
  const int bcol = ct * kBN + lrow;
  const uint16_t* asrc = arow < M ? p.a + static_cast<int64_t>(arow) * p.K + 8 * lpc : nullptr;
  const uint16_t* bsrc = nullptr;
  if (bcol < p.n0) bsrc = p.w0 + static_cast<int64_t>(bcol) * p.K + 8 * lpc;
  else if (bcol < n_tot) bsrc = p.w1 + static_cast<int64_t>(bcol - p.n0) * p.K + 8 * lpc;
  auto load = [&](int s, u32x4& av, u32x4& bv) {
    const u32x4 z = {0, 0, 0, 0};
    av = asrc ? *reinterpret_cast<const u32x4*>(asrc + s * kBK) : z;
    bv = bsrc ? *reinterpret_cast<const u32x4*>(bsrc + s * kBK) : z;
  };
  auto stash = [&](int buf, const u32x4& av, const u32x4& bv) {
    *reinterpret_cast<u32x4*>(&sa[buf][lrow * kRowB + 16 * lpc]) = av;
    *reinterpret_cast<u32x4*>(&sb[buf][lrow * kRowB + 16 * lpc]) = bv;
  };

  // operand rows of this lane: token 32 wm + lane % 32, column 32 wn + lane
  // % 32; reduction dims 16 kk + 8 (lane / 32) .. + 7 of the stage
  const int orow = 32 * wm + (lane & 31);
  const int ocol = 32 * wn + (lane & 31);
  const int okb = 16 * (lane >> 5);
  // kPF stages in flight in registers (slot j holds stage s_beg + j, then
  // + kPF, ...); each stage is copied to the LDS buffer of its parity just
  // before it is needed, and its slot refilled kPF stages ahead
  u32x4 ra[kPF], rb[kPF];
  static_for<kPF>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if (s_beg + j < s_end) load(s_beg + j, ra[j], rb[j]);
  });
  f32x16 acc = {};
  if (s_beg < s_end) {
    stash(0, ra[0], rb[0]);
    if (s_beg + kPF < s_end) load(s_beg + kPF, ra[0], rb[0]);
  }
  __syncthreads();
  for (int s0 = s_beg; s0 < s_end; s0 += kPF) {
    static_for<kPF>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int s = s0 + j;
      if (s >= s_end) return;
      const int buf = (s - s_beg) & 1;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const bf16x8 a8 = *reinterpret_cast<const bf16x8*>(&sa[buf][orow * kRowB + 32 * kk + okb]);
        const bf16x8 b8 = *reinterpret_cast<const bf16x8*>(&sb[buf][ocol * kRowB + 32 * kk + okb]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, acc, 0, 0, 0);
      }
      if (s + 1 < s_end) {
        constexpr int jn = (j + 1) % kPF;          // slot of stage s + 1
        stash(buf ^ 1, ra[jn], rb[jn]);
        if (s + 1 + kPF < s_end) load(s + 1 + kPF, ra[jn], rb[jn]);
      }
      __syncthreads();
    });
  }
  // accumulator register r of a 32x32 tile: row 8 (r / 4) + 4 (lane / 32) +
  // r % 4, column lane % 32
  const int col = ct * kBN + ocol;
  if (col >= n_tot) return;
  float* dst = p.part + static_cast<int64_t>(split) * M * n_tot + col;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = mt * kBM + 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row < M) dst[static_cast<int64_t>(row) * n_tot] = acc[r];
  }
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

struct EpiArgs {
  const float* qpart;     // [sq, N, H * D]
  const float* kpart;     // [sk, N, D + H]
  int32_t sq, sk, N, H, D, R;
  const float* cos;       // [N, R / 2]
  const float* sin;
  const float* k_norm;    // [D]
  float eps;
  uint16_t* q_out;        // [N, H, D] bf16
  uint16_t* k_out;        // [N, D] bf16 or null
  float* w_out;           // [N, H]
  const int64_t* slots;   // [N] or null (no cache write)
  int64_t num_slots;
  void* k_cache;
  float* k_scale;
  int32_t cache_dtype;
  float inv_sqrt_d;       // fl32(D^-1/2), FP8 path
};

// RoPE of a head vector held in LDS (v[0 .. D), D == 128) by one wave:
// element e of the result goes to lane e % 64, slot e / 64; pair (j, j + R/2)
// turns by the angle of cos_row[j] / sin_row[j]
__device__ __forceinline__ void rope_lds(const float* v, int R, const float* __restrict__ cos_row,
                                         const float* __restrict__ sin_row, int lane,
                                         float (&out)[2]) {
  const int h = R / 2;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = lane + 64 * m;
    float x = v[e];
    if (e < R) {
      const int j = e < h ? e : e - h;
      const float c = cos_row[j], s = sin_row[j];
      x = e < h ? v[e] * c - v[e + h] * s : v[e] * c + v[e - h] * s;
    }
    out[m] = x;
  }
}

// sum_{sp < n} p[sp * stride] in split order; the loads go out eight at a
// time ahead of their adds (a loop of dependent rounds would wait for each)
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int64_t stride, int n) {
  float s = 0.0f;
  int sp = 0;
  for (; sp + 8 <= n; sp += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(sp + i) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  for (; sp < n; ++sp) s += p[sp * stride];
  return s;
}

__global__ __launch_bounds__(256) void k_proj_epilogue(EpiArgs a, int32_t q_waves) {
  __shared__ float sv[4][128];
  const int lane = threadIdx.x & 63;
  const int wl = threadIdx.x >> 6;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + wl;    // global wave
  const int h2 = a.R / 2;
  float* v = sv[wl];
  if (gw < q_waves) {
    // ---- q: token t, head h
    const int t = static_cast<int>(gw / a.H), h = static_cast<int>(gw % a.H);
    const int64_t ld = static_cast<int64_t>(a.H) * a.D;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int e = lane + 64 * m;
      v[e] = sum_splits(a.qpart + static_cast<int64_t>(t) * ld + h * a.D + e,
                        static_cast<int64_t>(a.N) * ld, a.sq);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float o[2];
    rope_lds(v, a.R, a.cos + static_cast<int64_t>(t) * h2, a.sin + static_cast<int64_t>(t) * h2,
             lane, o);
#pragma unroll
    for (int m = 0; m < 2; ++m)
      a.q_out[(static_cast<int64_t>(t) * a.H + h) * a.D + lane + 64 * m] = to_bf16(o[m]);
    return;
  }
  // ---- k and w: token t
  const int64_t t = gw - q_waves;
  if (t >= a.N) return;
  const int nc = a.D + a.H;
  float x[2];
  float ss = 0.0f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = lane + 64 * m;
    const float s = sum_splits(a.kpart + t * nc + e, static_cast<int64_t>(a.N) * nc, a.sk);
    x[m] = s;
    ss = fmaf(s, s, ss);
  }
  // head weights
  for (int e = lane; e < a.H; e += 64) {
    a.w_out[t * a.H + e] =
        sum_splits(a.kpart + t * nc + a.D + e, static_cast<int64_t>(a.N) * nc, a.sk);
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv_rms = 1.0f / sqrtf(ss / static_cast<float>(a.D) + a.eps);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = lane + 64 * m;
    v[e] = x[m] * inv_rms * a.k_norm[e];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float o[2];
  rope_lds(v, a.R, a.cos + t * h2, a.sin + t * h2, lane, o);
  uint16_t kb[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    kb[m] = to_bf16(o[m]);
    if (a.k_out) a.k_out[t * a.D + lane + 64 * m] = kb[m];
  }
  if (!a.slots) return;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  if (a.cache_dtype == DSA_BF16) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
      static_cast<uint16_t*>(a.k_cache)[slot * a.D + lane + 64 * m] = kb[m];
  } else {
    // the FP8 path: the bf16 key rotated and quantised as dsa_rotate_quantize does
    float r[2] = {bf16_bits_to_f32(kb[0]), bf16_bits_to_f32(kb[1])};
    wave_rotate_quantize<2>(r, a.D, a.inv_sqrt_d,
                            static_cast<uint8_t*>(a.k_cache) + slot * a.D, a.k_scale + slot);
  }
}

}  // namespace

// splits of each K range so that the grid reaches about two workgroups per
// CU, with at least 8 stages per split
void prologue_splits(int32_t N, const dsa_prologue_dims* d, int* sq, int* sk) {
  const int mt = (N + kBM - 1) / kBM;
  const int qt = mt * ((d->n_heads * d->head_dim + kBN - 1) / kBN);
  const int kt = mt * ((d->head_dim + d->n_heads + kBN - 1) / kBN);
  auto pick = [](int tiles, int K) {
    int s = tiles >= 512 ? 1 : (512 + tiles - 1) / tiles;
    const int most = std::max(1, K / kBK / 8);
    return std::min(s, most);
  };
  *sq = pick(qt, d->q_lora_rank);
  *sk = pick(kt, d->hidden_dim);
}

size_t prologue_part_floats(int32_t N, const dsa_prologue_dims* d) {
  int sq, sk;
  prologue_splits(N, d, &sq, &sk);
  return static_cast<size_t>(sq) * N * d->n_heads * d->head_dim +
         static_cast<size_t>(sk) * N * (d->head_dim + d->n_heads);
}

hipError_t launch_prologue(int32_t N, const dsa_prologue_dims* d, const void* hidden,
                           const void* qa, const float* cos, const float* sin,
                           const void* wq_b, const void* wk, const void* wp,
                           const float* k_norm, const int64_t* slots, int64_t num_slots,
                           void* k_cache, float* k_scale, int cache_dtype, void* q_out,
                           void* k_out, float* w_out, float* part, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  int sq, sk;
  prologue_splits(N, d, &sq, &sk);
  const int mt = (N + kBM - 1) / kBM;
  const int HD = d->n_heads * d->head_dim;
  GemmPart pq{static_cast<const uint16_t*>(qa), static_cast<const uint16_t*>(wq_b), nullptr,
              HD, 0, d->q_lora_rank, sq, (HD + kBN - 1) / kBN, part};
  GemmPart pk{static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(wk),
              static_cast<const uint16_t*>(wp), d->head_dim, d->n_heads, d->hidden_dim, sk,
              (d->head_dim + d->n_heads + kBN - 1) / kBN,
              part + static_cast<size_t>(sq) * N * HD};
  const int q_tiles = mt * pq.col_tiles * sq;
  const int k_tiles = mt * pk.col_tiles * sk;
  k_proj_gemm<<<q_tiles + k_tiles, 256, 0, stream>>>(pq, pk, N, q_tiles);
  EpiArgs e{pq.part, pk.part, sq, sk, N, d->n_heads, d->head_dim, d->rope_dim, cos, sin,
            k_norm, d->eps, static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(k_out),
            w_out, slots, num_slots, k_cache, k_scale, cache_dtype,
            static_cast<float>(1.0 / std::sqrt(static_cast<double>(d->head_dim)))};
  const int64_t waves = static_cast<int64_t>(N) * d->n_heads + N;
  k_proj_epilogue<<<static_cast<unsigned>((waves + 3) / 4), 256, 0, stream>>>(
      e, N * d->n_heads);
  return hipGetLastError();
}

}  // namespace dsa

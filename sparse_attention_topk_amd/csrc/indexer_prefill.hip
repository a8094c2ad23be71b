// Indexer score for prefill-shaped batches (page "GLM5 TensorCast 适配设计",
// section "DSA Indexer fused semantic op": cache scoring, head-weight mixing
// and head reduction; section "Performance model design", bucket "q-k index
// score MMA"):
//
//     score[t, s] = sum_h w[t, h] * max(q[t, h, :] . k[s, :], 0)
//
// for every causal key s <= pos(t), into the same fp32 [N, row_stride]
// matrix (and, for rows past the top-k's register reach, the same per-chunk
// score ranges) as the decode-shaped pass, so the top-k is shared.
//
// Decode-shaped blocks of one or two tokens read every key tile once per
// token block; a prefill has thousands of query tokens over the same keys,
// so here each key is reused across 16 tokens.  A workgroup holds 16
// consecutive query tokens of one request (all 32 heads: 128 KB of queries
// in LDS, laid out as MFMA operands) and one chunk of keys.  Each of its 4
// waves keeps 64 keys in registers at a time and contracts them with every
// head on v_mfma_f32_16x16x32_bf16, keys on M and the 16 tokens on N: the
// accumulator leaves a lane one token and four keys of each 16-key block,
// so the token's head weights are per-lane registers and the ReLU-weighted
// head sum never leaves the lane.  The keys come from L2 (a prefill's key
// cache is a few MB and every token block of the request reads it); the
// next 64 keys are loaded while the current ones are multiplied.
#include <utility>

#include "common.h"

namespace dsa {
namespace {

constexpr int kPT = 16;                   // query tokens per workgroup
constexpr int kPH = 32;                   // heads
constexpr int kPD = 128;                  // dims per head
constexpr int kPWaves = 8;               // two per SIMD
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPKeysW = 64;               // keys a wave holds per step (two 32-key blocks)
constexpr int kPStep = kPWaves * kPKeysW; // keys per workgroup step (256)
constexpr int kStreamStore = 2;           // cache-policy bits of the score stores: nt
constexpr int kBidSpan = 64 * 64;         // keys whose block ids one lane vector holds
typedef float f32x4p __attribute__((ext_vector_type(4)));

template <typename F, int... I>
__device__ __forceinline__ void pstatic_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void pstatic_for(F&& f) {
  pstatic_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int N>
__device__ __forceinline__ void pwait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// min / max over lanes l, l ^ 16, l ^ 32, l ^ 48 (one token's four key
// quads), NaN skipped
__device__ __forceinline__ void quad_rows_minmax(float& lo, float& hi) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(lo), false, false);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(hi), __float_as_uint(hi), false, false);
  lo = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  hi = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  a = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(lo), false, false);
  b = __builtin_amdgcn_permlane32_swap(__float_as_uint(hi), __float_as_uint(hi), false, false);
  lo = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  hi = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One workgroup per 16-token block, over every key up to the block's last
// position (the queries are loaded once), blocks with the most keys
// dispatched first: blockIdx = (qbpr - 1 - qb) * num_reqs + request.
__global__ __launch_bounds__(kPThreads, 1) void k_score_prefill(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ kc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ block_table,
    int32_t max_blocks, int32_t block_size, int64_t num_slots, int32_t max_seq_len,
    int32_t qbpr, int32_t num_reqs, int32_t chunk_keys, float* __restrict__ scores,
    int64_t row_stride, float2* __restrict__ crange, int32_t range_stride, int32_t win_lo,
    int32_t win_hi) {
  // Queries as MFMA B operands of v_mfma_f32_32x32x16_bf16 whose 32 columns
  // are the 16 tokens x one pair of heads: block (p, s) is 1 KB at
  // 1024 (8 p + s); lane l's 16 bytes at 16 l hold token l % 16, head
  // 2 p + (l / 16) % 2, dims 16 s + 8 (l / 32) .. + 7.
  __shared__ __align__(16) uint8_t qs[kPH / 2 * 8 * 1024];
  __shared__ float wsh[kPT][kPH + 1];   // head weights [token][head], rows padded
  __shared__ float2 rsh[kPWaves][kPT];  // per-wave score ranges (long rows)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tl = lane & 15;             // this lane's token
  const int hp = (lane >> 4) & 1;       // its head of each pair
  const int hf = lane >> 5;             // its half of the K-step and of the key rows

  const int b = blockIdx.x % num_reqs;
  const int qb = qbpr - 1 - blockIdx.x / num_reqs;
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_blocks;
  // lane i: block id of 64-key group i of the 4096 keys from kbase (a group
  // never spans two cache blocks: block_size is a multiple of 64)
  auto bids = [&](int32_t kbase) -> int32_t {
    const int32_t blk = (kbase + 64 * lane) / block_size;
    return blk < max_blocks ? bt_row[blk] : -1;
  };
  int32_t bid_cur = bids(0);
  const int32_t L = min(seq_lens[b], max_seq_len);
  const int32_t tbeg = cu_q[b];
  const int32_t qlen = min(cu_q[b + 1] - tbeg, L);
  const int32_t t0 = qb * kPT;
  if (t0 >= qlen) return;
  const int nt = min(kPT, qlen - t0);
  // the block's tokens inside the window: tl_lo .. tl_hi - 1 (the others
  // are computed with the block but not stored)
  const int32_t tw = tbeg + t0;
  const int tl_lo = max(tw, win_lo) - tw, tl_hi = min(tw + nt, win_hi) - tw;
  if (tl_lo >= tl_hi) return;
  const int32_t pos0 = L - qlen + t0;
  const int32_t key_end = pos0 + nt;          // keys 0 .. key_end - 1
  if (key_end <= 0) return;
  int32_t bid_next = bids(kBidSpan);

  // ---- queries into LDS (DMA, read once: non-temporal), weights beside.
  // Wave w fills blocks w + W m (head pair (w + W m) / 8, K-step (w + W m) % 8).
  {
    const int64_t tok = tbeg + t0 + min(tl, nt - 1);
    const uint16_t* src = q + tok * (kPH * kPD) + hp * kPD + 8 * hf;
    pstatic_for<kPH / 2 * 8 / kPWaves>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      const int id = wave + kPWaves * m;
      __builtin_amdgcn_global_load_lds(
          src + 2 * (id >> 3) * kPD + 16 * (id & 7),
          (__attribute__((address_space(3))) void*)(qs + 1024 * id), 16, 0, 2);
    });
#pragma unroll
    for (int r = 0; r < kPT * kPH / kPThreads; ++r) {
      const int e = threadIdx.x + kPThreads * r;
      const int tt = e / kPH, h = e % kPH;
      wsh[tt][h] = w[(tbeg + t0 + min(tt, nt - 1)) * static_cast<int64_t>(kPH) + h];
    }
  }
  pwait_vm<0>();
  lds_barrier();
  asm volatile("" : "+v"(bid_cur), "+v"(bid_next));

  // ---- steps of kPStep keys; this wave's 32 at kPStep j + 32 wave
  const int nsteps = (key_end + kPStep - 1) / kPStep;
  const int32_t my_pos = pos0 + tl;
  // the wave's first slot in step j, or -1 (no cache block, or past the
  // block's keys: scores 0)
  auto step_slot = [&](int j) -> int64_t {
    const int32_t k0 = kPStep * j + kPKeysW * wave;
    const int32_t bid = __builtin_amdgcn_readlane(bid_cur, (k0 % kBidSpan) / 64);
    const int64_t s0 = static_cast<int64_t>(bid) * block_size + k0 % block_size;
    return (k0 < key_end && bid >= 0 && k0 / block_size < max_blocks &&
            s0 + kPKeysW <= num_slots) ? s0 : -1;
  };
  // key operand of block kb, K-step s: key 32 kb + l % 32, dims 16 s + 8 (l / 32)
  bf16x8 kcur[2][8], knext[2][8];
  // Loads and stores are issued unconditionally (a step without a cache
  // block reads row 0 and zeroes its scores; masked score lanes store out
  // of the buffer's range, which the hardware drops), so the compiler's
  // wait counts stay exact and the next step's key loads stay in flight
  // through the whole head loop.
  auto load_keys = [&](int64_t s0, bf16x8 (&dst)[2][8]) {
    const uint16_t* base = kc + ((s0 < 0 ? 0 : s0) + (lane & 31)) * kPD + 8 * hf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 8; ++st)
        dst[kb][st] = *reinterpret_cast<const bf16x8*>(base + 32 * kb * kPD + 16 * st);
  };
  // score rows of the block's tokens tl_lo .. tl_hi - 1 as one buffer: byte
  // offset 4 (row_stride (tl - tl_lo) + key).  The scores stream out
  // non-temporally, so the key cache keeps its place in L2.
  const __amdgpu_buffer_rsrc_t srows = __builtin_amdgcn_make_buffer_rsrc(
      scores + (tw + tl_lo - win_lo) * row_stride, 0,
      static_cast<int>(static_cast<uint32_t>((tl_hi - tl_lo) * row_stride * 4)), 0x00020000);
  // The key registers are re-defined by an empty asm once their loads are
  // in (here and after each step's copy), so the wait counts inside the
  // head loop never tie it to the step's own stores or next loads.
  auto settle = [&]() {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(kcur[kb][st]));
  };
  const uint32_t qlane = 16u * static_cast<uint32_t>(lane);
  auto qop = [&](int pair, int st) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(qs + 1024 * (8 * pair + st) + qlane);
  };
  auto fold = [&](const f32x16& c, f32x16& a, float wh) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // ReLU on the bits: a negative float is a negative integer
      const float v = __int_as_float(max(__float_as_int(c[r]), 0));
      a[r] = fmaf(wh, v, a[r]);
    }
  };

  float rmin = INFINITY, rmax = -INFINITY;
  int64_t s_cur = step_slot(0);
  load_keys(s_cur, kcur);
  settle();
  constexpr int kStepsPerSpan = kBidSpan / kPStep;
  for (int j = 0; j < nsteps; ++j) {
    // the next span's block ids come in a span ahead of their use (issued
    // ahead of this step's key loads, so waiting for those covers them)
    if ((j + 1) % kStepsPerSpan == 0) {
      bid_cur = bid_next;
      bid_next = bids(kBidSpan * ((j + 1) / kStepsPerSpan + 1));
    }
    const int64_t s_next = j + 1 < nsteps ? step_slot(j + 1) : -1;
    load_keys(s_next, knext);

    // acc[kb][r]: token tl, key 32 kb + 8 (r / 4) + 4 hf + r % 4, summed
    // over this lane's head of every pair.  Pair p's 16 MFMAs (both key
    // blocks, each query operand read once for both) run while the VALU
    // folds pair p - 1's logits (ReLU, times the token's weight); two pairs
    // per iteration with the logit registers alternating.
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    f32x16 ca[2], cb[2] = {f32x16{}, f32x16{}};
    float wb = 0.0f;
    // query operands through a ring of 4 registers, each read 3 K-steps
    // ahead of its use (the next pair's first 3 during this pair's last 3)
    bf16x8 qr[4];
    qr[0] = qop(0, 0);
    qr[1] = qop(0, 1);
    qr[2] = qop(0, 2);
    auto chain = [&](int pair, f32x16 (&c)[2]) {
      const int nx = pair + 1 < kPH / 2 ? pair + 1 : pair;
      c[0] = f32x16{};
      c[1] = f32x16{};
      pstatic_for<8>([&](auto sc) {
        constexpr int st = decltype(sc)::value;
        constexpr int ahead = st + 3;
        qr[ahead % 4] = ahead < 8 ? qop(pair, ahead) : qop(nx, ahead - 8);
        c[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[0][st], qr[st % 4], c[0], 0, 0, 0);
        c[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[1][st], qr[st % 4], c[1], 0, 0, 0);
      });
    };
    auto fold2 = [&](const f32x16 (&c)[2], float wh) {
      fold(c[0], acc[0], wh);
      fold(c[1], acc[1], wh);
    };
    auto interleave = [&]() {   // per K-step: a query read, two MFMAs, the fold's VALU between
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
    };
    for (int pr = 0; pr < kPH / 2; pr += 2) {
      const float wa = wsh[tl][2 * pr + hp];
      chain(pr, ca);
      fold2(cb, wb);                // pair pr - 1 (zeros, weight 0, for pr = 0)
      interleave();
      wb = wsh[tl][2 * pr + 2 + hp];
      chain(pr + 1, cb);
      fold2(ca, wa);                // pair pr
      interleave();
    }
    fold2(cb, wb);                  // the last pair
    // the other head of each pair sits in lane l ^ 16
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[kb][r]),
                                                        __float_as_uint(acc[kb][r]), false, false);
        acc[kb][r] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
      }

    // ---- scores: lane (tl, hp, hf) stores row groups 2 hp and 2 hp + 1 of
    // both blocks (keys k0 + 32 kb + 8 g + 4 hf .. + 3)
    const int32_t k0 = kPStep * j + kPKeysW * wave;
    const bool has_row = s_cur >= 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        f32x4p v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = acc[kb][4 * jj + i], x1 = acc[kb][8 + 4 * jj + i];
          v[i] = has_row ? (hp ? x1 : x0) : 0.0f;
        }
        const int32_t key = k0 + 32 * kb + 8 * (2 * hp + jj) + 4 * hf;
        if (crange) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool causal = key + i <= my_pos;
            rmin = fminf(rmin, causal ? v[i] : INFINITY);
            rmax = fmaxf(rmax, causal ? v[i] : -INFINITY);
          }
        }
        const bool keep = tl >= tl_lo && tl < tl_hi && key <= my_pos;
        const int off = keep ? static_cast<int>(4 * ((tl - tl_lo) * row_stride + key)) : -1;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), srows, off, 0, kStreamStore);
      }
    s_cur = s_next;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 8; ++st) kcur[kb][st] = knext[kb][st];
    settle();
    // a chunk's score ranges once its last step is done (uniform: crange,
    // chunk_keys and the step count are the same for every wave)
    if (crange && ((j + 1) * kPStep % chunk_keys == 0 || j + 1 == nsteps)) {
      quad_rows_minmax(rmin, rmax);
      if (lane < 16) rsh[wave][tl] = make_float2(rmin, rmax);
      lds_barrier();
      // entry e of the chunk covers waves e W / 4 .. (e + 1) W / 4 - 1
      if (threadIdx.x < kRangeParts * kPT) {
        const int e = threadIdx.x / kPT, tt = threadIdx.x % kPT;
        const int chunk = j * kPStep / chunk_keys;
        float2 r = rsh[e * (kPWaves / kRangeParts)][tt];
#pragma unroll
        for (int i = 1; i < kPWaves / kRangeParts; ++i) {
          const float2 o = rsh[e * (kPWaves / kRangeParts) + i][tt];
          r = make_float2(fminf(r.x, o.x), fmaxf(r.y, o.y));
        }
        if (tt >= tl_lo && tt < tl_hi)
          crange[(tw + tt - win_lo) * static_cast<int64_t>(range_stride) + chunk * kRangeParts + e] = r;
      }
      lds_barrier();
      rmin = INFINITY;
      rmax = -INFINITY;
    }
  }
}

}  // namespace

bool prefill_score_ok(const IndexerArgs& a) {
  // (a block of 64 keys must exist to stand in for missing ones; the score
  // rows of a token block are addressed with 32-bit byte offsets)
  return a.q_dtype == DSA_BF16 && a.cache_dtype == DSA_BF16 && a.n_heads == kPH &&
         a.d_idx == kPD && a.b.block_size % 64 == 0 && a.b.max_q_len >= kPT &&
         a.b.num_slots >= 64 && a.row_stride <= (1 << 24);
}

hipError_t launch_score_prefill(IndexerArgs& a, hipStream_t stream) {
  const dsa_batch& b = a.b;
  const int qbpr = (b.max_q_len + kPT - 1) / kPT;
  const int64_t grid = static_cast<int64_t>(b.num_reqs) * qbpr;
  // score ranges (rows past the top-k's register reach) per 2048 keys
  const int chunk_keys = 2048;
  static_assert(2048 % kPStep == 0, "a chunk is whole steps");
  static_assert(kPWaves % kRangeParts == 0, "range entries cover whole waves");
  const int nchunks = (b.max_seq_len + chunk_keys - 1) / chunk_keys;
  a.chunk_keys = chunk_keys;
  a.range_stride = nchunks * kRangeParts;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  k_score_prefill<<<static_cast<unsigned>(grid), kPThreads, 0, stream>>>(
      static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k_cache),
      b.seq_lens, b.cu_q, b.block_table, b.max_blocks, b.block_size, b.num_slots,
      b.max_seq_len, qbpr, b.num_reqs, chunk_keys, a.scores, a.row_stride,
      a.chunk_range, a.range_stride, a.win_lo, a.win_hi);
  return hipGetLastError();
}

}  // namespace dsa

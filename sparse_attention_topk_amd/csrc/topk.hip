// Deterministic per-row top-k (page "GLM5 TensorCast 适配设计", section "DSA
// Indexer fused semantic op": top-k selection, output width topk_limit, or
// min(topk_limit, active length); page "GLM5 full-stack LoRA", section 1:
// the selection must not depend on an unspecified tie order).
//
// Row t holds the scores of query token t over positions 0..pos(t).  The
// kernel selects the n = min(topk, pos + 1) positions that come first in the
// order (score descending, position ascending) and writes them in ascending
// position order, then -1 up to topk.
//
// One 1024-thread workgroup per row.  Scores become order-preserving 32-bit
// keys (-0.0 is folded into +0.0 first, so the two zeros tie and fall to the
// position rule).  The selection finds the threshold key T = the topk-th
// largest key and the count c_gt of keys strictly above it; the output is
// then every position with key > T plus the first topk - c_gt positions with
// key == T, in position order.
//
// Rows of up to 32768 keys stay in registers (each wave holds 2048
// consecutive positions, loaded 1 KB per instruction):
//  1. load, value range [vmin, vmax];
//  2. histogram over 2048 value-linear bins of [vmin, vmax] (the bin map is
//     monotone in the value, so every key in a higher bin is strictly
//     larger), LDS atomics; a suffix scan finds the bin holding rank topk;
//  3. one pass marks the positions of every higher bin in an LDS bitmap and
//     collects the threshold bin's (score, position) pairs; when there are
//     few they are ranked directly and the top ones marked too, otherwise an
//     exact 4 x 8-bit radix select over the row finds the threshold score;
//  4. the bitmap is emitted in position order after one workgroup-wide
//     scan of its popcounts.
// Longer rows stream from memory in every pass (same steps, radix select
// over candidates or the row, compaction by waves over contiguous spans).
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kKpt = 32;                       // keys per thread, register path
constexpr int kRegCap = kThreads * kKpt;       // 32768
static_assert(kRegCap == kTopkRegCap, "the score pass knows the register path's reach");
constexpr int kCandCap = 4096;
constexpr int kRankCap = 256;                  // threshold-bin keys ranked directly

__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;                 // -0.0 -> +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// LDS of a workgroup of T threads (the register path holds up to 32 T
// positions: one bitmap word per thread)
template <int T>
struct ShrT {
  uint32_t hist[kBins];
  uint32_t cand[kCandCap];
  uint32_t bm_sel[T];     // register path: selected positions
  uint32_t bm_eq[T];      // register path: positions scoring == T
  uint32_t wave_a[T / 64];
  uint32_t wave_b[T / 64];
  float red_min[T / 64];
  float red_max[T / 64];
  uint32_t ncand;
  uint32_t sel_bin;       // threshold bin
  uint32_t above_bin;     // keys in bins above it
  uint32_t digit;         // radix step result
  uint32_t digit_above;
};
using Shared = ShrT<kThreads>;

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Suffix scan helper: for a 256-bin histogram find digit d with
// above(d) < r <= above(d) + h[d] (above = sum of higher bins).  Wave 0
// scans; results land in s.digit / s.digit_above.
template <typename S>
__device__ __forceinline__ void find_digit(S& s, uint32_t r) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // lane owns digits 255 - 4*lane - i, i = 0..3 (top-down)
    uint32_t c[4];
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = s.hist[255 - 4 * lane - i];
      tot += c[i];
    }
    uint32_t incl = wave_scan_incl(tot);
    uint32_t above = incl - tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (above < r && r <= above + c[i]) {
        s.digit = 255 - 4 * lane - i;
        s.digit_above = above;
      }
      above += c[i];
    }
  }
}

__device__ __forceinline__ int bin_of(float v, float vmin, float inv) {
  float t = (v - vmin) * inv;
  // NaN (0 * inf when the range underflows) compares false -> bin 0;
  // the map stays monotone in v
  int b = t > 0.0f ? (t >= static_cast<float>(kBins) ? kBins - 1 : static_cast<int>(t)) : 0;
  return b;
}

// Workgroup-wide min / max of per-thread values (every thread gets both).
template <int T>
__device__ __forceinline__ void range_reduce(ShrT<T>& s, float& vmin, float& vmax) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  wave_minmax(vmin, vmax);
  if (lane == 0) {
    s.red_min[wave] = vmin;
    s.red_max[wave] = vmax;
  }
  lds_barrier();
  vmin = s.red_min[0];
  vmax = s.red_max[0];
#pragma unroll
  for (int wv = 1; wv < T / 64; ++wv) {
    vmin = fminf(vmin, s.red_min[wv]);
    vmax = fmaxf(vmax, s.red_max[wv]);
  }
}

// Thread tid owns the kBins / T bins from 2047 - (kBins / T) tid down; the
// bin holding rank r (counted from the top) and the number of keys above it
// go to s.sel_bin / s.above_bin.  Ends with a barrier.
template <int T>
__device__ __forceinline__ void find_threshold_bin(ShrT<T>& s, uint32_t r) {
  constexpr int kB = kBins / T;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t h[kB];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    h[i] = s.hist[kBins - 1 - kB * tid - i];
    tot += h[i];
  }
  uint32_t incl = wave_scan_incl(tot);
  if (lane == 63) s.wave_a[wave] = incl;
  lds_barrier();
  // the totals of the waves before this one, one per lane, summed with the
  // DPP scan (instead of a serial run of LDS reads)
  const uint32_t base = __builtin_amdgcn_readlane(
      wave_scan_incl(lane < wave ? s.wave_a[lane] : 0u), 63);
  uint32_t above = base + incl - tot;        // above bin 2047 - kB tid
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    if (above < r && r <= above + h[i]) {
      s.sel_bin = kBins - 1 - kB * tid - i;
      s.above_bin = above;
    }
    above += h[i];
  }
  lds_barrier();
}

// This thread's share of the row's score range (then reduced over the
// workgroup).  With the score pass's per-chunk ranges (rng: the row's
// entries, kRangeParts per chunk of chunk_keys keys) the chunks holding
// positions 0 .. L - 1 are combined; without them own(lo, hi) scans the
// keys.  Both give the exact min / max of the row's scores, NaN skipped.
// pre: entry threadIdx.x of the row, loaded early (before L was known).
template <int T, typename F>
__device__ __forceinline__ void row_range(const float2* __restrict__ rng, int32_t chunk_keys,
                                          int L, float2 pre, F&& own, float& vmin,
                                          float& vmax) {
  if (rng) {
    const int nent = ((L - 1) / chunk_keys + 1) * kRangeParts;
    const bool mine = static_cast<int>(threadIdx.x) < nent;
    vmin = mine ? pre.x : INFINITY;
    vmax = mine ? pre.y : -INFINITY;
    for (int e = threadIdx.x + T; e < nent; e += T) {
      const float2 r = rng[e];
      vmin = fminf(vmin, r.x);
      vmax = fmaxf(vmax, r.y);
    }
  } else {
    own(vmin, vmax);
  }
}

// Ranks the n threshold-bin candidates (values cval, positions cpos, in
// LDS) by (score descending, position ascending) and marks the r best in
// bm_sel.  Wave w ranks candidates 64 w + lane against every candidate,
// taken one at a time with v_readlane from a register copy (lane k of round
// k0 holds candidate k0 + k), eight per step; lanes past the last candidate
// hold (-inf, INT_MAX), which outranks no candidate, so a step needs no bound
// test.  n <= 64 * kWaves.
__device__ __forceinline__ void rank_direct(const float* cval, const int32_t* cpos, int n,
                                            uint32_t r, uint32_t* bm_sel) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (64 * wave >= n) return;
  const int c = 64 * wave + lane;
  const float mv = c < n ? cval[c] : 0.0f;
  const int32_t mp = c < n ? cpos[c] : 0;
  uint32_t rank = 0;
  for (int k0 = 0; k0 < n; k0 += 64) {
    const float ov = k0 + lane < n ? cval[k0 + lane] : -INFINITY;
    const int32_t op = k0 + lane < n ? cpos[k0 + lane] : INT32_MAX;
    const int m = min(64, n - k0);
    for (int k = 0; k < m; k += 8) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const float v = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ov), k + kk));
        const int32_t pk = __builtin_amdgcn_readlane(op, k + kk);
        rank += (v > mv || (v == mv && pk < mp)) ? 1u : 0u;
      }
    }
  }
  if (c < n && rank < r) atomicOr(&bm_sel[mp >> 5], 1u << (mp & 31));
}

// ------------------------------------------------------------ register path
// Position of register key (j, e) of a lane: wave w covers positions
// 2048 w .. 2048 w + 2047, its load j (0..7) the 256 positions from
// 2048 w + 256 j, lane l the 4 positions from there + 4 l.  Every load
// instruction reads 1 KB contiguous.
__device__ __forceinline__ int reg_pos(int wave, int lane, int j, int e) {
  return 2048 * wave + 256 * j + 4 * lane + e;
}

// Loads the first min(row_stride, 32768) scores of the row (the positions
// any register-path row can hold); issued before the row's length is known.
// Rows are padded to a multiple of 64 floats, so a float4 never straddles
// the end of the allocation.  Positions past the row's stride (>= its
// length, so replaced by NaN before use) re-read the row's last float4:
// every load is unconditional, and the eight go out back to back (loads
// under a branch each were waited for before the next was issued).
__device__ __forceinline__ void load_row_regs(const float* __restrict__ src,
                                              int64_t row_stride, float (&f)[kKpt]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kKpt / 4; ++j) {
    const int p = reg_pos(wave, lane, j, 0);
    const int64_t pc = p < row_stride ? p : row_stride - 4;
    const float4 v = *reinterpret_cast<const float4*>(src + pc);
    f[4 * j + 0] = v.x;
    f[4 * j + 1] = v.y;
    f[4 * j + 2] = v.z;
    f[4 * j + 3] = v.w;
  }
}

// Register path.  Scores are compared as floats: -0.0 == +0.0 as the tie
// rule needs, and the float order is the key order for the finite scores
// this path handles.  Absent positions (>= L) hold NaN, which min / max
// skip, every comparison rejects and the bin map sends to bin 0; the bin
// counts below correct for them.  The selection is recorded in a bitmap of
// positions (bit p & 31 of word p >> 5), emitted in position order at the
// end.
template <int T>
__device__ __forceinline__ void select_row_regs(ShrT<T>& s, float (&f)[kKpt], int L,
                                                int topk, const float2* __restrict__ rng,
                                                int32_t chunk_keys, float2 pre,
                                                int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // register key (j, e) is position 2048 wave + 256 j + 4 lane + e: word
  // 64 wave + 8 j + lane / 8, bit 4 (lane % 8) + e
  auto word_of = [&](int j) { return 64 * wave + 8 * j + (lane >> 3); };
  auto bit_of = [&](int e) { return 1u << (4 * (lane & 7) + e); };

  // ---- 1. range
  if (reg_pos(wave, lane, kKpt / 4 - 1, 3) >= L) {
#pragma unroll
    for (int j = 0; j < kKpt / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (reg_pos(wave, lane, j, e) >= L) f[4 * j + e] = __builtin_nanf("");
  }
  // 256-position blocks (wave-uniform: load j of a wave) lying wholly past
  // the row take no part in the passes below; the row's last block holds
  // the only NaNs that do, and they land in bin 0
  auto live = [&](int j) { return 2048 * wave + 256 * j < L; };
  const uint32_t absent = static_cast<uint32_t>((L + 255) / 256 * 256 - L);
  float vmin, vmax;
  row_range<T>(rng, chunk_keys, L, pre, [&](float& lo, float& hi) {
    lo = f[0];
    hi = f[0];
#pragma unroll
    for (int j = 1; j < kKpt; ++j) {
      lo = fminf(lo, f[j]);
      hi = fmaxf(hi, f[j]);
    }
  }, vmin, vmax);
  for (int i = tid; i < kBins; i += T) s.hist[i] = 0;
  s.bm_sel[tid] = 0;
  s.bm_eq[tid] = 0;
  if (tid == 0) s.ncand = 0;
  range_reduce<T>(s, vmin, vmax);

  uint32_t need = 0;          // positions still to take among those == T
  if (!(vmax > vmin)) {
    // every score is equal: the first topk positions
    need = static_cast<uint32_t>(topk);
#pragma unroll
    for (int j = 0; j < kKpt / 4; ++j) {
      if (!live(j)) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (f[4 * j + e] == vmax) atomicOr(&s.bm_eq[word_of(j)], bit_of(e));
    }
  } else {
    // ---- 2. histogram and threshold bin: 2048 value-linear bins of [vmin,
    // vmax], monotone in f; NaN lands in bin 0.  The map needs a finite,
    // non-zero inv and an offset below 2^23: a range narrower than about
    // 6e-36 (scores all in the subnormal range) overflows inv, one wider than
    // the largest float underflows it, and one narrower than about 1e-3 of
    // the scores' magnitude overflows the offset.  Such rows
    // (workgroup-uniform) take the exact radix select instead.
    const float inv = 8190.0f / (vmax - vmin);   // 4 per bin: see the bin map below
    const float off = -vmin * inv;
    const bool linear = inv > 0.0f && inv < INFINITY && fabsf(off) < 8388608.0f;
    bool ranked = false;     // the selection is complete without the radix select
    if (linear) {
      // t = x inv + off lies in [-0.5, 8190.5] for every key (|off| < 2^23
      // rounds by at most 1/2), and the key's counter sits at byte offset
      // trunc(t) & ~3: bin floor(t / 4), 0 .. 2047, monotone in x.  The
      // conversion (v_cvt_u32_f32) sends negative t and NaN to 0.
#pragma unroll
      for (int j = 0; j < kKpt / 4; ++j) {
        if (!live(j)) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t u;
          asm("v_cvt_u32_f32 %0, %1" : "=v"(u) : "v"(fmaf(f[4 * j + e], inv, off)));
          atomicAdd(reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(s.hist) +
                                                (u & 0x1FFCu)), 1u);
        }
      }
      lds_barrier();
      if (tid == T - 1) s.hist[0] -= absent;
      lds_barrier();
      find_threshold_bin<T>(s, static_cast<uint32_t>(topk));
      const int sel = static_cast<int>(s.sel_bin);
      const uint32_t above_bin = s.above_bin;
      const uint32_t bin_count = s.hist[sel];
      const uint32_t r = static_cast<uint32_t>(topk) - above_bin;

      if (bin_count <= static_cast<uint32_t>(kRankCap)) {
        // ---- 3a. one pass: keys of higher bins are taken, keys of the
        // threshold bin become (score, position) candidates.  With t the same
        // fma as in the bin map, bin > sel <=> t >= 4 (sel + 1) (sel < 2047)
        // and bin >= sel <=> t >= 4 sel (sel >= 1); for sel == 0 every non-NaN
        // key has bin >= sel, which t >= -inf expresses.  NaN fails every
        // test.  Flags are collected branch-free; the rare candidates are
        // appended after the pass.
        const float thr_above = sel == kBins - 1 ? INFINITY : static_cast<float>(4 * (sel + 1));
        const float thr_in = sel == 0 ? -INFINITY : static_cast<float>(4 * sel);
        // same values; the compiler is kept from holding the histogram pass's
        // 32 products in registers until here
        float inv2 = inv, off2 = off;
        asm volatile("" : "+v"(inv2), "+v"(off2));
        uint32_t cand_bits = 0;          // bit 4 j + e
#pragma unroll
        for (int j = 0; j < kKpt / 4; ++j) {
          if (!live(j)) continue;
          uint32_t take = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = fmaf(f[4 * j + e], inv2, off2);
            take |= t >= thr_above ? bit_of(e) : 0u;
            cand_bits |= (t >= thr_in && t < thr_above) ? (1u << (4 * j + e)) : 0u;
          }
          if (take) atomicOr(&s.bm_sel[word_of(j)], take);
        }
        float* cval = reinterpret_cast<float*>(s.cand);
        int32_t* cpos = reinterpret_cast<int32_t*>(s.cand + kRankCap);
        // the threshold bin holds few keys: groups of 4 keys where no lane
        // has one are skipped with one wave-uniform test
#pragma unroll
        for (int j = 0; j < kKpt / 4; ++j) {
          const uint32_t cj = (cand_bits >> (4 * j)) & 0xFu;
          if (__ballot(cj != 0u) == 0) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((cj >> e) & 1u) {
              const uint32_t slot = atomicAdd(&s.ncand, 1u);
              cval[slot] = f[4 * j + e];
              cpos[slot] = reg_pos(wave, lane, j, e);
            }
          }
        }
        lds_barrier();
        // ---- rank the candidates; the top r join the selection
        rank_direct(cval, cpos, static_cast<int>(bin_count), r, s.bm_sel);
        ranked = true;
      }
    }
    if (!ranked) {
      // ---- 3b. exact radix select of rank topk over the row's keys gives
      // the threshold score T and the count above it (the bitmaps are still
      // empty: a row comes here from step 2 before anything was marked)
      const int tid2 = tid;
      uint32_t rr = static_cast<uint32_t>(topk);
      uint32_t prefix = 0, mask = 0, gt_extra = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        lds_barrier();
        for (int i = tid2; i < 256; i += T) s.hist[i] = 0;
        lds_barrier();
#pragma unroll
        for (int j = 0; j < kKpt; ++j) {
          if (!live(j / 4)) continue;
          const uint32_t kk = float_key(f[j]);
          if (f[j] == f[j] && (kk & mask) == prefix)
            atomicAdd(&s.hist[(kk >> shift) & 255u], 1u);
        }
        lds_barrier();
        find_digit(s, rr);
        lds_barrier();
        const uint32_t d = s.digit;
        const uint32_t da = s.digit_above;
        rr -= da;
        gt_extra += da;
        prefix |= d << shift;
        mask |= 255u << shift;
      }
      const float thr = key_float(prefix);
      need = static_cast<uint32_t>(topk) - gt_extra;   // >= 1
#pragma unroll
      for (int j = 0; j < kKpt / 4; ++j) {
        if (!live(j)) continue;
        uint32_t gtm = 0, eqm = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (f[4 * j + e] > thr) gtm |= bit_of(e);
          if (f[4 * j + e] == thr) eqm |= bit_of(e);
        }
        if (gtm) atomicOr(&s.bm_sel[word_of(j)], gtm);
        if (eqm) atomicOr(&s.bm_eq[word_of(j)], eqm);
      }
    }
  }
  lds_barrier();

  // ---- 4. emission in position order: thread tid owns word tid (positions
  // 32 tid .. 32 tid + 31).  Counts of taken bits and of == T bits (packed
  // 16:16, totals <= 32768) are scanned across the workgroup; the first
  // `need` positions scoring == T join the taken ones.
  uint32_t w_sel = s.bm_sel[tid];
  const uint32_t w_eq = s.bm_eq[tid];
  const uint32_t packed = (static_cast<uint32_t>(__popc(w_sel)) << 16) |
                          static_cast<uint32_t>(__popc(w_eq));
  uint32_t incl = wave_scan_incl(packed);
  if (lane == 63) s.wave_b[wave] = incl;
  lds_barrier();
  const uint32_t base = __builtin_amdgcn_readlane(
      wave_scan_incl(lane < wave ? s.wave_b[lane] : 0u), 63);
  const uint32_t excl = base + incl - packed;
  const uint32_t eq_before = excl & 0xFFFFu;
  uint32_t o = (excl >> 16) + min(eq_before, need);
  if (w_eq && eq_before < need) {
    // the lowest (need - eq_before) bits of w_eq
    uint32_t m = w_eq;
    for (uint32_t c = need - eq_before; m && c; --c) {
      const uint32_t low = m & (0u - m);
      w_sel |= low;
      m ^= low;
    }
  }
  // bounded by the row width: the bitmap holds exactly topk positions when
  // the steps above agree, and a disagreement must not write past the row
  while (w_sel && o < static_cast<uint32_t>(topk)) {
    const int b = __builtin_ctz(w_sel);
    out[o++] = 32 * tid + b;
    w_sel &= w_sel - 1;
  }
}

// ------------------------------------------------------------ streaming path
// Streams keys 0 .. L-1 of a score row through f(i, key): 16-byte loads,
// kV per thread per round, the next round's loads in flight while a round
// is processed (two register buffers, no copies between them).  Loads past
// the row's end are clamped to its last 16 bytes (rows are padded to 64
// floats) and the keys past L are skipped, so every round issues the same
// loads and the compiler's wait counts stay exact.
constexpr int kV = 4;
constexpr int kRound = kV * 4 * kThreads;   // keys per round
// Streams positions beg .. end - 1 of a row through one wave in blocks of
// 256: f(block start, lane's float4) for each block in order, lane l
// holding positions 4 l .. 4 l + 3.  kSub blocks per round, two register
// buffers, loads clamped into the row like for_each_key's.
constexpr int kSub = 4;
template <typename F>
__device__ __forceinline__ void wave_blocks(const float* __restrict__ src, int beg,
                                            int end, int last4, F&& f) {
  const int lane = threadIdx.x & 63;
  auto load = [&](int base, float4 (&v)[kSub]) {
#pragma unroll
    for (int j = 0; j < kSub; ++j)
      v[j] = *reinterpret_cast<const float4*>(src + min(base + 256 * j + 4 * lane, last4));
  };
  auto run = [&](int base, const float4 (&v)[kSub]) {
#pragma unroll
    for (int j = 0; j < kSub; ++j)
      if (base + 256 * j < end) f(base + 256 * j, v[j]);
  };
  float4 A[kSub], B[kSub];
  load(beg, A);
  for (int base = beg; base < end; base += 2 * 256 * kSub) {
    load(base + 256 * kSub, B);
    run(base, A);
    load(base + 2 * 256 * kSub, A);
    run(base + 256 * kSub, B);
  }
}

template <typename F>
__device__ __forceinline__ void for_each_key(const float* __restrict__ src,
                                             int L, F&& f) {
  const int tid = threadIdx.x;
  const int last4 = ((L + 3) & ~3) - 4;
  auto load = [&](int base, float4 (&v)[kV]) {
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int i = min(base + 4 * (j * kThreads + tid), last4);
      v[j] = *reinterpret_cast<const float4*>(src + i);
    }
  };
  auto process = [&](int base, const float4 (&v)[kV]) {
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int i = base + 4 * (j * kThreads + tid);
      const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (i + q < L) f(i + q, float_key(e[q]));
    }
  };
  float4 A[kV], B[kV];
  load(0, A);
  for (int base = 0; base < L; base += 2 * kRound) {
    load(base + kRound, B);
    process(base, A);
    load(base + 2 * kRound, A);
    process(base + kRound, B);
  }
}

__device__ __forceinline__ void select_row_stream(Shared& s, const float* __restrict__ src, int L,
                                  int topk, const float2* __restrict__ rng,
                                  int32_t chunk_keys, float2 pre,
                                  int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- 1. range (a pass over the row only without the score pass's)
  float vmin, vmax;
  row_range<kThreads>(rng, chunk_keys, L, pre, [&](float& lo, float& hi) {
    lo = INFINITY;
    hi = -INFINITY;
    for_each_key(src, L, [&](int, uint32_t k) {
      const float f = key_float(k);
      lo = fminf(lo, f);
      hi = fmaxf(hi, f);
    });
  }, vmin, vmax);
  for (int i = tid; i < kBins; i += kThreads) s.hist[i] = 0;
  if (tid == 0) s.ncand = 0;
  range_reduce(s, vmin, vmax);

  uint32_t T;
  uint32_t c_gt;
  if (!(vmax > vmin)) {
    T = float_key(vmax);
    c_gt = 0;
  } else {
    // ---- 2. histogram and threshold bin
    const float inv = static_cast<float>(kBins) / (vmax - vmin);
    for_each_key(src, L, [&](int, uint32_t k) {
      atomicAdd(&s.hist[bin_of(key_float(k), vmin, inv)], 1u);
    });
    lds_barrier();
    find_threshold_bin(s, static_cast<uint32_t>(topk));
    const int sel = static_cast<int>(s.sel_bin);
    const uint32_t above_bin = s.above_bin;
    const uint32_t bin_count = s.hist[sel];
    const bool use_cand = bin_count <= kCandCap;
    if (use_cand) {
      for_each_key(src, L, [&](int, uint32_t k) {
        if (bin_of(key_float(k), vmin, inv) == sel) {
          const uint32_t slot = atomicAdd(&s.ncand, 1u);
          if (slot < kCandCap) s.cand[slot] = k;
        }
      });
    }
    lds_barrier();
    // ---- 3. exact radix select of rank r among the set
    uint32_t r = use_cand ? static_cast<uint32_t>(topk) - above_bin
                          : static_cast<uint32_t>(topk);
    const int n_set = use_cand ? min(static_cast<int>(s.ncand), kCandCap) : L;
    uint32_t prefix = 0, mask = 0, gt_extra = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kThreads) s.hist[i] = 0;
      lds_barrier();
      if (use_cand) {
        for (int i = tid; i < n_set; i += kThreads) {
          const uint32_t k = s.cand[i];
          if ((k & mask) == prefix) atomicAdd(&s.hist[(k >> shift) & 255u], 1u);
        }
      } else {
        for_each_key(src, L, [&](int, uint32_t k) {
          if ((k & mask) == prefix) atomicAdd(&s.hist[(k >> shift) & 255u], 1u);
        });
      }
      lds_barrier();
      find_digit(s, r);
      lds_barrier();
      const uint32_t d = s.digit;
      const uint32_t da = s.digit_above;
      r -= da;
      gt_extra += da;
      prefix |= d << shift;
      mask |= 255u << shift;
      lds_barrier();
    }
    T = prefix;
    c_gt = (use_cand ? above_bin : 0u) + gt_extra;
  }

  // ---- 4. ordered compaction over contiguous spans per wave: a wave
  // reads its span in blocks of 256 positions, lane l holding positions
  // 4 l .. 4 l + 3 of a block (16-byte loads, kSub blocks per round, the
  // next round in flight)
  const uint32_t need = static_cast<uint32_t>(topk) - c_gt;   // >= 1
  const int span = ((L + kWaves - 1) / kWaves + 255) & ~255;
  const int beg = wave * span;
  const int end = min(L, beg + span);
  const int last4 = ((L + 3) & ~3) - 4;
  // inclusive prefix sum over the wave's lanes
  auto wave_incl = [](uint32_t v) { return wave_scan_incl(v); };
  uint32_t n_gt = 0, n_eq = 0;
  wave_blocks(src, beg, end, last4, [&](int blk, const float4& v) {
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = blk + 4 * lane + q;
      const uint32_t k = float_key(e[q]);
      n_gt += (i < end && k > T) ? 1u : 0u;
      n_eq += (i < end && k == T) ? 1u : 0u;
    }
  });
  n_gt = __builtin_amdgcn_readlane(wave_scan_incl(n_gt), 63);   // the wave's totals
  n_eq = __builtin_amdgcn_readlane(wave_scan_incl(n_eq), 63);
  if (lane == 0) {
    s.wave_a[wave] = n_gt;
    s.wave_b[wave] = n_eq;
  }
  lds_barrier();
  uint32_t gt_before = 0, eq_run = 0;
  for (int wv = 0; wv < wave; ++wv) {
    gt_before += s.wave_a[wv];
    eq_run += s.wave_b[wv];
  }
  // positions taken before the next block, and == T positions seen
  uint32_t out_run = gt_before + min(eq_run, need);
  wave_blocks(src, beg, end, last4, [&](int blk, const float4& v) {
    const float e[4] = {v.x, v.y, v.z, v.w};
    bool gt[4], eq[4];
    uint32_t c_eq = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = blk + 4 * lane + q;
      const uint32_t k = float_key(e[q]);
      gt[q] = i < end && k > T;
      eq[q] = i < end && k == T;
      c_eq += eq[q] ? 1u : 0u;
    }
    // == T positions before this lane's, in position order
    const uint32_t eq_incl = wave_incl(c_eq);
    uint32_t eq_rank = eq_run + eq_incl - c_eq;
    bool take[4];
    uint32_t c_take = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      take[q] = gt[q] || (eq[q] && eq_rank < need);
      eq_rank += eq[q] ? 1u : 0u;
      c_take += take[q] ? 1u : 0u;
    }
    const uint32_t take_incl = wave_incl(c_take);
    uint32_t o = out_run + take_incl - c_take;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (take[q] && o < static_cast<uint32_t>(topk)) out[o] = blk + 4 * lane + q;
      o += take[q] ? 1u : 0u;
    }
    out_run += __builtin_amdgcn_readlane(take_incl, 63);
    eq_run += __builtin_amdgcn_readlane(eq_incl, 63);
  });
}

// ------------------------------------------------------------ long rows
// Rows of kRegCap < L <= kLongCap keys take the register path's steps with
// the keys streamed from memory, two passes over the row (the histogram,
// then one classification pass that marks every key of a higher bin in a
// position bitmap and collects the threshold bin's keys as candidates); the
// bitmaps live in dynamic LDS.  A row whose range the bin map cannot express,
// or whose threshold bin holds more than kCandCap keys, is left to the exact
// multi-pass path above (returns false before writing anything).
constexpr int kLongCap = 262144;

// Positions i .. i + 3 of a row (i a multiple of 4, i < L) as a float4,
// f(i, v), streamed kV float4 per thread per round with the next round in
// flight; entries at positions >= L hold clamped data the caller ignores.
template <typename F>
__device__ __forceinline__ void for_each_quad(const float* __restrict__ src, int L, F&& f) {
  const int tid = threadIdx.x;
  const int last4 = ((L + 3) & ~3) - 4;
  auto load = [&](int base, float4 (&v)[kV]) {
#pragma unroll
    for (int j = 0; j < kV; ++j)
      v[j] = *reinterpret_cast<const float4*>(src + min(base + 4 * (j * kThreads + tid), last4));
  };
  auto process = [&](int base, const float4 (&v)[kV]) {
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int i = base + 4 * (j * kThreads + tid);
      if (i < L) f(i, v[j]);
    }
  };
  float4 A[kV], B[kV];
  load(0, A);
  for (int base = 0; base < L; base += 2 * kRound) {
    load(base + kRound, B);
    process(base, A);
    load(base + 2 * kRound, A);
    process(base + kRound, B);
  }
}

// Emits, in position order, every position set in bm_sel plus the first
// `need` positions set in bm_eq (nwords words each, at most topk outputs).
// Thread tid owns the run of words wpt tid .. wpt tid + wpt - 1; the counts
// before each thread's run come from workgroup-wide scans.
__device__ __forceinline__ void emit_bitmaps(Shared& s, const uint32_t* bm_sel,
                                             const uint32_t* bm_eq, int nwords,
                                             uint32_t need, int topk,
                                             int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wpt = (nwords + kThreads - 1) / kThreads;
  const int w0 = min(nwords, wpt * tid);
  const int w1 = min(nwords, w0 + wpt);
  uint32_t c_sel = 0, c_eq = 0;
  for (int w = w0; w < w1; ++w) {
    c_sel += __popc(bm_sel[w]);
    c_eq += __popc(bm_eq[w]);
  }
  const uint32_t is = wave_scan_incl(c_sel);
  const uint32_t ie = wave_scan_incl(c_eq);
  if (lane == 63) {
    s.wave_a[wave] = is;
    s.wave_b[wave] = ie;
  }
  lds_barrier();
  const uint32_t bs = __builtin_amdgcn_readlane(
      wave_scan_incl(lane < wave ? s.wave_a[lane] : 0u), 63);
  const uint32_t be = __builtin_amdgcn_readlane(
      wave_scan_incl(lane < wave ? s.wave_b[lane] : 0u), 63);
  uint32_t eq_before = be + ie - c_eq;
  uint32_t o = bs + is - c_sel + min(eq_before, need);
  for (int w = w0; w < w1 && o < static_cast<uint32_t>(topk); ++w) {
    uint32_t ws = bm_sel[w];
    const uint32_t we = bm_eq[w];
    if (we && eq_before < need) {
      uint32_t m = we;              // its lowest (need - eq_before) bits join
      for (uint32_t c = need - eq_before; m && c; --c) {
        const uint32_t low = m & (0u - m);
        ws |= low;
        m ^= low;
      }
    }
    eq_before += __popc(we);
    while (ws && o < static_cast<uint32_t>(topk)) {
      out[o++] = 32 * w + __builtin_ctz(ws);
      ws &= ws - 1;
    }
  }
}

// dyn: [bm_sel: words_cap][bm_eq: words_cap][candidate positions: kCandCap]
__device__ __noinline__ bool select_row_long(Shared& s, uint32_t* __restrict__ dyn,
                                             int32_t words_cap, const float* __restrict__ src,
                                             int L, int topk, const float2* __restrict__ rng,
                                             int32_t chunk_keys, float2 pre,
                                             int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const int nwords = (L + 31) / 32;
  uint32_t* bm_sel = dyn;
  uint32_t* bm_eq = dyn + words_cap;
  int32_t* cpos = reinterpret_cast<int32_t*>(dyn + 2 * words_cap);
  float* cval = reinterpret_cast<float*>(s.cand);

  // ---- 1. range
  float vmin, vmax;
  row_range<kThreads>(rng, chunk_keys, L, pre, [&](float& lo, float& hi) {
    lo = INFINITY;
    hi = -INFINITY;
    for_each_quad(src, L, [&](int i, const float4& v) {
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool in = i + q < L;
        lo = fminf(lo, in ? e[q] : INFINITY);
        hi = fmaxf(hi, in ? e[q] : -INFINITY);
      }
    });
  }, vmin, vmax);
  for (int i = tid; i < kBins; i += kThreads) s.hist[i] = 0;
  for (int w = tid; w < nwords; w += kThreads) {
    bm_sel[w] = 0;
    bm_eq[w] = 0;
  }
  if (tid == 0) s.ncand = 0;
  range_reduce(s, vmin, vmax);
  if (!(vmax > vmin)) {
    // every score is equal: the first topk positions (L > topk here)
    for (int j = tid; j < topk; j += kThreads) out[j] = j;
    return true;
  }
  const float inv = static_cast<float>(kBins) / (vmax - vmin);
  const float off = -vmin * inv;
  if (!(inv > 0.0f && inv < INFINITY && off > -INFINITY && off < INFINITY)) return false;
  // bin = trunc(clamp(x inv + off, 0, 2047)), monotone in x (see the
  // register path)
  auto bin = [&](float x) {
    return static_cast<int>(fminf(fmaxf(fmaf(x, inv, off), 0.0f), kBins - 1.0f));
  };

  // ---- 2. histogram pass and threshold bin
  for_each_quad(src, L, [&](int i, const float4& v) {
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (i + q < L) atomicAdd(&s.hist[bin(e[q])], 1u);
  });
  lds_barrier();
  find_threshold_bin(s, static_cast<uint32_t>(topk));
  const int sel = static_cast<int>(s.sel_bin);
  const uint32_t above_bin = s.above_bin;
  const uint32_t r = static_cast<uint32_t>(topk) - above_bin;
  if (s.hist[sel] > static_cast<uint32_t>(kCandCap)) return false;

  // ---- 3. classification pass: a higher bin marks the position, the
  // threshold bin appends a candidate (same tests as the register path)
  const float thr_above = sel == kBins - 1 ? INFINITY : static_cast<float>(sel + 1);
  const float thr_in = sel == 0 ? -INFINITY : static_cast<float>(sel);
  for_each_quad(src, L, [&](int i, const float4& v) {
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t take = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float t = fmaf(e[q], inv, off);
      const bool in = i + q < L;
      take |= (in && t >= thr_above) ? (1u << q) : 0u;
      if (in && t >= thr_in && t < thr_above) {
        const uint32_t slot = atomicAdd(&s.ncand, 1u);
        if (slot < static_cast<uint32_t>(kCandCap)) {   // always: same test as the bins
          cval[slot] = e[q];
          cpos[slot] = i + q;
        }
      }
    }
    if (take) atomicOr(&bm_sel[i >> 5], take << (i & 31));
  });
  lds_barrier();

  // ---- 4. the r best candidates (as many as the threshold bin counted)
  const uint32_t n = min(s.ncand, static_cast<uint32_t>(kCandCap));
  uint32_t need = 0;
  if (n <= static_cast<uint32_t>(kRankCap)) {
    rank_direct(cval, cpos, static_cast<int>(n), r, bm_sel);
  } else {
    // exact radix select of rank r among the candidates' keys
    uint32_t rr = r, prefix = 0, mask = 0, gt_extra = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kThreads) s.hist[i] = 0;
      lds_barrier();
      for (int i = tid; i < static_cast<int>(n); i += kThreads) {
        const uint32_t k = float_key(cval[i]);
        if ((k & mask) == prefix) atomicAdd(&s.hist[(k >> shift) & 255u], 1u);
      }
      lds_barrier();
      find_digit(s, rr);
      lds_barrier();
      rr -= s.digit_above;
      gt_extra += s.digit_above;
      prefix |= s.digit << shift;
      mask |= 255u << shift;
      lds_barrier();
    }
    need = r - gt_extra;
    for (int i = tid; i < static_cast<int>(n); i += kThreads) {
      const uint32_t k = float_key(cval[i]);
      const int32_t p = cpos[i];
      if (k > prefix) atomicOr(&bm_sel[p >> 5], 1u << (p & 31));
      if (k == prefix) atomicOr(&bm_eq[p >> 5], 1u << (p & 31));
    }
  }
  lds_barrier();

  // ---- 5. emission in position order
  emit_bitmaps(s, bm_sel, bm_eq, nwords, need, topk, out);
  return true;
}

__global__ __launch_bounds__(kThreads, 1) void k_topk(
    const float* __restrict__ scores, int64_t row_stride,
    const float2* __restrict__ crange, int32_t range_stride, int32_t chunk_keys,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
    int32_t B, int32_t max_seq_len, int32_t topk, int32_t* __restrict__ out,
    int32_t words_cap, int32_t t_lo) {
  __shared__ Shared s;
  extern __shared__ uint32_t dyn[];   // long rows: words_cap > 0
  // query token t_lo + blockIdx.x; its score and range rows are row blockIdx.x
  const int t = t_lo + static_cast<int>(blockIdx.x);
  const float* src = scores + static_cast<int64_t>(blockIdx.x) * row_stride;
  // The request lookup (the largest b with cu_q[b] <= t, counted with a
  // ballot over 64 entries per load) reads its first entries before the
  // row is requested: loads return in order, so behind the row's 128 KB it
  // would wait for all of it before the length could even be asked for.
  const int lane = threadIdx.x & 63;
  const int32_t c0 = cu_q[lane < B ? lane : B];      // cu_q has B + 1 entries
  asm volatile("" ::: "memory");
  // the row's first 32768 scores are requested before its length is known
  float f[kKpt];
  load_row_regs(src, row_stride, f);
  // and the first kThreads of its score-range entries
  const float2* rng = crange ? crange + static_cast<int64_t>(blockIdx.x) * range_stride : nullptr;
  float2 pre = make_float2(INFINITY, -INFINITY);
  if (rng && static_cast<int>(threadIdx.x) < range_stride) pre = rng[threadIdx.x];
  int n = __popcll(__ballot(lane < B && c0 <= t));
  for (int b0 = 64; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const int32_t c = cu_q[bb < B ? bb : B];
    n += __popcll(__ballot(bb < B && c <= t));
  }
  const int b = n - 1 < 0 ? 0 : (n - 1 >= B ? B - 1 : n - 1);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  const int L = pos + 1;
  int32_t* orow = out + static_cast<int64_t>(t) * topk;
  if (L <= topk) {
    for (int j = threadIdx.x; j < topk; j += kThreads) orow[j] = j < L ? j : -1;
    return;
  }
  if (L <= kRegCap) {
    select_row_regs<kThreads>(s, f, L, topk, rng, chunk_keys, pre, orow);
    return;
  }
  if (L <= 32 * words_cap &&
      select_row_long(s, dyn, words_cap, src, L, topk, rng, chunk_keys, pre, orow))
    return;
  lds_barrier();
  select_row_stream(s, src, L, topk, rng, chunk_keys, pre, orow);
}

// Launches whose rows all fit 32 T positions (prefill-length rows): the
// register path on a workgroup of T threads, several rows per CU.
template <int T>
__global__ __launch_bounds__(T, 2048 / T) void k_topk_reg(
    const float* __restrict__ scores, int64_t row_stride,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
    int32_t B, int32_t max_seq_len, int32_t topk, int32_t* __restrict__ out, int32_t t_lo) {
  __shared__ ShrT<T> s;
  const int t = t_lo + static_cast<int>(blockIdx.x);
  const float* src = scores + static_cast<int64_t>(blockIdx.x) * row_stride;
  const int lane = threadIdx.x & 63;
  const int32_t c0 = cu_q[lane < B ? lane : B];      // cu_q has B + 1 entries
  asm volatile("" ::: "memory");
  float f[kKpt];
  load_row_regs(src, row_stride, f);
  int n = __popcll(__ballot(lane < B && c0 <= t));
  for (int b0 = 64; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const int32_t c = cu_q[bb < B ? bb : B];
    n += __popcll(__ballot(bb < B && c <= t));
  }
  const int b = n - 1 < 0 ? 0 : (n - 1 >= B ? B - 1 : n - 1);
  const int32_t pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
  const int L = pos + 1;
  int32_t* orow = out + static_cast<int64_t>(t) * topk;
  if (L <= topk) {
    for (int j = threadIdx.x; j < topk; j += T) orow[j] = j < L ? j : -1;
    return;
  }
  select_row_regs<T>(s, f, L, topk, nullptr, 0, make_float2(INFINITY, -INFINITY), orow);
}

}  // namespace

hipError_t launch_topk(const IndexerArgs& a, hipStream_t stream) {
  const int rows = a.win_hi - a.win_lo;      // the window's query tokens
  if (rows <= 0) return hipSuccess;
  if (a.b.max_seq_len <= 32 * 256) {
    k_topk_reg<256><<<rows, 256, 0, stream>>>(
        a.scores, a.row_stride, a.b.seq_lens, a.b.cu_q, a.b.num_reqs, a.b.max_seq_len,
        a.topk, a.topk_idx, a.win_lo);
    return hipGetLastError();
  }
  if (a.b.max_seq_len <= 32 * 512) {
    k_topk_reg<512><<<rows, 512, 0, stream>>>(
        a.scores, a.row_stride, a.b.seq_lens, a.b.cu_q, a.b.num_reqs, a.b.max_seq_len,
        a.topk, a.topk_idx, a.win_lo);
    return hipGetLastError();
  }
  // long rows' bitmaps and candidate positions in dynamic LDS, sized for the
  // longest row this launch can hold (none when every row fits registers)
  const int32_t words_cap = a.b.max_seq_len > kRegCap
                                ? (min(a.b.max_seq_len, kLongCap) + 31) / 32 : 0;
  const size_t dyn_bytes = words_cap > 0 ? (2 * static_cast<size_t>(words_cap) + kCandCap) * 4 : 0;
  k_topk<<<rows, kThreads, dyn_bytes, stream>>>(
      a.scores, a.row_stride, a.chunk_range, a.range_stride, a.chunk_keys, a.b.seq_lens,
      a.b.cu_q, a.b.num_reqs, a.b.max_seq_len, a.topk, a.topk_idx, words_cap, a.win_lo);
  return hipGetLastError();
}

}  // namespace dsa

// Indexer key-cache write (page "GLM5 TensorCast 适配设计", section "DSA
// Indexer fused semantic op": the op writes new keys into the paged indexer
// cache addressed by slot_mapping; on the FP8 path it writes e4m3 key codes
// plus a per-token scale; section "KV cache dtype and parallel-linear
// boundary fix": the cache dtype follows attention quantisation).
//
// One 64-lane wave per token.  F32/BF16: a straight copy.  FP8: the wave
// reduces amax = max |k| exactly, scale = fl32(amax / 448) (1 if amax == 0),
// each lane divides its elements by scale (IEEE fp32 division) and rounds to
// e4m3fn with round-to-nearest-even and saturation at +-448.
#include <cmath>
#include <type_traits>

#include "common.h"

namespace dsa {
namespace {

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p,
                                                       int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_copy_keys(const T* __restrict__ k_new,
                                                   int n_new, int d,
                                                   const int64_t* __restrict__ slots,
                                                   int64_t num_slots,
                                                   T* __restrict__ cache) {
  int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (tok >= n_new) return;
  int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  for (int e = lane; e < d; e += kWave)
    cache[slot * d + e] = k_new[static_cast<int64_t>(tok) * d + e];
}

template <typename T>
__global__ __launch_bounds__(256) void k_quant_keys(const T* __restrict__ k_new,
                                                    int n_new, int d,
                                                    const int64_t* __restrict__ slots,
                                                    int64_t num_slots,
                                                    uint8_t* __restrict__ cache,
                                                    float* __restrict__ scale) {
  int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (tok >= n_new) return;
  int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t src = static_cast<int64_t>(tok) * d;
  float amax = 0.0f;
  for (int e = lane; e < d; e += kWave)
    amax = fmaxf(amax, fabsf(load_as_f32(k_new, src + e)));
  for (int off = 32; off > 0; off >>= 1)
    amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  for (int e = lane; e < d; e += kWave) {
    float v = load_as_f32(k_new, src + e) / s;
    cache[slot * d + e] = static_cast<uint8_t>(f32_to_e4m3(v));
  }
  if (lane == 0) scale[slot] = s;
}

// Activation rotation and quantisation (page "GLM5 TensorCast 适配设计",
// section "DSA Indexer fused semantic op": the FP8 path's rotate_activation
// and activation quantisation; section "Performance model design", bucket
// 5).  One 64-lane wave per row of d = 32 .. 256 (a power of two) elements:
// element l + 64 m sits in lane l, slot m (EPL = max(1, d / 64) slots).  The
// orthonormal Hadamard transform runs as butterflies over h = 1, 2, ...,
// d / 2 in that order, (a, b) -> (a + b, a - b) for the pair (i, i + h) in
// each block of 2 h, rounded to fp32 at every stage, then one multiply by
// inv_sqrt_d = fl32(d^-1/2); pairs of h < 64 meet across lanes l and l ^ h,
// pairs of h >= 64 inside a lane.  The rotated row is then quantised like a
// key: amax, scale = fl32(amax / 448) (1 if amax == 0), e4m3(v / scale).
template <typename T, int EPL>
__global__ __launch_bounds__(256) void k_rotate_quantize(
    const T* __restrict__ x, int64_t n_rows, int d, float inv_sqrt_d,
    const int64_t* __restrict__ row_slots, int64_t num_out,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int64_t dst = row_slots ? row_slots[row] : row;
  if (dst < 0 || dst >= num_out) return;
  float v[EPL];
#pragma unroll
  for (int m = 0; m < EPL; ++m)
    v[m] = lane < d ? load_as_f32(x, row * d + lane + 64 * m) : 0.0f;
  wave_rotate_quantize<EPL>(v, d, inv_sqrt_d, codes + dst * d, scales + dst);
}

// Decodes e4m3 codes, 8 per thread, with the conversion and byte packing
// the indexer's FP8 path uses (n is a multiple of 8).
__global__ void k_fp8_decode_check(const uint8_t* __restrict__ codes,
                                   float* __restrict__ out, int n) {
  int i = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= n) return;
  const u32x2 raw = *reinterpret_cast<const u32x2*>(codes + i);
  bf16x8 v = fp8x8_to_bf16x8(raw[0], raw[1]);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[i + e] = static_cast<float>(v[e]);
}

}  // namespace

hipError_t launch_cache_write(const void* k_new, int k_dtype, int n_new,
                              int d, const int64_t* slots, int64_t num_slots,
                              void* k_cache, float* k_scale, int cache_dtype,
                              hipStream_t stream) {
  if (n_new == 0) return hipSuccess;
  dim3 grid((n_new + 3) / 4), block(256);
  if (cache_dtype == DSA_FP8_E4M3) {
    if (k_dtype == DSA_BF16)
      k_quant_keys<uint16_t><<<grid, block, 0, stream>>>(
          static_cast<const uint16_t*>(k_new), n_new, d, slots, num_slots,
          static_cast<uint8_t*>(k_cache), k_scale);
    else
      k_quant_keys<float><<<grid, block, 0, stream>>>(
          static_cast<const float*>(k_new), n_new, d, slots, num_slots,
          static_cast<uint8_t*>(k_cache), k_scale);
  } else if (cache_dtype == DSA_BF16) {
    k_copy_keys<uint16_t><<<grid, block, 0, stream>>>(
        static_cast<const uint16_t*>(k_new), n_new, d, slots, num_slots,
        static_cast<uint16_t*>(k_cache));
  } else {
    k_copy_keys<float><<<grid, block, 0, stream>>>(
        static_cast<const float*>(k_new), n_new, d, slots, num_slots,
        static_cast<float*>(k_cache));
  }
  return hipGetLastError();
}

hipError_t launch_rotate_quantize(const void* x, int x_dtype, int64_t n_rows, int d,
                                  const int64_t* row_slots, int64_t num_out, uint8_t* codes,
                                  float* scales, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  // fl32(d^-1/2): the double square root and reciprocal are correctly
  // rounded, then rounded once to float
  const float inv = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  const dim3 grid(static_cast<unsigned>((n_rows + 3) / 4)), block(256);
  auto go = [&](auto tag, auto epl) {
    using T = decltype(tag);
    constexpr int E = decltype(epl)::value;
    k_rotate_quantize<T, E><<<grid, block, 0, stream>>>(
        static_cast<const T*>(x), n_rows, d, inv, row_slots, num_out, codes, scales);
  };
  const int epl = d <= 64 ? 1 : d / 64;
  if (x_dtype == DSA_BF16) {
    if (epl == 1) go(uint16_t{}, std::integral_constant<int, 1>{});
    else if (epl == 2) go(uint16_t{}, std::integral_constant<int, 2>{});
    else go(uint16_t{}, std::integral_constant<int, 4>{});
  } else {
    if (epl == 1) go(float{}, std::integral_constant<int, 1>{});
    else if (epl == 2) go(float{}, std::integral_constant<int, 2>{});
    else go(float{}, std::integral_constant<int, 4>{});
  }
  return hipGetLastError();
}

hipError_t launch_fp8_decode_check(const uint8_t* codes, float* out, int n,
                                   hipStream_t stream) {
  if (n == 0) return hipSuccess;
  k_fp8_decode_check<<<(n / 8 + 255) / 256, 256, 0, stream>>>(codes, out, n);
  return hipGetLastError();
}

}  // namespace dsa

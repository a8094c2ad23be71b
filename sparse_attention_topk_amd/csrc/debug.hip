// Checked build (libdsa_debug.so, compiled with -DDSA_DEBUG).
//
// The release library trusts the device-resident metadata (kernels clamp or
// skip out-of-range values so that no memory outside the given buffers is
// touched, with unspecified results).  The checked build runs, on the
// caller's stream around every call:
//   * before: a validation of the metadata the call reads against the
//     host-side bounds of dsa_batch (seq_lens, cu_q, the block-table entries
//     in use, slot_mapping, the attention's index rows), and canary fills of
//     the outputs and of the workspace;
//   * after: a check that no output element still holds its canary and that
//     every indexer row is a valid selection (min(topk, pos + 1) ascending
//     positions in [0, pos], then -1).
// Violations set bits of a per-device fault word (DSA_FAULT_*), which
// dsa_debug_faults reads.  The kernels here are compiled into both
// libraries; only the checked build launches them.
#include "common.h"

namespace dsa {
namespace {

__device__ uint32_t g_faults;            // per device: DSA_FAULT_* bits since the last clear

__device__ __forceinline__ void raise_fault(uint32_t bits) {
  if (bits) atomicOr(&g_faults, bits);
}

// one workgroup per request
__global__ __launch_bounds__(256) void k_check_batch(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q, int32_t B,
    int32_t n_tokens, int32_t max_q_len, int32_t max_seq_len,
    const int32_t* __restrict__ block_table, int32_t max_blocks, int32_t block_size,
    int64_t num_slots) {
  const int b = blockIdx.x;
  const int32_t L = seq_lens[b];
  const int32_t c0 = cu_q[b], c1 = cu_q[b + 1];
  if (threadIdx.x == 0) {
    uint32_t f = 0;
    if (L < 0 || L > max_seq_len) f |= DSA_FAULT_SEQ_LENS;
    if (c1 < c0 || c1 - c0 > max_q_len || c1 - c0 > L) f |= DSA_FAULT_CU_Q;
    if (b == 0 && c0 != 0) f |= DSA_FAULT_CU_Q;
    if (b == B - 1 && c1 != n_tokens) f |= DSA_FAULT_CU_Q;
    raise_fault(f);
  }
  // the blocks that hold positions 0 .. L - 1
  const int32_t Lc = min(max(L, 0), max_seq_len);
  const int32_t nb = (Lc + block_size - 1) / block_size;
  if (threadIdx.x == 0 && nb > max_blocks) raise_fault(DSA_FAULT_BLOCK_TABLE);
  for (int i = threadIdx.x; i < min(nb, max_blocks); i += blockDim.x) {
    const int32_t bid = block_table[static_cast<int64_t>(b) * max_blocks + i];
    const int32_t used = min(block_size, Lc - i * block_size);
    if (bid < 0 || static_cast<int64_t>(bid) * block_size + used > num_slots)
      raise_fault(DSA_FAULT_BLOCK_TABLE);
  }
}

__global__ __launch_bounds__(256) void k_check_slots(const int64_t* __restrict__ slots,
                                                     int32_t n, int64_t num_slots) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t s = slots[i];
  if (s != -1 && (s < 0 || s >= num_slots)) raise_fault(DSA_FAULT_SLOT_MAPPING);
}

// position of query token t (request by binary search over cu_q)
__device__ __forceinline__ int32_t checked_pos(const int32_t* seq_lens, const int32_t* cu_q,
                                               int32_t B, int32_t t, int32_t max_seq_len) {
  const int b = request_of(cu_q, B, t);
  return query_pos(seq_lens, cu_q, b, t, max_seq_len);
}

// attention input rows: every entry -1 or in [0, pos]; one wave per row
__global__ __launch_bounds__(64) void k_check_topk_in(
    const int32_t* __restrict__ idx, int32_t topk, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, int32_t B, int32_t max_seq_len) {
  const int t = blockIdx.x;
  const int32_t pos = checked_pos(seq_lens, cu_q, B, t, max_seq_len);
  const int32_t* row = idx + static_cast<int64_t>(t) * topk;
  uint32_t f = 0;
  for (int j = threadIdx.x; j < topk; j += 64) {
    const int32_t v = row[j];
    if (v != -1 && (v < 0 || v > pos)) f |= DSA_FAULT_TOPK_INPUT;
  }
  raise_fault(f);
}

// indexer output rows: min(topk, pos + 1) ascending positions in [0, pos],
// then -1; the canary anywhere means an element was not written
__global__ __launch_bounds__(64) void k_check_topk_out(
    const int32_t* __restrict__ idx, int32_t topk, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, int32_t B, int32_t max_seq_len, int32_t canary) {
  const int t = blockIdx.x;
  const int32_t pos = checked_pos(seq_lens, cu_q, B, t, max_seq_len);
  const int32_t n = min(topk, max(pos + 1, 0));
  const int32_t* row = idx + static_cast<int64_t>(t) * topk;
  uint32_t f = 0;
  for (int j = threadIdx.x; j < topk; j += 64) {
    const int32_t v = row[j];
    if (v == canary) {
      f |= DSA_FAULT_UNWRITTEN;
    } else if (j < n) {
      if (v < 0 || v > pos || (j > 0 && row[j - 1] >= v)) f |= DSA_FAULT_TOPK_OUTPUT;
    } else if (v != -1) {
      f |= DSA_FAULT_TOPK_OUTPUT;
    }
  }
  raise_fault(f);
}

__global__ __launch_bounds__(256) void k_fill(uint8_t* __restrict__ p, int64_t bytes,
                                              uint32_t pattern) {
  const int64_t words = bytes / 4;
  uint32_t* w = reinterpret_cast<uint32_t*>(p);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < words; i += gridDim.x * 256ll)
    w[i] = pattern;
  const int64_t tail = blockIdx.x * 256ll + threadIdx.x;
  if (tail < bytes - 4 * words) p[4 * words + tail] = static_cast<uint8_t>(pattern >> (8 * tail));
}

template <typename T>
__global__ __launch_bounds__(256) void k_check_unwritten(const T* __restrict__ p, int64_t n,
                                                         T canary) {
  uint32_t f = 0;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += gridDim.x * 256ll)
    if (p[i] == canary) f = DSA_FAULT_UNWRITTEN;
  raise_fault(f);
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return static_cast<unsigned>(g < 1 ? 1 : (g > 1024 ? 1024 : g));
}

}  // namespace

hipError_t debug_check_batch(const dsa_batch& b, hipStream_t stream) {
  if (b.num_reqs <= 0) return hipSuccess;
  k_check_batch<<<b.num_reqs, 256, 0, stream>>>(b.seq_lens, b.cu_q, b.num_reqs, b.num_q_tokens,
                                                b.max_q_len, b.max_seq_len, b.block_table,
                                                b.max_blocks, b.block_size, b.num_slots);
  return hipGetLastError();
}

hipError_t debug_check_slots(const int64_t* slots, int32_t n, int64_t num_slots,
                             hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_check_slots<<<(n + 255) / 256, 256, 0, stream>>>(slots, n, num_slots);
  return hipGetLastError();
}

hipError_t debug_check_topk_in(const dsa_batch& b, const int32_t* idx, int32_t topk,
                               hipStream_t stream) {
  if (b.num_q_tokens <= 0 || topk <= 0) return hipSuccess;
  k_check_topk_in<<<b.num_q_tokens, 64, 0, stream>>>(idx, topk, b.seq_lens, b.cu_q,
                                                     b.num_reqs, b.max_seq_len);
  return hipGetLastError();
}

hipError_t debug_check_topk_out(const dsa_batch& b, const int32_t* idx, int32_t topk,
                                hipStream_t stream) {
  if (b.num_q_tokens <= 0 || topk <= 0) return hipSuccess;
  k_check_topk_out<<<b.num_q_tokens, 64, 0, stream>>>(idx, topk, b.seq_lens, b.cu_q,
                                                      b.num_reqs, b.max_seq_len, kCanaryIdx);
  return hipGetLastError();
}

hipError_t debug_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t stream) {
  if (!p || bytes == 0) return hipSuccess;
  k_fill<<<grid_for(static_cast<int64_t>(bytes / 4)), 256, 0, stream>>>(
      static_cast<uint8_t*>(p), static_cast<int64_t>(bytes), pattern);
  return hipGetLastError();
}

hipError_t debug_check_unwritten(const void* p, size_t n, int elem_bytes, uint32_t canary,
                                 hipStream_t stream) {
  if (!p || n == 0) return hipSuccess;
  const int64_t m = static_cast<int64_t>(n);
  if (elem_bytes == 2)
    k_check_unwritten<uint16_t><<<grid_for(m), 256, 0, stream>>>(
        static_cast<const uint16_t*>(p), m, static_cast<uint16_t>(canary));
  else
    k_check_unwritten<uint32_t><<<grid_for(m), 256, 0, stream>>>(
        static_cast<const uint32_t*>(p), m, canary);
  return hipGetLastError();
}

hipError_t debug_faults(uint32_t* faults, bool clear) {
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(faults, HIP_SYMBOL(g_faults), sizeof(uint32_t));
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_faults), &zero, sizeof(uint32_t));
}

}  // namespace dsa

// Debug check of a step's index arrays. The attention and cache-write calls
// never validate index contents (an out-of-range block id or slot is the
// caller's error there, and costs nothing to not check); this call counts
// such entries on the device, for callers that want to know before a step
// runs: context lengths outside [0, max_context_len], block ids that a call
// would read (the first ceil(L / 16) entries of a row) outside the pool, and
// slots past the pool (a negative slot means "no write" and is allowed).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mvk.h"

namespace {

constexpr int kCheckThreads = 1024;
constexpr int64_t kBlockTokens = 16;

// One workgroup: the arrays are walked in thread-strided loops, the counts
// meet in LDS, and thread t < 3 writes count t (so no zeroing is needed and
// the result does not depend on timing).
__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(
    long long* __restrict__ counts, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
    int32_t max_context_len, const int32_t* __restrict__ slot_mapping, int32_t num_slots,
    int32_t num_blocks) {
  __shared__ unsigned long long total[3];
  const int t = threadIdx.x;
  if (t < 3) total[t] = 0;
  __syncthreads();
  unsigned long long bad_len = 0, bad_block = 0, bad_slot = 0;
  for (int s = t; s < num_seqs; s += kCheckThreads) {
    const int32_t len = context_lens[s];
    bad_len += (len < 0 || len > max_context_len) ? 1u : 0u;
  }
  // the tokens a call reads: the length clamped to [0, max_context_len] and
  // to the row's width
  const int64_t cap = min((int64_t)max_context_len, (int64_t)max_blocks_per_seq * kBlockTokens);
  const int64_t entries = (int64_t)num_seqs * max_blocks_per_seq;
  for (int64_t e = t; e < entries; e += kCheckThreads) {
    const int64_t s = e / max_blocks_per_seq, j = e - s * max_blocks_per_seq;
    const int64_t len = min(max((int64_t)context_lens[s], (int64_t)0), cap);
    if (j * kBlockTokens < len) {
      const int32_t b = block_tables[e];
      bad_block += (b < 0 || b >= num_blocks) ? 1u : 0u;
    }
  }
  const int64_t pool_slots = (int64_t)num_blocks * kBlockTokens;
  for (int i = t; i < num_slots; i += kCheckThreads)
    bad_slot += (int64_t)slot_mapping[i] >= pool_slots ? 1u : 0u;
  if (bad_len) atomicAdd(&total[0], bad_len);
  if (bad_block) atomicAdd(&total[1], bad_block);
  if (bad_slot) atomicAdd(&total[2], bad_slot);
  __syncthreads();
  if (t < 3) counts[t] = (long long)total[t];
}

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

}  // namespace

extern "C" int32_t mvk_check_indices(int64_t* counts, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     const int32_t* slot_mapping, int32_t num_slots,
                                     int32_t num_blocks, void* stream) {
  if (!counts || !aligned(counts, 8)) return MVK_ERR_INVALID_ARGUMENT;
  if (num_seqs < 0 || num_slots < 0 || max_context_len < 0 || num_blocks <= 0)
    return MVK_ERR_INVALID_ARGUMENT;
  if (num_seqs > 0 && (!block_tables || !context_lens || max_blocks_per_seq <= 0 ||
                       !aligned(block_tables, 4) || !aligned(context_lens, 4)))
    return MVK_ERR_INVALID_ARGUMENT;
  if (num_slots > 0 && (!slot_mapping || !aligned(slot_mapping, 4))) return MVK_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(check_indices_kernel, dim3(1), dim3(kCheckThreads), 0, (hipStream_t)stream,
                     (long long*)counts, block_tables, context_lens, num_seqs,
                     num_seqs > 0 ? max_blocks_per_seq : 1, max_context_len, slot_mapping,
                     num_slots, num_blocks);
  return hipGetLastError() == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

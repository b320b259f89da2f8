// Paged cache write: scatter new K/V token rows into their physical slots.
//
// A slot is a flat row index of the pool: the pool [num_blocks, 16, Hkv, D]
// is num_blocks*16 rows of Hkv*D elements, so slot = block*16 + offset
// addresses row `slot` directly (16-token blocks: mini-vllm write-up, section
// "2. 分页KV缓存（PagedAttention）"; K/V pools with block before head:
// "关键工程决策", item 3). The copy moves raw 16-byte vectors, so the pools
// receive the source bits unchanged.
#include "device_common.h"
#include "launch.h"

namespace mvk {

// One thread per 16-byte vector of a row; consecutive threads cover
// consecutive bytes of one row, so both the read of key/value and the write
// into the slot are fully coalesced. K and V are handled by the same thread.
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int32_t num_tokens,
    int32_t row_vecs, int64_t num_slots) {
  const int64_t total = (int64_t)num_tokens * row_vecs;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int32_t t = (int32_t)(i / row_vecs);
    const int32_t c = (int32_t)(i - (int64_t)t * row_vecs);
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;  // padding / out of range: no write
    const int64_t dst = (int64_t)slot * row_vecs + c;
    const uint4 kv = key[i];
    const uint4 vv = value[i];
    k_cache[dst] = kv;
    v_cache[dst] = vv;
  }
}

hipError_t launch_cache_write(const void* key, const void* value, void* k_cache, void* v_cache,
                              const int32_t* slot_mapping, int32_t num_tokens, int32_t row_vecs,
                              int64_t num_slots, hipStream_t stream) {
  const int64_t total = (int64_t)num_tokens * row_vecs;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 waves per CU
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const uint4*)key, (const uint4*)value, (uint4*)k_cache, (uint4*)v_cache,
                     slot_mapping, num_tokens, row_vecs, num_slots);
  return hipGetLastError();
}

}  // namespace mvk

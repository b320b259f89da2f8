// C ABI entry points: host-side validation, partition planning and dispatch.
// Nothing here touches the GPU before every argument has been checked.
#include <math.h>
#include <stdint.h>

#include "../../include/mvk.h"
#include "launch.h"

namespace {

constexpr int32_t kBlock = 16;
constexpr int32_t kMaxPartition = 65536;
constexpr int32_t kMaxGridYZ = 65535;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int32_t round_up16(int64_t x) { return (int32_t)((x + kBlock - 1) / kBlock * kBlock); }

// Partition length when the caller leaves the choice to the library. Short
// contexts run in one pass (no workspace, no merge kernel); longer ones are cut
// into 512-token partitions, which keeps every workgroup's wave busy with 8
// blocks while giving long sequences enough workgroups to fill 256 CUs.
int32_t default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  (void)num_seqs;
  (void)num_kv_heads;
  if (max_context_len <= 512) return max_context_len <= 0 ? kBlock : round_up16(max_context_len);
  return 512;
}

struct Plan {
  int32_t partition_tokens;
  int32_t num_parts;
  size_t workspace_bytes;
};

int32_t check_sizes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_context_len, int32_t partition_tokens, Plan* plan) {
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_kv_heads > kMaxGridYZ || max_context_len < 0)
    return MVK_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return MVK_ERR_INVALID_ARGUMENT;
  if (partition_tokens != 0 &&
      (partition_tokens < kBlock || partition_tokens > kMaxPartition || partition_tokens % kBlock))
    return MVK_ERR_INVALID_ARGUMENT;
  if (!mvk::decode_supported(head_dim, num_q_heads / num_kv_heads)) return MVK_ERR_UNSUPPORTED;
  const int32_t p = partition_tokens ? partition_tokens
                                     : default_partition(num_seqs, num_kv_heads, max_context_len);
  int64_t parts = ((int64_t)max_context_len + p - 1) / p;
  if (parts < 1) parts = 1;
  plan->partition_tokens = p;
  plan->num_parts = (int32_t)parts;
  plan->workspace_bytes =
      parts > 1 ? (size_t)num_seqs * num_q_heads * (size_t)parts * (size_t)(head_dim + 2) * 4u : 0;
  return MVK_OK;
}

}  // namespace

extern "C" {

int32_t mvk_abi_version(void) { return MVK_ABI_VERSION; }

const char* mvk_status_string(int32_t status) {
  switch (status) {
    case MVK_OK: return "ok";
    case MVK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MVK_ERR_UNSUPPORTED: return "unsupported configuration";
    case MVK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MVK_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int32_t mvk_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                              const int32_t* slot_mapping, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t dtype, void* stream) {
  if (dtype != MVK_F16 && dtype != MVK_BF16) return MVK_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return MVK_ERR_INVALID_ARGUMENT;
  if (block_size != kBlock || (head_dim != 64 && head_dim != 128)) return MVK_ERR_UNSUPPORTED;
  if ((int64_t)num_blocks * kBlock > INT32_MAX) return MVK_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return MVK_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(slot_mapping))
    return MVK_ERR_INVALID_ARGUMENT;
  if (k_cache == v_cache) return MVK_ERR_INVALID_ARGUMENT;
  const int64_t row_vecs = (int64_t)num_kv_heads * head_dim * 2 / 16;
  if (row_vecs > INT32_MAX) return MVK_ERR_INVALID_ARGUMENT;
  hipError_t err = mvk::launch_cache_write(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                           (int32_t)row_vecs, (int64_t)num_blocks * kBlock,
                                           (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

int32_t mvk_paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_context_len, int32_t partition_tokens,
                                           size_t* workspace_bytes,
                                           int32_t* chosen_partition_tokens) {
  if (!workspace_bytes) return MVK_ERR_INVALID_ARGUMENT;
  Plan plan;
  const int32_t st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                 partition_tokens, &plan);
  if (st != MVK_OK) return st;
  *workspace_bytes = plan.workspace_bytes;
  if (chosen_partition_tokens) *chosen_partition_tokens = plan.partition_tokens;
  return MVK_OK;
}

int32_t mvk_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   float scale, int32_t dtype, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != MVK_F16 && dtype != MVK_BF16) return MVK_ERR_INVALID_ARGUMENT;
  if (block_size != kBlock) return MVK_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || !isfinite(scale))
    return MVK_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
    return MVK_ERR_INVALID_ARGUMENT;
  Plan plan;
  const int32_t st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                 partition_tokens, &plan);
  if (st != MVK_OK) return st;
  if (num_seqs == 0) return MVK_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens))
    return MVK_ERR_INVALID_ARGUMENT;
  if (out == q || out == k_cache || out == v_cache) return MVK_ERR_INVALID_ARGUMENT;
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return MVK_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return MVK_ERR_INVALID_ARGUMENT;
  }

  mvk::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t n_state = (size_t)num_seqs * num_q_heads * (size_t)plan.num_parts;
  a.ws_ml = plan.workspace_bytes ? (float*)workspace : nullptr;
  a.ws_o = plan.workspace_bytes ? (float*)workspace + n_state * 2 : nullptr;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.partition_tokens = plan.partition_tokens;
  a.num_parts = plan.num_parts;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  a.dtype = dtype;
  hipError_t err = mvk::launch_paged_decode(a, (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

}  // extern "C"

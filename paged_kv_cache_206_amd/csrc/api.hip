// C ABI entry points: host-side validation, partition planning and dispatch.
// Nothing here touches the GPU before every argument has been checked.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "mvk.h"
#include "launch.h"

namespace {

constexpr int32_t kBlock = 16;
constexpr int32_t kMinWaves = 4;
// a wave prefetches its table entries into one VGPR: at most 64 blocks per
// wave, so a partition holds at most 64 * 16 * (waves per workgroup) tokens
constexpr int32_t kMaxPartition = 64 * 16 * kMinWaves;
constexpr int32_t kMaxGridYZ = 65535;
// A multi-partition batch whose dense (partition, KV head, sequence) grid
// would exceed this many workgroups runs in work-list mode: most of such a
// grid would be partitions past short contexts, each costing a dispatch and a
// load only to exit.
constexpr int64_t kGridLimit = 16384;
// Shortest longest-context (tokens) for which a single-pass grid is
// dispatched longest sequence first.
constexpr int32_t kMinOrderedContext = 1024;
// Workgroups (over all KV heads) that walk the work list.
constexpr int64_t kListWorkgroups = 4096;
// Any workspace starts with this many bytes of partition counters, one int32
// per (sequence, KV head), and nothing else is ever stored there: every call
// returns the counters it used to zero, so a workspace zero-filled once stays
// valid for calls of any shape. Batches with more (sequence, KV head) pairs
// than the region holds merge their partitions with a separate kernel.
constexpr size_t kCounterRegion = 65536;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int32_t round_up16(int64_t x) { return (int32_t)((x + kBlock - 1) / kBlock * kBlock); }

// Partition length when the caller leaves the choice to the library: the
// longest of 4096 / 2048 / 1024 / 512 / 256 tokens whose (sequence, KV head,
// partition) grid still has at least kMinWorkgroups workgroups (4 per CU),
// capped by the longest context; 256 tokens when none has. Long partitions
// mean fewer partial states to merge; the floor keeps all CUs streaming.
// (Measured on MI355X: 256-token single pass for 60 x 8 short contexts,
// 2048 single pass for 256 x 4 contexts of <= 2048, 4096 for 32 x 8 x 32768
// and for skewed batches.)
constexpr int64_t kMinWorkgroups = 1024;

int32_t default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  if (max_context_len <= 0) return kBlock;
  const int32_t cap = round_up16(max_context_len);
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  for (int32_t p = kMaxPartition; p >= 256; p /= 2) {
    const int64_t parts = ((int64_t)max_context_len + p - 1) / p;
    if (units * parts >= kMinWorkgroups) return p < cap ? p : cap;
  }
  return cap < 256 ? cap : 256;
}

// Partition length (tokens) the library chooses for batches that run in
// work-list mode.
constexpr int32_t kWorkListPartition = 3072;

// Waves per workgroup: 8 for the longest partitions (more bytes in flight per
// workgroup), else 4.
int32_t default_waves(int32_t partition_tokens) {
  return partition_tokens >= kWorkListPartition ? 8 : 4;
}

struct Plan {
  int32_t partition_tokens;
  int32_t num_parts;
  int32_t waves;
  int32_t longest_first;
  int32_t detect_shared;
  bool work_list;
  int32_t list_workgroups;
  size_t counter_bytes;    // the counter region at the start of the workspace
  bool use_counters;       // merge partitions in the partition kernel
  size_t partial_bytes;    // partial (m, l, o) states, after the counters
  size_t workspace_bytes;  // counters + partial states + work list
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
  int32_t p = partition_tokens ? partition_tokens
                               : default_partition(num_seqs, num_kv_heads, max_context_len);
  if (!partition_tokens && p == kMaxPartition) {
    // A batch whose dense grid at the longest partitions would run in
    // work-list mode (a few very long sequences among many short ones) takes
    // 3072-token partitions, with the same 8 waves. Measured on MI355X, 512
    // sequences up to 131072 tokens: 4096-token partitions 362.6 us, 3072
    // 351.5 us, 2048 374 us (the longest sequence's items are then short
    // enough to balance against the rest, and not so many that their merge
    // and per-item round trips dominate).
    const int64_t parts0 = ((int64_t)max_context_len + p - 1) / p;
    if (parts0 > 1 && (int64_t)num_seqs * parts0 * num_kv_heads > kGridLimit) p = kWorkListPartition;
  }
  // a function of the partition length alone, so that a caller passing the
  // length the library chose gets the same plan
  const int32_t waves = default_waves(p);
  int64_t parts = ((int64_t)max_context_len + p - 1) / p;
  if (parts < 1) parts = 1;
  if (parts > kMaxGridYZ) return MVK_ERR_INVALID_ARGUMENT;  // grid z
  plan->partition_tokens = p;
  plan->num_parts = (int32_t)parts;
  plan->waves = waves;
  plan->partial_bytes =
      parts > 1 ? (size_t)num_seqs * num_q_heads * (size_t)parts * (size_t)(head_dim + 2) * 4u : 0;
  const int64_t dense = (int64_t)num_seqs * parts * num_kv_heads;
  plan->work_list = parts > 1 && dense > kGridLimit;
  // One partition per sequence, a batch the decode kernel can rank in every
  // workgroup (at most 256 sequences), and contexts long enough that the
  // ranking's extra memory round trip at the start of every workgroup
  // (about 1.5 us) is repaid: dispatch longest first. Measured on MI355X:
  // 256 x 4 items of 512-2048 tokens 71.5 -> 68.6 us; 60 x 8 items of
  // 64-256 tokens 11.2 -> 12.1 us (so short contexts keep batch order).
  // Dense grids of split sequences (long contexts, where a shared prefix is
  // many blocks) look for blocks shared with a neighbouring sequence and
  // keep those cached; the lookup costs more than it saves on short contexts
  // and on work lists (measured with it on everywhere: Llama-7B shape 534.6
  // -> 526 us, the Qwen3 shape 11.24 -> 11.89 us, the skewed batch 351 ->
  // 363 us).
  plan->detect_shared = parts > 1 && !plan->work_list;
  plan->longest_first = parts == 1 && num_seqs <= mvk::kMaxOrderedSeqs &&
                        max_context_len >= kMinOrderedContext;
  if (!plan->work_list && dense > INT32_MAX) return MVK_ERR_INVALID_ARGUMENT;
  const int64_t per_head = (kListWorkgroups + num_kv_heads - 1) / num_kv_heads;
  plan->list_workgroups = (int32_t)(per_head < num_seqs * parts ? per_head : num_seqs * parts);
  // Where partitions merge. In the partition kernel (the last partition of a
  // (sequence, KV head) to finish merges) saves the merge kernel's launch but
  // makes every partition wait for its partial state to reach memory; that
  // pays off when few sequences are split, i.e. in work-list mode, and costs
  // more than it saves when every sequence is split (dense grids).
  const bool merge_in_kernel = plan->work_list;
  plan->counter_bytes = parts > 1 ? kCounterRegion : 0;
  plan->use_counters = parts > 1 && merge_in_kernel &&
                       (size_t)num_seqs * num_kv_heads * 4u <= kCounterRegion;
  plan->workspace_bytes = plan->counter_bytes + plan->partial_bytes +
                          (plan->work_list
                               ? (size_t)(1 + num_kv_heads + 2 * num_seqs * parts) * 4u
                               : 0);
  return MVK_OK;
}

// ------------------------------------------------ multi-query (several new tokens)

// Query tokens per sequence that one call accepts: verification of K draft
// tokens and short prefill chunks. Longer chunks are prefill's job.
constexpr int32_t kMaxQueryLen = 1024;
constexpr int32_t kMqRowTile = 16;  // (new token, query head) rows per workgroup

struct MqPlan {
  int32_t partition_tokens;
  int32_t num_parts;
  int32_t waves;
  int32_t tiles;           // 16-row tiles per workgroup
  int32_t row_groups;      // workgroups per (sequence, KV head, partition)
  int32_t longest_first;   // as in decode: single pass, <= 256 sequences, long contexts
  int32_t detect_shared;   // as in decode: sequences split into several partitions
  size_t workspace_bytes;  // partial (m, l, o) states, when sequences are split
};

int32_t check_mq_sizes(int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_context_len, int32_t partition_tokens, MqPlan* plan) {
  if (num_seqs < 0 || num_query_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      max_context_len < 0 || max_query_len < 1 || max_query_len > kMaxQueryLen)
    return MVK_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return MVK_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_query_tokens > (int64_t)num_seqs * max_query_len)
    return MVK_ERR_INVALID_ARGUMENT;
  if (partition_tokens != 0 &&
      (partition_tokens < kBlock || partition_tokens > kMaxPartition || partition_tokens % kBlock))
    return MVK_ERR_INVALID_ARGUMENT;
  const int32_t group = num_q_heads / num_kv_heads;
  if (!mvk::decode_supported(head_dim, group)) return MVK_ERR_UNSUPPORTED;
  // A workgroup takes up to 4 row tiles (2 with head_dim 128, whose tiles
  // need twice the registers), so each block it loads serves all its rows.
  const int32_t tiles_needed = (max_query_len * group + kMqRowTile - 1) / kMqRowTile;
  const int32_t max_tiles = head_dim == 64 ? 4 : 2;
  int32_t tiles = 1;
  while (tiles < tiles_needed && tiles < max_tiles) tiles *= 2;
  const int32_t row_groups = (tiles_needed + tiles - 1) / tiles;
  const int64_t units = (int64_t)num_seqs * row_groups;  // workgroups per KV head and partition
  int32_t p = partition_tokens
                  ? partition_tokens
                  : default_partition((int32_t)(units < INT32_MAX ? units : INT32_MAX),
                                      num_kv_heads, max_context_len);
  // Four waves at every partition length: with two tiles per workgroup the
  // kernel holds about 230 VGPRs (two waves per SIMD), and eight-wave
  // workgroups measured slower on long contexts (Llama-7B shape, 4096-token
  // partitions: 652 vs 623 us with 5 new tokens).
  const int32_t waves = 4;
  int64_t parts = ((int64_t)max_context_len + p - 1) / p;
  if (parts < 1) parts = 1;
  if (units * num_kv_heads * parts > INT32_MAX) return MVK_ERR_INVALID_ARGUMENT;  // 1-D grid
  plan->partition_tokens = p;
  plan->num_parts = (int32_t)parts;
  plan->waves = waves;
  plan->tiles = tiles;
  plan->row_groups = row_groups;
  // Row groups of one (sequence, KV head) read the same blocks: in the
  // XCD-contiguous order they share an L2, in longest-first order they would
  // not, so several row groups keep that order.
  plan->detect_shared = parts > 1;
  plan->longest_first = parts == 1 && row_groups == 1 && num_seqs <= mvk::kMaxOrderedSeqs &&
                        max_context_len >= kMinOrderedContext;
  plan->workspace_bytes = parts > 1 ? (size_t)num_query_tokens * num_q_heads * (size_t)parts *
                                          (size_t)(head_dim + 2) * 4u
                                    : 0;
  return MVK_OK;
}


// ------------------------------------------------ planned decode (plan once per step)

// Bins (workgroups of mvk::kPlanWaves waves) of a decode plan: as many as the
// chip runs at once (one per CU at head_dim 128 with g >= 2, whose kernel
// holds two waves per SIMD; two per CU elsewhere, four waves per SIMD), more
// when the items would not fit their waves, and no more than there are
// (sequence, KV head) items. Contexts up to kPlanWaves * kPlanMaxBlocks
// blocks (7168 tokens) are covered.
constexpr int32_t kCus = 256;

struct PlanGeom {
  int32_t bins;
  int32_t desc_ints;
  size_t bytes;
};

int32_t plan_geometry(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t max_context_len, PlanGeom* g) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_kv_heads > kMaxGridYZ ||
      max_context_len < 0)
    return MVK_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return MVK_ERR_INVALID_ARGUMENT;
  const int32_t group = num_q_heads / num_kv_heads;
  if (!mvk::decode_supported(head_dim, group)) return MVK_ERR_UNSUPPORTED;
  if (num_seqs > mvk::kPlanMaxSeqs || num_kv_heads > mvk::kPlanMaxKvHeads) return MVK_ERR_UNSUPPORTED;
  const int64_t items = (int64_t)num_seqs * num_kv_heads;
  const int32_t waves_per_simd = (head_dim == 64 || group == 1) ? 4 : 2;
  const int64_t cap = (int64_t)kCus * (4 * waves_per_simd / mvk::kPlanWaves);
  // an item needs a wave per kPlanMaxBlocks blocks, so a bin holds at most
  // kPlanWaves / that many items; batches with more items than the resident
  // bins hold take more bins (a second round of workgroups)
  const int64_t blocks = ((int64_t)max_context_len + kBlock - 1) / kBlock;
  int64_t waves_per_item = (blocks + mvk::kPlanMaxBlocks - 1) / mvk::kPlanMaxBlocks;
  if (waves_per_item < 1) waves_per_item = 1;
  if (waves_per_item > mvk::kPlanWaves) return MVK_ERR_UNSUPPORTED;
  const int64_t items_per_bin = mvk::kPlanWaves / waves_per_item;
  int64_t bins = (items + items_per_bin - 1) / items_per_bin;
  if (bins < cap) bins = cap;
  if (bins > items) bins = items;
  if (bins > INT32_MAX / (mvk::kPlanWaves * mvk::kPlanDescInts)) return MVK_ERR_UNSUPPORTED;
  g->bins = (int32_t)bins;
  g->desc_ints = blocks <= mvk::kPlanShortDescInts - mvk::kPlanHdrInts ? mvk::kPlanShortDescInts
                                                                      : mvk::kPlanDescInts;
  g->bytes = (size_t)bins * mvk::kPlanWaves * g->desc_ints * 4u;
  return MVK_OK;
}

// ------------------------------------------- static scratch (allocation-free calls)
// The allocation-free decode entry point keeps its partial states, partition
// counters and work list in this array instead of a caller workspace. Every
// GPU the library runs on holds its own copy until the process ends. In host
// code the name `scratch` is only a host-side stand-in for the symbol: its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the GPU that `stream` runs on
// (the current device for the NULL stream). The first call on a device also
// enqueues, on `stream`, a kernel that zero-fills the counter region at its
// start (the partition counters must start at zero; every completed call
// leaves them at zero again).
hipError_t scratch_for_stream(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t err = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    err = hipGetDevice(&cur);
    if (err != hipSuccess) return err;
    if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err == hipSuccess) err = mvk::launch_zero_fill(p, kCounterRegion, stream);
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int32_t decode_impl(void* out, const void* q, void* k_cache, void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, const void* new_key,
                    const void* new_value, const int32_t* slot_mapping, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t max_context_len, float scale, int32_t dtype,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, bool use_scratch) {
  if (dtype != MVK_F16 && dtype != MVK_BF16) return MVK_ERR_INVALID_ARGUMENT;
  if (block_size != kBlock) return MVK_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || !isfinite(scale))
    return MVK_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
    return MVK_ERR_INVALID_ARGUMENT;
  Plan plan{};
  const int32_t st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                 partition_tokens, &plan);
  if (st != MVK_OK) return st;
  if (num_seqs == 0) return MVK_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens))
    return MVK_ERR_INVALID_ARGUMENT;
  if (out == q || out == k_cache || out == v_cache || k_cache == v_cache)
    return MVK_ERR_INVALID_ARGUMENT;
  if (new_key || new_value || slot_mapping) {  // fused cache write: all three or none
    if (!new_key || !new_value || !slot_mapping) return MVK_ERR_INVALID_ARGUMENT;
    if (!aligned16(new_key) || !aligned16(new_value) || !aligned4(slot_mapping))
      return MVK_ERR_INVALID_ARGUMENT;
    if ((int64_t)num_blocks * kBlock > INT32_MAX) return MVK_ERR_INVALID_ARGUMENT;
  }
  if (plan.workspace_bytes > 0) {
    if (use_scratch) {
      // allocation-free entry point: the library's static per-GPU scratch
      if (plan.workspace_bytes > kScratchBytes) return MVK_ERR_SCRATCH_LIMIT;
      void* ptr = nullptr;
      const hipError_t err = scratch_for_stream(stream, &ptr);
      if (err != hipSuccess) return MVK_ERR_HIP;
      workspace = ptr;
      workspace_bytes = kScratchBytes;
    } else {
      if (!workspace || workspace_bytes < plan.workspace_bytes) return MVK_ERR_WORKSPACE_TOO_SMALL;
      if (!aligned16(workspace)) return MVK_ERR_INVALID_ARGUMENT;
    }
  }

  mvk::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.new_key = new_key;
  a.new_value = new_value;
  a.slot_mapping = slot_mapping;
  const size_t n_state = (size_t)num_seqs * num_q_heads * (size_t)plan.num_parts;
  char* partials = (char*)workspace + plan.counter_bytes;
  a.ws_ml = plan.partial_bytes ? (float*)partials : nullptr;
  a.ws_o = plan.partial_bytes ? (float*)partials + n_state * 2 : nullptr;
  a.counters = plan.use_counters ? (int32_t*)workspace : nullptr;
  a.items = plan.work_list ? (int32_t*)(partials + plan.partial_bytes) : nullptr;
  a.list_workgroups = plan.list_workgroups;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.partition_tokens = plan.partition_tokens;
  a.num_parts = plan.num_parts;
  a.waves = plan.waves;
  a.longest_first = plan.longest_first;
  a.detect_shared = plan.detect_shared;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  a.dtype = dtype;
  hipError_t err = mvk::launch_paged_decode(a, stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
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
    case MVK_ERR_OUT_OF_BLOCKS: return "not enough free KV blocks";
    case MVK_ERR_SCRATCH_LIMIT:
      return "needs more scratch than the library's static per-GPU array holds "
             "(mvk_paged_attention_scratch_limit)";
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

size_t mvk_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t head_dim, int32_t max_context_len) {
  size_t most = 0;
  bool any = false;
  for (int32_t g = 1; g <= 8; g *= 2) {
    if (num_q_heads <= 0 || num_q_heads % g != 0) continue;
    Plan plan{};
    if (check_sizes(num_seqs, num_q_heads, num_q_heads / g, head_dim, max_context_len, 0, &plan) !=
        MVK_OK)
      continue;
    any = true;
    if (plan.workspace_bytes > most) most = plan.workspace_bytes;
  }
  return any ? most : SIZE_MAX;
}

int32_t mvk_paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_context_len, int32_t partition_tokens,
                                           size_t* workspace_bytes,
                                           int32_t* chosen_partition_tokens) {
  if (!workspace_bytes) return MVK_ERR_INVALID_ARGUMENT;
  Plan plan{};
  const int32_t st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                 partition_tokens, &plan);
  if (st != MVK_OK) return st;
  *workspace_bytes = plan.workspace_bytes;
  if (chosen_partition_tokens) *chosen_partition_tokens = plan.partition_tokens;
  return MVK_OK;
}

int32_t mvk_paged_attention_decode(void* out, const void* q, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const void* new_key, const void* new_value,
                                   const int32_t* slot_mapping, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   float scale, int32_t dtype, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, new_key, new_value,
                     slot_mapping, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_tokens, workspace, workspace_bytes, (hipStream_t)stream, false);
}

int32_t mvk_paged_attention_plan_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, size_t* plan_bytes) {
  if (!plan_bytes) return MVK_ERR_INVALID_ARGUMENT;
  PlanGeom g{};
  const int32_t st =
      plan_geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, &g);
  if (st != MVK_OK) return st;
  *plan_bytes = g.bytes;
  return MVK_OK;
}

int32_t mvk_paged_attention_plan(void* plan, size_t plan_bytes, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* slot_mapping,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t max_context_len, void* stream) {
  PlanGeom g{};
  const int32_t st =
      plan_geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, &g);
  if (st != MVK_OK) return st;
  if (max_blocks_per_seq <= 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
    return MVK_ERR_INVALID_ARGUMENT;
  if (g.bins == 0) return MVK_OK;
  if (!plan || !block_tables || !context_lens) return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(plan) || !aligned4(block_tables) || !aligned4(context_lens) ||
      (slot_mapping && !aligned4(slot_mapping)))
    return MVK_ERR_INVALID_ARGUMENT;
  if (plan_bytes < g.bytes) return MVK_ERR_WORKSPACE_TOO_SMALL;
  mvk::DecodePlanArgs a{};
  a.plan = (int32_t*)plan;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.slot_mapping = slot_mapping;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_bins = g.bins;
  a.desc_ints = g.desc_ints;
  const hipError_t err = mvk::launch_decode_plan(a, (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

int32_t mvk_paged_attention_decode_planned(void* out, const void* q, void* k_cache,
                                           void* v_cache, const void* new_key,
                                           const void* new_value, const void* plan,
                                           size_t plan_bytes, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_context_len,
                                           float scale, int32_t dtype, void* stream) {
  if (dtype != MVK_F16 && dtype != MVK_BF16) return MVK_ERR_INVALID_ARGUMENT;
  if (block_size != kBlock) return MVK_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || !isfinite(scale)) return MVK_ERR_INVALID_ARGUMENT;
  PlanGeom g{};
  const int32_t st =
      plan_geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, &g);
  if (st != MVK_OK) return st;
  if (g.bins == 0) return MVK_OK;
  if (!out || !q || !k_cache || !v_cache || !plan) return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(plan))
    return MVK_ERR_INVALID_ARGUMENT;
  if (out == q || out == k_cache || out == v_cache || k_cache == v_cache)
    return MVK_ERR_INVALID_ARGUMENT;
  if (plan_bytes < g.bytes) return MVK_ERR_WORKSPACE_TOO_SMALL;
  if (new_key || new_value) {  // fused cache write at the plan's slots: both rows or none
    if (!new_key || !new_value || !aligned16(new_key) || !aligned16(new_value))
      return MVK_ERR_INVALID_ARGUMENT;
    if ((int64_t)num_blocks * kBlock > INT32_MAX) return MVK_ERR_INVALID_ARGUMENT;
  }
  mvk::PlannedDecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.new_key = new_key;
  a.new_value = new_value;
  a.plan = (const int32_t*)plan;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.num_bins = g.bins;
  a.desc_ints = g.desc_ints;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  a.dtype = dtype;
  const hipError_t err = mvk::launch_paged_decode_planned(a, (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

int32_t mvk_paged_attention_decode_noalloc(void* out, const void* q, void* k_cache,
                                           void* v_cache, const int32_t* block_tables,
                                           const int32_t* context_lens, const void* new_key,
                                           const void* new_value, const int32_t* slot_mapping,
                                           int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t num_blocks,
                                           int32_t max_blocks_per_seq, int32_t max_context_len,
                                           float scale, int32_t dtype, int32_t partition_tokens,
                                           void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, new_key, new_value,
                     slot_mapping, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_tokens, nullptr, 0, (hipStream_t)stream, true);
}

size_t mvk_paged_attention_scratch_limit(void) { return kScratchBytes; }

int32_t mvk_paged_attention_multi_query_workspace_size(
    int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len, int32_t partition_tokens,
    size_t* workspace_bytes, int32_t* chosen_partition_tokens) {
  if (!workspace_bytes) return MVK_ERR_INVALID_ARGUMENT;
  MqPlan plan{};
  const int32_t st = check_mq_sizes(num_seqs, num_query_tokens, max_query_len, num_q_heads,
                                    num_kv_heads, head_dim, max_context_len, partition_tokens,
                                    &plan);
  if (st != MVK_OK) return st;
  *workspace_bytes = plan.workspace_bytes;
  if (chosen_partition_tokens) *chosen_partition_tokens = plan.partition_tokens;
  return MVK_OK;
}

int32_t mvk_paged_attention_multi_query(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, int32_t dtype,
    int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != MVK_F16 && dtype != MVK_BF16) return MVK_ERR_INVALID_ARGUMENT;
  if (block_size != kBlock) return MVK_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || !isfinite(scale))
    return MVK_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
    return MVK_ERR_INVALID_ARGUMENT;
  MqPlan plan{};
  const int32_t st = check_mq_sizes(num_seqs, num_query_tokens, max_query_len, num_q_heads,
                                    num_kv_heads, head_dim, max_context_len, partition_tokens,
                                    &plan);
  if (st != MVK_OK) return st;
  if (num_seqs == 0 || num_query_tokens == 0) return MVK_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens) || !aligned4(query_start))
    return MVK_ERR_INVALID_ARGUMENT;
  if (out == q || out == k_cache || out == v_cache || k_cache == v_cache)
    return MVK_ERR_INVALID_ARGUMENT;
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return MVK_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return MVK_ERR_INVALID_ARGUMENT;
  }

  mvk::MultiQueryArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  const size_t n_state = (size_t)num_query_tokens * num_q_heads * (size_t)plan.num_parts;
  a.ws_ml = plan.workspace_bytes ? (float*)workspace : nullptr;
  a.ws_o = plan.workspace_bytes ? (float*)workspace + n_state * 2 : nullptr;
  a.num_seqs = num_seqs;
  a.num_query_tokens = num_query_tokens;
  a.max_query_len = max_query_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.partition_tokens = plan.partition_tokens;
  a.num_parts = plan.num_parts;
  a.tiles = plan.tiles;
  a.row_groups = plan.row_groups;
  a.longest_first = plan.longest_first;
  a.detect_shared = plan.detect_shared;
  a.waves = plan.waves;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  a.dtype = dtype;
  hipError_t err = mvk::launch_paged_multi_query(a, (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

int32_t mvk_paged_attention_multi_query_planned(
    void* out, const void* q, const void* k_cache, const void* v_cache, const void* plan,
    size_t plan_bytes, const int32_t* query_start, int32_t num_seqs, int32_t num_query_tokens,
    int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale, int32_t dtype,
    void* stream) {
  if (dtype != MVK_F16 && dtype != MVK_BF16) return MVK_ERR_INVALID_ARGUMENT;
  if (block_size != kBlock) return MVK_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || !isfinite(scale)) return MVK_ERR_INVALID_ARGUMENT;
  if (num_query_tokens < 0 || max_query_len < 1 || max_query_len > kMaxQueryLen)
    return MVK_ERR_INVALID_ARGUMENT;
  PlanGeom g{};
  const int32_t st =
      plan_geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, &g);
  if (st != MVK_OK) return st;
  if ((int64_t)num_query_tokens > (int64_t)num_seqs * max_query_len)
    return MVK_ERR_INVALID_ARGUMENT;
  const int32_t group = num_q_heads / num_kv_heads;
  // one 16-row MFMA tile per item; head_dim 128 with g = 1 runs four waves
  // per SIMD in the plan's bins, too few registers for the tile
  if (max_query_len * group > kMqRowTile || (head_dim == 128 && group == 1))
    return MVK_ERR_UNSUPPORTED;
  if (g.bins == 0 || num_query_tokens == 0) return MVK_OK;
  if (!out || !q || !k_cache || !v_cache || !plan || !query_start) return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(plan) || !aligned4(query_start))
    return MVK_ERR_INVALID_ARGUMENT;
  if (out == q || out == k_cache || out == v_cache || k_cache == v_cache)
    return MVK_ERR_INVALID_ARGUMENT;
  if (plan_bytes < g.bytes) return MVK_ERR_WORKSPACE_TOO_SMALL;
  mvk::PlannedMultiQueryArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.plan = (const int32_t*)plan;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_query_tokens = num_query_tokens;
  a.max_query_len = max_query_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.num_bins = g.bins;
  a.desc_ints = g.desc_ints;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  a.dtype = dtype;
  const hipError_t err = mvk::launch_paged_multi_query_planned(a, (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

int32_t mvk_prefill_attention(void* out, const void* q, const void* key, const void* value,
                              void* k_cache, void* v_cache, const int32_t* slot_mapping,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_tokens,
                              int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              float scale, int32_t dtype, void* stream) {
  if (dtype != MVK_F16 && dtype != MVK_BF16) return MVK_ERR_INVALID_ARGUMENT;
  if (block_size != kBlock) return MVK_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_tokens < 0 || max_seqlen < 0 ||
      num_q_heads <= 0 || num_q_heads > kMaxGridYZ || num_kv_heads <= 0 || !isfinite(scale))
    return MVK_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return MVK_ERR_INVALID_ARGUMENT;
  if (!mvk::decode_supported(head_dim, num_q_heads / num_kv_heads)) return MVK_ERR_UNSUPPORTED;
  // The prefill kernel takes the running maximum of the raw dot products and
  // scales it afterwards, which is the maximum of the scaled logits only for
  // a positive scale.
  if (!(scale > 0.0f)) return MVK_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens > (int64_t)num_seqs * max_seqlen) return MVK_ERR_INVALID_ARGUMENT;
  // a prompt's K/V rows are addressed with 32-bit byte offsets
  if (((int64_t)max_seqlen + 256) * num_kv_heads * head_dim * 2 > INT32_MAX)
    return MVK_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return MVK_OK;
  if (!out || !q || !key || !value || !cu_seqlens) return MVK_ERR_INVALID_ARGUMENT;
  if (!aligned16(out) || !aligned16(q) || !aligned16(key) || !aligned16(value) ||
      !aligned4(cu_seqlens))
    return MVK_ERR_INVALID_ARGUMENT;
  if (out == q || out == key || out == value) return MVK_ERR_INVALID_ARGUMENT;
  if (slot_mapping) {  // the fused cache write
    if (!k_cache || !v_cache || k_cache == v_cache || num_blocks <= 0) return MVK_ERR_INVALID_ARGUMENT;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned4(slot_mapping))
      return MVK_ERR_INVALID_ARGUMENT;
    if ((int64_t)num_blocks * kBlock > INT32_MAX) return MVK_ERR_INVALID_ARGUMENT;
    if (out == k_cache || out == v_cache) return MVK_ERR_INVALID_ARGUMENT;
  }
  mvk::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.key = key;
  a.value = value;
  a.k_cache = slot_mapping ? k_cache : nullptr;
  a.v_cache = slot_mapping ? v_cache : nullptr;
  a.slot_mapping = slot_mapping;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_seqlen = max_seqlen;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = slot_mapping ? num_blocks : 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  a.dtype = dtype;
  hipError_t err = mvk::launch_prefill(a, (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

int32_t mvk_stream_read_probe(const void* src, size_t bytes, void* sink, int32_t workgroups,
                              void* stream) {
  if (!src || !sink || !aligned16(src) || !aligned4(sink)) return MVK_ERR_INVALID_ARGUMENT;
  if (bytes < 16 || bytes % 16 || bytes > (size_t(1) << 31)) return MVK_ERR_INVALID_ARGUMENT;
  if (workgroups < 1 || workgroups > kMaxGridYZ) return MVK_ERR_INVALID_ARGUMENT;
  const hipError_t err = mvk::launch_stream_read(src, (uint32_t)bytes, (uint32_t*)sink, workgroups,
                                                 (hipStream_t)stream);
  return err == hipSuccess ? MVK_OK : MVK_ERR_HIP;
}

}  // extern "C"

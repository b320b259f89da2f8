// Internal launchers behind the C ABI (host side). Arguments are already
// validated by the entry points in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mvk {

// Zero-fills `bytes` (a multiple of 16) bytes at `dst` with a kernel on
// `stream` (a kernel rather than a memset node, so that it can be captured
// into a graph and replayed).
hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t stream);

// Read-only streaming probe over [src, src + bytes) (bytes < 4 GiB, a multiple
// of 16) with `workgroups` workgroups of 256 threads; workgroup i stores one
// word to sink[i].
hipError_t launch_stream_read(const void* src, uint32_t bytes, uint32_t* sink, int32_t workgroups,
                              hipStream_t stream);

hipError_t launch_cache_write(const void* key, const void* value, void* k_cache, void* v_cache,
                              const int32_t* slot_mapping, int32_t num_tokens, int32_t row_vecs,
                              int64_t num_slots, hipStream_t stream);

// Largest batch whose single-pass decode grid is dispatched longest sequence
// first (the decode kernel ranks the batch's sequences in every workgroup).
constexpr int32_t kMaxOrderedSeqs = 256;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* new_key;          // fused cache write (nullptr = none): [S, Hkv, D]
  const void* new_value;
  const int32_t* slot_mapping;  // [S]
  float* ws_ml;  // [S, Hq, num_parts, 2] (running max in log2 units, denominator)
  float* ws_o;   // [S, Hq, num_parts, D] normalised partial outputs
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int32_t num_blocks, max_blocks_per_seq, max_context_len;
  int32_t partition_tokens, num_parts;
  int32_t waves;     // waves per workgroup (4 or 8)
  int32_t longest_first; // single-pass grid dispatched longest sequence first (see Shape)
  int32_t detect_shared; // blocks shared with a neighbouring sequence keep the default cache policy
  int32_t* items;    // work list (count, one dispatch counter per KV head, then (seq, part)
                     // pairs); nullptr = grid mode
  int32_t* counters; // per (seq, KV head) partition counters (zero between calls), or
                     // nullptr: partitions are merged by a separate kernel
  int32_t list_workgroups;  // workgroups per KV head in work-list mode
  float scale_log2;  // scale * log2(e): logits are kept in base-2 units
  int32_t dtype;
};

// Kernel variants are instantiated for these group sizes and head dims.
bool decode_supported(int32_t head_dim, int32_t group);

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

// Planned single-pass decode: a plan built once per decode step (block
// tables, lengths and new-token slots of the step) that every layer's call
// reads. The plan is num_bins * kPlanWaves descriptors of desc_ints ints:
// kPlanShortDescInts (one 128-byte line) when no sequence has more than
// kPlanShortDescInts - kPlanHdrInts blocks, kPlanDescInts otherwise, so a
// batch of short contexts reads half the plan bytes per call.
constexpr int32_t kPlanWaves = 8;          // waves per bin (workgroup)
constexpr int32_t kPlanDescInts = 64;      // ints per wave descriptor (longest form)
constexpr int32_t kPlanShortDescInts = 32;  // the short form
constexpr int32_t kPlanHdrInts = 8;        // descriptor header; the rest are block ids
constexpr int32_t kPlanMaxBlocks = kPlanDescInts - kPlanHdrInts;  // blocks per wave
constexpr int32_t kPlanMaxSeqs = 1024;   // sequences one plan ranks (in LDS)
constexpr int32_t kPlanMaxKvHeads = 256;  // KV heads of a planned batch

// Descriptor header fields (ints 0..7); the rest are the wave's block ids.
enum : int {
  kDescSeq = 0,       // sequence (negative: idle wave)
  kDescHead = 1,      // KV head
  kDescTokBegin = 2,  // first token of the wave's run (a multiple of 16)
  kDescTokEnd = 3,    // one past its last token
  kDescSlot = 4,      // the sequence's new-token slot (fused cache write), or -1
  kDescWaves = 5,     // first wave of the item (bits 0-7), waves of the item (bits 8-15)
  kDescLen = 6,       // the sequence's context length
  kDescFlags = 7,     // the wave's part in the fused cache write
};

struct DecodePlanArgs {
  int32_t* plan;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* slot_mapping;  // nullptr: no new-token slots recorded
  int32_t num_seqs, num_kv_heads, max_blocks_per_seq, max_context_len, num_bins;
  int32_t desc_ints;  // kPlanShortDescInts or kPlanDescInts
};

hipError_t launch_decode_plan(const DecodePlanArgs& a, hipStream_t stream);

struct PlannedDecodeArgs {
  void* out;
  const void* q;
  void* k_cache;
  void* v_cache;
  const void* new_key;    // fused cache write (nullptr = none), at the plan's slots
  const void* new_value;
  const int32_t* plan;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_context_len, num_bins;
  int32_t desc_ints;  // the plan's descriptor size
  float scale_log2;
  int32_t dtype;
};

hipError_t launch_paged_decode_planned(const PlannedDecodeArgs& a, hipStream_t stream);

// Multi-query attention through a decode plan built without new-token slots
// (single-pass batches, n * g <= 16 rows per item): every wave streams its
// descriptor's blocks for all n * g query rows of its item.
struct PlannedMultiQueryArgs {
  void* out;                   // [T, Hq, D]
  const void* q;               // [T, Hq, D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* plan;
  const int32_t* query_start;  // [S + 1]
  int32_t num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim;
  int32_t num_blocks, max_context_len, num_bins;
  int32_t desc_ints;           // the plan's descriptor size
  float scale_log2;
  int32_t dtype;
};

hipError_t launch_paged_multi_query_planned(const PlannedMultiQueryArgs& a, hipStream_t stream);

struct MultiQueryArgs {
  void* out;                   // [T, Hq, D]
  const void* q;               // [T, Hq, D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // [S + 1]: sequence s owns query rows [query_start[s], query_start[s+1])
  float* ws_ml;  // [T, Hq, num_parts, 2] (running max in log2 units, denominator)
  float* ws_o;   // [T, Hq, num_parts, D] normalised partial outputs
  int32_t num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim;
  int32_t num_blocks, max_blocks_per_seq, max_context_len;
  int32_t partition_tokens, num_parts;
  int32_t tiles;       // 16-row MFMA tiles per workgroup (1, 2, or 4 with head_dim 64)
  int32_t row_groups;  // groups of 16 * tiles (new token, query head) rows per (sequence, KV head)
  int32_t waves;       // waves per workgroup (4 or 8)
  int32_t longest_first;  // single-pass grid dispatched longest sequence first
  int32_t detect_shared;  // blocks shared with a neighbouring sequence keep the default cache policy
  float scale_log2;
  int32_t dtype;
};

hipError_t launch_paged_multi_query(const MultiQueryArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;                    // [T, Hq, D]
  const void* q;                // [T, Hq, D]
  const void* key;              // [T, Hkv, D] the prompts' new K/V rows
  const void* value;
  void* k_cache;                // pools, written at slot_mapping (nullptr slot_mapping: no write)
  void* v_cache;
  const int32_t* slot_mapping;  // [T] or nullptr
  const int32_t* cu_seqlens;    // [S + 1]: prompt s owns rows [cu_seqlens[s], cu_seqlens[s+1])
  int32_t num_seqs, num_tokens, max_seqlen, num_q_heads, num_kv_heads, head_dim, num_blocks;
  float scale_log2;
  int32_t dtype;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace mvk

/*
 * mvk.h - C ABI of the MI355X (gfx950) paged KV-cache attention library.
 *
 * Two operations make up one decode step of a paged KV cache:
 *
 *   mvk_reshape_and_cache       scatter the step's new K/V rows into their
 *                               physical slots of the block pools;
 *   mvk_paged_attention_decode  each sequence's single new query token attends
 *                               over its whole cached context, read block by
 *                               block through its block table.
 *
 * Where the operations come from (web pages on small vLLM re-implementations):
 *   - "从零手写 vLLM 核心：mini-vllm 项目深度解析", section "2. 分页KV缓存（PagedAttention）":
 *     the KV cache is cut into fixed 16-token blocks managed like pages of
 *     virtual memory, which lets sequences share physical blocks (prefix cache);
 *   - same page, "关键工程决策", item 1: every layer reads its own cache length;
 *     item 2: in steady state every running request is in one batched decode;
 *     item 3: K and V pools are separate, layer-first, with the block dimension
 *     ahead of the KV-head dimension, and attention receives views of them;
 *   - micro-vLLM wiki, feature list and API example: the attention operator is
 *     a swappable backend (this library is one), block_size = 16.
 *
 * Conventions shared by every entry point
 *   - Pointers to tensors are DEVICE pointers owned by the caller. The library
 *     allocates nothing and keeps no state between calls (the one exception is
 *     mvk_paged_attention_decode_noalloc's static scratch), and is thread-safe.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously; MVK_OK means "arguments valid and kernels launched".
 *     A fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is launched and nothing is written.
 *   - Tensors are dense and row-major; every tensor pointer must be 16-byte
 *     aligned.
 *   - dtype: MVK_F16 (IEEE binary16) or MVK_BF16 (bfloat16). q, the pools,
 *     key/value and out all share it.
 *   - Pool layout (one layer): [num_blocks, block_size, num_kv_heads, head_dim].
 *     Token t of sequence s lives in physical block block_tables[s][t / 16] at
 *     offset t % 16. A flat slot number is block * 16 + offset.
 *   - Device-side index contents (block ids, slots, lengths) are not checked on
 *     the host (mvk_check_indices counts bad entries on the device, on
 *     request). The kernels never access memory outside the buffers described
 *     by the size arguments: an out-of-range block id is read as block 0 and an
 *     out-of-range slot is not written; the affected output is then unspecified.
 */
#ifndef MVK_H
#define MVK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MVK_ABI_VERSION 8

typedef enum mvk_status {
    MVK_OK = 0,
    MVK_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misaligned tensor */
    MVK_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, group size, block size */
    MVK_ERR_WORKSPACE_TOO_SMALL = 3,
    MVK_ERR_HIP = 4,                /* a HIP launch reported an error */
    MVK_ERR_OUT_OF_BLOCKS = 5,      /* block manager: not enough free KV blocks */
    MVK_ERR_SCRATCH_LIMIT = 6       /* allocation-free call: the sizes need more than the
                                       library's static scratch (mvk_paged_attention_scratch_limit) */
} mvk_status;

typedef enum mvk_dtype {
    MVK_F16 = 0,
    MVK_BF16 = 1
} mvk_dtype;

/* Version of this ABI (MVK_ABI_VERSION of the built library). */
int32_t mvk_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* mvk_status_string(int32_t status);

/*
 * mvk_reshape_and_cache - write one step's new K and V rows into the pools.
 *
 * Defines: for every i < num_tokens with s = slot_mapping[i] >= 0,
 *   k_cache[s / 16][s % 16][:][:] = key[i][:][:]  and the same for V.
 * The copy is raw (no conversion), so the pools receive the exact bits.
 * (Paged cache with fixed 16-token blocks: mini-vllm write-up, section
 * "2. 分页KV缓存（PagedAttention）"; pool layout: "关键工程决策", item 3.)
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim], dtype, read only.
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim], dtype;
 *   v_cache       only the addressed rows are written.
 *   slot_mapping  int32 [num_tokens]; negative = padding, skipped. A slot at or
 *                 past num_blocks * block_size is skipped. Two tokens with the
 *                 same slot leave that row holding one of them (unspecified).
 *   block_size    must be 16.  head_dim: 64 or 128.  num_tokens == 0 is a no-op.
 * Errors: MVK_ERR_INVALID_ARGUMENT (null/misaligned pointers, negative sizes,
 * bad dtype), MVK_ERR_UNSUPPORTED (block_size, head_dim), MVK_ERR_HIP.
 */
int32_t mvk_reshape_and_cache(const void* key, const void* value,
                              void* k_cache, void* v_cache,
                              const int32_t* slot_mapping,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks,
                              int32_t dtype, void* stream);

/*
 * mvk_paged_attention_workspace_size - bytes of scratch that
 * mvk_paged_attention_decode needs for these sizes.
 *
 * Long contexts are cut into partitions of `partition_tokens` tokens (a
 * multiple of 16; 0 lets the library choose from num_seqs, num_kv_heads and
 * max_context_len). When a sequence spans more than one partition, each
 * partition's partial softmax state (running max, denominator, normalised
 * output; float32) goes to the workspace, and the partitions are merged either
 * by a second kernel of the same call or, for skewed batches, by the last
 * partition of a (sequence, KV head) to finish, counted in a 64 KiB counter
 * region at the start of the workspace that holds nothing else. Skewed
 * batches also keep a compact list of their non-empty partitions there.
 *
 *   *workspace_bytes          receives the size (0 when no split is needed).
 *   *chosen_partition_tokens  receives the partition length that the decode
 *                             call will use for the same arguments (may be NULL).
 * Errors: as for mvk_paged_attention_decode's size checks.
 */
int32_t mvk_paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_context_len, int32_t partition_tokens,
                                           size_t* workspace_bytes,
                                           int32_t* chosen_partition_tokens);

/*
 * mvk_paged_attention_workspace_bytes - workspace bytes that suffice for
 * mvk_paged_attention_decode with these sizes and the library's choice of
 * partition length (partition_tokens = 0), whatever the number of KV heads:
 * the largest of mvk_paged_attention_workspace_size's answers over every
 * supported group size num_q_heads / num_kv_heads (1, 2, 4, 8). A caller that
 * knows num_kv_heads gets the exact size from mvk_paged_attention_workspace_size.
 * Returns SIZE_MAX when no group size gives valid sizes (e.g. head_dim not 64
 * or 128, negative sizes).
 */
size_t mvk_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t head_dim, int32_t max_context_len);

/*
 * mvk_paged_attention_decode - one batched decode step of paged attention,
 * optionally with that step's cache write fused in.
 *
 * Defines, for every sequence s, query head j and d < head_dim, with
 * L = context_lens[s], g = num_q_heads / num_kv_heads and h = j / g
 * (consecutive query heads share a KV head):
 *   z_t        = scale * sum_d q[s][j][d] * K_t[h][d]        for t < L,
 *   out[s][j]  = sum_t softmax(z)_t * V_t[h]
 * where K_t / V_t are token t's rows fetched through block_tables[s]. The new
 * token of this step counts in L and must be in the pools when attention reads
 * it: stored earlier with mvk_reshape_and_cache, or passed in new_key /
 * new_value / slot_mapping (below). L == 0 gives an all-zero row. Arithmetic
 * is float32 (products, logits, softmax, accumulation); out is rounded to
 * nearest-even. (Method: mini-vllm write-up, "2. 分页KV缓存（PagedAttention）"
 * and "关键工程决策" items 1-3; micro-vLLM wiki, paged-attention backend.)
 *
 *   out           [num_seqs, num_q_heads, head_dim], dtype, written.
 *   q             [num_seqs, num_q_heads, head_dim], dtype.
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim], dtype; read,
 *   v_cache       and written only by the fused cache write.
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; entries past
 *                 ceil(L / 16) are never read (any value).
 *   context_lens  int32 [num_seqs]; each must be <= max_context_len (tokens
 *                 past it are ignored).
 *   new_key,      fused cache write, all three NULL or all three set:
 *   new_value     [num_seqs, num_kv_heads, head_dim], dtype: row s is sequence
 *   slot_mapping  s's token of this step; int32 [num_seqs] its flat slot
 *                 (negative = no write). The rows are stored exactly as
 *                 mvk_reshape_and_cache(new_key, new_value, ..., num_seqs)
 *                 would store them (bit-exact), and sequence s's attention
 *                 sees row s wherever its slot lies in s's own context. A slot
 *                 that lies in another sequence's context is stored, but what
 *                 that other sequence reads for it in the same call is
 *                 unspecified (a paged allocator never appends into a block
 *                 another sequence reads).
 *   max_context_len  host-side upper bound of context_lens; sizes the split.
 *                 Must be <= max_blocks_per_seq * 16.
 *   scale         finite float multiplier of the raw dot products.
 *   partition_tokens  0 = library choice, else a multiple of 16 in [16, 4096].
 *   workspace     device scratch of workspace_bytes (from
 *                 mvk_paged_attention_workspace_size with the same sizes and
 *                 partition_tokens); may be NULL when that size is 0. Owned by
 *                 the caller. It must be zero-filled before its first use
 *                 (e.g. hipMemset at allocation); every call that completes
 *                 leaves it ready for the next one, so it can be reused
 *                 without clearing. It must not be shared by calls that may
 *                 run concurrently.
 *   head_dim 64 or 128; num_q_heads / num_kv_heads in {1, 2, 4, 8};
 *   block_size 16.  num_seqs == 0 is a no-op.
 * Unused pool slots and the unread tail of a sequence's last block may hold
 * any bits, NaN included: they do not reach the output.
 * The output does not depend on the order in which the GPU runs work items:
 * repeated calls with the same inputs give identical bits, and a fused call
 * gives the same bits as the cache write followed by the unfused call.
 * Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_UNSUPPORTED,
 * MVK_ERR_WORKSPACE_TOO_SMALL, MVK_ERR_HIP.
 */
int32_t mvk_paged_attention_decode(void* out, const void* q,
                                   void* k_cache, void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const void* new_key, const void* new_value,
                                   const int32_t* slot_mapping,
                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   float scale, int32_t dtype, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Planned decode: the layout of a decode step's work computed once per step
 * and reused by every layer's decode call of that step.
 *
 * In steady state every running sequence is in one batched decode step, and
 * every layer runs that step over its own pools with the same block tables,
 * context lengths and new-token slots ("从零手写 vLLM 核心：mini-vllm 项目深度解析",
 * "关键工程决策" items 1-3). mvk_paged_attention_plan reads those arrays once
 * per step on the device: it ranks the sequences by length, deals the
 * (sequence, KV head) items to workgroups that carry equal numbers of blocks
 * (long items paired with short ones), splits each workgroup's waves over its
 * items, and records for every wave its sequence, KV head, token range and the
 * physical ids of its blocks. Each mvk_paged_attention_decode_planned call
 * then starts streaming K/V after one load per wave, with no per-layer
 * ranking or table walk.
 *
 * Scope: single-pass batches (each (sequence, KV head) item is done by one
 * workgroup): at most 1024 sequences and 256 KV heads, and contexts short
 * enough for the items of a workgroup (mvk_paged_attention_plan_size returns
 * MVK_ERR_UNSUPPORTED otherwise; mvk_paged_attention_decode covers every
 * batch). The plan is a snapshot: it holds copies of the block ids, lengths
 * and slots as they are when the plan kernel runs (stream order); later
 * changes to those arrays do not reach planned calls until the next plan.
 */

/* Bytes of device memory a plan for these sizes takes (*plan_bytes).
 * Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_UNSUPPORTED (outside the planned
 * path's scope: use mvk_paged_attention_decode). */
int32_t mvk_paged_attention_plan_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, size_t* plan_bytes);

/*
 * mvk_paged_attention_plan - build a step's plan into `plan` (device memory of
 * plan_bytes >= mvk_paged_attention_plan_size; caller-owned; 16-byte
 * aligned), asynchronously on `stream`.
 *   block_tables  int32 [num_seqs, max_blocks_per_seq] (device), as for decode.
 *   context_lens  int32 [num_seqs] (device); values are clamped into
 *                 [0, max_context_len].
 *   slot_mapping  int32 [num_seqs] (device) or NULL: each sequence's new-token
 *                 slot, used by planned calls that fuse the cache write.
 *   max_context_len  host-side bound of context_lens, <= max_blocks_per_seq * 16.
 * num_seqs == 0 is a no-op. Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_UNSUPPORTED,
 * MVK_ERR_WORKSPACE_TOO_SMALL (plan_bytes), MVK_ERR_HIP.
 */
int32_t mvk_paged_attention_plan(void* plan, size_t plan_bytes, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* slot_mapping,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t max_context_len, void* stream);

/*
 * mvk_paged_attention_decode_planned - one layer's decode step through a plan.
 *
 * Computes what mvk_paged_attention_decode computes (same definition,
 * arithmetic and rounding) for the block tables, context lengths and slots the
 * plan was built from; num_seqs, num_q_heads, num_kv_heads, head_dim and
 * max_context_len must be those of the plan call. With new_key / new_value
 * ([num_seqs, num_kv_heads, head_dim]; both or neither) the step's cache write
 * is fused in at the plan's slots (none when the plan had no slot_mapping),
 * bit-exact as mvk_reshape_and_cache. The summation order differs from the
 * unplanned call's, so the two may differ in the last bits (both within the
 * same bound of the exact result); planned calls with the same plan and inputs
 * give identical bits.
 *   out, q, k_cache, v_cache, scale, dtype, block_size: as for decode.
 *   plan, plan_bytes: a plan built by mvk_paged_attention_plan (stream order).
 * Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_UNSUPPORTED,
 * MVK_ERR_WORKSPACE_TOO_SMALL (plan_bytes), MVK_ERR_HIP.
 */
int32_t mvk_paged_attention_decode_planned(void* out, const void* q, void* k_cache,
                                           void* v_cache, const void* new_key,
                                           const void* new_value, const void* plan,
                                           size_t plan_bytes, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_context_len,
                                           float scale, int32_t dtype, void* stream);

/*
 * mvk_paged_attention_decode_noalloc - mvk_paged_attention_decode without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, semantics, kernels and output bits as
 * mvk_paged_attention_decode with the same partition_tokens; the partial
 * states, partition counters and work list that a split call keeps in the
 * workspace go to a static device array of the library instead
 * (mvk_paged_attention_scratch_limit() bytes per GPU, held from the first such
 * call on a GPU until the process ends). The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.
 *   - Every call on one GPU shares that GPU's array. Calls that may overlap on
 *     one GPU (different streams without ordering, several threads) race on it
 *     and give unspecified results; calls ordered on one stream are safe.
 *   - The first call on a GPU also enqueues, on `stream`, a kernel that clears
 *     the counter region of the array; every completed call leaves the
 *     counters at zero again.
 * Errors: as mvk_paged_attention_decode, with MVK_ERR_SCRATCH_LIMIT (nothing
 * launched) when these sizes would need a larger workspace than the array
 * (mvk_paged_attention_workspace_size gives the need), and MVK_ERR_HIP when the
 * array's device address cannot be obtained.
 */
int32_t mvk_paged_attention_decode_noalloc(void* out, const void* q,
                                           void* k_cache, void* v_cache,
                                           const int32_t* block_tables, const int32_t* context_lens,
                                           const void* new_key, const void* new_value,
                                           const int32_t* slot_mapping,
                                           int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t num_blocks,
                                           int32_t max_blocks_per_seq, int32_t max_context_len,
                                           float scale, int32_t dtype, int32_t partition_tokens,
                                           void* stream);

/* Bytes of the static per-GPU scratch array of mvk_paged_attention_decode_noalloc. */
size_t mvk_paged_attention_scratch_limit(void);

/*
 * mvk_paged_attention_multi_query_workspace_size - bytes of scratch that
 * mvk_paged_attention_multi_query needs for these sizes (0 when no sequence
 * is split into partitions), and the partition length it will use.
 * Arguments as for mvk_paged_attention_multi_query. Errors: as for its size
 * checks.
 */
int32_t mvk_paged_attention_multi_query_workspace_size(int32_t num_seqs, int32_t num_query_tokens,
                                                       int32_t max_query_len, int32_t num_q_heads,
                                                       int32_t num_kv_heads, int32_t head_dim,
                                                       int32_t max_context_len,
                                                       int32_t partition_tokens,
                                                       size_t* workspace_bytes,
                                                       int32_t* chosen_partition_tokens);

/*
 * mvk_paged_attention_multi_query - paged attention for several new tokens
 * per sequence, causal among them: the target model's verification pass of
 * speculative decoding, which scores the last accepted token and K draft
 * tokens in one forward pass ("从零手写 vLLM 核心：mini-vllm 项目深度解析",
 * section "推测解码原理"), and a short prefill chunk over a cached prefix.
 *
 * Defines, for sequence s with L = context_lens[s] cached tokens of which the
 * last n = query_start[s+1] - query_start[s] are new (their K/V rows already
 * in the pools, e.g. written by mvk_reshape_and_cache), for new token
 * i < n (query row t = query_start[s] + i, position L - n + i), query head j
 * and h = j / g:
 *   out[t][j] = sum_{u <= L-n+i} softmax_u(scale * q[t][j] . K_u[h]) V_u[h]
 * Arithmetic, rounding, block addressing and GQA grouping are those of
 * mvk_paged_attention_decode; with n = 1 for every sequence the result equals
 * the decode call's.
 *
 *   out, q        [num_query_tokens, num_q_heads, head_dim], dtype; out written.
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim], dtype; read.
 *   v_cache
 *   block_tables  int32 [num_seqs, max_blocks_per_seq] (as for decode).
 *   context_lens  int32 [num_seqs]; each <= max_context_len, and >= its n.
 *   query_start   int32 [num_seqs + 1], on the device: 0 = query_start[0] <=
 *                 ... <= query_start[num_seqs] = num_query_tokens; every
 *                 n <= max_query_len and n <= L. A sequence with n = 0 has
 *                 no rows. (n > L is not checked on the device: such rows see
 *                 only the positions that exist, or none, and are then zero.
 *                 Offsets outside [0, num_query_tokens] are clamped into it
 *                 and n to max_query_len, so inconsistent values give wrong
 *                 rows but no access outside q, out or the workspace.)
 *   max_query_len host-side bound of n, in [1, 1024].
 *   max_context_len, scale, dtype, partition_tokens: as for decode.
 *   workspace     device scratch of workspace_bytes (from the query above with
 *                 the same sizes); may be NULL when that size is 0; owned by
 *                 the caller, needs no clearing, not shared by concurrent calls.
 *   head_dim 64 or 128; num_q_heads / num_kv_heads in {1, 2, 4, 8};
 *   block_size 16. num_seqs == 0 or num_query_tokens == 0 is a no-op.
 * Unread pool slots may hold any bits. Repeated calls give identical bits.
 * Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_UNSUPPORTED,
 * MVK_ERR_WORKSPACE_TOO_SMALL, MVK_ERR_HIP.
 */
int32_t mvk_paged_attention_multi_query(void* out, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables,
                                        const int32_t* context_lens,
                                        const int32_t* query_start,
                                        int32_t num_seqs, int32_t num_query_tokens,
                                        int32_t max_query_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks,
                                        int32_t max_blocks_per_seq, int32_t max_context_len,
                                        float scale, int32_t dtype, int32_t partition_tokens,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * mvk_paged_attention_multi_query_planned - the multi-query call through a
 * step's plan (mvk_paged_attention_plan), for single-pass batches: the same
 * definition and arithmetic as mvk_paged_attention_multi_query (the rows'
 * summation order differs, so results may differ in the last bits; both are
 * within the same bound of the exact result), with the (sequence, KV head)
 * items dealt to workgroups by the plan instead of one workgroup per item.
 * A speculative-verification step runs every layer over the same block
 * tables, context lengths and query offsets, so the plan is built once per
 * step as for decode
 * ("从零手写 vLLM 核心：mini-vllm 项目深度解析", "推测解码原理" and
 * "关键工程决策" items 1-3).
 *   plan, plan_bytes  a plan built by mvk_paged_attention_plan from this
 *                 call's block_tables and context_lens with slot_mapping =
 *                 NULL, the same num_seqs, num_q_heads, num_kv_heads, head_dim
 *                 and max_context_len (stream order). A plan built with new-
 *                 token slots is a decode step's (its runs end before each
 *                 sequence's last position): every output row of a sequence
 *                 with a slot is then written as NaN.
 *   out, q, k_cache, v_cache, query_start, num_query_tokens, max_query_len,
 *   scale, dtype, block_size, num_blocks: as for mvk_paged_attention_multi_query.
 * Scope: the plan's (mvk_paged_attention_plan_size), max_query_len * g <= 16,
 * and not head_dim 128 with g = 1 (MVK_ERR_UNSUPPORTED otherwise;
 * mvk_paged_attention_multi_query covers every batch). No workspace.
 * num_seqs == 0 or num_query_tokens == 0 is a no-op. Repeated calls give
 * identical bits. Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_UNSUPPORTED,
 * MVK_ERR_WORKSPACE_TOO_SMALL (plan_bytes), MVK_ERR_HIP.
 */
int32_t mvk_paged_attention_multi_query_planned(void* out, const void* q, const void* k_cache,
                                                const void* v_cache, const void* plan,
                                                size_t plan_bytes, const int32_t* query_start,
                                                int32_t num_seqs, int32_t num_query_tokens,
                                                int32_t max_query_len, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t num_blocks,
                                                int32_t max_context_len, float scale,
                                                int32_t dtype, void* stream);

/*
 * mvk_prefill_attention - causal self-attention of new prompts, with their
 * K/V rows stored into the paged pools in the same call: the pass a request
 * runs over its whole prompt when it is admitted, before it decodes
 * ("从零手写 vLLM 核心：mini-vllm 项目深度解析", section "1. 连续批处理" and
 * "关键工程决策" item 2).
 *
 * Defines, for prompt s owning rows lo = cu_seqlens[s] .. cu_seqlens[s+1]-1,
 * its token t (row lo + t), query head j and h = j / g:
 *   out[lo+t][j] = sum_{u <= t} softmax_u(scale * q[lo+t][j] . key[lo+u][h]) value[lo+u][h]
 * and, when slot_mapping is given, stores key[r] / value[r] at flat slot
 * slot_mapping[r] of k_cache / v_cache exactly as mvk_reshape_and_cache would
 * (negative slots skipped). Attention reads the key/value tensors, not the
 * pools. Arithmetic and rounding as for mvk_paged_attention_decode.
 *
 *   out, q        [num_tokens, num_q_heads, head_dim], dtype; out written.
 *   key, value    [num_tokens, num_kv_heads, head_dim], dtype.
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim], dtype;
 *   v_cache       written at slot_mapping; ignored (may be NULL) without it.
 *   slot_mapping  int32 [num_tokens] or NULL (no cache write).
 *   cu_seqlens    int32 [num_seqs + 1], on the device: 0 = cu_seqlens[0] <=
 *                 ... <= cu_seqlens[num_seqs] = num_tokens, every prompt
 *                 length <= max_seqlen (host-side bound that sizes the grid).
 *                 Offsets outside [0, num_tokens] are clamped into it (no
 *                 access outside the token arrays; rows of a prompt longer
 *                 than the grid covers are not computed).
 *   scale         finite and > 0 (MVK_ERR_UNSUPPORTED otherwise: the kernel takes
 *                 the running maximum of the raw dot products and scales it).
 *   head_dim 64 or 128; num_q_heads / num_kv_heads in {1, 2, 4, 8};
 *   block_size 16. num_seqs == 0 or num_tokens == 0 is a no-op.
 *   A prompt's rows are addressed with 32-bit byte offsets: (max_seqlen + 256)
 *   * num_kv_heads * head_dim * 2 above INT32_MAX is MVK_ERR_UNSUPPORTED.
 *   Inputs are finite numbers: the kernel is compiled without NaN semantics,
 *   so a NaN in q, key or value gives an unspecified output (it is not
 *   guaranteed to propagate).
 * Repeated calls give identical bits.
 * Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_UNSUPPORTED, MVK_ERR_HIP.
 */
int32_t mvk_prefill_attention(void* out, const void* q, const void* key, const void* value,
                              void* k_cache, void* v_cache, const int32_t* slot_mapping,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_tokens,
                              int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              float scale, int32_t dtype, void* stream);

/*
 * mvk_stream_read_probe - measurement aid: a read-only streaming kernel over
 * `bytes` bytes of device memory at `src`, with the same 16-byte loads and
 * non-temporal cache policy as the attention kernels' K/V streams, giving the
 * practical HBM read rate that their byte rates are compared with. Workgroup
 * i of `workgroups` (256 threads each) writes one uint32 to sink[i] so that no
 * load is dead; nothing else is written.
 *   src   device, 16-byte aligned; bytes a multiple of 16 in [16, 2^31].
 *   sink  device uint32 [workgroups]; workgroups in [1, 65535].
 * Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_HIP.
 */
int32_t mvk_stream_read_probe(const void* src, size_t bytes, void* sink, int32_t workgroups,
                              void* stream);

/*
 * mvk_check_indices - debug check of a step's index arrays, the optional
 * device-side check the calls above skip (they never read index contents for
 * validation). One small kernel counts, asynchronously on `stream`:
 *   counts[0]  context lengths outside [0, max_context_len];
 *   counts[1]  block ids a call would read (entries j < ceil(L / 16) of row s,
 *              L = context_lens[s] clamped to [0, min(max_context_len,
 *              16 * max_blocks_per_seq)]) outside [0, num_blocks);
 *   counts[2]  slots >= 16 * num_blocks (a negative slot means no write).
 * Arguments (device pointers):
 *   counts        int64 [3], 8-byte aligned; written by the kernel (no prior
 *                 zeroing needed); read it after synchronising the stream.
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; context_lens int32
 *                 [num_seqs] (both may be NULL when num_seqs == 0).
 *   slot_mapping  int32 [num_slots] (NULL allowed when num_slots == 0).
 *   num_blocks > 0 (the pool's blocks); max_context_len >= 0.
 * Allocates nothing; reads only the entries described above.
 * Errors: MVK_ERR_INVALID_ARGUMENT, MVK_ERR_HIP.
 */
int32_t mvk_check_indices(int64_t* counts, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t max_context_len,
                          const int32_t* slot_mapping, int32_t num_slots, int32_t num_blocks,
                          void* stream);

/*
 * Block manager (host side): which physical 16-token blocks each sequence
 * owns, the block tables and slot mappings the calls above read, prefix
 * sharing of full blocks, and release, eviction and rollback. The KV-cache
 * manager owns logical blocks, block tables, the prefix cache, and block
 * allocation and release (micro-vLLM wiki, layer description
 * "KVCacheManager", feature list "Paged KV Cache、prefix cache 和请求抢占");
 * blocks are allocated on demand, shared through prefix caching, and
 * admission stays correct when blocks are scarce ("从零手写 vLLM 核心：
 * mini-vllm 项目深度解析", section "2. 分页KV缓存（PagedAttention）");
 * speculative decoding needs KV rollback (same write-up, "工程启示").
 *
 * Rules:
 *  - A slot is a flat pool row: block * 16 + offset; token t of a sequence is
 *    in table[t / 16] at offset t % 16.
 *  - A full block is identified by the chained hash of its parent block and
 *    its 16 token ids (checked against the ids on a hit). A new sequence
 *    shares the cached blocks of its longest cached full-block prefix; the
 *    block holding its last prompt token is always its own. Shared blocks are
 *    reference counted.
 *  - A released block goes to the back of the free queue; a block with a hash
 *    stays findable until the queue hands it out again (least recently
 *    released first). A sequence's blocks are released newest first, so its
 *    prefix stays cached longest.
 *  - Rollback drops a sequence's newest tokens and never modifies a block
 *    another sequence shares (MVK_ERR_INVALID_ARGUMENT instead).
 * Host memory only; not thread-safe (one manager per scheduler thread).
 * Errors: MVK_ERR_INVALID_ARGUMENT (NULL manager or output, unknown or
 * duplicate seq_id, bad sizes), MVK_ERR_OUT_OF_BLOCKS (nothing was changed).
 */
typedef struct mvk_block_manager mvk_block_manager;

/* A manager of num_blocks blocks of block_size (16) tokens, all free; prefix
 * sharing on when prefix_cache != 0. NULL on bad sizes (num_blocks must be in
 * 1 .. INT32_MAX / 16) or no memory. A sequence holds at most INT32_MAX / 2
 * tokens (MVK_ERR_INVALID_ARGUMENT beyond). */
mvk_block_manager* mvk_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_cache);
void mvk_bm_destroy(mvk_block_manager* m);

/* Blocks in the free queue (cached ones included); -1 for a NULL manager. */
int32_t mvk_bm_num_free(const mvk_block_manager* m);

/* Whether a prompt of num_tokens token ids could be admitted now: MVK_OK or
 * MVK_ERR_OUT_OF_BLOCKS; *cached_tokens (may be NULL) receives how many of its
 * leading tokens are already cached. Changes nothing. */
int32_t mvk_bm_can_admit(const mvk_block_manager* m, const int32_t* token_ids,
                         int32_t num_tokens, int32_t* cached_tokens);

/* Admit a prompt as sequence seq_id: share its cached prefix blocks, allocate
 * the rest. *cached_tokens (may be NULL) receives the shared prefix length in
 * tokens (its K/V rows need not be recomputed). */
int32_t mvk_bm_admit(mvk_block_manager* m, int64_t seq_id, const int32_t* token_ids,
                     int32_t num_tokens, int32_t* cached_tokens);

/* Append one token (a decode step or a draft token); *slot receives its slot. */
int32_t mvk_bm_append(mvk_block_manager* m, int64_t seq_id, int32_t token_id, int32_t* slot);

/* Drop the sequence's newest num_tokens tokens (rejected drafts). */
int32_t mvk_bm_rollback(mvk_block_manager* m, int64_t seq_id, int32_t num_tokens);

/* Release a finished or preempted sequence. */
int32_t mvk_bm_release(mvk_block_manager* m, int64_t seq_id);

/* Tokens and blocks the sequence holds (either pointer may be NULL). */
int32_t mvk_bm_seq_info(const mvk_block_manager* m, int64_t seq_id, int32_t* num_tokens,
                        int32_t* num_blocks);

/* The sequence's block table into table[0 .. max_blocks), -1 past its blocks. */
int32_t mvk_bm_block_table(const mvk_block_manager* m, int64_t seq_id, int32_t* table,
                           int32_t max_blocks);

/* Slots of the sequence's tokens first_token .. first_token + count - 1. */
int32_t mvk_bm_slots(const mvk_block_manager* m, int64_t seq_id, int32_t first_token,
                     int32_t count, int32_t* slots);

/* Reference count of a block (0 = free); -1 for a bad manager or block. */
int32_t mvk_bm_block_ref(const mvk_block_manager* m, int32_t block);

#ifdef __cplusplus
}
#endif

#endif /* MVK_H */

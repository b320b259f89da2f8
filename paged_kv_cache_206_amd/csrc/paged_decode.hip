// Paged-attention decode for gfx950 (CDNA4), wave64.
//
// Method (mini-vllm write-up, "2. 分页KV缓存（PagedAttention）" and
// "关键工程决策" items 1-3): every sequence's single new query token attends
// over its cached context, whose K and V rows sit in fixed 16-token blocks of
// separate pools [num_blocks, 16, Hkv, D] and are found through the
// sequence's block table.
//
// Work decomposition: one workgroup per (partition, KV head, sequence). It
// serves all g = Hq/Hkv query heads of the GQA group, so each K/V row fetched
// from HBM is used g times. The partition's blocks are dealt round-robin to
// the W waves of the workgroup; every wave first fetches all of its block-table
// entries with one vector load (issued together with the context length, the
// query rows and the new K/V row, so the prologue costs one round trip), then
// streams its blocks with the next blocks' K/V loads in flight while the
// current block is computed.
//
// Fused cache write (both policies): when the call brings the step's new K/V
// rows, the block holding a sequence's new slot takes that row from registers
// instead of memory, and wave 0 of partition 0 stores it once (the store of
// record), so attention never waits for its own write.
//
// Per-block compute, two policies:
//  * MFMA (g >= 2): logits as S^T = K Q^T with v_mfma_f32_16x16x32 (16 tokens x
//    16 head slots, zero-padded past g), whose result layout (lane l holds
//    tokens 4*(l/16)+i of head l%16) is exactly the A-operand layout of the PV
//    product O += P V with v_mfma_f32_16x16x16. V rows are loaded coalesced
//    (four full rows per instruction) and transposed into token pairs with
//    v_perm_b32. P is rounded to the storage type for the PV product; the
//    denominator sums the same rounded values.
//  * VALU (g = 1): lanes (rg, c) read 16-byte chunk c of token rows; v_dot2
//    partial dots are summed over the row with DPP; PV accumulates in float32.
//
// Softmax: online normaliser (Milakov & Gimelshein 2018) in base-2 units
// (logit * scale * log2 e). The running reference max moves only when a logit
// exceeds it by more than kLazyRescale, so accumulator rescaling is rare;
// out = acc / l is exact for any reference. Partial states (per lane group,
// per wave, per partition) are merged with the log-sum-exp rule
// (FlashAttention, Dao et al. 2022): M = max m_i, l = sum l_i 2^(m_i - M),
// o = sum o_i 2^(m_i - M) / l, always in a fixed order, so results are
// bitwise reproducible.
#include <type_traits>

#include "attention_mfma.h"
#include "attention_valu.h"
#include "device_common.h"
#include "launch.h"
#include "ordering.h"

namespace mvk {

// Blocks whose loads are in flight per wave. Two keep HBM busy with two
// waves per SIMD; four (measured) only add registers and delay the first
// block's compute.
constexpr int kPrefetch = 2;

struct Shape {
  int32_t num_seqs;
  int32_t num_kv_heads, num_blocks, max_blocks, max_context_len, partition_tokens, num_parts;
  float scale_log2;
  int32_t longest_first; // single-pass grids of <= kMaxOrderedSeqs sequences: (rank, KV head) in dispatch order
};


// Optional fused cache write: row s of new_key/new_value ([S, Hkv, D]) is
// sequence s's token of this step, stored at flat slot slots[s] (negative =
// none). Passed as separate __restrict__ kernel arguments: restrict on struct
// members is not seen, and a possibly-aliased slot would be re-read through
// the vector path with a wait on every load before it.

// ------------------------------------------------------------ one work item
// Attention of sequence s, KV head h over partition `part` (tokens
// [part*P, min((part+1)*P, L))): the final row if the context fits in one
// partition, else this partition's partial state. Every wave of the workgroup
// calls it with the same arguments (it contains a barrier).
template <int DT, int D, int G, int W, int NPF, bool USE_MFMA, bool FUSED, bool SHARED>
__device__ __forceinline__ void decode_item(
    int s, int h, int part, uint16_t* __restrict__ out, float* __restrict__ ws_ml,
    float* __restrict__ ws_o, const uint16_t* __restrict__ q, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const Shape& sh,
    const uint16_t* __restrict__ new_key, const uint16_t* __restrict__ new_value,
    const int32_t* __restrict__ slots, int32_t* __restrict__ counters, float (*sm_o)[G * D],
    float (*sm_m)[G], float (*sm_l)[G], int* sm_last, uint4* sm_nk, uint4* sm_nv) {
  using Policy = typename std::conditional<USE_MFMA, MfmaPolicy<DT, D, G>, ValuPolicy<DT, D, G>>::type;
  using E = Elem<DT>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int P = sh.partition_tokens;
  const int t_begin = part * P;
  const int b_begin = t_begin / kBlockTokens;

  // Prologue: every load it needs (context length, fused slot, this wave's
  // table entries, the query rows, the step's new K/V row) is issued before
  // anything waits on one of them, so together they cost one memory round
  // trip. Lane k takes table entry b_begin + wave + k*W; the row is read only
  // below max_blocks, and entries past the context are never used.
  const int len = context_lens[s];
  int slot = -1;
  if constexpr (FUSED) slot = slots[s];
  const int part_blocks = min(P / kBlockTokens, sh.max_blocks - b_begin);
  const int32_t* table = block_tables + (size_t)s * sh.max_blocks;
  int ent = 0, ent_prev = -1, ent_next = -1;
  if (wave + lane * W < part_blocks) {
    const int e = b_begin + wave + lane * W;
    ent = table[e];
    if constexpr (SHARED) {  // the same logical blocks of the neighbouring sequences
      if (s > 0) ent_prev = table[e - sh.max_blocks];
      if (s + 1 < sh.num_seqs) ent_next = table[e + sh.max_blocks];
    }
  }
  const int Hq = sh.num_kv_heads * G;
  const uint32_t row_bytes = (uint32_t)sh.num_kv_heads * D * 2u;  // one token row of the pool
  const size_t new_src = ((size_t)s * sh.num_kv_heads + h) * D;
  Policy pol;
  pol.init(q, (size_t)s * Hq + (size_t)h * G, lane, row_bytes);
  // The step's new K/V row of this KV head: wave 0 fetches it here and stages
  // it in LDS below, where the block that holds it takes it from (so it does
  // not occupy registers through the block loop).
  uint4 nk16 = make_uint4(0u, 0u, 0u, 0u), nv16 = nk16;
  if constexpr (FUSED) {
    if (wave == 0 && lane < D / 8) {
      nk16 = *(const uint4*)(new_key + new_src + lane * 8);
      nv16 = *(const uint4*)(new_value + new_src + lane * 8);
    }
  }

  const int L = min(len, sh.max_context_len);
  const bool has_new = FUSED && slot >= 0 && slot < sh.num_blocks * kBlockTokens;
  const int blk_new = has_new ? slot / kBlockTokens : -1;
  if constexpr (FUSED) pol.row_new = has_new ? slot % kBlockTokens : -1;
  const size_t new_dst = (size_t)(has_new ? slot : 0) * sh.num_kv_heads * D + (size_t)h * D;
  // the store of record of this KV head's slice: wave 0 of partition 0
  const bool writer = has_new && part == 0 && wave == 0;
  if (t_begin >= L) {  // uniform over the workgroup
    if constexpr (FUSED) {
      if (writer && lane < D / 8) {
        *(uint4*)(k_cache + new_dst + lane * 8) = nk16;
        *(uint4*)(v_cache + new_dst + lane * 8) = nv16;
      }
    }
    if (part == 0) {   // empty context: the row is defined as zeros
      const size_t row0 = ((size_t)s * Hq + (size_t)h * G) * D;
      for (int idx = threadIdx.x; idx < G * D; idx += W * 64) out[row0 + idx] = 0;
    }
    return;
  }
  const int t_end = min(t_begin + P, L);
  const int nblk = (t_end - t_begin + kBlockTokens - 1) / kBlockTokens;
  const int my_blocks = nblk > wave ? (nblk - wave + W - 1) / W : 0;
  const size_t block_bytes = (size_t)row_bytes * kBlockTokens;

  if constexpr (FUSED) {
    if (wave == 0 && lane < D / 8) {
      sm_nk[lane] = nk16;
      sm_nv[lane] = nv16;
    }
  }

  const char* kbase = (const char*)(k_cache + (size_t)h * D);
  const char* vbase = (const char*)(v_cache + (size_t)h * D);
  // NPF fragments in rotation: the loads of the next NPF-1 blocks are in
  // flight while a block is computed, and no register copy of in-flight data
  // is ever needed (the rotation is unrolled, so every fragment index is
  // static). Each block is read through a buffer descriptor covering only its
  // rows that hold context tokens, so rows past the context (any bits, NaN
  // included) read as zeros. Steps past the last block issue their loads
  // through an empty descriptor: they return zeros without touching memory,
  // which keeps the load count of every step the same.
  typename Policy::Frag f[NPF];
  auto tok_of = [&](int k) { return (b_begin + wave + k * W) * kBlockTokens; };
  auto block_of = [&](int k) {
    int blk = __builtin_amdgcn_readlane(ent, min(k, my_blocks - 1));
    return ((unsigned)blk < (unsigned)sh.num_blocks) ? blk : 0;
  };
  uint64_t shared = 0;
  if constexpr (SHARED) shared = shared_blocks(ent, ent_prev, ent_next);
  auto load_block = [&](typename Policy::Frag& fr, int k) {
    const bool real = k < my_blocks;
    const int blk = block_of(k);
    k = min(k, my_blocks - 1);
    const int rows = min(kBlockTokens, t_end - tok_of(k));
    const uint32_t extent = real ? (uint32_t)(rows - 1) * row_bytes + D * 2u : 0u;
    const size_t o = (size_t)blk * block_bytes;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + o, extent), vr = make_rsrc(vbase + o, extent);
    if (SHARED && ((shared >> k) & 1u)) pol.template load<kDefaultLoad>(fr, kr, vr, row_bytes);
    else pol.template load<kStreamLoad>(fr, kr, vr, row_bytes);
  };
  auto is_new = [&](int k) { return FUSED && block_of(k) == blk_new; };
  if (my_blocks > 0) {
#pragma unroll
    for (int j = 0; j < NPF - 1; ++j) load_block(f[j], j);
  }
  if constexpr (FUSED) __syncthreads();  // the new row is in LDS before any block needs it
  if (my_blocks > 0) {
    for (int k0 = 0;; k0 += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        const int k = k0 + j;
        load_block(f[(j + NPF - 1) % NPF], k + NPF - 1);
        pol.process(f[j], tok_of(k), t_end, sh.scale_log2, is_new(k), sm_nk, sm_nv);
        if (k + 1 >= my_blocks) goto blocks_done;
      }
    }
  blocks_done:;
  }
  if constexpr (FUSED) {
    if (writer && lane < D / 8) {   // the store of record
      *(uint4*)(k_cache + new_dst + lane * 8) = sm_nk[lane];
      *(uint4*)(v_cache + new_dst + lane * 8) = sm_nv[lane];
    }
  }
  pol.to_lds(sm_m[wave], sm_l[wave], sm_o[wave]);
  __syncthreads();

  // Merge the waves; write the final row, or this partition's partial state.
  const int parts_of_seq = (L + P - 1) / P;
  for (int idx = threadIdx.x; idx < G * D; idx += W * 64) {
    const int j = idx / D;
    const int d = idx % D;
    float mm = sm_m[0][j];
#pragma unroll
    for (int w = 1; w < W; ++w) mm = fmaxf(mm, sm_m[w][j]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = fast_exp2(sm_m[w][j] - mm);
      lsum = fmaf(sm_l[w][j], f, lsum);
      o = fmaf(sm_o[w][idx], f, o);
    }
    const float r = lsum > 0.0f ? o / lsum : 0.0f;
    const size_t hq = (size_t)s * Hq + (size_t)h * G + j;
    if (parts_of_seq == 1) {
      out[hq * D + d] = E::round(r);
    } else {
      const size_t slot = hq * sh.num_parts + part;
      publish(ws_o + slot * D + d, r);
      if (d == 0) {
        publish(ws_ml + slot * 2, mm);
        publish(ws_ml + slot * 2 + 1, lsum);
      }
    }
  }

  // Several partitions, merged in this launch: each workgroup publishes its
  // partial state and counts itself in; the last of the sequence's partitions
  // to arrive (whichever it is) merges all of them in partition order, so the
  // result does not depend on arrival order, and resets the counter to zero
  // for the next call. No workgroup ever waits for another.
  //
  // Memory ordering. The partial states are written and read only with
  // agent-scope atomic stores and loads (publish / collect: sc1 accesses,
  // coherent across the XCDs' L2s by themselves), so the two halves of a
  // release / acquire pair that the merge needs are done explicitly instead
  // of with agent-scope fences, which would write back or invalidate this
  // XCD's whole L2 and cost more than the merge saves:
  //  * writer: every wave waits for its own publish stores to complete
  //    (s_waitcnt vmcnt(0): a store counts as complete once it is visible at
  //    agent scope), then the barrier, then one thread's counter increment
  //    (an agent-scope atomic read-modify-write). The barrier also keeps the
  //    compiler from moving the increment above the waits. So every store a
  //    workgroup published is visible device-wide before its increment is.
  //  * reader: the workgroup whose increment returns parts - 1 has seen every
  //    other increment of this counter before its own, hence every store
  //    published before them. Its collect loads are issued only after the
  //    increment returned (its value reaches them through LDS, a barrier and
  //    a branch; the GPU does not issue loads speculatively), and as
  //    agent-scope loads they cannot be served from a stale cache line.
  // The counter is reset by that workgroup; the next call is a later kernel,
  // ordered after this one by the stream.
  if (parts_of_seq > 1 && counters != nullptr) {
    int32_t* ctr = counters + (size_t)s * sh.num_kv_heads + h;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int done = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *sm_last = done == parts_of_seq - 1;
    }
    __syncthreads();
    if (*sm_last) {
      for (int idx = threadIdx.x; idx < G * D; idx += W * 64) {
        const int j = idx / D;
        const int d = idx % D;
        const size_t hq = (size_t)s * Hq + (size_t)h * G + j;
        const float* ml = ws_ml + hq * sh.num_parts * 2;
        const float* o = ws_o + hq * sh.num_parts * D + d;
        float mm = -INFINITY;
        for (int p = 0; p < parts_of_seq; ++p) mm = fmaxf(mm, collect(ml + 2 * p));
        float acc = 0.0f, tot = 0.0f;
#pragma unroll 4
        for (int p = 0; p < parts_of_seq; ++p) {
          const float w = collect(ml + 2 * p + 1) * fast_exp2(collect(ml + 2 * p) - mm);
          acc = fmaf(w, collect(o + (size_t)p * D), acc);
          tot += w;
        }
        out[hq * D + d] = E::round(tot > 0.0f ? acc / tot : 0.0f);
      }
      if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------ the kernel
// Grid mode (items == nullptr): grid (S, Hkv, num_parts), one item per
// workgroup; workgroups whose partition starts past their context exit.
// Work-list mode: grid (X, Hkv); the plan kernel has written the count and
// the (sequence, partition) items of all non-empty partitions, and workgroup
// x takes items x, x+X, ... so no workgroup is launched for nothing.
// Waves per SIMD the register allocation must allow. Four (<= 128 VGPRs)
// keep every workgroup of a 1024-workgroup grid of 4-wave groups resident
// at once: at 129 VGPRs the TinyLlama-shaped grid ran a quarter of its
// workgroups as a late second round (79 us instead of 67). The D = 128
// kernels with g >= 2 would spill at 128 and take two (the compiler then
// settles at three for VALU, two for MFMA).
template <int D, int G>
constexpr int kMinWavesPerSimd = (D == 64 || G == 1) ? 4 : 2;

template <int DT, int D, int G, int W, int NPF, bool USE_MFMA, bool FUSED, bool SHARED>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(kMinWavesPerSimd<D, G>))) void paged_decode_partition_kernel(
    uint16_t* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const uint16_t* __restrict__ q, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t* __restrict__ items, Shape sh,
    const uint16_t* __restrict__ new_key, const uint16_t* __restrict__ new_value,
    const int32_t* __restrict__ slots, int32_t* __restrict__ counters) {
  __shared__ float sm_o[W][G * D];
  __shared__ float sm_m[W][G];
  __shared__ float sm_l[W][G];
  __shared__ int sm_last;
  __shared__ int sm_claim;            // work-list mode: the item this workgroup claimed
  __shared__ uint4 sm_new[2][D / 8];  // the step's new K and V row (fused write)
  if (items == nullptr) {
    // Workgroups are dealt round-robin to the 8 XCDs in dispatch order; remap
    // so that each XCD runs a contiguous range of (sequence fastest, then KV
    // head, then partition) items. Sequences that share prefix blocks then
    // read them on the same XCD at about the same time, from its L2.
    const uint32_t n = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t i = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int S = gridDim.x, H = gridDim.y;
    int s, h, part;
    if (sh.longest_first) {
      s = __builtin_amdgcn_readfirstlane(
          sequence_of_rank(context_lens, S, (int)(i / H), sh.max_context_len));
      h = i % H;
      part = 0;
    } else {
      const uint32_t v = xcd_contiguous(i, n);
      s = v % S;
      h = (v / S) % H;
      part = v / (S * H);
    }
    decode_item<DT, D, G, W, NPF, USE_MFMA, FUSED, SHARED>(s, h, part, out, ws_ml, ws_o, q, k_cache, v_cache,
                                               block_tables, context_lens, sh, new_key,
                                               new_value, slots, counters, sm_o, sm_m, sm_l,
                                               &sm_last, sm_new[0], sm_new[1]);
    return;
  }
  // Claim items one at a time through this KV head's dispatch counter; every
  // workgroup stops at its first claim past the end of the list.
  const int count = items[0];
  int32_t* next = items + 1 + blockIdx.y;
  const int32_t* pairs = items + 1 + sh.num_kv_heads;
  for (;;) {
    if (threadIdx.x == 0) sm_claim = atomicAdd(next, 1);
    __syncthreads();
    const int i = sm_claim;
    if (i >= count) break;  // uniform over the workgroup
    const int s = pairs[2 * i];
    const int part = pairs[2 * i + 1];
    decode_item<DT, D, G, W, NPF, USE_MFMA, FUSED, SHARED>(s, blockIdx.y, part, out, ws_ml, ws_o, q, k_cache,
                                               v_cache, block_tables, context_lens, sh, new_key,
                                               new_value, slots, counters, sm_o, sm_m, sm_l,
                                               &sm_last, sm_new[0], sm_new[1]);
    __syncthreads();  // the LDS of this item is read before the next item writes it
  }
}

// Work list for work-list mode: items[0] = count, items[1 .. Hkv] = one
// dispatch counter per KV head (reset here), then (sequence, partition)
// pairs, one per partition that holds context tokens (one partition for an
// empty context, which writes its zero row). Full partitions (every one but
// a sequence's last) come first, then the last partitions, each group in
// sequence order. Workgroups claim items through the counters, so the
// longest items start first and each later item goes to whichever
// workgroup is free (list scheduling). One workgroup of kPlanThreads
// threads: each thread counts both kinds over a contiguous range of
// sequences, workgroup-wide exclusive scans give every thread its two output
// offsets, then each thread writes its own items.
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void paged_decode_plan_kernel(
    int32_t* __restrict__ items, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_kv_heads, int32_t max_context_len, int32_t partition_tokens) {
  __shared__ int32_t sums_full[kPlanThreads];
  __shared__ int32_t sums_last[kPlanThreads];
  const int t = threadIdx.x;
  const int per = (num_seqs + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(t * per, num_seqs);
  const int s1 = min(s0 + per, num_seqs);
  auto parts_of = [&](int s) {
    const int L = min(context_lens[s], max_context_len);
    return L > 0 ? (L + partition_tokens - 1) / partition_tokens : 1;
  };
  int n_full = 0;
  for (int s = s0; s < s1; ++s) n_full += parts_of(s) - 1;
  const int n_last = s1 - s0;
  sums_full[t] = n_full;
  sums_last[t] = n_last;
  __syncthreads();
  // Hillis-Steele inclusive scans over the per-thread counts
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int vf = t >= off ? sums_full[t - off] : 0;
    const int vl = t >= off ? sums_last[t - off] : 0;
    __syncthreads();
    sums_full[t] += vf;
    sums_last[t] += vl;
    __syncthreads();
  }
  const int total_full = sums_full[kPlanThreads - 1];
  int pos_full = sums_full[t] - n_full;
  int pos_last = total_full + sums_last[t] - n_last;
  int32_t* pairs = items + 1 + num_kv_heads;
  for (int s = s0; s < s1; ++s) {
    const int parts = parts_of(s);
    for (int p = 0; p + 1 < parts; ++p, ++pos_full) {
      pairs[2 * pos_full] = s;
      pairs[2 * pos_full + 1] = p;
    }
    pairs[2 * pos_last] = s;
    pairs[2 * pos_last + 1] = parts - 1;
    ++pos_last;
  }
  for (int h = t; h < num_kv_heads; h += kPlanThreads) items[1 + h] = 0;
  if (t == kPlanThreads - 1) items[0] = total_full + sums_last[t];
}

// Merge the partitions of every (sequence, KV head) whose context spans more
// than one partition, for the g query heads of the group. Phase 1: the
// per-partition weights w_p = l_p 2^(m_p - M) and their sum, one thread per
// (head, partition), into LDS. Phase 2: one thread per (head, d) accumulates
// sum_p w_p o_p[d] in partition order, with independent loads in flight.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxParts = 512;  // partitions merged per pass through LDS

template <int DT, int D, int G>
__global__ __launch_bounds__(kMergeThreads) void paged_decode_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, int32_t num_kv_heads, int32_t max_context_len,
    int32_t partition_tokens, int32_t num_parts) {
  using E = Elem<DT>;
  __shared__ float sm_w[G][kMergeMaxParts];
  __shared__ float sm_max[G];
  const int s = blockIdx.y;
  const int h = blockIdx.x;
  const int L = min(context_lens[s], max_context_len);
  const int parts = (L + partition_tokens - 1) / partition_tokens;
  if (parts <= 1) return;  // written directly by the partition kernel
  const int Hq = num_kv_heads * G;
  const size_t hq0 = (size_t)s * Hq + (size_t)h * G;
  const int t = threadIdx.x;

  constexpr int R = (G * D + kMergeThreads - 1) / kMergeThreads;  // outputs per thread
  float acc[R], tot[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = tot[r] = 0.0f;

  // max over the partitions of each head: one wave per head, lanes over p
  for (int j = t / 64; j < G; j += kMergeThreads / 64) {
    const int lane = t % 64;
    const float* ml = ws_ml + (hq0 + j) * num_parts * 2;
    float mm = -INFINITY;
    for (int p = lane; p < parts; p += 64) mm = fmaxf(mm, ml[2 * p]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
    if (lane == 0) sm_max[j] = mm;
  }
  __syncthreads();
  for (int p0 = 0; p0 < parts; p0 += kMergeMaxParts) {
    const int np = min(kMergeMaxParts, parts - p0);
    for (int idx = t; idx < G * np; idx += kMergeThreads) {
      const int j = idx / np, p = p0 + idx % np;
      const float* ml = ws_ml + ((hq0 + j) * num_parts + p) * 2;
      sm_w[j][p - p0] = ml[1] * fast_exp2(ml[0] - sm_max[j]);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = t + r * kMergeThreads;
      if (idx < G * D) {
        const int j = idx / D, d = idx % D;
        const float* o = ws_o + ((hq0 + j) * num_parts + p0) * D + d;
        float a = acc[r], tw = tot[r];
#pragma unroll 8
        for (int p = 0; p < np; ++p) {
          const float w = sm_w[j][p];
          a = fmaf(w, o[(size_t)p * D], a);
          tw += w;
        }
        acc[r] = a;
        tot[r] = tw;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = t + r * kMergeThreads;
    if (idx < G * D) {
      const int j = idx / D, d = idx % D;
      out[(hq0 + j) * D + d] = E::round(tot[r] > 0.0f ? acc[r] / tot[r] : 0.0f);
    }
  }
}

template <int DT, int D, int G, int W, int NPF, bool USE_MFMA, bool FUSED, bool SHARED>
static hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  Shape sh{a.num_seqs, a.num_kv_heads, a.num_blocks, a.max_blocks_per_seq, a.max_context_len,
           a.partition_tokens, a.num_parts, a.scale_log2, a.longest_first};
  dim3 grid((unsigned)a.num_seqs, (unsigned)a.num_kv_heads, (unsigned)a.num_parts);
  if (a.items != nullptr) {
    hipLaunchKernelGGL(paged_decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.items,
                       a.context_lens, a.num_seqs, a.num_kv_heads, a.max_context_len,
                       a.partition_tokens);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    grid = dim3((unsigned)a.list_workgroups, (unsigned)a.num_kv_heads, 1u);
  }
  hipLaunchKernelGGL((paged_decode_partition_kernel<DT, D, G, W, NPF, USE_MFMA, FUSED, SHARED>), grid,
                     dim3(W * 64), 0, stream, (uint16_t*)a.out, a.ws_ml, a.ws_o,
                     (const uint16_t*)a.q, (uint16_t*)a.k_cache, (uint16_t*)a.v_cache,
                     a.block_tables, a.context_lens, a.items, sh,
                     (const uint16_t*)a.new_key, (const uint16_t*)a.new_value, a.slot_mapping,
                     a.counters);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_parts <= 1 || a.counters != nullptr) return err;
  dim3 mgrid((unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((paged_decode_merge_kernel<DT, D, G>), mgrid, dim3(kMergeThreads), 0, stream,
                     (uint16_t*)a.out, a.ws_ml, a.ws_o, a.context_lens, a.num_kv_heads,
                     a.max_context_len, a.partition_tokens, a.num_parts);
  return hipGetLastError();
}

// Blocks shared with a neighbouring sequence are looked for (and kept
// cached) only in the kernels of split long-context grids: the choice
// between two load variants costs the other shapes 4-7 % even when nothing
// is shared, so it is a separate instantiation.
template <int DT, int D, int G, int W, bool MFMA>
static hipError_t launch_shared(const DecodeArgs& a, bool fused, hipStream_t stream) {
  if (a.detect_shared) {
    return fused ? launch_typed<DT, D, G, W, kPrefetch, MFMA, true, true>(a, stream)
                 : launch_typed<DT, D, G, W, kPrefetch, MFMA, false, true>(a, stream);
  }
  return fused ? launch_typed<DT, D, G, W, kPrefetch, MFMA, true, false>(a, stream)
               : launch_typed<DT, D, G, W, kPrefetch, MFMA, false, false>(a, stream);
}

template <int DT, int D, int G>
static hipError_t launch_waves(const DecodeArgs& a, hipStream_t stream) {
  // MFMA from g = 2 on: at g = 2 it takes the Qwen3-shaped call (60 x 8 short
  // contexts, head_dim 128) from 11.54 to 11.15 us on MI355X, and the skewed
  // batch stays within 1 %; a single head (g = 1) would fill 1 of 16 rows.
  constexpr bool kMfma = G >= 2;
  const bool fused = a.new_key != nullptr;
  switch (a.waves) {
    case 4: return launch_shared<DT, D, G, 4, kMfma>(a, fused, stream);
    case 8: return launch_shared<DT, D, G, 8, kMfma>(a, fused, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
static hipError_t launch_group(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_waves<DT, D, 1>(a, stream);
    case 2: return launch_waves<DT, D, 2>(a, stream);
    case 4: return launch_waves<DT, D, 4>(a, stream);
    case 8: return launch_waves<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(int32_t head_dim, int32_t group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (a.dtype == 0) {
    return a.head_dim == 64 ? launch_group<0, 64>(a, group, stream)
                            : launch_group<0, 128>(a, group, stream);
  }
  return a.head_dim == 64 ? launch_group<1, 64>(a, group, stream)
                          : launch_group<1, 128>(a, group, stream);
}

}  // namespace mvk

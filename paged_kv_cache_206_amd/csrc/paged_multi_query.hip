// Multi-query paged attention for gfx950 (CDNA4), wave64: each sequence
// brings n_s >= 1 new query tokens, the last n_s of its context_lens[s] = L
// cached tokens, and new token i (position L - n_s + i) attends causally over
// positions 0 .. L - n_s + i.
//
// Method ("从零手写 vLLM 核心：mini-vllm 项目深度解析", section "推测解码原理"):
// the target model of speculative decoding scores the last accepted token and
// K draft tokens of every sequence in one forward pass; a prefill chunk
// appended to a cached prefix has the same shape. The cache is the paged one
// of the decode kernel (same page, "2. 分页KV缓存（PagedAttention）" and
// "关键工程决策" item 3): 16-token blocks of separate K/V pools
// [num_blocks, 16, Hkv, D] found through per-sequence block tables.
//
// Work decomposition: the n_s * g rows of a (sequence, KV head) - row i*g + j
// is new token i with query head j of the group - are cut into tiles of 16
// rows, one MFMA tile each (attention_mfma.h), and a workgroup takes NT tiles
// (up to 64 rows for D = 64, 32 for D = 128), so that every block it loads
// serves all its rows. One workgroup per (row group, sequence, KV head,
// partition); the partition's blocks are dealt round-robin to its W waves,
// which stream them two at a time as in decode. Row groups beyond the first
// (more rows than one workgroup takes) read the same blocks and are adjacent
// in the XCD-contiguous order, so they read them from the XCD's L2. Each row
// carries its own causal limit, so rows of one tile see different numbers of
// tokens of the same block.
//
// Long contexts: partial (m, l, o) states per (query row, partition) go to
// the workspace and a second kernel merges them with the log-sum-exp rule
// in partition order.
#include "attention_mfma.h"
#include "device_common.h"
#include "launch.h"
#include "ordering.h"

namespace mvk {

namespace {

constexpr int kMqRows = 16;      // query rows per MFMA tile
constexpr int kMqPrefetch = 2;   // blocks whose loads are in flight per wave
constexpr int kMqMergeThreads = 256;

struct MqShape {
  int32_t num_seqs, num_kv_heads, num_blocks, max_blocks, max_context_len, max_query_len;
  int32_t partition_tokens, num_parts, row_groups, num_query_tokens;
  float scale_log2;
  int32_t longest_first;  // single-pass grid dispatched longest sequence first (ordering.h)
};

// Sequence s's query rows [first, first + n): query_start clamped to [0, T]
// and n to max_query_len, so inconsistent offsets never index outside q, out
// or the partial states.
__device__ __forceinline__ void mq_rows(int qs0, int qs1, int num_query_tokens, int max_query_len,
                                        int& first, int& n) {
  first = min(max(qs0, 0), num_query_tokens);
  const int last = min(max(qs1, first), num_query_tokens);
  n = min(last - first, max_query_len);
}
__device__ __forceinline__ void mq_rows(int qs0, int qs1, const MqShape& sh, int& first, int& n) {
  mq_rows(qs0, qs1, sh.num_query_tokens, sh.max_query_len, first, n);
}

// A work item, from the XCD-contiguous item index: row group fastest, then
// sequence, KV head, partition.
struct MqItem {
  int rg, s, h, part;
};

__device__ __forceinline__ MqItem mq_item(uint32_t v, const MqShape& sh) {
  MqItem it;
  it.rg = v % sh.row_groups;
  v /= sh.row_groups;
  it.s = v % sh.num_seqs;
  v /= sh.num_seqs;
  it.h = v % sh.num_kv_heads;
  it.part = v / sh.num_kv_heads;
  return it;
}

// Query row r of a (sequence, KV head) with n new tokens is new token r / G,
// query head h*G + r % G: its index in the [T, Hq] row space.
template <int G>
__device__ __forceinline__ size_t mq_out_row(int first_token, int r, int h, int Hq) {
  return (size_t)(first_token + r / G) * Hq + (size_t)h * G + r % G;
}

// Waves per SIMD the register allocation must allow: each tile's query
// operands and accumulators take about 50 (D = 64) or 100 (D = 128) VGPRs.
template <int D, int NT>
constexpr int kMqMinWavesPerSimd = (D == 64 && NT == 1) ? 4 : 2;

template <int DT, int D, int G, int W, int NT, bool SHARED>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(kMqMinWavesPerSimd<D, NT>)))
void paged_mq_partition_kernel(uint16_t* __restrict__ out, float* __restrict__ ws_ml,
                               float* __restrict__ ws_o, const uint16_t* __restrict__ q,
                               const uint16_t* __restrict__ k_cache,
                               const uint16_t* __restrict__ v_cache,
                               const int32_t* __restrict__ block_tables,
                               const int32_t* __restrict__ context_lens,
                               const int32_t* __restrict__ query_start, MqShape sh) {
  using Policy = MfmaPolicy<DT, D, kMqRows>;
  using E = Elem<DT>;
  constexpr int NPF = kMqPrefetch;
  __shared__ float sm_o[W][kMqRows * D];
  __shared__ float sm_m[W][kMqRows];
  __shared__ float sm_l[W][kMqRows];

  MqItem it;
  if (sh.longest_first) {  // (row group fastest, KV head, sequence rank), one partition
    const uint32_t i = blockIdx.x;
    it.rg = i % sh.row_groups;
    it.h = (i / sh.row_groups) % sh.num_kv_heads;
    it.part = 0;
    it.s = __builtin_amdgcn_readfirstlane(sequence_of_rank(
        context_lens, sh.num_seqs, (int)(i / ((uint32_t)sh.row_groups * sh.num_kv_heads)),
        sh.max_context_len));
  } else {
    it = mq_item(xcd_contiguous(blockIdx.x, gridDim.x), sh);
  }
  const int s = it.s, h = it.h, part = it.part;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int Hq = sh.num_kv_heads * G;
  const int P = sh.partition_tokens;
  const int t_begin = part * P;
  const int b_begin = t_begin / kBlockTokens;

  // Prologue: context length, query range and this wave's table entries
  // (lane k <- block b_begin + wave + k*W) are fetched together.
  const int len = context_lens[s];
  const int qs0 = query_start[s];
  const int qs1 = query_start[s + 1];
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

  const int L = min(len, sh.max_context_len);
  int first, n_new;
  mq_rows(qs0, qs1, sh, first, n_new);
  const int rows = n_new * G;
  const int r0 = it.rg * (NT * kMqRows);
  if (r0 >= rows) return;  // no query rows in this group (uniform over the workgroup)
  const int nrow = min(NT * kMqRows, rows - r0);
  if (t_begin >= L) {      // no context in this partition
    if (part == 0) {       // empty context: every row is zero
      for (int idx = threadIdx.x; idx < nrow * D; idx += W * 64)
        out[mq_out_row<G>(first, r0 + idx / D, h, Hq) * D + idx % D] = 0;
    }
    return;
  }
  const int t_end = min(t_begin + P, L);
  const int nblk = (t_end - t_begin + kBlockTokens - 1) / kBlockTokens;
  const int my_blocks = nblk > wave ? (nblk - wave + W - 1) / W : 0;

  // This lane's row slot in tile t: new token i = r / G sees tokens below
  // L - n + i + 1.
  const uint32_t row_bytes = (uint32_t)sh.num_kv_heads * D * 2u;
  const size_t block_bytes = (size_t)row_bytes * kBlockTokens;
  Policy pol[NT];
  int row_end[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = r0 + t * kMqRows + (lane & 15);
    const bool valid = r < rows;
    pol[t].init_rows(valid ? q + mq_out_row<G>(first, r, h, Hq) * D : nullptr, lane, row_bytes);
    row_end[t] = valid ? min(t_end, L - n_new + r / G + 1) : 0;
  }

  const char* kbase = (const char*)(k_cache + (size_t)h * D);
  const char* vbase = (const char*)(v_cache + (size_t)h * D);
  if (my_blocks > 0) {
    // The decode kernel's streaming: NPF fragments in rotation, each block
    // read through a buffer descriptor that covers only its context rows
    // (rows past the context read as zeros), steps past the last block
    // issuing loads through an empty descriptor.
    typename Policy::Frag f[NPF];
    uint64_t shared = 0;
    if constexpr (SHARED) shared = shared_blocks(ent, ent_prev, ent_next);
    auto tok_of = [&](int k) { return (b_begin + wave + k * W) * kBlockTokens; };
    auto load_block = [&](typename Policy::Frag& fr, int k) {
      const bool real = k < my_blocks;
      k = min(k, my_blocks - 1);
      int blk = __builtin_amdgcn_readlane(ent, k);
      blk = ((unsigned)blk < (unsigned)sh.num_blocks) ? blk : 0;
      const int nrows = min(kBlockTokens, t_end - tok_of(k));
      const uint32_t extent = real ? (uint32_t)(nrows - 1) * row_bytes + D * 2u : 0u;
      const size_t o = (size_t)blk * block_bytes;
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + o, extent), vr = make_rsrc(vbase + o, extent);
      if (SHARED && ((shared >> k) & 1u)) pol[0].template load<kDefaultLoad>(fr, kr, vr, row_bytes);
      else pol[0].template load<kStreamLoad>(fr, kr, vr, row_bytes);
    };
#pragma unroll
    for (int j = 0; j < NPF - 1; ++j) load_block(f[j], j);
    for (int k0 = 0;; k0 += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        const int k = k0 + j;
        load_block(f[(j + NPF - 1) % NPF], k + NPF - 1);
        pol[0].arrange(f[j]);
#pragma unroll
        for (int t = 0; t < NT; ++t) pol[t].step(f[j], tok_of(k), row_end[t], sh.scale_log2);
        if (k + 1 >= my_blocks) goto blocks_done;
      }
    }
  blocks_done:;
  }
  // Merge the waves in order, one tile at a time through LDS; write each
  // row, or its partial state.
  const int parts_of_seq = (L + P - 1) / P;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tr0 = r0 + t * kMqRows;
    const int tnrow = min(kMqRows, rows - tr0);   // uniform: rows of this tile in use
    if (tnrow <= 0) break;
    if (t > 0) __syncthreads();                   // the previous tile's LDS has been read
    pol[t].to_lds(sm_m[wave], sm_l[wave], sm_o[wave]);
    __syncthreads();
    for (int idx = threadIdx.x; idx < tnrow * D; idx += W * 64) {
      const int rl = idx / D;
      const int d = idx % D;
      float mm = sm_m[0][rl];
#pragma unroll
      for (int w = 1; w < W; ++w) mm = fmaxf(mm, sm_m[w][rl]);
      float lsum = 0.0f, o = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float fw = fast_exp2(sm_m[w][rl] - mm);
        lsum = fmaf(sm_l[w][rl], fw, lsum);
        o = fmaf(sm_o[w][rl * D + d], fw, o);
      }
      const float res = lsum > 0.0f ? o / lsum : 0.0f;
      const size_t orow = mq_out_row<G>(first, tr0 + rl, h, Hq);
      if (parts_of_seq == 1) {
        out[orow * D + d] = E::round(res);
      } else {
        const size_t slot = orow * sh.num_parts + part;
        ws_o[slot * D + d] = res;
        if (d == 0) {
          ws_ml[slot * 2] = mm;
          ws_ml[slot * 2 + 1] = lsum;
        }
      }
    }
  }
}

// Workgroups over (row group, sequence, KV head) x chunks of the group's
// outputs, for sequences that span several partitions; each thread merges one
// output element, so all of its partition loads are in flight at once:
// out = sum_p w_p o_p / sum_p w_p with w_p = l_p 2^(m_p - max m), over the
// partitions in index order. A partition that holds none of a row's visible
// tokens has l_p = 0 and weighs nothing.
template <int DT, int D, int G, int NT>
__global__ __launch_bounds__(kMqMergeThreads) void paged_mq_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start,
    MqShape sh) {
  using E = Elem<DT>;
  const MqItem it = mq_item(blockIdx.x, sh);
  const int s = it.s, h = it.h;
  const int L = min(context_lens[s], sh.max_context_len);
  const int P = sh.partition_tokens;
  const int parts = (L + P - 1) / P;
  if (parts <= 1) return;  // the partition kernel wrote these rows
  int first, n_new;
  mq_rows(query_start[s], query_start[s + 1], sh, first, n_new);
  const int rows = n_new * G;
  const int r0 = it.rg * (NT * kMqRows);
  if (r0 >= rows) return;
  const int nrow = min(NT * kMqRows, rows - r0);
  const int Hq = sh.num_kv_heads * G;
  const int idx = blockIdx.y * kMqMergeThreads + threadIdx.x;
  if (idx < nrow * D) {
    const int d = idx % D;
    const size_t orow = mq_out_row<G>(first, r0 + idx / D, h, Hq);
    const float* ml = ws_ml + orow * sh.num_parts * 2;
    const float* o = ws_o + orow * sh.num_parts * D + d;
    // unrolled so that a chunk's loads are in flight together
    float mm = -INFINITY;
#pragma unroll 8
    for (int p = 0; p < parts; ++p) mm = fmaxf(mm, ml[2 * p]);
    float acc = 0.0f, tot = 0.0f;
#pragma unroll 8
    for (int p = 0; p < parts; ++p) {
      const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - mm);
      acc = fmaf(w, o[(size_t)p * D], acc);
      tot += w;
    }
    out[orow * D + d] = E::round(tot > 0.0f ? acc / tot : 0.0f);
  }
}

template <int DT, int D, int G, int W, int NT, bool SHARED>
hipError_t launch_mq_typed(const MultiQueryArgs& a, hipStream_t stream) {
  MqShape sh{a.num_seqs,       a.num_kv_heads,  a.num_blocks,       a.max_blocks_per_seq,
             a.max_context_len, a.max_query_len, a.partition_tokens, a.num_parts,
             a.row_groups,      a.num_query_tokens, a.scale_log2, a.longest_first};
  const int64_t items = (int64_t)a.row_groups * a.num_seqs * a.num_kv_heads * a.num_parts;
  hipLaunchKernelGGL((paged_mq_partition_kernel<DT, D, G, W, NT, SHARED>), dim3((unsigned)items),
                     dim3(W * 64), 0, stream, (uint16_t*)a.out, a.ws_ml, a.ws_o,
                     (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                     (const uint16_t*)a.v_cache, a.block_tables, a.context_lens, a.query_start,
                     sh);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_parts <= 1) return err;
  const int64_t groups = (int64_t)a.row_groups * a.num_seqs * a.num_kv_heads;
  const unsigned chunks = (NT * kMqRows * D + kMqMergeThreads - 1) / kMqMergeThreads;
  hipLaunchKernelGGL((paged_mq_merge_kernel<DT, D, G, NT>), dim3((unsigned)groups, chunks),
                     dim3(kMqMergeThreads), 0, stream, (uint16_t*)a.out, a.ws_ml, a.ws_o,
                     a.context_lens, a.query_start, sh);
  return hipGetLastError();
}

template <int DT, int D, int G, int NT>
hipError_t launch_mq_waves(const MultiQueryArgs& a, hipStream_t stream) {
  switch (a.waves) {
    case 4: return a.detect_shared ? launch_mq_typed<DT, D, G, 4, NT, true>(a, stream)
                                   : launch_mq_typed<DT, D, G, 4, NT, false>(a, stream);
    case 8: return a.detect_shared ? launch_mq_typed<DT, D, G, 8, NT, true>(a, stream)
                                   : launch_mq_typed<DT, D, G, 8, NT, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D, int G>
hipError_t launch_mq_tiles(const MultiQueryArgs& a, hipStream_t stream) {
  switch (a.tiles) {
    case 1: return launch_mq_waves<DT, D, G, 1>(a, stream);
    case 2: return launch_mq_waves<DT, D, G, 2>(a, stream);
    case 4:
      if constexpr (D == 64) return launch_mq_waves<DT, D, G, 4>(a, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_mq_group(const MultiQueryArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_mq_tiles<DT, D, 1>(a, stream);
    case 2: return launch_mq_tiles<DT, D, 2>(a, stream);
    case 4: return launch_mq_tiles<DT, D, 4>(a, stream);
    case 8: return launch_mq_tiles<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------ planned multi-query
// The same rows through a decode plan (paged_decode_planned.hip, one per
// step, built from the step's block tables and context lengths without
// new-token slots), for items of at most 16 query rows (n * g <= 16): the
// plan deals the (sequence, KV head) items to bins of kPlanWaves waves with
// equal block counts and gives every wave a descriptor (item, token run,
// block ids). Each wave streams its blocks once for the n * g rows of its
// item, one 16-row MFMA tile whose rows carry their own causal limits, and
// the item's waves merge through LDS (log-sum-exp rule, waves in order).
// (Items of up to 32 rows in two tiles measured no faster than the unplanned
// kernel: 15.7 against 15.3 us for 12 new tokens on the Qwen3 shape.) A plan
// built with new-token slots is a decode step's: it ends the run of a
// sequence's last wave before the sequence's last position (that step
// computes the token from its new row), so this kernel refuses it by writing
// the item's rows as NaN.
struct MqPlannedShape {
  int32_t num_seqs, num_kv_heads, num_blocks, max_context_len, max_query_len, num_query_tokens;
  int32_t desc_ints;
  float scale_log2;
};

// The plan's bins assume the planned decode kernel's occupancy: two waves
// per SIMD at head_dim 128 with g >= 2 (one bin per CU), four otherwise.
template <int D, int G>
constexpr int kMqPlannedWavesPerSimd = (D == 64 || G == 1) ? 4 : 2;

// Merge of the N waves wb .. wb+N-1 of an item for its rows [0, nrow):
// element (r, d) is sum_w o_w 2^(m_w - M) / sum_w l_w 2^(m_w - M), waves in
// order, M their largest reference.
template <int N, int G, int D, int DT>
__device__ __forceinline__ void mq_merge_item(uint16_t* __restrict__ out,
                                              const float (*sm_o)[kMqRows * D],
                                              const float (*sm_m)[kMqRows],
                                              const float (*sm_l)[kMqRows], int wb, int wave,
                                              int lane, int first, int nrow, int h, int Hq,
                                              bool refuse) {
  using E = Elem<DT>;
  // a lane's elements are idx, idx + 64 N, ...; at head_dim 128 the reads of
  // kBatch of them are issued before any is combined, so the lane waits for
  // LDS once per batch instead of once per element (Qwen3 shape, 5 / 8 new
  // tokens: 11.18 -> 11.03 / 12.40 -> 12.06 us per call); at 64 that measured
  // slightly slower (TinyLlama shape, 2 new tokens: 57.32 -> 57.46 us), so
  // those lanes take one element at a time
  constexpr int kBatch = D == 128 ? (N <= 4 ? 4 : 2) : 1;
  const int total = nrow * D;
  for (int base = (wave - wb) * 64 + lane; base < total; base += kBatch * N * 64) {
    float m[kBatch][N], l[kBatch][N], o[kBatch][N];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      // past the last element a lane reads the last one again and stores nothing
      const int idx = min(base + e * N * 64, total - 1);
      const int rl = idx / D;
      const int d = idx % D;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        m[e][n] = sm_m[wb + n][rl];
        l[e][n] = sm_l[wb + n][rl];
        o[e][n] = sm_o[wb + n][rl * D + d];
      }
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int idx = base + e * N * 64;
      float mm = m[e][0];
#pragma unroll
      for (int n = 1; n < N; ++n) mm = fmaxf(mm, m[e][n]);
      float lsum = 0.0f, acc = 0.0f;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float fct = fast_exp2(m[e][n] - mm);
        lsum = fmaf(l[e][n], fct, lsum);
        acc = fmaf(o[e][n], fct, acc);
      }
      const float res =
          refuse ? __builtin_nanf("") : lsum > 0.0f ? acc * __builtin_amdgcn_rcpf(lsum) : 0.0f;
      if (idx < total) out[mq_out_row<G>(first, idx / D, h, Hq) * D + idx % D] = E::round(res);
    }
  }
}

template <int DT, int D, int G, int W, int NPF>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(
    kMqPlannedWavesPerSimd<D, G>))) void paged_mq_planned_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ query_start,
    MqPlannedShape sh) {
  using Policy = MfmaPolicy<DT, D, kMqRows>;
  __shared__ float sm_o[W][kMqRows * D];
  __shared__ float sm_m[W][kMqRows];
  __shared__ float sm_l[W][kMqRows];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // lane k holds descriptor int k; every field is clamped into range, so an
  // inconsistent plan gives wrong rows but no access outside the buffers
  const int dv = lane < sh.desc_ints ? plan[((size_t)blockIdx.x * W + wave) * sh.desc_ints + lane] : -1;
  const int s_raw = __builtin_amdgcn_readlane(dv, kDescSeq);
  const int h_raw = __builtin_amdgcn_readlane(dv, kDescHead);
  const bool active = s_raw >= 0 && s_raw < sh.num_seqs && h_raw >= 0 && h_raw < sh.num_kv_heads;
  const int s = active ? s_raw : 0;
  const int h = active ? h_raw : 0;
  const int L = min(max(__builtin_amdgcn_readlane(dv, kDescLen), 0), sh.max_context_len);
  const int tb = min(max(__builtin_amdgcn_readlane(dv, kDescTokBegin), 0), L) & ~(kBlockTokens - 1);
  const int te = min(max(__builtin_amdgcn_readlane(dv, kDescTokEnd), tb), L);
  const int nblk =
      active ? min((te - tb + kBlockTokens - 1) / kBlockTokens, sh.desc_ints - kPlanHdrInts) : 0;
  const int wv = __builtin_amdgcn_readlane(dv, kDescWaves);
  const int wb = min(wv & 0xff, W - 1);
  const int wn = min(max((wv >> 8) & 0xff, 1), W - wb);
  const bool in_item = active && wave >= wb && wave < wb + wn;
  const bool refuse = __builtin_amdgcn_readlane(dv, kDescSlot) >= 0;  // a plan with slots

  const int Hq = sh.num_kv_heads * G;
  const uint32_t row_bytes = (uint32_t)sh.num_kv_heads * D * 2u;
  const size_t block_bytes = (size_t)row_bytes * kBlockTokens;
  const char* kbase = (const char*)(k_cache + (size_t)h * D);
  const char* vbase = (const char*)(v_cache + (size_t)h * D);
  Policy pol;
  pol.init_rows(nullptr, lane, row_bytes);  // lane layout, empty state
  int first = 0, n_new = 0;
  if (in_item) {
    typename Policy::Frag f[NPF];
    auto block_of = [&](int k) {
      const int blk = __builtin_amdgcn_readlane(dv, kPlanHdrInts + min(k, max(nblk - 1, 0)));
      return ((unsigned)blk < (unsigned)sh.num_blocks) ? blk : 0;
    };
    // rows of block k past te read as zero; steps past the last block load
    // through an empty descriptor (zeros, no memory access)
    auto load_block = [&](typename Policy::Frag& fr, int k) {
      const bool real = k < nblk;
      const int blk = block_of(k);
      const int kk = min(k, max(nblk - 1, 0));
      const int rows = min(kBlockTokens, te - (tb + kk * kBlockTokens));
      const uint32_t extent = real ? (uint32_t)(rows - 1) * row_bytes + D * 2u : 0u;
      const size_t o = (size_t)blk * block_bytes;
      pol.template load<kStreamLoad>(fr, make_rsrc(kbase + o, extent),
                                     make_rsrc(vbase + o, extent), row_bytes);
    };
    // The K/V stream starts first (it needs only the descriptor); the query
    // rows need the sequence's query offsets, one more round trip.
#pragma unroll
    for (int j = 0; j < NPF; ++j) load_block(f[j], j);
    __builtin_amdgcn_sched_barrier(0);
    mq_rows(query_start[s], query_start[s + 1], sh.num_query_tokens, sh.max_query_len, first,
            n_new);
    // row r = lane % 16 of the item (new token r / G, query head h*G + r % G)
    // sees the tokens below L - n + r/G + 1
    const int r = lane & 15;
    const bool valid = r < n_new * G;
    if (valid) {
      const uint16_t* qr = q + mq_out_row<G>(first, r, h, Hq) * D;
#pragma unroll
      for (int ks = 0; ks < Policy::NKS; ++ks)
        pol.qop[ks] = *(const uint4*)(qr + 32 * ks + 8 * pol.q4);
    }
    const int row_end = valid ? min(te, L - n_new + r / G + 1) : 0;
    auto process = [&](typename Policy::Frag& fr, int tok0) {
      pol.arrange(fr);
      pol.step(fr, tok0, row_end, sh.scale_log2);
    };
    // as in the planned decode: groups of NPF blocks whose refills are all
    // real, then the last one or two groups, which skip the steps and
    // refills past nblk
    int k = 0;
    for (; k + 2 * NPF <= nblk; k += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        process(f[j], tb + (k + j) * kBlockTokens);
        __builtin_amdgcn_sched_barrier(0);
        load_block(f[j], k + j + NPF);
      }
    }
    for (; k < nblk; k += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        if (k + j < nblk) process(f[j], tb + (k + j) * kBlockTokens);
        __builtin_amdgcn_sched_barrier(0);
        if (k + j + NPF < nblk) load_block(f[j], k + j + NPF);
      }
    }
    pol.to_lds(sm_m[wave], sm_l[wave], sm_o[wave]);
  }
  lds_barrier();  // every wave of the workgroup takes part
  const int nrow = min(kMqRows, n_new * G);
  if (!in_item || nrow <= 0) return;
  switch (wn) {
    case 1: mq_merge_item<1, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
    case 2: mq_merge_item<2, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
    case 3: mq_merge_item<3, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
    case 4: mq_merge_item<4, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
    case 5: mq_merge_item<5, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
    case 6: mq_merge_item<6, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
    case 7: mq_merge_item<7, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
    default: mq_merge_item<8, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, first, nrow, h, Hq, refuse); break;
  }
}

// Blocks in flight per wave: three, the planned decode's choice for its MFMA tile.
constexpr int kMqPlannedPrefetch = 3;

template <int DT, int D, int G>
hipError_t launch_mq_planned_typed(const PlannedMultiQueryArgs& a, hipStream_t stream) {
  if constexpr (D == 128 && G == 1) {
    return hipErrorInvalidValue;  // four waves per SIMD leave too few registers
  } else {
    MqPlannedShape sh{a.num_seqs,      a.num_kv_heads,     a.num_blocks, a.max_context_len,
                      a.max_query_len, a.num_query_tokens, a.desc_ints,  a.scale_log2};
    hipLaunchKernelGGL((paged_mq_planned_kernel<DT, D, G, kPlanWaves, kMqPlannedPrefetch>),
                       dim3((unsigned)a.num_bins), dim3(kPlanWaves * 64), 0, stream,
                       (uint16_t*)a.out, (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                       (const uint16_t*)a.v_cache, a.plan, a.query_start, sh);
    return hipGetLastError();
  }
}

template <int DT, int D>
hipError_t launch_mq_planned_group(const PlannedMultiQueryArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_mq_planned_typed<DT, D, 1>(a, stream);
    case 2: return launch_mq_planned_typed<DT, D, 2>(a, stream);
    case 4: return launch_mq_planned_typed<DT, D, 4>(a, stream);
    case 8: return launch_mq_planned_typed<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_paged_multi_query(const MultiQueryArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (a.dtype == 0) {
    return a.head_dim == 64 ? launch_mq_group<0, 64>(a, group, stream)
                            : launch_mq_group<0, 128>(a, group, stream);
  }
  return a.head_dim == 64 ? launch_mq_group<1, 64>(a, group, stream)
                          : launch_mq_group<1, 128>(a, group, stream);
}


hipError_t launch_paged_multi_query_planned(const PlannedMultiQueryArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (a.dtype == 0) {
    return a.head_dim == 64 ? launch_mq_planned_group<0, 64>(a, group, stream)
                            : launch_mq_planned_group<0, 128>(a, group, stream);
  }
  return a.head_dim == 64 ? launch_mq_planned_group<1, 64>(a, group, stream)
                          : launch_mq_planned_group<1, 128>(a, group, stream);
}

}  // namespace mvk

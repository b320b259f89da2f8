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
// the workgroup's waves.
//
// Lane layout inside a wave (16-byte loads, one token row = D*2 bytes):
//   LPR = D/8 lanes cover one token row (8 for D=64, 16 for D=128),
//   RG  = 64/LPR token rows per wave-wide load, TPL = 16/RG loads per block.
// Lane (rg, c) reads chunk c (8 elements) of token rows rg, rg+RG, ... of each
// block, for K and for V: every load instruction reads whole rows, fully
// coalesced. QK partial dots use v_dot2 (two fp16/bf16 products accumulated
// in float32) and are summed over the LPR lanes of a row with DPP.
//
// Softmax: online normaliser (Milakov & Gimelshein 2018) kept per row group,
// in base-2 units (logit * scale * log2 e). The running reference max is only
// moved when a logit exceeds it by more than kLazyRescale, so rescaling of
// the accumulators is rare; out = acc / l is exact for any reference.
// Partial states of the row groups, then of the waves, then of the
// partitions are merged with the log-sum-exp rule (FlashAttention, Dao et
// al. 2022): M = max m_i, l = sum l_i 2^(m_i - M), o = sum o_i 2^(m_i - M) / l.
// Merges run in a fixed order, so results are bitwise reproducible.
#include "device_common.h"
#include "launch.h"

namespace mvk {

constexpr int kWaves = 4;               // waves per workgroup
constexpr float kNegBig = -1.0e30f;     // "no token seen yet" (finite, so 2^(a-b) never sees inf-inf)
constexpr float kLazyRescale = 8.0f;    // let p = 2^(z - m) grow up to 2^8 before rescaling

template <int DT, int D, int G>
__global__ __launch_bounds__(kWaves * 64) void paged_decode_partition_kernel(
    uint16_t* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t num_kv_heads, int32_t num_blocks,
    int32_t max_blocks, int32_t max_context_len, int32_t partition_tokens, int32_t num_parts,
    float scale_log2) {
  using E = Elem<DT>;
  constexpr int LPR = D / 8;
  constexpr int RG = 64 / LPR;
  constexpr int TPL = kBlockTokens / RG;

  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];

  const int part = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rg = lane / LPR;
  const int c = lane % LPR;

  // lengths past the host-side bound are clamped: the table row, the grid and
  // the workspace are all sized from max_context_len (<= max_blocks * 16)
  const int L = min(context_lens[s], max_context_len);
  const int t_begin = part * partition_tokens;
  if (t_begin >= L) {  // whole workgroup leaves together, before any barrier
    if (part == 0) {   // empty context: the row is defined as zeros
      const size_t row0 = ((size_t)s * num_kv_heads * G + (size_t)h * G) * D;
      for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) out[row0 + idx] = 0;
    }
    return;
  }
  const int t_end = min(t_begin + partition_tokens, L);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = (t_end + kBlockTokens - 1) / kBlockTokens;

  const int Hq = num_kv_heads * G;
  const size_t row_stride = (size_t)num_kv_heads * D;  // elements between token rows
  const uint16_t* kbase = k_cache + (size_t)h * D + c * 8;
  const uint16_t* vbase = v_cache + (size_t)h * D + c * 8;
  const int32_t* table = block_tables + (size_t)s * max_blocks;

  uint4 qv[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    qv[j] = *(const uint4*)(q + ((size_t)s * Hq + (size_t)h * G + j) * D + c * 8);

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegBig;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
  }

  for (int b = b_begin + wave; b < b_end; b += kWaves) {
    int blk = table[b];
    blk = ((unsigned)blk < (unsigned)num_blocks) ? blk : 0;
    uint4 kv[TPL], vv[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const size_t row = (size_t)blk * kBlockTokens + i * RG + rg;
      kv[i] = *(const uint4*)(kbase + row * row_stride);
      vv[i] = *(const uint4*)(vbase + row * row_stride);
    }
    const int tok0 = b * kBlockTokens + rg;  // token of load i is tok0 + i*RG
    const bool partial_block = (b + 1) * kBlockTokens > t_end;
    if (partial_block) {
      // rows past the context may hold anything (NaN included): zero the V
      // words so that 0 * garbage never reaches the accumulators
#pragma unroll
      for (int i = 0; i < TPL; ++i)
        if (tok0 + i * RG >= t_end) vv[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    float z[G][TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const bool valid = tok0 + i * RG < t_end;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = E::dot2(qv[j].x, kv[i].x, 0.0f);
        d = E::dot2(qv[j].y, kv[i].y, d);
        d = E::dot2(qv[j].z, kv[i].z, d);
        d = E::dot2(qv[j].w, kv[i].w, d);
        d = group_sum<LPR>(d);
        z[j][i] = valid ? d * scale_log2 : -INFINITY;
      }
    }

#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mx = z[j][0];
#pragma unroll
      for (int i = 1; i < TPL; ++i) mx = fmaxf(mx, z[j][i]);
      if (mx > m[j] + kLazyRescale) {
        const float a = fast_exp2(m[j] - mx);
        l[j] *= a;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] *= a;
        m[j] = mx;
      }
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const float p = fast_exp2(z[j][i] - m[j]);
        l[j] += p;
        const uint32_t w[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[j][2 * e] = fmaf(p, E::lo(w[e]), acc[j][2 * e]);
          acc[j][2 * e + 1] = fmaf(p, E::hi(w[e]), acc[j][2 * e + 1]);
        }
      }
    }
  }

  // Merge the RG row groups of this wave (lanes c, c+LPR, ... hold the same
  // output chunk for different tokens).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = __shfl_xor(m[j], off);
      const float lo = __shfl_xor(l[j], off);
      const float mm = fmaxf(m[j], mo);
      const float a = fast_exp2(m[j] - mm);
      const float bb = fast_exp2(mo - mm);
      l[j] = l[j] * a + lo * bb;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] * a + __shfl_xor(acc[j][e], off) * bb;
      m[j] = mm;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][j][c * 8 + e] = acc[j][e];
      if (c == 0) {
        sm_m[wave][j] = m[j];
        sm_l[wave][j] = l[j];
      }
    }
  }
  __syncthreads();

  // Merge the waves; write the final row, or this partition's partial state.
  const int parts_of_seq = (L + partition_tokens - 1) / partition_tokens;
  for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) {
    const int j = idx / D;
    const int d = idx % D;
    float mm = sm_m[0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][j]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm_m[w][j] - mm);
      lsum = fmaf(sm_l[w][j], f, lsum);
      o = fmaf(sm_acc[w][j][d], f, o);
    }
    const float r = lsum > 0.0f ? o / lsum : 0.0f;
    const size_t hq = (size_t)s * Hq + (size_t)h * G + j;
    if (parts_of_seq == 1) {
      out[hq * D + d] = E::round(r);
    } else {
      const size_t slot = hq * num_parts + part;
      ws_o[slot * D + d] = r;
      if (d == 0) {
        ws_ml[slot * 2] = mm;
        ws_ml[slot * 2 + 1] = lsum;
      }
    }
  }
}

// Merge the partitions of every (sequence, query head) whose context spans
// more than one partition. One thread per output element; partitions are
// combined in index order.
template <int DT, int D>
__global__ __launch_bounds__(256) void paged_decode_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, int32_t num_q_heads, int32_t max_context_len,
    int32_t partition_tokens, int32_t num_parts) {
  using E = Elem<DT>;
  const int s = blockIdx.y;
  const int L = min(context_lens[s], max_context_len);
  const int parts = (L + partition_tokens - 1) / partition_tokens;
  if (parts <= 1) return;  // written directly by the partition kernel
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= num_q_heads * D) return;
  const int j = idx / D;
  const int d = idx % D;
  const size_t hq = (size_t)s * num_q_heads + j;
  const float* ml = ws_ml + hq * num_parts * 2;
  const float* o = ws_o + hq * num_parts * D + d;
  float mm = ml[0];
  for (int p = 1; p < parts; ++p) mm = fmaxf(mm, ml[2 * p]);
  float lsum = 0.0f, acc = 0.0f;
  for (int p = 0; p < parts; ++p) {
    const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - mm);
    lsum += w;
    acc = fmaf(w, o[(size_t)p * D], acc);
  }
  out[hq * D + d] = E::round(lsum > 0.0f ? acc / lsum : 0.0f);
}

template <int DT, int D, int G>
static hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.num_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((paged_decode_partition_kernel<DT, D, G>), grid, dim3(kWaves * 64), 0, stream,
                     (uint16_t*)a.out, a.ws_ml, a.ws_o, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_tables,
                     a.context_lens, a.num_kv_heads, a.num_blocks, a.max_blocks_per_seq,
                     a.max_context_len, a.partition_tokens, a.num_parts, a.scale_log2);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_parts <= 1) return err;
  dim3 mgrid((unsigned)((a.num_q_heads * D + 255) / 256), (unsigned)a.num_seqs);
  hipLaunchKernelGGL((paged_decode_merge_kernel<DT, D>), mgrid, dim3(256), 0, stream,
                     (uint16_t*)a.out, a.ws_ml, a.ws_o, a.context_lens, a.num_q_heads,
                     a.max_context_len, a.partition_tokens, a.num_parts);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_group(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_typed<DT, D, 1>(a, stream);
    case 2: return launch_typed<DT, D, 2>(a, stream);
    case 4: return launch_typed<DT, D, 4>(a, stream);
    case 8: return launch_typed<DT, D, 8>(a, stream);
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

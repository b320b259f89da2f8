// Prefill attention for gfx950 (CDNA4), wave64: causal self-attention of new
// prompts, with the prompts' K/V rows stored into the paged pools in the same
// call.
//
// Method ("从零手写 vLLM 核心：mini-vllm 项目深度解析", section "1. 连续批处理"
// and "关键工程决策" item 2): a request admitted to the batch first runs one
// forward pass over its whole prompt (prefill), after which it decodes one
// token per step against its cache. In that pass token t of a prompt attends
// over the prompt's tokens 0..t, and every token's K/V row goes to the slot
// the block manager gave it (same page, "2. 分页KV缓存（PagedAttention）").
//
// Work decomposition: one workgroup of 4 waves per (64 query tokens, query
// head, prompt); wave w owns 16 of the query tokens, one MFMA tile
// (attention_mfma.h), for the whole pass, so no wave merges with another.
// The workgroup walks the prompt's K/V rows from token 0 up to its last query
// token in tiles of 64 tokens staged in LDS; each wave runs the tile's 16-token
// blocks below its own causal limit through the MFMA tile, with the limit of
// every row (token t sees tokens <= t). The K/V rows come from the new
// key/value tensors (contiguous per prompt), not through the block table:
// they are this pass's own rows. Later query tiles carry more work and are
// dispatched first.
//
// LDS rows are padded to D + 8 elements (D*2 + 16 bytes): a 16-row MFMA
// operand read then touches each of the 64 banks once.
#include "attention_mfma.h"
#include "device_common.h"
#include "launch.h"

namespace mvk {

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfRows = 16 * kPfWaves;  // query tokens per workgroup
constexpr int kPfKvTile = 64;           // K/V tokens per LDS tile

struct PfShape {
  int32_t num_q_heads, num_kv_heads, num_blocks, query_tiles;
  float scale_log2;
};

template <int DT, int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
                    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                    const int32_t* __restrict__ slots, const int32_t* __restrict__ cu_seqlens,
                    PfShape sh) {
  using Policy = MfmaPolicy<DT, D, 16>;
  using E = Elem<DT>;
  constexpr int RH = D + 8;                  // LDS row pitch in 16-bit elements
  constexpr uint32_t kPitch = RH * 2u;       // ... in bytes
  constexpr int kChunks = D / 8;             // 16-byte chunks per row
  constexpr size_t kTileBytes = (size_t)kPfKvTile * RH * 2;
  constexpr size_t kStateBytes = (size_t)kPfWaves * 16 * D * 4;
  constexpr size_t kSmem = 2 * kTileBytes > kStateBytes ? 2 * kTileBytes : kStateBytes;
  // K and V tiles during the pass; each wave's output state after it
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ float sm_m[kPfWaves][16];
  __shared__ float sm_l[kPfWaves][16];
  uint16_t* sk = (uint16_t*)smem;
  uint16_t* sv = (uint16_t*)(smem + kTileBytes);
  float* sm_o = (float*)smem;

  const int s = blockIdx.z;
  const int j = blockIdx.y;                             // query head
  const int qt = sh.query_tiles - 1 - (int)blockIdx.x;  // latest (heaviest) tiles first
  const int lo = cu_seqlens[s];
  const int n = cu_seqlens[s + 1] - lo;
  const int q0 = qt * kPfRows;
  if (q0 >= n) return;  // uniform over the workgroup
  const int h = j / G;
  const int Hq = sh.num_q_heads, Hkv = sh.num_kv_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q_end = min(n, q0 + kPfRows);  // the workgroup's query tokens: [q0, q_end)

  // Cache write: the first query head of each KV head stores this tile's
  // tokens' rows of that KV head (every row exactly once over the grid).
  if (slots != nullptr && j % G == 0) {
    for (int idx = threadIdx.x; idx < (q_end - q0) * kChunks; idx += kPfWaves * 64) {
      const int t = q0 + idx / kChunks;
      const int c = idx % kChunks;
      const int slot = slots[lo + t];
      if (slot >= 0 && slot < sh.num_blocks * kBlockTokens) {
        const size_t src = ((size_t)(lo + t) * Hkv + h) * D + c * 8;
        const size_t dst = ((size_t)slot * Hkv + h) * D + c * 8;
        *(uint4*)(k_cache + dst) = *(const uint4*)(key + src);
        *(uint4*)(v_cache + dst) = *(const uint4*)(value + src);
      }
    }
  }

  // This wave's 16 query tokens; row r16 is token qw0 + r16 and sees tokens
  // below qw0 + r16 + 1.
  const int qw0 = q0 + wave * 16;
  const int r16 = lane & 15;
  const bool valid = qw0 + r16 < n;
  Policy pol;
  pol.init_rows(valid ? q + ((size_t)(lo + qw0 + r16) * Hq + j) * D : nullptr, lane, kPitch);
  const int row_end = valid ? qw0 + r16 + 1 : 0;
  const int wave_end = min(n, qw0 + 16);  // no row of this wave sees past this

  for (int kt0 = 0; kt0 < q_end; kt0 += kPfKvTile) {
    __syncthreads();  // the previous tile has been read
    for (int idx = threadIdx.x; idx < kPfKvTile * kChunks; idx += kPfWaves * 64) {
      const int r = idx / kChunks;
      const int c = idx % kChunks;
      const int t = kt0 + r;
      uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = kk;
      if (t < q_end) {
        const size_t src = ((size_t)(lo + t) * Hkv + h) * D + c * 8;
        kk = *(const uint4*)(key + src);
        vv = *(const uint4*)(value + src);
      }
      *(uint4*)(sk + r * RH + c * 8) = kk;
      *(uint4*)(sv + r * RH + c * 8) = vv;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kPfKvTile / 16; ++b) {
      const int tok0 = kt0 + 16 * b;
      if (tok0 >= wave_end) break;  // uniform over the wave
      typename Policy::Frag f;
      pol.load_lds(f, (const char*)(sk + 16 * b * RH), (const char*)(sv + 16 * b * RH), kPitch);
      pol.step(f, tok0, row_end, sh.scale_log2);
    }
  }

  // Each wave normalises and writes its own rows.
  __syncthreads();  // the last tile has been read: the LDS takes the states
  pol.to_lds(sm_m[wave], sm_l[wave], sm_o + (size_t)wave * 16 * D);
  __syncthreads();
  const float* so = sm_o + (size_t)wave * 16 * D;
  for (int idx = lane; idx < 16 * D; idx += 64) {
    const int rl = idx / D;
    const int d = idx % D;
    if (qw0 + rl >= n) break;  // rows are in order: the rest are past the prompt
    const float l = sm_l[wave][rl];
    out[((size_t)(lo + qw0 + rl) * Hq + j) * D + d] = E::round(l > 0.0f ? so[idx] / l : 0.0f);
  }
}

template <int DT, int D, int G>
hipError_t launch_prefill_typed(const PrefillArgs& a, hipStream_t stream) {
  PfShape sh{a.num_q_heads, a.num_kv_heads, a.num_blocks,
             (a.max_seqlen + kPfRows - 1) / kPfRows, a.scale_log2};
  dim3 grid((unsigned)sh.query_tiles, (unsigned)a.num_q_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((prefill_kernel<DT, D, G>), grid, dim3(kPfWaves * 64), 0, stream,
                     (uint16_t*)a.out, (const uint16_t*)a.q, (const uint16_t*)a.key,
                     (const uint16_t*)a.value, (uint16_t*)a.k_cache, (uint16_t*)a.v_cache,
                     a.slot_mapping, a.cu_seqlens, sh);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_prefill_group(const PrefillArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefill_typed<DT, D, 1>(a, stream);
    case 2: return launch_prefill_typed<DT, D, 2>(a, stream);
    case 4: return launch_prefill_typed<DT, D, 4>(a, stream);
    case 8: return launch_prefill_typed<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int32_t prefill_rows_per_workgroup() { return kPfRows; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (a.dtype == 0) {
    return a.head_dim == 64 ? launch_prefill_group<0, 64>(a, group, stream)
                            : launch_prefill_group<0, 128>(a, group, stream);
  }
  return a.head_dim == 64 ? launch_prefill_group<1, 64>(a, group, stream)
                          : launch_prefill_group<1, 128>(a, group, stream);
}

}  // namespace mvk

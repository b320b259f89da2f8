// Longest-first dispatch order for single-pass grids (decode and
// multi-query kernels, gfx950).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace mvk {

// A single-pass grid (one partition per sequence) is dispatched longest
// sequence first: dispatch index i serves KV head i % Hkv (decode; the
// multi-query kernel puts its row groups fastest) of the sequence of rank
// i / Hkv, ranked by block count (descending), ties by index
// (ascending). The workgroups are dealt round-robin to the XCDs and, within
// an XCD, to its CUs, so every CU receives a long item with a short one and
// every XCD the same mix; with the sequences in batch order a CU could get
// two long items while another got two short ones. Measured on MI355X with
// the batch sorted by the caller (no ranking in the kernel): 60 x 8 items of
// 4-16 blocks 11.18 -> 10.4 us, 256 x 4 items of 32-128 blocks 70.5 ->
// 66.8 us. Ranking in the kernel adds a memory round trip to the start of
// every workgroup, which only the long items repay (the planner's choice).
constexpr int kOrderKeys = kMaxOrderedSeqs / 64;  // keys per lane

// The sequence of rank r: a radix select over unique 32-bit keys (block count
// in the high bits, S - 1 - s in the low bits, so a larger key ranks first)
// that every wave runs on its own, with ballots and scalar counts only: no
// LDS, no barrier, the same answer in every wave and workgroup.
__device__ __forceinline__ int sequence_of_rank(const int32_t* __restrict__ context_lens, int S, int r,
                                                int max_context_len) {
  const int lane = threadIdx.x & 63;
  const int idx_bits = 32 - __builtin_clz((unsigned)max(S - 1, 1));
  const int max_blocks = (max_context_len + kBlockTokens - 1) / kBlockTokens;
  const int blk_bits = 32 - __builtin_clz((unsigned)max(max_blocks, 1));
  const int nk = (S + 63) / 64;  // key slots in use (uniform)
  // Every lane loads all its lengths at once (indexes clamped into the batch,
  // so no load is conditional and one wait covers them all).
  int Lraw[kOrderKeys];
#pragma unroll
  for (int k = 0; k < kOrderKeys; ++k) Lraw[k] = context_lens[min(lane + 64 * k, S - 1)];
  uint32_t key[kOrderKeys];
  bool valid[kOrderKeys];
#pragma unroll
  for (int k = 0; k < kOrderKeys; ++k) {
    const int s = lane + 64 * k;
    valid[k] = s < S;
    const int L = valid[k] ? min(max(Lraw[k], 0), max_context_len) : 0;
    key[k] = ((uint32_t)((L + kBlockTokens - 1) / kBlockTokens) << idx_bits) |
             (uint32_t)(valid[k] ? S - 1 - s : 0);
  }
  uint32_t prefix = 0;
  int rem = r;
  for (int b = idx_bits + blk_bits - 1; b >= 0; --b) {  // uniform loop
    const uint32_t want = (prefix | (1u << b)) >> b;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kOrderKeys; ++k) {
      if (k < nk) cnt += __builtin_popcountll(__ballot(valid[k] && (key[k] >> b) == want));
    }
    if (rem < cnt) prefix |= 1u << b;
    else rem -= cnt;
  }
  return S - 1 - (int)(prefix & ((1u << idx_bits) - 1u));
}

}  // namespace mvk

// Planned paged-attention decode for gfx950 (CDNA4), wave64: the work of a
// decode step is laid out once per step (a plan), and every layer's decode
// call of that step reads it.
//
// Method (mini-vllm write-up, "2. 分页KV缓存（PagedAttention）" and
// "关键工程决策" items 1-3): every running sequence's single new query token
// attends over its cached context, read block by block through its block
// table; in steady state all running sequences form one batched decode step,
// and every layer of the model runs that same step over its own pools with
// the same block tables and lengths. The plan exploits exactly that: the
// tables and lengths are read, ranked and dealt out once per step instead of
// once per layer.
//
// Work decomposition (single pass: every (sequence, KV head) item is done by
// one workgroup, so no partial state leaves the workgroup):
//  * The plan kernel ranks the sequences by block count (longest first, ties
//    by index) and deals the items (rank-major, KV head fastest) to B bins
//    in boustrophedon rounds: round k gives item k*B + p to bin p on even
//    rounds and to bin B-1-p on odd ones, so each bin pairs long items with
//    short ones and all bins carry about the same number of blocks.
//  * A bin is one workgroup of W waves. Its waves are split over its items
//    to keep the largest number of blocks any wave streams small (greedy:
//    each item gets the waves its descriptors need, then every spare wave
//    goes to the item whose waves carry the most blocks each), and each wave
//    takes a contiguous run of its item's blocks.
//  * Each wave's work is one descriptor: sequence, KV head, token range,
//    the sequence's new-token slot and context length, its item's wave
//    range, and the physical ids of its blocks (copied from the block
//    table); 32 ints (one 128-byte line, up to 24 blocks) when no sequence
//    has more blocks, 64 otherwise. The decode kernel's wave fetches it with
//    one load, so K/V loads start after a single round trip, and no wave
//    ranks or searches anything.
//  * The waves of an item merge their online-softmax states through LDS
//    (log-sum-exp rule, fixed order) and write the item's rows.
// Per-block compute is the MFMA tile (g >= 2) or the VALU policy (g = 1).
// The fused cache write costs the block loop nothing: in a decode step the
// new token is the sequence's last position, so the wave holding the last
// block reads the blocks up to the token before it (the buffer descriptor
// ends there, so the slot's old bits are never read); that wave starts its
// online-softmax state from the new row, taken as the first token while its
// block loads are in flight, and stores the row. A slot elsewhere in the item's blocks
// is stored first by the wave that reads that block, which waits for the
// store before its loads; a sequence appends only into its own blocks, which
// no other sequence reads (the paged allocator's rule), so no other wave
// depends on the store.
#include <type_traits>

#include "attention_mfma.h"
#include "attention_valu.h"
#include "device_common.h"
#include "launch.h"

namespace mvk {

namespace {

// Descriptor fields: kDesc* (launch.h); the rest (24 or 56 ints) are block ids.

// Parts in the fused cache write (descriptor int kDescFlags), set by the plan
// per item: when the new slot is the sequence's position L-1 (a decode
// step's own token), the wave holding the last block stops before it,
// starts its state from the new row (append), and stores it; when the slot is in one of the item's other blocks, the wave holding
// that block stores the row first and reads its blocks after the store has
// completed (store first); otherwise the item's first wave stores it.
enum : int { kFlagAppend = 1, kFlagStore = 2, kFlagStoreFirst = 4 };

constexpr int kBinThreads = 512;

template <int D, int G>
constexpr int kPlannedWavesPerSimd = (D == 64 || G == 1) ? 4 : 2;

struct PlannedShape {
  int32_t num_seqs, num_kv_heads, num_blocks, max_context_len;
  int32_t desc_ints;  // kPlanShortDescInts or kPlanDescInts
  float scale_log2;
};

// Merge of the N waves wb .. wb+N-1 of an item (N known at compile time, so
// only their LDS slots are read and every loop unrolls): element (j, d) of
// the item's g x D outputs is sum_w o_w 2^(m_w - M) / sum_w l_w 2^(m_w - M),
// waves in order, M their largest reference; the division is one reciprocal
// of the denominator (the output is rounded to 16 bits). Lane x of the
// item's waves takes elements x, x + 64 N, ...: with fewer than g D / 64
// waves a lane has several, and all of their reads are issued before any is
// combined, so the lane waits for LDS once instead of once per element.
template <int N, int W, int G, int D, int DT>
__device__ __forceinline__ void merge_item(uint16_t* __restrict__ out, const float (*sm_o)[G * D],
                                           const float (*sm_m)[G], const float (*sm_l)[G], int wb,
                                           int wave, int lane, int s, int h, int Hq) {
  using E = Elem<DT>;
  constexpr int kPer = (G * D + N * 64 - 1) / (N * 64);  // elements per lane, at most
  const int first = (wave - wb) * 64 + lane;
  if ((wave - wb) * 64 >= G * D) return;  // a wave with no elements (uniform)
  float m[kPer][N], l[kPer][N], o[kPer][N];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    // past the last element a lane reads the last one again and stores nothing
    const int idx = min(first + e * N * 64, G * D - 1);
    const int j = idx / D;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      m[e][n] = sm_m[wb + n][j];
      l[e][n] = sm_l[wb + n][j];
      o[e][n] = sm_o[wb + n][idx];
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = first + e * N * 64;
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
    if (idx < G * D)
      out[((size_t)s * Hq + (size_t)h * G) * D + idx] =
          E::round(lsum > 0.0f ? acc * __builtin_amdgcn_rcpf(lsum) : 0.0f);
  }
}

template <int DT, int D, int G, int W, int NPF, bool USE_MFMA, bool FUSED>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(
    kPlannedWavesPerSimd<D, G>))) void paged_decode_planned_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, const int32_t* __restrict__ plan, PlannedShape sh,
    const uint16_t* __restrict__ new_key, const uint16_t* __restrict__ new_value) {
  using Policy =
      typename std::conditional<USE_MFMA, MfmaPolicy<DT, D, G>, ValuPolicy<DT, D, G>>::type;
  __shared__ float sm_o[W][G * D];
  __shared__ float sm_m[W][G];
  __shared__ float sm_l[W][G];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // lane k holds descriptor int k (lanes past a short descriptor load nothing)
  const int dv = lane < sh.desc_ints ? plan[((size_t)blockIdx.x * W + wave) * sh.desc_ints + lane] : -1;
  const int s_raw = __builtin_amdgcn_readlane(dv, kDescSeq);
  const int h_raw = __builtin_amdgcn_readlane(dv, kDescHead);
  // every field is clamped into range, so an inconsistent plan gives wrong
  // rows but no access outside the buffers
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

  const int Hq = sh.num_kv_heads * G;
  const uint32_t row_bytes = (uint32_t)sh.num_kv_heads * D * 2u;
  const size_t block_bytes = (size_t)row_bytes * kBlockTokens;
  Policy pol;
  int slot = -1, flags = 0;
  if constexpr (FUSED) {
    slot = __builtin_amdgcn_readlane(dv, kDescSlot);
    flags = __builtin_amdgcn_readlane(dv, kDescFlags);
  }
  const bool has_new = FUSED && in_item && slot >= 0 && slot < sh.num_blocks * kBlockTokens;
  const bool append = has_new && (flags & kFlagAppend);
  const bool store = has_new && (flags & (kFlagStore | kFlagStoreFirst));
  const bool store_first = has_new && (flags & kFlagStoreFirst);
  const size_t new_dst = (size_t)(has_new ? slot : 0) * sh.num_kv_heads * D + (size_t)h * D;

  const char* kbase = (const char*)(k_cache + (size_t)h * D);
  const char* vbase = (const char*)(v_cache + (size_t)h * D);
  typename Policy::Frag f[NPF];
  auto block_of = [&](int k) {
    const int blk = __builtin_amdgcn_readlane(dv, kPlanHdrInts + min(k, max(nblk - 1, 0)));
    return ((unsigned)blk < (unsigned)sh.num_blocks) ? blk : 0;
  };
  // Rows of block k that hold context tokens are read through its buffer
  // descriptor; rows past te read as zero, and steps past the last block
  // load through an empty descriptor (zeros, no memory access).
  auto load_block = [&](typename Policy::Frag& fr, int k) {
    const bool real = k < nblk;
    const int blk = block_of(k);
    const int kk = min(k, max(nblk - 1, 0));
    const int rows = min(kBlockTokens, te - (tb + kk * kBlockTokens));
    const uint32_t extent = real ? (uint32_t)(rows - 1) * row_bytes + D * 2u : 0u;
    const size_t o = (size_t)blk * block_bytes;
    pol.template load<kStreamLoad>(fr, make_rsrc(kbase + o, extent), make_rsrc(vbase + o, extent),
                                   row_bytes);
  };

  if (in_item) {
    pol.init(q, (size_t)s * Hq + (size_t)h * G, lane, row_bytes);
    if constexpr (FUSED) {
      if (append || store) {
        const size_t src = ((size_t)s * sh.num_kv_heads + h) * D;
        pol.load_new_row(new_key + src, new_value + src);
      }
      if (store_first) {
        // the slot lies in one of this wave's blocks: store the row, and let
        // the block loads below start only once the store has completed
        pol.store_new_row(k_cache + new_dst, v_cache + new_dst);
        __builtin_amdgcn_s_waitcnt(0);
      }
    }
    // Loads complete in issue order: the query and new-row loads go out
    // before the K/V stream, so the first block is computed as soon as it
    // lands instead of after the blocks issued ahead of a late query load.
    __builtin_amdgcn_sched_barrier(0);
    // NPF blocks in flight from here on (empty descriptors past the last
    // block): block k's buffer is refilled with block k + NPF right after
    // block k is computed.
#pragma unroll
    for (int j = 0; j < NPF; ++j) load_block(f[j], j);
    if constexpr (FUSED) {
      // The new token enters the state before any block (it waits only for
      // the query and new-row loads, while the block loads are in flight),
      // and its row is stored at once: no wave of this item reads its slot.
      if (append) pol.seed_row(sh.scale_log2);
      if (store && !store_first) pol.store_new_row(k_cache + new_dst, v_cache + new_dst);
    }
    // Steady state: groups of NPF blocks whose refills are all real blocks,
    // with no branch around a load, so every path keeps the same loads in
    // flight and each block waits only for its own. Then the last one or two
    // groups, which skip the steps and refills past nblk (their waits are
    // coarser, but a short run gains more from issuing no empty loads).
    int k = 0;
    for (; k + 2 * NPF <= nblk; k += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        pol.process_plain(f[j], tb + (k + j) * kBlockTokens, te, sh.scale_log2);
        // the refill stays behind the block's last reads, so it reuses the
        // block's registers instead of alternating between two sets
        __builtin_amdgcn_sched_barrier(0);
        load_block(f[j], k + j + NPF);
      }
    }
    for (; k < nblk; k += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        if (k + j < nblk) pol.process_plain(f[j], tb + (k + j) * kBlockTokens, te, sh.scale_log2);
        __builtin_amdgcn_sched_barrier(0);
        if (k + j + NPF < nblk) load_block(f[j], k + j + NPF);
      }
    }
  }
  if (in_item) pol.to_lds(sm_m[wave], sm_l[wave], sm_o[wave]);
  lds_barrier();  // the writer's pool stores and any other global traffic stay in flight
  if (!in_item) return;

  // The item's waves merge their states (log-sum-exp rule, waves in order)
  // and write its g output rows; an empty context gives zeros.
  switch (wn) {
    case 1: merge_item<1, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
    case 2: merge_item<2, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
    case 3: merge_item<3, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
    case 4: merge_item<4, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
    case 5: merge_item<5, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
    case 6: merge_item<6, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
    case 7: merge_item<7, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
    default: merge_item<8, W, G, D, DT>(out, sm_o, sm_m, sm_l, wb, wave, lane, s, h, Hq); break;
  }
}

// One workgroup per bin. Every workgroup ranks the whole batch in LDS (at
// most kPlanMaxSeqs sequences), assembles its own bin and writes its W
// descriptors; workgroups do not communicate.
struct BinShape {
  int32_t num_seqs, num_kv_heads, max_blocks, max_context_len, num_bins;
  int32_t desc_ints;  // kPlanShortDescInts or kPlanDescInts
  // reciprocals rounded up, ceil(2^32 / d), for divisions as a multiply-high
  // (exact for n / d while n * d < 2^32): d = num_kv_heads (0 when it is
  // one, whose reciprocal does not fit in 32 bits) and d = the block ids a
  // descriptor holds
  uint32_t kv_rcp, ids_rcp;
};
static_assert((uint64_t)kPlanMaxSeqs * kPlanMaxKvHeads * kPlanMaxKvHeads < (1ull << 32),
              "the plan's multiply-high division needs i * num_kv_heads < 2^32");

template <int W>
__global__ __launch_bounds__(kBinThreads) void paged_decode_plan_bins_kernel(
    int32_t* __restrict__ plan, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ slots, BinShape ps) {
  __shared__ int32_t nblk[kPlanMaxSeqs];
  __shared__ int32_t lens[kPlanMaxSeqs];
  __shared__ int32_t slot_of[kPlanMaxSeqs];
  __shared__ int32_t appends[kPlanMaxSeqs];  // the slot is the sequence's position L-1
  __shared__ __attribute__((aligned(16))) int32_t keys[kPlanMaxSeqs];
  __shared__ int32_t rank_of[kPlanMaxSeqs];
  __shared__ int32_t seq_of_rank[kPlanMaxSeqs];
  __shared__ int32_t hdr[W][kPlanHdrInts];
  __shared__ int32_t holds[W];  // the wave's blocks include its item's new slot (not at L-1)
  static_assert(W * W <= 64 && kBinThreads >= 64, "one lane per spare-wave candidate in wave 0");
  const int t = threadIdx.x;
  const int S = ps.num_seqs;
  if (t < W) holds[t] = 0;
  const int S4 = (S + 3) & ~3;
  // Each thread's sequences (at most kPlanMaxSeqs / kBinThreads): the block
  // that holds position L-1 is loaded here and compared only after the
  // ranking, so that load's round trip overlaps the LDS work (the barriers
  // below order LDS only and leave global loads in flight).
  constexpr int kPer = kPlanMaxSeqs / kBinThreads;
  int tail_blk[kPer], tail_slot[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int s = t + r * kBinThreads;
    tail_blk[r] = -1;
    tail_slot[r] = -1;
    if (s >= S4) continue;
    int key = -1;  // padding: never larger than a real key
    if (s < S) {
      const int L = min(max(context_lens[s], 0), ps.max_context_len);
      const int nb = (L + kBlockTokens - 1) / kBlockTokens;
      const int slot = slots != nullptr ? slots[s] : -1;
      lens[s] = L;
      nblk[s] = nb;
      slot_of[s] = slot;
      rank_of[s] = 0;
      if (L > 0 && slot >= 0) {
        tail_blk[r] = block_tables[(size_t)s * ps.max_blocks + (L - 1) / kBlockTokens];
        tail_slot[r] = (L - 1) % kBlockTokens;
      }
      // unique key, larger = earlier: more blocks first, then lower index
      key = (nb << 10) | (kPlanMaxSeqs - 1 - s);
    }
    keys[s] = key;
  }
  lds_barrier();
  // rank = number of larger keys (a permutation of 0..S-1). Sequence s gets
  // P = kBinThreads / S threads (at least one), each counting over its slice of the
  // keys four at a time; the slices' counts meet in LDS.
  {
    const int P = S <= kBinThreads ? kBinThreads / S : 1;
    const int chunks = S4 / 4;
    const int per = (chunks + P - 1) / P;  // 4-key chunks per slice
    for (int w = t; w < S * P; w += kBinThreads) {
      const int s = w / P, p = w % P;
      const int mine = keys[s];
      const int c1 = min(chunks, (p + 1) * per);
      int cnt = 0;
#pragma unroll 8
      for (int c = p * per; c < c1; ++c) {
        const int4 k4 = *(const int4*)(keys + 4 * c);
        cnt += (k4.x > mine) + (k4.y > mine) + (k4.z > mine) + (k4.w > mine);
      }
      if (cnt) atomicAdd(&rank_of[s], cnt);
    }
  }
  lds_barrier();
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int s = t + r * kBinThreads;
    if (s < S) {
      seq_of_rank[rank_of[s]] = s;
      // the slot is the sequence's position L-1
      appends[s] = tail_blk[r] >= 0 && slot_of[s] == tail_blk[r] * kBlockTokens + tail_slot[r];
    }
  }
  lds_barrier();
  if (t < 64) {
    // Wave 0 assembles the bin and lanes t < W write the header of wave t.
    // Lane k < W looks up item slot k: round k's item, present when that
    // round reaches this bin (the present slots are a prefix).
    const int N = S * ps.num_kv_heads;
    const int B = ps.num_bins;
    const int max_ids = ps.desc_ints - kPlanHdrInts;  // block ids a descriptor holds
    const int b = blockIdx.x;
    // i / num_kv_heads as a multiply-high: exact, since i * hkv < 2^32 for
    // i < kPlanMaxSeqs * kPlanMaxKvHeads
    const uint32_t hkv = (uint32_t)ps.num_kv_heads;
    int s = 0, h = 0, nb = 0, w0 = 0;
    {
      const int i = t * B + ((t & 1) ? B - 1 - b : b);
      if (t < W && t * B < N && i < N) {
        const int r = hkv > 1u ? (int)__umulhi((uint32_t)i, ps.kv_rcp) : i;
        s = seq_of_rank[r];
        h = i - r * (int)hkv;
        nb = nblk[s];
        // every item gets the waves its descriptors need (at least one)
        w0 = max(1, (int)__umulhi((uint32_t)(nb + max_ids - 1), ps.ids_rcp));
      }
    }
    int used = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) used += __builtin_amdgcn_readlane(w0, k);
    const int spare = W - used;  // the host sizes the bins so that used <= W
    const int items = __popcll(__ballot(t < W && w0 > 0));  // the present slots, a prefix
    // The spare waves go one at a time to the item whose waves carry the
    // most blocks each (the first such item on ties). Item k's j-th spare
    // wave would be taken at a load of nb_k / (w0_k + j) blocks per wave,
    // which falls as j grows, so these steps take exactly the `spare`
    // largest candidates (k, j), ordered by that load, then k, then j. Lane
    // k * W + j holds candidate (k, j) and counts the larger ones among the
    // items * spare candidates (at most 16: each item takes a wave). A load is
    // compared as nb * (420 / waves): an exact integer, since every wave
    // count a candidate has (1 .. W - 1) divides 420; the quotients are
    // packed 9 bits each into one constant.
    static_assert(W <= 8, "420 / waves covers wave counts up to 7");
    constexpr uint64_t kPer420 = 420ull | 210ull << 9 | 140ull << 18 | 105ull << 27 |
                                 84ull << 36 | 70ull << 45 | 60ull << 54;
    const int kc = t / W, jc = t % W;
    const int nbc = __shfl(nb, kc), w0c = __shfl(w0, kc);
    const int den = min(max(w0c + jc, 1), 7);
    const int per420 = (int)((kPer420 >> (9 * (den - 1))) & 511u);
    const bool cand = w0c > 0 && jc < spare;
    const int key = cand ? ((nbc * per420) << 6) | (63 - t) : -1;  // unique, larger = earlier
    int above = 0;
    for (int k2 = 0; k2 < items; ++k2) {
      for (int j2 = 0; j2 < spare; ++j2) above += __builtin_amdgcn_readlane(key, k2 * W + j2) > key;
    }
    const uint64_t taken = __ballot(cand && above < spare);
    // lane k < W: item k's wave count
    const int iw = w0 + __popcll((taken >> ((t % W) * W)) & ((1ull << W) - 1));
    // wave t's item: items take consecutive waves in slot order
    int wb = 0, item = -1, is = 0, ih = 0, inb = 0, wn = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int iwk = __builtin_amdgcn_readlane(iw, k);
      const int sk = __builtin_amdgcn_readlane(s, k);
      const int hk = __builtin_amdgcn_readlane(h, k);
      const int nbk = __builtin_amdgcn_readlane(nb, k);
      const bool mine = item < 0 && iwk > 0 && t < wb + iwk;
      if (mine) {
        item = k;
        is = sk;
        ih = hk;
        inb = nbk;
        wn = iwk;
      }
      if (item < 0) wb += iwk;
    }
    if (t < W) {
      int* hw = hdr[t];
      if (item < 0) {
#pragma unroll
        for (int k = 0; k < kPlanHdrInts; ++k) hw[k] = 0;
        hw[kDescSeq] = -1;
      } else {
        const int x = t - wb;
        const int b0 = (int)((uint32_t)(x * inb) / (uint32_t)wn);
        const int b1 = (int)((uint32_t)((x + 1) * inb) / (uint32_t)wn);
        const bool last = x == wn - 1;
        const bool app = appends[is] != 0;
        hw[kDescSeq] = is;
        hw[kDescHead] = ih;
        hw[kDescTokBegin] = b0 * kBlockTokens;
        // the append wave's blocks end before the new token
        hw[kDescTokEnd] = min(b1 * kBlockTokens, lens[is] - (app && last ? 1 : 0));
        hw[kDescSlot] = slot_of[is];
        hw[kDescWaves] = wb | (wn << 8);
        hw[kDescLen] = lens[is];
        // provisional: the store-first holder, if any, is found below
        hw[kDescFlags] = slot_of[is] < 0 ? 0
                         : app ? (last ? kFlagAppend | kFlagStore : 0)
                               : (x == 0 ? kFlagStore : 0);
      }
    }
  }
  lds_barrier();
  // block ids; a wave whose blocks include its item's new slot (when that is
  // not the append case) is marked as the store-first holder
  const int dn = ps.desc_ints;
  int32_t* desc = plan + (size_t)blockIdx.x * W * dn;
  for (int idx = t; idx < W * dn; idx += kBinThreads) {
    const int w = idx / dn;
    const int k = idx % dn;
    if (k < kPlanHdrInts) continue;
    const int s = hdr[w][kDescSeq];
    const int tb = hdr[w][kDescTokBegin];
    const int n = s >= 0 ? max(hdr[w][kDescTokEnd] - tb + kBlockTokens - 1, 0) / kBlockTokens : 0;
    const int j = k - kPlanHdrInts;
    const int v = j < n ? block_tables[(size_t)s * ps.max_blocks + tb / kBlockTokens + j] : -1;
    if (j < n && slot_of[s] >= 0 && !appends[s] && v == slot_of[s] / kBlockTokens) holds[w] = 1;
    desc[idx] = v;
  }
  lds_barrier();
  if (t < W) {
    int flags = hdr[t][kDescFlags];
    const int s = hdr[t][kDescSeq];
    if (s >= 0 && slot_of[s] >= 0 && !appends[s]) {
      const int wb = hdr[t][kDescWaves] & 0xff, wn = (hdr[t][kDescWaves] >> 8) & 0xff;
      bool any = false;
      for (int w = wb; w < wb + wn; ++w) any = any || holds[w] != 0;
      if (any) flags = holds[t] ? kFlagStoreFirst : 0;   // the holder stores, nobody else
    }
#pragma unroll
    for (int k = 0; k < kPlanHdrInts; ++k) desc[t * dn + k] = k == kDescFlags ? flags : hdr[t][k];
  }
}

template <int DT, int D, int G, int W, int NPF, bool MFMA>
hipError_t launch_planned_typed(const PlannedDecodeArgs& a, hipStream_t stream) {
  PlannedShape sh{a.num_seqs, a.num_kv_heads, a.num_blocks, a.max_context_len, a.desc_ints,
                  a.scale_log2};
  if (a.new_key != nullptr) {
    hipLaunchKernelGGL((paged_decode_planned_kernel<DT, D, G, W, NPF, MFMA, true>),
                       dim3((unsigned)a.num_bins), dim3(W * 64), 0, stream, (uint16_t*)a.out,
                       (const uint16_t*)a.q, (uint16_t*)a.k_cache, (uint16_t*)a.v_cache, a.plan, sh,
                       (const uint16_t*)a.new_key, (const uint16_t*)a.new_value);
  } else {
    hipLaunchKernelGGL((paged_decode_planned_kernel<DT, D, G, W, NPF, MFMA, false>),
                       dim3((unsigned)a.num_bins), dim3(W * 64), 0, stream, (uint16_t*)a.out,
                       (const uint16_t*)a.q, (uint16_t*)a.k_cache, (uint16_t*)a.v_cache, a.plan, sh,
                       nullptr, nullptr);
  }
  return hipGetLastError();
}

// Blocks in flight per wave: three for the MFMA tile (g >= 2): at head_dim
// 128 that fits the two-waves-per-SIMD register budget (a plan of short
// contexts gives each wave at most three blocks, all then in flight at
// once), at head_dim 64 it stays within 128 VGPRs (four waves per SIMD;
// TinyLlama shape 58.8 -> 58.0 us); two for the VALU policy (g = 1).
template <int D, int G>
constexpr int kPlannedPrefetch = G >= 2 ? 3 : 2;

template <int DT, int D, int G>
hipError_t launch_planned_group(const PlannedDecodeArgs& a, hipStream_t stream) {
  constexpr bool kMfma = G >= 2;
  return launch_planned_typed<DT, D, G, kPlanWaves, kPlannedPrefetch<D, G>, kMfma>(a, stream);
}

template <int DT, int D>
hipError_t launch_planned_dim(const PlannedDecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_planned_group<DT, D, 1>(a, stream);
    case 2: return launch_planned_group<DT, D, 2>(a, stream);
    case 4: return launch_planned_group<DT, D, 4>(a, stream);
    case 8: return launch_planned_group<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_plan(const DecodePlanArgs& a, hipStream_t stream) {
  const uint32_t hkv = (uint32_t)a.num_kv_heads;
  const uint32_t ids = (uint32_t)(a.desc_ints - kPlanHdrInts);
  BinShape ps{a.num_seqs, a.num_kv_heads, a.max_blocks_per_seq, a.max_context_len, a.num_bins,
              a.desc_ints, hkv > 1u ? 0xFFFFFFFFu / hkv + 1u : 0u, 0xFFFFFFFFu / ids + 1u};
  hipLaunchKernelGGL((paged_decode_plan_bins_kernel<kPlanWaves>), dim3((unsigned)a.num_bins),
                     dim3(kBinThreads), 0, stream, a.plan, a.block_tables, a.context_lens,
                     a.slot_mapping, ps);
  return hipGetLastError();
}

hipError_t launch_paged_decode_planned(const PlannedDecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (a.dtype == 0) {
    return a.head_dim == 64 ? launch_planned_dim<0, 64>(a, group, stream)
                            : launch_planned_dim<0, 128>(a, group, stream);
  }
  return a.head_dim == 64 ? launch_planned_dim<1, 64>(a, group, stream)
                          : launch_planned_dim<1, 128>(a, group, stream);
}

}  // namespace mvk

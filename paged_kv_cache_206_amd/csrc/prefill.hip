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
// Work decomposition: one workgroup of W = 4 waves per (32 W query tokens,
// query head, prompt). Wave w owns two 16-row tiles, query tokens [16w,
// 16w + 16) and [16W + 16w, 16W + 16w + 16) of the workgroup's range, so the
// waves reach the causal diagonal at similar depths. The workgroup walks the
// prompt's K/V rows from token 0 to its last query token in 64-token tiles,
// double buffered in LDS: the next tile streams from memory straight into
// LDS while the current one is computed, and one barrier per tile separates
// the two. The K/V rows come from the new key/value tensors (contiguous per
// prompt), not through the block table: they are this pass's own rows.
// Later query ranges carry more work and are dispatched first.
//
// Per 32 K/V tokens a wave runs, for each of its tiles:
//   S^T = K Q^T     two v_mfma_f32_16x16x32 chains (16 tokens x 16 rows each);
//                   lane l holds tokens 4*(l/16)+i (+16) of row l%16
//   online softmax  base 2, reference max raised lazily (by more than
//                   kLazyRescale), masking only on blocks that cross the
//                   diagonal; p rounded to the storage type (v_cvt_pk_*)
//   O += P V        v_mfma_f32_16x16x32 with the 32 tokens as the reduction
//                   index. The 8 p values a lane holds are exactly its
//                   A-operand slots once the reduction index is ordered
//                   (tokens 4*q4..4*q4+3, then 16+4*q4..16+4*q4+3) for lane
//                   group q4; each B operand (those 8 tokens of one V
//                   column) comes from two transposed LDS reads
//                   (ds_read_b64_tr_b16) of the row-major V tile.
//   l += P 1        one more MFMA against a ones operand sums the same rounded
//                   p per row, in the output's own layout.
// The K/V fragments a wave reads from LDS serve both of its tiles.
//
// LDS: K and V tiles are row-major, loaded straight from the prompt's rows
// (buffer loads to LDS), with the 16-byte chunks of each row permuted (swz_k,
// swz_v) so that the operand reads meet no bank conflicts; the two tile
// buffers are separate arrays (see the main loop).
#include "attention_mfma.h"
#include "device_common.h"
#include "launch.h"

namespace mvk {

namespace {

typedef __bf16 pf_bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 pf_f16x2_t __attribute__((ext_vector_type(2)));
typedef float pf_f32x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

template <int DT> struct PfMath;
template <> struct PfMath<0> {  // binary16
  static constexpr uint32_t kOnes = 0x3C003C00u;
  static __device__ __forceinline__ uint32_t pack(float a, float b) {  // round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(pf_f32x2_t{a, b}, pf_f16x2_t));
  }
  static __device__ __forceinline__ f32x4_t mma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct PfMath<1> {  // bfloat16
  static constexpr uint32_t kOnes = 0x3F803F80u;
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(pf_f32x2_t{a, b}, pf_bf16x2_t));
  }
  static __device__ __forceinline__ f32x4_t mma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

struct PfShape {
  int32_t num_q_heads, num_kv_heads, num_blocks, query_tiles, num_tokens;
  float scale_log2;
};


template <int DT, int D>
struct PfTile {
  static constexpr int kWaves = 4;                 // waves per workgroup
  static constexpr int kTiles = 2;                 // 16-row query tiles per wave
  static constexpr int kRows = 16 * kTiles * kWaves;  // query tokens per workgroup
  static constexpr int kKvTile = 64;               // K/V tokens per LDS tile
  static constexpr int NKS = D / 32;               // QK reduction steps of 32
  static constexpr int NE = D / 16;                // PV output column groups
  static constexpr int kChunks = D / 8;            // 16-byte chunks per row
  static constexpr int kTileBytes = kKvTile * D * 2;  // one K or V tile, row-major
  static constexpr int kBufBytes = 2 * kTileBytes;    // K tile, then V tile
  // 1 KB LDS-DMA loads (64 lanes x 16 bytes) per wave for one K or V tile
  static constexpr int kDmaPerWave = kKvTile * kChunks / 64 / kWaves;
  static_assert(kDmaPerWave * kWaves * 64 == kKvTile * kChunks, "tile split into 1 KB loads");
};

// gfx950 LDS instructions, wrapped in plain device functions (called from
// the kernel template, a direct builtin call would also have to instantiate
// in the host compilation, which lacks these target features):
// 16 bytes per lane from a buffer straight into LDS (lane l writes bytes
// 16 l .. 16 l + 15 after `lds`), and a transposed 16-bit read (lane n of
// each 16-lane group gets element n % 4 of the 8-byte reads of lanes
// 4 k + n / 4, k = 0..3).
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Chunk swizzles of the row-major K and V tiles (16-byte chunk c of row r
// sits at chunk position c ^ swz_k(r) of its row in K, c ^ swz_v(r) in V),
// chosen so that the operand reads meet no bank conflicts: a K operand read
// takes one chunk of 16 consecutive rows; a V transposed read takes two
// adjacent chunks of 8 consecutive rows. 256-byte rows (D = 128) start on the same bank, so the
// swizzle alone separates them; 128-byte rows (D = 64) alternate between two
// bank halves, so rows of one parity are separated. Both repeat every 16
// rows. (A single swizzle meeting both patterns on paper, ((u % (KC/2)) << 1)
// | bit log2(KC/2) of u with u the row, or the row / 2 at D = 64, measured
// about one conflict cycle per two conflict-free ones on gfx950.)
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

// Four waves per SIMD at head_dim 64 (at most 128 VGPRs; 122 used): its
// exponentials make it the VALU-bound shape, and more resident waves hide
// more of the step's chain (against three waves per SIMD, 6.09 -> 5.75 ms
// for 256 x 2048 tokens when first measured); two at 128 (214 VGPRs).
template <int DT, int D, int G>
__global__ __launch_bounds__((PfTile<DT, D>::kWaves * 64)) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2)))
void prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
                    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                    const int32_t* __restrict__ slots, const int32_t* __restrict__ cu_seqlens,
                    PfShape sh) {
  using T = PfTile<DT, D>;
  using Mth = PfMath<DT>;
  using E = Elem<DT>;
  constexpr int NKS = T::NKS, NE = T::NE, KC = T::kChunks;
  constexpr int kPfKvTile = T::kKvTile;
  constexpr int kPfWaves = T::kWaves, kPfRows = T::kRows, NT = T::kTiles;
  __shared__ __attribute__((aligned(16))) char smem0[T::kBufBytes];
  __shared__ __attribute__((aligned(16))) char smem1[T::kBufBytes];

  // Workgroups are dealt round-robin to the XCDs in dispatch order; remap so
  // that each XCD runs whole (query head, prompt) groups. Their query ranges
  // then share K/V tiles in one L2, and every XCD gets the same mix of heavy
  // and light ranges (with the range index fastest and no remap, XCD k would
  // get ranges k and k + 8 of every group: 2.4x more work on some XCDs).
  const uint32_t n_wg = gridDim.x * gridDim.y * gridDim.z;
  const uint32_t v =
      xcd_contiguous(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), n_wg);
  const int s = v / (gridDim.x * gridDim.y);
  const int j = (v / gridDim.x) % gridDim.y;                // query head
  const int qt = sh.query_tiles - 1 - (int)(v % gridDim.x);  // latest (heaviest) ranges first
  // prompt s's rows [lo, lo + n), clamped to [0, T] so that inconsistent
  // offsets never index outside the token arrays
  const int lo = min(max(cu_seqlens[s], 0), sh.num_tokens);
  const int n = min(max(cu_seqlens[s + 1], lo), sh.num_tokens) - lo;
  const int q0 = qt * kPfRows;
  if (q0 >= n) return;  // uniform over the workgroup
  const int h = j / G;
  const int Hq = sh.num_q_heads, Hkv = sh.num_kv_heads;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  const int q_end = min(n, q0 + kPfRows);  // the workgroup's query tokens: [q0, q_end)
  const float sl2 = sh.scale_log2;

  // Cache write: the first query head of each KV head stores the workgroup's
  // tokens' rows of that KV head (every row exactly once over the grid).
  if (slots != nullptr && j % G == 0) {
    for (int idx = tid; idx < (q_end - q0) * T::kChunks; idx += kPfWaves * 64) {
      const int t = q0 + idx / T::kChunks;
      const int c = idx % T::kChunks;
      const int slot = slots[lo + t];
      if (slot >= 0 && slot < sh.num_blocks * kBlockTokens) {
        const size_t src = ((size_t)(lo + t) * Hkv + h) * D + c * 8;
        const size_t dst = ((size_t)slot * Hkv + h) * D + c * 8;
        *(uint4*)(k_cache + dst) = *(const uint4*)(key + src);
        *(uint4*)(v_cache + dst) = *(const uint4*)(value + src);
      }
    }
  }

  // This wave's two tiles: rows rb[t] + r16 (B operand: row r16's query).
  int rb[NT];
  uint4 qop[NT][NKS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    rb[t] = q0 + 16 * kPfWaves * t + 16 * wave;
    const int row = rb[t] + r16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qop[t][ks] = row < n ? *(const uint4*)(q + ((size_t)(lo + row) * Hq + j) * D + 32 * ks + 8 * q4)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  f32x4_t acc[NT][NE], lacc[NT];
  // nm: minus row r16's reference maximum (scaled, base 2), the addend of
  // every exponent
  float nm[NT];
  // thr: the raw logit above which the scaled one passes the reference by
  // more than kLazyRescale, (kLazyRescale - nm) / sl2 (sl2 > 0), so that each
  // step tests its raw maximum with one compare
  const float inv_sl2 = 1.0f / sl2;
  float thr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[t][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    nm[t] = -kNegBig;
    thr[t] = (kLazyRescale + kNegBig) * inv_sl2;
  }
  uint4 ones = make_uint4(Mth::kOnes, Mth::kOnes, Mth::kOnes, Mth::kOnes);
  // kept in registers (as a known constant the compiler rebuilds it with
  // three moves before every use)
  asm volatile("" : "+v"(ones.x), "+v"(ones.y), "+v"(ones.z), "+v"(ones.w));

  // Staging: the K and V tiles go from the prompt's rows straight into LDS
  // (buffer loads to LDS, 1 KB per instruction, lane l filling bytes 16 l ..
  // 16 l + 15 of it), so no registers hold a tile in flight. Lane l of load i
  // fills chunk position p = 64 i + l of the tile: row p / KC, chunk
  // (p % KC) ^ swz_k(row) (swz_v for V) of that token's row. Each tile's descriptors start at
  // its first row and end at row q_end: rows past it (the tail of the last
  // tile) read as zero, and the per-lane offsets are the same for every tile.
  const uint32_t row_stride = (uint32_t)Hkv * D * 2;
  const uint16_t* kbase = key + (size_t)lo * Hkv * D;
  const uint16_t* vbase = value + (size_t)lo * Hkv * D;
  uint32_t koff_dma[T::kDmaPerWave], voff_dma[T::kDmaPerWave];
#pragma unroll
  for (int i = 0; i < T::kDmaPerWave; ++i) {
    const int p = 64 * (wave * T::kDmaPerWave + i) + lane;
    const int row = p / KC, pos = p % KC;
    const uint32_t trow = (uint32_t)row * row_stride + (uint32_t)h * D * 2;
    koff_dma[i] = trow + 16u * (pos ^ swz_k<D>(row));
    voff_dma[i] = trow + 16u * (pos ^ swz_v<D>(row));
  }
  auto fetch = [&](char* base, int kt0) __attribute__((always_inline)) {
    const uint32_t skip = (uint32_t)kt0 * row_stride;
    const uint32_t bytes = (uint32_t)q_end * row_stride - skip;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc((const char*)kbase + skip, bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const char*)vbase + skip, bytes);
#pragma unroll
    for (int i = 0; i < T::kDmaPerWave; ++i) {
      const int gi = wave * T::kDmaPerWave + i;  // this wave's i-th 1 KB piece of a tile
      load_to_lds16(krs, base + 1024 * gi, koff_dma[i]);
      load_to_lds16(vrs, base + T::kTileBytes + 1024 * gi, voff_dma[i]);
    }
  };

  // Per-lane byte offsets of the operand reads within a K or V tile, the
  // same for both buffers and every 32-token half (the swizzles repeat every
  // 16 rows); kept opaque so that the compiler adds each buffer's address as
  // an instruction offset instead of holding one register per buffer
  int kofs[NKS], vofs[NE];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kofs[ks] = 16 * (r16 * KC + ((4 * ks + q4) ^ swz_k<D>(r16)));
    asm volatile("" : "+v"(kofs[ks]));
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int t0 = 4 * q4 + ((lane & 15) >> 2);
    const int c = 2 * e + ((lane & 3) >> 1);
    vofs[e] = 16 * (t0 * KC + (c ^ swz_v<D>(t0))) + 8 * (lane & 1);
    asm volatile("" : "+v"(vofs[e]));
  }

  // Reads of one 32-token half of a K/V tile: the K fragments of its two
  // 16-token blocks and the V fragments of its 32 tokens
  auto read_frags = [&](const char* sk, const int hoff, uint4 (&kf)[2][NKS], uint4 (&vf)[NE])
      __attribute__((always_inline)) {
    const char* sv = sk + T::kTileBytes;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kf[b][ks] = *(const uint4*)(sk + kofs[ks] + 16 * KC * (hoff + 16 * b));
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      // two transposed reads: lane j of a 16-lane group reads 4 columns
      // (16 e + 4 (j % 4) ...) of token row t0 + j / 4; the hardware hands
      // lane n column 16 e + n of the four rows, so slots 0-3 hold tokens
      // 4 q4 .. 4 q4 + 3 and slots 4-7 tokens 16 + 4 q4 .. 16 + 4 q4 + 3
      const char* vp = sv + vofs[e] + 16 * KC * hoff;
      const uint2 a = lds_read_tr16(vp), b = lds_read_tr16(vp + 16 * 16 * KC);
      vf[e] = make_uint4(a.x, a.y, b.x, b.y);
    }
  };
  auto qk = [&](const uint4 (&kf)[2][NKS], int t, float (&z)[8]) __attribute__((always_inline)) {
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      s0 = Mth::mma(kf[0][ks], qop[t][ks], s0);
      s1 = Mth::mma(kf[1][ks], qop[t][ks], s1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = s0[i];
      z[4 + i] = s1[i];
    }
  };
  auto max8 = [](const float (&z)[8]) __attribute__((always_inline)) {
    return fmaxf(fmaxf(fmaxf(fmaxf(z[0], z[1]), z[2]), fmaxf(fmaxf(z[3], z[4]), z[5])),
                 fmaxf(z[6], z[7]));
  };
  // Raise tile t's reference to the row maximum where it passed the old one
  // by more than kLazyRescale, scaling the row's sums by 2^(m_old - m_new)
  auto rescale = [&](int t, float mx) __attribute__((always_inline)) {
    // the 4 lanes of a row (l, l^16, l^32, l^48) agree on its new reference
    float bm = mx * sl2;
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mold = -nm[t];
    const float mnew = bm > mold + kLazyRescale ? bm : mold;
    const float alpha = fast_exp2(mold - mnew);
    nm[t] = -mnew;
    thr[t] = (kLazyRescale + mnew) * inv_sl2;
    // output rows 4*q4+i take the factor of the lane that holds row 4*q4+i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __shfl(alpha, 4 * q4 + i);
      lacc[t][i] *= a;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[t][e][i] *= a;
    }
  };
  auto accumulate = [&](int t, const float (&z)[8], const uint4 (&vf)[NE]) __attribute__((always_inline)) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(z[i], sl2, nm[t]));
    const uint4 pa = make_uint4(Mth::pack(p[0], p[1]), Mth::pack(p[2], p[3]),
                                Mth::pack(p[4], p[5]), Mth::pack(p[6], p[7]));
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[t][e] = Mth::mma(pa, vf[e], acc[t][e]);
    lacc[t] = Mth::mma(pa, ones, lacc[t]);
  };

  // One 32-token step of the K/V tile in buffer sk (tokens tok0 .., hoff
  // into the tile): a tile wholly above the diagonal (or past the prompt's
  // end) is skipped, and tokens past a row's own are masked where the step
  // crosses a tile's diagonal.
  auto step = [&](const char* sk, const int tok0, const int hoff) __attribute__((always_inline)) {
    bool act[NT];
    bool any = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      act[t] = rb[t] < n && tok0 <= rb[t] + 15;
      any = any || act[t];
    }
    if (!any) return;  // uniform over the wave
    uint4 kf[2][NKS], vf[NE];
    read_frags(sk, hoff, kf, vf);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (!act[t]) continue;
      float z[8];
      qk(kf, t, z);
      if (tok0 + 31 > rb[t]) {  // the 32 tokens cross this tile's diagonal
        // row r16 sees tokens up to its own: this lane's tokens tok0 + 4 q4 + i
        // (+ 16) are visible while i (+ 16) < vis
        const int vis = rb[t] + r16 + 1 - (tok0 + 4 * q4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= vis) z[i] = -INFINITY;
          if (16 + i >= vis) z[4 + i] = -INFINITY;
        }
      }
      // raise the reference only where a scaled logit passes it by more than
      // kLazyRescale: the raw maximum against thr (sl2 > 0, so the raw
      // maximum scales to the scaled one)
      const float mx = max8(z);
      if (__any(mx > thr[t])) rescale(t, mx);
      accumulate(t, z, vf);
    }
  };

  // Two LDS buffers, used alternately: the next tile streams into one while
  // the other is computed. They are separate arrays so that the compiler can
  // tell the loads into one from the reads of the other (with one array it
  // makes every read wait for all of this wave's loads, the next tile's
  // included); the explicit wait for this wave's loads and the barrier after
  // each tile order the rest.
  const int ntiles = (q_end + kPfKvTile - 1) / kPfKvTile;
  fetch(smem0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have reached LDS
  lds_barrier();
  for (int kt = 0; kt < ntiles; kt += 2) {
    if (kt + 1 < ntiles) fetch(smem1, (kt + 1) * kPfKvTile);
    step(smem0, kt * kPfKvTile, 0);
    step(smem0, kt * kPfKvTile + 32, 32);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile are in LDS
    lds_barrier();
    if (kt + 1 >= ntiles) break;
    if (kt + 2 < ntiles) fetch(smem0, (kt + 2) * kPfKvTile);
    step(smem1, (kt + 1) * kPfKvTile, 0);
    step(smem1, (kt + 1) * kPfKvTile + 32, 32);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
  }

  // Output rows rb[t] + 4*q4 + i, columns 16e + r16: divided by the row's sum.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rb[t] + 4 * q4 + i;
      if (row < n) {
        const float inv = 1.0f / lacc[t][i];
        uint16_t* o = out + ((size_t)(lo + row) * Hq + j) * D + r16;
#pragma unroll
        for (int e = 0; e < NE; ++e) o[16 * e] = E::round(acc[t][e][i] * inv);
      }
    }
  }
}

template <int DT, int D, int G>
hipError_t launch_prefill_typed(const PrefillArgs& a, hipStream_t stream) {
  using T = PfTile<DT, D>;
  PfShape sh{a.num_q_heads, a.num_kv_heads, a.num_blocks,
             (a.max_seqlen + T::kRows - 1) / T::kRows, a.num_tokens, a.scale_log2};
  dim3 grid((unsigned)sh.query_tiles, (unsigned)a.num_q_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((prefill_kernel<DT, D, G>), grid, dim3(T::kWaves * 64), 0, stream,
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

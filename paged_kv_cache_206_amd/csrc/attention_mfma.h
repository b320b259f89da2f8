// MFMA attention tile for gfx950: one wave computes, for up to 16 query rows
// and one 16-token block, the logits S^T = K Q^T, the online softmax update
// and O += P V. Used by the decode kernel (rows = the g query heads of a KV
// head) and by the multi-query kernel (rows = (new token, query head) pairs).
//
// Layouts: S^T = K Q^T on v_mfma_f32_16x16x32 (16 tokens x 16 row slots,
// zero-padded past the rows in use); its result layout (lane l holds tokens
// 4*(l/16)+i of row l%16) is exactly the A-operand layout of
// v_mfma_f32_16x16x16 for O += P V. V rows are loaded coalesced (four full
// rows per instruction) and transposed into token pairs with v_perm_b32. P
// is rounded to the storage type for the PV product; the denominator sums
// the same rounded values. The softmax is the online normaliser (Milakov &
// Gimelshein 2018) in base-2 units; its reference max moves only when a
// logit passes it by more than kLazyRescale.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace mvk {

constexpr float kNegBig = -1.0e30f;   // "no token seen yet" (finite: 2^(a-b) never sees inf-inf)
constexpr float kLazyRescale = 8.0f;  // p = 2^(z - m) may grow up to 2^8 before rescaling

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT> struct Mma;
template <> struct Mma<0> {  // binary16
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<1> {  // bfloat16
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
};

// Byte selectors for v_perm_b32(hi_src, lo_src, sel): gather the low (resp.
// high) 16-bit halves of lo_src and hi_src into one word, lo_src's first.
constexpr uint32_t kPermLoHalves = 0x05040100u;
constexpr uint32_t kPermHiHalves = 0x07060302u;

// ------------------------------------------------------------ MFMA policy
template <int DT, int D, int G>
struct MfmaPolicy {
  static_assert(G >= 1 && G <= 16, "one 16-row tile holds the whole group");
  static constexpr int NKS = D / 32;  // QK k-steps of 32
  static constexpr int VW = D / 16;   // V elements per lane per token row (8 or 4)
  static constexpr int NE = VW;       // PV products (16 output columns each)
  using VT = typename std::conditional<D == 128, uint4, uint2>::type;

  // K is loaded in whole 128-byte lines and rearranged (arrange) into the
  // QK operand layout: operand ks of lane l is K[token l%16][32*ks + 8*(l/16)
  // .. +7]. Load 2*h+T of lane l reads token 8*T + l%8, 16-byte chunk
  // 8*h + l/16 + 4*((l%16)/8) of the row: each instruction covers line h of
  // 8 token rows.
  struct Frag {
    uint4 k[NKS];  // as loaded; after arrange(), the QK operands
    VT v[4];       // V[token 4*(l/16)+i][VW*(l%16) .. +VW-1]
  };

  uint4 qop[NKS];
  uint4 nk_ov[NKS];  // the step's new K row pieces of this lane (load_new_row)
  VT nv_ov;          // and its new V row piece
  f32x4_t acc[NE];
  float m, lsum;
  int r16, q4;
  uint32_t koff, voff;  // per-lane byte offsets inside a block (loop invariant)
  int row_new;          // offset of the step's new row inside its block (fused write)

  // Lane layout, empty state, and row r16's query (q_row: that row's D
  // elements, or nullptr for a row slot no query fills).
  __device__ __forceinline__ void init_rows(const uint16_t* q_row, int lane, uint32_t row_bytes) {
    r16 = lane & 15;
    q4 = lane >> 4;
    koff = (lane & 7) * row_bytes + 16u * (q4 + 4 * ((lane & 15) >> 3));
    voff = 4u * q4 * row_bytes + 2u * VW * r16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qop[ks] = q_row != nullptr ? *(const uint4*)(q_row + 32 * ks + 8 * q4)
                                 : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = kNegBig;
    lsum = 0.0f;
  }

  // Decode: row slot j < G is query head j of the group (rows q_row0 + j of q).
  __device__ __forceinline__ void init(const uint16_t* q, size_t q_row0, int lane,
                                       uint32_t row_bytes) {
    const int r = lane & 15;
    init_rows(r < G ? q + (q_row0 + r) * D : nullptr, lane, row_bytes);
  }

  // kr/vr: this KV head's slice of one block (a scalar descriptor; every lane
  // adds its fixed offset); rows past the context read as 0
  template <int POL>
  __device__ __forceinline__ void load(Frag& f, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                       uint32_t row_bytes) const {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      f.k[ks] = buffer_load16<POL>(kr, koff + 128u * (ks >> 1) + 8u * (ks & 1) * row_bytes);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (D == 128) f.v[i] = buffer_load16<POL>(vr, voff + i * row_bytes);
      else f.v[i] = buffer_load8<POL>(vr, voff + i * row_bytes);
    }
  }

  // Loaded K lines -> QK operands. For line h, load A = k[2h] holds tokens
  // 0-7 and B = k[2h+1] tokens 8-15; operand 2h takes A's first half-row and
  // B's chunks from 8 lanes away, operand 2h+1 the reverse.
  __device__ __forceinline__ void arrange(Frag& f) const {
#pragma unroll
    for (int h = 0; h < NKS / 2; ++h) {
      const uint4 a = f.k[2 * h], b = f.k[2 * h + 1];
      f.k[2 * h] = make_uint4(swap_half_rows<kDppBanksHi>(a.x, b.x), swap_half_rows<kDppBanksHi>(a.y, b.y),
                              swap_half_rows<kDppBanksHi>(a.z, b.z), swap_half_rows<kDppBanksHi>(a.w, b.w));
      f.k[2 * h + 1] =
          make_uint4(swap_half_rows<kDppBanksLo>(b.x, a.x), swap_half_rows<kDppBanksLo>(b.y, a.y),
                     swap_half_rows<kDppBanksLo>(b.z, a.z), swap_half_rows<kDppBanksLo>(b.w, a.w));
    }
  }

  // Decode: every row slot j < G sees the block's tokens below t_end.
  // nk/nv: the step's new K/V row of this KV head in LDS, as 16-byte chunks
  __device__ __forceinline__ void process(Frag& f, int tok0, int t_end, float scale_log2, bool sub,
                                          const uint4* nk, const uint4* nv) {
    arrange(f);
    if (sub) {  // this block holds the new row: take it from LDS, not memory
      if (r16 == row_new) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) f.k[ks] = nk[4 * ks + q4];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * q4 + i == row_new) f.v[i] = ((const VT*)nv)[r16];
      }
    }
    step(f, tok0, r16 < G ? t_end : 0, scale_log2);
  }

  // The step's new K/V row of this KV head (nk_row / nv_row: its D elements)
  // for the planned kernel, which takes the new token before the blocks
  // (seed_row) and stores the row (store_new_row) instead of taking it in
  // place of a pool row: every lane loads the K pieces of its quarter
  // (elements 32*ks + 8*q4 .. +7, the layout of its query operand) and the
  // V piece of its columns (VW*r16 .. +VW-1, the layout of its accumulators).
  __device__ __forceinline__ void load_new_row(const uint16_t* nk_row, const uint16_t* nv_row) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) nk_ov[ks] = *(const uint4*)(nk_row + 32 * ks + 8 * q4);
    nv_ov = *(const VT*)(nv_row + VW * r16);
  }

  // Store the row loaded by load_new_row: lanes of row slot 0 write K,
  // lanes of quarter 0 write V.
  __device__ __forceinline__ void store_new_row(uint16_t* k_dst, uint16_t* v_dst) const {
    if (r16 == 0) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) *(uint4*)(k_dst + 32 * ks + 8 * q4) = nk_ov[ks];
    }
    if (q4 == 0) *(VT*)(v_dst + VW * r16) = nv_ov;
  }

  // Start the empty online-softmax state from the new row of load_new_row
  // as its first token, for the rows below G: the reference is the row's
  // logit (the quarters' partial dot products summed across the four lanes
  // of a row), its weight exp2(0) = 1 is counted once per row in the
  // denominator, and O = v_new. Later tokens are added by step() as usual.
  __device__ __forceinline__ void seed_row(float scale_log2) {
    using E = Elem<DT>;
    float d = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      d = E::dot2(qop[ks].x, nk_ov[ks].x, d);
      d = E::dot2(qop[ks].y, nk_ov[ks].y, d);
      d = E::dot2(qop[ks].z, nk_ov[ks].z, d);
      d = E::dot2(qop[ks].w, nk_ov[ks].w, d);
    }
    d += __shfl_xor(d, 16);
    d += __shfl_xor(d, 32);
    if (r16 < G) {
      m = d * scale_log2;
      if (q4 == 0) lsum = 1.0f;
    }
    // acc[2k][i], acc[2k+1][i]: head 4*q4+i, columns VW*r16+2k, +2k+1
    const uint32_t* w = (const uint32_t*)&nv_ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * q4 + i < G) {
#pragma unroll
        for (int k = 0; k < VW / 2; ++k) {
          acc[2 * k][i] = E::lo(w[k]);
          acc[2 * k + 1][i] = E::hi(w[k]);
        }
      }
    }
  }

  // A block with no new-row substitution.
  __device__ __forceinline__ void process_plain(Frag& f, int tok0, int t_end, float scale_log2) {
    arrange(f);
    step(f, tok0, r16 < G ? t_end : 0, scale_log2);
  }

  // One block of 16 tokens starting at tok0 (K already arranged); this lane's
  // row slot r16 sees the tokens below row_end (its own limit: causal masks
  // differ per row).
  __device__ __forceinline__ void step(Frag& f, int tok0, int row_end, float scale_log2) {
    using M = Mma<DT>;
    using E = Elem<DT>;
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sc = M::qk(f.k[ks], qop[ks], sc);

    const int tb = tok0 + 4 * q4;  // this lane's tokens: tb + i, head r16
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = tb + i < row_end ? sc[i] * scale_log2 : -INFINITY;

    const float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    if (__any(mx > m + kLazyRescale)) {
      // new reference for every head whose block max passed the threshold;
      // the 4 lanes of a head (l, l^16, l^32, l^48) agree on it
      float bm = fmaxf(mx, __shfl_xor(mx, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mnew = bm > m + kLazyRescale ? bm : m;
      const float alpha = fast_exp2(m - mnew);
      lsum *= alpha;
      m = mnew;
      // acc element i holds head 4*q4+i, whose factor lives in lane 4*q4+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, 4 * q4 + i);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e][i] *= a;
      }
    }
    uint32_t pw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint16_t p0 = E::round(fast_exp2(z[2 * i] - m));
      const uint16_t p1 = E::round(fast_exp2(z[2 * i + 1] - m));
      pw[i] = (uint32_t)p0 | ((uint32_t)p1 << 16);
      lsum += E::lo(pw[i]) + E::hi(pw[i]);
    }
    const uint2 pa = make_uint2(pw[0], pw[1]);

    const uint32_t* w0 = (const uint32_t*)&f.v[0];
    const uint32_t* w1 = (const uint32_t*)&f.v[1];
    const uint32_t* w2 = (const uint32_t*)&f.v[2];
    const uint32_t* w3 = (const uint32_t*)&f.v[3];
#pragma unroll
    for (int k = 0; k < VW / 2; ++k) {
      const uint2 blo = make_uint2(__builtin_amdgcn_perm(w1[k], w0[k], kPermLoHalves),
                                   __builtin_amdgcn_perm(w3[k], w2[k], kPermLoHalves));
      const uint2 bhi = make_uint2(__builtin_amdgcn_perm(w1[k], w0[k], kPermHiHalves),
                                   __builtin_amdgcn_perm(w3[k], w2[k], kPermHiHalves));
      acc[2 * k] = M::pv(pa, blo, acc[2 * k]);
      acc[2 * k + 1] = M::pv(pa, bhi, acc[2 * k + 1]);
    }
  }

  // Hand the wave's state to LDS: m/l per head, unnormalised o per head.
  __device__ __forceinline__ void to_lds(float* sm_m, float* sm_l, float* sm_o) {
    float l = lsum + __shfl_xor(lsum, 16);
    l += __shfl_xor(l, 32);
    if (q4 == 0 && r16 < G) {
      sm_m[r16] = m;
      sm_l[r16] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 4 * q4 + i;
      if (head < G) {
#pragma unroll
        for (int e = 0; e < NE; ++e) sm_o[head * D + VW * r16 + e] = acc[e][i];
      }
    }
  }
};

}  // namespace mvk

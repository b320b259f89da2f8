// VALU attention policy for gfx950 (wave64), used where a GQA group is a
// single query head (g = 1), which would fill one row of a 16-row MFMA tile:
// lanes (rg, c) read 16-byte chunk c of token rows rg, rg + RG, ...; v_dot2
// partial dots are summed over a row with DPP; the softmax is the online
// normaliser in base-2 units with a lazily raised reference max; PV
// accumulates in float32.
#pragma once

#include "attention_mfma.h"
#include "device_common.h"

namespace mvk {

template <int DT, int D, int G>
struct ValuPolicy {
  static constexpr int LPR = D / 8;              // lanes per token row (16-byte chunks)
  static constexpr int RG = 64 / LPR;            // token rows per wave-wide load
  static constexpr int TPL = kBlockTokens / RG;  // loads per block

  struct Frag {
    uint4 k[TPL];
    uint4 v[TPL];
  };

  uint4 qv[G];
  uint4 nk_ov, nv_ov;  // the step's new K / V row chunk of this lane (load_new_row)
  float m[G], l[G], acc[G][8];
  int rg, c;
  uint32_t off;  // per-lane byte offset inside a block (loop invariant)
  int row_new;   // offset of the step's new row inside its block (fused write)

  __device__ __forceinline__ void init(const uint16_t* q, size_t q_row0, int lane,
                                       uint32_t row_bytes) {
    rg = lane / LPR;
    c = lane % LPR;
    off = rg * row_bytes + 16u * c;
#pragma unroll
    for (int j = 0; j < G; ++j) qv[j] = *(const uint4*)(q + (q_row0 + j) * D + c * 8);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      m[j] = kNegBig;
      l[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
    }
  }

  template <int POL>
  __device__ __forceinline__ void load(Frag& f, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                       uint32_t row_bytes) const {
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint32_t o = off + i * RG * row_bytes;
      f.k[i] = buffer_load16<POL>(kr, o);
      f.v[i] = buffer_load16<POL>(vr, o);
    }
  }

  // nk/nv: the step's new K/V row of this KV head in LDS, as 16-byte chunks
  __device__ __forceinline__ void process(Frag& f, int tok0, int t_end, float scale_log2, bool sub,
                                          const uint4* nk, const uint4* nv) {
    if (sub) {  // this block holds the new row: take it from LDS, not memory
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        if (i * RG + rg == row_new) {
          f.k[i] = nk[c];
          f.v[i] = nv[c];
        }
      }
    }
    compute(f, tok0, t_end, scale_log2);
  }

  // The step's new K/V row (this KV head's D elements) for the planned
  // kernel: every lane loads chunk c, the chunk its rows cover.
  __device__ __forceinline__ void load_new_row(const uint16_t* nk_row, const uint16_t* nv_row) {
    nk_ov = *(const uint4*)(nk_row + 8 * c);
    nv_ov = *(const uint4*)(nv_row + 8 * c);
  }

  // Store the row loaded by load_new_row (the lanes of row group 0).
  __device__ __forceinline__ void store_new_row(uint16_t* k_dst, uint16_t* v_dst) const {
    if (rg == 0) {
      *(uint4*)(k_dst + 8 * c) = nk_ov;
      *(uint4*)(v_dst + 8 * c) = nv_ov;
    }
  }

  // Start the empty online-softmax state from the new row as the first
  // token, held by row group 0 (each row group keeps its own state until
  // to_lds merges them): reference = its logit, weight 1, O = v_new.
  __device__ __forceinline__ void seed_row(float scale_log2) {
    using E = Elem<DT>;
    const uint32_t w[4] = {nv_ov.x, nv_ov.y, nv_ov.z, nv_ov.w};
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float d = E::dot2(qv[j].x, nk_ov.x, 0.0f);
      d = E::dot2(qv[j].y, nk_ov.y, d);
      d = E::dot2(qv[j].z, nk_ov.z, d);
      d = E::dot2(qv[j].w, nk_ov.w, d);
      const float z = group_sum<LPR>(d) * scale_log2;
      if (rg == 0) {
        m[j] = z;
        l[j] = 1.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[j][2 * e] = E::lo(w[e]);
          acc[j][2 * e + 1] = E::hi(w[e]);
        }
      }
    }
  }

  __device__ __forceinline__ void process_plain(Frag& f, int tok0, int t_end, float scale_log2) {
    compute(f, tok0, t_end, scale_log2);
  }

  __device__ __forceinline__ void compute(Frag& f, int tok0, int t_end, float scale_log2) {
    using E = Elem<DT>;
    const int tb = tok0 + rg;  // token of load i is tb + i*RG
    float z[G][TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const bool valid = tb + i * RG < t_end;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = E::dot2(qv[j].x, f.k[i].x, 0.0f);
        d = E::dot2(qv[j].y, f.k[i].y, d);
        d = E::dot2(qv[j].z, f.k[i].z, d);
        d = E::dot2(qv[j].w, f.k[i].w, d);
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
        const uint32_t w[4] = {f.v[i].x, f.v[i].y, f.v[i].z, f.v[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[j][2 * e] = fmaf(p, E::lo(w[e]), acc[j][2 * e]);
          acc[j][2 * e + 1] = fmaf(p, E::hi(w[e]), acc[j][2 * e + 1]);
        }
      }
    }
  }

  __device__ __forceinline__ void to_lds(float* sm_m, float* sm_l, float* sm_o) {
    // merge the RG row groups (lanes c, c+LPR, ... hold the same output chunk)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float mo = __shfl_xor(m[j], off);
        const float lo = __shfl_xor(l[j], off);
        const float mm = fmaxf(m[j], mo);
        const float a = fast_exp2(m[j] - mm);
        const float b = fast_exp2(mo - mm);
        l[j] = l[j] * a + lo * b;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] * a + __shfl_xor(acc[j][e], off) * b;
        m[j] = mm;
      }
    }
    if (rg == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_o[j * D + c * 8 + e] = acc[j][e];
        if (c == 0) {
          sm_m[j] = m[j];
          sm_l[j] = l[j];
        }
      }
    }
  }
};

}  // namespace mvk

// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mvk {

constexpr int kBlockTokens = 16;  // tokens per KV block
constexpr uint32_t kXcds = 8;     // accelerator complex dies of an MI355X

// Workgroups are dealt round-robin to the 8 XCDs in dispatch order. Dispatch
// index i of n maps to the item index returned here, so that each XCD runs a
// contiguous range of items (and items that read the same data share an L2).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t i, uint32_t n) {
  const uint32_t xcd = i % kXcds, per = n / kXcds, rem = n % kXcds;
  return xcd * per + min(xcd, rem) + i / kXcds;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// Storage types. DT 0 = IEEE binary16, DT 1 = bfloat16; both are 16-bit words.
template <int DT> struct Elem;

template <> struct Elem<0> {
  // a.lo*b.lo + a.hi*b.hi + c, products and sum in float32 (v_dot2c_f32_f16)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  // float32 -> binary16, round to nearest even
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

template <> struct Elem<1> {
  // a.lo*b.lo + a.hi*b.hi + c in float32 (v_dot2c_f32_bf16)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), c, false);
  }
  // bfloat16 is the top half of a float32: widening is a shift / mask
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  // float32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + num_bytes): loads through it take a
// scalar descriptor plus a 32-bit per-lane byte offset, and every byte at or
// past num_bytes reads as zero. Word 3 selects 32-bit data format, which raw
// (untyped) loads require to be non-zero.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           kBufferWord3);
}

// Cache policy of a buffer load (the instruction's cache-policy bits).
// kStreamLoad sets the non-temporal bit: the lines it brings into L2 are the
// first to be replaced. The K/V streams of decode and multi-query use it:
// each of their load instructions consumes whole 128-byte lines that no
// other load of the workgroup reads again, so keeping them in L2 only
// displaces the block tables, query rows and partial states that are read
// again. Measured on MI355X: decode calls 6-11 % faster on every workload
// shape; blocks shared by several sequences (a common prefix) leave L2
// sooner and are fetched from memory somewhat more often. It costs time
// where an instruction reads half lines whose other half the next
// instruction reads, which is why the MFMA tile loads K in whole lines.
constexpr int kDefaultLoad = 0;
constexpr int kStreamLoad = 2;

template <int POLICY = kDefaultLoad>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY));
}

template <int POLICY = kDefaultLoad>
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POLICY));
}

// Blocks a sequence shares with a neighbour in the batch. Lane k holds
// entry k of a wave's block list (ent) and the entries at the same logical
// positions of the previous and next sequences' tables (-1 where there is
// none); bit k of the result is set when block k is also one of theirs.
// Sequences that share a prefix (a common prompt, parallel samples) sit next
// to each other in a batch, and their shared blocks are read by several
// workgroups at about the same time: those loads keep the default cache
// policy, so the blocks stay in L2 for the other readers, while every other
// block streams (kStreamLoad). A false match only changes a cache policy.
__device__ __forceinline__ uint64_t shared_blocks(int ent, int ent_prev, int ent_next) {
  return __ballot(ent == ent_prev || ent == ent_next);
}

// Device-coherent float store / load (relaxed atomics at device scope): they
// bypass the per-XCD L2's non-coherent state, so a value published by one
// workgroup is seen by a workgroup on another XCD without any cache-wide
// writeback or invalidate.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float collect(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier that orders LDS only: each wave's LDS writes complete
// before the barrier and are visible to every wave after it, while its
// global loads and stores stay in flight (a full __syncthreads also waits
// for them, which puts a memory round trip before the code that follows).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane moves inside a 16-lane DPP row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xF, 0xF, false);
}

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15-i within each 16 lanes
constexpr int kDppRowRor8 = 0x128;    // lane i <- lane (i+8) mod 16 within each 16 lanes
constexpr int kDppBanksLo = 0x3;      // bank mask: lanes 0-7 of each 16-lane row
constexpr int kDppBanksHi = 0xC;      // bank mask: lanes 8-15 of each 16-lane row

// Lanes of each 16-lane row in the banks selected by BANKS take x's value
// from the lane 8 places away in the same row; the other lanes keep old.
template <int BANKS>
__device__ __forceinline__ uint32_t swap_half_rows(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, kDppRowRor8, 0xF, BANKS, false);
}

// Sum over each aligned group of N lanes (N = 8 or 16); every lane of the
// group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp_mov<kDppRowMirror>(x);
  return x;
}

}  // namespace mvk

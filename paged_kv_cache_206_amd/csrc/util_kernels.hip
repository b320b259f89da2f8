// Small utility kernels: a zero fill for library-owned scratch, and a
// read-only streaming probe that measures the practical HBM read ceiling the
// attention kernels are compared against.
#include "device_common.h"
#include "launch.h"

namespace mvk {

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ dst, int64_t vecs) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < vecs; i += stride)
    dst[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t stream) {
  const int64_t vecs = (int64_t)(bytes / 16);
  if (vecs == 0) return hipSuccess;
  int64_t blocks = (vecs + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4*)dst,
                     vecs);
  return hipGetLastError();
}

// Streaming read: every thread reads kUnroll 16-byte vectors per iteration
// (all issued before any is consumed), with the same non-temporal cache
// policy as the attention kernels' K/V streams, and folds them into one word;
// each workgroup stores one word to `sink` so that no load is dead. Workgroups
// walk the buffer in grid-sized strides, so consecutive workgroups read
// consecutive 64 KiB pieces.
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(
    const void* __restrict__ src, uint32_t bytes, uint32_t* __restrict__ sink) {
  // bytes at or past `bytes` read as zero through the descriptor
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, bytes);
  uint32_t acc = 0;
  const uint32_t piece = kProbeThreads * kProbeUnroll * 16u;  // bytes per workgroup step
  for (uint64_t base = (uint64_t)blockIdx.x * piece; base < bytes;
       base += (uint64_t)gridDim.x * piece) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      v[u] = buffer_load16<kStreamLoad>(
          rs, (uint32_t)base + (uint32_t)(u * kProbeThreads + threadIdx.x) * 16u);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < kProbeThreads / 64; ++i) w ^= red[i];
    sink[blockIdx.x] = w;
  }
}

hipError_t launch_stream_read(const void* src, uint32_t bytes, uint32_t* sink, int32_t workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0,
                     stream, src, bytes, sink);
  return hipGetLastError();
}

}  // namespace mvk

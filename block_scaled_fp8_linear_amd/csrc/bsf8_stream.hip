// Plain read of a device buffer, for measurement only: the achievable HBM read
// rate on the same bytes as a GEMV, the rate the GEMV's own is compared with.
// Each lane reads four 16-byte words per pass, grid-strided so that every wave
// instruction covers 1 KiB of consecutive bytes.  Each block stores the XOR of
// what it read into its own sink word (a plain store: one shared word updated
// by atomics from every block serialises them and would dominate the time),
// so the loads cannot be dropped and the sink XOR equals the buffer's.  The
// loads are non-temporal: among the read patterns timed on 26 MB (256 to 1024
// threads per block, 2 to 16 loads per lane in flight, grid-strided or
// block-contiguous, one pass or a persistent grid of 256 to 2048 blocks) this
// one was the fastest (6.2 us; the same pattern without nt 6.7 us, the others
// 6.6 to 8.3 us).
#include <hip/hip_runtime.h>

#include "bsf8_internal.h"

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

namespace bsf8 {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * kStreamThreads;
  uint32_t acc = 0;
  for (int64_t base = int64_t(blockIdx.x) * kStreamThreads + threadIdx.x; base < n16; base += stride * kStreamUnroll) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = base + u * stride;
      const v4u t = i < n16 ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p) + i) : v4u{0, 0, 0, 0};
      v[u] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kStreamThreads / 64];
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kStreamThreads / 64; ++w) t ^= red[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

bsf8_status launch_read_stream(const void* p, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = int64_t(kStreamThreads) * kStreamUnroll;
  int64_t grid = (n16 + per_block - 1) / per_block;
  if (grid > BSF8_READ_STREAM_SINK_WORDS) grid = BSF8_READ_STREAM_SINK_WORDS;
  hipLaunchKernelGGL(read_stream_kernel, dim3(unsigned(grid)), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint4*>(p), n16, sink);
  return device_status(hipGetLastError(), "read_stream launch");
}

}  // namespace bsf8

// Dense copy of a block-scaled weight, the load step of the resident=False arm.
//
// ("th#1803: the consumer half of the layout gate", section "What lands": with
//  resident=False the loader upcasts the weight ahead of time instead of keeping
//  the FP8 bytes; "FP8 Native Serving", section "Native FP8 vs dequant-to-BF16":
//  the dequantized operand is BF16.)
//
// Wd[col0_i + r, k] = dec(q_i[r, k]) * s_i[r / 128, k / 128] for every member i,
// formed as one F32 product (exact for BF16 scales: 4 + 8 significant bits fit
// in 24) and written as F32 or rounded to nearest-even BF16.  Every E4M3 value is
// exact in BF16, so the decode goes through v_cvt_scalef32_pk_bf16_fp8 with a
// unit scale and widens to F32 by a shift.
//
// HBM-bound: each thread turns 16 weight bytes into 16 outputs; consecutive
// threads take consecutive 16-byte pieces of a row, so reads and writes are
// contiguous per wave.  The member and scale lookups are a few scalar-cached
// loads per thread.  The copy is written once and read by a later GEMM, so
// its stores are non-temporal (Q/K/V, three copies in turn: 28.7 -> 25.9 us);
// each weight byte is read once, so the loads are non-temporal too (26.2 ->
// 24.2 us).
#include <hip/hip_runtime.h>

#include "bsf8_internal.h"

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

namespace bsf8 {
namespace {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

constexpr int UP_THREADS = 256;

struct UpcastArgs {
  WeightDev w;
  void* out;
  int64_t ldo;        // elements
  uint32_t chunks;    // 16-element pieces per row: ceil(K / 16)
  uint32_t total;     // rows x chunks
};

template <bool SBF16>
__device__ __forceinline__ float scale_at(const void* s, int64_t idx) {
  if (SBF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(s)[idx]) << 16);
  return static_cast<const float*>(s)[idx];
}

__device__ __forceinline__ float bf16_to_f32(__bf16 b) {
  return __uint_as_float(uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const v2bf r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, r);
}

// VEC: K % 16 == 0, 16-byte aligned weights, output rows and base.
template <bool VEC, bool SBF16, bool OBF16>
__global__ __launch_bounds__(UP_THREADS) void upcast_kernel(UpcastArgs a) {
  const uint32_t idx = blockIdx.x * uint32_t(UP_THREADS) + threadIdx.x;
  if (idx >= a.total) return;
  const uint32_t row = idx / a.chunks;
  const int k0 = int(idx - row * a.chunks) * 16;
  int mi = 0;
  while (mi + 1 < a.w.n_members && int(row) >= a.w.m[mi + 1].col0) ++mi;
  const MemberDev mem = a.w.m[mi];
  const int r = int(row) - mem.col0;
  const int K = a.w.K;
  const int n = min(16, K - k0);
  const float s = scale_at<SBF16>(mem.s, int64_t(r >> 7) * a.w.s_rs + int64_t(k0 >> 7) * a.w.s_cs);
  const uint8_t* src = mem.w + int64_t(r) * K + k0;

  uint32_t q[4] = {0, 0, 0, 0};
  if (VEC) {
    const v4u u = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src));
    q[0] = u.x; q[1] = u.y; q[2] = u.z; q[3] = u.w;
  } else {
    for (int i = 0; i < n; ++i) q[i >> 2] |= uint32_t(src[i]) << (8 * (i & 3));
  }
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2bf lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, false);
    const v2bf hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, true);
    v[4 * i] = bf16_to_f32(lo[0]) * s;
    v[4 * i + 1] = bf16_to_f32(lo[1]) * s;
    v[4 * i + 2] = bf16_to_f32(hi[0]) * s;
    v[4 * i + 3] = bf16_to_f32(hi[1]) * s;
  }

  const int64_t off = int64_t(row) * a.ldo + k0;
  if (OBF16) {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = bf16_pair(v[2 * i], v[2 * i + 1]);
    uint16_t* dst = static_cast<uint16_t*>(a.out) + off;
    if (VEC) {
      __builtin_nontemporal_store(u4v{p[0], p[1], p[2], p[3]}, reinterpret_cast<u4v*>(dst));
      __builtin_nontemporal_store(u4v{p[4], p[5], p[6], p[7]}, reinterpret_cast<u4v*>(dst) + 1);
    } else {
      for (int i = 0; i < n; ++i) dst[i] = uint16_t(p[i >> 1] >> (16 * (i & 1)));
    }
  } else {
    float* dst = static_cast<float*>(a.out) + off;
    if (VEC) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_nontemporal_store(u4v{__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                                        __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3])},
                                    reinterpret_cast<u4v*>(dst) + i);
    } else {
      for (int i = 0; i < n; ++i) dst[i] = v[i];
    }
  }
}

using UpcastKernel = void (*)(UpcastArgs);

template <bool VEC>
UpcastKernel pick(bool sbf16, bool obf16) {
  if (sbf16) return obf16 ? upcast_kernel<VEC, true, true> : upcast_kernel<VEC, true, false>;
  return obf16 ? upcast_kernel<VEC, false, true> : upcast_kernel<VEC, false, false>;
}

}  // namespace

bsf8_status launch_upcast(const WeightDev& w, int64_t n_total, bool vec, void* out, bool out_bf16, int64_t ldo,
                          hipStream_t stream) {
  UpcastArgs a{};
  a.w = w;
  a.out = out;
  a.ldo = ldo;
  a.chunks = uint32_t((w.K + 15) / 16);
  const int64_t total = n_total * int64_t(a.chunks);
  if (total >= (int64_t(1) << 32) - UP_THREADS) {
    set_error("UNSUPPORTED: upcast of %lld 16-element pieces exceeds 2^32", (long long)total);
    return BSF8_E_UNSUPPORTED;
  }
  a.total = uint32_t(total);
  const dim3 grid(unsigned((total + UP_THREADS - 1) / UP_THREADS));
  const UpcastKernel kern = vec ? pick<true>(w.scale_bf16 != 0, out_bf16) : pick<false>(w.scale_bf16 != 0, out_bf16);
  hipLaunchKernelGGL(kern, grid, dim3(UP_THREADS), 0, stream, a);
  return device_status(hipGetLastError(), "upcast launch");
}

}  // namespace bsf8

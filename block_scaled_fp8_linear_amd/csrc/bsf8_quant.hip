// Per-token 1x128 activation quantization to OCP E4M3 (gfx950).
//
// ("Module w8a8_prefill", section "WHY (#917 / #928)": per-token F32 scales over
//  groups of 128 channels; "FP8 Native Serving", section "FP8 E4M3: range and
//  quirks": finite range +-448, no infinity.)
//
// One group of 128 channels is handled by the lanes of one 16-byte load each:
// 32 lanes of 4 F32 channels (half a wave) or 16 lanes of 8 BF16 channels (a
// quarter), so every global access is a coalesced 16-byte load and a 4- or
// 8-byte store.  (With BF16 in 8-byte loads the fused GLU step, which reads
// the gate and the up half, ran at 33.5 us where this layout takes less;
// see the launch.)  A slot of lanes takes two or four consecutive groups (four
// for large tensors) and issues all their loads before processing any, so
// each lane has several loads in flight.
// The group amax is a butterfly inside the group's lanes.  The arithmetic is
// the defined one: s = max(amax, 1e-10) / 448 in F32 (IEEE division, hipcc's
// default), f = x / s with the IEEE F32 quotient, clamp to +-448, then the
// hardware RNE conversion v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950), which keeps
// the sign of zero.  The quotient is formed as fl32(x * r) in F64 with
// r = fl64(1 / s) computed once per group, which is exactly the IEEE F32
// quotient.  Write x = X 2^a and s = S 2^b with integer significands (S below
// 2^24, s is normal) and let m = (2n + 1) 2^(c-1) be an F32 rounding midpoint
// next to q = x / s, 2^c the F32 spacing there.  x/s - m equals
// (X 2^a - (2n + 1) S 2^(b+c-1)) / (S 2^b), which is never zero (a quotient of
// two 24-bit numbers is not a 25-bit odd significand) and, as q >= 2^(c+23)
// forces a >= b + c - 1, is a multiple of 2^(b+c-1) / (S 2^b): relative to q
// at least 2^-25 / S > 2^-49 (for a subnormal q at least 2^-174 in absolute
// terms).  fl64(x * r) is within 2^-51.9 of x / s relative (below 2^-178
// absolute for subnormal q), so both round to the same F32 value, zero's sign
// included.  Per channel that is two conversions and one F64 multiply instead
// of the F32 division's ten instructions.  The kernel is HBM-bound for plain activations: 4 (or 2)
// bytes in and 1 byte out per channel, plus 4 bytes per group.
//
// The GLU instance is the step between the dense FFN's gate/up GEMM and its
// down GEMM ("Module w8a8_prefill", preamble: the gate/up/down prefill arm):
// it reads the gate/up output [M, 2F] (gate in columns [0, F), up in [F, 2F)),
// forms h = silu(gate) * up in registers and quantizes h, so the activated
// tensor never goes to memory.  The activation is the gated SiLU of the Qwen
// dense FFN (the pages do not name one), evaluated in a fixed, overflow-free
// order so that the codes are reproducible: e = exp(-|g|) in F64 rounded to
// F32, t = 1 + e, q = g / t (g >= 0) or (g * e) / t, h = q * u, each an IEEE
// F32 operation.  Per channel: 2 x 4 (or 2 x 2) bytes in, 1 byte out.
#include <hip/hip_runtime.h>

#include "bsf8_internal.h"

namespace bsf8 {
namespace {

constexpr int kQuantThreads = 256;
constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxFloor = 1e-10f;
// 128-element groups per 32-lane half-wave: 4 from 2^18 groups on, else 2
// (more, smaller blocks: X [1024, 17408] 19.1 -> 18.0 us, X [1024, 5120]
// 7.5 -> 6.9 us, the GLU step 35.1 -> 33.5 us; X [8192, 7168] keeps 4, 56.4
// against 59.6 us with 2).
constexpr int64_t kManyGroups = int64_t(1) << 18;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// EPL consecutive values (one 16-byte load: 8 BF16 or 4 F32) at element off;
// zeros from element `valid` on.
template <bool BF16, int EPL>
__device__ __forceinline__ void load_lane(const void* x, int64_t off, int valid, bool vec_ok, float (&v)[EPL]) {
  static_assert(EPL * (BF16 ? 2 : 4) == 16, "one 16-byte load per lane");
  if (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + off;
    if (valid == EPL && vec_ok) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[j] = j < valid ? bf16_to_f32(p[j]) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(x) + off;
    if (valid == EPL && vec_ok) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[j] = j < valid ? p[j] : 0.0f;
    }
  }
}

// four channels of the quantizer's unit of work, kept for the activation alone
template <bool BF16>
__device__ __forceinline__ void load4(const void* x, int64_t off, int valid, bool vec_ok, float v[4]) {
  if (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + off;
    if (valid == 4 && vec_ok) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = __uint_as_float(u.x << 16);
      v[1] = __uint_as_float(u.x & 0xFFFF0000u);
      v[2] = __uint_as_float(u.y << 16);
      v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = j < valid ? bf16_to_f32(p[j]) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(x) + off;
    if (valid == 4 && vec_ok) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = j < valid ? p[j] : 0.0f;
    }
  }
}

// h = silu(g) * u in the fixed order above (no contraction: no product is
// followed by an add).
__device__ __forceinline__ float silu_glu(float g, float u) {
  const float e = static_cast<float>(exp(-fabs(static_cast<double>(g))));
  const float t = 1.0f + e;
  const float q = g >= 0.0f ? g / t : (g * e) / t;
  return q * u;
}

// GLU: x is the gate/up output; K = F, the up half starts at column K.
template <bool BF16, bool GLU, int kGroupsPerSlot>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(const void* __restrict__ x, int32_t M, int32_t K,
                                                                  int64_t ldx, uint8_t* __restrict__ xq, int64_t ldq,
                                                                  float* __restrict__ xs, int64_t xs_sm, int64_t xs_sk,
                                                                  int32_t Kb,
                                                                  int32_t x_vec, int32_t q_vec) {
  // A group of 128 channels is held by LPG aligned lanes, EPL channels each
  // (one 16-byte load: 32 lanes of 4 F32 or 16 lanes of 8 BF16), so a wave has
  // SLOTS group slots.  Each slot quantizes kGroupsPerSlot consecutive groups
  // (row-major over tokens and groups), loading all of them before any is
  // processed so that several loads per lane are in flight.
  constexpr int EPL = BF16 ? 8 : 4;
  constexpr int LPG = kBlock / EPL;
  constexpr int SLOTS = 64 / LPG;
  const int lane = threadIdx.x & 63;
  const int lg = lane & (LPG - 1);
  const int64_t n_groups = int64_t(M) * Kb;
  const int64_t g0 =
      ((int64_t(blockIdx.x) * (kQuantThreads / 64) + (threadIdx.x >> 6)) * SLOTS + lane / LPG) * kGroupsPerSlot;
  // Token row and group column of the slot's first group: one division, in 32
  // bits whenever the group count allows (a 64-bit division is about a hundred
  // instructions, as many as the arithmetic of the group's channels); the
  // following groups step along the row and wrap to the next ones.
  int64_t mrow0;
  int32_t gcol0;
  if (n_groups <= int64_t(INT32_MAX)) {
    const uint32_t gg = uint32_t(g0), q = gg / uint32_t(Kb);
    mrow0 = q;
    gcol0 = int32_t(gg - q * uint32_t(Kb));
  } else {
    mrow0 = g0 / Kb;
    gcol0 = int32_t(g0 - mrow0 * Kb);
  }
  float v[kGroupsPerSlot][EPL];
  int64_t mrow[kGroupsPerSlot];
  int32_t gcol[kGroupsPerSlot], kk[kGroupsPerSlot], valid[kGroupsPerSlot];
#pragma unroll
  for (int j = 0; j < kGroupsPerSlot; ++j) {
    const int64_t gi = g0 + j;
    const bool live = gi < n_groups;
    int32_t gc = gcol0 + j;
    int64_t mr = mrow0;
#pragma unroll
    for (int t = 0; t < j; ++t)   // at most j rows further on (when Kb < j + 1)
      if (gc >= Kb) {
        gc -= Kb;
        ++mr;
      }
    mrow[j] = live ? mr : 0;
    gcol[j] = live ? gc : 0;
    kk[j] = gcol[j] * kBlock + lg * EPL;
    valid[j] = live ? max(0, min(EPL, K - kk[j])) : 0;
    load_lane<BF16, EPL>(x, mrow[j] * ldx + kk[j], valid[j], x_vec != 0, v[j]);
    if (GLU) {
      float u[EPL];
      load_lane<BF16, EPL>(x, mrow[j] * ldx + K + kk[j], valid[j], x_vec != 0, u);
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[j][e] = silu_glu(v[j][e], u[e]);   // lanes past K: silu(0) * 0 = 0
    }
  }
#pragma unroll
  for (int j = 0; j < kGroupsPerSlot; ++j) {
    if (g0 + j >= n_groups) break;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
#pragma unroll
    for (int d = LPG / 2; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, LPG));
    const float s = fmaxf(amax, kAmaxFloor) / kE4M3Max;
    const double rs = 1.0 / static_cast<double>(s);   // fl64(1 / s), once per group
    uint32_t packed[EPL / 4];
#pragma unroll
    for (int w = 0; w < EPL / 4; ++w) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float qv = static_cast<float>(static_cast<double>(v[j][4 * w + e]) * rs);   // = the IEEE F32 quotient v / s
        f[e] = fminf(fmaxf(qv, -kE4M3Max), kE4M3Max);
      }
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], pk, true);
      packed[w] = uint32_t(pk);
    }
    uint8_t* q = xq + mrow[j] * ldq + kk[j];
    if (valid[j] == EPL && q_vec) {
      if (EPL == 8)
        *reinterpret_cast<uint2*>(q) = make_uint2(packed[0], packed[EPL / 4 - 1]);
      else
        *reinterpret_cast<uint32_t*>(q) = packed[0];
    } else {
      for (int e = 0; e < valid[j]; ++e) q[e] = uint8_t(packed[e >> 2] >> (8 * (e & 3)));
    }
    if (lg == 0) xs[mrow[j] * xs_sm + gcol[j] * xs_sk] = s;
  }
}

// The activation itself, h = silu(g) * u in F32, for callers that need it
// unquantized (the W8A16 down projection at decode).  One thread per four
// channels of a token; y is the gate/up output [M, 2F], h is [M, F] (pitch ldh).
template <bool BF16>
__global__ __launch_bounds__(kQuantThreads) void glu_act_kernel(const void* __restrict__ y, int32_t M, int32_t F,
                                                                int64_t ldy, float* __restrict__ h, int64_t ldh,
                                                                int32_t y_vec, int32_t h_vec) {
  const int32_t per_row = (F + 3) >> 2;
  const int64_t i = int64_t(blockIdx.x) * kQuantThreads + threadIdx.x;
  if (i >= int64_t(M) * per_row) return;
  const int64_t m = i / per_row;
  const int32_t f0 = int32_t(i - m * per_row) * 4;
  const int valid = min(4, F - f0);
  float g[4], u[4];
  load4<BF16>(y, m * ldy + f0, valid, y_vec != 0, g);
  load4<BF16>(y, m * ldy + F + f0, valid, y_vec != 0, u);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = silu_glu(g[e], u[e]);
  float* out = h + m * ldh + f0;
  if (valid == 4 && h_vec) {
    *reinterpret_cast<float4*>(out) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    for (int e = 0; e < valid; ++e) out[e] = v[e];
  }
}

}  // namespace

namespace {

// glu: x is the gate/up output [M, 2K] and the quantized tensor is silu(gate) * up.
bsf8_status launch_quant(const void* x, bool x_bf16, bool glu, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                         int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, hipStream_t stream) {
  const int32_t Kb = int32_t((K + kBlock - 1) / kBlock);
  const int64_t n_groups = M * Kb;
  const int gph = n_groups >= kManyGroups ? 4 : 2;
  const int slots_per_wave = x_bf16 ? 4 : 2;   // 16 or 32 lanes per group
  const int64_t per_block = int64_t(kQuantThreads / 64) * slots_per_wave * gph;
  const int64_t grid64 = (n_groups + per_block - 1) / per_block;
  if (grid64 > INT32_MAX) {
    set_error("UNSUPPORTED: %lld activation groups", (long long)n_groups);
    return BSF8_E_UNSUPPORTED;
  }
  const int grid = int(grid64);
  const size_t esz = x_bf16 ? 2 : 4;
  const int64_t epl = x_bf16 ? 8 : 4;   // channels per lane: one 16-byte load
  // 16-byte loads: the base, every row and (GLU) the up half's offset aligned
  const int x_vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && ((ldx * int64_t(esz)) % 16 == 0) &&
                    (!glu || K % epl == 0);
  // a lane's epl codes in one store
  const int q_vec = (reinterpret_cast<uintptr_t>(xq) % epl == 0) && (ldq % epl == 0);
  using Kern = void (*)(const void*, int32_t, int32_t, int64_t, uint8_t*, int64_t, float*, int64_t, int64_t, int32_t,
                        int32_t, int32_t);
  const Kern kern = gph == 4 ? (x_bf16 ? (glu ? quant_act_kernel<true, true, 4> : quant_act_kernel<true, false, 4>)
                                       : (glu ? quant_act_kernel<false, true, 4> : quant_act_kernel<false, false, 4>))
                             : (x_bf16 ? (glu ? quant_act_kernel<true, true, 2> : quant_act_kernel<true, false, 2>)
                                       : (glu ? quant_act_kernel<false, true, 2> : quant_act_kernel<false, false, 2>));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kQuantThreads), 0, stream, x, int32_t(M), int32_t(K), ldx, xq, ldq, xs,
                     xs_sm, xs_sk, Kb, x_vec, q_vec);
  return device_status(hipGetLastError(), glu ? "quant_glu launch" : "quant_act launch");
}

}  // namespace

bsf8_status launch_quant_act(const void* x, bool x_bf16, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                             int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, hipStream_t stream) {
  return launch_quant(x, x_bf16, false, M, K, ldx, xq, ldq, xs, xs_sm, xs_sk, stream);
}

bsf8_status launch_quant_glu(const void* y, bool y_bf16, int64_t M, int64_t F, int64_t ldy, uint8_t* xq,
                             int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, hipStream_t stream) {
  return launch_quant(y, y_bf16, true, M, F, ldy, xq, ldq, xs, xs_sm, xs_sk, stream);
}

}  // namespace bsf8

namespace bsf8 {

bsf8_status launch_glu_act(const void* y, bool y_bf16, int64_t M, int64_t F, int64_t ldy, float* h, int64_t ldh,
                           hipStream_t stream) {
  const int64_t threads = M * ((F + 3) / 4);
  const int64_t grid64 = (threads + kQuantThreads - 1) / kQuantThreads;
  if (grid64 > INT32_MAX || F > INT32_MAX || M > INT32_MAX) {
    set_error("UNSUPPORTED: %lld x %lld activations", (long long)M, (long long)F);
    return BSF8_E_UNSUPPORTED;
  }
  const size_t esz = y_bf16 ? 2 : 4;
  const int y_vec = (reinterpret_cast<uintptr_t>(y) % (4 * esz) == 0) && ((ldy * esz) % (4 * esz) == 0) && F % 4 == 0;
  const int h_vec = (reinterpret_cast<uintptr_t>(h) % 16 == 0) && (ldh % 4 == 0);
  hipLaunchKernelGGL(y_bf16 ? glu_act_kernel<true> : glu_act_kernel<false>, dim3(unsigned(grid64)),
                     dim3(kQuantThreads), 0, stream, y, int32_t(M), int32_t(F), ldy, h, ldh, y_vec, h_vec);
  return device_status(hipGetLastError(), "glu_act launch");
}

}  // namespace bsf8

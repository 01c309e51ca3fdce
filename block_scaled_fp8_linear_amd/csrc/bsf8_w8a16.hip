// W8A16/F32 block operator: F32 activations, resident E4M3 weights, the block
// multiplier applied inside the reduction, F32 accumulation.
//
// ("Qwen checkpoints with block FP8 weights", block-path paragraph: original
//  quantized weights stay resident, block multipliers inside the projection
//  reduction, F32 activations and accumulation, no requantization; operator
//  paragraph: one operator for decode and prefill, grouped members keep their
//  own block-row origin.)
//
// Design for CDNA4.  At decode sizes this is an HBM stream of the weight bytes.
// Kernels by token count (16-byte aligned operands):
//  * 1 token: F32 FMAs on the vector ALUs against weights decoded exactly to
//    F32 in registers (w8a16_m1_kernel; w8a16_m1_ring_kernel beyond five chunks
//    per wave);
//  * 2 to 16 tokens: the few-token MFMA kernel (w8a16_small_m_kernel);
//  * (the W8A8 arm's E4M3 activations at one to 48 tokens take the same
//    two kernels: codes decoded exactly, each chunk partial scaled by activation
//    scale x weight scale);
//  * many tokens, once 256-row x 64-token tiles fill half the compute units:
//    the LDS-staged GEMM (w8a16_gemm_kernel);
//  * the tokens in between, or any unaligned operand: the general MFMA kernel.
// A plain F32 FMA loop needs ~M FMAs per weight byte, which beyond four tokens
// outweighs the stream, so there the products run on the BF16 matrix cores
// without losing any activation bit:
//  * every E4M3 value is exact in BF16 (v_cvt_scalef32_pk_bf16_fp8, scale 1.0);
//  * every F32 activation is split exactly as x = hi + mid + lo with three BF16
//    values (truncate to the top 16 bits twice; each remainder is exact in F32
//    and the last one has at most 8 significant bits);
//  * BF16 x BF16 products are exact in F32 and the MFMA accumulates in F32.
//  So the arithmetic is F32 activations times exact FP8 weights with F32
//  accumulation, as the pages state, at about three BF16 MFMAs per 16x16x32 step.
//  (Inputs below ~2^-100 in magnitude may lose their lowest remainder bits.)
//
// Work decomposition of the general kernel (the others, described where they
// are defined, follow the same pattern; no inter-block traffic):
//  * A block owns 32 consecutive rows of one member (two 16-row MFMA tiles,
//    member-local, so each tile lies in one row of that member's scale grid
//    and its weight scale is one scalar per 128-wide K chunk), up to 16 tokens,
//    and all of K.  Its 8 waves split K: wave w takes a contiguous run of
//    128-wide chunks.  Per chunk a lane loads its two 16-byte pieces of each of
//    the two row tiles and 32 activations, splits the activations into three
//    BF16 B fragments in registers (shared by both row tiles), converts the
//    weights and issues 24 MFMAs; the chunk partial is scaled by the tile's
//    weight scale into the F32 accumulator.  Loads run one chunk ahead.
//  * The 8 per-wave partial tiles are added in LDS in wave order (a fixed
//    order, so results are reproducible) and stored.
//  * At decode shapes (N = 8144 rows -> 256 blocks of 32 rows) that is about
//    one block per CU, and the weight stream is the only HBM traffic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <string>
#include <type_traits>

#include "bsf8_internal.h"

// Raw buffer load of 16 bytes; an offset past the resource's size reads zeros.
typedef int bsf8_w16_v4i __attribute__((ext_vector_type(4)));
__device__ bsf8_w16_v4i bsf8_raw_buffer_load_b128(bsf8_w16_v4i rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ int bsf8_raw_buffer_load_b32(bsf8_w16_v4i rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.i32");
__device__ short bsf8_raw_buffer_load_b16(bsf8_w16_v4i rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.i16");

namespace bsf8 {
namespace {

// Cache policy (the buffer instructions' aux field) of the weight loads.  The
// few-token kernels read every weight byte once per launch, so their loads are
// non-temporal (nt): 5120x5120 at one token 8.5 -> 7.7 us, Q/K/V 11.4 -> 10.2
// us, the FFN down projection 24.4 -> 22.5 us.  The general kernel reads each
// weight row once per token tile and keeps the default policy (nt made it
// 324 -> 445 us at M = 512).
constexpr int kStreamLoadAux = 2;   // nt
constexpr int kReuseLoadAux = 0;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef bsf8_w16_v4i v4i;

__device__ __forceinline__ v4i make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32)));
  r[2] = __builtin_amdgcn_readfirstlane(int(bytes));
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint4 as_u4(v4i v) { return make_uint4(uint32_t(v[0]), uint32_t(v[1]), uint32_t(v[2]), uint32_t(v[3])); }
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int RT = 2;            // 16-row MFMA tiles per block (and per wave)
constexpr int ROWS = 16 * RT;    // weight rows per block
constexpr int COLS = 16;         // tokens per block
constexpr int CHUNK = 128;       // K per chunk (one scale block)
constexpr int TERMS = 3;
constexpr int STEPS = CHUNK / 32;  // MFMA K-steps per chunk
constexpr int MAX_KB = 1024;       // K up to 131072 (scale row staged in LDS)

struct Args {
  WeightDev w;
  TileMap tm;          // 32-row tiles per member; tiles = row tiles x token tiles
  const void* x;
  void* y;
  int64_t ldx;
  int64_t ldy;
  int32_t M;
  int32_t col_tiles;
  int32_t chunks_per_wave;
  int32_t x_bf16;
  int32_t y_bf16;
  int32_t rows_per_block;   // few-token VALU kernels: rows of a block (at most 8 G)
  // E4M3-activation instances (the W8A8 arm at one to 48 tokens): the
  // per-token group scales, element (m, kb) at xs[m * xs_sm + kb * xs_sk]
  const float* xs;
  int64_t xs_sm;
  int64_t xs_sk;
};

// Activation kinds of the few-token VALU kernels: F32 and BF16 activations (the
// W8A16 arm), or E4M3 codes with per-token 1x128 group scales (the W8A8 arm:
// the products of decoded codes are exact in F32, each chunk's partial is
// scaled by activation scale x weight scale), or one token of F32 / BF16
// activations that the one-token kernels quantize to those codes and scales
// themselves (the W8A8 arm with the activation quantization in the same call).
constexpr int XK_F32 = 0, XK_BF16 = 1, XK_E4M3 = 2, XK_F32Q = 3, XK_BF16Q = 4;
template <int XK>
constexpr bool xk_quantize() { return XK == XK_F32Q || XK == XK_BF16Q; }
// bytes per activation element in memory
template <int XK>
constexpr uint32_t xk_bytes() { return XK == XK_E4M3 ? 1u : XK == XK_BF16 || XK == XK_BF16Q ? 2u : 4u; }
// 16-byte activation loads per lane and chunk in the one-token kernels' main loop
// (a quantizing instance reads the codes it staged, one 16-byte piece)
template <int XK>
constexpr int xk_loads() { return XK == XK_E4M3 || xk_quantize<XK>() ? 1 : XK == XK_BF16 ? 2 : 4; }

// ---- Per-token 1x128 activation quantization inside the one-token kernels
// ("Module w8a8_prefill", WHY: amax / 448 per 128-wide group of a token, E4M3
// with round-to-nearest-even, saturating).  A wave quantizes its own K range
// once before it streams weights: lane slot q of a round takes 16-byte piece
// q % 8 (16 activations) of chunk q / 8, so the 8 lanes of a chunk hold its
// group, and writes the 16 codes and, from its first lane, the group's scale
// to the wave's LDS region; the main loop then reads them as it would read
// quantized activations from memory.  The arithmetic is the activation
// quantizer's, step for step, so codes and scales are bit-identical to its
// output: s = max(amax, 1e-10) / 448 as an IEEE F32 division, the quotient x / s
// formed exactly as fl32(x * fl64(1 / s)) (the quantizer's comments show why
// that is the IEEE F32 quotient), clamped to +-448 in the same order, rounded
// by v_cvt_pk_fp8_f32.  Values past K load as zeros, as there.
constexpr int QROUND_MAX = 8;                        // 64 slots per round: up to 64 chunks per wave
constexpr int QCHUNKS_MAX = QROUND_MAX * 64 / 8;

// Issues the loads of RB rounds of slots from slot r0 (16 activations of one
// piece per lane and round, raw); zeros past the range or past K.
template <int XK, int RB>
__device__ __forceinline__ void quant_issue(v4i rx, uint32_t x_bytes, int K, int c_begin, int nch, int lane, int r0,
                                            uint4 (&raw)[RB][4]) {
  constexpr uint32_t XE = xk_bytes<XK>();
  constexpr int NL = XE == 4 ? 4 : 2;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int slot = r0 + 64 * b + lane;
    const int cl = slot >> 3, pc = slot & 7;
    const uint32_t k = uint32_t(c_begin + cl) * CHUNK + 16u * pc;
    const bool ok = cl < nch && int(k) < K;
#pragma unroll
    for (int q = 0; q < NL; ++q) raw[b][q] = as_u4(bsf8_raw_buffer_load_b128(rx, int(ok ? k * XE + 16u * q : x_bytes), 0, 0));
  }
}

// Quantizes the slots whose loads quant_issue made: a lane's 16 values are an
// eighth of its chunk's group (8 aligned lanes); the codes and the group's
// scale go to the wave's LDS region, codes[slot] and scales[chunk], for the
// region's cap chunks.
template <int XK, int RB>
__device__ __forceinline__ void quant_store(int nch, int cap, int lane, int r0, const uint4 (&raw)[RB][4],
                                            uint4* codes, float* scales) {
  constexpr bool W4 = xk_bytes<XK>() == 4;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    float v[16];
#pragma unroll
    for (int q = 0; q < (W4 ? 4 : 2); ++q) {
      const uint32_t w4[4] = {raw[b][q].x, raw[b][q].y, raw[b][q].z, raw[b][q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (W4) {
          v[4 * q + e] = __uint_as_float(w4[e]);
        } else {
          v[8 * q + 2 * e] = __uint_as_float(w4[e] << 16);
          v[8 * q + 2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
        }
      }
    }
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(v[e]));
#pragma unroll
    for (int d = 1; d < 8; d <<= 1) am = fmaxf(am, __shfl_xor(am, d));
    const float s = fmaxf(am, 1e-10f) / 448.0f;
    const double rs = 1.0 / static_cast<double>(s);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        f[e] = fminf(fmaxf(static_cast<float>(static_cast<double>(v[4 * q + e]) * rs), -448.0f), 448.0f);
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], packed, true);
      w[q] = uint32_t(packed);
    }
    // slots past the range hold zero codes, so a chunk read past it adds nothing
    const int slot = r0 + 64 * b + lane;
    if (slot < cap * 8) {
      codes[slot] = make_uint4(w[0], w[1], w[2], w[3]);
      if ((slot & 7) == 0) scales[slot >> 3] = s;
    }
  }
}

template <bool SBF16>
__device__ __forceinline__ float load_scale(const void* s, int64_t idx) {
  if (SBF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(s)[idx]) << 16);
  return static_cast<const float*>(s)[idx];
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// K offsets held by lane group gq within a 128-wide chunk: two runs of 16,
// [16 gq, 16 gq + 16) and [64 + 16 gq, 64 + 16 gq + 16).  K-step s uses
// elements (s >> 1) * 64 + 16 gq + (s & 1) * 8 + j, j < 8, on BOTH operands,
// so every k is covered once whatever order the MFMA sums in.

// 16 weight bytes of one row at K offset k; zeros past K or for a missing row.
template <bool ALIGNED>
__device__ __forceinline__ uint4 load_w16(const uint8_t* row, int k, int K, bool ok) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (!ok) return v;
  const int n = K - k;
  if (ALIGNED) {
    if (n >= 16) v = *reinterpret_cast<const uint4*>(row + k);
  } else if (n > 0) {
    uint32_t b[4] = {0, 0, 0, 0};
    const int cnt = n < 16 ? n : 16;
    for (int i = 0; i < cnt; ++i) b[i >> 2] |= uint32_t(row[k + i]) << (8 * (i & 3));
    v = make_uint4(b[0], b[1], b[2], b[3]);
  }
  return v;
}

// 16 activations of one token starting at K offset k, as F32; zeros past K or for a missing token.
template <bool ALIGNED, bool bf16>
__device__ __forceinline__ void load_x16(const void* x, int64_t off, int n, bool ok, float v[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = 0.f;
  if (!ok || n <= 0) return;
  if (ALIGNED && n < 16) return;   // K % 16 == 0: a 16-run is either whole or past K
  if (bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + off;
    if (ALIGNED) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 u = reinterpret_cast<const uint4*>(p)[q];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[q * 8 + 2 * h] = __uint_as_float(w[h] << 16);
          v[q * 8 + 2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
        }
      }
    } else {
      for (int j = 0; j < 16 && j < n; ++j) v[j] = __uint_as_float(uint32_t(p[j]) << 16);
    }
  } else {
    const float* p = static_cast<const float*>(x) + off;
    if (ALIGNED) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 u = reinterpret_cast<const float4*>(p)[q];
        v[4 * q] = u.x; v[4 * q + 1] = u.y; v[4 * q + 2] = u.z; v[4 * q + 3] = u.w;
      }
    } else {
      for (int j = 0; j < 16 && j < n; ++j) v[j] = p[j];
    }
  }
}

// x = hi + mid + lo exactly, each a BF16 (top 16 bits of an F32); returns the
// three terms of 8 activations packed as BF16 pairs.
__device__ __forceinline__ void split8(const float* v, v8bf& t0, v8bf& t1, v8bf& t2) {
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t hb = __float_as_uint(v[j]) & 0xFFFF0000u;
    const float r1 = v[j] - __uint_as_float(hb);
    const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
    h[j] = hb;
    m[j] = mb;
    l[j] = __float_as_uint(r1 - __uint_as_float(mb));
  }
  uint32_t p0[4], p1[4], p2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p0[q] = (h[2 * q] >> 16) | (h[2 * q + 1] & 0xFFFF0000u);
    p1[q] = (m[2 * q] >> 16) | (m[2 * q + 1] & 0xFFFF0000u);
    p2[q] = (l[2 * q] >> 16) | (l[2 * q + 1] & 0xFFFF0000u);
  }
  t0 = __builtin_bit_cast(v8bf, make_uint4(p0[0], p0[1], p0[2], p0[3]));
  t1 = __builtin_bit_cast(v8bf, make_uint4(p1[0], p1[1], p1[2], p1[3]));
  t2 = __builtin_bit_cast(v8bf, make_uint4(p2[0], p2[1], p2[2], p2[3]));
}

__device__ __forceinline__ v8bf cvt8(uint32_t lo, uint32_t hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool ALIGNED, bool XBF16, bool SBF16, int RTT>
__global__ __launch_bounds__(THREADS) void w8a16_kernel(Args a) {
  constexpr int RT = RTT;          // 16-row MFMA tiles per block (and per wave)
  constexpr int ROWS = 16 * RT;    // weight rows per block (32 or 64: within one 128-row scale block)
  __shared__ __attribute__((aligned(16))) float red[WAVES][RT][64][4];
  __shared__ float srow[MAX_KB];   // this block's row of the scale grid

  // ---- block -> (member, 32-row tile, token tile)
  const int tile = blockIdx.x;
  int mi = 0;
  while (mi + 1 < a.w.n_members && tile >= a.tm.tile0[mi + 1]) ++mi;
  const int local = tile - a.tm.tile0[mi];
  const int rtile = local % a.tm.n_tiles[mi];
  const int ct = local / a.tm.n_tiles[mi];
  const MemberDev mem = a.w.m[mi];
  const int K = a.w.K, Kb = a.w.Kb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so the chunk loop is scalar
  const int l16 = lane & 15, gq = lane >> 4;
  // The block's 16-row tiles lie in one 128-row block (ROWS divides 128), so
  // the block uses one row of the member's scale grid: stage it in LDS once.
  {
    const int64_t sr = int64_t((rtile * ROWS) >> 7) * a.w.s_rs;
    for (int i = tid; i < Kb; i += THREADS) srow[i] = load_scale<SBF16>(mem.s, sr + int64_t(i) * a.w.s_cs);
  }
  __syncthreads();
  const int c_begin = min(Kb, wave * a.chunks_per_wave);
  const int c_end = min(Kb, c_begin + a.chunks_per_wave);

  // weight rows of this lane in the two row tiles, and their scale rows
  // (A lane's weight row l16 and the outputs it accumulates, rows 4*gq + r for
  // token l16, are different things; the scale belongs to the whole block.)
  const uint8_t* wrow[RT];
  bool row_ok[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r0 = rtile * ROWS + t * 16;
    row_ok[t] = r0 + l16 < mem.rows;
    wrow[t] = mem.w + int64_t(row_ok[t] ? r0 + l16 : 0) * K;
  }
  // activations of this lane's token
  const int m = ct * COLS + l16;
  const bool m_ok = m < a.M;
  const int64_t x_base = int64_t(m_ok ? m : 0) * a.ldx;

  v4f acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 wv[RT][2];
  float xv[2][16];
  // Aligned path: buffer loads whose out-of-range offsets (missing rows, tokens
  // past M, K past the end) read zeros, so no load sits behind a branch and the
  // compiler can count the one-chunk-ahead prefetch instead of draining it.
  const uint32_t w_bytes = uint32_t(mem.rows) * uint32_t(K);
  const uint32_t x_esz = XBF16 ? 2u : 4u;
  const uint32_t x_bytes = uint32_t(a.M) * uint32_t(a.ldx) * x_esz;
  const v4i rw = make_rsrc(mem.w, w_bytes);
  const v4i rx = make_rsrc(a.x, x_bytes);
  auto load_chunk = [&](int c) {
    const int k0 = c * CHUNK + gq * 16, k1 = k0 + 64;
    if (ALIGNED) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int rb = (rtile * ROWS + t * 16 + l16) * K;
        wv[t][0] = as_u4(bsf8_raw_buffer_load_b128(rw, (row_ok[t] && k0 < K) ? rb + k0 : int(w_bytes), 0, kReuseLoadAux));
        wv[t][1] = as_u4(bsf8_raw_buffer_load_b128(rw, (row_ok[t] && k1 < K) ? rb + k1 : int(w_bytes), 0, kReuseLoadAux));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = h ? k1 : k0;
        const int xo = int((x_base + kk) * x_esz);
        const bool ok = m_ok && kk < K;
        if (XBF16) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint4 u = as_u4(bsf8_raw_buffer_load_b128(rx, ok ? xo + 16 * q : int(x_bytes), 0, 0));
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              xv[h][q * 8 + 2 * e] = __uint_as_float(w4[e] << 16);
              xv[h][q * 8 + 2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 u = as_u4(bsf8_raw_buffer_load_b128(rx, ok ? xo + 16 * q : int(x_bytes), 0, 0));
            xv[h][4 * q] = __uint_as_float(u.x);
            xv[h][4 * q + 1] = __uint_as_float(u.y);
            xv[h][4 * q + 2] = __uint_as_float(u.z);
            xv[h][4 * q + 3] = __uint_as_float(u.w);
          }
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        wv[t][0] = load_w16<ALIGNED>(wrow[t], k0, K, row_ok[t]);
        wv[t][1] = load_w16<ALIGNED>(wrow[t], k1, K, row_ok[t]);
      }
      load_x16<ALIGNED, XBF16>(a.x, x_base + k0, K - k0, m_ok, xv[0]);
      load_x16<ALIGNED, XBF16>(a.x, x_base + k1, K - k1, m_ok, xv[1]);
    }
  };

  if (c_begin < c_end) load_chunk(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    uint4 cw[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t) { cw[t][0] = wv[t][0]; cw[t][1] = wv[t][1]; }
    const float sw = srow[c];
    v8bf b[TERMS][STEPS];
    split8(&xv[0][0], b[0][0], b[1][0], b[2][0]);
    split8(&xv[0][8], b[0][1], b[1][1], b[2][1]);
    split8(&xv[1][0], b[0][2], b[1][2], b[2][2]);
    split8(&xv[1][8], b[0][3], b[1][3], b[2][3]);
    if (c + 1 < c_end) load_chunk(c + 1);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const v8bf af[STEPS] = {cvt8(cw[t][0].x, cw[t][0].y), cvt8(cw[t][0].z, cw[t][0].w),
                              cvt8(cw[t][1].x, cw[t][1].y), cvt8(cw[t][1].z, cw[t][1].w)};
      v4f pt[TERMS];
#pragma unroll
      for (int u = 0; u < TERMS; ++u) pt[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int u = 0; u < TERMS; ++u) pt[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], b[u][s], pt[u], 0, 0, 0);
      acc[t] += (pt[0] + pt[1] + pt[2]) * sw;
    }
  }

  // ---- add the 8 waves' partial tiles in wave order and store
#pragma unroll
  for (int t = 0; t < RT; ++t) *reinterpret_cast<v4f*>(&red[wave][t][lane][0]) = acc[t];
  __syncthreads();
#pragma unroll
  for (int o = tid; o < RT * 256; o += THREADS) {
    const int t = o >> 8;               // row tile
    const int ln = (o >> 2) & 63;       // lane of that tile
    const int r = o & 3;                // element
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w][t][ln][r];
    const int row = rtile * ROWS + t * 16 + 4 * (ln >> 4) + r;   // member-local output feature
    const int mo = ct * COLS + (ln & 15);
    if (row < mem.rows && mo < a.M) {
      const int64_t off = int64_t(mo) * a.ldy + mem.col0 + row;
      if (a.y_bf16) static_cast<uint16_t*>(a.y)[off] = f32_to_bf16_rne(sum);
      else static_cast<float*>(a.y)[off] = sum;
    }
  }
}


// ---------------------------------------------------------------------------
// Few tokens (M <= 16, 16-byte aligned operands; E4M3 codes up to 48): the
// decode-size kernel.  The
// general kernel's loads put each lane on one weight row (16 rows x 64 bytes
// per instruction) and its activation loads fill 16 token lanes even when
// most are past M; at decode sizes those load patterns, not the arithmetic,
// set its speed.  Here, per wave and K chunk:
//  * weights are loaded by 8 lanes per 128-byte row (full cache lines per
//    instruction), written to a wave-private LDS buffer when their chunk comes
//    up and read back in the MFMA layout;
//  * activations are loaded compactly (32 lanes per F32 token, 16 per BF16
//    token, 8 per token of E4M3 codes), each lane splits (or decodes) only what
//    it loaded, and the BF16 terms go to a wave-private LDS scratch in fragment
//    order; tokens past M read a zero row;
//  * SM_RING chunks of both operands are in flight per wave in registers, one
//    chunk: each chunk is about 8 KiB per wave (weights and activations), and
//    with more in flight the memory system only queues the requests (W
//    [5120, 5120] at M = 8: 13.9 us with 3 chunks, 13.0 with 2, 11.0 with 1;
//    Q/K/V at M = 8 with BF16 activations 10.9 -> 8.6 us);
//    loads retire in issue order, so each slot's loads are issued together and
//    slots in chunk order (scheduling barriers keep them grouped), and chunks
//    past the wave's range get past-the-end offsets (zeros, no traffic).
//    A slot is refilled as soon as its registers are written to LDS, before
//    the chunk's fragment reads, MFMAs and epilogue, which then overlap the
//    next chunk's load (refilled after them, W [5120, 5120] took 8.7 / 11.0 us
//    at two / eight F32 tokens and 8.4 / 8.6 us at two / eight E4M3 tokens,
//    now 7.7 / 10.3 and 7.7 / 7.9; the FFN down projection 21.5 / 27.7 and
//    21.2 / 21.4 us, now 18.2 / 25.6 and 18.6 / 18.9).
//    (Copies straight into LDS would save the registers, but the compiler then
//    waits for every copy in flight before any other LDS access of the wave.)
//  * the chunk scales of the wave's range are loaded once, first;
//  * the three BF16 terms of F32 activations are not three MFMA passes: they
//    fill the MFMA's otherwise idle token columns.  Column g holds term g / M of
//    token g % M, so M <= 5 takes one 16-column pass, M <= 8 two and M <= 16
//    three (a third and a sixth of the general kernel's MFMAs at five and
//    eight tokens).  Each column keeps its own F32 accumulator over the chunks,
//    and a token's three columns are added once, when the waves' partial tiles
//    are reduced (with three passes, in the activation scratch: the weight
//    buffers hold two);
//  * E4M3 codes (the W8A8 arm) decode exactly to one BF16 term, column = token,
//    and the epilogue scales each chunk partial by activation scale x weight
//    scale, the activation scale of the lane's column token loaded with the
//    chunk's slot (W [5120, 5120] at two to eight tokens 8.3-8.8 us, where the
//    F32-matrix-core kernel took 9.9 us at two to four and the GEMM 16.2 us
//    from five on; grouped Q/K/V 9.7-10.0 us against 13.0 / 19.3 us).
// In a chunk, lane group gq owns the 32 contiguous K bytes [32 gq, 32 gq + 32)
// of both operands, and K-step s of the 16x16x32 MFMA the 8 at 32 gq + 8 s.
// LDS layouts (16-byte pieces, bank-conflict free for the fragment reads):
//  weight buffer: row r of the wave's 32 at r * 128, piece p at p ^ s(r), with s
//  the permutation of r & 7 that puts even rows on {0, 1, 4, 5} and odd rows on
//  {2, 3, 6, 7}, so a fragment read's 16 lanes over two lane groups hit all 64
//  banks once (with s(r) = (r >> 1) & 7 they collide in pairs);
//  activation scratch (one row per token plus a zero row, 256 bytes each, per
//  term): term u, token t at u * (rows * 256) + t * 256, piece p at
//  p ^ ((u M + t) & 15) (the column index of that term and token in its pass).
// Per-chunk scaling and the wave-order reduction are those of the general
// kernel.
// ---------------------------------------------------------------------------
constexpr int SM_MAXM = 16;   // F32 (three columns per token, three passes) and BF16 activations
// 17 to 32 aligned F32 or BF16 tokens: two launches, the first 16 tokens on the
// few-token kernel and the rest on whichever kernel their count takes, each
// streaming the whole weight.  Against the general kernel in one launch:
// grouped Q/K/V at 17 / 24 / 32 tokens 35.0 / 35.3 / 36.4 -> 25.7 / 28.4 /
// 32.8 us, W [5120, 5120] 22.3 / 28.4 / 33.3 -> 22.1 / 24.7 / 28.8 us, the FFN
// down projection 57.4 / 75.5 / 97.7 -> 54.5 / 62.5 / 73.9 us.  (One launch
// with both token groups on the grid's second dimension reached 28.5 / 29.7 /
// 31.0, 26.1 / 26.6 / 27.4 and 66.0 / 67.6 / 71.1 us: the second group finds
// little of the weight still cached, and a 1-token group costs a full one.)
// At 48 tokens the general kernel is as fast (W [5120, 5120] 34.0 against
// 42.8 us in three launches).
constexpr int SM_SPLIT_MAXM = 32;
// E4M3 codes take one column per token, so three 16-column passes hold 48
// (W [5120, 5120] at 33-48 tokens 17.2-17.4 -> 13.0-13.7 us against the
// GEMM, grouped Q/K/V 20.9-21.5 -> 14.7-16.1 us)
constexpr int SM_MAXM_Q8 = 48;
__device__ __forceinline__ int sm_swz(int r) { return ((r & 1) << 1) | ((r >> 1) & 1) | (r & 4); }
constexpr int SM_ROW_BYTES = CHUNK * 2;        // one token's chunk as BF16
constexpr int SM_RING = 1;                    // chunks in flight per wave (the kernel takes any depth)
constexpr int SM_SCALE_REGS = 2;               // chunk scales per wave: up to 128 (K up to 131072 with 8 waves)
constexpr int SM_WBUF = ROWS * CHUNK;          // a wave's weight bytes per chunk: 4 KiB

template <int XK, bool SBF16, int NXI, int NP, int SM_DEPTH>
__global__ __launch_bounds__(THREADS) void w8a16_small_m_kernel(Args a) {
  constexpr bool XBF16 = XK == XK_BF16, XQ8 = XK == XK_E4M3;
  constexpr int NT = XK == XK_F32 ? TERMS : 1;   // a BF16 activation, or a decoded E4M3 code, is its own single term
  static_assert(NP >= 1 && NP <= 3, "one to three 16-column MFMA passes");
  constexpr int LPT = XQ8 ? 8 : XBF16 ? 16 : 32;  // lanes per token in a compact load
  constexpr int EPL = XQ8 ? 16 : XBF16 ? 8 : 4;   // activations per lane in a compact load
  // tokens per launch: one column per token for E4M3 codes and BF16, three for
  // F32 (eight tokens in two passes, sixteen in three)
  constexpr int MAXM = NT == 1 ? 16 * NP : NP == 3 ? 16 : 8;
  constexpr int ZERO_ROW = MAXM;                     // scratch row that stays zero
  constexpr int TERM_BYTES = (MAXM + 1) * SM_ROW_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t wbuf[WAVES][SM_WBUF];
  __shared__ __attribute__((aligned(16))) uint8_t scratch[WAVES][NT * TERM_BYTES];
  // the waves' partial tiles are reduced in the weight buffers, or in the
  // activation scratch when they do not fit there (three passes)
  constexpr bool RED_IN_WBUF = sizeof(float) * WAVES * RT * NP * 64 * 4 <= sizeof(uint8_t) * WAVES * SM_WBUF;
  static_assert(RED_IN_WBUF || sizeof(float) * WAVES * RT * NP * 64 * 4 <= sizeof(uint8_t) * WAVES * NT * TERM_BYTES,
                "reduction fits the buffers");

  const int tile = blockIdx.x;
  int mi = 0;
  while (mi + 1 < a.w.n_members && tile >= a.tm.tile0[mi + 1]) ++mi;
  const int rtile = tile - a.tm.tile0[mi];
  const MemberDev mem = a.w.m[mi];
  const int K = a.w.K, Kb = a.w.Kb, M = a.M;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, gq = lane >> 4;
  const int c_begin = min(Kb, wave * a.chunks_per_wave);
  const int c_end = min(Kb, c_begin + a.chunks_per_wave);
  // the block's rows: [row0, rend), at most 32, in two 16-row MFMA tiles (rows
  // past rend masked); they use at most two rows of the scale grid, the second
  // from row `split` on
  const int row0 = rtile * a.rows_per_block;
  const int rend = min(mem.rows, row0 + a.rows_per_block);
  const int srow = row0 >> 7;
  const int split = (srow + 1) << 7;
  const int64_t soff0 = int64_t(srow) * a.w.s_rs;
  const int64_t soff1 = int64_t(min(srow + 1, ((mem.rows + 127) >> 7) - 1)) * a.w.s_rs;

  uint8_t* sc = scratch[wave];
  for (int i = lane; i < NT * TERM_BYTES / 16; i += 64) reinterpret_cast<uint4*>(sc)[i] = make_uint4(0, 0, 0, 0);

  const int xt = lane / LPT;                     // token within a compact load
  const int xk = (lane % LPT) * EPL;             // first K element of the lane in the chunk
  // B operand column of this lane in pass p: g = 16 p + l16 is term g / M of
  // token g % M; columns past the last read the zero row of term 0.  The
  // 16-byte slots of term u's row of token t are permuted by the key
  // (u M + t) & 15, which differs across the 16 columns of a pass, so a
  // fragment read never meets two rows on one bank (term rows lie a multiple
  // of 256 bytes apart); the zero row takes key 15, which no live column of
  // its pass uses.
  int boff[NP], bkey[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int g = 16 * p + l16;
    const int u = g / M;
    const int tk = g - u * M;
    const bool ok = u < NT;
    boff[p] = ok ? u * TERM_BYTES + tk * SM_ROW_BYTES : ZERO_ROW * SM_ROW_BYTES;
    bkey[p] = ok ? g & 15 : 15;
  }
  // weight loads: lane L takes piece L & 7 of row (L >> 3) + 8 q of the wave's 32
  const int crow = lane >> 3;
  const int cpiece = lane & 7;
  uint8_t* const wb = wbuf[wave];

  v4f acc[RT][NP];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[t][p] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 xr[SM_DEPTH][NXI];
  uint4 wr[SM_DEPTH][2 * RT];
  const uint32_t w_bytes = uint32_t(mem.rows) * uint32_t(K);
  const uint32_t x_esz = XQ8 ? 1u : XBF16 ? 2u : 4u;
  const uint32_t x_bytes = uint32_t(M) * uint32_t(a.ldx) * x_esz;
  const uint32_t s_esz = SBF16 ? 2u : 4u;
  const uint32_t s_bytes = (a.w.s_rs ? uint32_t((mem.rows + 127) >> 7) * uint32_t(Kb) : 1u) * s_esz;
  const v4i rw = make_rsrc(mem.w, w_bytes);
  const v4i rx = make_rsrc(a.x, x_bytes);
  const v4i rs = make_rsrc(mem.s, s_bytes);
  // E4M3 activations: the group scale of this lane's column token in each
  // pass (token 16 p + l16) for each chunk, loaded with its slot
  const uint32_t xs_bytes = XQ8 ? uint32_t(((int64_t(M) - 1) * a.xs_sm + int64_t(Kb - 1) * a.xs_sk + 1) * 4) : 0u;
  const v4i rxs = make_rsrc(a.xs, xs_bytes);
  uint32_t sar[SM_DEPTH][NP];

  // The weight scales of this wave's chunks, one per lane (chunk c_begin +
  // 64 h + lane), loaded first: as the oldest loads, waiting for them never
  // waits for a ring slot.  Raw bits; converted where used.
  uint32_t sraw[2][SM_SCALE_REGS];
#pragma unroll
  for (int h = 0; h < SM_SCALE_REGS; ++h) {
    const int c = c_begin + 64 * h + lane;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int so = c < c_end ? int(((v ? soff1 : soff0) + int64_t(c) * a.w.s_cs) * s_esz) : int(s_bytes);
      sraw[v][h] = SBF16 ? uint32_t(uint16_t(bsf8_raw_buffer_load_b16(rs, so, 0, 0)))
                         : uint32_t(bsf8_raw_buffer_load_b32(rs, so, 0, 0));
    }
  }
  auto chunk_scale = [&](int c, int v) {   // c - c_begin is wave-uniform
    const int i = c - c_begin;
    uint32_t bits = 0;
#pragma unroll
    for (int h = 0; h < SM_SCALE_REGS; ++h)
      if ((i >> 6) == h) bits = __builtin_amdgcn_readlane(sraw[v][h], i & 63);
    return c < c_end ? __uint_as_float(SBF16 ? bits << 16 : bits) : 0.f;
  };
  // which of this lane's accumulator rows (16 t + 4 gq + e) use the second grid row
  uint32_t hi_rows = 0;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (row0 + 16 * t + 4 * gq + e >= split) hi_rows |= 1u << (4 * t + e);

  auto issue = [&](int c, int d) {
    const bool live = c < c_end;
    if (XQ8) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int tk = 16 * p + l16;
        const bool ok = live && tk < M;
        sar[d][p] = uint32_t(bsf8_raw_buffer_load_b32(
            rxs, ok ? int((int64_t(tk) * a.xs_sm + int64_t(c) * a.xs_sk) * 4) : int(xs_bytes), 0, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int t = i * (64 / LPT) + xt;
      const int k = c * CHUNK + xk;
      const bool ok = live && t < M && k < K;
      xr[d][i] = as_u4(bsf8_raw_buffer_load_b128(rx, ok ? int((int64_t(t) * a.ldx + k) * x_esz) : int(x_bytes), 0, 0));
    }
#pragma unroll
    for (int q = 0; q < 2 * RT; ++q) {
      const int row = row0 + 8 * q + crow;
      const int k = c * CHUNK + 16 * cpiece;
      const bool ok = live && row < rend && k < K;
      wr[d][q] = as_u4(bsf8_raw_buffer_load_b128(rw, ok ? row * K + k : int(w_bytes), 0, kStreamLoadAux));
    }
  };

#pragma unroll
  for (int d = 0; d < SM_DEPTH; ++d) {
    issue(c_begin + d, d);
    __builtin_amdgcn_sched_barrier(0);   // keep the slots in chunk order
  }
  for (int c0 = c_begin; c0 < c_end; c0 += SM_DEPTH) {
#pragma unroll
    for (int d = 0; d < SM_DEPTH; ++d) {
      const int c = c0 + d;
      const float sw0 = chunk_scale(c, 0), sw1 = chunk_scale(c, 1);
      // split this lane's activations and write the terms in fragment order
#pragma unroll
      for (int i = 0; i < NXI; ++i) {
        const int t = i * (64 / LPT) + xt;
        // slot of this lane's 16-byte K piece in term u's row: piece ^ ((u M + t) & 15)
        auto at = [&](int u) { return sc + u * TERM_BYTES + t * SM_ROW_BYTES +
                                      ((xk >> 3) ^ ((u * M + t) & 15)) * 16 + (xk & 7) * 2; };
        if (XQ8) {
          // 16 codes, decoded exactly to BF16: pieces xk / 8 and xk / 8 + 1 of the token's row
          const uint4 q = xr[d][i];
          const v8bf lo = cvt8(q.x, q.y), hi = cvt8(q.z, q.w);
          uint8_t* row = sc + t * SM_ROW_BYTES;
          const int key = t & 15;   // u M + t with u = 0
          *reinterpret_cast<uint4*>(row + (((xk >> 3) ^ key) * 16)) = __builtin_bit_cast(uint4, lo);
          *reinterpret_cast<uint4*>(row + ((((xk >> 3) + 1) ^ key) * 16)) = __builtin_bit_cast(uint4, hi);
        } else if (XBF16) {
          *reinterpret_cast<uint4*>(at(0)) = xr[d][i];
        } else {
          const float v[4] = {__uint_as_float(xr[d][i].x), __uint_as_float(xr[d][i].y), __uint_as_float(xr[d][i].z),
                              __uint_as_float(xr[d][i].w)};
          uint32_t h[4], m[4], l[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t hb = __float_as_uint(v[j]) & 0xFFFF0000u;
            const float r1 = v[j] - __uint_as_float(hb);
            const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
            h[j] = hb;
            m[j] = mb;
            l[j] = __float_as_uint(r1 - __uint_as_float(mb));
          }
          *reinterpret_cast<uint2*>(at(0)) = make_uint2((h[0] >> 16) | (h[1] & 0xFFFF0000u), (h[2] >> 16) | (h[3] & 0xFFFF0000u));
          *reinterpret_cast<uint2*>(at(1)) =
              make_uint2((m[0] >> 16) | (m[1] & 0xFFFF0000u), (m[2] >> 16) | (m[3] & 0xFFFF0000u));
          *reinterpret_cast<uint2*>(at(2)) =
              make_uint2((l[0] >> 16) | (l[1] & 0xFFFF0000u), (l[2] >> 16) | (l[3] & 0xFFFF0000u));
        }
      }
      // weights: to LDS in rows (read back in the MFMA layout below)
#pragma unroll
      for (int q = 0; q < 2 * RT; ++q) {
        const int rr = 8 * q + crow;
        *reinterpret_cast<uint4*>(wb + rr * CHUNK + ((cpiece ^ sm_swz(rr)) * 16)) = wr[d][q];
      }
      uint32_t sa_now[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) sa_now[p] = XQ8 ? sar[d][p] : 0u;
      // the slot's registers are free: refill it now, so this chunk's
      // fragment reads, MFMAs and epilogue overlap the next chunk's load
      __builtin_amdgcn_sched_barrier(0);
      issue(c + SM_DEPTH, d);
      __builtin_amdgcn_sched_barrier(0);
      // B fragments: K-step st holds K = 32 gq + 8 st + j
      v8bf b[NP][STEPS];
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        const int kc = 4 * gq + st;
#pragma unroll
        for (int p = 0; p < NP; ++p)
          b[p][st] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(sc + boff[p] + ((kc ^ bkey[p]) * 16)));
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int rr = 16 * t + l16;
        const int sw8 = sm_swz(rr);
        const uint4 lo = *reinterpret_cast<const uint4*>(wb + rr * CHUNK + (((2 * gq) ^ sw8) * 16));
        const uint4 hi = *reinterpret_cast<const uint4*>(wb + rr * CHUNK + (((2 * gq + 1) ^ sw8) * 16));
        const v8bf af[STEPS] = {cvt8(lo.x, lo.y), cvt8(lo.z, lo.w), cvt8(hi.x, hi.y), cvt8(hi.z, hi.w)};
        v4f pt[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) pt[p] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
          for (int p = 0; p < NP; ++p) pt[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st], b[p][st], pt[p], 0, 0, 0);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          v4f s4;
          if (XQ8) {
            // the W8A8 epilogue: block partial x (act scale x weight scale)
            const float sa = __uint_as_float(sa_now[p]);
            const float m0 = sa * sw0, m1 = sa * sw1;
#pragma unroll
            for (int e = 0; e < 4; ++e) s4[e] = (hi_rows >> (4 * t + e)) & 1u ? m1 : m0;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) s4[e] = (hi_rows >> (4 * t + e)) & 1u ? sw1 : sw0;
          }
          acc[t][p] += pt[p] * s4;
        }
      }
    }
  }
  // the ring's last refills (chunks past the range) are still in flight, and
  // the reduction reuses the weight buffers once every wave is done with them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- add the 8 waves' partial tiles in wave order, then a token's term
  // columns (smallest first), and store
  float(*red)[RT * NP][64][4] =
      reinterpret_cast<float(*)[RT * NP][64][4]>(RED_IN_WBUF ? &wbuf[0][0] : &scratch[0][0]);
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int p = 0; p < NP; ++p) *reinterpret_cast<v4f*>(&red[wave][t * NP + p][lane][0]) = acc[t][p];
  __syncthreads();
  const int rr = tid & 31;             // row of the block
  const int t = rr >> 4, i = rr & 15;  // row tile, row within the MFMA tile
#pragma unroll
  for (int tb = 0; tb < MAXM; tb += 16) {   // 16 token slots at a time
  const int tok = tb + (tid >> 5);
  if (tok < M) {
    float part[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int g = u * M + tok;       // column of term u
      const int p = g >> 4;
      const int ln = 16 * (i >> 2) + (g & 15);
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) s += red[w][t * NP + p][ln][i & 3];
      part[u] = s;
    }
    float sum = part[NT - 1];
#pragma unroll
    for (int u = NT - 2; u >= 0; --u) sum += part[u];
    const int row = row0 + rr;
    if (row < rend) {
      const int64_t off = int64_t(tok) * a.ldy + mem.col0 + row;
      if (a.y_bf16) static_cast<uint16_t*>(a.y)[off] = f32_to_bf16_rne(sum);
      else static_cast<float*>(a.y)[off] = sum;
    }
  }
  }
}


// ---------------------------------------------------------------------------
// One token (M = 1, 16-byte aligned operands): plain F32 dot products on the
// vector ALUs.  At one token the matrix unit saves nothing (each weight byte
// is used once) and its fragment layout costs a transpose of the weights
// through LDS; here a weight row's 128-byte K chunk is loaded by 8 lanes
// (16 bytes each, full lines), decoded exactly to F32 in registers
// (v_cvt_scalef32_pk_f32_fp8, unit scale) and multiplied by the 16
// activations that lane holds for that chunk, so there is no LDS traffic until
// the final reduction.  A block owns rb consecutive rows of one member, taken
// as G groups of 8 (the last group partly masked when rb < 8 G; rb is chosen
// so that the grid is about one block per compute unit), and all of K;
// its 8 waves split K into contiguous chunk ranges and every load of a wave is
// issued before any arithmetic.  The chunk partial of each row is scaled by
// its block scale (a block's rows span at most two rows of the grid, each
// lane picks its own) into an F32 accumulator; lanes of a row are added by
// shuffles and the 8 waves' partials in LDS in wave order (reproducible).
// ---------------------------------------------------------------------------
constexpr int M1_MAX_G = 4;

template <int XK, bool SBF16, int G, int CPW>
__global__ __launch_bounds__(THREADS) void w8a16_m1_kernel(Args a) {
  constexpr bool XBF16 = XK == XK_BF16, XQ8 = XK == XK_E4M3, XQD = xk_quantize<XK>();
  static_assert(!XQD || CPW * 8 <= 64, "a quantizing wave's range is one round of slots");
  __shared__ float red[WAVES][G * 8];
  __shared__ uint4 qcodes[WAVES][XQD ? CPW * 8 : 1];   // quantizing instances: the wave's codes and scales
  __shared__ float qscl[WAVES][XQD ? CPW : 1];
  const int tile = blockIdx.x;
  int mi = 0;
  while (mi + 1 < a.w.n_members && tile >= a.tm.tile0[mi + 1]) ++mi;
  const int rtile = tile - a.tm.tile0[mi];
  const MemberDev mem = a.w.m[mi];
  const int K = a.w.K, Kb = a.w.Kb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jp = lane & 7;    // 16-byte piece of a 128-byte chunk
  const int rl = lane >> 3;   // row within an 8-row group
  const int row0 = rtile * a.rows_per_block;
  const int rend = min(mem.rows, row0 + a.rows_per_block);   // rows from rend on: masked lanes
  const int c_begin = min(Kb, wave * CPW);
  const int c_end = min(Kb, c_begin + CPW);

  const uint32_t w_bytes = uint32_t(mem.rows) * uint32_t(K);
  const v4i rw = make_rsrc(mem.w, w_bytes);
  constexpr uint32_t XE = xk_bytes<XK>();
  const uint32_t x_bytes = uint32_t(K) * XE;
  const v4i rx = make_rsrc(a.x, x_bytes);
  constexpr int XL = xk_loads<XK>();   // 16-byte activation loads per chunk piece

  // ---- the chunk scales of the (at most two) grid rows the block's rows use,
  // issued first and without branches, so that waiting for them never waits
  // for the weight stream behind them (loads retire in order)
  const int nb = (mem.rows + 127) >> 7;
  const int srow = row0 >> 7;
  const int srow1 = min(srow + 1, nb - 1);
  // raw bits now, widened to F32 at use (a conversion here would wait for the loads)
  uint32_t sc0[CPW], sc1[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int chunk = min(c_begin + c, Kb - 1);
    const int64_t i0 = int64_t(srow) * a.w.s_rs + int64_t(chunk) * a.w.s_cs;
    const int64_t i1 = int64_t(srow1) * a.w.s_rs + int64_t(chunk) * a.w.s_cs;
    if (SBF16) {
      sc0[c] = static_cast<const uint16_t*>(mem.s)[i0];
      sc1[c] = static_cast<const uint16_t*>(mem.s)[i1];
    } else {
      sc0[c] = static_cast<const uint32_t*>(mem.s)[i0];
      sc1[c] = static_cast<const uint32_t*>(mem.s)[i1];
    }
  }
  // the token's group scale of each chunk (E4M3 activations)
  float sa[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) sa[c] = XQ8 ? a.xs[int64_t(min(c_begin + c, Kb - 1)) * a.xs_sk] : 1.f;
  __builtin_amdgcn_sched_barrier(0);

  // ---- a quantizing instance's activations go out first: they arrive long
  // before the weights and are quantized while the weight stream is in flight
  // (loads retire in order, so a wait for them never covers weights)
  uint4 qraw[1][4];
  if constexpr (XQD) quant_issue<XK, 1>(rx, x_bytes, K, c_begin, c_end - c_begin, lane, 0, qraw);
  __builtin_amdgcn_sched_barrier(0);

  // ---- every load of the wave: weights, activations (kept ahead of all arithmetic)
  uint4 wv[CPW][G];
  uint4 xr[CPW][XL];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int chunk = c_begin + c;
    const int k = chunk * CHUNK + 16 * jp;
    const bool live = chunk < c_end && k < K;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int r = row0 + 8 * g + rl;
      const uint32_t off = live && r < rend ? uint32_t(r) * uint32_t(K) + uint32_t(k) : w_bytes;
      wv[c][g] = as_u4(bsf8_raw_buffer_load_b128(rw, int(off), 0, kStreamLoadAux));
    }
    if (!XQD) {
#pragma unroll
      for (int q = 0; q < XL; ++q) {
        const uint32_t off = live ? uint32_t(k) * XE + 16u * q : x_bytes;
        xr[c][q] = as_u4(bsf8_raw_buffer_load_b128(rx, int(off), 0, 0));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XQD) {
    quant_store<XK, 1>(c_end - c_begin, CPW, lane, 0, qraw, qcodes[wave], qscl[wave]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      xr[c][0] = qcodes[wave][8 * c + jp];
      sa[c] = qscl[wave][c];
    }
  }

  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    float xv[16];
    if (XQ8 || XQD) {
      const uint32_t x4[4] = {xr[c][0].x, xr[c][0].y, xr[c][0].z, xr[c][0].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x4[e], 1.0f, false);
        const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x4[e], 1.0f, true);
        xv[4 * e] = lo[0];
        xv[4 * e + 1] = lo[1];
        xv[4 * e + 2] = hi[0];
        xv[4 * e + 3] = hi[1];
      }
    } else if (XBF16) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t w4[4] = {xr[c][q].x, xr[c][q].y, xr[c][q].z, xr[c][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[8 * q + 2 * e] = __uint_as_float(w4[e] << 16);
          xv[8 * q + 2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[4 * q] = __uint_as_float(xr[c][q].x);
        xv[4 * q + 1] = __uint_as_float(xr[c][q].y);
        xv[4 * q + 2] = __uint_as_float(xr[c][q].z);
        xv[4 * q + 3] = __uint_as_float(xr[c][q].w);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t w4[4] = {wv[c][g].x, wv[c][g].y, wv[c][g].z, wv[c][g].w};
      float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w4[e], 1.0f, false);
        const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w4[e], 1.0f, true);
        p[0] = fmaf(xv[4 * e], lo[0], p[0]);
        p[1] = fmaf(xv[4 * e + 1], lo[1], p[1]);
        p[2] = fmaf(xv[4 * e + 2], hi[0], p[2]);
        p[3] = fmaf(xv[4 * e + 3], hi[1], p[3]);
      }
      const int r = row0 + 8 * g + rl;
      const uint32_t sb = (r >> 7) == srow ? sc0[c] : sc1[c];
      const float sw = __uint_as_float(SBF16 ? sb << 16 : sb);
      acc[g] = fmaf((p[0] + p[1]) + (p[2] + p[3]), XQ8 || XQD ? sa[c] * sw : sw, acc[g]);
    }
  }
  // ---- rows: the 8 lanes of a row, then the 8 waves in order
#pragma unroll
  for (int g = 0; g < G; ++g) {
    acc[g] += __shfl_xor(acc[g], 1);
    acc[g] += __shfl_xor(acc[g], 2);
    acc[g] += __shfl_xor(acc[g], 4);
    if (jp == 0) red[wave][8 * g + rl] = acc[g];
  }
  __syncthreads();
  if (tid < G * 8) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w][tid];
    const int row = row0 + tid;
    if (row < rend) {
      const int64_t off = mem.col0 + row;
      if (a.y_bf16) static_cast<uint16_t*>(a.y)[off] = f32_to_bf16_rne(sum);
      else static_cast<float*>(a.y)[off] = sum;
    }
  }
}


// ---------------------------------------------------------------------------
// One token with a long K (more than five chunks per wave, e.g. an FFN down
// projection at decode, K = 17408): the one-token kernel's layout, but a wave
// keeps a ring of D chunk slots in flight instead of issuing all of its loads
// at once.  Each slot's loads (the row groups' 16-byte pieces and the lane's
// activations) are issued together and slots in chunk order; after a chunk is
// used its slot is refilled with the chunk D further on (loads retire in
// issue order, so waiting for one chunk never waits for a later one), and
// chunks past the wave's range read past-the-end offsets (zeros, no traffic).
// The weight scales (and the token's activation scales for E4M3 activations)
// of the wave's chunks are loaded first, one chunk per lane, and picked per
// chunk with a lane read.
// Ring depth: a slot holds about 3 KiB of weights per wave plus the lane's
// activations (4 KiB per wave for F32, 2 for BF16, 1 for E4M3), and the
// fastest depth is the one that keeps about 14-16 MB in flight over the
// chip, beyond which requests only queue: FFN down [5120, 17408] at one token
// with F32 activations took 22.5 / 20.2 / 19.7 / 19.1 us at depth 4 / 3 / 2 /
// 1, with E4M3 activations 20.4 / 18.3 / 17.3 / 19.4 us (the plain read of
// the same bytes 17.3 us).
// ---------------------------------------------------------------------------
// (a quantizing instance's slot holds weights only: its activations are staged
// in LDS before the stream starts, so it takes the E4M3 depth)
template <int XK>
constexpr int m1r_depth() { return XK == XK_F32 ? 1 : 2; }
constexpr int QRB = 4;   // rounds of quantization slots issued together by the ring kernel (32 chunks)

template <int XK, bool SBF16, int G, int D>
__global__ __launch_bounds__(THREADS) void w8a16_m1_ring_kernel(Args a) {
  constexpr bool XBF16 = XK == XK_BF16, XQ8 = XK == XK_E4M3, XQD = xk_quantize<XK>();
  __shared__ float red[WAVES][G * 8];
  // quantizing instances: the wave's codes and scales (at most QCHUNKS_MAX chunks per wave)
  __shared__ uint4 qcodes[WAVES][XQD ? QCHUNKS_MAX * 8 : 1];
  __shared__ float qscl[WAVES][XQD ? QCHUNKS_MAX : 1];
  const int tile = blockIdx.x;
  int mi = 0;
  while (mi + 1 < a.w.n_members && tile >= a.tm.tile0[mi + 1]) ++mi;
  const int rtile = tile - a.tm.tile0[mi];
  const MemberDev mem = a.w.m[mi];
  const int K = a.w.K, Kb = a.w.Kb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jp = lane & 7;
  const int rl = lane >> 3;
  const int row0 = rtile * a.rows_per_block;
  const int rend = min(mem.rows, row0 + a.rows_per_block);
  const int c_begin = min(Kb, wave * a.chunks_per_wave);
  const int c_end = min(Kb, c_begin + a.chunks_per_wave);

  const uint32_t w_bytes = uint32_t(mem.rows) * uint32_t(K);
  const v4i rw = make_rsrc(mem.w, w_bytes);
  constexpr uint32_t XE = xk_bytes<XK>();
  const uint32_t x_bytes = uint32_t(K) * XE;
  const v4i rx = make_rsrc(a.x, x_bytes);
  constexpr int XL = XQD ? 1 : xk_loads<XK>();

  // ---- scales of the wave's chunks, chunk c_begin + 64 h + lane in register h
  const int nb = (mem.rows + 127) >> 7;
  const int srow = row0 >> 7;
  const int srow1 = min(srow + 1, nb - 1);
  uint32_t s0[SM_SCALE_REGS], s1[SM_SCALE_REGS];
  float sav[SM_SCALE_REGS];
#pragma unroll
  for (int h = 0; h < SM_SCALE_REGS; ++h) {
    const int chunk = min(c_begin + 64 * h + lane, Kb - 1);
    const int64_t i0 = int64_t(srow) * a.w.s_rs + int64_t(chunk) * a.w.s_cs;
    const int64_t i1 = int64_t(srow1) * a.w.s_rs + int64_t(chunk) * a.w.s_cs;
    if (SBF16) {
      s0[h] = static_cast<const uint16_t*>(mem.s)[i0];
      s1[h] = static_cast<const uint16_t*>(mem.s)[i1];
    } else {
      s0[h] = static_cast<const uint32_t*>(mem.s)[i0];
      s1[h] = static_cast<const uint32_t*>(mem.s)[i1];
    }
    sav[h] = XQ8 ? a.xs[int64_t(chunk) * a.xs_sk] : 1.f;
  }
  // raw bits of chunk c's scale for grid row v (c - c_begin is wave-uniform); 0 past the range
  auto wscale = [&](int c, int v) {
    const int i = c - c_begin;
    uint32_t bits = 0;
#pragma unroll
    for (int h = 0; h < SM_SCALE_REGS; ++h)
      if ((i >> 6) == h) bits = __builtin_amdgcn_readlane(v ? s1[h] : s0[h], i & 63);
    return c < c_end ? __uint_as_float(SBF16 ? bits << 16 : bits) : 0.f;
  };
  auto ascale = [&](int c) {
    const int i = c - c_begin;
    float v = 1.f;
#pragma unroll
    for (int h = 0; h < SM_SCALE_REGS; ++h)
      if ((i >> 6) == h) v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sav[h]), i & 63));
    return v;
  };
  __builtin_amdgcn_sched_barrier(0);

  // ---- a quantizing instance's first QRB rounds of activations go out before
  // the weight stream (quantized while it is in flight; loads retire in order)
  const int nch = c_end - c_begin;
  uint4 qraw[XQD ? QRB : 1][4];
  if constexpr (XQD) quant_issue<XK, QRB>(rx, x_bytes, K, c_begin, nch, lane, 0, qraw);
  __builtin_amdgcn_sched_barrier(0);

  uint4 wv[D][G];
  uint4 xr[D][XL];
  auto issue = [&](int c, int d) {
    const int k = c * CHUNK + 16 * jp;
    const bool live = c < c_end && k < K;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int r = row0 + 8 * g + rl;
      const uint32_t off = live && r < rend ? uint32_t(r) * uint32_t(K) + uint32_t(k) : w_bytes;
      wv[d][g] = as_u4(bsf8_raw_buffer_load_b128(rw, int(off), 0, kStreamLoadAux));
    }
    if (!XQD) {
#pragma unroll
      for (int q = 0; q < XL; ++q) {
        const uint32_t off = live ? uint32_t(k) * XE + 16u * q : x_bytes;
        xr[d][q] = as_u4(bsf8_raw_buffer_load_b128(rx, int(off), 0, 0));
      }
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) {
    issue(c_begin + d, d);
    __builtin_amdgcn_sched_barrier(0);   // keep the slots in chunk order
  }
  if constexpr (XQD) {
    quant_store<XK, QRB>(nch, QCHUNKS_MAX, lane, 0, qraw, qcodes[wave], qscl[wave]);
    // a range beyond QRB rounds (more than 32 chunks per wave): the rest in
    // further batches, whose loads wait behind the first weight slots
    for (int r0 = 64 * QRB; r0 < nch * 8; r0 += 64 * QRB) {
      quant_issue<XK, QRB>(rx, x_bytes, K, c_begin, nch, lane, r0, qraw);
      quant_store<XK, QRB>(nch, QCHUNKS_MAX, lane, r0, qraw, qcodes[wave], qscl[wave]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }

  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
  for (int c0 = c_begin; c0 < c_end; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = c0 + d;
      const float sw0 = wscale(c, 0), sw1 = wscale(c, 1);
      // a quantizing instance's codes and scale of chunk c, from LDS (zeros past the range)
      const int cq = min(c - c_begin, QCHUNKS_MAX - 1);
      const uint4 qc = XQD && c < c_end ? qcodes[wave][8 * cq + jp] : make_uint4(0, 0, 0, 0);
      const float sa = XQ8 ? ascale(c) : XQD ? (c < c_end ? qscl[wave][cq] : 0.f) : 1.f;
      float xv[16];
      if (XQ8 || XQD) {
        const uint4 cx = XQD ? qc : xr[d][0];
        const uint32_t x4[4] = {cx.x, cx.y, cx.z, cx.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x4[e], 1.0f, false);
          const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x4[e], 1.0f, true);
          xv[4 * e] = lo[0];
          xv[4 * e + 1] = lo[1];
          xv[4 * e + 2] = hi[0];
          xv[4 * e + 3] = hi[1];
        }
      } else if (XBF16) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t w4[4] = {xr[d][q].x, xr[d][q].y, xr[d][q].z, xr[d][q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[8 * q + 2 * e] = __uint_as_float(w4[e] << 16);
            xv[8 * q + 2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[4 * q] = __uint_as_float(xr[d][q].x);
          xv[4 * q + 1] = __uint_as_float(xr[d][q].y);
          xv[4 * q + 2] = __uint_as_float(xr[d][q].z);
          xv[4 * q + 3] = __uint_as_float(xr[d][q].w);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t w4[4] = {wv[d][g].x, wv[d][g].y, wv[d][g].z, wv[d][g].w};
        float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w4[e], 1.0f, false);
          const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w4[e], 1.0f, true);
          p[0] = fmaf(xv[4 * e], lo[0], p[0]);
          p[1] = fmaf(xv[4 * e + 1], lo[1], p[1]);
          p[2] = fmaf(xv[4 * e + 2], hi[0], p[2]);
          p[3] = fmaf(xv[4 * e + 3], hi[1], p[3]);
        }
        const int r = row0 + 8 * g + rl;
        const float sw = (r >> 7) == srow ? sw0 : sw1;
        acc[g] = fmaf((p[0] + p[1]) + (p[2] + p[3]), XQ8 || XQD ? sa * sw : sw, acc[g]);
      }
      __builtin_amdgcn_sched_barrier(0);
      issue(c + D, d);   // refill this slot
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // ---- rows: the 8 lanes of a row, then the 8 waves in order
#pragma unroll
  for (int g = 0; g < G; ++g) {
    acc[g] += __shfl_xor(acc[g], 1);
    acc[g] += __shfl_xor(acc[g], 2);
    acc[g] += __shfl_xor(acc[g], 4);
    if (jp == 0) red[wave][8 * g + rl] = acc[g];
  }
  __syncthreads();
  if (tid < G * 8) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w][tid];
    const int row = row0 + tid;
    if (row < rend) {
      const int64_t off = mem.col0 + row;
      if (a.y_bf16) static_cast<uint16_t*>(a.y)[off] = f32_to_bf16_rne(sum);
      else static_cast<float*>(a.y)[off] = sum;
    }
  }
}



// ---------------------------------------------------------------------------
// Many tokens (aligned operands): an LDS-staged tile of 256 weight rows x 64
// tokens per block, so each weight byte is read once per 64 tokens and each
// activation once per 256 rows.  Per 128-wide K chunk the block copies the
// chunk's weight bytes (256 rows x 128 bytes) and activations (64 tokens x 128,
// F32 or BF16) through registers into one of two LDS stages; a chunk's loads go
// out two chunks before its use.  Its 8 waves split the tile 2
// (row halves of 128) x 4 (token quarters of 16); per 32-wide K step a wave
// reads 8 weight fragments (decoded exactly to BF16) and the token fragment's
// three BF16 terms and issues 8 x 3 MFMAs.  F32 activations are split into the
// three exact terms (as in the general kernel) once per value and block, when
// the chunk is stored: three BF16 planes, so a stage holds 32 KiB of weights
// and 48 KiB of activations and the two stages fill the 160 KiB LDS (splitting
// per wave instead, each token fragment being split by both row halves, cost
// 134 against 112 us at M = 512 in a timing variant without the split).  A wave's 128 rows lie in one
// 128-row block of its member's scale grid (tiles start at member-local
// multiples of 256), so after the chunk's 4 steps each 16x16 partial is scaled
// by one multiplier into the F32 accumulator: the arithmetic is the block
// operator's, per-chunk partial then block scale.
//
// LDS layouts (16-byte units XOR-swizzled so fragment reads are
// conflict-free): weight row r at r * 128, unit u at (u ^ ((r >> 1) & 7)) * 16
// (16 lanes reading 8 bytes of 16 consecutive rows meet 32 distinct 8-byte
// slots of the 256 bytes the 64 banks span); in each activation plane, token t
// at t * 256, unit u (8 BF16) at (u ^ (t & 15)) * 16 (16 lanes reading 16 bytes
// of 16 consecutive tokens meet 16 distinct units).
// ---------------------------------------------------------------------------
constexpr int GW_ROWS = 256;
constexpr int GW_TOKS = 64;
constexpr int GW_THREADS = 512;

struct GemmArgs {
  WeightDev w;
  int32_t rt0[kMaxMembers + 1];   // first 256-row tile of each member; rt0[n_members] = row tiles
  int32_t m_tiles;                // 64-token tiles
  const void* x;
  void* y;
  int64_t ldx;
  int64_t ldy;
  int32_t M;
  int32_t y_bf16;
  int32_t y_vec;                  // 16-byte (F32) / 8-byte (BF16) output stores allowed
  // split-K: blocks [s * tiles, (s + 1) * tiles) take K chunks [s * kb_per_split,
  // + kb_per_split) and, with more than one split, write their F32 partial of y
  // to ws + s * M * ldws (same row and column indexing as y); a second kernel
  // adds the splits in order
  int32_t splits;
  int32_t kb_per_split;
  float* ws;
  int64_t ldws;
};

template <bool XBF16, bool SBF16>
__global__ __launch_bounds__(GW_THREADS) void w8a16_gemm_kernel(GemmArgs a) {
  constexpr int XE = XBF16 ? 2 : 4;
  constexpr int NT = XBF16 ? 1 : 3;                     // BF16 planes of the activations
  constexpr int PLANE = GW_TOKS * CHUNK * 2;            // 16 KiB: 64 tokens x 128 BF16
  constexpr int A_BYTES = GW_ROWS * CHUNK;              // 32 KiB
  constexpr int STAGE = A_BYTES + NT * PLANE;           // 80 KiB (F32: two stages fill the LDS) / 48 KiB
  constexpr int A_PER = A_BYTES / 16 / GW_THREADS;      // 16-byte pieces per thread: 4
  constexpr int B_PER = GW_TOKS * CHUNK * XE / 16 / GW_THREADS;   // 4 (F32: 16 consecutive values) / 2
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tiles = a.rt0[a.w.n_members] * a.m_tiles;
  const int sp = blockIdx.x / tiles, bt = blockIdx.x - sp * tiles;
  const int R = bt / a.m_tiles, T = bt - R * a.m_tiles;
  int mi = 0;
  while (mi + 1 < a.w.n_members && R >= a.rt0[mi + 1]) ++mi;
  const MemberDev mem = a.w.m[mi];
  const int K = a.w.K, Kb = a.w.Kb;
  const int kb_begin = sp * a.kb_per_split, kb_end = min(Kb, kb_begin + a.kb_per_split);
  const int r0 = (R - a.rt0[mi]) * GW_ROWS;   // member-local first row
  const int t0 = T * GW_TOKS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 1, wc = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4;

  // ---- copies of chunk kb into a register slot, then into a stage.  Buffer loads:
  // a piece past a member's rows, past K or past M reads an offset beyond the
  // resource (zeros, no traffic), so every chunk issues the same loads.
  const uint32_t w_bytes = uint32_t(mem.rows) * uint32_t(K);
  const v4i rw = make_rsrc(mem.w, w_bytes);
  const uint32_t x_bytes = uint32_t(a.M) * uint32_t(a.ldx) * XE;
  const v4i rx = make_rsrc(a.x, x_bytes);
  uint4 ra[A_PER], rb[B_PER];
  // per piece, its byte offset in chunk 0 (past the resource for rows past the
  // member's end and tokens past M) and the first K element it holds; chunk kb
  // adds kb * 128 elements through the instruction's scalar offset
  uint32_t aoff[A_PER], boff[B_PER];
  int ak[A_PER], bk[B_PER];
#pragma unroll
  for (int j = 0; j < A_PER; ++j) {
    const int pc = tid + GW_THREADS * j;
    const int row = pc >> 3, u = pc & 7;
    ak[j] = u * 16;
    aoff[j] = r0 + row < mem.rows ? uint32_t(r0 + row) * uint32_t(K) + uint32_t(ak[j]) : w_bytes;
  }
  // activations: F32, thread (t, q) = (tid / 8, tid % 8) holds elements [16 q, 16 q + 16)
  // of token t (4 pieces); BF16, the thread holds elements [8 u, 8 u + 8) of token
  // t for u = 2 (tid % 8) and u + 1
  const int bt_t = tid >> 3, bt_q = tid & 7;
#pragma unroll
  for (int j = 0; j < B_PER; ++j) {
    bk[j] = XBF16 ? (2 * bt_q + j) * 8 : 16 * bt_q + 4 * j;
    boff[j] = t0 + bt_t < a.M ? (uint32_t(t0 + bt_t) * uint32_t(a.ldx) + uint32_t(bk[j])) * uint32_t(XE) : x_bytes;
  }
  auto load = [&](int kb) {
    const int kt = K - kb * CHUNK;   // K elements left from this chunk on (<= 0 past the last)
    const int sa = __builtin_amdgcn_readfirstlane(kb * CHUNK), sx = __builtin_amdgcn_readfirstlane(kb * CHUNK * XE);
#pragma unroll
    for (int j = 0; j < A_PER; ++j)
      ra[j] = as_u4(bsf8_raw_buffer_load_b128(rw, ak[j] < kt ? int(aoff[j]) : int(w_bytes), sa, kReuseLoadAux));
#pragma unroll
    for (int j = 0; j < B_PER; ++j)
      rb[j] = as_u4(bsf8_raw_buffer_load_b128(rx, bk[j] < kt ? int(boff[j]) : int(x_bytes), sx, 0));
  };
  auto store = [&](uint8_t* st) {
#pragma unroll
    for (int j = 0; j < A_PER; ++j) {
      const int pc = tid + GW_THREADS * j;
      const int row = pc >> 3, u = pc & 7;
      *reinterpret_cast<uint4*>(st + row * CHUNK + ((u ^ ((row >> 1) & 7)) << 4)) = ra[j];
    }
    // activation plane p, token t: 16 units of 8 BF16, unit u at (u ^ (t & 15)) * 16
    uint8_t* bp = st + A_BYTES + bt_t * (CHUNK * 2);
    if (XBF16) {
#pragma unroll
      for (int j = 0; j < B_PER; ++j)
        *reinterpret_cast<uint4*>(bp + (((2 * bt_q + j) ^ (bt_t & 15)) << 4)) = rb[j];
    } else {
      // the exact three-term split, once per value and block
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float xv[8] = {__uint_as_float(rb[2 * h].x), __uint_as_float(rb[2 * h].y), __uint_as_float(rb[2 * h].z),
                             __uint_as_float(rb[2 * h].w), __uint_as_float(rb[2 * h + 1].x),
                             __uint_as_float(rb[2 * h + 1].y), __uint_as_float(rb[2 * h + 1].z),
                             __uint_as_float(rb[2 * h + 1].w)};
        v8bf t3[3];
        split8(xv, t3[0], t3[1], t3[2]);
        const int pos = ((2 * bt_q + h) ^ (bt_t & 15)) << 4;
#pragma unroll
        for (int p = 0; p < 3; ++p) *reinterpret_cast<v8bf*>(bp + p * PLANE + pos) = t3[p];
      }
    }
  };

  // the wave's scale-grid row (its 128 rows lie in one block row; a half past the
  // member's last row reads the last grid row, its rows being zeros)
  const int srow = min((r0 + wr * 128) >> 7, (mem.rows - 1) >> 7);
  auto wscale = [&](int kb) {
    const int64_t i = int64_t(srow) * a.w.s_rs + int64_t(kb) * a.w.s_cs;
    return SBF16 ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(mem.s)[i]) << 16)
                 : static_cast<const float*>(mem.s)[i];
  };

  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  // chunk kb goes through stage (kb - kb_begin) & 1: loaded into registers two
  // chunks before its use and stored into its stage one chunk before; past the
  // split's range a load reads chunk Kb (zeros, no traffic)
  load(kb_begin);
  store(lds);
  load(kb_begin + 1 < kb_end ? kb_begin + 1 : Kb);
  const int tw = wc * 16 + l16;   // the lane's token within the tile (B fragments)
  // the fragments of K step st: 8 weight fragments decoded to BF16 and the token
  // fragment's BF16 terms (one per plane)
  auto frag = [&](const uint8_t* cur, int st, v8bf (&af)[8], v8bf (&bt)[3]) {
    const int ub = 4 * st + g;   // K elements [32 st + 8 g, + 8): one unit of each plane
#pragma unroll
    for (int p = 0; p < NT; ++p)
      bt[p] = *reinterpret_cast<const v8bf*>(cur + A_BYTES + p * PLANE + tw * (CHUNK * 2) + ((ub ^ (tw & 15)) << 4));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // row 16 i + l16 of the wave's half, K bytes 32 st + 8 g
      const int row = wr * 128 + 16 * i + l16;
      const int u = 2 * st + (g >> 1);
      const uint2 wq =
          *reinterpret_cast<const uint2*>(cur + row * CHUNK + ((u ^ ((row >> 1) & 7)) << 4) + ((g & 1) << 3));
      af[i] = cvt8(wq.x, wq.y);
    }
  };
  // a chunk: per K step the fragments, then its MFMAs with the terms outermost,
  // so 8 independent MFMAs sit between two that share an accumulator
  auto compute = [&](const uint8_t* cur, int kb) {
    const float sw = wscale(kb);
    v4f pr[8];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      v8bf af[8], bt[3];
      frag(cur, st, af, bt);
#pragma unroll
      for (int tm = 0; tm < NT; ++tm)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pr[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bt[tm],
                                                          (st == 0 && tm == 0) ? v4f{0.f, 0.f, 0.f, 0.f} : pr[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = fmaf(pr[i][r], sw, acc[i][r]);
  };
  for (int kb = kb_begin; kb < kb_end; ++kb) {
    const int j = kb - kb_begin;
    __syncthreads();   // chunk kb's stage is complete; chunk kb - 1's reads are done
    if (kb + 1 < kb_end) store(lds + ((j + 1) & 1) * STAGE);
    load(kb + 2 < kb_end ? kb + 2 : Kb);
    compute(lds + (j & 1) * STAGE, kb);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- store: lane holds rows 16 i + 4 g + r (r < 4) of the wave's half, token l16 of its quarter
  const int t = t0 + wc * 16 + l16;
  if (t >= a.M) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = r0 + wr * 128 + 16 * i + 4 * g;   // member-local row of register 0
    const int nvalid = mem.rows - n;
    if (nvalid <= 0) continue;
    if (a.splits > 1) {   // this split's F32 partial
      float* wp = a.ws + int64_t(sp) * a.M * a.ldws + int64_t(t) * a.ldws + mem.col0 + n;
      for (int r = 0; r < 4 && r < nvalid; ++r) wp[r] = acc[i][r];
      continue;
    }
    const int64_t off = int64_t(t) * a.ldy + mem.col0 + n;
    if (a.y_bf16) {
      uint16_t* yp = static_cast<uint16_t*>(a.y) + off;
      if (nvalid >= 4 && a.y_vec) {
        *reinterpret_cast<uint2*>(yp) = make_uint2(uint32_t(f32_to_bf16_rne(acc[i][0])) | (uint32_t(f32_to_bf16_rne(acc[i][1])) << 16),
                                                   uint32_t(f32_to_bf16_rne(acc[i][2])) | (uint32_t(f32_to_bf16_rne(acc[i][3])) << 16));
      } else {
        for (int r = 0; r < 4 && r < nvalid; ++r) yp[r] = f32_to_bf16_rne(acc[i][r]);
      }
    } else {
      float* yp = static_cast<float*>(a.y) + off;
      if (nvalid >= 4 && a.y_vec) {
        *reinterpret_cast<float4*>(yp) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      } else {
        for (int r = 0; r < 4 && r < nvalid; ++r) yp[r] = acc[i][r];
      }
    }
  }
}

struct Plan {
  TileMap tm;
  int col_tiles;
  int tiles;
  int chunks_per_wave;
  int rt;   // general kernel: 16-row tiles per block
};

// The general kernel re-reads a block's tokens for every row block, so from
// this many tokens on (aligned operands) it takes 64-row blocks: half the
// activation traffic per weight byte, twice the matrix work per split.
constexpr int GEN_WIDE_M = 64;

// Compute units of the current device (cached per device).
int w16_device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// The one-token kernels' shape: rows per block (rb), 8-row groups per block
// (g = ceil(rb / 8)) and chunks per wave; g = 0 when they do not apply.
struct M1Shape {
  int g;
  int rb;
  int cpw;
  bool ring;   // more than five chunks per wave: the ring kernel
  TileMap tm;
  int tiles;
};

M1Shape m1_shape(const WeightDev& w, bool aligned, int64_t M) {
  M1Shape m{};
  if (!aligned || M != 1) return m;
  m.ring = w.Kb > WAVES * 5;
  m.cpw = m.ring ? (w.Kb + WAVES - 1) / WAVES : w.Kb <= WAVES * 4 ? 4 : 5;
  // the fewest rows in [16, 32] that keep the grid within one block per
  // compute unit, so every unit streams about the same bytes (W [5120, 5120]:
  // 20 rows, 256 blocks, 9.3 -> 8.8 us; whole 8-row groups would give 24 rows
  // and 214 blocks); the last group of a block may be partly masked
  const int cus = w16_device_cus();
  m.rb = 8 * M1_MAX_G;
  for (int rb = 16; rb < 8 * M1_MAX_G; ++rb) {
    int64_t n = 0;
    for (int i = 0; i < w.n_members; ++i) n += (w.m[i].rows + rb - 1) / rb;
    if (n <= cus) {
      m.rb = rb;
      break;
    }
  }
  m.g = (m.rb + 7) / 8;
  int t = 0;
  for (int i = 0; i < w.n_members; ++i) {
    m.tm.tile0[i] = t;
    m.tm.n_tiles[i] = (w.m[i].rows + m.rb - 1) / m.rb;
    t += m.tm.n_tiles[i];
  }
  m.tm.tile0[w.n_members] = t;
  m.tiles = t;
  return m;
}

// Whether one token takes the one-token kernels: not with four 8-row groups
// per block and every load issued at once (25-32 rows per block, five chunks
// per wave), where a wave holds 20 weight loads in flight and the requests
// queue; the few-token kernel, one chunk in flight per wave, is faster there
// (grouped Q/K/V at one token, 32-row blocks: 10.2 -> 9.9 us with F32
// activations, 10.15 -> 9.62 us with E4M3 codes; W [5120, 5120] keeps the
// one-token kernel, 7.7 against 8.5 us, with three groups of 20 rows).
bool m1_preferred(const M1Shape& m1) { return m1.g != 0 && (m1.ring || m1.g < 4); }


// The few-token MFMA kernel's rows per block: the fewest in [16, 32] that keep
// the grid within one block per compute unit (W [5120, 5120]: 20 rows, 256
// blocks, where 32-row blocks leave 96 units idle), else 32.
struct SmallShape {
  int rb;
  TileMap tm;
  int tiles;
};

SmallShape small_shape(const WeightDev& w) {
  SmallShape sh{};
  const int cus = w16_device_cus();
  sh.rb = ROWS;
  for (int rb = 16; rb < ROWS; ++rb) {
    int64_t n = 0;
    for (int i = 0; i < w.n_members; ++i) n += (w.m[i].rows + rb - 1) / rb;
    if (n <= cus) {
      sh.rb = rb;
      break;
    }
  }
  int t = 0;
  for (int i = 0; i < w.n_members; ++i) {
    sh.tm.tile0[i] = t;
    sh.tm.n_tiles[i] = (w.m[i].rows + sh.rb - 1) / sh.rb;
    t += sh.tm.n_tiles[i];
  }
  sh.tm.tile0[w.n_members] = t;
  sh.tiles = t;
  return sh;
}

Plan make_plan(const WeightDev& w, int64_t M, bool aligned = false) {
  Plan p{};
  p.rt = aligned && M >= GEN_WIDE_M ? 4 : RT;
  const int rows = 16 * p.rt;
  p.col_tiles = int((M + COLS - 1) / COLS);
  int t = 0;
  for (int i = 0; i < w.n_members; ++i) {
    p.tm.tile0[i] = t;
    p.tm.n_tiles[i] = (w.m[i].rows + rows - 1) / rows;
    t += p.tm.n_tiles[i] * p.col_tiles;
  }
  p.tm.tile0[w.n_members] = t;
  p.tiles = t;
  p.chunks_per_wave = (w.Kb + WAVES - 1) / WAVES;
  return p;
}

typedef void (*KernelFn)(Args);


int gemm_row_tiles(const WeightDev& w, int32_t* rt0);

// The split-K sum of the W8A16 GEMM: y[m, c] = the splits' F32 partials added
// in split order, for the N output columns of every token, then rounded to y's
// type.  One thread per output.
struct W16ReduceArgs {
  const float* ws;
  int64_t ldws;
  int64_t split_stride;   // M * ldws
  void* y;
  int64_t ldy;
  int32_t M;
  int32_t N;
  int32_t splits;
  int32_t y_bf16;
};

__global__ __launch_bounds__(256) void w8a16_splitk_reduce_kernel(W16ReduceArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(a.M) * a.N) return;
  const int m = int(idx / a.N), c = int(idx - int64_t(m) * a.N);
  const float* p = a.ws + int64_t(m) * a.ldws + c;
  float v = p[0];
  for (int s = 1; s < a.splits; ++s) v += p[int64_t(s) * a.split_stride];
  const int64_t off = int64_t(m) * a.ldy + c;
  if (a.y_bf16) static_cast<uint16_t*>(a.y)[off] = f32_to_bf16_rne(v);
  else static_cast<float*>(a.y)[off] = v;
}

// The LDS-staged GEMM kernel runs for aligned operands when its grid fills at
// least half the compute units: a block takes about the same time whatever
// the grid (grouped Q/K/V: 121-130 us from 64 to 512 tokens), so with fewer
// blocks the general kernel, which splits K inside many small blocks, is
// faster (44 / 84 us at 64 / 128 tokens against 121 us; at 256 tokens 164
// against 122 us, at 512 325 against 129 us).
//
// Split-K: when the tile grid leaves half the compute units or more idle,
// K is cut into up to 8 ranges of at least 4 chunks, as many as keep the grid
// within one block per compute unit, the splits write F32 partials to the workspace and a second kernel
// adds them in order; the GEMM then also takes 33 to 63 tokens (one partly
// filled token tile).
struct W16Split {
  int splits;
  int kb_per_split;
};

W16Split w16_split(const WeightDev& w, int64_t M) {
  const int64_t blocks = int64_t(gemm_row_tiles(w, nullptr)) * ((M + GW_TOKS - 1) / GW_TOKS);
  const int cus = w16_device_cus();
  int s = 1;
  // the most splits that keep the grid within one round of blocks (one per unit)
  if (2 * blocks <= cus) s = int(std::min<int64_t>({cus / blocks, 8, w.Kb / 4}));
  s = std::max(s, 1);
  const int kps = (w.Kb + s - 1) / s;
  return W16Split{(w.Kb + kps - 1) / kps, kps};
}

bool gemm_applies(const WeightDev& w, bool aligned, int64_t M) {
  if (!aligned || M <= SM_SPLIT_MAXM) return false;
  const int64_t blocks = int64_t(gemm_row_tiles(w, nullptr)) * ((M + GW_TOKS - 1) / GW_TOKS);
  return 2 * blocks >= w16_device_cus() || (M >= 33 && w16_split(w, M).splits > 1);
}

int64_t w16_n_total(const WeightDev& w) {
  int64_t n = 0;
  for (int i = 0; i < w.n_members; ++i) n = std::max<int64_t>(n, int64_t(w.m[i].col0) + w.m[i].rows);
  return n;
}

// the split partials' row pitch: N rounded up to 4 floats
int64_t w16_ldws(const WeightDev& w) { return (w16_n_total(w) + 3) / 4 * 4; }

int gemm_row_tiles(const WeightDev& w, int32_t* rt0) {
  int t = 0;
  for (int i = 0; i < w.n_members; ++i) {
    if (rt0) rt0[i] = t;
    t += (w.m[i].rows + GW_ROWS - 1) / GW_ROWS;
  }
  if (rt0) rt0[w.n_members] = t;
  return t;
}

bsf8_status launch_gemm(const WeightDev& w, const void* x, bool x_bf16, int64_t M, int64_t ldx, void* y, bool y_bf16,
                        int64_t ldy, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  GemmArgs a{};
  a.w = w;
  const int rt = gemm_row_tiles(w, a.rt0);
  a.m_tiles = int32_t((M + GW_TOKS - 1) / GW_TOKS);
  a.x = x;
  a.y = y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int32_t(M);
  a.y_bf16 = y_bf16 ? 1 : 0;
  // vector stores of 4 outputs need every member's 4-row runs to start aligned
  const int ye = y_bf16 ? 2 : 4;
  bool vec = reinterpret_cast<uintptr_t>(y) % (4 * ye) == 0 && ldy % 4 == 0;
  for (int i = 0; i < w.n_members; ++i) vec = vec && w.m[i].col0 % 4 == 0;
  a.y_vec = vec ? 1 : 0;
  const W16Split sp = w16_split(w, M);
  a.splits = sp.splits;
  a.kb_per_split = sp.kb_per_split;
  a.ldws = w16_ldws(w);
  a.ws = static_cast<float*>(workspace);
  const int64_t blocks = int64_t(rt) * a.m_tiles * sp.splits;
  if (blocks == 0) return BSF8_OK;
  if (blocks >= (int64_t(1) << 31)) {
    set_error("UNSUPPORTED: %lld blocks", (long long)blocks);
    return BSF8_E_UNSUPPORTED;
  }
  if (sp.splits > 1 && (workspace == nullptr ||
                        workspace_bytes < size_t(sp.splits) * size_t(M) * size_t(a.ldws) * sizeof(float))) {
    set_error("WORKSPACE: %d split-K partials of [%lld, %lld] F32 need a workspace", sp.splits, (long long)M,
              (long long)a.ldws);
    return BSF8_E_WORKSPACE;
  }
  const bool sb = w.scale_bf16 != 0;
  auto k = x_bf16 ? (sb ? w8a16_gemm_kernel<true, true> : w8a16_gemm_kernel<true, false>)
                  : (sb ? w8a16_gemm_kernel<false, true> : w8a16_gemm_kernel<false, false>);
  hipLaunchKernelGGL(k, dim3(unsigned(blocks)), dim3(GW_THREADS), 0, stream, a);
  bsf8_status st = device_status(hipGetLastError(), "w8a16_gemm launch");
  if (st != BSF8_OK || sp.splits == 1) return st;
  W16ReduceArgs r{};
  r.ws = a.ws;
  r.ldws = a.ldws;
  r.split_stride = M * a.ldws;
  r.y = y;
  r.ldy = ldy;
  r.M = int32_t(M);
  r.N = int32_t(w16_n_total(w));
  r.splits = sp.splits;
  r.y_bf16 = y_bf16 ? 1 : 0;
  const int64_t n = M * int64_t(r.N);
  hipLaunchKernelGGL(w8a16_splitk_reduce_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, r);
  return device_status(hipGetLastError(), "w8a16 split-K reduce launch");
}

}  // namespace

// the split-K partials of the GEMM (an upper bound over the paths: operands that
// are not 16-byte aligned take kernels without a workspace)
size_t w8a16_workspace_bytes(const WeightDev& w, int64_t M) {
  if (!gemm_applies(w, true, M)) return 0;
  const W16Split sp = w16_split(w, M);
  return sp.splits > 1 ? size_t(sp.splits) * size_t(M) * size_t(w16_ldws(w)) * sizeof(float) : 0;
}

std::string describe_w8a16(const WeightDev& w, bool aligned, int64_t M) {
  if (!gemm_applies(w, aligned, M) && aligned && M > SM_MAXM && M <= SM_SPLIT_MAXM)
    return "two launches, tokens [0, " + std::to_string(SM_MAXM) + ") then [" + std::to_string(SM_MAXM) + ", " +
           std::to_string(M) + "): " + describe_w8a16(w, aligned, SM_MAXM) + " ;; " +
           describe_w8a16(w, aligned, M - SM_MAXM);
  if (gemm_applies(w, aligned, M)) {
    char b[448];
    const int rt = gemm_row_tiles(w, nullptr);
    snprintf(b, sizeof(b),
             "arm=w8a16 arithmetic=f32 activations (exact 3-term bf16 split) x e4m3 weights, f32 accumulate, "
             "mfma_f32_16x16x32_bf16 | kernel=w8a16_gemm tile=%dx%d waves=8 lds=2 stages (register-staged copies) "
             "split_k=%d (%d chunks per split%s) | M=%lld blocks=%lld",
             GW_ROWS, GW_TOKS, w16_split(w, M).splits, w16_split(w, M).kb_per_split,
             w16_split(w, M).splits > 1 ? ", F32 partials added in split order by a second kernel" : "", (long long)M,
             (long long)rt * ((M + GW_TOKS - 1) / GW_TOKS) * w16_split(w, M).splits);
    return b;
  }
  const M1Shape m1 = m1_shape(w, aligned, M > 0 ? M : 1);
  if (m1_preferred(m1)) {
    char b1[448];
    snprintf(b1, sizeof(b1),
             "arm=w8a16 arithmetic=f32 activations x e4m3 weights (exact f32 decode), f32 fma accumulate | "
             "kernel=%s rows=%d (8-row groups=%d) waves=%d (in-block split-K, %d chunks/wave, %s, "
             "8 lanes per 128-byte row piece, no LDS transpose) | M=%lld blocks=%d",
             m1.ring ? "w8a16_m1_ring" : "w8a16_m1", m1.rb, m1.g, WAVES, m1.cpw,
             m1.ring ? "load ring of 1 chunk (F32 activations) or 2 (BF16)" : "all loads first",
             (long long)(M > 0 ? M : 1), m1.tiles);
    return b1;
  }
  const Plan p = make_plan(w, M > 0 ? M : 1, aligned);
  const bool small = aligned && M >= 1 && M <= SM_MAXM;
  char ring[160] = "";
  if (small)
    snprintf(ring, sizeof(ring), ", %d-chunk load ring, compact activations split in LDS, F32 terms in MFMA columns",
             SM_RING);
  char buf[512];
  snprintf(buf, sizeof(buf),
           "arm=w8a16 arithmetic=f32 activations (exact 3-term bf16 split) x e4m3 weights, f32 accumulate, "
           "mfma_f32_16x16x32_bf16 | kernel=%s rows=%d tokens=%d waves=%d (in-block split-K, %d chunks/wave%s) "
           "path=%s | M=%lld blocks=%d",
           small ? "w8a16_small_m" : "w8a16", small ? small_shape(w).rb : 16 * p.rt, small ? SM_MAXM : COLS, WAVES,
           p.chunks_per_wave, ring, aligned ? "aligned16" : "bytewise", (long long)M,
           small ? small_shape(w).tiles : p.tiles);
  return buf;
}

bsf8_status launch_w8a16(const WeightDev& w, bool aligned, const void* x, bool x_bf16, int64_t M, int64_t ldx,
                         void* y, bool y_bf16, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (w.Kb > MAX_KB) {
    set_error("UNSUPPORTED: K above %d", MAX_KB * CHUNK);
    return BSF8_E_UNSUPPORTED;
  }
  // buffer offsets are 32-bit: operands of 2 GiB or more take the byte-wise path
  if (M * ldx * (x_bf16 ? 2 : 4) >= (int64_t(1) << 31)) aligned = false;
  for (int i = 0; i < w.n_members; ++i)
    if (int64_t(w.m[i].rows) * w.K >= (int64_t(1) << 31)) aligned = false;
  const Plan p = make_plan(w, M, aligned);
  if (p.tiles == 0) return BSF8_OK;
  if (gemm_applies(w, aligned, M)) return launch_gemm(w, x, x_bf16, M, ldx, y, y_bf16, ldy, ws, ws_bytes, stream);
  if (aligned && M > SM_MAXM && M <= SM_SPLIT_MAXM) {
    // rows SM_MAXM on of x start 16-byte aligned too (ldx * element size is a multiple of 16)
    const bsf8_status st = launch_w8a16(w, true, x, x_bf16, SM_MAXM, ldx, y, y_bf16, ldy, nullptr, 0, stream);
    if (st != BSF8_OK) return st;
    return launch_w8a16(w, true, static_cast<const uint8_t*>(x) + SM_MAXM * ldx * (x_bf16 ? 2 : 4), x_bf16,
                        M - SM_MAXM, ldx, static_cast<uint8_t*>(y) + SM_MAXM * ldy * (y_bf16 ? 2 : 4), y_bf16, ldy,
                        nullptr, 0, stream);
  }
  const M1Shape m1 = m1_shape(w, aligned, M);
  if (m1_preferred(m1)) {
    Args a{};
    a.w = w;
    a.tm = m1.tm;
    a.x = x;
    a.y = y;
    a.ldx = ldx;
    a.ldy = ldy;
    a.M = int32_t(M);
    a.col_tiles = 1;
    a.chunks_per_wave = m1.cpw;
    a.rows_per_block = m1.rb;
    a.x_bf16 = x_bf16 ? 1 : 0;
    a.y_bf16 = y_bf16 ? 1 : 0;
    const bool sb = w.scale_bf16 != 0;
#define BSF8_M1(G, C)                                                                                         \
  (x_bf16 ? (sb ? w8a16_m1_kernel<XK_BF16, true, G, C> : w8a16_m1_kernel<XK_BF16, false, G, C>)               \
          : (sb ? w8a16_m1_kernel<XK_F32, true, G, C> : w8a16_m1_kernel<XK_F32, false, G, C>))
#define BSF8_MR(G)                                                                                              \
  (x_bf16 ? (sb ? w8a16_m1_ring_kernel<XK_BF16, true, G, m1r_depth<XK_BF16>()>                           \
                 : w8a16_m1_ring_kernel<XK_BF16, false, G, m1r_depth<XK_BF16>()>)                          \
          : (sb ? w8a16_m1_ring_kernel<XK_F32, true, G, m1r_depth<XK_F32>()>                               \
                : w8a16_m1_ring_kernel<XK_F32, false, G, m1r_depth<XK_F32>()>))
    auto k1 = m1.ring ? (m1.g == 2 ? BSF8_MR(2) : m1.g == 3 ? BSF8_MR(3) : BSF8_MR(4))
              : m1.cpw == 4 ? (m1.g == 2 ? BSF8_M1(2, 4) : m1.g == 3 ? BSF8_M1(3, 4) : BSF8_M1(4, 4))
                            : (m1.g == 2 ? BSF8_M1(2, 5) : m1.g == 3 ? BSF8_M1(3, 5) : BSF8_M1(4, 5));
#undef BSF8_M1
#undef BSF8_MR
    hipLaunchKernelGGL(k1, dim3(m1.tiles), dim3(THREADS), 0, stream, a);
    return device_status(hipGetLastError(), "w8a16_m1 launch");
  }
  Args a{};
  a.w = w;
  a.tm = p.tm;
  a.x = x;
  a.y = y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int32_t(M);
  a.col_tiles = p.col_tiles;
  a.chunks_per_wave = p.chunks_per_wave;
  a.x_bf16 = x_bf16 ? 1 : 0;
  a.y_bf16 = y_bf16 ? 1 : 0;
  auto kern = w8a16_kernel<true, false, true, RT>;
  const bool sb = w.scale_bf16 != 0;
  int grid = p.tiles;
  if (aligned && M <= SM_MAXM) {
    const SmallShape sh = small_shape(w);
    a.tm = sh.tm;
    a.rows_per_block = sh.rb;
    grid = sh.tiles;
    // compact activation loads: 2 F32 (4 BF16) tokens per 16-byte-per-lane load,
    // and 3 M term columns of F32 tokens in 16-column MFMA passes (one up to
    // M = 5, two up to 8, three up to 16: W [5120, 5120] at five tokens 10.9 ->
    // 9.9 us with one pass instead of two); a BF16 token is one column
#define BSF8_SMALL(XK, NXI, NP) \
  (sb ? w8a16_small_m_kernel<XK, true, NXI, NP, SM_RING> : w8a16_small_m_kernel<XK, false, NXI, NP, SM_RING>)
    if (x_bf16) {
      kern = M <= 4 ? BSF8_SMALL(XK_BF16, 1, 1) : M <= 8 ? BSF8_SMALL(XK_BF16, 2, 1) : BSF8_SMALL(XK_BF16, 4, 1);
    } else if (M <= 5) {
      kern = M <= 2 ? BSF8_SMALL(XK_F32, 1, 1) : M <= 4 ? BSF8_SMALL(XK_F32, 2, 1) : BSF8_SMALL(XK_F32, 3, 1);
    } else if (M <= 8) {
      kern = BSF8_SMALL(XK_F32, 4, 2);
    } else {
      kern = BSF8_SMALL(XK_F32, 8, 3);
    }
#undef BSF8_SMALL
  } else if (aligned && p.rt == 4) {
    if (x_bf16) kern = sb ? w8a16_kernel<true, true, true, 4> : w8a16_kernel<true, true, false, 4>;
    else kern = sb ? w8a16_kernel<true, false, true, 4> : w8a16_kernel<true, false, false, 4>;
  } else if (aligned) {
    if (x_bf16) kern = sb ? w8a16_kernel<true, true, true, RT> : w8a16_kernel<true, true, false, RT>;
    else kern = sb ? w8a16_kernel<true, false, true, RT> : w8a16_kernel<true, false, false, RT>;
  } else {
    if (x_bf16) kern = sb ? w8a16_kernel<false, true, true, RT> : w8a16_kernel<false, true, false, RT>;
    else kern = sb ? w8a16_kernel<false, false, true, RT> : w8a16_kernel<false, false, false, RT>;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), 0, stream, a);
  return device_status(hipGetLastError(), "w8a16 launch");
}

// The W8A8 arm at one to 48 tokens: the same weight streams with E4M3
// activations (the one-token kernels, and from two tokens the few-token
// kernel).  A decoded code times a decoded weight is exact in F32 (and the
// BF16 matrix cores add such products exactly into F32), so a chunk partial is
// the method's block partial summed in another order, and it is scaled by
// activation scale x weight scale as the F32 epilogue states.  At these token
// counts a matrix-core GEMM tile would read the weight for 1 to 32 useful
// columns out of 128 or 256.
bool w8a8_stream_applies(const WeightDev& w, bool aligned, int64_t M, int64_t ldq) {
  // (the streaming kernels hold a wave's chunk scales in two registers per lane: K up to 131072)
  if (!aligned || M < 1 || M > SM_MAXM_Q8 || w.Kb > MAX_KB || M * ldq >= (int64_t(1) << 31)) return false;
  for (int i = 0; i < w.n_members; ++i)
    if (int64_t(w.m[i].rows) * w.K >= (int64_t(1) << 31)) return false;
  return M > 1 || m1_shape(w, true, M).g != 0;
}

std::string describe_w8a8_stream(const WeightDev& w, int64_t M) {
  if (M > 1 || !m1_preferred(m1_shape(w, true, M))) {
    const SmallShape sh = small_shape(w);
    char b[512];
    snprintf(b, sizeof(b),
             "arm=w8a8 arithmetic=e4m3 codes decoded exactly to bf16 x e4m3 weights decoded exactly to bf16, "
             "mfma_f32_16x16x32_bf16 (column = token), f32 chunk partials x (act scale x weight scale) | "
             "kernel=w8a16_small_m<e4m3> rows=%d tokens<=%d waves=%d (in-block split-K, weights 8 lanes per "
             "128-byte row through a wave-private LDS transpose, %d chunk in flight per wave) | M=%lld blocks=%d",
             sh.rb, SM_MAXM_Q8, WAVES, SM_RING, (long long)M, sh.tiles);
    return b;
  }
  const M1Shape m1 = m1_shape(w, true, M);
  char b[448];
  snprintf(b, sizeof(b),
           "arm=w8a8 arithmetic=e4m3 x e4m3 decoded exactly to f32, f32 fma chunk partials x (act scale x weight "
           "scale) | kernel=%s<e4m3> rows=%d (8-row groups=%d) waves=%d (in-block split-K, %d chunks/wave, %s, "
           "8 lanes per 128-byte row piece, no LDS transpose%s) | M=%lld blocks=%d",
           m1.ring ? "w8a16_m1_ring" : "w8a16_m1", m1.rb, m1.g, WAVES, m1.cpw,
           m1.ring ? "2-chunk load ring" : "all loads first", "", (long long)M, m1.tiles);
  return b;
}

bsf8_status launch_w8a8_stream(const WeightDev& w, const uint8_t* xq, int64_t ldq, const float* xs, int64_t xs_sm,
                               int64_t xs_sk, int64_t M, void* y, bool y_bf16, int64_t ldy, hipStream_t stream) {
  if (M > 1 || !m1_preferred(m1_shape(w, true, M))) {
    const SmallShape sh = small_shape(w);
    Args a{};
    a.w = w;
    a.tm = sh.tm;
    a.x = xq;
    a.y = y;
    a.ldx = ldq;
    a.ldy = ldy;
    a.M = int32_t(M);
    a.col_tiles = 1;
    a.chunks_per_wave = (w.Kb + WAVES - 1) / WAVES;
    a.rows_per_block = sh.rb;
    a.y_bf16 = y_bf16 ? 1 : 0;
    a.xs = xs;
    a.xs_sm = xs_sm;
    a.xs_sk = xs_sk;
    const bool sb = w.scale_bf16 != 0;
    // 8 tokens of codes per compact load (one load per lane up to 8 tokens, two
    // up to 16, four up to 32, six up to 48) and 16 tokens per MFMA pass
#define BSF8_SQ8(NXI, NP) \
  (sb ? w8a16_small_m_kernel<XK_E4M3, true, NXI, NP, SM_RING> : w8a16_small_m_kernel<XK_E4M3, false, NXI, NP, SM_RING>)
    auto k = M <= 8 ? BSF8_SQ8(1, 1) : M <= 16 ? BSF8_SQ8(2, 1) : M <= 32 ? BSF8_SQ8(4, 2) : BSF8_SQ8(6, 3);
#undef BSF8_SQ8
    hipLaunchKernelGGL(k, dim3(sh.tiles), dim3(THREADS), 0, stream, a);
    return device_status(hipGetLastError(), "w8a8 few-token launch");
  }
  const M1Shape m1 = m1_shape(w, true, M);
  if (m1.g == 0) {
    set_error("UNSUPPORTED: no one-token streaming shape for this weight");
    return BSF8_E_UNSUPPORTED;
  }
  Args a{};
  a.w = w;
  a.tm = m1.tm;
  a.x = xq;
  a.y = y;
  a.ldx = ldq;
  a.ldy = ldy;
  a.M = int32_t(M);
  a.col_tiles = 1;
  a.chunks_per_wave = m1.cpw;
  a.rows_per_block = m1.rb;
  a.x_bf16 = 0;
  a.y_bf16 = y_bf16 ? 1 : 0;
  a.xs = xs;
  a.xs_sm = xs_sm;
  a.xs_sk = xs_sk;
  const bool sb = w.scale_bf16 != 0;
#define BSF8_Q1(G, C) (sb ? w8a16_m1_kernel<XK_E4M3, true, G, C> : w8a16_m1_kernel<XK_E4M3, false, G, C>)
#define BSF8_QR(G) \
  (sb ? w8a16_m1_ring_kernel<XK_E4M3, true, G, m1r_depth<XK_E4M3>()>                                     \
      : w8a16_m1_ring_kernel<XK_E4M3, false, G, m1r_depth<XK_E4M3>()>)
  auto k1 = m1.ring ? (m1.g == 2 ? BSF8_QR(2) : m1.g == 3 ? BSF8_QR(3) : BSF8_QR(4))
            : m1.cpw == 4 ? (m1.g == 2 ? BSF8_Q1(2, 4) : m1.g == 3 ? BSF8_Q1(3, 4) : BSF8_Q1(4, 4))
                          : (m1.g == 2 ? BSF8_Q1(2, 5) : m1.g == 3 ? BSF8_Q1(3, 5) : BSF8_Q1(4, 5));
#undef BSF8_Q1
#undef BSF8_QR
  hipLaunchKernelGGL(k1, dim3(m1.tiles), dim3(THREADS), 0, stream, a);
  return device_status(hipGetLastError(), "w8a8 streaming launch");
}

// The W8A8 arm with the activation quantization in the same call, at one token:
// the one-token kernels (and their load-ring form) quantize each wave's K range
// of the token into LDS before the weight stream lands (see quant_issue) and
// then run as on quantized activations, so codes, scales and results are those
// of bsf8_quant_act followed by bsf8_linear_w8a8, bit for bit, and the codes
// never go to memory.  More tokens do not pay: every block would quantize all
// of them again (at four tokens 40 values per lane, with their quotients in
// F64, 3-4 us of ALU work per wave ahead of the first chunk).
bool w8a8_dyn_stream_applies(const WeightDev& w, bool aligned, int64_t M, int64_t ldx_bytes) {
  if (M != 1 || !w8a8_stream_applies(w, aligned, M, ldx_bytes)) return false;
  const M1Shape m1 = m1_shape(w, true, M);
  return m1.g != 0 && (!m1.ring || m1.cpw <= QCHUNKS_MAX);
}

std::string describe_w8a8_dyn_stream(const WeightDev& w, int64_t M) {
  const M1Shape m1 = m1_shape(w, true, M);
  char b[640];
  snprintf(b, sizeof(b),
           "arm=w8a8-dynamic arithmetic=f32/bf16 activations quantized per token 1x128 to e4m3 by each wave for "
           "its K range into LDS (codes never stored), e4m3 x e4m3 decoded exactly to f32, f32 fma chunk partials "
           "x (act scale x weight scale) | kernel=%s<quantizing> rows=%d (8-row groups=%d) waves=%d (in-block "
           "split-K, %d chunks/wave, %s, 8 lanes per 128-byte row piece) | M=%lld blocks=%d",
           m1.ring ? "w8a16_m1_ring" : "w8a16_m1", m1.rb, m1.g, WAVES, m1.cpw,
           m1.ring ? "2-chunk load ring" : "all loads first", (long long)M, m1.tiles);
  return b;
}

bsf8_status launch_w8a8_dyn_stream(const WeightDev& w, const void* x, bool x_bf16, int64_t M, int64_t ldx, void* y,
                                   bool y_bf16, int64_t ldy, hipStream_t stream) {
  const M1Shape m1 = m1_shape(w, true, M);
  if (M != 1 || m1.g == 0 || (m1.ring && m1.cpw > QCHUNKS_MAX)) {
    set_error("UNSUPPORTED: the quantizing streaming kernels take one token and at most %d chunks per wave",
              QCHUNKS_MAX);
    return BSF8_E_UNSUPPORTED;
  }
  Args a{};
  a.w = w;
  a.tm = m1.tm;
  a.x = x;
  a.y = y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = 1;
  a.col_tiles = 1;
  a.chunks_per_wave = m1.cpw;
  a.rows_per_block = m1.rb;
  a.x_bf16 = x_bf16 ? 1 : 0;
  a.y_bf16 = y_bf16 ? 1 : 0;
  const bool sb = w.scale_bf16 != 0;
#define BSF8_D1(XK, G, C) (sb ? w8a16_m1_kernel<XK, true, G, C> : w8a16_m1_kernel<XK, false, G, C>)
#define BSF8_DR(XK, G) \
  (sb ? w8a16_m1_ring_kernel<XK, true, G, m1r_depth<XK>()> : w8a16_m1_ring_kernel<XK, false, G, m1r_depth<XK>()>)
#define BSF8_DSEL(XK)                                                                                    \
  (m1.ring ? (m1.g == 2 ? BSF8_DR(XK, 2) : m1.g == 3 ? BSF8_DR(XK, 3) : BSF8_DR(XK, 4))                \
   : m1.cpw == 4 ? (m1.g == 2 ? BSF8_D1(XK, 2, 4) : m1.g == 3 ? BSF8_D1(XK, 3, 4) : BSF8_D1(XK, 4, 4)) \
                 : (m1.g == 2 ? BSF8_D1(XK, 2, 5) : m1.g == 3 ? BSF8_D1(XK, 3, 5) : BSF8_D1(XK, 4, 5)))
  auto k1 = x_bf16 ? BSF8_DSEL(XK_BF16Q) : BSF8_DSEL(XK_F32Q);
#undef BSF8_DSEL
#undef BSF8_DR
#undef BSF8_D1
  hipLaunchKernelGGL(k1, dim3(m1.tiles), dim3(THREADS), 0, stream, a);
  return device_status(hipGetLastError(), "w8a8 dynamic streaming launch");
}

}  // namespace bsf8

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
// A plain F32 FMA loop needs ~M FMAs per weight byte, which at M = 8 exceeds the
// FP32 VALU rate before HBM is saturated, so the products run on the BF16
// matrix cores without losing any activation bit:
//  * every E4M3 value is exact in BF16 (v_cvt_scalef32_pk_bf16_fp8, scale 1.0);
//  * every F32 activation is split exactly as x = hi + mid + lo with three BF16
//    values (truncate to the top 16 bits twice; each remainder is exact in F32
//    and the last one has at most 8 significant bits);
//  * BF16 x BF16 products are exact in F32 and the MFMA accumulates in F32.
//  So the arithmetic is F32 activations times exact FP8 weights with F32
//  accumulation, as the pages state, at about three BF16 MFMAs per 16x16x32 step.
//  (Inputs below ~2^-100 in magnitude may lose their lowest remainder bits.)
//
// Work decomposition:
//  * A block (8 waves) owns one 128-row group of one member (exactly one row of
//    that member's scale grid, so the weight scale is a block-uniform scalar per
//    128-wide K chunk), 16 tokens, and a range of K chunks.
//  * Per chunk, the block splits its 16x128 activation slice once into LDS
//    (shared by all 8 waves); each wave streams its own 16 weight rows x 128
//    bytes straight from HBM into registers (two 16-byte loads per lane),
//    converts them and issues 12 MFMAs (4 K-steps x 3 terms); the chunk partial
//    is scaled by the block's weight scale into the F32 accumulator.
//  * Decode shapes have too few 128-row groups to fill 256 CUs, so K is split
//    across blocks.  Each block writes its partial tile to the workspace; the
//    last block to arrive (device-scope counter) adds the partials in split
//    order and stores Y, so the result does not depend on arrival order, and
//    resets the counter to zero for the next call.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>

#include "bsf8_internal.h"

namespace bsf8 {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int ROWS = 128;        // weight rows per block (one scale-grid row)
constexpr int COLS = 16;         // tokens per block
constexpr int CHUNK = 128;       // K per chunk (one scale block)
constexpr int TERMS = 3;
constexpr int STEPS = CHUNK / 32;                        // MFMA K-steps per chunk
constexpr int SPLIT_BYTES = TERMS * STEPS * 64 * 16;     // 12 KiB of BF16 fragments per chunk
constexpr int TARGET_BLOCKS = 512;

struct Args {
  WeightDev w;
  TileMap tm;          // row groups per member, tiles = groups x col tiles
  const void* x;
  void* y;
  float* partial;      // [tiles][splits][ROWS][COLS]
  uint32_t* counter;   // [tiles]
  int64_t ldx;
  int64_t ldy;
  int32_t M;
  int32_t col_tiles;
  int32_t splits;
  int32_t chunks_per_split;
  int32_t x_bf16;
  int32_t y_bf16;
};

__device__ __forceinline__ float load_scale(const void* s, int64_t idx, int bf16) {
  if (bf16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(s)[idx]) << 16);
  return static_cast<const float*>(s)[idx];
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// K offset (within a chunk) of element j of K-step s held by lane group gq.
// Both MFMA operands use this same map, so the dot product covers every k once.
__device__ __forceinline__ int kmap(int s, int gq, int j) { return (s >> 1) * 64 + gq * 16 + (s & 1) * 8 + j; }

// Four activations (k .. k+3 of one token) as F32; zeros past K or past M.
template <bool ALIGNED>
__device__ __forceinline__ void load_x4(const Args& a, int m, int k, int K, float v[4]) {
  v[0] = v[1] = v[2] = v[3] = 0.f;
  if (m >= a.M) return;
  const int n = K - k;
  if (n <= 0) return;
  const int64_t off = int64_t(m) * a.ldx + k;
  if (a.x_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(a.x) + off;
    if (ALIGNED && n >= 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = __uint_as_float(u.x << 16);
      v[1] = __uint_as_float(u.x & 0xFFFF0000u);
      v[2] = __uint_as_float(u.y << 16);
      v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      for (int j = 0; j < 4 && j < n; ++j) v[j] = __uint_as_float(uint32_t(p[j]) << 16);
    }
  } else {
    const float* p = static_cast<const float*>(a.x) + off;
    if (ALIGNED && n >= 4) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else {
      for (int j = 0; j < 4 && j < n; ++j) v[j] = p[j];
    }
  }
}

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

__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

// Split 4 activations into three BF16 terms and store them into the fragment
// layout: lane (token c, group gq) of K-step s owns 16 bytes at
// ((t * STEPS + s) * 64 + gq * 16 + c) * 16.
__device__ __forceinline__ void split_store(uint8_t* buf, int c, int k4, const float v[4]) {
  uint32_t t0[4], t1[4], t2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t xb = __float_as_uint(v[j]);
    const uint32_t hb = xb & 0xFFFF0000u;
    const float r1 = v[j] - __uint_as_float(hb);
    const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(mb);
    t0[j] = hb;
    t1[j] = mb;
    t2[j] = __float_as_uint(r2);
  }
  const int s = ((k4 >> 6) << 1) | ((k4 >> 3) & 1);
  const int gq = (k4 >> 4) & 3;
  const int jbyte = (k4 & 7) * 2;  // 0 or 8
  const int slot = (gq * 16 + c) * 16 + jbyte;
  uint2 w0 = make_uint2(pack_hi16(t0[0], t0[1]), pack_hi16(t0[2], t0[3]));
  uint2 w1 = make_uint2(pack_hi16(t1[0], t1[1]), pack_hi16(t1[2], t1[3]));
  uint2 w2 = make_uint2(pack_hi16(t2[0], t2[1]), pack_hi16(t2[2], t2[3]));
  *reinterpret_cast<uint2*>(buf + (0 * STEPS + s) * 1024 + slot) = w0;
  *reinterpret_cast<uint2*>(buf + (1 * STEPS + s) * 1024 + slot) = w1;
  *reinterpret_cast<uint2*>(buf + (2 * STEPS + s) * 1024 + slot) = w2;
}

__device__ __forceinline__ v8bf cvt8(uint32_t lo, uint32_t hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool ALIGNED>
__global__ __launch_bounds__(THREADS) void w8a16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t xsplit[2][SPLIT_BYTES];
  __shared__ int last_flag;

  // ---- block -> (member, row group, token tile, K split)
  const int splits = a.splits;
  const int bid = blockIdx.x;
  const int ks = bid % splits;
  const int tile = bid / splits;
  int mi = 0;
  while (mi + 1 < a.w.n_members && tile >= a.tm.tile0[mi + 1]) ++mi;
  const int local = tile - a.tm.tile0[mi];
  const int rg = local % a.tm.n_tiles[mi];
  const int ct = local / a.tm.n_tiles[mi];
  const MemberDev mem = a.w.m[mi];
  const int K = a.w.K, Kb = a.w.Kb;
  const int c_begin = ks * a.chunks_per_split;
  const int c_end = min(Kb, c_begin + a.chunks_per_split);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, gq = lane >> 4;

  // splitter role: thread -> (token c, 4 consecutive k)
  const int sc = tid >> 5;             // 0..15
  const int sk4 = (tid & 31) * 4;      // 0..124
  const int sm = ct * COLS + sc;

  // weight role: wave -> 16 rows; lane -> row l16, two 16-byte pieces
  const int row = rg * ROWS + wave * 16 + l16;
  const bool row_ok = row < mem.rows;
  const uint8_t* wrow = mem.w + int64_t(row_ok ? row : 0) * K;
  const int64_t s_base = int64_t(rg) * Kb;

  v4f acc = {0.f, 0.f, 0.f, 0.f};

  float xv[4];
  uint4 w0 = make_uint4(0, 0, 0, 0), w1 = w0;
  if (c_begin < c_end) {
    load_x4<ALIGNED>(a, sm, c_begin * CHUNK + sk4, K, xv);
    w0 = load_w16<ALIGNED>(wrow, c_begin * CHUNK + gq * 16, K, row_ok);
    w1 = load_w16<ALIGNED>(wrow, c_begin * CHUNK + 64 + gq * 16, K, row_ok);
  }
  for (int c = c_begin; c < c_end; ++c) {
    uint8_t* buf = xsplit[c & 1];
    split_store(buf, sc, sk4, xv);
    const bool more = c + 1 < c_end;
    if (more) load_x4<ALIGNED>(a, sm, (c + 1) * CHUNK + sk4, K, xv);
    __syncthreads();
    const uint4 p0 = w0, p1 = w1;
    if (more) {
      w0 = load_w16<ALIGNED>(wrow, (c + 1) * CHUNK + gq * 16, K, row_ok);
      w1 = load_w16<ALIGNED>(wrow, (c + 1) * CHUNK + 64 + gq * 16, K, row_ok);
    }
    const float sw = load_scale(mem.s, s_base + c, a.w.scale_bf16);
    const v8bf af[STEPS] = {cvt8(p0.x, p0.y), cvt8(p0.z, p0.w), cvt8(p1.x, p1.y), cvt8(p1.z, p1.w)};
    v4f pt[TERMS];
#pragma unroll
    for (int t = 0; t < TERMS; ++t) pt[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int t = 0; t < TERMS; ++t) {
        const v8bf bfr = *reinterpret_cast<const v8bf*>(buf + ((t * STEPS + s) * 64 + lane) * 16);
        pt[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bfr, pt[t], 0, 0, 0);
      }
    }
    acc += (pt[0] + pt[1] + pt[2]) * sw;
  }

  // ---- output: lane holds rows 4*gq + r of the wave's 16, token l16
  const int out_row0 = rg * ROWS + wave * 16 + 4 * gq;   // member-local
  const int m = ct * COLS + l16;
  auto store_y = [&](const v4f& v) {
    if (m >= a.M) return;
    const int nvalid = mem.rows - out_row0;
    if (nvalid <= 0) return;
    const int64_t off = int64_t(m) * a.ldy + mem.col0 + out_row0;
    if (a.y_bf16) {
      uint16_t* y = static_cast<uint16_t*>(a.y) + off;
      for (int r = 0; r < 4 && r < nvalid; ++r) y[r] = f32_to_bf16_rne(v[r]);
    } else {
      float* y = static_cast<float*>(a.y) + off;
      if (nvalid >= 4 && (reinterpret_cast<uintptr_t>(y) & 15) == 0)
        *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
      else
        for (int r = 0; r < 4 && r < nvalid; ++r) y[r] = v[r];
    }
  };

  if (splits == 1) {
    store_y(acc);
    return;
  }

  // ---- split-K: publish the partial, the last block to arrive reduces in order
  float* part = a.partial + (int64_t(tile) * splits + ks) * (ROWS * COLS);
#pragma unroll
  for (int r = 0; r < 4; ++r) part[(wave * 16 + 4 * gq + r) * COLS + l16] = acc[r];
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.counter + tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == uint32_t(splits - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  v4f sum = {0.f, 0.f, 0.f, 0.f};
  const float* base = a.partial + int64_t(tile) * splits * (ROWS * COLS);
  for (int s = 0; s < splits; ++s) {
    const float* p = base + int64_t(s) * (ROWS * COLS);
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[r] += __builtin_nontemporal_load(p + (wave * 16 + 4 * gq + r) * COLS + l16);
  }
  store_y(sum);
  if (tid == 0) __hip_atomic_store(a.counter + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Plan {
  TileMap tm;
  int col_tiles;
  int tiles;
  int splits;
  int chunks_per_split;
  int blocks;
  size_t counter_bytes;
  size_t partial_bytes;
};

Plan make_plan(const WeightDev& w, int64_t M) {
  Plan p{};
  p.col_tiles = int((M + COLS - 1) / COLS);
  int t = 0;
  for (int i = 0; i < w.n_members; ++i) {
    p.tm.tile0[i] = t;
    p.tm.n_tiles[i] = (w.m[i].rows + ROWS - 1) / ROWS;
    t += p.tm.n_tiles[i] * p.col_tiles;
  }
  p.tm.tile0[w.n_members] = t;
  p.tiles = t;
  const int want = (TARGET_BLOCKS + t - 1) / t;
  const int cps = want <= 1 ? w.Kb : (w.Kb + want - 1) / want;
  p.chunks_per_split = cps < 1 ? 1 : cps;
  p.splits = (w.Kb + p.chunks_per_split - 1) / p.chunks_per_split;
  p.blocks = p.tiles * p.splits;
  if (p.splits > 1) {
    p.counter_bytes = ((size_t(p.tiles) * 4 + 255) / 256) * 256;
    p.partial_bytes = size_t(p.tiles) * p.splits * ROWS * COLS * sizeof(float);
  }
  return p;
}

}  // namespace

size_t w8a16_workspace_bytes(const WeightDev& w, int64_t M) {
  const Plan p = make_plan(w, M);
  return p.counter_bytes + p.partial_bytes;
}

std::string describe_w8a16(const WeightDev& w, bool aligned, int64_t M) {
  const Plan p = make_plan(w, M > 0 ? M : 1);
  char buf[320];
  snprintf(buf, sizeof(buf),
           "arm=w8a16 arithmetic=f32 activations (exact 3-term bf16 split) x e4m3 weights, f32 accumulate, "
           "mfma_f32_16x16x32_bf16 | kernel=w8a16 rows=%d tokens=%d waves=%d k_splits=%d chunks_per_split=%d "
           "path=%s | M=%lld blocks=%d",
           ROWS, COLS, WAVES, p.splits, p.chunks_per_split, aligned ? "aligned16" : "bytewise", (long long)M,
           p.blocks);
  return buf;
}

bsf8_status launch_w8a16(const WeightDev& w, bool aligned, const void* x, bool x_bf16, int64_t M, int64_t ldx,
                         void* y, bool y_bf16, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
  const Plan p = make_plan(w, M);
  if (p.blocks == 0) return BSF8_OK;
  Args a{};
  a.w = w;
  a.tm = p.tm;
  a.x = x;
  a.y = y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int32_t(M);
  a.col_tiles = p.col_tiles;
  a.splits = p.splits;
  a.chunks_per_split = p.chunks_per_split;
  a.x_bf16 = x_bf16 ? 1 : 0;
  a.y_bf16 = y_bf16 ? 1 : 0;
  if (p.splits > 1) {
    if (ws == nullptr || ws_bytes < p.counter_bytes + p.partial_bytes) {
      set_error("WORKSPACE: %zu bytes needed", p.counter_bytes + p.partial_bytes);
      return BSF8_E_WORKSPACE;
    }
    a.counter = static_cast<uint32_t*>(ws);
    a.partial = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.counter_bytes);
  }
  if (aligned)
    hipLaunchKernelGGL(w8a16_kernel<true>, dim3(p.blocks), dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(w8a16_kernel<false>, dim3(p.blocks), dim3(THREADS), 0, stream, a);
  return device_status(hipGetLastError(), "w8a16 launch");
}

}  // namespace bsf8

// W8A8 block-scaled GEMM on the gfx950 FP8 matrix cores.
//
// ("Module w8a8_prefill", section "WHY (#917 / #928)": FP8 x FP8 products
//  accumulated in F32, each 128-wide K slice rescaled by the token's group scale
//  times the weight block scale in an F32 epilogue; "FP8 Native Serving",
//  section "Native FP8 vs dequant-to-BF16": FP8 operands go straight into the
//  matrix unit and results become BF16 only when written back.)
//
// Design for CDNA4:
//  * Y^T tile = W tile . Xq^T: the weight rows are the MFMA A operand (16 rows
//    of N) and the quantized tokens the B operand (16 columns of M).  Both are
//    K-contiguous in HBM, exactly what v_mfma_f32_16x16x128_f8f6f4 reads per
//    lane (32 consecutive K bytes of one row), so neither operand is repacked.
//  * One 16x16x128 MFMA covers exactly one 128-wide scale block, so its result
//    is the block partial P of the method; the epilogue is one FMA per output
//    per K block: acc += P * (sa[m,kb] * sw[row block,kb]).
//  * Block tile 256 (N) x 128 (M), four waves of 128 x 64.  Tiles are laid out
//    member by member from each member's own row 0, so a wave's 128 rows are
//    exactly one row of that member's scale grid: sw is one scalar per wave and
//    K block (member-local origins come for free).
//  * Operands are staged through LDS, double-buffered, 128 bytes per row per K
//    block with the 16-byte chunks XOR-swizzled by (row & 7), which makes both
//    the staging writes and the MFMA fragment reads bank-conflict free.
//  * Tails: rows past a member's end, tokens past M and K bytes past K are
//    loaded as zeros (so a NaN code beyond K can never reach a product) and
//    never stored.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>

#include "bsf8_internal.h"

namespace bsf8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = 256;        // weight rows per block tile
constexpr int BM = 128;        // tokens per block tile
constexpr int KBYTES = 128;    // one scale block of K
constexpr int THREADS = 256;
constexpr int WN = 128;        // rows per wave
constexpr int WM = 64;         // tokens per wave
constexpr int TI = WN / 16;    // 8 MFMA row tiles per wave
constexpr int TJ = WM / 16;    // 4 MFMA column tiles per wave
constexpr int A_CHUNKS = BN * KBYTES / 16 / THREADS;  // 8 16-byte chunks per thread
constexpr int B_CHUNKS = BM * KBYTES / 16 / THREADS;  // 4
constexpr int STAGE_BYTES = (BN + BM) * KBYTES;        // 48 KiB

struct GemmArgs {
  WeightDev w;
  TileMap tm;
  const uint8_t* xq;
  const float* xs;
  void* y;
  int64_t ldq;
  int64_t ldxs;
  int64_t ldy;
  int32_t M;
  int32_t m_tiles;
  int32_t y_bf16;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * KBYTES + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ float load_scale(const void* s, int64_t idx, int bf16) {
  if (bf16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(s)[idx]) << 16);
  return static_cast<const float*>(s)[idx];
}

// 16 bytes of one row starting at K offset k (bytes past K are zero).
template <bool ALIGNED>
__device__ __forceinline__ uint4 load_chunk(const uint8_t* row, int k, int K, bool row_ok) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (!row_ok) return v;
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

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool ALIGNED>
__global__ __launch_bounds__(THREADS) void w8a8_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

  // ---- tile of this block: member, row tile, token tile
  const int t = blockIdx.x;
  int mi = 0;
  while (mi + 1 < a.w.n_members && t >= a.tm.tile0[mi + 1]) ++mi;
  const int local = t - a.tm.tile0[mi];
  const int nt = local % a.tm.n_tiles[mi];
  const int mt = local / a.tm.n_tiles[mi];
  const MemberDev mem = a.w.m[mi];
  const int n0 = nt * BN;
  const int m0 = mt * BM;
  const int K = a.w.K, Kb = a.w.Kb, M = a.M;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4;

  // ---- staging geometry: each thread owns fixed (row, chunk) slots
  // Thread tid always stages chunk (tid & 7) of rows (tid >> 3) + 32 i.
  const int ch16 = (tid & 7) * 16;
  const uint8_t* a_row[A_CHUNKS];
  bool a_ok[A_CHUNKS];
  int a_dst[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + THREADS * i, row = c >> 3, ch = c & 7;
    a_ok[i] = (n0 + row) < mem.rows;
    a_row[i] = mem.w + int64_t(a_ok[i] ? n0 + row : 0) * K;
    a_dst[i] = swz(row, ch);
  }
  const uint8_t* b_row[B_CHUNKS];
  bool b_ok[B_CHUNKS];
  int b_dst[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int c = tid + THREADS * i, row = c >> 3, ch = c & 7;
    b_ok[i] = (m0 + row) < M;
    b_row[i] = a.xq + int64_t(b_ok[i] ? m0 + row : 0) * a.ldq;
    b_dst[i] = BN * KBYTES + swz(row, ch);
  }

  // ---- scales: one weight scale per wave and K block, one token scale per column tile
  const int srow = (n0 + wn * WN) >> 7;
  const int nb = (mem.rows + 127) >> 7;
  const bool srow_ok = srow < nb;
  const int64_t s_base = int64_t(srow_ok ? srow : 0) * Kb;
  const float* xs_row[TJ];
  bool m_ok[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int m = m0 + wm * WM + 16 * j + l16;
    m_ok[j] = m < M;
    xs_row[j] = a.xs + int64_t(m_ok[j] ? m : 0) * a.ldxs;
  }

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ra[A_CHUNKS], rb[B_CHUNKS];
  auto gload = [&](int kb) {
    const int k = kb * KBYTES + ch16;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) ra[i] = load_chunk<ALIGNED>(a_row[i], k, K, a_ok[i]);
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) rb[i] = load_chunk<ALIGNED>(b_row[i], k, K, b_ok[i]);
  };
  auto lstore = [&](int stage) {
    uint8_t* base = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<uint4*>(base + a_dst[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<uint4*>(base + b_dst[i]) = rb[i];
  };

  gload(0);
  lstore(0);
  __syncthreads();

  float sw_next = srow_ok ? load_scale(mem.s, s_base, a.w.scale_bf16) : 0.f;
  float sa_next[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) sa_next[j] = m_ok[j] ? xs_row[j][0] : 0.f;

  for (int kb = 0; kb < Kb; ++kb) {
    const int stage = kb & 1;
    const bool more = kb + 1 < Kb;
    if (more) gload(kb + 1);
    float s[TJ];
    const float sw = sw_next;
#pragma unroll
    for (int j = 0; j < TJ; ++j) s[j] = sa_next[j] * sw;
    if (more) {
      sw_next = srow_ok ? load_scale(mem.s, s_base + kb + 1, a.w.scale_bf16) : 0.f;
#pragma unroll
      for (int j = 0; j < TJ; ++j) sa_next[j] = m_ok[j] ? xs_row[j][kb + 1] : 0.f;
    }

    const uint8_t* As = smem + stage * STAGE_BYTES;
    const uint8_t* Bs = As + BN * KBYTES;
    v8i bf[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = wm * WM + 16 * j + l16;
      const uint4 lo = *reinterpret_cast<const uint4*>(Bs + swz(r, 2 * g));
      const uint4 hi = *reinterpret_cast<const uint4*>(Bs + swz(r, 2 * g + 1));
      bf[j] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = wn * WN + 16 * i + l16;
      const uint4 lo = *reinterpret_cast<const uint4*>(As + swz(r, 2 * g));
      const uint4 hi = *reinterpret_cast<const uint4*>(As + swz(r, 2 * g + 1));
      const v8i af = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                       0, 0, 0);
        acc[i][j] += p * s[j];
      }
    }
    if (more) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- store: lane holds rows 4*(lane/16)+r of each 16x16 tile, column lane%16
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int m = m0 + wm * WM + 16 * j + l16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int n = n0 + wn * WN + 16 * i + 4 * g;
      const int64_t off = int64_t(m) * a.ldy + mem.col0 + n;
      const int nvalid = mem.rows - n;
      if (nvalid <= 0) continue;
      if (a.y_bf16) {
        uint16_t* y = static_cast<uint16_t*>(a.y) + off;
        const uint16_t b0 = f32_to_bf16_rne(acc[i][j][0]), b1 = f32_to_bf16_rne(acc[i][j][1]);
        const uint16_t b2 = f32_to_bf16_rne(acc[i][j][2]), b3 = f32_to_bf16_rne(acc[i][j][3]);
        if (nvalid >= 4 && (reinterpret_cast<uintptr_t>(y) & 7) == 0) {
          *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(b0) | (uint32_t(b1) << 16), uint32_t(b2) | (uint32_t(b3) << 16));
        } else {
          y[0] = b0;
          if (nvalid > 1) y[1] = b1;
          if (nvalid > 2) y[2] = b2;
          if (nvalid > 3) y[3] = b3;
        }
      } else {
        float* y = static_cast<float*>(a.y) + off;
        if (nvalid >= 4 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
          *reinterpret_cast<float4*>(y) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
          y[0] = acc[i][j][0];
          if (nvalid > 1) y[1] = acc[i][j][1];
          if (nvalid > 2) y[2] = acc[i][j][2];
          if (nvalid > 3) y[3] = acc[i][j][3];
        }
      }
    }
  }
}

struct Plan {
  TileMap tm;
  int m_tiles;
  int blocks;
};

Plan make_plan(const WeightDev& w, int64_t M) {
  Plan p{};
  p.m_tiles = int((M + BM - 1) / BM);
  int t = 0;
  for (int i = 0; i < w.n_members; ++i) {
    p.tm.tile0[i] = t;
    p.tm.n_tiles[i] = (w.m[i].rows + BN - 1) / BN;
    t += p.tm.n_tiles[i] * p.m_tiles;
  }
  p.tm.tile0[w.n_members] = t;
  p.blocks = t;
  return p;
}

}  // namespace

size_t w8a8_workspace_bytes(const WeightDev&, int64_t) { return 0; }

std::string describe_w8a8(const WeightDev& w, bool aligned, int64_t M) {
  const Plan p = make_plan(w, M > 0 ? M : 1);
  char buf[256];
  snprintf(buf, sizeof(buf),
           "arm=w8a8 arithmetic=e4m3xe4m3 mfma_f32_16x16x128_f8f6f4, f32 per-128-K epilogue | kernel=w8a8_gemm "
           "tile=%dx%d waves=4 lds=2x%dKiB path=%s | M=%lld blocks=%d",
           BN, BM, STAGE_BYTES / 1024, aligned ? "aligned16" : "bytewise", (long long)M, p.blocks);
  return buf;
}

bsf8_status launch_w8a8(const WeightDev& w, bool aligned, const uint8_t* xq, int64_t ldq, const float* xs,
                        int64_t ldxs, int64_t M, void* y, bool y_bf16, int64_t ldy, void*, size_t,
                        hipStream_t stream) {
  const Plan p = make_plan(w, M);
  if (p.blocks == 0) return BSF8_OK;
  GemmArgs a{};
  a.w = w;
  a.tm = p.tm;
  a.xq = xq;
  a.xs = xs;
  a.y = y;
  a.ldq = ldq;
  a.ldxs = ldxs;
  a.ldy = ldy;
  a.M = int32_t(M);
  a.m_tiles = p.m_tiles;
  a.y_bf16 = y_bf16 ? 1 : 0;
  if (aligned)
    hipLaunchKernelGGL(w8a8_gemm_kernel<true>, dim3(p.blocks), dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(w8a8_gemm_kernel<false>, dim3(p.blocks), dim3(THREADS), 0, stream, a);
  return device_status(hipGetLastError(), "w8a8_gemm launch");
}

}  // namespace bsf8

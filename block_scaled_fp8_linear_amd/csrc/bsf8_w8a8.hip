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

#include <atomic>
#include <cstdio>
#include <mutex>
#include <string>
#include <type_traits>

#include "bsf8_internal.h"

// buffer_load ... lds: each lane's 16 bytes land at lds + 16 * lane (the LLVM intrinsic).
typedef int bsf8_v4i __attribute__((ext_vector_type(4)));
__device__ void bsf8_raw_buffer_load_lds(bsf8_v4i rsrc, __attribute__((address_space(3))) uint32_t* lds, int size,
                                         int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
// Raw buffer load of 16 bytes into registers; an offset past the resource's size reads zeros.
__device__ bsf8_v4i bsf8_raw_buffer_load_b128(bsf8_v4i rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

namespace bsf8 {
namespace {

typedef bsf8_v4i v4i;
typedef uint32_t __attribute__((address_space(3)))* lds_u32_ptr;
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
  int64_t xs_sm;   // activation scale (m, kb) at xs[m * xs_sm + kb * xs_sk]
  int64_t xs_sk;
  int64_t ldy;
  int32_t M;
  int32_t m_tiles;
  int32_t y_bf16;
};

// 16-byte chunk c of row r lives at chunk position c ^ s(r), with s a
// permutation of r & 7 that sends even rows to {0, 1, 4, 5} and odd rows to
// {2, 3, 6, 7}.  A fragment read (ds_read_b128) has lane (l, g) fetch chunk
// 2g or 2g + 1 of row r0 + l: eight consecutive rows then sit on eight
// distinct positions, and the 16 accesses of rows r0..r0+7 under two adjacent
// lane groups (chunks c and c + 2) cover all 16 (row parity, position) pairs,
// i.e. all 64 four-byte banks.  Measured with SQ_LDS_BANK_CONFLICT: 3 % of the
// LDS's active cycles are conflict stalls, against 48 % with s(r) = (r >> 1) & 7
// and with s(r) = r & 7.  s depends on r & 7 only, so an 8-row copy slab
// fetches the same chunk pattern whatever its position.
__device__ __forceinline__ int swz_pos(int row, int chunk) {
  return chunk ^ (((row & 1) << 1) | ((row >> 1) & 1) | (row & 4));
}
__device__ __forceinline__ int swz(int row, int chunk) { return row * KBYTES + (swz_pos(row, chunk) << 4); }

__device__ __forceinline__ float load_scale(const void* s, int64_t idx, int bf16) {
  if (bf16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(s)[idx]) << 16);
  return static_cast<const float*>(s)[idx];
}

template <bool SBF16>
__device__ __forceinline__ float load_scale_t(const void* s, int64_t idx) {
  if (SBF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(s)[idx]) << 16);
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

// F32 -> BF16 with round-to-nearest-even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction per pair; NaN stays NaN).
typedef __bf16 bsf8_v2bf16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bsf8_v2bf16 r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, r);
}


// Four consecutive outputs of one token (nvalid of them exist) as F32 or BF16 (RNE).
__device__ __forceinline__ void store4(void* yv, int bf16, int64_t off, int nvalid, const v4f& v) {
  if (bf16) {
    uint16_t* y = static_cast<uint16_t*>(yv) + off;
    const uint32_t p01 = bf16_pair(v[0], v[1]), p23 = bf16_pair(v[2], v[3]);
    if (nvalid >= 4 && (reinterpret_cast<uintptr_t>(y) & 7) == 0) {
      *reinterpret_cast<uint2*>(y) = make_uint2(p01, p23);
    } else {
      y[0] = uint16_t(p01);
      if (nvalid > 1) y[1] = uint16_t(p01 >> 16);
      if (nvalid > 2) y[2] = uint16_t(p23);
      if (nvalid > 3) y[3] = uint16_t(p23 >> 16);
    }
  } else {
    float* y = static_cast<float*>(yv) + off;
    if (nvalid >= 4 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
      *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      y[0] = v[0];
      if (nvalid > 1) y[1] = v[1];
      if (nvalid > 2) y[2] = v[2];
      if (nvalid > 3) y[3] = v[3];
    }
  }
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
  const int64_t s_base = int64_t(srow_ok ? srow : 0) * a.w.s_rs;
  const float* xs_row[TJ];
  bool m_ok[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int m = m0 + wm * WM + 16 * j + l16;
    m_ok[j] = m < M;
    xs_row[j] = a.xs + int64_t(m_ok[j] ? m : 0) * a.xs_sm;
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
      sw_next = srow_ok ? load_scale(mem.s, s_base + int64_t(kb + 1) * a.w.s_cs, a.w.scale_bf16) : 0.f;
#pragma unroll
      for (int j = 0; j < TJ; ++j) sa_next[j] = m_ok[j] ? xs_row[j][int64_t(kb + 1) * a.xs_sk] : 0.f;
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
      const int nvalid = mem.rows - n;
      if (nvalid <= 0) continue;
      store4(a.y, a.y_bf16, int64_t(m) * a.ldy + mem.col0 + n, nvalid, acc[i][j]);
    }
  }
}


// ---------------------------------------------------------------------------
// Fast path (K % 16 == 0, 16-byte aligned operands): 512 threads, a T x T
// block tile (T = 256, or 128 for small grids), eight waves of T/2 x T/4 (two
// per SIMD, so one wave's epilogue and
// LDS traffic overlap the other's MFMAs), operands copied HBM -> LDS by
// buffer_load ... lds without passing through registers.  Out-of-range rows,
// tokens and K bytes are given an offset past the buffer's end, which the
// buffer unit returns as zeros.
// ---------------------------------------------------------------------------

constexpr int FTHREADS = 512;
// Operand copies: 1 KiB wave copies (8 rows x 128 bytes) per stage, T/8 weight
// slabs and T/8 token slabs, issued by waves 0-3 between the MFMAs of their
// chains.  The vector memory unit takes a 1 KiB copy about as fast as it
// moves it, so a wave that issues its sixteen copies in one burst stalls for
// most of a K block; spread over the chain, the stalls overlap MFMAs of both
// waves of the SIMD.  Waves 0-3 are the older wave of each SIMD pair and win
// most MFMA issue slots, so their chains, and the copies in them, run early.
// (Copies spread over all eight waves go out late: the younger waves' chains
// lag behind.)
constexpr int F_COPIERS = 4;
// The block tile: T weight rows x T tokens over 2 x 4 waves.  T = 256 is the
// main tile; T = 128 serves grids that 256 x 256 tiles would leave mostly to
// split-K (Q/K/V [8144, 5120] at M = 512: 64 tiles split 4 ways, 43.9 us,
// against 256 whole 128 x 128 tiles, 34.7 us).  A 128 x 128 K block reads
// 12 KiB of fragments per wave for an eighth of the MFMAs, so per FLOP it is
// slower (about 0.55 of a 256 x 256 step for a quarter of the work); the plan
// takes whichever its cost model finds cheaper.
template <int T>
struct FTile {
  static constexpr int BN = T, BM = T;                // weight rows and tokens per block tile
  static constexpr int WN = BN / 2, WM = BM / 4;      // per wave
  static constexpr int TI = WN / 16, TJ = WM / 16;    // 16 x 16 MFMA tiles per wave
  static constexpr int SA = BN * KBYTES + BM * KBYTES;  // offset of the token scales in a stage
  static constexpr int STAGE = SA + BM * 4;             // operands + token scales
  static constexpr int A_LOADS = BN / 8 / F_COPIERS;    // weight slabs per copying wave
  static constexpr int B_LOADS = BM / 8 / F_COPIERS;    // token slabs per copying wave
};
constexpr int XCDS = 8;
// Row tiles per L2 group: 16 when there are at most 4 token tiles (M <= 1024)
// and more tiles than one round, else 8 (measured: gate/up at M = 1024,
// 544 tiles, 170 -> 166 us with 16; the M = 8192 prefill keeps 8, 794 -> 798
// us with 16; the M = 1024 down projection, 80 tiles all split, 92 -> 93 us).
int group_rows_for(int m_tiles, int tiles, int cus) { return m_tiles <= 4 && tiles > cus ? 16 : 8; }
constexpr int F_MAX_KB = 1024;  // K up to 131072 on the fast path

struct FastArgs {
  WeightDev w;
  int32_t rt0[kMaxMembers + 1];   // first row tile (T rows) of each member
  const uint8_t* xq;
  const float* xs;
  void* y;
  int64_t ldq;
  int64_t xs_sm;   // activation scale (m, kb) at xs[m * xs_sm + kb * xs_sk]
  int64_t xs_sk;
  int64_t ldy;
  int32_t M;
  int32_t m_tiles;
  int32_t rt_total;
  int32_t y_bf16;
  int32_t y_vec;   // y, ldy and every member's column offset allow 16-byte stores
  int32_t y_nt;    // the output exceeds half the Infinity Cache: store it non-temporally
  int32_t group_rows;   // row tiles per L2 group
  // split-K for the row tiles from rt_split0 on: their K blocks are cut into
  // `splits` ranges of kb_per_split; split s of tile (R, mt) writes its F32
  // partial tile to ws + s * M * ldws, columns (R - rt_split0) * T + [0, T),
  // and a second kernel adds the partials.  Row tiles below rt_split0 run
  // whole and write y.
  int32_t splits;
  int32_t kb_per_split;
  int32_t rt_split0;
  float* ws;
  int64_t ldws;
};

__device__ __forceinline__ v4i make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32)));
  r[2] = __builtin_amdgcn_readfirstlane(int(bytes));
  r[3] = 0x00020000;
  return r;
}

constexpr int F_OUT_PITCH = 144;  // bytes per token row of the store staging (128 + 16: no bank conflicts)

// Writes a wave's 16 STI x 16 STJ result tile through LDS so that each lane stores 16
// contiguous bytes of one token row (8 lanes fill a 128-byte line).  In the
// MFMA layout a lane holds 4 consecutive outputs of one token, and 16 lanes of
// one instruction touch 16 rows, which turns into many small partial-line
// writes.  `buf` is this wave's 16 STJ x F_OUT_PITCH staging area; the tile goes
// out in rounds of 128 bytes per token row (4 row tiles of bf16, 2 of f32).
//
// NT: non-temporal stores, for an output too large to stay in the Infinity
// Cache for its consumer anyway; they keep it from evicting the operands the
// GEMM is still reading (M = 8192, N = 18432: 302 MB of output, 2-3 % faster).
typedef unsigned int bsf8_u4v __attribute__((ext_vector_type(4)));
template <int STI, int STJ, bool YBF16, bool NT = false>
__device__ __forceinline__ void store_tile_via_lds(const v4f (&acc)[STI][STJ], uint8_t* buf, void* y, int64_t ldy,
                                                   int64_t col0, int n_base, int n_end, int m_base, int M, int lane) {
  constexpr int ESZ = YBF16 ? 2 : 4;
  constexpr int PER_ROUND = 128 / (16 * ESZ);  // row tiles per round
  constexpr int EPC = 16 / ESZ;                // elements per 16-byte chunk
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i0 = 0; i0 < STI; i0 += PER_ROUND) {
#pragma unroll
    for (int j = 0; j < STJ; ++j) {
#pragma unroll
      for (int ii = 0; ii < PER_ROUND; ++ii) {
        const v4f& v = acc[i0 + ii][j];
        uint8_t* dst = buf + (16 * j + l16) * F_OUT_PITCH + (ii * 16 + 4 * g) * ESZ;
        if (YBF16) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2 * STJ; ++t) {   // the wave's 16 STJ token rows, 8 at a time
      const int row = 8 * t + (lane >> 3), ch = lane & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(buf + row * F_OUT_PITCH + ch * 16);
      const int m = m_base + row;
      const int n = n_base + i0 * 16 + ch * EPC;
      const int nvalid = n_end - n;
      if (m >= M || nvalid <= 0) continue;
      uint8_t* out = static_cast<uint8_t*>(y) + (int64_t(m) * ldy + col0 + n) * ESZ;
      if (nvalid >= EPC) {
        if (NT)
          __builtin_nontemporal_store(bsf8_u4v{v.x, v.y, v.z, v.w}, reinterpret_cast<bsf8_u4v*>(out));
        else
          *reinterpret_cast<uint4*>(out) = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < nvalid; ++e) {
          if (YBF16)
            reinterpret_cast<uint16_t*>(out)[e] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
          else
            reinterpret_cast<uint32_t*>(out)[e] = w[e];
        }
      }
    }
  }
}

// Dense arm: two BF16 MFMAs per 32-byte fragment pair.  A fragment holds 16
// BF16 values of one row (chunks 2g and 2g + 1 of its 128-byte K block); the
// first MFMA takes chunk 2g as its K group g and the second chunk 2g + 1, on
// both operands alike, so the pair sums every K element of the block once.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void mfma_bf16_pair(v4f& c, const v8i& a, const v8i& b) {
  const v8bf a0 = __builtin_bit_cast(v8bf, __builtin_shufflevector(a, a, 0, 1, 2, 3));
  const v8bf a1 = __builtin_bit_cast(v8bf, __builtin_shufflevector(a, a, 4, 5, 6, 7));
  const v8bf b0 = __builtin_bit_cast(v8bf, __builtin_shufflevector(b, b, 0, 1, 2, 3));
  const v8bf b1 = __builtin_bit_cast(v8bf, __builtin_shufflevector(b, b, 4, 5, 6, 7));
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, c, 0, 0, 0);
}

// KFULL: K is a multiple of 128 bytes, so no copy needs the ragged-K test.
// DENSE: BF16 operands without scales (the upcast weight of the resident=False
// arm times BF16 activations): w.K counts bytes (2 per element), the MFMAs
// accumulate in place, and there are no scales to stage or apply.
template <int T, bool SBF16, bool KFULL, bool DENSE>
__global__ __launch_bounds__(FTHREADS) void w8a8_gemm_fast_kernel(FastArgs a) {
  using C = FTile<T>;
  constexpr int FBN = C::BN, FBM = C::BM, F_SA = C::SA, F_STAGE = C::STAGE;
  constexpr int F_A_LOADS = C::A_LOADS, F_B_LOADS = C::B_LOADS;
  constexpr int WN = C::WN, WM = C::WM, TI = C::TI, TJ = C::TJ;
  // Two separate stage arrays (not one array indexed by stage): the compiler
  // must wait for in-flight LDS copies before any LDS read it cannot prove
  // disjoint from them, and distinct objects let it see that reading stage 0
  // does not touch the copy landing in stage 1.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[F_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[F_STAGE];
  __shared__ float wscale[2][F_MAX_KB];   // the block's two rows of the weight scale grid

  // ---- XCD-aware tile order.  Blocks are dealt to the 8 XCDs round robin, and
  // each XCD runs its blocks in order.  Two kinds of work are dealt evenly to
  // every XCD, whole tiles first and split tiles (K ranges of the last row
  // tiles) after them; within each kind an XCD walks a contiguous run of
  // tiles in groups of group_rows row tiles x all token tiles, so blocks that
  // run together share operands in that XCD's L2.  Split work walks
  // (split, row tile) pairs split-major: a group shares one K range.
  const int nblk = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b % XCDS;
  const int l = b / XCDS;
  const int split_rows = a.rt_total - a.rt_split0;
  const int n_whole = a.rt_split0 * a.m_tiles;
  int start_whole = 0, start_split = 0;
  for (int y = 0; y < xcd; ++y) {
    const int ny = (nblk - y + XCDS - 1) / XCDS, nwy = (n_whole - y + XCDS - 1) / XCDS;
    start_whole += nwy;
    start_split += ny - nwy;
  }
  const int n_whole_here = (n_whole - xcd + XCDS - 1) / XCDS;
  const bool whole = l < n_whole_here;
  const int v = whole ? start_whole + l : start_split + (l - n_whole_here);
  const int vr_total = whole ? a.rt_split0 : split_rows * a.splits;
  const int GROUP_ROWS = a.group_rows;
  const int gsz = GROUP_ROWS * a.m_tiles;
  const int grp = v / gsz;
  const int in_grp = v - grp * gsz;
  const int g_rows = min(GROUP_ROWS, vr_total - grp * GROUP_ROWS);
  const int VR = grp * GROUP_ROWS + in_grp % g_rows;
  const int mt = in_grp / g_rows;
  const int split = whole ? 0 : VR / split_rows;
  const int R = whole ? VR : a.rt_split0 + (VR - split * split_rows);
  int mi = 0;
  while (mi + 1 < a.w.n_members && R >= a.rt0[mi + 1]) ++mi;
  const MemberDev mem = a.w.m[mi];
  const int n0 = (R - a.rt0[mi]) * FBN;
  const int m0 = mt * FBM;
  const int K = a.w.K, Kb = a.w.Kb, M = a.M;
  const int kb_begin = whole ? 0 : split * a.kb_per_split;
  const int kb_end = whole ? Kb : min(Kb, kb_begin + a.kb_per_split);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4;

  // ---- buffer resources and per-lane copy offsets (fixed per K block but for kb*128)
  const uint32_t a_bytes = uint32_t(mem.rows) * uint32_t(K);
  const uint32_t b_bytes = uint32_t(M) * uint32_t(a.ldq);
  const v4i ra = make_rsrc(mem.w, a_bytes);
  const v4i rb = make_rsrc(a.xq, b_bytes);
  // the scales' extent in bytes (below 2^31: the plan checks it)
  const uint32_t s_bytes = uint32_t(((int64_t(M) - 1) * a.xs_sm + int64_t(Kb - 1) * a.xs_sk + 1) * 4);
  const v4i rs = make_rsrc(a.xs, s_bytes);
  // waves 0..T/64-1 each copy the scales of 64 tokens (one 4-byte element per
  // lane).  Lane L fetches token 16 (L & 3) + (L >> 2) of its wave's 64, so the
  // four scales a compute lane of a 64-token wave needs (tokens l16 + 16 j,
  // j = 0..3) sit in one 16-byte LDS word (a 32-token wave's two, in 8 bytes).  With K-major scales (xs_sm = 1) a wave's copy reads
  // 256 contiguous bytes; token-major, 64 words a row pitch apart.
  const bool s_wave = wave < FBM / 64;
  const int s_tok = m0 + wave * 64 + 16 * (lane & 3) + (lane >> 2);
  const bool s_ok = s_wave && s_tok < M;
  const int s_off = s_ok ? s_tok * int(a.xs_sm) * 4 : 0;
  const int s_kstep = int(a.xs_sk) * 4;
  // Lane L of a 1 KiB wave copy fills chunk position L & 7 of row L >> 3 of its
  // 8-row slab; since the swizzle depends on r & 7 only, the logical chunk it
  // fetches is the same for every slab.
  const int crow = lane >> 3;
  const uint32_t ch_lane = uint32_t(swz_pos(crow, lane & 7) * 16);
  const int cw = wave;              // copier index (valid when copier)
  const bool copier = F_COPIERS * 64 >= FTHREADS || wave < F_COPIERS;
  const int a_row0 = n0 + cw * F_A_LOADS * 8 + crow;   // row of slab i is a_row0 + 8 i
  const int b_row0 = m0 + cw * F_B_LOADS * 8 + crow;
  // Copy number c (0 .. F_A_LOADS + F_B_LOADS - 1) of K block kb into a stage:
  // the first F_A_LOADS are weight slabs, the rest token slabs.
  // Row parts of the copy offsets, per lane; a row past the operand's end
  // lands past the buffer's end (zeros), so only a ragged K needs a test.
  // The K block's part goes through a scalar register, which keeps the
  // compiler from holding every copy's offset in its own vector register.
  const uint32_t a_lane = uint32_t(a_row0) * uint32_t(K);
  const uint32_t b_lane = uint32_t(b_row0) * uint32_t(a.ldq);
  auto issue_one = [&](int kb, uint8_t* base, int c) {
    const uint32_t kbo = uint32_t(kb) * KBYTES;
    if (c < F_A_LOADS) {
      const int i = c;
      const uint32_t ch = ch_lane;
      const uint32_t sc = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(8 * i) * uint32_t(K) + kbo)));
      const uint32_t off = KFULL || kbo + ch < uint32_t(K) ? a_lane + ch + sc : a_bytes;
      bsf8_raw_buffer_load_lds(ra, (lds_u32_ptr)(base + (cw * F_A_LOADS + i) * 1024), 16, int(off), 0, 0, 0);
    } else {
      const int i = c - F_A_LOADS;
      const uint32_t ch = ch_lane;
      const uint32_t sc = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(8 * i) * uint32_t(a.ldq) + kbo)));
      const uint32_t off = KFULL || kbo + ch < uint32_t(K) ? b_lane + ch + sc : b_bytes;
      bsf8_raw_buffer_load_lds(rb, (lds_u32_ptr)(base + FBN * KBYTES + (cw * F_B_LOADS + i) * 1024), 16, int(off), 0,
                               0, 0);
    }
  };
  auto issue_scales = [&](int kb, uint8_t* base) {
    if constexpr (!DENSE) {
      if (s_wave) {
        const int off = s_ok ? s_off + kb * s_kstep : int(s_bytes);
        bsf8_raw_buffer_load_lds(rs, (lds_u32_ptr)(base + F_SA + wave * 256), 4, off, 0, 0, 0);
      }
    }
  };
  auto issue = [&](int kb, uint8_t* base) {
    if (copier) {
#pragma unroll
      for (int c = 0; c < F_A_LOADS + F_B_LOADS; ++c) issue_one(kb, base, c);
    }
    issue_scales(kb, base);
  };

  // The first K block's copies go out before the weight scales are staged, so
  // the two memory latencies overlap (the first step's barrier covers both).
  issue(kb_begin, stage0);

  // ---- weight scales: rows (n0 >> 7) and (n0 >> 7) + 1 of the member's grid
  // (one per wave half of a 256-row tile; a 128-row tile uses the first),
  // staged in LDS once; a missing row reads as zero
  if constexpr (!DENSE) {
    const int nb = (mem.rows + 127) >> 7;
    for (int i = tid; i < 2 * Kb; i += FTHREADS) {
      const int h = i >= Kb, kb = i - h * Kb;
      const int srow = (n0 >> 7) + h;
      wscale[h][kb] = srow < nb ? load_scale_t<SBF16>(mem.s, int64_t(srow) * a.w.s_rs + int64_t(kb) * a.w.s_cs) : 0.f;
    }
  }

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};


  // LDS fragment reads of a stage (swizzled 128-byte rows).
  auto read_b = [&](const uint8_t* st, int j) {
    const uint8_t* Bs = st + FBN * KBYTES;
    const int r = wm * WM + 16 * j + l16;
    const uint4 lo = *reinterpret_cast<const uint4*>(Bs + swz(r, 2 * g));
    const uint4 hi = *reinterpret_cast<const uint4*>(Bs + swz(r, 2 * g + 1));
    return v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
  };
  auto read_a = [&](const uint8_t* st, int i) {
    const int r = wn * WN + 16 * i + l16;
    const uint4 lo = *reinterpret_cast<const uint4*>(st + swz(r, 2 * g));
    const uint4 hi = *reinterpret_cast<const uint4*>(st + swz(r, 2 * g + 1));
    return v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
  };
  // A block's B fragments and first A fragment, in the order its chain needs
  // them.
  auto read_head = [&](const uint8_t* st, v8i(&bfx)[TJ], v8i& a0) __attribute__((always_inline)) {
    bfx[0] = read_b(st, 0);
    a0 = read_a(st, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 1; j < TJ; ++j) bfx[j] = read_b(st, j);
    __builtin_amdgcn_sched_barrier(0);
  };

  // One K block, kb, in stage `cur`; block kb + 1 lands in `nxt`.  Its B
  // fragments (bf) and first A fragment (af[0]) were read before it started.
  // The block barrier sits at MFMA BARQ of the chain, the first MFMA of the
  // last row tile, when every read of `cur` has been made: past it `cur` may
  // be refilled (with block kb + 2), and the copies of block kb + 1 have
  // landed, so the next block's first A fragment is read at once and each of
  // its B fragments right after the last MFMA that uses the current one; the
  // last row tile's MFMAs cover those reads and the next chain starts without
  // waiting on a burst of LDS reads.  A copying wave issues two copies per
  // MFMA: block kb + 2's first NTAIL right after the barrier (into `cur`),
  // the rest over the next chain's first MFMAs, so every copy has most of a K
  // block to land.  (One copy per MFMA over the chain's first MFMAs was slower
  // on weights streamed from HBM; all sixteen at once stall the copying wave.)
  // Near the end of the range the copies repeat the last block (in bounds,
  // never read), so the chain needs no test.
  constexpr int BARQ = (TI - 1) * TJ;
  constexpr int NCOPY = F_A_LOADS + F_B_LOADS;
  constexpr int CPM = 2;
  constexpr int NTAIL = (TI * TJ - BARQ) * CPM;
  static_assert(NTAIL <= NCOPY && (NCOPY - NTAIL) % CPM == 0 && (NCOPY - NTAIL) / CPM <= BARQ, "copies fit the chain");
  auto step = [&](int kb, const uint8_t* cur, uint8_t* nxt, v8i(&bf)[TJ], v8i(&af)[2],
                  auto copy_tag) __attribute__((always_inline)) {
    constexpr bool COPY = decltype(copy_tag)::value;
    const int k1 = min(kb + 1, kb_end - 1);
    const int k2 = min(kb + 2, kb_end - 1);
    if (kb + 1 < kb_end) issue_scales(kb + 1, nxt);   // the next block's token scales
    float sw = 0.f;
    float4 sa = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (!DENSE) {
      sw = wscale[WN >= 128 ? wn : 0][kb];   // a 128-row tile lies in one scale row
      if constexpr (TJ == 4) {
        sa = *reinterpret_cast<const float4*>(cur + F_SA + wm * 256 + 16 * l16);
      } else {
        // 32 tokens per wave: tokens 32 wm + 16 j + l16, j = 0, 1, sit at
        // positions 4 l16 + 2 (wm & 1) + j of their 64-token copy group
        const float2 s2 = *reinterpret_cast<const float2*>(cur + F_SA + (wm >> 1) * 256 + 16 * l16 + 8 * (wm & 1));
        sa = make_float4(s2.x, s2.y, 0.f, 0.f);
      }
    }
    float s[TJ];
    // The 32 MFMAs of the K block run as one rotated chain: the epilogue FMAs
    // that consume MFMA q's partial are issued after MFMA q + 2 (three
    // 4-register partial buffers), far enough behind for its result to be ready
    // without wait states, and the A fragment of row tile i + 1 is read from LDS
    // while tile i's MFMAs run.
    constexpr int LAG = 2;
    v4f part[LAG + 1];
#pragma unroll
    for (int q = 0; q < TI * TJ + LAG; ++q) {
      if (q < TI * TJ) {
        const int i = q / TJ, j = q % TJ;
        if (q == BARQ) {
          // this wave's copies into `nxt` have landed and its reads of `cur`
          // are done; after the barrier everyone's are
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          af[0] = read_a(nxt, 0);
        }
        if (j == 0 && i + 1 < TI) af[(i + 1) & 1] = read_a(cur, i + 1);
        if constexpr (DENSE)
          mfma_bf16_pair(acc[i][j], af[i & 1], bf[j]);
        else
          part[q % (LAG + 1)] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i & 1], bf[j],
                                                                               v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        if (q >= BARQ) bf[j] = read_b(nxt, j);   // its last use in this block was the MFMA above
      }
      if constexpr (COPY) {
        if (q >= BARQ && q < TI * TJ) {
#pragma unroll
          for (int t = 0; t < CPM; ++t) issue_one(k2, const_cast<uint8_t*>(cur), CPM * (q - BARQ) + t);
        }
        if (q < (NCOPY - NTAIL) / CPM) {
#pragma unroll
          for (int t = 0; t < CPM; ++t) issue_one(k1, nxt, NTAIL + CPM * q + t);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!DENSE) {
        if (q == LAG) {   // the scale products, first needed here
          s[0] = sa.x * sw;
          s[1] = sa.y * sw;
          if constexpr (TJ == 4) {
            s[2] = sa.z * sw;
            s[3] = sa.w * sw;
          }
        }
        if (q >= LAG) {
          const int c = q - LAG, ci = c / TJ, cj = c % TJ;
          acc[ci][cj] += part[c % (LAG + 1)] * s[cj];
        }
      }
      // (the scheduling barriers keep each MFMA ahead of the FMAs issued after it)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The second block's first copies (the ones a chain issues after its
  // barrier), then the first block's head fragments.
  if (copier) {
    const int k1 = min(kb_begin + 1, kb_end - 1);
#pragma unroll
    for (int c = 0; c < NTAIL; ++c) issue_one(k1, stage1, c);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  v8i bf[TJ], af[2];
  read_head(stage0, bf, af[0]);

  // Copying waves and the others run separate copies of the main loop and
  // the store, so no MFMA chain holds a branch (a branch in the chain costs
  // the register allocator dearly).
  auto finish = [&](auto copy_tag) __attribute__((always_inline)) {
    for (int kb = kb_begin; kb < kb_end; kb += 2) {
      step(kb, stage0, stage1, bf, af, copy_tag);
      if (kb + 1 < kb_end) step(kb + 1, stage1, stage0, bf, af, copy_tag);
    }

    // ---- store
    if (!whole || a.y_vec) {
      // every wave is done reading both stages
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      uint8_t* buf = (wave < 4 ? stage0 : stage1) + (wave & 3) * (WM * F_OUT_PITCH);
      if (!whole)
        store_tile_via_lds<TI, TJ, false>(acc, buf, a.ws + int64_t(split) * M * a.ldws, a.ldws,
                                  int64_t(R - a.rt_split0) * FBN - n0, n0 + wn * WN, mem.rows, m0 + wm * WM, M, lane);
      else if (a.y_bf16 && a.y_nt)
        store_tile_via_lds<TI, TJ, true, true>(acc, buf, a.y, a.ldy, mem.col0, n0 + wn * WN, mem.rows, m0 + wm * WM, M, lane);
      else if (a.y_bf16)
        store_tile_via_lds<TI, TJ, true>(acc, buf, a.y, a.ldy, mem.col0, n0 + wn * WN, mem.rows, m0 + wm * WM, M, lane);
      else if (a.y_nt)
        store_tile_via_lds<TI, TJ, false, true>(acc, buf, a.y, a.ldy, mem.col0, n0 + wn * WN, mem.rows, m0 + wm * WM, M, lane);
      else
        store_tile_via_lds<TI, TJ, false>(acc, buf, a.y, a.ldy, mem.col0, n0 + wn * WN, mem.rows, m0 + wm * WM, M, lane);
      return;
    }
    // unaligned output: lane holds rows 4*(lane/16)+r of each 16x16 tile, column lane%16
  #pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = m0 + wm * WM + 16 * j + l16;
      if (m >= M) continue;
  #pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int n = n0 + wn * WN + 16 * i + 4 * g;
        const int nvalid = mem.rows - n;
        if (nvalid <= 0) continue;
        store4(a.y, a.y_bf16, int64_t(m) * a.ldy + mem.col0 + n, nvalid, acc[i][j]);
      }
    }
  };
  if (copier) finish(std::true_type{});
  else finish(std::false_type{});
}

// Split-K partial sums: for workspace column c (row tile R = rt_split0 +
// c / T, member i holding R, row n of member i), y[m, col0_i + n] = sum over
// s = 0 .. S-1, in that order, of ws[s][m][c].  One thread per 4 columns.
struct ReduceArgs {
  const float* ws;
  int64_t ldws;
  int64_t split_stride;  // M * ldws
  void* y;
  int64_t ldy;
  int32_t M;
  int32_t splits;
  int32_t y_bf16;
  int32_t n_members;
  int32_t rt_split0;
  int32_t tile_n;       // weight rows per block tile (T)
  int32_t rt0[kMaxMembers + 1];
  int32_t rows[kMaxMembers];
  int32_t col0[kMaxMembers];
};

__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceArgs a) {
  const int64_t c4_per_row = a.ldws / 4;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(a.M) * c4_per_row) return;
  const int m = int(idx / c4_per_row);
  const int c = int(idx - int64_t(m) * c4_per_row) * 4;
  const int R = a.rt_split0 + c / a.tile_n;
  int i = 0;
  while (i + 1 < a.n_members && R >= a.rt0[i + 1]) ++i;
  const int n = (R - a.rt0[i]) * a.tile_n + c % a.tile_n;
  const int nvalid = a.rows[i] - n;
  if (nvalid <= 0) return;
  const float* p = a.ws + int64_t(m) * a.ldws + c;
  float4 t = *reinterpret_cast<const float4*>(p);
  for (int sp = 1; sp < a.splits; ++sp) {
    const float4 u = *reinterpret_cast<const float4*>(p + sp * a.split_stride);
    t.x += u.x;
    t.y += u.y;
    t.z += u.z;
    t.w += u.w;
  }
  store4(a.y, a.y_bf16, int64_t(m) * a.ldy + a.col0[i] + n, nvalid, v4f{t.x, t.y, t.z, t.w});
}

struct Plan {
  bool fast;
  int tile;           // fast kernel: the block tile T (T x T)
  TileMap tm;         // register-staged kernel: member tiles
  int32_t rt0[kMaxMembers + 1];
  int rt_total;
  int m_tiles;
  int blocks;
  int splits;         // fast kernel: K ranges of each split row tile (1: none)
  int kb_per_split;
  int rt_split0;      // first split row tile (rt_total when none)
  int64_t ldws;       // split workspace row pitch (floats)
  size_t ws_bytes;
};

// Compute units of the current device (cached per device).
int device_cus() {
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

// Split-K where the tile grid leaves compute units idle: every tile when there
// are fewer tiles than compute units, else the row tiles of the last, partly
// filled round.  Cost model in units of one 256 x 256 tile-K-block step (about
// 1.6 us of GPU time at full occupancy): whole tiles run ceil(n / CUs) rounds
// of Kb steps, split tiles ceil(n * S / CUs) rounds of ceil(Kb / S) steps, and
// each split partial tile costs `part` (0.06 step for 256 x 256) to write and
// read back, plus two steps for the second kernel; every round of blocks adds
// four steps of start-up and result stores.  A 128 x 128 K block costs `step`
// = 0.555 of a 256 x 256 one and its partial tile 0.015.  (Without the round
// term the model gives 23 / 31 / 43 / 58 us for Q/K/V [8144, 5120] at M =
// 128 / 256 / 512 / 1024 on 256 x 256 tiles, against 25 / 31 / 44 / 59
// measured; the round term only weighs plans with different round counts,
// and with it the cheaper tile was picked on all 18 shapes timed both ways.)
constexpr double kRoundSteps = 4.0;
struct SplitChoice {
  int splits;
  int split_rows;
  double cost;
};

SplitChoice choose_splits(int rt_total, int m_tiles, int Kb, int cus, double step, double part) {
  const int tiles = rt_total * m_tiles;
  const int tail = tiles <= cus ? tiles : tiles % cus;
  const int rounds = (tiles + cus - 1) / cus;
  SplitChoice best{1, 0, double(rounds) * (Kb * step + kRoundSteps)};
  if (tail == 0) return best;
  const int split_rows = tiles <= cus ? rt_total : (tail + m_tiles - 1) / m_tiles;
  const int whole = (rt_total - split_rows) * m_tiles;
  const int split_tiles = split_rows * m_tiles;
  for (int sp = 2; sp <= 8; ++sp) {
    const int kps = (Kb + sp - 1) / sp;
    if (kps < 4) break;
    const int r_whole = (whole + cus - 1) / cus;
    const int r_split = int((int64_t(split_tiles) * sp + cus - 1) / cus);
    const double cost = r_whole * (Kb * step + kRoundSteps) + r_split * (kps * step + kRoundSteps) +
                        part * sp * split_tiles + 2.0;
    if (cost < best.cost - 1e-9) best = SplitChoice{sp, split_rows, cost};
  }
  return best;
}

// The direct-copy kernel addresses each operand with 32-bit byte offsets from
// its base, so every member, the activation block and its scales must stay
// below 2^31 bytes.
// (xs_extent: elements spanned by the activation scales; -1: M x Kb.)
Plan make_plan(const WeightDev& w, bool aligned, int64_t M, int64_t ldq, int64_t xs_extent = -1) {
  Plan p{};
  if (xs_extent < 0) xs_extent = M * w.Kb;
  bool fits = M * ldq < (int64_t(1) << 31) && xs_extent * 4 < (int64_t(1) << 31);
  for (int i = 0; i < w.n_members; ++i) fits = fits && int64_t(w.m[i].rows) * w.K < (int64_t(1) << 31);
  p.fast = aligned && fits && w.Kb <= F_MAX_KB;
  if (p.fast) {
    // the tile (256 or 128) with the lower modelled cost, 256 on a tie
    SplitChoice sc{};
    for (const int T : {256, 128}) {
      const int m_tiles = int((M + T - 1) / T);
      int r = 0;
      for (int i = 0; i < w.n_members; ++i) r += (w.m[i].rows + T - 1) / T;
      const SplitChoice c = T == 256 ? choose_splits(r, m_tiles, w.Kb, device_cus(), 1.0, 0.06)
                                     : choose_splits(r, m_tiles, w.Kb, device_cus(), 0.555, 0.015);
      if (T == 256 || c.cost < sc.cost - 1e-9) {
        sc = c;
        p.tile = T;
      }
    }
    const int T = p.tile;
    p.m_tiles = int((M + T - 1) / T);
    int r = 0;
    for (int i = 0; i < w.n_members; ++i) {
      p.rt0[i] = r;
      r += (w.m[i].rows + T - 1) / T;
    }
    for (int i = w.n_members; i <= kMaxMembers; ++i) p.rt0[i] = r;
    p.rt_total = r;
    p.kb_per_split = (w.Kb + sc.splits - 1) / sc.splits;
    p.splits = (w.Kb + p.kb_per_split - 1) / p.kb_per_split;  // no empty split
    const int split_rows = p.splits > 1 ? sc.split_rows : 0;
    p.rt_split0 = r - split_rows;
    p.ldws = int64_t(split_rows) * T;
    p.blocks = p.rt_split0 * p.m_tiles + split_rows * p.m_tiles * p.splits;
    p.ws_bytes = p.splits > 1 ? size_t(p.splits) * size_t(M) * size_t(p.ldws) * sizeof(float) : 0;
    return p;
  }
  p.splits = 1;
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

// An upper bound over the paths a call may take: the split plan of the fast
// kernel for packed activations (the register-staged kernel needs none).
size_t w8a8_workspace_bytes(const WeightDev& w, int64_t M) {
  if (M <= 0) return 0;
  return make_plan(w, true, M, w.K).ws_bytes;
}

std::string describe_w8a8(const WeightDev& w, bool aligned, int64_t M) {
  if (w8a8_stream_applies(w, aligned, M > 0 ? M : 1, w.K)) return describe_w8a8_stream(w, M > 0 ? M : 1);
  const Plan p = make_plan(w, aligned, M > 0 ? M : 1, w.K);
  char buf[320];
  if (p.fast)
    snprintf(buf, sizeof(buf),
             "arm=w8a8 arithmetic=e4m3xe4m3 mfma_f32_16x16x128_f8f6f4, f32 per-128-K epilogue | "
             "kernel=w8a8_gemm_fast tile=%dx%d waves=8 lds=2x%dKiB (two stage arrays) buffer_load_lds "
             "xcd_groups=%d split_k=%d split_row_tiles=%d | M=%lld blocks=%d",
             p.tile, p.tile, (p.tile == 256 ? FTile<256>::STAGE : FTile<128>::STAGE) / 1024,
             group_rows_for(p.m_tiles, p.rt_total * p.m_tiles, device_cus()), p.splits,
             p.rt_total - p.rt_split0, (long long)M, p.blocks);
  else
    snprintf(buf, sizeof(buf),
             "arm=w8a8 arithmetic=e4m3xe4m3 mfma_f32_16x16x128_f8f6f4, f32 per-128-K epilogue | "
             "kernel=w8a8_gemm tile=%dx%d waves=4 lds=2x%dKiB path=%s | M=%lld blocks=%d",
             BN, BM, STAGE_BYTES / 1024, aligned ? "aligned16" : "bytewise", (long long)M, p.blocks);
  return buf;
}

namespace {

// Fast-kernel launch (and the split-K reduction when the plan splits).
bsf8_status launch_fast(const Plan& p, const WeightDev& w, bool dense, const uint8_t* xq, int64_t ldq,
                        const float* xs, int64_t xs_sm, int64_t xs_sk, int64_t M, void* y, bool y_bf16, int64_t ldy,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  FastArgs a{};
  a.w = w;
  for (int i = 0; i <= kMaxMembers; ++i) a.rt0[i] = p.rt0[i];
  a.xq = xq;
  a.xs = xs;
  a.y = y;
  a.ldq = ldq;
  a.xs_sm = xs_sm;
  a.xs_sk = xs_sk;
  a.ldy = ldy;
  a.M = int32_t(M);
  a.m_tiles = p.m_tiles;
  a.rt_total = p.rt_total;
  a.group_rows = group_rows_for(p.m_tiles, p.rt_total * p.m_tiles, device_cus());
  a.y_bf16 = y_bf16 ? 1 : 0;
  const int64_t esz = y_bf16 ? 2 : 4;
  bool vec = (reinterpret_cast<uintptr_t>(y) & 15) == 0 && (ldy * esz) % 16 == 0;
  for (int i = 0; i < w.n_members; ++i) vec = vec && (w.m[i].col0 * esz) % 16 == 0;
  a.y_vec = vec ? 1 : 0;
  a.y_nt = M * int64_t(w.m[w.n_members - 1].col0 + w.m[w.n_members - 1].rows) * esz > (int64_t(128) << 20) ? 1 : 0;
  a.splits = p.splits;
  a.kb_per_split = p.kb_per_split;
  a.rt_split0 = p.rt_split0;
  a.ldws = p.ldws;
  if (p.splits > 1) {
    if (ws == nullptr || ws_bytes < p.ws_bytes || (reinterpret_cast<uintptr_t>(ws) & 255) != 0) {
      set_error("WORKSPACE: split-K needs %zu bytes of 256-byte aligned workspace", p.ws_bytes);
      return BSF8_E_WORKSPACE;
    }
    a.ws = static_cast<float*>(ws);
  }
  const bool kfull = w.K % KBYTES == 0;
  using Kern = void (*)(FastArgs);
  Kern kern;
#define BSF8_FAST(T)                                                                                          \
  (dense ? (kfull ? w8a8_gemm_fast_kernel<T, false, true, true> : w8a8_gemm_fast_kernel<T, false, false, true>) \
   : w.scale_bf16 ? (kfull ? w8a8_gemm_fast_kernel<T, true, true, false> : w8a8_gemm_fast_kernel<T, true, false, false>) \
                  : (kfull ? w8a8_gemm_fast_kernel<T, false, true, false> : w8a8_gemm_fast_kernel<T, false, false, false>))
  kern = p.tile == 256 ? BSF8_FAST(256) : BSF8_FAST(128);
#undef BSF8_FAST
  hipLaunchKernelGGL(kern, dim3(p.blocks), dim3(FTHREADS), 0, stream, a);
  bsf8_status st = device_status(hipGetLastError(), dense ? "dense_gemm launch" : "w8a8_gemm_fast launch");
  if (st != BSF8_OK || p.splits == 1) return st;
  ReduceArgs r{};
  r.ws = a.ws;
  r.ldws = p.ldws;
  r.split_stride = M * p.ldws;
  r.y = y;
  r.ldy = ldy;
  r.M = int32_t(M);
  r.splits = p.splits;
  r.y_bf16 = y_bf16 ? 1 : 0;
  r.n_members = w.n_members;
  r.rt_split0 = p.rt_split0;
  r.tile_n = p.tile;
  for (int i = 0; i <= kMaxMembers; ++i) r.rt0[i] = p.rt0[i];
  for (int i = 0; i < w.n_members; ++i) {
    r.rows[i] = w.m[i].rows;
    r.col0[i] = w.m[i].col0;
  }
  const int64_t threads = M * (p.ldws / 4);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, r);
  return device_status(hipGetLastError(), "splitk_reduce launch");
}

// The dense BF16 weight [N, K] as the fast kernel's single member: rows of
// 2K bytes, no scales.
WeightDev dense_weight(const uint16_t* wd, int64_t N, int64_t K) {
  WeightDev w{};
  w.m[0].w = reinterpret_cast<const uint8_t*>(wd);
  w.m[0].s = nullptr;
  w.m[0].rows = int32_t(N);
  w.m[0].col0 = 0;
  w.n_members = 1;
  w.K = int32_t(2 * K);
  w.Kb = int32_t((2 * K + KBYTES - 1) / KBYTES);
  return w;
}

}  // namespace

bool dense_supported(int64_t N, int64_t K, int64_t M, int64_t ldx) {
  if (N <= 0 || K <= 0 || N > INT32_MAX || 2 * K > int64_t(F_MAX_KB) * KBYTES) return false;
  return make_plan(dense_weight(nullptr, N, K), true, M > 0 ? M : 1, 2 * ldx).fast;
}

size_t dense_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  if (M <= 0 || !dense_supported(N, K, M, K)) return 0;
  return make_plan(dense_weight(nullptr, N, K), true, M, 2 * K).ws_bytes;
}

std::string describe_dense(int64_t N, int64_t K, int64_t M) {
  const int64_t m = M > 0 ? M : 1;
  if (!dense_supported(N, K, m, K)) return "arm=dense unsupported shape";
  const Plan p = make_plan(dense_weight(nullptr, N, K), true, m, 2 * K);
  char buf[320];
  snprintf(buf, sizeof(buf),
           "arm=dense arithmetic=bf16xbf16 mfma_f32_16x16x32_bf16 (two per 128-byte K block), f32 accumulate | "
           "kernel=w8a8_gemm_fast<dense> tile=%dx%d waves=8 buffer_load_lds xcd_groups=%d split_k=%d "
           "split_row_tiles=%d | M=%lld blocks=%d | dense weight N=%lld K=%lld bf16",
           p.tile, p.tile, group_rows_for(p.m_tiles, p.rt_total * p.m_tiles, device_cus()), p.splits,
           p.rt_total - p.rt_split0, (long long)m, p.blocks, (long long)N,
           (long long)K);
  return buf;
}

bsf8_status launch_dense(const uint16_t* wd, int64_t N, int64_t K, const uint16_t* x, int64_t M, int64_t ldx,
                         void* y, bool y_bf16, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
  const WeightDev w = dense_weight(wd, N, K);
  const Plan p = make_plan(w, true, M, 2 * ldx);
  if (!p.fast) {
    set_error("UNSUPPORTED: dense GEMM shape N=%lld K=%lld M=%lld", (long long)N, (long long)K, (long long)M);
    return BSF8_E_UNSUPPORTED;
  }
  if (p.blocks == 0) return BSF8_OK;
  return launch_fast(p, w, true, reinterpret_cast<const uint8_t*>(x), 2 * ldx, nullptr, 0, 0, M, y, y_bf16, ldy,
                     ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry point (bsf8_linear_w8a8_noalloc): the
// split-K partial tiles go here instead of a caller workspace.  Each device
// holds its own copy of this array from the library's load until the process
// ends.  Its name is only a host-side stand-in: kernels are given the device
// address hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.  Nothing in it needs to start at zero (every split
// writes the whole partial tile it later reads), and calls that overlap in
// time on one device share it, so they race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[BSF8_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

bsf8_status w8a8_noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices) {
    set_error("DEVICE: device index %d beyond the %d the no-allocation scratch table covers", dev, kScratchDevices);
    return BSF8_E_DEVICE;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
      if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255) != 0) {
        set_error("DEVICE: the no-allocation scratch has no 256-byte aligned device address");
        return BSF8_E_DEVICE;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return BSF8_OK;
}

bsf8_status launch_w8a8(const WeightDev& w, bool aligned, const uint8_t* xq, int64_t ldq, const float* xs,
                        int64_t xs_sm, int64_t xs_sk, int64_t M, void* y, bool y_bf16, int64_t ldy, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  if (w8a8_stream_applies(w, aligned, M, ldq))
    return launch_w8a8_stream(w, xq, ldq, xs, xs_sm, xs_sk, M, y, y_bf16, ldy, stream);
  const Plan p = make_plan(w, aligned, M, ldq, (M - 1) * xs_sm + (w.Kb - 1) * xs_sk + 1);
  if (p.blocks == 0) return BSF8_OK;
  if (p.fast) return launch_fast(p, w, false, xq, ldq, xs, xs_sm, xs_sk, M, y, y_bf16, ldy, ws, ws_bytes, stream);
  GemmArgs a{};
  a.w = w;
  a.tm = p.tm;
  a.xq = xq;
  a.xs = xs;
  a.y = y;
  a.ldq = ldq;
  a.xs_sm = xs_sm;
  a.xs_sk = xs_sk;
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

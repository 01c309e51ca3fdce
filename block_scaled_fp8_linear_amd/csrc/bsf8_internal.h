// Internal declarations shared by the host side and the kernel launchers of libbsf8.
// Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "bsf8.h"

namespace bsf8 {

constexpr int kBlock = 128;       // weight_block_size and activation group width
constexpr int kMaxMembers = BSF8_MAX_MEMBERS;

// One grouped member as the kernels see it (passed by value in kernel args).
struct MemberDev {
  const uint8_t* w;   // [rows, K] E4M3 bytes, row stride K
  const void* s;      // BF16 or F32 scales: the [ceil(rows/128), Kb] grid, or one per-tensor value
  int32_t rows;       // N_i
  int32_t col0;       // R_i: first output feature of this member in Y
};

struct WeightDev {
  MemberDev m[kMaxMembers];
  int32_t n_members;
  int32_t K;
  int32_t Kb;          // ceil(K/128)
  int32_t scale_bf16;  // 1: BF16 scales, 0: F32 scales
  // Scale of (128-row block r, 128-wide K block kb) is s[r * s_rs + kb * s_cs]:
  // (Kb, 1) for a block grid, (0, 0) for a per-tensor scale (the degenerate
  // block that covers the whole tensor).
  int32_t s_rs;
  int32_t s_cs;
};

// Per-launch tile table: member i owns tiles [tile0[i], tile0[i+1]).
struct TileMap {
  int32_t tile0[kMaxMembers + 1];
  int32_t n_tiles[kMaxMembers];  // row tiles of member i
};

void set_error(const char* fmt, ...);
bsf8_status device_status(hipError_t e, const char* what);

// Kernel launchers (one per .hip translation unit).
// Activation scales: element (m, kb) at xs[m * xs_sm + kb * xs_sk] (token-major
// or K-major, checked by the host layer).
bsf8_status launch_quant_act(const void* x, bool x_bf16, int64_t M, int64_t K, int64_t ldx,
                             uint8_t* xq, int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, hipStream_t stream);

bsf8_status launch_quant_glu(const void* y, bool y_bf16, int64_t M, int64_t F, int64_t ldy, uint8_t* xq,
                             int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, hipStream_t stream);
bsf8_status launch_glu_act(const void* y, bool y_bf16, int64_t M, int64_t F, int64_t ldy, float* h, int64_t ldh,
                           hipStream_t stream);

size_t w8a16_workspace_bytes(const WeightDev& w, int64_t M);
bsf8_status launch_w8a16(const WeightDev& w, bool aligned, const void* x, bool x_bf16, int64_t M,
                         int64_t ldx, void* y, bool y_bf16, int64_t ldy, void* ws, size_t ws_bytes,
                         hipStream_t stream);
std::string describe_w8a16(const WeightDev& w, bool aligned, int64_t M);

size_t w8a8_workspace_bytes(const WeightDev& w, int64_t M);
bsf8_status launch_w8a8(const WeightDev& w, bool aligned, const uint8_t* xq, int64_t ldq, const float* xs,
                        int64_t xs_sm, int64_t xs_sk, int64_t M, void* y, bool y_bf16, int64_t ldy, void* ws,
                        size_t ws_bytes, hipStream_t stream);
std::string describe_w8a8(const WeightDev& w, bool aligned, int64_t M);
// The W8A8 arm at one to 48 tokens runs the W8A16 file's streaming kernels
// with E4M3 activations (no workspace).
bool w8a8_stream_applies(const WeightDev& w, bool aligned, int64_t M, int64_t ldq);
std::string describe_w8a8_stream(const WeightDev& w, int64_t M);
bsf8_status launch_w8a8_stream(const WeightDev& w, const uint8_t* xq, int64_t ldq, const float* xs, int64_t xs_sm,
                               int64_t xs_sk, int64_t M, void* y, bool y_bf16, int64_t ldy, hipStream_t stream);
// The one-token kernels quantizing F32 or BF16 activations themselves (the
// W8A8 arm with the activation quantization in the same call; ldx_bytes is the
// activations' row pitch in bytes).
bool w8a8_dyn_stream_applies(const WeightDev& w, bool aligned, int64_t M, int64_t ldx_bytes);
std::string describe_w8a8_dyn_stream(const WeightDev& w, int64_t M);
bsf8_status launch_w8a8_dyn_stream(const WeightDev& w, const void* x, bool x_bf16, int64_t M, int64_t ldx, void* y,
                                   bool y_bf16, int64_t ldy, hipStream_t stream);
// Device address of this device's copy of the no-allocation scratch array
// (BSF8_NOALLOC_SCRATCH_BYTES bytes), looked up once per device.
bsf8_status w8a8_noalloc_scratch(void** ptr);

// Dense arm: the upcast copy and the BF16 GEMM over it (the fast W8A8 kernel's
// dense instance).
bsf8_status launch_upcast(const WeightDev& w, int64_t n_total, bool vec, void* out, bool out_bf16, int64_t ldo,
                          hipStream_t stream);
bool dense_supported(int64_t N, int64_t K, int64_t M, int64_t ldx);
size_t dense_workspace_bytes(int64_t N, int64_t K, int64_t M);
std::string describe_dense(int64_t N, int64_t K, int64_t M);
bsf8_status launch_dense(const uint16_t* wd, int64_t N, int64_t K, const uint16_t* x, int64_t M, int64_t ldx,
                         void* y, bool y_bf16, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream);

bsf8_status launch_read_stream(const void* p, int64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace bsf8

// The opaque handle of the ABI.
struct bsf8_weight {
  bsf8::WeightDev dev;
  int64_t n_total;
  int64_t rows[bsf8::kMaxMembers];
  int64_t col0[bsf8::kMaxMembers];
  int64_t srow0[bsf8::kMaxMembers];  // B_i: origin of member i in the stacked grids
  bool aligned16;                    // K % 16 == 0 and every weight pointer 16-byte aligned
  bool per_tensor;                   // one scale per member (per-tensor layout) instead of a block grid
};

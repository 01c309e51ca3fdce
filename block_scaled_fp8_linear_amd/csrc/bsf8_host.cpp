// Host side of libbsf8: status names, the header-only validator, weight handles,
// argument checks and dispatch to the kernel launchers.  No device memory is
// touched here except through the launchers.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "bsf8_internal.h"

namespace bsf8 {

static thread_local std::string g_last_error;
static thread_local std::string g_describe;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

bsf8_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSF8_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return BSF8_E_DEVICE;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static bsf8_status fail(bsf8_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(bsf8_status_name(s)) + ": " + buf;
  return s;
}

// The member's scale leaf: the block grid, or the per-tensor weight_scale.
static const bsf8_tensor_desc* scale_leaf(const bsf8_member_desc& m) { return m.scale_inv ? m.scale_inv : m.scale; }

static bool shape_is(const bsf8_tensor_desc* t, int64_t a, int64_t b) {
  return t->rank == 2 && t->shape[0] == a && t->shape[1] == b;
}

// Header-only validation.  The order of the checks is the precedence the ABI
// documents, so every bad input has exactly one status.
static bsf8_status validate_impl(const bsf8_decl* decl, const bsf8_member_desc* members, int32_t n) {
  if (decl == nullptr || (members == nullptr && n > 0)) return fail(BSF8_E_INVALID_ARG, "null descriptor");
  if (n < 1 || n > kMaxMembers) return fail(BSF8_E_GROUP, "%d members (1..%d allowed)", n, kMaxMembers);
  const bool per_tensor = decl->quant_method_fp8 && decl->block_n == 0 && decl->block_k == 0;
  if (!decl->quant_method_fp8 || (!per_tensor && (decl->block_n != kBlock || decl->block_k != kBlock)))
    return fail(BSF8_E_DECL,
                "declaration is not quant_method fp8 with weight_block_size [128,128] or per-tensor (got fp8=%d, [%d,%d])",
                decl->quant_method_fp8, decl->block_n, decl->block_k);
  for (int i = 0; i < n; ++i) {
    const bsf8_member_desc& m = members[i];
    const bsf8_tensor_desc& w = m.weight;
    if (w.rank < 0 || w.rank > 4) return fail(BSF8_E_INVALID_ARG, "member %d: weight rank %d", i, w.rank);
    if (w.dtype == BSF8_DT_F8_E5M2) return fail(BSF8_E_WEIGHT_E5M2, "member %d: E5M2 weight", i);
    if (w.dtype != BSF8_DT_F8_E4M3) return fail(BSF8_E_WEIGHT_DTYPE, "member %d: weight dtype %d is not F8_E4M3", i, w.dtype);
    if (w.rank != 2) return fail(BSF8_E_WEIGHT_RANK, "member %d: weight rank %d", i, w.rank);
    if (w.shape[0] <= 0 || w.shape[1] <= 0)
      return fail(BSF8_E_WEIGHT_EMPTY, "member %d: weight shape [%lld,%lld]", i, (long long)w.shape[0], (long long)w.shape[1]);
    if (m.scale_inv == nullptr && m.scale == nullptr) return fail(BSF8_E_SCALE_MISSING, "member %d: FP8 weight without a scale", i);
    if (m.scale_inv != nullptr && m.scale != nullptr)
      return fail(BSF8_E_SCALE_AMBIGUOUS, "member %d: both a block grid and a row/tensor scale", i);
    const bsf8_tensor_desc* leaf = m.scale_inv ? m.scale_inv : m.scale;
    if (leaf->rank < 0 || leaf->rank > 4) return fail(BSF8_E_INVALID_ARG, "member %d: scale rank %d", i, leaf->rank);
    if (per_tensor) {
      // one weight_scale value for the whole tensor (rank 0, or rank 1 of one element)
      if (m.scale_inv != nullptr)
        return fail(BSF8_E_DECL, "member %d: a weight_scale_inv grid under a per-tensor declaration", i);
      if (leaf->rank == 1 && leaf->shape[0] != 1) return fail(BSF8_E_SCALE_ROWWISE, "member %d: rank-1 (row-wise) scale", i);
      if (leaf->rank > 1) return fail(BSF8_E_SCALE_RANK, "member %d: per-tensor scale of rank %d", i, leaf->rank);
      if (leaf->dtype != BSF8_DT_BF16 && leaf->dtype != BSF8_DT_F32)
        return fail(BSF8_E_SCALE_DTYPE, "member %d: scale dtype %d is not BF16/F32", i, leaf->dtype);
      continue;
    }
    if (leaf->rank == 1) return fail(BSF8_E_SCALE_ROWWISE, "member %d: rank-1 (row-wise) scale", i);
    if (leaf->rank == 0 && m.scale != nullptr) return fail(BSF8_E_SCALE_PER_TENSOR, "member %d: per-tensor scale", i);
    if (leaf->rank != 2) return fail(BSF8_E_SCALE_RANK, "member %d: scale rank %d", i, leaf->rank);
    if (leaf->dtype != BSF8_DT_BF16 && leaf->dtype != BSF8_DT_F32)
      return fail(BSF8_E_SCALE_DTYPE, "member %d: scale dtype %d is not BF16/F32", i, leaf->dtype);
    const int64_t nb = ceil_div(w.shape[0], kBlock), kb = ceil_div(w.shape[1], kBlock);
    if (!shape_is(leaf, nb, kb) && shape_is(leaf, kb, nb))
      return fail(BSF8_E_SCALE_TRANSPOSED, "member %d: grid [%lld,%lld] is the transpose of [%lld,%lld]", i,
                  (long long)leaf->shape[0], (long long)leaf->shape[1], (long long)nb, (long long)kb);
    if (!shape_is(leaf, nb, kb))
      return fail(BSF8_E_SCALE_GRID, "member %d: grid [%lld,%lld] != [%lld,%lld]", i, (long long)leaf->shape[0],
                  (long long)leaf->shape[1], (long long)nb, (long long)kb);
    if (m.scale != nullptr)
      return fail(BSF8_E_SCALE_GRID, "member %d: a block-shaped weight_scale leaf is not a weight_scale_inv grid", i);
  }
  const int64_t k0 = members[0].weight.shape[1];
  const int32_t dt0 = scale_leaf(members[0])->dtype;
  for (int i = 1; i < n; ++i) {
    if (members[i].weight.shape[1] != k0) return fail(BSF8_E_GROUP, "member %d: K differs from member 0", i);
    if (scale_leaf(members[i])->dtype != dt0) return fail(BSF8_E_GROUP, "member %d: scale dtype differs from member 0", i);
  }
  for (int i = 0; i < n; ++i) {
    const uintptr_t wa = reinterpret_cast<uintptr_t>(members[i].weight.data);
    if (wa % 16 != 0) return fail(BSF8_E_ALIGNMENT, "member %d: weight address not 16-byte aligned", i);
    const uintptr_t sa = reinterpret_cast<uintptr_t>(scale_leaf(members[i])->data);
    const uintptr_t esz = scale_leaf(members[i])->dtype == BSF8_DT_BF16 ? 2 : 4;
    if (sa % esz != 0) return fail(BSF8_E_ALIGNMENT, "member %d: scale address not element aligned", i);
  }
  return BSF8_OK;
}

static bool dtype_ok(int32_t dt, bool f32, bool bf16) {
  return (f32 && dt == BSF8_DT_F32) || (bf16 && dt == BSF8_DT_BF16);
}

}  // namespace bsf8

using namespace bsf8;

extern "C" {

int32_t bsf8_abi_version(void) { return BSF8_ABI_VERSION; }

const char* bsf8_status_name(bsf8_status s) {
  switch (s) {
    case BSF8_OK: return "OK";
    case BSF8_E_INVALID_ARG: return "INVALID_ARG";
    case BSF8_E_GROUP: return "GROUP";
    case BSF8_E_DECL: return "DECL";
    case BSF8_E_WEIGHT_E5M2: return "WEIGHT_E5M2";
    case BSF8_E_WEIGHT_DTYPE: return "WEIGHT_DTYPE";
    case BSF8_E_WEIGHT_RANK: return "WEIGHT_RANK";
    case BSF8_E_WEIGHT_EMPTY: return "WEIGHT_EMPTY";
    case BSF8_E_SCALE_MISSING: return "SCALE_MISSING";
    case BSF8_E_SCALE_AMBIGUOUS: return "SCALE_AMBIGUOUS";
    case BSF8_E_SCALE_ROWWISE: return "SCALE_ROWWISE";
    case BSF8_E_SCALE_PER_TENSOR: return "SCALE_PER_TENSOR";
    case BSF8_E_SCALE_RANK: return "SCALE_RANK";
    case BSF8_E_SCALE_DTYPE: return "SCALE_DTYPE";
    case BSF8_E_SCALE_TRANSPOSED: return "SCALE_TRANSPOSED";
    case BSF8_E_SCALE_GRID: return "SCALE_GRID";
    case BSF8_E_ALIGNMENT: return "ALIGNMENT";
    case BSF8_E_UNSUPPORTED: return "UNSUPPORTED";
    case BSF8_E_WORKSPACE: return "WORKSPACE";
    case BSF8_E_DEVICE: return "DEVICE";
  }
  return "UNKNOWN";
}

const char* bsf8_last_error(void) { return g_last_error.c_str(); }

bsf8_status bsf8_validate(const bsf8_decl* decl, const bsf8_member_desc* members, int32_t n_members) {
  return validate_impl(decl, members, n_members);
}

bsf8_status bsf8_weight_create(const bsf8_decl* decl, const bsf8_member_desc* members, int32_t n_members,
                               bsf8_weight** out) {
  if (out == nullptr) return fail(BSF8_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  bsf8_status st = validate_impl(decl, members, n_members);
  if (st != BSF8_OK) return st;
  const int64_t K = members[0].weight.shape[1];
  int64_t total = 0;
  for (int i = 0; i < n_members; ++i) {
    if (members[i].weight.data == nullptr || scale_leaf(members[i])->data == nullptr)
      return fail(BSF8_E_INVALID_ARG, "member %d: a handle needs device addresses", i);
    total += members[i].weight.shape[0];
  }
  if (K > INT32_MAX / 2 || total > INT32_MAX / 2)
    return fail(BSF8_E_UNSUPPORTED, "N or K beyond 2^30");
  bsf8_weight* h = new bsf8_weight();
  std::memset(&h->dev, 0, sizeof(h->dev));
  h->dev.n_members = n_members;
  h->dev.K = static_cast<int32_t>(K);
  h->dev.Kb = static_cast<int32_t>(ceil_div(K, kBlock));
  h->dev.scale_bf16 = scale_leaf(members[0])->dtype == BSF8_DT_BF16 ? 1 : 0;
  h->per_tensor = members[0].scale_inv == nullptr;
  h->dev.s_rs = h->per_tensor ? 0 : h->dev.Kb;
  h->dev.s_cs = h->per_tensor ? 0 : 1;
  h->aligned16 = (K % 16) == 0;
  int64_t col = 0, srow = 0;
  for (int i = 0; i < n_members; ++i) {
    const int64_t rows = members[i].weight.shape[0];
    h->dev.m[i].w = static_cast<const uint8_t*>(members[i].weight.data);
    h->dev.m[i].s = scale_leaf(members[i])->data;
    h->dev.m[i].rows = static_cast<int32_t>(rows);
    h->dev.m[i].col0 = static_cast<int32_t>(col);
    h->rows[i] = rows;
    h->col0[i] = col;
    h->srow0[i] = srow;
    col += rows;
    srow += h->per_tensor ? 1 : ceil_div(rows, kBlock);
  }
  h->n_total = total;
  *out = h;
  return BSF8_OK;
}

void bsf8_weight_destroy(bsf8_weight* w) { delete w; }

bsf8_status bsf8_weight_geometry(const bsf8_weight* w, int64_t* n_total, int64_t* k, int32_t* n_members) {
  if (w == nullptr) return fail(BSF8_E_INVALID_ARG, "null handle");
  if (n_total) *n_total = w->n_total;
  if (k) *k = w->dev.K;
  if (n_members) *n_members = w->dev.n_members;
  return BSF8_OK;
}

bsf8_status bsf8_weight_scale_row(const bsf8_weight* w, int64_t n, int32_t* member, int64_t* local_row,
                                  int64_t* stacked_row) {
  if (w == nullptr) return fail(BSF8_E_INVALID_ARG, "null handle");
  if (n < 0 || n >= w->n_total) return fail(BSF8_E_INVALID_ARG, "row %lld outside [0,%lld)", (long long)n, (long long)w->n_total);
  for (int i = w->dev.n_members - 1; i >= 0; --i) {
    if (n >= w->col0[i]) {
      const int64_t r = w->per_tensor ? 0 : (n - w->col0[i]) / kBlock;
      if (member) *member = i;
      if (local_row) *local_row = r;
      if (stacked_row) *stacked_row = w->srow0[i] + r;
      return BSF8_OK;
    }
  }
  return fail(BSF8_E_INVALID_ARG, "row not found");
}

// The two accepted activation scale layouts: token-major (xs_sk == 1, rows of
// at least Kb) and K-major (xs_sm == 1, rows of at least M).
static bool scale_layout_ok(int64_t M, int64_t Kb, int64_t xs_sm, int64_t xs_sk) {
  return (xs_sk == 1 && xs_sm >= Kb) || (xs_sm == 1 && xs_sk >= M);
}

bsf8_status bsf8_quant_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                           int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, void* stream) {
  if (M < 0 || K < 0) return fail(BSF8_E_INVALID_ARG, "negative size");
  if (!dtype_ok(x_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "x dtype %d (F32 or BF16)", x_dtype);
  if (M == 0 || K == 0) return BSF8_OK;
  if (x == nullptr || xq == nullptr || xs == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (ldx < K || ldq < K) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  if (!scale_layout_ok(M, ceil_div(K, kBlock), xs_sm, xs_sk))
    return fail(BSF8_E_INVALID_ARG, "xs strides (%lld, %lld): neither token-major nor K-major", (long long)xs_sm,
                (long long)xs_sk);
  if (M > INT32_MAX || K > INT32_MAX / 2) return fail(BSF8_E_UNSUPPORTED, "M or K too large");
  const size_t esz = x_dtype == BSF8_DT_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(x) % esz || reinterpret_cast<uintptr_t>(xs) % 4)
    return fail(BSF8_E_ALIGNMENT, "x or xs not element aligned");
  return launch_quant_act(x, x_dtype == BSF8_DT_BF16, M, K, ldx, xq, ldq, xs, xs_sm, xs_sk,
                          static_cast<hipStream_t>(stream));
}

bsf8_status bsf8_quant_glu(const void* y, int32_t y_dtype, int64_t M, int64_t F, int64_t ldy, uint8_t* xq,
                           int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, void* stream) {
  if (M < 0 || F < 0) return fail(BSF8_E_INVALID_ARG, "negative size");
  if (!dtype_ok(y_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "y dtype %d (F32 or BF16)", y_dtype);
  if (M == 0 || F == 0) return BSF8_OK;
  if (y == nullptr || xq == nullptr || xs == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (ldy < 2 * F || ldq < F) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  if (!scale_layout_ok(M, ceil_div(F, kBlock), xs_sm, xs_sk))
    return fail(BSF8_E_INVALID_ARG, "xs strides (%lld, %lld): neither token-major nor K-major", (long long)xs_sm,
                (long long)xs_sk);
  if (M > INT32_MAX || F > INT32_MAX / 4) return fail(BSF8_E_UNSUPPORTED, "M or F too large");
  const size_t esz = y_dtype == BSF8_DT_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(y) % esz || reinterpret_cast<uintptr_t>(xs) % 4)
    return fail(BSF8_E_ALIGNMENT, "y or xs not element aligned");
  return launch_quant_glu(y, y_dtype == BSF8_DT_BF16, M, F, ldy, xq, ldq, xs, xs_sm, xs_sk,
                          static_cast<hipStream_t>(stream));
}

bsf8_status bsf8_glu_act(const void* y, int32_t y_dtype, int64_t M, int64_t F, int64_t ldy, float* h, int64_t ldh,
                         void* stream) {
  if (M < 0 || F < 0) return fail(BSF8_E_INVALID_ARG, "negative size");
  if (!dtype_ok(y_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "y dtype %d (F32 or BF16)", y_dtype);
  if (M == 0 || F == 0) return BSF8_OK;
  if (y == nullptr || h == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (ldy < 2 * F || ldh < F) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  if (M > INT32_MAX || F > INT32_MAX / 4) return fail(BSF8_E_UNSUPPORTED, "M or F too large");
  const size_t esz = y_dtype == BSF8_DT_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(y) % esz || reinterpret_cast<uintptr_t>(h) % 4)
    return fail(BSF8_E_ALIGNMENT, "y or h not element aligned");
  return launch_glu_act(y, y_dtype == BSF8_DT_BF16, M, F, ldy, h, ldh, static_cast<hipStream_t>(stream));
}

// Workspace of the two-step form of bsf8_linear_w8a8_dynamic: the codes (row
// pitch K rounded up to 16 bytes), the K-major scales, then the W8A8 call's own
// workspace, each from a 256-byte boundary.
struct DynLayout {
  int64_t ldq;
  size_t xs_off, gemm_off, gemm_bytes, total;
};
static size_t round256(size_t n) { return (n + 255) & ~size_t(255); }
static DynLayout dyn_layout(const WeightDev& d, int64_t M) {
  DynLayout L{};
  L.ldq = (int64_t(d.K) + 15) & ~int64_t(15);
  L.xs_off = round256(size_t(M) * size_t(L.ldq));
  L.gemm_off = L.xs_off + round256(size_t(M) * size_t(d.Kb) * sizeof(float));
  L.gemm_bytes = w8a8_workspace_bytes(d, M);
  L.total = L.gemm_off + L.gemm_bytes;
  return L;
}

bsf8_status bsf8_workspace_size(const bsf8_weight* w, int32_t arm, int64_t M, size_t* bytes) {
  if (w == nullptr || bytes == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (M < 0) return fail(BSF8_E_INVALID_ARG, "negative M");
  if (arm == BSF8_ARM_W8A16) *bytes = M ? w8a16_workspace_bytes(w->dev, M) : 0;
  else if (arm == BSF8_ARM_W8A8) *bytes = M ? w8a8_workspace_bytes(w->dev, M) : 0;
  else if (arm == BSF8_ARM_DENSE) *bytes = M ? dense_workspace_bytes(w->n_total, w->dev.K, M) : 0;
  else if (arm == BSF8_ARM_W8A8_DYNAMIC) *bytes = M ? dyn_layout(w->dev, M).total : 0;
  else return fail(BSF8_E_INVALID_ARG, "arm %d", arm);
  return BSF8_OK;
}

bsf8_status bsf8_upcast(const bsf8_weight* w, void* out, int32_t out_dtype, int64_t ldo, void* stream) {
  if (w == nullptr || out == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (!dtype_ok(out_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "out dtype %d (F32 or BF16)", out_dtype);
  if (ldo < w->dev.K) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  const size_t esz = out_dtype == BSF8_DT_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(out) % esz) return fail(BSF8_E_ALIGNMENT, "out not element aligned");
  const bool vec = w->aligned16 && reinterpret_cast<uintptr_t>(out) % 16 == 0 && (ldo * int64_t(esz)) % 16 == 0;
  return launch_upcast(w->dev, w->n_total, vec, out, out_dtype == BSF8_DT_BF16, ldo, static_cast<hipStream_t>(stream));
}

bsf8_status bsf8_dense_workspace_size(int64_t N, int64_t K, int64_t M, size_t* bytes) {
  if (bytes == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (N <= 0 || K <= 0 || M < 0) return fail(BSF8_E_INVALID_ARG, "sizes N=%lld K=%lld M=%lld", (long long)N,
                                             (long long)K, (long long)M);
  *bytes = dense_workspace_bytes(N, K, M);
  return BSF8_OK;
}

bsf8_status bsf8_linear_dense(const uint16_t* wd, int64_t N, int64_t K, const uint16_t* x, int64_t M, int64_t ldx,
                              void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (N <= 0 || K <= 0 || M < 0) return fail(BSF8_E_INVALID_ARG, "sizes N=%lld K=%lld M=%lld", (long long)N,
                                             (long long)K, (long long)M);
  if (!dtype_ok(y_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "y dtype %d (F32 or BF16)", y_dtype);
  if (M == 0) return BSF8_OK;
  if (wd == nullptr || x == nullptr || y == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (ldx < K || ldy < N) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  const size_t ye = y_dtype == BSF8_DT_F32 ? 4 : 2;
  if (K % 8 || ldx % 8 || reinterpret_cast<uintptr_t>(wd) % 16 || reinterpret_cast<uintptr_t>(x) % 16)
    return fail(BSF8_E_ALIGNMENT, "dense GEMM needs K and ldx multiples of 8 and 16-byte aligned wd and x");
  if (reinterpret_cast<uintptr_t>(y) % ye) return fail(BSF8_E_ALIGNMENT, "y not element aligned");
  if (!dense_supported(N, K, M, ldx))
    return fail(BSF8_E_UNSUPPORTED, "dense GEMM shape N=%lld K=%lld M=%lld ldx=%lld (K <= 65536 and operands "
                "below 2 GiB)", (long long)N, (long long)K, (long long)M, (long long)ldx);
  const size_t need = dense_workspace_bytes(N, K, M);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(BSF8_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (workspace != nullptr && reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(BSF8_E_ALIGNMENT, "workspace not 256-byte aligned");
  return launch_dense(wd, N, K, x, M, ldx, y, y_dtype == BSF8_DT_BF16, ldy, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream));
}

bsf8_status bsf8_linear_w8a16(const bsf8_weight* w, const void* x, int32_t x_dtype, int64_t M, int64_t ldx,
                              void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (w == nullptr) return fail(BSF8_E_INVALID_ARG, "null handle");
  if (M < 0) return fail(BSF8_E_INVALID_ARG, "negative M");
  if (!dtype_ok(x_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "x dtype %d (F32 or BF16)", x_dtype);
  if (!dtype_ok(y_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "y dtype %d (F32 or BF16)", y_dtype);
  if (M == 0) return BSF8_OK;
  if (x == nullptr || y == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (ldx < w->dev.K || ldy < w->n_total) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  if (M > INT32_MAX / 2) return fail(BSF8_E_UNSUPPORTED, "M too large");
  const size_t xe = x_dtype == BSF8_DT_F32 ? 4 : 2, ye = y_dtype == BSF8_DT_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(x) % xe || reinterpret_cast<uintptr_t>(y) % ye)
    return fail(BSF8_E_ALIGNMENT, "x or y not element aligned");
  const size_t need = w8a16_workspace_bytes(w->dev, M);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(BSF8_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (workspace != nullptr && reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(BSF8_E_ALIGNMENT, "workspace not 256-byte aligned");
  const bool aligned = w->aligned16 && (reinterpret_cast<uintptr_t>(x) % 16 == 0) && ((ldx * xe) % 16 == 0);
  return launch_w8a16(w->dev, aligned, x, x_dtype == BSF8_DT_BF16, M, ldx, y, y_dtype == BSF8_DT_BF16, ldy,
                      workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

bsf8_status bsf8_linear_w8a8(const bsf8_weight* w, const uint8_t* xq, int64_t ldq, const float* xs, int64_t xs_sm,
                             int64_t xs_sk,
                             int64_t M, void* y, int32_t y_dtype, int64_t ldy, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (w == nullptr) return fail(BSF8_E_INVALID_ARG, "null handle");
  if (M < 0) return fail(BSF8_E_INVALID_ARG, "negative M");
  if (!dtype_ok(y_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "y dtype %d (F32 or BF16)", y_dtype);
  if (M == 0) return BSF8_OK;
  if (xq == nullptr || xs == nullptr || y == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (ldq < w->dev.K || ldy < w->n_total) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  if (!scale_layout_ok(M, w->dev.Kb, xs_sm, xs_sk))
    return fail(BSF8_E_INVALID_ARG, "xs strides (%lld, %lld): neither token-major nor K-major", (long long)xs_sm,
                (long long)xs_sk);
  if (M > INT32_MAX / 2) return fail(BSF8_E_UNSUPPORTED, "M too large");
  const size_t ye = y_dtype == BSF8_DT_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(xs) % 4 || reinterpret_cast<uintptr_t>(y) % ye)
    return fail(BSF8_E_ALIGNMENT, "xs or y not element aligned");
  const size_t need = w8a8_workspace_bytes(w->dev, M);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(BSF8_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (workspace != nullptr && reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(BSF8_E_ALIGNMENT, "workspace not 256-byte aligned");
  const bool aligned = w->aligned16 && (reinterpret_cast<uintptr_t>(xq) % 16 == 0) && (ldq % 16 == 0);
  return launch_w8a8(w->dev, aligned, xq, ldq, xs, xs_sm, xs_sk, M, y, y_dtype == BSF8_DT_BF16, ldy, workspace,
                     workspace_bytes, static_cast<hipStream_t>(stream));
}

bsf8_status bsf8_linear_w8a8_dynamic(const bsf8_weight* w, const void* x, int32_t x_dtype, int64_t M, int64_t ldx,
                                     void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (w == nullptr) return fail(BSF8_E_INVALID_ARG, "null handle");
  if (M < 0) return fail(BSF8_E_INVALID_ARG, "negative M");
  if (!dtype_ok(x_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "x dtype %d (F32 or BF16)", x_dtype);
  if (!dtype_ok(y_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "y dtype %d (F32 or BF16)", y_dtype);
  if (M == 0) return BSF8_OK;
  if (x == nullptr || y == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (ldx < w->dev.K || ldy < w->n_total) return fail(BSF8_E_INVALID_ARG, "leading dimension too small");
  if (M > INT32_MAX / 2) return fail(BSF8_E_UNSUPPORTED, "M too large");
  const size_t xe = x_dtype == BSF8_DT_F32 ? 4 : 2, ye = y_dtype == BSF8_DT_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(x) % xe || reinterpret_cast<uintptr_t>(y) % ye)
    return fail(BSF8_E_ALIGNMENT, "x or y not element aligned");
  const bool x_bf16 = x_dtype == BSF8_DT_BF16, y_bf16 = y_dtype == BSF8_DT_BF16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool aligned = w->aligned16 && (reinterpret_cast<uintptr_t>(x) % 16 == 0) && ((ldx * int64_t(xe)) % 16 == 0);
  if (w8a8_dyn_stream_applies(w->dev, aligned, M, ldx * int64_t(xe)))
    return launch_w8a8_dyn_stream(w->dev, x, x_bf16, M, ldx, y, y_bf16, ldy, st);
  // two steps: the quantizer into the workspace, then the W8A8 kernels
  const DynLayout L = dyn_layout(w->dev, M);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(BSF8_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace ? workspace_bytes : 0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(BSF8_E_ALIGNMENT, "workspace not 256-byte aligned");
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint8_t* xq = base;
  float* xs = reinterpret_cast<float*>(base + L.xs_off);
  const bsf8_status s1 = launch_quant_act(x, x_bf16, M, w->dev.K, ldx, xq, L.ldq, xs, 1, M, st);
  if (s1 != BSF8_OK) return s1;
  return launch_w8a8(w->dev, w->aligned16, xq, L.ldq, xs, 1, M, M, y, y_bf16, ldy,
                     L.gemm_bytes ? base + L.gemm_off : nullptr, L.gemm_bytes, st);
}

bsf8_status bsf8_linear_w8a8_noalloc(const bsf8_weight* w, const uint8_t* xq, int64_t ldq, const float* xs,
                                     int64_t xs_sm, int64_t xs_sk, int64_t M, void* y, int32_t y_dtype, int64_t ldy,
                                     void* stream) {
  if (w == nullptr) return fail(BSF8_E_INVALID_ARG, "null handle");
  if (M < 0) return fail(BSF8_E_INVALID_ARG, "negative M");
  if (!dtype_ok(y_dtype, true, true)) return fail(BSF8_E_INVALID_ARG, "y dtype %d (F32 or BF16)", y_dtype);
  if (M == 0) return BSF8_OK;
  const size_t need = w8a8_workspace_bytes(w->dev, M);
  if (need > size_t(BSF8_NOALLOC_SCRATCH_BYTES))
    return fail(BSF8_E_WORKSPACE,
                "this call needs %zu bytes of split-K partials; the no-allocation entry point holds %zu "
                "(BSF8_NOALLOC_SCRATCH_BYTES): call bsf8_linear_w8a8 with a workspace instead",
                need, size_t(BSF8_NOALLOC_SCRATCH_BYTES));
  void* scratch = nullptr;
  const bsf8_status st = w8a8_noalloc_scratch(&scratch);
  if (st != BSF8_OK) return st;
  return bsf8_linear_w8a8(w, xq, ldq, xs, xs_sm, xs_sk, M, y, y_dtype, ldy, scratch,
                          size_t(BSF8_NOALLOC_SCRATCH_BYTES), stream);
}

bsf8_status bsf8_read_stream(const void* p, int64_t bytes, uint32_t* sink, void* stream) {
  if (p == nullptr || sink == nullptr) return fail(BSF8_E_INVALID_ARG, "null pointer");
  if (bytes < 0) return fail(BSF8_E_INVALID_ARG, "negative size");
  if (reinterpret_cast<uintptr_t>(p) % 16 || bytes % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
    return fail(BSF8_E_ALIGNMENT, "read_stream needs a 16-byte aligned pointer and size");
  if (bytes == 0) return BSF8_OK;
  return launch_read_stream(p, bytes, sink, static_cast<hipStream_t>(stream));
}

const char* bsf8_describe(const bsf8_weight* w, int32_t arm, int64_t M) {
  if (w == nullptr) return nullptr;
  char geo[256];
  snprintf(geo, sizeof(geo), " | weight N=%lld K=%d members=%d scales=%s%s", (long long)w->n_total, w->dev.K,
           w->dev.n_members, w->dev.scale_bf16 ? "bf16" : "f32", w->per_tensor ? " per-tensor" : "");
  if (arm == BSF8_ARM_W8A16) g_describe = describe_w8a16(w->dev, w->aligned16, M) + geo;
  else if (arm == BSF8_ARM_W8A8) g_describe = describe_w8a8(w->dev, w->aligned16, M) + geo;
  else if (arm == BSF8_ARM_DENSE) g_describe = describe_dense(w->n_total, w->dev.K, M) + geo;
  else if (arm == BSF8_ARM_W8A8_DYNAMIC)
    g_describe = (w8a8_dyn_stream_applies(w->dev, w->aligned16, M > 0 ? M : 1, int64_t(w->dev.K) * 4)
                      ? describe_w8a8_dyn_stream(w->dev, M > 0 ? M : 1)
                      : "quant_act into the workspace (K-major scales), then " + describe_w8a8(w->dev, w->aligned16, M)) +
                  geo;
  else g_describe = "unknown arm";
  return g_describe.c_str();
}

}  // extern "C"

/*
 * bsf8.h -- C ABI of libbsf8: the block-scaled FP8 linear projection Y = X . W^T
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (sources cited by page title and section):
 *   - Weights are E4M3 bytes of shape [N,K] (row n = output feature, K contiguous),
 *     kept exactly as the checkpoint stores them, with one scale per 128x128 block
 *     on a ceil-divided grid [ceil(N/128), ceil(K/128)].  The scale multiplies the
 *     decoded value; it is not a reciprocal.  BF16 scales widen exactly to F32.
 *     ("Qwen checkpoints with block FP8 weights", layout and operator paragraphs;
 *      "th#1803 ... hf.fp8-blockwise@1", section "What lands".)
 *   - W8A16/F32 arm: F32 activations and F32 accumulation, the block multiplier
 *     applied inside the reduction, neither operand requantized.
 *     ("Qwen checkpoints with block FP8 weights", block-path paragraph.)
 *   - W8A8 arm: activations quantized per token in 1x128 groups to E4M3 with an
 *     F32 scale each; FP8 x FP8 products accumulated in F32; every 128-wide K
 *     slice rescaled by activation scale x weight scale in an F32 epilogue.
 *     ("Module w8a8_prefill", section "WHY (#917 / #928)".)
 *   - Grouped tensors (fused QKV, gate/up) keep each member's own block-row
 *     origin; the output concatenates the members along N.
 *     ("Qwen checkpoints with block FP8 weights", operator paragraph.)
 *
 * Conventions for every call:
 *   - Pointers named x, xq, xs, y, workspace and the tensor descriptors' data are
 *     DEVICE addresses on the current HIP device.  Descriptors themselves live
 *     in host memory and are read during the call only.
 *   - The caller owns all memory.  A weight handle BORROWS the weight and scale
 *     device pointers it was created from; they must stay valid and unchanged
 *     until bsf8_weight_destroy.  The library never copies, repacks, rescales or
 *     quantizes weights on its own; bsf8_upcast writes a dense copy into caller
 *     memory when asked.
 *   - No call allocates device memory, frees it or synchronizes the device.
 *     Compute calls are asynchronous and ordered on the given stream
 *     (a hipStream_t passed as void*; NULL = the default stream).
 *   - Errors are returned as bsf8_status; nothing is thrown across the ABI.
 *     bsf8_last_error() gives a thread-local sentence for the last failure.
 *   - Element layouts are row-major with a leading dimension counted in
 *     elements (ldx, ldq, ldy), except the activation scales, which take two
 *     strides (see BSF8 activation scale layout below).
 *   - M == 0 is a successful no-op for every compute call.
 */
#ifndef BSF8_H
#define BSF8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSF8_ABI_VERSION 1
#define BSF8_MAX_MEMBERS 8

typedef enum bsf8_status {
  BSF8_OK = 0,
  BSF8_E_INVALID_ARG = 1,       /* null pointer, negative size, bad dtype/arm enum, ld too small */
  BSF8_E_GROUP = 2,             /* 0 or more than 8 members; members disagree on K or scale dtype */
  BSF8_E_DECL = 3,              /* declaration is not quant_method fp8 with weight_block_size [128,128] */
  BSF8_E_WEIGHT_E5M2 = 4,       /* E5M2 weight encoding */
  BSF8_E_WEIGHT_DTYPE = 5,      /* weight is not F8_E4M3 (e.g. a dense BF16 tree) */
  BSF8_E_WEIGHT_RANK = 6,       /* weight is not rank 2 */
  BSF8_E_WEIGHT_EMPTY = 7,      /* a weight dimension is zero */
  BSF8_E_SCALE_MISSING = 8,     /* FP8 weight with neither scale leaf */
  BSF8_E_SCALE_AMBIGUOUS = 9,   /* both a block grid and a row/tensor scale leaf */
  BSF8_E_SCALE_ROWWISE = 10,    /* a rank-1 scale (one scale per row) */
  BSF8_E_SCALE_PER_TENSOR = 11, /* a rank-0 weight_scale (per-tensor layout, not this format) */
  BSF8_E_SCALE_RANK = 12,       /* any other scale rank than 2 */
  BSF8_E_SCALE_DTYPE = 13,      /* scale grid is not BF16 or F32 */
  BSF8_E_SCALE_TRANSPOSED = 14, /* grid shaped [Kb,Nb] instead of [Nb,Kb] */
  BSF8_E_SCALE_GRID = 15,       /* any other grid shape (mis-blocked, floor-divided, ...) */
  BSF8_E_ALIGNMENT = 16,        /* weight address not 16-byte aligned, scale not element aligned,
                                   or an activation/output address or ld not aligned as a call needs */
  BSF8_E_UNSUPPORTED = 17,      /* a dtype combination this build does not implement */
  BSF8_E_WORKSPACE = 18,        /* workspace missing or smaller than bsf8_workspace_size reports */
  BSF8_E_DEVICE = 19            /* HIP error at launch; see bsf8_last_error() */
} bsf8_status;

typedef enum bsf8_dtype {
  BSF8_DT_INVALID = 0,
  BSF8_DT_F8_E4M3 = 1,
  BSF8_DT_F8_E5M2 = 2,
  BSF8_DT_BF16 = 3,
  BSF8_DT_F16 = 4,
  BSF8_DT_F32 = 5,
  BSF8_DT_U8 = 6,
  BSF8_DT_OTHER = 7
} bsf8_dtype;

typedef enum bsf8_arm {
  BSF8_ARM_W8A16 = 0,  /* F32 activations, F32 accumulation */
  BSF8_ARM_W8A8 = 1,   /* per-token 1x128 E4M3 activations, F32 epilogue */
  BSF8_ARM_DENSE = 2,  /* the handle's upcast dense BF16 copy times BF16 activations (bsf8_linear_dense);
                          for bsf8_workspace_size and bsf8_describe */
  BSF8_ARM_W8A8_DYNAMIC = 3  /* W8A8 on F32 or BF16 activations quantized in the same call
                                (bsf8_linear_w8a8_dynamic) */
} bsf8_arm;

/* Header-level description of one tensor.  data may be NULL for a header-only
 * check (bsf8_validate); bsf8_weight_create needs device addresses. */
typedef struct bsf8_tensor_desc {
  int32_t dtype;      /* bsf8_dtype */
  int32_t rank;       /* 0..4 */
  int64_t shape[4];   /* first `rank` entries used */
  const void* data;   /* device address or NULL */
} bsf8_tensor_desc;

/* One member of a (possibly grouped) weight.  scale_inv is the block-grid leaf
 * (weight_scale_inv); scale is the row-wise / per-tensor leaf (weight_scale)
 * that other FP8 layouts use.  Either may be NULL. */
typedef struct bsf8_member_desc {
  bsf8_tensor_desc weight;
  const bsf8_tensor_desc* scale_inv;
  const bsf8_tensor_desc* scale;
} bsf8_member_desc;

/* The checkpoint's quantization_config as declared.  block_n = block_k = 0
 * declares the per-tensor layout (no weight_block_size: one weight_scale per
 * tensor, read as the degenerate block that covers the whole tensor; "FP8
 * Native Serving", section "The two FP8 checkpoint shapes"). */
typedef struct bsf8_decl {
  int32_t quant_method_fp8;  /* nonzero when quant_method is "fp8" */
  int32_t block_n;           /* weight_block_size[0], or 0 for per-tensor */
  int32_t block_k;           /* weight_block_size[1], or 0 for per-tensor */
} bsf8_decl;

typedef struct bsf8_weight bsf8_weight;

/* ABI version of the loaded library (BSF8_ABI_VERSION it was built with). */
int32_t bsf8_abi_version(void);

/* Stable upper-case name of a status ("OK", "SCALE_TRANSPOSED", ...). Never NULL. */
const char* bsf8_status_name(bsf8_status s);

/* Thread-local sentence describing the last non-OK status of this thread. */
const char* bsf8_last_error(void);

/*
 * bsf8_validate -- geometry validation from headers alone, before any weight
 * byte is read or uploaded.
 * ("Qwen checkpoints with block FP8 weights", operator paragraph: E5M2,
 *  ambiguous row/block scales, malformed grids and incompatible declarations
 *  are refused before upload; "th#1803", sections "What lands" (headers only)
 *  and "Why the refusals matter more than the load" (row-wise trees,
 *  transposed or mis-blocked grids, FP8 without a scale, rank-1 scales,
 *  configs that disagree with the bytes are refused by name).)
 *
 * decl, members: host pointers; n_members in 1..8.  Reads no device memory.
 * Returns exactly one status; the precedence is
 *   GROUP (member count) > DECL > per member in index order
 *   [WEIGHT_E5M2 > WEIGHT_DTYPE > WEIGHT_RANK > WEIGHT_EMPTY > SCALE_MISSING >
 *    SCALE_AMBIGUOUS > SCALE_ROWWISE > SCALE_PER_TENSOR > SCALE_RANK >
 *    SCALE_DTYPE > SCALE_TRANSPOSED > SCALE_GRID]
 *   > GROUP (K or scale dtype differ across members) > ALIGNMENT (non-NULL data
 *   not 16-byte aligned for weights, not element aligned for scales).
 * A square grid (Nb == Kb) given transposed has the right shape and cannot be
 * detected from headers; it is accepted.
 * Under a per-tensor declaration (block 0 x 0) each member needs a scale
 * (weight_scale) leaf holding one BF16 or F32 value (rank 0, or rank 1 of
 * shape [1]); a scale_inv grid disagrees with the declaration (DECL), a
 * longer rank-1 leaf is SCALE_ROWWISE and a higher rank SCALE_RANK.  A rank-0
 * scale under the [128,128] declaration stays SCALE_PER_TENSOR.
 */
bsf8_status bsf8_validate(const bsf8_decl* decl, const bsf8_member_desc* members, int32_t n_members);

/*
 * bsf8_weight_create -- validate (as bsf8_validate) and build an immutable
 * handle over borrowed device pointers.  Every weight and scale data pointer
 * must be non-NULL.  Host-only: no device access.
 * Member i owns output rows [R_i, R_i + N_i) with R_i = sum_{j<i} N_j; its
 * scale grid is its own [ceil(N_i/128), ceil(K/128)] array (member-local
 * origin), or, per-tensor, its own single value used for every block.  On
 * failure *out is set to NULL.
 */
bsf8_status bsf8_weight_create(const bsf8_decl* decl, const bsf8_member_desc* members,
                               int32_t n_members, bsf8_weight** out);

/* Release a handle (host memory only).  NULL is ignored. */
void bsf8_weight_destroy(bsf8_weight* w);

/* Geometry of a handle: total output features N = sum N_i, K, member count. */
bsf8_status bsf8_weight_geometry(const bsf8_weight* w, int64_t* n_total, int64_t* k, int32_t* n_members);

/*
 * bsf8_weight_scale_row -- for output feature n in [0, N), the member index and
 * the row of that member's scale grid the kernels use: (n - R_i) / 128.
 * Also returns the row of the members' grids stacked in member order,
 * B_i + (n - R_i) / 128 with B_i = sum_{j<i} ceil(N_j/128).  For a
 * per-tensor weight the local row is 0 and the stacked row is i (one value
 * per member).  Host-only.
 */
bsf8_status bsf8_weight_scale_row(const bsf8_weight* w, int64_t n, int32_t* member,
                                  int64_t* local_row, int64_t* stacked_row);

/*
 * BSF8 activation scale layout.  The per-token group scales xs are a logical
 * [M, ceil(K/128)] F32 array whose element (m, kb) sits at
 * xs[m * xs_sm + kb * xs_sk] (strides in elements).  Two layouts are accepted:
 *   token-major: xs_sk == 1 and xs_sm >= ceil(K/128)  (row m = token m's scales,
 *                as the quantizer of "Module w8a8_prefill" writes them);
 *   K-major:     xs_sm == 1 and xs_sk >= M            (row kb = every token's
 *                scale of block kb, token index contiguous: the transposed
 *                copy that "Module w8a8_prefill", section "Reachability",
 *                makes for its cuBLASLt path).
 * (When M == 1 or ceil(K/128) == 1 either test may hold.)  Any other pair is
 * INVALID_ARG.  The W8A8 product reads a K block's 256 token scales at a time:
 * K-major makes that one contiguous kilobyte, token-major 256 separate words,
 * so K-major is the faster input; results are identical.
 */

/*
 * bsf8_quant_act -- per-token 1x128 group quantization of activations.
 * ("Module w8a8_prefill", section "WHY (#917 / #928)": per-token FP32 scales
 *  over 1x128 groups; "FP8 Native Serving", section "FP8 E4M3: range and
 *  quirks": E4M3 range +-448, no infinity.)
 *
 * x   : [M, K] with leading dimension ldx (elements), dtype F32 or BF16.
 * xq  : [M, K] E4M3 bytes out, leading dimension ldq (bytes).
 * xs  : [M, ceil(K/128)] F32 scales out, strides xs_sm, xs_sk (elements; the
 *       activation scale layout above).
 * For token m and group g (channels 128g .. min(128g+128, K) - 1):
 *   amax = max |x|;  s = amax' / 448 with amax' = max(amax, 1e-10f) (IEEE F32);
 *   q = round-to-nearest-even E4M3 of clamp(x / s, -448, 448) (IEEE F32
 *   division), sign of zero kept.  xs holds s, the dequantization multiplier.
 * Results are bit-exact: one byte pattern and one scale per input.
 * Non-finite inputs are outside the defined domain.
 * Errors: INVALID_ARG (null, negative, ld < K, a scale layout other than the
 *         two above, bad dtype), DEVICE.
 */
bsf8_status bsf8_quant_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                           uint8_t* xq, int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, void* stream);

/*
 * bsf8_quant_glu -- the step between the dense FFN's gate/up GEMM and its down
 * GEMM: y [M, >= 2F] (leading dimension ldy, F32 or BF16) holds the gate
 * outputs in columns [0, F) and the up outputs in [F, 2F) (a gate/up weight
 * grouped as gate then up gives exactly this); the call writes the down GEMM's
 * quantized input, xq [M, F] and xs [M, ceil(F/128)] (strides xs_sm, xs_sk),
 * as bsf8_quant_act would
 * for h = silu(gate) * up, without writing h.
 * ("Module w8a8_prefill", preamble and section "WHY (#917 / #928)": the
 *  gate/up/down prefill arm; the down GEMM consumes per-token 1x128 E4M3
 *  activations.  The pages do not name the activation: this is the gated SiLU
 *  of the Qwen dense FFN.)
 * h is formed in F32 in a fixed order, so the codes are reproducible:
 *   e = exp(-|g|) evaluated in F64 and rounded to F32;  t = 1 + e;
 *   q = g / t (g >= 0) or (g * e) / t (g < 0);  h = q * u,
 * each an IEEE F32 operation; then quantized exactly as bsf8_quant_act does.
 * Errors: INVALID_ARG (null, negative, ldy < 2F, ldq < F, a scale layout other
 * than the two accepted, bad dtype), ALIGNMENT (y not element aligned), DEVICE.
 */
bsf8_status bsf8_quant_glu(const void* y, int32_t y_dtype, int64_t M, int64_t F, int64_t ldy, uint8_t* xq,
                           int64_t ldq, float* xs, int64_t xs_sm, int64_t xs_sk, void* stream);

/*
 * bsf8_glu_act -- the same activation as bsf8_quant_glu, written out instead of
 * quantized: h[m, f] = silu(y[m, f]) * y[m, F + f] as F32, h [M, F] with leading
 * dimension ldh (elements).  For a down projection that takes F32 activations
 * (the W8A16 arm at decode, where the activation is not quantized).
 * ("Module w8a8_prefill", preamble: the gate/up/down dense FFN; "Qwen
 *  checkpoints with block FP8 weights", block-path paragraph: the W8A16 arm takes
 *  F32 activations.)  Same evaluation, bit for bit, as bsf8_quant_glu's h.
 * Errors: INVALID_ARG (null, negative, ldy < 2F, ldh < F, bad dtype), ALIGNMENT
 * (y or h not element aligned), UNSUPPORTED (M or F too large), DEVICE.
 */
bsf8_status bsf8_glu_act(const void* y, int32_t y_dtype, int64_t M, int64_t F, int64_t ldy, float* h, int64_t ldh,
                         void* stream);

/*
 * bsf8_workspace_size -- device workspace bytes a compute call of this handle
 * needs for M tokens on the given arm (0 when none).  The W8A8 arm uses one
 * when its tile grid is too small to occupy the device (few tokens against few
 * output features, long K): K is then cut into S ranges, each range's F32
 * partial tile goes to the workspace (S x M x N floats, N rounded up per member
 * to a multiple of 4), and a second kernel adds them in range order, so results
 * do not depend on timing.  The W8A16 arm does the same from 33 tokens while
 * its GEMM's tiles cannot cover half the device (S x M x N floats, N rounded
 * up to a multiple of 4); up to 32 tokens it needs none.  The size depends on the device's compute-unit count
 * (the current device).  No initialization is needed; every call overwrites
 * what it reads.  Calls that overlap in time must not share a workspace.  The
 * buffer must be 256-byte aligned.
 */
bsf8_status bsf8_workspace_size(const bsf8_weight* w, int32_t arm, int64_t M, size_t* bytes);

/*
 * bsf8_linear_w8a16 -- Y[m, R_i + r] = sum_kb S_i[r/128, kb] * sum_{k in kb} x[m,k] * dec(W_i[r,k])
 * with F32 activations (BF16 accepted and widened exactly) and F32
 * accumulation; weights used as stored, no operand requantized.
 * ("Qwen checkpoints with block FP8 weights", block-path and operator
 *  paragraphs; "FP8 Native Serving", section "Native FP8 vs dequant-to-BF16":
 *  the weights are decoded where they are consumed, not in a copy.)
 * Kernels (aligned operands): one token runs F32 FMAs on the vector ALUs
 * against weights decoded exactly to F32 (any K); more tokens run the BF16
 * matrix cores on an exact three-term split of each F32 activation (a
 * weight-streaming kernel up to sixteen tokens, and for 17 to 32 two of its
 * launches, 16 tokens then the rest; from 33 tokens an LDS-staged GEMM, split
 * over K into a workspace while its tiles are too few to fill the device).
 *
 * x : [M, K] F32 or BF16, leading dimension ldx (elements), 16-byte aligned
 *     rows when K allows.
 * y : [M, N] F32 or BF16 (RNE), leading dimension ldy (elements).
 * workspace: device buffer of at least bsf8_workspace_size(w, W8A16, M) bytes
 *     (may be NULL when that size is 0).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE.
 */
bsf8_status bsf8_linear_w8a16(const bsf8_weight* w, const void* x, int32_t x_dtype, int64_t M, int64_t ldx,
                              void* y, int32_t y_dtype, int64_t ldy,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsf8_linear_w8a8 -- for each 128-wide K slice kb:
 *   P = sum_{k in kb} dec(xq[m,k]) * dec(W_i[r,k])   (products exact, F32 sum)
 *   acc += P * (xs[m,kb] * S_i[r/128, kb])          (F32 epilogue)
 * then Y[m, R_i + r] = acc rounded to y_dtype (F32, or BF16 with RNE).
 * ("Module w8a8_prefill", section "WHY (#917 / #928)"; "FP8 Native Serving",
 *  section "Native FP8 vs dequant-to-BF16": FP8 operands through the matrix
 *  unit, BF16 only when results are written back.)
 * Kernels (aligned operands): up to 48 tokens the weight streams through the
 * W8A16 arm's one-token and few-token kernels with the codes decoded exactly
 * (the same exact products, each slice partial scaled as above); from 49
 * tokens the FP8 matrix-core GEMM (256x256 or 128x128 tiles, split-K when the
 * tile grid leaves compute units idle, the partials added in split order).
 *
 * xq, xs: exactly what bsf8_quant_act writes (ldq bytes; xs in either
 *         activation scale layout, strides xs_sm, xs_sk).
 * y : [M, N] BF16 or F32, leading dimension ldy (elements).
 * workspace: as for bsf8_linear_w8a16 with arm W8A8.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE.
 */
bsf8_status bsf8_linear_w8a8(const bsf8_weight* w, const uint8_t* xq, int64_t ldq, const float* xs,
                             int64_t xs_sm, int64_t xs_sk, int64_t M, void* y, int32_t y_dtype, int64_t ldy,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsf8_linear_w8a8_dynamic -- the W8A8 arm on unquantized activations: x is
 * quantized per token in 1x128 groups exactly as bsf8_quant_act does (amax /
 * 448, E4M3 round-to-nearest-even, saturating) and the product is then that
 * of bsf8_linear_w8a8; the result is bit-identical to those two calls.
 * ("Module w8a8_prefill", section "WHY (#917 / #928)": the per-token group
 *  quantization that feeds the FP8 product, and the product itself.)
 * One token, with the weight and x 16-byte aligned and the one-token streaming
 * kernels applicable (K up to 65536), is quantized inside those kernels: each
 * wave quantizes its K range into LDS before its weights land, the codes and
 * scales never go to memory and no workspace is used.  Otherwise (more tokens,
 * where every block would quantize all of x again) the codes (row pitch K
 * rounded up to 16 bytes) and the K-major scales go to the start of the
 * workspace and the W8A8 kernels read them from there.
 *
 * x : [M, K] F32 or BF16, leading dimension ldx (elements); read only.
 * y : [M, N] BF16 or F32, leading dimension ldy (elements).
 * workspace: device buffer of bsf8_workspace_size(w, BSF8_ARM_W8A8_DYNAMIC, M)
 *     bytes, 256-byte aligned; that size covers the two-step path, and the
 *     buffer may be NULL when the call quantizes inside the one-token kernels.
 * Errors: INVALID_ARG, ALIGNMENT, UNSUPPORTED, WORKSPACE (a workspace is needed
 * and missing or too small), DEVICE.
 */
bsf8_status bsf8_linear_w8a8_dynamic(const bsf8_weight* w, const void* x, int32_t x_dtype, int64_t M, int64_t ldx,
                                     void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * bsf8_linear_w8a8_noalloc -- bsf8_linear_w8a8 without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, kernels and results as bsf8_linear_w8a8; where
 * that call would use a workspace (split-K partial tiles), this one uses a
 * fixed array of BSF8_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * every device it runs on until the process ends (its device address is looked
 * up once per device, on the first call made with that device current).
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device race and must be ordered by the caller (one stream, or
 * events).  Nothing in the array needs clearing between calls.
 * Errors: as bsf8_linear_w8a8, and WORKSPACE when the call would need more than
 * BSF8_NOALLOC_SCRATCH_BYTES of partials (bsf8_workspace_size with arm W8A8
 * tells), before anything is launched; DEVICE when the array's address cannot
 * be obtained.
 */
#define BSF8_NOALLOC_SCRATCH_BYTES (64u << 20)
bsf8_status bsf8_linear_w8a8_noalloc(const bsf8_weight* w, const uint8_t* xq, int64_t ldq, const float* xs,
                                     int64_t xs_sm, int64_t xs_sk, int64_t M, void* y, int32_t y_dtype, int64_t ldy,
                                     void* stream);

/*
 * bsf8_describe -- one line naming the arithmetic and kernel configuration a
 * call with this handle, arm and M would run, with the handle's geometry.
 * ("Qwen checkpoints with block FP8 weights", block-path paragraph: report the
 *  compute path next to the checkpoint identity; "Module w8a8_prefill",
 *  section "ACCURACY": make visible which arithmetic ran.)
 * Returns a pointer to thread-local storage valid until the next call on the
 * same thread; NULL only for a NULL handle.
 */
const char* bsf8_describe(const bsf8_weight* w, int32_t arm, int64_t M);

/*
 * The resident=False arm: upcast at load, then a dense BF16 product.
 * ("th#1803: the consumer half of the layout gate", section "What lands": with
 *  resident=False the loader upcasts the weight ahead of time instead of
 *  keeping the FP8 bytes; "FP8 Native Serving", section "Native FP8 vs
 *  dequant-to-BF16": the dequantized operand is BF16 and the product runs on
 *  BF16 matrix units.)
 *
 * bsf8_upcast -- write the dense copy of the handle's weight:
 *   out[R_i + r, k] = dec(W_i[r, k]) * S_i[r/128, k/128]   (per-tensor: * s_i)
 * for every member i (rows in member order, as the output features of the other
 * arms).  Each value is one F32 product (exact for BF16 scales) written as F32,
 * or rounded to nearest-even BF16 (out_dtype BSF8_DT_BF16).  out: device
 * [n_total, ldo] of out_dtype, ldo >= K, caller-owned; columns K..ldo-1 are not
 * written.  One pass over the weight bytes (HBM-bound), asynchronous on
 * `stream`.  Errors: INVALID_ARG (null, dtype, ldo), ALIGNMENT (out not element
 * aligned), UNSUPPORTED (more than 2^32 16-element pieces).
 *
 * bsf8_linear_dense -- Y[m, n] = sum_k x[m, k] * wd[n, k] for BF16 wd [N, K]
 * (row-major, row pitch K: bsf8_upcast's output with ldo = K) and BF16 x [M, K]
 * with row pitch ldx; BF16 x BF16 products accumulated in F32 on the BF16
 * matrix cores; y F32 or BF16 (RNE) [M, ldy].  Needs K and ldx multiples of 8,
 * wd and x 16-byte aligned (ALIGNMENT otherwise), K <= 65536 and each operand
 * below 2 GiB (UNSUPPORTED otherwise).  A workspace of
 * bsf8_dense_workspace_size bytes (256-byte aligned) is needed when the tile
 * grid is split over K, as for the W8A8 arm; M == 0 is a no-op.
 */
bsf8_status bsf8_upcast(const bsf8_weight* w, void* out, int32_t out_dtype, int64_t ldo, void* stream);
bsf8_status bsf8_dense_workspace_size(int64_t N, int64_t K, int64_t M, size_t* bytes);
bsf8_status bsf8_linear_dense(const uint16_t* wd, int64_t N, int64_t K, const uint16_t* x, int64_t M, int64_t ldx,
                              void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Header-only checkpoint inspection ("th#1803: the consumer half of the layout
 * gate", sections "What lands": verification from safetensors headers alone,
 * before any weight byte is read; "Why the refusals matter more than the
 * load" and "Proof": row-wise, transposed-grid, scale-less and dense trees are
 * refused by name.  "Qwen checkpoints with block FP8 weights", layout
 * paragraph: the declaration and the weight / weight_scale_inv leaves.)
 *
 * bsf8_parse_quant_config -- read quant_method and weight_block_size from a
 * checkpoint config: json_text is a NUL-terminated JSON object, either the
 * model config holding a "quantization_config" object or that object itself.
 * out->quant_method_fp8 = (quant_method == "fp8"); block_n / block_k from
 * weight_block_size, or 0 / 0 when it is absent or null (the per-tensor
 * reading).  Host-only.  Errors: INVALID_ARG (null argument, malformed JSON,
 * not an object), DECL (no quant_method string, or a weight_block_size that is
 * not a pair of positive integers).
 *
 * bsf8_inspect_safetensors -- read the 8-byte header length and the JSON
 * header of the safetensors file at `path` (nothing after the header) and
 * list its linear units: every "<prefix>.weight" tensor stored as F8_E4M3 /
 * F8_E5M2, or with a "<prefix>.weight_scale_inv" or "<prefix>.weight_scale"
 * sibling.  Other tensors (dense BF16/F16 weights such as the output head,
 * norms, biases) keep their own representation and are not units.  Each unit
 * carries header descriptors (data = NULL), the file offsets of its bytes and
 * the status bsf8_validate gives it alone under *decl.  units: caller array of
 * `capacity` records (may be NULL when capacity is 0); *n_units = the number
 * of units in the file (records past `capacity` are not written).  Host-only.
 * Returns OK when every unit validates; else the first refusing unit's status
 * in header order (bsf8_last_error names the unit); WEIGHT_DTYPE when the file
 * has two-dimensional weights but no unit (a dense tree).  Errors also:
 * INVALID_ARG (null argument, unreadable file, header length outside
 * [2, BSF8_SAFETENSORS_MAX_HEADER], malformed header JSON).
 */
#define BSF8_SAFETENSORS_MAX_HEADER 100000000
typedef struct bsf8_unit {
  char prefix[256];            /* tensor name without ".weight" (NUL-terminated) */
  int32_t prefix_truncated;    /* 1 when the name did not fit */
  int32_t status;              /* bsf8_status of this unit alone */
  bsf8_tensor_desc weight;
  bsf8_tensor_desc scale_inv;  /* valid when has_scale_inv */
  bsf8_tensor_desc scale;      /* valid when has_scale */
  int32_t has_scale_inv;
  int32_t has_scale;
  int64_t weight_offset;       /* byte offset of the weight's data in the file */
  int64_t scale_offset;        /* of the scale leaf present (scale_inv first), -1 when none */
} bsf8_unit;
bsf8_status bsf8_parse_quant_config(const char* json_text, bsf8_decl* out);
bsf8_status bsf8_inspect_safetensors(const char* path, const bsf8_decl* decl, bsf8_unit* units, int32_t capacity,
                                     int32_t* n_units);

/*
 * bsf8_read_stream -- measurement aid, not part of the projection: reads
 * `bytes` bytes at `p` as a plain coalesced stream.  Timed on a GEMV's weight
 * bytes it gives the achievable read rate to compare the GEMV's rate with.
 * p: device pointer, 16-byte aligned; bytes: a multiple of 16, >= 0.
 * sink: device array of BSF8_READ_STREAM_SINK_WORDS 4-byte words the caller
 * owns.  The launch uses min(ceil(bytes / 16 KiB), BSF8_READ_STREAM_SINK_WORDS)
 * blocks; block b overwrites sink[b] with the XOR of the 4-byte words it read
 * and words past the last block are left as they were, so the XOR of a sink
 * zeroed beforehand equals the XOR of the buffer's words.  Stream-ordered;
 * allocates nothing.  Errors: INVALID_ARG (null pointer, negative size),
 * ALIGNMENT, DEVICE.
 */
#define BSF8_READ_STREAM_SINK_WORDS 2048
bsf8_status bsf8_read_stream(const void* p, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSF8_H */

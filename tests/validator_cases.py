"""Header-level validator cases shared by the oracle pin test and the C-ABI test.

Each case: (id, quant_method, block, members, expected status name).  Members
are lists of dicts: weight (dtype, shape, addr), scale_inv / scale (dtype,
shape, addr) or None.  Expectations follow the refusal list of the pages
(Qwen checkpoints with block FP8 weights, operator/grid/refusal paragraph;
th#1803 PR, sections 'Why the refusals matter more than the load' and 'Proof')
and the precedence stated in the oracle's ``validate`` docstring.
"""


def T(dtype, shape, addr=None):
    return dict(dtype=dtype, shape=list(shape), addr=addr)


def mem(wshape=(128, 256), wdt="F8_E4M3", sinv=None, s=None, waddr=None):
    return dict(weight=T(wdt, wshape, waddr), scale_inv=sinv, scale=s)


GOOD = mem(sinv=T("BF16", (1, 2)))

CASES = [
    ("page_example_ok", "fp8", (128, 128), [GOOD], "OK"),
    ("f32_scales_ok", "fp8", (128, 128), [mem(sinv=T("F32", (1, 2)))], "OK"),
    ("tails_ok", "fp8", (128, 128), [mem((5000, 4000), sinv=T("BF16", (40, 32)))], "OK"),
    ("square_transposed_undetectable", "fp8", (128, 128), [mem((5120, 5120), sinv=T("BF16", (40, 40)))], "OK"),
    ("grouped_qkv_ok", "fp8", (128, 128),
     [mem((6144, 5120), sinv=T("BF16", (48, 40))), mem((1000, 5120), sinv=T("BF16", (8, 40))),
      mem((1000, 5120), sinv=T("BF16", (8, 40)))], "OK"),
    ("no_members", "fp8", (128, 128), [], "GROUP"),
    ("nine_members", "fp8", (128, 128), [GOOD] * 9, "GROUP"),
    ("decl_not_fp8", "int8", (128, 128), [GOOD], "DECL"),
    ("decl_block_64", "fp8", (64, 64), [GOOD], "DECL"),
    ("decl_block_rect", "fp8", (128, 64), [GOOD], "DECL"),
    ("e5m2_weight", "fp8", (128, 128), [mem(wdt="F8_E5M2", sinv=T("BF16", (1, 2)))], "WEIGHT_E5M2"),
    ("dense_bf16_tree", "fp8", (128, 128), [mem(wdt="BF16", sinv=T("BF16", (1, 2)))], "WEIGHT_DTYPE"),
    ("dense_bf16_no_scale", "fp8", (128, 128), [mem(wdt="BF16")], "WEIGHT_DTYPE"),
    ("weight_rank3", "fp8", (128, 128), [mem((2, 128, 256), sinv=T("BF16", (1, 2)))], "WEIGHT_RANK"),
    ("weight_rank1", "fp8", (128, 128), [mem((256,), sinv=T("BF16", (1, 2)))], "WEIGHT_RANK"),
    ("weight_empty", "fp8", (128, 128), [mem((0, 256), sinv=T("BF16", (0, 2)))], "WEIGHT_EMPTY"),
    ("missing_scale", "fp8", (128, 128), [mem()], "SCALE_MISSING"),
    ("ambiguous_row_and_block", "fp8", (128, 128), [mem(sinv=T("BF16", (1, 2)), s=T("F32", (128,)))], "SCALE_AMBIGUOUS"),
    ("rowwise_tree", "fp8", (128, 128), [mem(s=T("F32", (128,)))], "SCALE_ROWWISE"),
    ("rank1_scale_inv", "fp8", (128, 128), [mem(sinv=T("BF16", (2,)))], "SCALE_ROWWISE"),
    ("per_tensor_scale", "fp8", (128, 128), [mem(s=T("F32", ()))], "SCALE_PER_TENSOR"),
    ("rank0_scale_inv", "fp8", (128, 128), [mem(sinv=T("F32", ()))], "SCALE_RANK"),
    ("rank3_scale", "fp8", (128, 128), [mem(sinv=T("BF16", (1, 1, 2)))], "SCALE_RANK"),
    ("scale_f16", "fp8", (128, 128), [mem(sinv=T("F16", (1, 2)))], "SCALE_DTYPE"),
    ("scale_e4m3", "fp8", (128, 128), [mem(sinv=T("F8_E4M3", (1, 2)))], "SCALE_DTYPE"),
    ("transposed_grid", "fp8", (128, 128), [mem(sinv=T("BF16", (2, 1)))], "SCALE_TRANSPOSED"),
    ("transposed_tail_grid", "fp8", (128, 128), [mem((5000, 4000), sinv=T("BF16", (32, 40)))], "SCALE_TRANSPOSED"),
    ("floor_grid", "fp8", (128, 128), [mem((5000, 4000), sinv=T("BF16", (39, 31)))], "SCALE_GRID"),
    ("mis_blocked_64", "fp8", (128, 128), [mem(sinv=T("BF16", (2, 4)))], "SCALE_GRID"),
    ("block_leaf_under_plain_name", "fp8", (128, 128), [mem(s=T("F32", (1, 2)))], "SCALE_GRID"),
    ("group_k_mismatch", "fp8", (128, 128), [GOOD, mem((128, 384), sinv=T("BF16", (1, 3)))], "GROUP"),
    ("group_scale_dtype_mismatch", "fp8", (128, 128), [GOOD, mem(sinv=T("F32", (1, 2)))], "GROUP"),
    ("second_member_bad_first", "fp8", (128, 128), [GOOD, mem(sinv=T("BF16", (2, 1)))], "SCALE_TRANSPOSED"),
    ("member_order_precedence", "fp8", (128, 128),
     [mem(sinv=T("BF16", (1, 3))), mem(wdt="F8_E5M2", sinv=T("BF16", (1, 2)))], "SCALE_GRID"),
    ("decl_before_member", "fp8", (64, 128), [mem(wdt="F8_E5M2")], "DECL"),
    ("e5m2_before_missing_scale", "fp8", (128, 128), [mem(wdt="F8_E5M2")], "WEIGHT_E5M2"),
    ("weight_misaligned", "fp8", (128, 128), [mem(sinv=T("BF16", (1, 2), 4096), waddr=4104)], "ALIGNMENT"),
    ("scale_misaligned", "fp8", (128, 128), [mem(sinv=T("F32", (1, 2), 4098), waddr=4096)], "ALIGNMENT"),
    ("aligned_addresses_ok", "fp8", (128, 128), [mem(sinv=T("BF16", (1, 2), 4098), waddr=8192)], "OK"),
    ("grid_before_alignment", "fp8", (128, 128), [mem(sinv=T("BF16", (1, 3), 4096), waddr=4104)], "SCALE_GRID"),
    # Per-tensor layout (FP8 Native Serving, 'The two FP8 checkpoint shapes': one
    # weight_scale per tensor, the degenerate block), declared as block (0, 0).
    ("per_tensor_f32_scalar_ok", "fp8", (0, 0), [mem(s=T("F32", ()))], "OK"),
    ("per_tensor_one_element_ok", "fp8", (0, 0), [mem(s=T("F32", (1,)))], "OK"),
    ("per_tensor_bf16_scalar_ok", "fp8", (0, 0), [mem(s=T("BF16", ()))], "OK"),
    ("per_tensor_group_ok", "fp8", (0, 0), [mem(s=T("F32", ())), mem((1000, 256), s=T("F32", ()))], "OK"),
    ("per_tensor_decl_with_grid", "fp8", (0, 0), [mem(sinv=T("BF16", (1, 2)))], "DECL"),
    ("per_tensor_decl_rowwise", "fp8", (0, 0), [mem(s=T("F32", (128,)))], "SCALE_ROWWISE"),
    ("per_tensor_decl_rank2", "fp8", (0, 0), [mem(s=T("F32", (1, 1)))], "SCALE_RANK"),
    ("per_tensor_decl_f16", "fp8", (0, 0), [mem(s=T("F16", ()))], "SCALE_DTYPE"),
    ("per_tensor_decl_missing", "fp8", (0, 0), [mem()], "SCALE_MISSING"),
    ("per_tensor_decl_e5m2", "fp8", (0, 0), [mem(wdt="F8_E5M2", s=T("F32", ()))], "WEIGHT_E5M2"),
    ("per_tensor_group_dtype_mismatch", "fp8", (0, 0), [mem(s=T("F32", ())), mem(s=T("BF16", ()))], "GROUP"),
    ("per_tensor_scale_misaligned", "fp8", (0, 0), [mem(s=T("F32", (), 4098), waddr=4096)], "ALIGNMENT"),
    ("decl_half_zero_block", "fp8", (0, 128), [mem(s=T("F32", ()))], "DECL"),
]

"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* the library loads and exports every function include/bsf8.h declares;
* the C++ validator returns the oracle's status on every validator case;
* handles over placeholder addresses report the geometry and the member-local
  scale rows the oracle derives;
* argument errors are refused before any launch, and M == 0 is a no-op.
"""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_linear_amd as B
import oracle as O
from test_oracle_validate import to_oracle
from validator_cases import CASES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "bsf8.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsf8_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = B.lib()
    names = header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == {e[0] for e in B.EXPORTS}


def test_abi_version_and_status_names():
    L = B.lib()
    assert L.bsf8_abi_version() == 1
    want = ["OK", "INVALID_ARG", "GROUP", "DECL", "WEIGHT_E5M2", "WEIGHT_DTYPE", "WEIGHT_RANK", "WEIGHT_EMPTY",
            "SCALE_MISSING", "SCALE_AMBIGUOUS", "SCALE_ROWWISE", "SCALE_PER_TENSOR", "SCALE_RANK", "SCALE_DTYPE",
            "SCALE_TRANSPOSED", "SCALE_GRID", "ALIGNMENT", "UNSUPPORTED", "WORKSPACE", "DEVICE"]
    assert [B.status_name(i) for i in range(len(want))] == want


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_validator_matches_oracle(case):
    _, qm, block, members, want = case
    assert B.validate(qm, block, members) == want
    assert O.validate(qm, block, to_oracle(members)) == want


def _handle(rows, K, sdt="BF16", base=1 << 40):
    members, addr = [], base
    for r in rows:
        nb, kb = O.scale_grid_shape(r, K)
        members.append(dict(weight=dict(dtype="F8_E4M3", shape=(r, K), addr=addr),
                            scale_inv=dict(dtype=sdt, shape=(nb, kb), addr=addr + (1 << 32))))
        addr += 1 << 33
    decl = B._decl()
    arr, keep = B._members_array(members)
    h = ctypes.c_void_p()
    st = B.lib().bsf8_weight_create(ctypes.byref(decl), arr, len(members), ctypes.byref(h))
    return st, h


def test_handle_geometry_and_member_local_rows():
    rows = [6144, 1000, 1000]
    st, h = _handle(rows, 5120)
    assert st == 0
    L = B.lib()
    try:
        n, k, nm = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        assert L.bsf8_weight_geometry(h, ctypes.byref(n), ctypes.byref(k), ctypes.byref(nm)) == 0
        assert (n.value, k.value, nm.value) == (8144, 5120, 3)
        R, Bo = O.member_table(rows)
        for row in [0, 127, 128, 6143, 6144, 7143, 7144, 7167, 7271, 7272, 8143]:
            mi, lr, sr = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
            assert L.bsf8_weight_scale_row(h, row, ctypes.byref(mi), ctypes.byref(lr), ctypes.byref(sr)) == 0
            assert sr.value == O.stacked_scale_row(row, rows)
            assert lr.value == (row - R[mi.value]) // 128
        # V's first row sits on stacked scale row 56, where a global n/128 grid would say 55
        mi, lr, sr = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
        L.bsf8_weight_scale_row(h, 7144, ctypes.byref(mi), ctypes.byref(lr), ctypes.byref(sr))
        assert (mi.value, lr.value, sr.value) == (2, 0, 56) and 7144 // 128 == 55
        assert L.bsf8_weight_scale_row(h, 8144, ctypes.byref(mi), ctypes.byref(lr), ctypes.byref(sr)) == 1
        d = L.bsf8_describe(h, 0, 1).decode()
        assert "w8a16" in d and "K=5120" in d and "members=3" in d
        # W8A16 plans by token count: the few-token kernel to 16, two of its
        # launches (16, then the rest) to 32, then the LDS-staged GEMM, split over
        # K while its tile grid is small (32 row tiles x 1 token tile x 8 splits)
        assert "kernel=w8a16_small_m " in L.bsf8_describe(h, 0, 16).decode()
        d = L.bsf8_describe(h, 0, 24).decode()
        assert d.startswith("two launches, tokens [0, 16) then [16, 24): ") and d.count("kernel=w8a16_small_m ") == 2, d
        # (one token on this grouped weight also takes the few-token kernel: 32-row blocks)
        assert L.bsf8_describe(h, 0, 17).decode().startswith("two launches, tokens [0, 16) then [16, 17): ")
        d = L.bsf8_describe(h, 0, 33).decode()
        assert "kernel=w8a16_gemm " in d and "split_k=8 (5 chunks per split" in d and "blocks=256" in d, d
        b33 = ctypes.c_size_t()
        assert L.bsf8_workspace_size(h, 0, 33, ctypes.byref(b33)) == 0 and b33.value == 8 * 33 * 8144 * 4
        assert L.bsf8_workspace_size(h, 0, 32, ctypes.byref(b33)) == 0 and b33.value == 0
        d = L.bsf8_describe(h, 1, 512).decode()
        assert "w8a8" in d and "e4m3" in d
    finally:
        L.bsf8_weight_destroy(h)


def test_workspace_sizes():
    L = B.lib()
    st, h = _handle([5120], 5120)
    assert st == 0
    try:
        b = ctypes.c_size_t()
        assert L.bsf8_workspace_size(h, 0, 8, ctypes.byref(b)) == 0 and b.value == 0
        assert L.bsf8_workspace_size(h, 0, 0, ctypes.byref(b)) == 0 and b.value == 0
        # W8A8 split-K: the workspace holds S partial tiles of every split row
        # tile; its size agrees with the plan the handle describes (256 compute
        # units are assumed when no device is present)
        for M in (1024, 8192):
            assert L.bsf8_workspace_size(h, 1, M, ctypes.byref(b)) == 0
            d = L.bsf8_describe(h, 1, M).decode()
            sk = int(re.search(r"split_k=(\d+)", d).group(1))
            rows = int(re.search(r"split_row_tiles=(\d+)", d).group(1))
            tile = int(re.search(r"tile=(\d+)x", d).group(1))
            assert b.value == (sk * M * rows * tile * 4 if sk > 1 else 0), (M, d)
        # 20 row tiles x 4 token tiles < 256 units: every tile is split
        assert "split_k=3 split_row_tiles=20" in L.bsf8_describe(h, 1, 1024).decode()
        # one to 48 tokens stream the weight with E4M3 activations and use no
        # workspace; the size reported stays an upper bound over the paths
        assert "w8a16_m1<e4m3>" in L.bsf8_describe(h, 1, 1).decode()
        for M in (2, 4, 8, 16, 17, 32, 33, 48):
            d = L.bsf8_describe(h, 1, M).decode()
            assert "kernel=w8a16_small_m<e4m3>" in d and "e4m3 codes decoded exactly to bf16" in d, d
            assert L.bsf8_workspace_size(h, 1, M, ctypes.byref(b)) == 0
        assert "w8a8_gemm" in L.bsf8_describe(h, 1, 49).decode()
        assert L.bsf8_workspace_size(h, 7, 8, ctypes.byref(b)) == 1
    finally:
        L.bsf8_weight_destroy(h)


def test_dynamic_w8a8_workspace_describe_and_refusals():
    """bsf8_linear_w8a8_dynamic: its workspace is the two-step form's (codes at a
    16-byte row pitch, K-major scales, the W8A8 call's own workspace, each from a
    256-byte boundary); one token describes the quantizing one-token kernel, more
    the quantizer and then the W8A8 kernels; bad arguments are refused before any
    launch, a missing workspace wherever the two-step form is needed."""
    L = B.lib()
    st, h = _handle([5120], 5120)
    assert st == 0
    r256 = lambda n: (n + 255) // 256 * 256
    try:
        b, w8 = ctypes.c_size_t(), ctypes.c_size_t()
        for M in (1, 4, 5, 1024):
            assert L.bsf8_workspace_size(h, B.ARM_W8A8_DYNAMIC, M, ctypes.byref(b)) == 0
            assert L.bsf8_workspace_size(h, B.ARM_W8A8, M, ctypes.byref(w8)) == 0
            assert b.value == r256(M * 5120) + r256(M * 40 * 4) + w8.value, M
        assert L.bsf8_workspace_size(h, B.ARM_W8A8_DYNAMIC, 0, ctypes.byref(b)) == 0 and b.value == 0
        d1 = L.bsf8_describe(h, B.ARM_W8A8_DYNAMIC, 1).decode()
        assert "arm=w8a8-dynamic" in d1 and "kernel=w8a16_m1<quantizing>" in d1, d1
        d3 = L.bsf8_describe(h, B.ARM_W8A8_DYNAMIC, 3).decode()
        assert d3.startswith("quant_act into the workspace") and "kernel=w8a16_small_m<e4m3>" in d3, d3
        d49 = L.bsf8_describe(h, B.ARM_W8A8_DYNAMIC, 49).decode()
        assert d49.startswith("quant_act into the workspace") and "w8a8_gemm" in d49, d49
        fake = ctypes.c_void_p(1 << 40)
        ws_fake = ctypes.c_void_p(1 << 41)
        call = lambda x, dt, M, ldx, ws=None, wsb=0: B.status_name(
            L.bsf8_linear_w8a8_dynamic(h, x, dt, M, ldx, fake, B.DT_BF16, 5120, ws, wsb, None))
        assert call(fake, B.DT_F32, 0, 5120) == "OK"
        assert call(fake, B.DT_F32, -1, 5120) == "INVALID_ARG"
        assert call(fake, B.DT_F16, 2, 5120) == "INVALID_ARG"
        assert call(fake, B.DT_F32, 2, 5119) == "INVALID_ARG"
        assert call(None, B.DT_F32, 2, 5120) == "INVALID_ARG"
        assert call(ctypes.c_void_p((1 << 40) + 2), B.DT_F32, 1, 5120) == "ALIGNMENT"
        # two or five tokens, or one with x only element-aligned: the two-step form, refused without a workspace
        assert call(fake, B.DT_F32, 5, 5120) == "WORKSPACE"
        assert call(fake, B.DT_F32, 2, 5120) == "WORKSPACE"
        assert call(ctypes.c_void_p((1 << 40) + 4), B.DT_F32, 1, 5120) == "WORKSPACE"
        assert L.bsf8_workspace_size(h, B.ARM_W8A8_DYNAMIC, 5, ctypes.byref(b)) == 0
        assert call(fake, B.DT_F32, 5, 5120, ws_fake, b.value - 1) == "WORKSPACE"
        assert call(fake, B.DT_F32, 5, 5120, ctypes.c_void_p((1 << 41) + 16), b.value) == "ALIGNMENT"
    finally:
        L.bsf8_weight_destroy(h)


def test_compute_calls_refuse_bad_arguments_without_launching():
    L = B.lib()
    st, h = _handle([128], 256)
    assert st == 0
    try:
        fake = ctypes.c_void_p(1 << 40)
        # M == 0: success, nothing launched
        assert L.bsf8_linear_w8a16(h, fake, B.DT_F32, 0, 256, fake, B.DT_F32, 128, None, 0, None) == 0
        assert L.bsf8_linear_w8a8(h, fake, 256, fake, 2, 1, 0, fake, B.DT_BF16, 128, None, 0, None) == 0
        assert L.bsf8_quant_act(fake, B.DT_F32, 0, 256, 256, fake, 256, fake, 2, 1, None) == 0
        # refusals
        assert B.status_name(L.bsf8_linear_w8a16(h, fake, B.DT_F32, -1, 256, fake, B.DT_F32, 128, None, 0, None)) == "INVALID_ARG"
        assert B.status_name(L.bsf8_linear_w8a16(h, fake, B.DT_F16, 4, 256, fake, B.DT_F32, 128, None, 0, None)) == "INVALID_ARG"
        assert B.status_name(L.bsf8_linear_w8a16(h, fake, B.DT_F32, 4, 255, fake, B.DT_F32, 128, None, 0, None)) == "INVALID_ARG"
        assert B.status_name(L.bsf8_linear_w8a8(h, fake, 256, fake, 1, 1, 4, fake, B.DT_BF16, 128, None, 0, None)) == "INVALID_ARG"
        assert B.status_name(L.bsf8_linear_w8a8(h, None, 256, fake, 2, 1, 4, fake, B.DT_BF16, 128, None, 0, None)) == "INVALID_ARG"
        assert B.status_name(L.bsf8_quant_act(fake, B.DT_F32, 4, 256, 100, fake, 256, fake, 2, 1, None)) == "INVALID_ARG"
        assert B.status_name(L.bsf8_quant_act(ctypes.c_void_p((1 << 40) + 2), B.DT_F32, 4, 256, 256, fake, 256, fake, 2, 1, None)) == "ALIGNMENT"
        assert B.status_name(L.bsf8_linear_w8a16(None, fake, B.DT_F32, 4, 256, fake, B.DT_F32, 128, None, 0, None)) == "INVALID_ARG"
        assert "INVALID_ARG" in L.bsf8_last_error().decode()
        # activation scale layouts: only token-major (sk = 1, sm >= Kb) and K-major (sm = 1, sk >= M)
        for sm, sk in ((3, 2), (1, 3), (2, 0), (0, 1), (-2, 1)):
            assert B.status_name(L.bsf8_linear_w8a8(h, fake, 256, fake, sm, sk, 4, fake, B.DT_BF16, 128, None, 0,
                                                    None)) == "INVALID_ARG", (sm, sk)
            assert B.status_name(L.bsf8_quant_act(fake, B.DT_F32, 4, 256, 256, fake, 256, fake, sm, sk,
                                                  None)) == "INVALID_ARG", (sm, sk)
            assert B.status_name(L.bsf8_quant_glu(fake, B.DT_BF16, 4, 256, 512, fake, 256, fake, sm, sk,
                                                  None)) == "INVALID_ARG", (sm, sk)
        assert "neither token-major nor K-major" in L.bsf8_last_error().decode()
    finally:
        L.bsf8_weight_destroy(h)


def test_create_needs_device_addresses():
    members = [dict(weight=dict(dtype="F8_E4M3", shape=(128, 256)), scale_inv=dict(dtype="BF16", shape=(1, 2)))]
    decl = B._decl()
    arr, keep = B._members_array(members)
    h = ctypes.c_void_p()
    assert B.status_name(B.lib().bsf8_weight_create(ctypes.byref(decl), arr, 1, ctypes.byref(h))) == "INVALID_ARG"
    assert not h.value


def test_read_stream_refusals():
    L = B.lib()
    fake = ctypes.c_void_p(1 << 40)
    assert B.status_name(L.bsf8_read_stream(None, 16, fake, None)) == "INVALID_ARG"
    assert B.status_name(L.bsf8_read_stream(fake, -16, fake, None)) == "INVALID_ARG"
    assert B.status_name(L.bsf8_read_stream(fake, 24, fake, None)) == "ALIGNMENT"
    assert B.status_name(L.bsf8_read_stream(ctypes.c_void_p((1 << 40) + 8), 16, fake, None)) == "ALIGNMENT"
    assert L.bsf8_read_stream(fake, 0, fake, None) == 0


def test_read_stream_sink_size_matches_header():
    with open(os.path.join(ROOT, "include", "bsf8.h")) as f:
        hdr = f.read()
    assert int(re.search(r"#define BSF8_READ_STREAM_SINK_WORDS (\d+)", hdr).group(1)) == B.READ_STREAM_SINK_WORDS


def test_dense_arm_refuses_bad_arguments_without_launching():
    L = B.lib()
    st, h = _handle([128, 300], 256)
    assert st == 0
    fake = ctypes.c_void_p(1 << 40)
    name = lambda s: B.status_name(s)
    try:
        # upcast: dtype, leading dimension, null, element alignment
        assert name(L.bsf8_upcast(h, fake, B.DT_F16, 256, None)) == "INVALID_ARG"
        assert name(L.bsf8_upcast(h, fake, B.DT_BF16, 255, None)) == "INVALID_ARG"
        assert name(L.bsf8_upcast(h, None, B.DT_BF16, 256, None)) == "INVALID_ARG"
        assert name(L.bsf8_upcast(None, fake, B.DT_BF16, 256, None)) == "INVALID_ARG"
        assert name(L.bsf8_upcast(h, ctypes.c_void_p((1 << 40) + 2), B.DT_F32, 256, None)) == "ALIGNMENT"
        # dense product
        args = lambda N=512, K=256, x=fake, M=4, ldx=256, ydt=B.DT_F32, ldy=512, ws=None, wsb=0: \
            L.bsf8_linear_dense(fake, N, K, x, M, ldx, fake, ydt, ldy, ws, wsb, None)
        assert args(M=0) == 0
        assert name(args(M=-1)) == "INVALID_ARG"
        assert name(args(ydt=B.DT_F16)) == "INVALID_ARG"
        assert name(args(ldx=255)) == "INVALID_ARG"
        assert name(args(ldy=511)) == "INVALID_ARG"
        assert name(args(x=None)) == "INVALID_ARG"
        assert name(args(K=250, ldx=256)) == "ALIGNMENT"
        assert name(args(ldx=260)) == "ALIGNMENT"
        assert name(args(x=ctypes.c_void_p((1 << 40) + 8))) == "ALIGNMENT"
        assert name(args(K=65544, ldx=65544)) == "UNSUPPORTED"
        # one row tile, four token rows: the plan splits K, so a workspace is required
        b = ctypes.c_size_t()
        assert L.bsf8_dense_workspace_size(512, 4096, 4, ctypes.byref(b)) == 0 and b.value > 0
        assert name(args(K=4096, ldx=4096)) == "WORKSPACE"
        assert name(L.bsf8_dense_workspace_size(0, 4096, 4, ctypes.byref(b))) == "INVALID_ARG"
        # the handle's dense arm describes and sizes the product over its dense copy (N = 428)
        assert L.bsf8_workspace_size(h, B.ARM_DENSE, 4, ctypes.byref(b)) == 0
        w2 = ctypes.c_size_t()
        assert L.bsf8_dense_workspace_size(428, 256, 4, ctypes.byref(w2)) == 0 and w2.value == b.value
        d = L.bsf8_describe(h, B.ARM_DENSE, 4).decode()
        assert "arm=dense" in d and "N=428 K=256" in d
    finally:
        L.bsf8_weight_destroy(h)


def test_quant_glu_refuses_bad_arguments_without_launching():
    L = B.lib()
    fake = ctypes.c_void_p(1 << 40)
    name = lambda s: B.status_name(s)
    assert L.bsf8_quant_glu(fake, B.DT_BF16, 0, 256, 512, fake, 256, fake, 2, 1, None) == 0
    assert L.bsf8_quant_glu(fake, B.DT_BF16, 4, 0, 512, fake, 256, fake, 2, 1, None) == 0
    assert name(L.bsf8_quant_glu(fake, B.DT_BF16, -1, 256, 512, fake, 256, fake, 2, 1, None)) == "INVALID_ARG"
    assert name(L.bsf8_quant_glu(fake, B.DT_F16, 4, 256, 512, fake, 256, fake, 2, 1, None)) == "INVALID_ARG"
    assert name(L.bsf8_quant_glu(fake, B.DT_BF16, 4, 256, 511, fake, 256, fake, 2, 1, None)) == "INVALID_ARG"
    assert name(L.bsf8_quant_glu(fake, B.DT_BF16, 4, 256, 512, fake, 255, fake, 2, 1, None)) == "INVALID_ARG"
    assert name(L.bsf8_quant_glu(fake, B.DT_BF16, 4, 257, 514, fake, 257, fake, 2, 1, None)) == "INVALID_ARG"
    assert name(L.bsf8_quant_glu(None, B.DT_BF16, 4, 256, 512, fake, 256, fake, 2, 1, None)) == "INVALID_ARG"
    assert name(L.bsf8_quant_glu(ctypes.c_void_p((1 << 40) + 2), B.DT_F32, 4, 256, 512, fake, 256, fake, 2, 1,
                                 None)) == "ALIGNMENT"


def test_binding_refuses_host_tensors_before_any_library_call():
    """Host (CPU) tensors never reach the library: their addresses are not device
    memory, so the binding raises ValueError first, for every call that takes a
    tensor, and also rejects activation codes of any dtype other than E4M3 bytes."""
    import types

    import torch
    codes = torch.zeros((256, 256), dtype=torch.uint8)
    grid = torch.ones((2, 2), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.BlockFP8Weight([(codes, grid)])
    x = torch.zeros((4, 256), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.quant_act(x)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.quant_glu(torch.zeros((4, 512), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.linear_dense(torch.zeros((8, 64), dtype=torch.bfloat16), torch.zeros((2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.read_stream(torch.zeros(64, dtype=torch.int32), torch.zeros(B.READ_STREAM_SINK_WORDS, dtype=torch.int32))
    # A handle that claims a GPU: host activations, outputs and workspaces are refused.
    fake = types.SimpleNamespace(device=torch.device("cuda", 0), K=256, n_total=256, handle=None,
                                 workspace=lambda arm, M: (None, 0))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.linear_w8a16(fake, x)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.linear_w8a8(fake, torch.zeros((4, 256), dtype=torch.uint8), torch.ones((4, 2), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.upcast(fake, out=torch.empty((256, 256), dtype=torch.bfloat16))


def test_binding_checks_activation_code_dtype():
    """xq must hold E4M3 bytes (uint8 or float8_e4m3fn): an int8 or float tensor of the
    right shape is refused by dtype.  The predicate the calls use is checked directly on
    meta tensors, since no device tensor exists without a GPU."""
    import torch
    for dt, ok in ((torch.uint8, True), (torch.float8_e4m3fn, True), (torch.int8, False), (torch.float32, False),
                   (torch.float8_e5m2, False)):
        assert B._codes_dtype_ok(torch.empty((2, 2), dtype=dt, device="meta")) == ok, dt

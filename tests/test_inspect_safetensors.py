"""Header-only checkpoint inspection (CPU): real safetensors files written by the
safetensors package, read back by bsf8_inspect_safetensors from their headers.

("th#1803: the consumer half of the layout gate", sections "What lands" and
"Proof": a tiny tree verifies from headers alone with the grid derived per unit,
down_proj [128,256] -> scale [1,2]; row-wise, transposed-grid and dense trees are
refused by name.  Each unit's status is also checked against the oracle's
validator on descriptors read from the header with Python's own JSON reader.)
"""
import json
import os
import struct

import pytest
import torch

import block_scaled_fp8_linear_amd as B
import oracle as O
from safetensors.torch import save_file


def f8(shape):
    return torch.zeros(shape, dtype=torch.float8_e4m3fn)


def bf16(shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(shape):
    return torch.zeros(shape, dtype=torch.float32)


def tiny_tree(**over):
    t = {
        "model.layers.0.self_attn.q_proj.weight": f8((256, 256)),
        "model.layers.0.self_attn.q_proj.weight_scale_inv": bf16((2, 2)),
        "model.layers.0.mlp.down_proj.weight": f8((128, 256)),
        "model.layers.0.mlp.down_proj.weight_scale_inv": bf16((1, 2)),
        "model.layers.0.input_layernorm.weight": bf16((256,)),
        "lm_head.weight": bf16((512, 256)),
    }
    t.update(over)
    return {k: v for k, v in t.items() if v is not None}


def write(tmp_path, name, tensors):
    p = os.path.join(str(tmp_path), name)
    save_file(tensors, p)
    return p


def header_of(path):
    with open(path, "rb") as f:
        n = struct.unpack("<Q", f.read(8))[0]
        return n, json.loads(f.read(n))


def oracle_status(hdr, prefix, quant_method, block):
    w = hdr[prefix + ".weight"]
    si = hdr.get(prefix + ".weight_scale_inv")
    sc = hdr.get(prefix + ".weight_scale")
    T = lambda e: O.TensorDesc(e["dtype"], e["shape"])
    m = O.MemberDesc(T(w), T(si) if si else None, T(sc) if sc else None)
    return O.validate(quant_method, block, [m])


def check_against_oracle(path, units, quant_method="fp8", block=(128, 128)):
    n, hdr = header_of(path)
    for u in units:
        assert u["status"] == oracle_status(hdr, u["prefix"], quant_method, block), u["prefix"]
        assert u["weight_offset"] == 8 + n + hdr[u["prefix"] + ".weight"]["data_offsets"][0]


def test_good_tree_verifies_from_headers(tmp_path):
    p = write(tmp_path, "good.safetensors", tiny_tree())
    st, units = B.inspect_safetensors(p)
    assert st == "OK"
    by = {u["prefix"]: u for u in units}
    # dense BF16 tensors (norm, output head) keep their representation: not units
    assert set(by) == {"model.layers.0.self_attn.q_proj", "model.layers.0.mlp.down_proj"}
    d = by["model.layers.0.mlp.down_proj"]
    assert d["weight"] == dict(dtype="F8_E4M3", shape=(128, 256))
    assert d["scale_inv"] == dict(dtype="BF16", shape=(1, 2)) and d["scale"] is None
    assert O.scale_grid_shape(128, 256) == (1, 2)
    check_against_oracle(p, units)


def test_header_alone_is_enough(tmp_path):
    """A file cut right after its header (no tensor byte at all) inspects the same."""
    p = write(tmp_path, "good.safetensors", tiny_tree())
    n, _ = header_of(p)
    q = os.path.join(str(tmp_path), "header_only.safetensors")
    with open(p, "rb") as f, open(q, "wb") as g:
        g.write(f.read(8 + n))
    assert B.inspect_safetensors(q) == B.inspect_safetensors(p)


@pytest.mark.parametrize("name,over,expect,bad", [
    ("rowwise", {"model.layers.0.mlp.down_proj.weight_scale_inv": None,
                 "model.layers.0.mlp.down_proj.weight_scale": f32((128,))}, "SCALE_ROWWISE", "model.layers.0.mlp.down_proj"),
    ("transposed", {"model.layers.0.mlp.down_proj.weight_scale_inv": bf16((2, 1))}, "SCALE_TRANSPOSED",
     "model.layers.0.mlp.down_proj"),
    ("mis_blocked", {"model.layers.0.mlp.down_proj.weight_scale_inv": bf16((2, 4))}, "SCALE_GRID",
     "model.layers.0.mlp.down_proj"),
    ("no_scale", {"model.layers.0.mlp.down_proj.weight_scale_inv": None}, "SCALE_MISSING",
     "model.layers.0.mlp.down_proj"),
    ("e5m2", {"model.layers.0.self_attn.q_proj.weight": torch.zeros((256, 256), dtype=torch.float8_e5m2)},
     "WEIGHT_E5M2", "model.layers.0.self_attn.q_proj"),
    ("rank1_grid", {"model.layers.0.mlp.down_proj.weight_scale_inv": bf16((2,))}, "SCALE_ROWWISE",
     "model.layers.0.mlp.down_proj"),
])
def test_refusals_by_name(tmp_path, name, over, expect, bad):
    p = write(tmp_path, name + ".safetensors", tiny_tree(**over))
    st, units = B.inspect_safetensors(p)
    assert st == expect
    by = {u["prefix"]: u for u in units}
    assert by[bad]["status"] == expect
    assert all(u["status"] == "OK" for u in units if u["prefix"] != bad)
    check_against_oracle(p, units)


def test_dense_tree_is_refused(tmp_path):
    t = {"model.layers.0.mlp.down_proj.weight": bf16((128, 256)), "lm_head.weight": bf16((512, 256)),
         "model.norm.weight": bf16((256,))}
    p = write(tmp_path, "dense.safetensors", t)
    st, units = B.inspect_safetensors(p)
    assert st == "WEIGHT_DTYPE" and units == []


def test_per_tensor_tree(tmp_path):
    t = {"model.layers.0.mlp.down_proj.weight": f8((128, 256)), "model.layers.0.mlp.down_proj.weight_scale": f32(()),
         "model.layers.0.mlp.up_proj.weight": f8((256, 128)), "model.layers.0.mlp.up_proj.weight_scale": f32((1,))}
    p = write(tmp_path, "per_tensor.safetensors", t)
    st, units = B.inspect_safetensors(p, block=(0, 0))
    assert st == "OK" and len(units) == 2
    check_against_oracle(p, units, block=(0, 0))
    # under the 128x128 block declaration: a scalar scale is a per-tensor scale,
    # a one-element vector reads as a row-wise one; the first refusal is reported
    st, units = B.inspect_safetensors(p)
    assert st == "SCALE_PER_TENSOR"
    assert [u["status"] for u in units] == ["SCALE_PER_TENSOR", "SCALE_ROWWISE"]
    check_against_oracle(p, units)


def test_declaration_must_match(tmp_path):
    p = write(tmp_path, "good.safetensors", tiny_tree())
    st, units = B.inspect_safetensors(p, block=(64, 64))
    assert st == "DECL" and all(u["status"] == "DECL" for u in units)
    st, _ = B.inspect_safetensors(p, quant_method="int8")
    assert st == "DECL"


def test_malformed_files_raise(tmp_path):
    bad_json = os.path.join(str(tmp_path), "bad_json.safetensors")
    body = b'{"a": {"dtype": "F8_E4M3", "shape": [1, 2], "data_offsets": [0, 2]'
    with open(bad_json, "wb") as f:
        f.write(struct.pack("<Q", len(body)) + body)
    short = os.path.join(str(tmp_path), "short.safetensors")
    with open(short, "wb") as f:
        f.write(struct.pack("<Q", 1000) + b"{}")
    for path in (bad_json, short, os.path.join(str(tmp_path), "missing.safetensors")):
        with pytest.raises(B.BSF8Error) as e:
            B.inspect_safetensors(path)
        assert e.value.name == "INVALID_ARG"


@pytest.mark.parametrize("text,expect", [
    ('{"quantization_config": {"quant_method": "fp8", "weight_block_size": [128, 128], "activation_scheme": "dynamic"}}',
     ("fp8", (128, 128))),
    ('{"quant_method": "fp8", "weight_block_size": [128, 128]}', ("fp8", (128, 128))),
    ('{"quant_method": "fp8"}', ("fp8", (0, 0))),
    ('{"quant_method": "fp8", "weight_block_size": null}', ("fp8", (0, 0))),
    ('{"quant_method": "compressed-tensors", "weight_block_size": [128, 128]}', ("other", (128, 128))),
    ('{"hidden_size": 256, "quantization_config": {"quant_method": "fp8", "weight_block_size": [64, 128]}}',
     ("fp8", (64, 128))),
])
def test_quant_config(text, expect):
    assert B.parse_quant_config(text) == expect


@pytest.mark.parametrize("text,name", [
    ('{"weight_block_size": [128, 128]}', "DECL"),
    ('{"quant_method": "fp8", "weight_block_size": [128]}', "DECL"),
    ('{"quant_method": "fp8", "weight_block_size": [128, -1]}', "DECL"),
    ('[1, 2]', "INVALID_ARG"),
    ('{"quant_method": "fp8",', "INVALID_ARG"),
])
def test_quant_config_refusals(text, name):
    with pytest.raises(B.BSF8Error) as e:
        B.parse_quant_config(text)
    assert e.value.name == name


def _raw_file(tmp_path, name, header: dict, pad: int = 0):
    body = json.dumps(header).encode()
    p = os.path.join(str(tmp_path), name)
    with open(p, "wb") as f:
        f.write(struct.pack("<Q", len(body)) + body + b"\0" * pad)
    return p


GOOD_UNIT = {"down.weight": {"dtype": "F8_E4M3", "shape": [128, 256], "data_offsets": [0, 32768]},
             "down.weight_scale_inv": {"dtype": "BF16", "shape": [1, 2], "data_offsets": [32768, 32772]}}


@pytest.mark.parametrize("case,entry", [
    ("negative_begin", {"dtype": "F8_E4M3", "shape": [128, 256], "data_offsets": [-16, 32752]}),
    ("begin_after_end", {"dtype": "F8_E4M3", "shape": [128, 256], "data_offsets": [32768, 0]}),
    ("span_too_short", {"dtype": "F8_E4M3", "shape": [128, 256], "data_offsets": [0, 32767]}),
    ("span_too_long", {"dtype": "F8_E4M3", "shape": [128, 256], "data_offsets": [0, 65536]}),
    ("dimension_2_31", {"dtype": "F8_E4M3", "shape": [2 ** 31, 1], "data_offsets": [0, 2 ** 31]}),
    ("element_count_overflow", {"dtype": "F8_E4M3", "shape": [2 ** 31 - 1] * 3, "data_offsets": [0, 1]}),
    ("offset_above_int64", {"dtype": "F8_E4M3", "shape": [128, 256], "data_offsets": [0, 10 ** 20]}),
    ("dimension_above_int64", {"dtype": "F8_E4M3", "shape": [10 ** 19, 1], "data_offsets": [0, 1]}),
    ("offset_near_int64_max", {"dtype": "U8", "shape": [16],
                               "data_offsets": [2 ** 63 - 20, 2 ** 63 - 4]}),
])
def test_malformed_offsets_and_shapes_are_refused(tmp_path, case, entry):
    """data_offsets must satisfy 0 <= begin <= end with end - begin = numel x element size,
    every dimension must be an integer in [0, 2^31), and integers beyond int64 are not
    integers: each such header is refused as malformed (no offset is ever returned)."""
    hdr = dict(GOOD_UNIT)
    hdr["down.weight"] = entry
    p = _raw_file(tmp_path, f"{case}.safetensors", hdr)
    with pytest.raises(B.BSF8Error) as e:
        B.inspect_safetensors(p)
    assert e.value.name == "INVALID_ARG", e.value


def test_hand_written_header_verifies(tmp_path):
    """The same hand-written header with consistent offsets verifies and reports the offsets."""
    p = _raw_file(tmp_path, "ok.safetensors", GOOD_UNIT)
    st, units = B.inspect_safetensors(p)
    n = len(json.dumps(GOOD_UNIT).encode())
    assert st == "OK" and len(units) == 1
    assert units[0]["weight_offset"] == 8 + n and units[0]["scale_offset"] == 8 + n + 32768
    assert units[0]["weight"]["shape"] == (128, 256) and units[0]["scale_inv"]["shape"] == (1, 2)

"""Python binding of libbsf8, the block-scaled FP8 linear projection for MI355X.

Argument marshalling only: every step of the projection runs in the HIP
library (``libbsf8.so``, built by ``python -m block_scaled_fp8_linear_amd.build``).
PyTorch supplies device memory and the current stream.  There is no CPU path:
if the library is missing, importing works but every call raises.

Entry points mirror ``include/bsf8.h``:

* ``validate(...)``                     header-only geometry check, returns a status name
* ``BlockFP8Weight(members, ...)``      handle over borrowed device tensors
* ``quant_act(x)``                      per-token 1x128 E4M3 quantization -> (xq, xs)
* ``linear_w8a16(w, x)``                F32-activation arm
* ``linear_w8a8(w, xq, xs)``            FP8 x FP8 arm with F32 epilogue
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# BSF8_LIBRARY may name another build of the same library (the host-sanitized
# build the CPU tests run under); by default the in-tree libbsf8.so is loaded.
LIB_PATH = os.environ.get("BSF8_LIBRARY") or os.path.join(_HERE, "libbsf8.so")

DT_INVALID, DT_F8_E4M3, DT_F8_E5M2, DT_BF16, DT_F16, DT_F32, DT_U8, DT_OTHER = range(8)
ARM_W8A16, ARM_W8A8, ARM_DENSE, ARM_W8A8_DYNAMIC = 0, 1, 2, 3
DTYPE_NAMES = {"F8_E4M3": DT_F8_E4M3, "F8_E5M2": DT_F8_E5M2, "BF16": DT_BF16, "F16": DT_F16,
               "F32": DT_F32, "U8": DT_U8}
MAX_MEMBERS = 8
BLOCK = 128


class BSF8Error(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status, self.name, self.detail = status, name, detail


class TensorDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rank", ctypes.c_int32), ("shape", ctypes.c_int64 * 4),
                ("data", ctypes.c_void_p)]


class MemberDesc(ctypes.Structure):
    _fields_ = [("weight", TensorDesc), ("scale_inv", ctypes.POINTER(TensorDesc)),
                ("scale", ctypes.POINTER(TensorDesc))]


class Decl(ctypes.Structure):
    _fields_ = [("quant_method_fp8", ctypes.c_int32), ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32)]


class Unit(ctypes.Structure):
    _fields_ = [("prefix", ctypes.c_char * 256), ("prefix_truncated", ctypes.c_int32), ("status", ctypes.c_int32),
                ("weight", TensorDesc), ("scale_inv", TensorDesc), ("scale", TensorDesc),
                ("has_scale_inv", ctypes.c_int32), ("has_scale", ctypes.c_int32),
                ("weight_offset", ctypes.c_int64), ("scale_offset", ctypes.c_int64)]


_lib = None

# (name, restype, argtypes) of every entry point the header declares.
EXPORTS = [
    ("bsf8_abi_version", ctypes.c_int32, []),
    ("bsf8_status_name", ctypes.c_char_p, [ctypes.c_int]),
    ("bsf8_last_error", ctypes.c_char_p, []),
    ("bsf8_validate", ctypes.c_int, [ctypes.POINTER(Decl), ctypes.POINTER(MemberDesc), ctypes.c_int32]),
    ("bsf8_weight_create", ctypes.c_int, [ctypes.POINTER(Decl), ctypes.POINTER(MemberDesc), ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_void_p)]),
    ("bsf8_weight_destroy", None, [ctypes.c_void_p]),
    ("bsf8_weight_geometry", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                            ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]),
    ("bsf8_weight_scale_row", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    ("bsf8_quant_act", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    ("bsf8_workspace_size", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                           ctypes.POINTER(ctypes.c_size_t)]),
    ("bsf8_linear_w8a16", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("bsf8_linear_w8a8", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    ("bsf8_linear_w8a8_dynamic", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("bsf8_linear_w8a8_noalloc", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]),
    ("bsf8_describe", ctypes.c_char_p, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64]),
    ("bsf8_read_stream", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    ("bsf8_parse_quant_config", ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(Decl)]),
    ("bsf8_inspect_safetensors", ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(Decl), ctypes.POINTER(Unit),
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    ("bsf8_quant_glu", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    ("bsf8_glu_act", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    ("bsf8_upcast", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]),
    ("bsf8_dense_workspace_size", ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    ("bsf8_linear_dense", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
]


def lib() -> ctypes.CDLL:
    """Load libbsf8.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m block_scaled_fp8_linear_amd.build` "
                              "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in EXPORTS:
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_name(st: int) -> str:
    return lib().bsf8_status_name(st).decode()


def _check(st: int, what: str):
    if st != 0:
        raise BSF8Error(st, status_name(st), f"{what}: {lib().bsf8_last_error().decode()}")


def _tdesc(dtype, shape, addr) -> TensorDesc:
    d = TensorDesc()
    d.dtype = DTYPE_NAMES[dtype] if isinstance(dtype, str) else int(dtype)
    d.rank = len(shape)
    for i, s in enumerate(shape):
        d.shape[i] = int(s)
    d.data = int(addr) if addr else None
    return d


def _members_array(members: Sequence[dict]):
    """members: dicts with 'weight' (dtype, shape, addr) and optional 'scale_inv' / 'scale'."""
    keep = []
    arr = (MemberDesc * max(1, len(members)))()
    for i, m in enumerate(members):
        w = m["weight"]
        arr[i].weight = _tdesc(w["dtype"], w["shape"], w.get("addr"))
        for leaf in ("scale_inv", "scale"):
            s = m.get(leaf)
            if s is not None:
                d = _tdesc(s["dtype"], s["shape"], s.get("addr"))
                keep.append(d)
                setattr(arr[i], leaf, ctypes.pointer(d))
    return arr, keep


def _decl(quant_method: str = "fp8", block=(BLOCK, BLOCK)) -> Decl:
    d = Decl()
    d.quant_method_fp8 = 1 if quant_method == "fp8" else 0
    d.block_n, d.block_k = int(block[0]), int(block[1])
    return d


def validate(quant_method: str, block, members: Sequence[dict]) -> str:
    """Header-only validation (no device access); returns the status name."""
    decl = _decl(quant_method, block)
    arr, _keep = _members_array(members)
    return status_name(lib().bsf8_validate(ctypes.byref(decl), arr, len(members)))


# ------------------------------------------------------- checkpoint headers

_DT_NAME = {v: k for k, v in DTYPE_NAMES.items()}


def parse_quant_config(json_text: str) -> Tuple[str, Tuple[int, int]]:
    """(quant_method as 'fp8' or 'other', weight_block_size) from a config's JSON text;
    the block is (0, 0) when no weight_block_size is declared (per-tensor reading)."""
    d = Decl()
    _check(lib().bsf8_parse_quant_config(json_text.encode(), ctypes.byref(d)), "parse_quant_config")
    return ("fp8" if d.quant_method_fp8 else "other"), (d.block_n, d.block_k)


def _desc_dict(t: TensorDesc) -> dict:
    return dict(dtype=_DT_NAME.get(t.dtype, "OTHER"), shape=tuple(t.shape[i] for i in range(t.rank)))


def inspect_safetensors(path: str, quant_method: str = "fp8", block=(BLOCK, BLOCK)):
    """Header-only inspection of one safetensors file (no tensor byte is read).

    Returns (status name of the whole file, list of units); each unit is a dict
    with prefix, weight / scale_inv / scale descriptors, data offsets and its
    own status name."""
    L = lib()
    decl = _decl(quant_method, block)
    n = ctypes.c_int32()
    st = L.bsf8_inspect_safetensors(path.encode(), ctypes.byref(decl), None, 0, ctypes.byref(n))
    if status_name(st) == "INVALID_ARG":
        _check(st, "inspect_safetensors")
    units = (Unit * max(1, n.value))()
    st = L.bsf8_inspect_safetensors(path.encode(), ctypes.byref(decl), units, n.value, ctypes.byref(n))
    out = []
    for u in units[:n.value]:
        out.append(dict(prefix=u.prefix.decode(), status=status_name(u.status), weight=_desc_dict(u.weight),
                        scale_inv=_desc_dict(u.scale_inv) if u.has_scale_inv else None,
                        scale=_desc_dict(u.scale) if u.has_scale else None,
                        weight_offset=u.weight_offset, scale_offset=u.scale_offset))
    return status_name(st), out


# ------------------------------------------------------------------ torch glue

def _torch():
    import torch
    return torch


def _dt_of(t) -> int:
    torch = _torch()
    return {torch.float32: DT_F32, torch.bfloat16: DT_BF16, torch.float16: DT_F16, torch.uint8: DT_U8,
            torch.float8_e4m3fn: DT_F8_E4M3, torch.float8_e5m2: DT_F8_E5M2}.get(t.dtype, DT_OTHER)


def _on_device(device, **tensors):
    """Refuse, before any library call, a tensor that is not a GPU tensor on ``device``.

    The library takes raw device addresses: a host tensor's address would reach
    a kernel as if it were device memory, so every tensor argument is checked
    here (None entries are skipped)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (got one on {t.device})")
        if device is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _codes_dtype_ok(t) -> bool:
    torch = _torch()
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


class BlockFP8Weight:
    """Immutable handle over a (possibly grouped) block-FP8 weight on the GPU.

    ``members``: list of (weight, scale_inv) device tensors; weight is uint8 or
    float8_e4m3fn [N_i, K] (contiguous), scale_inv is bfloat16 or float32
    [ceil(N_i/128), ceil(K/128)] (contiguous).  With ``block=(0, 0)`` the
    weight is per-tensor scaled instead: each member's scale is its single
    ``weight_scale`` value (a 0-d or one-element tensor), read as one block that
    covers the whole member.  The tensors are borrowed: this object keeps
    references so they stay alive, and never modifies them.
    """

    def __init__(self, members: Sequence[Tuple[object, object]], quant_method: str = "fp8", block=(BLOCK, BLOCK)):
        L = lib()
        descs = []
        self._tensors = []
        leaf = "scale" if tuple(int(b) for b in block) == (0, 0) else "scale_inv"
        self.per_tensor = leaf == "scale"
        if len(members) == 0:
            raise ValueError("a weight needs at least one member")
        dev0 = members[0][0].device
        for i, (w, s) in enumerate(members):
            _on_device(dev0 if dev0.type == "cuda" else None, **{f"member {i} weight": w, f"member {i} scale": s})
            if not (w.is_contiguous() and s.is_contiguous()):
                raise ValueError("weights and scale grids must be contiguous")
            wdt = DT_F8_E4M3 if _dt_of(w) in (DT_U8, DT_F8_E4M3) else _dt_of(w)
            descs.append({"weight": dict(dtype=wdt, shape=tuple(w.shape), addr=w.data_ptr()),
                          leaf: dict(dtype=_dt_of(s), shape=tuple(s.shape), addr=s.data_ptr())})
            self._tensors += [w, s]
        decl = _decl(quant_method, block)
        arr, keep = _members_array(descs)
        h = ctypes.c_void_p()
        _check(L.bsf8_weight_create(ctypes.byref(decl), arr, len(descs), ctypes.byref(h)), "weight_create")
        self._h = h
        self.device = members[0][0].device
        n, k, nm = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(L.bsf8_weight_geometry(h, ctypes.byref(n), ctypes.byref(k), ctypes.byref(nm)), "geometry")
        self.n_total, self.K, self.n_members = n.value, k.value, nm.value
        self._ws: Dict[tuple, object] = {}

    @property
    def handle(self):
        return self._h

    @property
    def members(self):
        """The borrowed (weight, scale_inv) device tensors, in member order."""
        return [(self._tensors[i], self._tensors[i + 1]) for i in range(0, len(self._tensors), 2)]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.bsf8_weight_destroy(h)
            self._h = None

    def describe(self, arm: int, M: int) -> str:
        return lib().bsf8_describe(self._h, arm, M).decode()

    def scale_row(self, n: int) -> Tuple[int, int, int]:
        mi, lr, sr = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().bsf8_weight_scale_row(self._h, n, ctypes.byref(mi), ctypes.byref(lr), ctypes.byref(sr)),
               "scale_row")
        return mi.value, lr.value, sr.value

    def workspace_size(self, arm: int, M: int) -> int:
        b = ctypes.c_size_t()
        _check(lib().bsf8_workspace_size(self._h, arm, M, ctypes.byref(b)), "workspace_size")
        return b.value

    def workspace(self, arm: int, M: int):
        """A zero-filled device workspace, cached per stream and grown on demand."""
        torch = _torch()
        need = self.workspace_size(arm, M)
        if need == 0:
            return None, 0
        key = _stream_ptr(self.device)
        ws = self._ws.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws, ws.numel()


def _out(out, M, N, dtype, device):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=dtype, device=device)
    if out.dtype != dtype or out.dim() != 2 or out.shape[0] != M or out.shape[1] < N or out.stride(1) != 1:
        raise ValueError("out must be [M, >=N] with unit column stride and the requested dtype")
    return out


def scales_kmajor(M: int, Kb: int, device):
    """An uninitialised [M, Kb] float32 scale tensor in the K-major layout (token index
    contiguous: strides (1, M)), the layout the W8A8 product reads fastest."""
    torch = _torch()
    return torch.empty((Kb, M), dtype=torch.float32, device=device).t()


def quant_act(x, xq=None, xs=None):
    """Per-token 1x128 E4M3 quantization of x [M,K] (float32 or bfloat16) -> (xq uint8 [M,K], xs f32 [M,Kb]).
    xs may be any [M, Kb] float32 view in the token-major or the K-major layout; by default
    it is a new K-major one."""
    torch = _torch()
    _on_device(None, x=x)
    _on_device(x.device, xq=xq, xs=xs)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    Kb = -(-K // BLOCK)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = scales_kmajor(M, Kb, x.device)
    if tuple(xq.shape) != (M, K) or tuple(xs.shape) != (M, Kb) or xs.dtype != torch.float32:
        raise ValueError(f"xq must be [M, K] = [{M}, {K}] and xs float32 [M, Kb] = [{M}, {Kb}]")
    if not _codes_dtype_ok(xq) or xq.stride(1) != 1:
        raise ValueError("xq must be uint8 or float8_e4m3fn with unit column stride")
    _check(lib().bsf8_quant_act(x.data_ptr(), _dt_of(x), M, K, x.stride(0), xq.data_ptr(), xq.stride(0),
                                xs.data_ptr(), xs.stride(0), xs.stride(1), _stream_ptr(x.device)), "quant_act")
    return xq, xs


def quant_glu(y, xq=None, xs=None):
    """Gate/up output y [M, 2F] (gate then up; float32 or bfloat16) -> the down projection's
    quantized input for silu(gate) * up: (xq uint8 [M, F], xs f32 [M, ceil(F/128)]; xs as for quant_act)."""
    torch = _torch()
    _on_device(None, y=y)
    _on_device(y.device, xq=xq, xs=xs)
    if y.dim() != 2 or y.stride(1) != 1 or y.shape[1] % 2:
        raise ValueError("y must be 2-D with an even number of columns and unit column stride")
    M, F = y.shape[0], y.shape[1] // 2
    Fb = -(-F // BLOCK)
    if xq is None:
        xq = torch.empty((M, F), dtype=torch.uint8, device=y.device)
    if xs is None:
        xs = scales_kmajor(M, Fb, y.device)
    if tuple(xq.shape) != (M, F) or tuple(xs.shape) != (M, Fb) or xs.dtype != torch.float32:
        raise ValueError(f"xq must be [M, F] = [{M}, {F}] and xs float32 [M, Fb] = [{M}, {Fb}]")
    if not _codes_dtype_ok(xq) or xq.stride(1) != 1:
        raise ValueError("xq must be uint8 or float8_e4m3fn with unit column stride")
    _check(lib().bsf8_quant_glu(y.data_ptr(), _dt_of(y), M, F, y.stride(0), xq.data_ptr(), xq.stride(0),
                                xs.data_ptr(), xs.stride(0), xs.stride(1), _stream_ptr(y.device)), "quant_glu")
    return xq, xs


def glu_act(y, out=None):
    """Gate/up output y [M, 2F] (gate then up; float32 or bfloat16) -> h = silu(gate) * up as float32 [M, F],
    the same values quant_glu quantizes."""
    torch = _torch()
    _on_device(None, y=y)
    _on_device(y.device, out=out)
    if y.dim() != 2 or y.stride(1) != 1 or y.shape[1] % 2:
        raise ValueError("y must be 2-D with an even number of columns and unit column stride")
    M, F = y.shape[0], y.shape[1] // 2
    if out is None:
        out = torch.empty((M, F), dtype=torch.float32, device=y.device)
    if out.dtype != torch.float32 or out.dim() != 2 or tuple(out.shape) != (M, F) or out.stride(1) != 1:
        raise ValueError(f"out must be float32 [M, F] = [{M}, {F}] with unit column stride")
    _check(lib().bsf8_glu_act(y.data_ptr(), _dt_of(y), M, F, y.stride(0), out.data_ptr(), out.stride(0),
                              _stream_ptr(y.device)), "glu_act")
    return out


def linear_w8a16(w: BlockFP8Weight, x, out_dtype=None, out=None, workspace=None):
    """F32-activation arm: y [M, N] = x . dequant(W)^T (float32 output unless out_dtype says bfloat16)."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    _on_device(w.device, x=x, out=out, workspace=workspace[0] if workspace is not None else None)
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[1] != w.K:
        raise ValueError("x must be [M, K] with unit column stride")
    M = x.shape[0]
    y = _out(out, M, w.n_total, out_dtype, x.device)
    ws, wsb = workspace if workspace is not None else w.workspace(ARM_W8A16, M)
    _check(lib().bsf8_linear_w8a16(w.handle, x.data_ptr(), _dt_of(x), M, x.stride(0), y.data_ptr(), _dt_of(y),
                                   y.stride(0), ws.data_ptr() if ws is not None else None, wsb,
                                   _stream_ptr(x.device)), "linear_w8a16")
    return y


def linear_w8a8(w: BlockFP8Weight, xq, xs, out_dtype=None, out=None, workspace=None):
    """FP8 x FP8 arm with F32 epilogue: y [M, N] (bfloat16 output unless out_dtype says float32)."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _on_device(w.device, xq=xq, xs=xs, out=out, workspace=workspace[0] if workspace is not None else None)
    Kb = -(-w.K // BLOCK)
    if (xq.dim() != 2 or xq.shape[1] != w.K or xq.stride(1) != 1 or tuple(xs.shape) != (xq.shape[0], Kb)
            or xs.dtype != torch.float32):
        raise ValueError("xq must be [M, K] with unit column stride and xs float32 [M, ceil(K/128)]")
    if not _codes_dtype_ok(xq):
        raise ValueError("xq must be uint8 or float8_e4m3fn (the quantizer's E4M3 bytes)")
    M = xq.shape[0]
    y = _out(out, M, w.n_total, out_dtype, xq.device)
    ws, wsb = workspace if workspace is not None else w.workspace(ARM_W8A8, M)
    _check(lib().bsf8_linear_w8a8(w.handle, xq.data_ptr(), xq.stride(0), xs.data_ptr(), xs.stride(0), xs.stride(1), M,
                                  y.data_ptr(), _dt_of(y), y.stride(0),
                                  ws.data_ptr() if ws is not None else None, wsb, _stream_ptr(xq.device)),
           "linear_w8a8")
    return y


def linear_w8a8_dynamic(w: BlockFP8Weight, x, out_dtype=None, out=None, workspace=None):
    """W8A8 arm on unquantized activations: x (float32 or bfloat16 [M, K]) is quantized per
    token in 1x128 groups as quant_act does and multiplied as linear_w8a8 does, bit for bit,
    in one call (bfloat16 output unless out_dtype says float32).  One aligned token is
    quantized inside the weight-streaming kernels; more go through the workspace."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _on_device(w.device, x=x, out=out, workspace=workspace[0] if workspace is not None else None)
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[1] != w.K:
        raise ValueError("x must be [M, K] with unit column stride")
    M = x.shape[0]
    y = _out(out, M, w.n_total, out_dtype, x.device)
    ws, wsb = workspace if workspace is not None else w.workspace(ARM_W8A8_DYNAMIC, M)
    _check(lib().bsf8_linear_w8a8_dynamic(w.handle, x.data_ptr(), _dt_of(x), M, x.stride(0), y.data_ptr(),
                                          _dt_of(y), y.stride(0), ws.data_ptr() if ws is not None else None, wsb,
                                          _stream_ptr(x.device)), "linear_w8a8_dynamic")
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20   # BSF8_NOALLOC_SCRATCH_BYTES in include/bsf8.h


def linear_w8a8_noalloc(w: BlockFP8Weight, xq, xs, out):
    """linear_w8a8 for callers that cannot allocate: ``out`` (bfloat16 or float32 [M, >=N])
    must be given, and split-K partials go to the library's fixed per-device scratch
    instead of a workspace.  Calls that overlap in time on one device race."""
    torch = _torch()
    if out is None:
        raise ValueError("out must be given: the no-allocation call allocates nothing")
    _on_device(w.device, xq=xq, xs=xs, out=out)
    Kb = -(-w.K // BLOCK)
    if (xq.dim() != 2 or xq.shape[1] != w.K or xq.stride(1) != 1 or tuple(xs.shape) != (xq.shape[0], Kb)
            or xs.dtype != torch.float32):
        raise ValueError("xq must be [M, K] with unit column stride and xs float32 [M, ceil(K/128)]")
    if not _codes_dtype_ok(xq):
        raise ValueError("xq must be uint8 or float8_e4m3fn (the quantizer's E4M3 bytes)")
    M = xq.shape[0]
    y = _out(out, M, w.n_total, out.dtype, xq.device)
    _check(lib().bsf8_linear_w8a8_noalloc(w.handle, xq.data_ptr(), xq.stride(0), xs.data_ptr(), xs.stride(0),
                                          xs.stride(1), M, y.data_ptr(), _dt_of(y), y.stride(0),
                                          _stream_ptr(xq.device)), "linear_w8a8_noalloc")
    return y


def upcast(w: BlockFP8Weight, out_dtype=None, out=None):
    """Dense copy [N, K] of the weight (bfloat16 unless out_dtype says float32): the resident=False load step."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _on_device(w.device, out=out)
    if out is None:
        out = torch.empty((w.n_total, w.K), dtype=out_dtype, device=w.device)
    if out.dtype != out_dtype or out.dim() != 2 or out.shape[0] != w.n_total or out.shape[1] < w.K \
            or out.stride(1) != 1:
        raise ValueError("out must be [N, >=K] with unit column stride and the requested dtype")
    _check(lib().bsf8_upcast(w.handle, out.data_ptr(), _dt_of(out), out.stride(0), _stream_ptr(out.device)), "upcast")
    return out


def dense_workspace_size(N: int, K: int, M: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().bsf8_dense_workspace_size(N, K, M, ctypes.byref(b)), "dense_workspace_size")
    return b.value


def linear_dense(wd, x, out_dtype=None, out=None, workspace=None):
    """Dense arm: y [M, N] = x . wd^T for bfloat16 wd [N, K] (contiguous) and bfloat16 x [M, K]
    (float32 output unless out_dtype says bfloat16).  ``workspace``: a uint8 device tensor of at
    least dense_workspace_size bytes, allocated here when omitted."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    _on_device(None, wd=wd)
    _on_device(wd.device, x=x, out=out, workspace=workspace)
    if wd.dim() != 2 or not wd.is_contiguous() or wd.dtype != torch.bfloat16:
        raise ValueError("wd must be a contiguous bfloat16 [N, K] tensor")
    N, K = wd.shape
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[1] != K or x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16 [M, K] with unit column stride")
    M = x.shape[0]
    y = _out(out, M, N, out_dtype, x.device)
    need = dense_workspace_size(N, K, M)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib().bsf8_linear_dense(wd.data_ptr(), N, K, x.data_ptr(), M, x.stride(0), y.data_ptr(), _dt_of(y),
                                   y.stride(0), workspace.data_ptr() if workspace is not None else None,
                                   workspace.numel() if workspace is not None else 0, _stream_ptr(x.device)),
           "linear_dense")
    return y


__all__ = ["BSF8Error", "BlockFP8Weight", "validate", "quant_act", "quant_glu", "glu_act", "linear_w8a16", "linear_w8a8",
           "linear_w8a8_dynamic", "linear_w8a8_noalloc", "NOALLOC_SCRATCH_BYTES", "upcast",
           "linear_dense", "dense_workspace_size", "lib", "status_name", "ARM_W8A16", "ARM_W8A8", "ARM_DENSE",
           "ARM_W8A8_DYNAMIC",
           "EXPORTS", "LIB_PATH", "MAX_MEMBERS", "scales_kmajor"]


READ_STREAM_SINK_WORDS = 2048  # BSF8_READ_STREAM_SINK_WORDS in include/bsf8.h


def read_stream(buf, sink):
    """Measurement aid: a plain read of ``buf``'s bytes on the current stream.

    ``sink``: int32 device tensor of at least READ_STREAM_SINK_WORDS words; the
    launch overwrites its leading words with per-block XORs of what it read."""
    _on_device(None, buf=buf)
    _on_device(buf.device, sink=sink)
    if sink.numel() * sink.element_size() < 4 * READ_STREAM_SINK_WORDS:
        raise ValueError(f"read_stream sink needs {READ_STREAM_SINK_WORDS} 4-byte words")
    _check(lib().bsf8_read_stream(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                  _stream_ptr(buf.device)), "read_stream")

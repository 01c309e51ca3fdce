"""Every entry point captured into one HIP graph, replayed against eager results.

A serving loop records its calls once and replays them, so each kernel path
must give the same bits from a replay as from an eager call, also when the
state it shares (a split-K workspace, the no-allocation scratch) was written
by other calls in between.  One graph holds a call of every kernel family:
the W8A16 one-token, ring, few-token, general and LDS-staged GEMM kernels;
W8A8 through the one-token and few-token streaming kernels and the GEMM with
split-K partials; W8A8 on unquantized activations (quantized inside the
one-token kernel, or into the workspace before the W8A8 kernels); the quantizer, the
fused GLU quantizer and the activation alone; the upcast and the dense product.  Between replays the outputs are
overwritten and eager calls reuse the same workspace and scratch with other
inputs; after every replay each output must equal its eager bits.
"""
import pytest

import block_scaled_fp8_linear_amd as B
import synth
from gpu_util import banner, device, member_to_device, torch

pytestmark = pytest.mark.gpu

SEED = 240


def _weight(name, rows, K):
    m = synth.random_code_weight(SEED, name, rows, K)
    return B.BlockFP8Weight([member_to_device(m)])


def _x(name, M, K, dtype=None):
    t = torch()
    x = t.from_numpy(synth.gaussian_activations(SEED, name, M, K)).to(device())
    return x if dtype is None else x.to(dtype)


def _bits(y):
    t = torch()
    return y.view(t.int16) if y.element_size() == 2 else y.view(t.int32) if y.element_size() == 4 else y


def test_graph_of_every_kernel_family_replays_eager_bits():
    t = torch()
    d = device()
    w_a = _weight("graph_WA", 2048, 2048)      # decode-sized: one, three and seven tokens; split-K W8A8
    w_g = _weight("graph_WG", 4096, 1024)      # 16 row tiles x 8 token tiles at M = 512: the LDS-staged GEMM
    w_r = _weight("graph_WR", 512, 8192)       # eight chunks per wave at one token: the ring kernel
    w_s = _weight("graph_WS", 512, 768)        # six chunks: 40 tokens on the general kernel

    # (name, weight, M, arm): F32 activations; the W8A8 calls quantize their own x first
    calls = [("w8a16_m1", w_a, 1, B.ARM_W8A16), ("w8a16_m3", w_a, 3, B.ARM_W8A16), ("w8a16_m7", w_a, 7, B.ARM_W8A16),
             ("w8a16_m40", w_a, 40, B.ARM_W8A16), ("w8a16_general_m40", w_s, 40, B.ARM_W8A16),
             ("w8a16_gemm_m512", w_g, 512, B.ARM_W8A16),
             ("w8a16_ring_m1", w_r, 1, B.ARM_W8A16),
             ("w8a8_m1", w_a, 1, B.ARM_W8A8), ("w8a8_m3", w_a, 3, B.ARM_W8A8), ("w8a8_split_m64", w_a, 64, B.ARM_W8A8),
             ("w8a8_dyn_m1", w_a, 1, B.ARM_W8A8_DYNAMIC), ("w8a8_dyn_m3", w_a, 3, B.ARM_W8A8_DYNAMIC),
             ("w8a8_dyn_m64", w_a, 64, B.ARM_W8A8_DYNAMIC)]
    describes = {}
    state = {}
    for name, w, M, arm in calls:
        x = _x(f"graph_X_{name}", M, w.K)
        y = t.empty((M, w.n_total), dtype=t.float32 if arm == B.ARM_W8A16 else t.bfloat16, device=d)
        ws = w.workspace(arm, M)      # allocated before capture
        xq = xs = None
        if arm == B.ARM_W8A8:
            xq = t.empty((M, w.K), dtype=t.uint8, device=d)
            xs = B.scales_kmajor(M, -(-w.K // 128), d)
        state[name] = (w, M, arm, x, y, ws, xq, xs)
        describes[name] = w.describe(arm, M)
        banner(f"graph case {name}: {describes[name]}")
    joined = " ".join(describes.values())
    for kernel in ("kernel=w8a16_m1 ", "kernel=w8a16_m1_ring", "kernel=w8a16_small_m<e4m3>", "kernel=w8a16_small_m",
                   "kernel=w8a16_gemm ", "kernel=w8a16 rows=", "w8a16_m1<e4m3>", "kernel=w8a8_gemm_fast", "w8a16_m1<quantizing>",
                   "arm=w8a8-dynamic", "quant_act into the workspace"):
        assert kernel in joined, (kernel, describes)
    assert "split_k=1 " not in describes["w8a8_split_m64"], describes["w8a8_split_m64"]
    # the W8A16 GEMM split over K, with its reduction kernel, in the graph too
    assert "kernel=w8a16_gemm " in describes["w8a16_m40"] and "split_k=1 " not in describes["w8a16_m40"], \
        describes["w8a16_m40"]

    # the fused GLU step and the activation alone on a gate/up output [64, 2 x 640] (a ragged last group)
    yglu = _x("graph_Yglu", 64, 2 * 640, t.bfloat16)
    gq = t.empty((64, 640), dtype=t.uint8, device=d)
    gs = B.scales_kmajor(64, 5, d)
    gh = t.empty((64, 640), dtype=t.float32, device=d)
    # the dense arm: the upcast copy of w_a and the BF16 product at M = 16 (split over K)
    wd = t.empty((w_a.n_total, w_a.K), dtype=t.bfloat16, device=d)
    xd = _x("graph_Xdense", 16, w_a.K, t.bfloat16)
    yd = t.empty((16, w_a.n_total), dtype=t.float32, device=d)
    dws = t.empty(max(1, B.dense_workspace_size(w_a.n_total, w_a.K, 16)), dtype=t.uint8, device=d)
    # the no-allocation entry point (split-K partials in the library's scratch)
    na = state["w8a8_split_m64"]
    yna = t.empty_like(na[4])

    def run_all():
        for name, (w, M, arm, x, y, ws, xq, xs) in state.items():
            if arm == B.ARM_W8A16:
                B.linear_w8a16(w, x, out=y, workspace=ws)
            elif arm == B.ARM_W8A8_DYNAMIC:
                B.linear_w8a8_dynamic(w, x, out=y, workspace=ws)
            else:
                B.quant_act(x, xq, xs)
                B.linear_w8a8(w, xq, xs, out=y, workspace=ws)
        B.quant_glu(yglu, gq, gs)
        B.glu_act(yglu, out=gh)
        B.upcast(w_a, out=wd)
        B.linear_dense(wd, xd, out=yd, workspace=dws)
        B.linear_w8a8_noalloc(na[0], na[6], na[7], out=yna)

    def outputs():
        outs = {name: s[4] for name, s in state.items()}
        outs.update({f"{n}_xq": s[6] for n, s in state.items() if s[6] is not None})
        outs.update({f"{n}_xs": s[7] for n, s in state.items() if s[7] is not None})
        outs.update(glu_q=gq, glu_s=gs, glu_h=gh, upcast=wd, dense=yd, noalloc=yna)
        return outs

    banner("graph: eager reference")
    run_all()
    t.cuda.synchronize()
    ref = {k: _bits(v).clone() for k, v in outputs().items()}
    assert t.equal(_bits(yna), _bits(na[4])), "no-allocation and workspace W8A8 differ"

    banner("graph: capture")
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        run_all()

    # eager calls between replays that rewrite the shared state with other inputs
    other_x = _x("graph_X_other", 64, w_a.K)
    other_q, other_s = B.quant_act(other_x)
    other_y = t.empty_like(na[4])
    for rep in range(3):
        for v in outputs().values():
            v.fill_(3)
        B.linear_w8a8(w_a, other_q, other_s, out=other_y, workspace=na[5])
        B.linear_w8a8_noalloc(w_a, other_q, other_s, out=other_y)
        t.cuda.synchronize()
        banner(f"graph: replay {rep}")
        g.replay()
        t.cuda.synchronize()
        for k, v in outputs().items():
            assert t.equal(_bits(v), ref[k]), (rep, k)

"""Seeded synthetic inputs for the block-scaled FP8 linear projection.

This module is shared by the parity tests, the bench and the oracle's timing
leg.  It holds no arithmetic of the projection itself: it draws random numbers
(NumPy ``Generator(PCG64)``) and, where a workload needs a block-FP8
checkpoint, it plays the part of the ahead-of-time checkpoint converter using
PyTorch's own ``bfloat16`` and ``float8_e4m3fn`` casts.  The pages place weight
quantization outside the load/compute path (python-gen-worker PR "th#1803 ...
hf.fp8-blockwise@1", section "Why the refusals matter more than the load": no
quantization at load, conversion happens ahead of time), so neither the oracle
nor the HIP kernels take part in making these inputs.

Every tensor is drawn from its own child of ``SeedSequence(20260000 + config)``
keyed by a stable tensor name, so any tensor can be regenerated on its own.

Workloads (synthetic stand-ins for the pages' Qwen-class projections):

* config 1, tiny: W [128,256] codes uniform over the 254 finite E4M3 codes,
  BF16 scales 2^u with u ~ U(-10,-4), X [8,256] N(0,1).
* config 2, decode GEMV: W [5120,5120] and [5000,4000] from BF16 N(0,0.02)
  quantized per 128x128 block (scale = amax/448); X N(0,1) with 1% of the
  channels multiplied by 20; M in {1,4,8}.
* config 3, dense-FFN prefill: M=1024, gate/up = two members of 17408 rows
  (K=5120), down = [5120,17408]; X as in config 2.
* config 4, grouped QKV: members Q [6144,5120], K [1000,5120], V [1000,5120],
  each on its own ceil-divided grid; M in {1,512}.
* config 5, large prefill: M=8192, K=7168, N=18432; per-block weight gain
  LogNormal(0, 1.5); per-token activation magnitude 10^U(-2,2).
"""
from __future__ import annotations

import hashlib
import zlib
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

BLOCK = 128
E4M3_MAX = 448.0

# Shapes of the five workloads.  Members are (rows, K).
CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny", members=[(128, 256)], M=[8]),
    2: dict(name="decode_gemv", members=[(5120, 5120)], alt_members=[(5000, 4000)], M=[1, 4, 8]),
    3: dict(name="dense_ffn_prefill", gate_up=[(17408, 5120), (17408, 5120)],
            down=[(5120, 17408)], M=[1024]),
    4: dict(name="grouped_qkv", members=[(6144, 5120), (1000, 5120), (1000, 5120)], M=[1, 512]),
    5: dict(name="large_prefill", members=[(18432, 7168)], M=[8192]),
}


def rng_for(config: int, tensor: str) -> np.random.Generator:
    """Independent PCG64 stream for ``tensor`` of ``config``.

    The child index is a CRC32 of the tensor name, so adding a tensor never
    shifts the stream of another.
    """
    ss = np.random.SeedSequence(20260000 + int(config))
    child = np.random.SeedSequence(entropy=ss.entropy, spawn_key=(zlib.crc32(tensor.encode()),))
    return np.random.Generator(np.random.PCG64(child))


# ---------------------------------------------------------------- activations

def gaussian_activations(config: int, tensor: str, M: int, K: int,
                         outlier_frac: float = 0.01, outlier_gain: float = 20.0) -> np.ndarray:
    """X [M,K] float32 ~ N(0,1); ceil(frac*K) fixed channels multiplied by ``gain``.

    The outlier channels are the same for every token (a seeded permutation of
    the K channels), which is the structure transformer activations show.
    """
    g = rng_for(config, tensor)
    x = g.standard_normal((M, K), dtype=np.float32)
    n_out = int(np.ceil(outlier_frac * K)) if outlier_frac > 0 else 0
    if n_out:
        cols = rng_for(config, tensor + "/outlier_channels").permutation(K)[:n_out]
        x[:, cols] *= np.float32(outlier_gain)
    return x


def spread_activations(config: int, tensor: str, M: int, K: int,
                       lo: float = -2.0, hi: float = 2.0) -> np.ndarray:
    """X [M,K] float32: token m is 10^{u_m} N(0,1), u_m ~ U(lo,hi)."""
    g = rng_for(config, tensor)
    x = g.standard_normal((M, K), dtype=np.float32)
    u = rng_for(config, tensor + "/token_gain").uniform(lo, hi, size=(M, 1))
    return (x * np.power(10.0, u)).astype(np.float32)


# -------------------------------------------------------------------- weights

@dataclass
class BlockFP8Member:
    """One member of a (possibly grouped) block-FP8 weight, as a checkpoint stores it."""
    codes: np.ndarray            # uint8 [N,K], E4M3 bit patterns
    scale_bits: np.ndarray       # uint16 [ceil(N/128), ceil(K/128)] BF16 bit patterns
    source: Optional[np.ndarray] = None  # float32 [N,K] pre-quantization values, when kept

    @property
    def shape(self):
        return self.codes.shape

    def scale_f32(self) -> np.ndarray:
        """BF16 scale bits widened to float32 (bits << 16; exact)."""
        return (self.scale_bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_round_torch(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (RNE) -> float32, using PyTorch's cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def convert_checkpoint(w: np.ndarray, keep_source: bool = False) -> BlockFP8Member:
    """Ahead-of-time block-FP8 conversion of a float32 weight, as a converter would do it.

    Per 128x128 block (partial at the tails): scale = bf16(amax/448); codes =
    fp8_e4m3fn(clip(w/scale, +-448)) with PyTorch's casts; an all-zero block
    gets scale 0 and zero codes.  Runs in row bands to bound memory.
    """
    import torch
    N, K = w.shape
    Nb, Kb = -(-N // BLOCK), -(-K // BLOCK)
    codes = np.empty((N, K), np.uint8)
    sbits = np.empty((Nb, Kb), np.uint16)
    Kp = Kb * BLOCK
    for rb in range(Nb):
        r0, r1 = rb * BLOCK, min(N, rb * BLOCK + BLOCK)
        band = torch.from_numpy(np.ascontiguousarray(w[r0:r1], dtype=np.float32))
        if Kp != K:
            band_p = torch.zeros((r1 - r0, Kp), dtype=torch.float32)
            band_p[:, :K] = band
        else:
            band_p = band
        amax = band_p.abs().view(r1 - r0, Kb, BLOCK).amax(dim=(0, 2))           # [Kb]
        s = (amax / E4M3_MAX).to(torch.bfloat16)                               # [Kb] bf16
        sbits[rb] = s.view(torch.int16).numpy().view(np.uint16)
        s32 = s.to(torch.float32)
        safe = torch.where(s32 > 0, s32, torch.ones_like(s32))
        q = (band_p.view(r1 - r0, Kb, BLOCK) / safe[None, :, None]).clamp(-E4M3_MAX, E4M3_MAX)
        q = torch.where((s32 > 0)[None, :, None], q, torch.zeros_like(q))
        codes[r0:r1] = q.view(r1 - r0, Kp)[:, :K].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return BlockFP8Member(codes=codes, scale_bits=sbits, source=(w if keep_source else None))


def gaussian_weight(config: int, tensor: str, N: int, K: int, std: float = 0.02,
                    keep_source: bool = False) -> BlockFP8Member:
    """BF16 N(0,std) source weight, block-quantized (configs 2-4)."""
    g = rng_for(config, tensor)
    w = _bf16_round_torch(g.standard_normal((N, K), dtype=np.float32) * np.float32(std))
    return convert_checkpoint(w, keep_source=keep_source)


def heavy_tailed_weight(config: int, tensor: str, N: int, K: int, std: float = 0.02,
                        sigma: float = 1.5, keep_source: bool = False) -> BlockFP8Member:
    """Source 0.02 * g_b * N(0,1) with a LogNormal(0, sigma^2) gain per 128x128 block (config 5)."""
    g = rng_for(config, tensor)
    Nb, Kb = -(-N // BLOCK), -(-K // BLOCK)
    gain = rng_for(config, tensor + "/block_gain").lognormal(0.0, sigma, size=(Nb, Kb)).astype(np.float32)
    w = np.empty((N, K), np.float32)
    for rb in range(Nb):
        r0, r1 = rb * BLOCK, min(N, rb * BLOCK + BLOCK)
        band = g.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(std)
        band *= np.repeat(gain[rb], BLOCK)[:K][None, :]
        w[r0:r1] = band
    w = _bf16_round_torch(w)
    return convert_checkpoint(w, keep_source=keep_source)


def uniform_code_weight(config: int, tensor: str, N: int, K: int,
                        log2_lo: float = -10.0, log2_hi: float = -4.0) -> BlockFP8Member:
    """Codes uniform over the 254 finite E4M3 patterns; BF16 scales 2^u, u ~ U(lo,hi) (config 1)."""
    g = rng_for(config, tensor)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = finite[g.integers(0, finite.size, size=(N, K))]
    Nb, Kb = -(-N // BLOCK), -(-K // BLOCK)
    u = rng_for(config, tensor + "/scales").uniform(log2_lo, log2_hi, size=(Nb, Kb)).astype(np.float32)
    sbits = _bf16_bits_torch(np.exp2(u).astype(np.float32))
    return BlockFP8Member(codes=codes, scale_bits=sbits)


def random_code_weight(config: int, tensor: str, N: int, K: int, scale_log2: Sequence[float] = (-10.0, -4.0),
                       positive_only: bool = False, finite_only: bool = True) -> BlockFP8Member:
    """Random codes (optionally only positive ones) with log-uniform BF16 scales; for edge fixtures."""
    g = rng_for(config, tensor)
    pool = [c for c in range(256) if not (finite_only and c in (0x7F, 0xFF))]
    if positive_only:
        pool = [c for c in pool if c < 0x80 and c != 0]
    pool = np.array(pool, np.uint8)
    codes = pool[g.integers(0, pool.size, size=(N, K))]
    Nb, Kb = -(-N // BLOCK), -(-K // BLOCK)
    u = rng_for(config, tensor + "/scales").uniform(scale_log2[0], scale_log2[1], size=(Nb, Kb)).astype(np.float32)
    sbits = _bf16_bits_torch(np.exp2(u).astype(np.float32))
    return BlockFP8Member(codes=codes, scale_bits=sbits)


# ------------------------------------------------------------------ workloads

@dataclass
class Workload:
    name: str
    members: List[BlockFP8Member]
    x: np.ndarray                              # float32 [M,K]
    meta: dict = field(default_factory=dict)

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return sum(m.codes.shape[0] for m in self.members)


def config1() -> Workload:
    w = uniform_code_weight(1, "W", 128, 256)
    x = gaussian_activations(1, "X", 8, 256, outlier_frac=0.0)
    return Workload("tiny_128x256_m8", [w], x)


def config2(M: int, shape=(5120, 5120)) -> Workload:
    N, K = shape
    w = gaussian_weight(2, f"W{N}x{K}", N, K)
    x = gaussian_activations(2, f"X{K}", 8, K)[:M].copy()
    return Workload(f"decode_gemv_{N}x{K}_m{M}", [w], x)


def config3_gate_up(M: int = 1024) -> Workload:
    g = gaussian_weight(3, "W_gate", 17408, 5120)
    u = gaussian_weight(3, "W_up", 17408, 5120)
    x = gaussian_activations(3, "X_gate_up", M, 5120)
    return Workload(f"ffn_gate_up_m{M}", [g, u], x)


def config3_down(M: int = 1024) -> Workload:
    d = gaussian_weight(3, "W_down", 5120, 17408)
    x = gaussian_activations(3, "X_down", M, 17408)
    return Workload(f"ffn_down_m{M}", [d], x)


def config4(M: int) -> Workload:
    q = gaussian_weight(4, "W_q", 6144, 5120)
    k = gaussian_weight(4, "W_k", 1000, 5120)
    v = gaussian_weight(4, "W_v", 1000, 5120)
    x = gaussian_activations(4, "X", 512, 5120)[:M].copy()
    return Workload(f"grouped_qkv_m{M}", [q, k, v], x)


def config5(M: int = 8192) -> Workload:
    w = heavy_tailed_weight(5, "W", 18432, 7168)
    x = spread_activations(5, "X", M, 7168)
    return Workload(f"large_prefill_m{M}", [w], x)


def sha256_of(*arrays: np.ndarray) -> str:
    """Fixture hash: sha256 over the raw bytes of each array in order."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()

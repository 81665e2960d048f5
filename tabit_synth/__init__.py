"""Seeded synthetic inputs and workload tables for the timestep-adaptive-bit linear.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds random draws, shape tables and bit reinterpretation only:
no step of the method's arithmetic (no rotation, quantization, masking or
GEMM) lives here, so the oracle and the HIP path stay independent.

Workload shapes follow the diffusion transformers the TASQ pages evaluate on
(PixArt-Sigma, SANA-1.6B, SDXL-Turbo; TASQ gist.science summary, section 4
"Resultados Experimentais") and the CogVideoX-2B video DiT of 6Bit-Diffusion
(gist.science summary, section 4).  No checkpoint or dataset is used: weights
and activations are drawn from fixed seeds with the distributions stated in
each config below.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np
import torch

FMT_INT8 = 0
FMT_MXFP4 = 1

# Outlier channels: 8 input-channel indices from a seeded permutation, scaled
# x20 for every token before the bf16 cast ("long-tailed with prominent
# outliers": HQ-DM gist.science summary, section 1).
OUTLIER_SEED = 7
N_OUTLIERS = 8
OUTLIER_GAIN = 20.0
WEIGHT_STD = 0.02


# --------------------------------------------------------------------------
# bit plumbing
# --------------------------------------------------------------------------
def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a CPU bfloat16 tensor (no arithmetic)."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(u: np.ndarray) -> torch.Tensor:
    """Inverse of :func:`bf16_bits`."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16)


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------
def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def outlier_channels(K: int) -> np.ndarray:
    return np.sort(_rng(OUTLIER_SEED).permutation(K)[: min(N_OUTLIERS, K)])


def gen_activation(M: int, K: int, seed: int, sigma: float = 1.0,
                   outliers: bool = True) -> torch.Tensor:
    """X ~ N(0, sigma^2) in fp32, outlier channels x20, cast to bf16 (CPU)."""
    x = _rng(seed).standard_normal((M, K), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if outliers and M > 0:
        x[:, outlier_channels(K)] *= np.float32(OUTLIER_GAIN)
    return torch.from_numpy(x).to(torch.bfloat16)


def gen_weight(N: int, K: int, seed: int, std: float = WEIGHT_STD) -> torch.Tensor:
    """W ~ N(0, std^2) in fp32, cast to bf16 (CPU).  nn.Linear layout [N, K]."""
    w = _rng(10_000 + seed).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return torch.from_numpy(w).to(torch.bfloat16)


def gen_int8(shape: Tuple[int, ...], seed: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Uniform int8 codes in [lo, hi] (for direct GEMM tests)."""
    return _rng(seed).integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int8)


def gen_scales(n: int, seed: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    """Positive fp32 scales, log-uniform in [lo, hi]."""
    u = _rng(seed).random(n)
    return np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.float32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    M: int       # tokens
    N: int       # output features
    K: int       # input features


@dataclasses.dataclass
class Workload:
    name: str
    layers: List[Layer]          # one entry per linear, in execution order
    steps: int                   # denoising steps T
    had_block: int               # block Hadamard size b (0 = no rotation)
    k_bits: np.ndarray           # uint8 [T, L]
    fmt: np.ndarray              # uint8 [T, L]

    @property
    def num_layers(self) -> int:
        return len(self.layers)

    def ops_per_schedule(self) -> int:
        return int(sum(2 * l.M * l.N * l.K for l in self.layers)) * self.steps


def _blocks(M: int, block_shapes, n_blocks: int, prefix: str) -> List[Layer]:
    out = []
    for bi in range(n_blocks):
        for lname, (N, K) in block_shapes:
            out.append(Layer(f"{prefix}{bi}.{lname}", M, N, K))
    return out


def c1_single_linear() -> Workload:
    """64 tokens x 1152, one 1152x1152 linear, b=64, 4 steps k=[0,2,4,3]."""
    layers = [Layer("lin", 64, 1152, 1152)]
    k = np.array([[0], [2], [4], [3]], dtype=np.uint8)
    return Workload("single_linear_64x1152x1152", layers, 4, 64, k, np.zeros_like(k))


def c2_pixart_sigma(had_block: int = 0) -> Workload:
    """PixArt-Sigma-shaped stack: 28 blocks, hidden 1152, 4096 tokens, 20 steps.

    k drawn per (layer, step): k = 0 with probability p0(t) = 0.9 - 0.8 t/(T-1),
    else uniform on {1..4}; seed 20 (early steps biased to full precision).
    """
    shapes = [("qkv", (3456, 1152)), ("out", (1152, 1152)),
              ("mlp_up", (4608, 1152)), ("mlp_down", (1152, 4608))]
    layers = _blocks(4096, shapes, 28, "blk")
    T, L = 20, len(layers)
    rng = _rng(20)
    k = np.zeros((T, L), dtype=np.uint8)
    for t in range(T):
        p0 = 0.9 - 0.8 * t / (T - 1)
        u = rng.random(L)
        draw = rng.integers(1, 5, size=L)
        k[t] = np.where(u < p0, 0, draw).astype(np.uint8)
    return Workload("pixart_sigma_28x1152_tok4096_T20", layers, T, had_block, k,
                    np.zeros_like(k))


def c3_sana(had_block: int = 0) -> Workload:
    """SANA-1.6B-shaped stack: 20 blocks, hidden 2240, 1024 tokens, 20 steps, k~U{0..5} seed 30."""
    shapes = [("qkv", (6720, 2240)), ("out", (2240, 2240)),
              ("mlp_up", (5600, 2240)), ("mlp_down", (2240, 5600))]
    layers = _blocks(1024, shapes, 20, "blk")
    T, L = 20, len(layers)
    k = _rng(30).integers(0, 6, size=(T, L)).astype(np.uint8)
    return Workload("sana_20x2240_tok1024_T20", layers, T, had_block, k, np.zeros_like(k))


def c4_sdxl_turbo(had_block: int = 0) -> Workload:
    """SDXL-Turbo-shaped UNet transformer linears, batch 4.

    Stage h640: 16384 tokens (4 x 4096); stage h1280: 4096 tokens (4 x 1024);
    10 transformer blocks per stage; QKV h->3h, out h->h, GEGLU up h->8h
    (value and gate fused), down 4h->h.  4 steps, k = t for every layer.
    """
    s640 = [("qkv", (1920, 640)), ("out", (640, 640)),
            ("geglu_up", (5120, 640)), ("down", (640, 2560))]
    s1280 = [("qkv", (3840, 1280)), ("out", (1280, 1280)),
             ("geglu_up", (10240, 1280)), ("down", (1280, 5120))]
    layers = _blocks(16384, s640, 10, "h640.blk") + _blocks(4096, s1280, 10, "h1280.blk")
    T, L = 4, len(layers)
    k = np.repeat(np.arange(T, dtype=np.uint8)[:, None], L, axis=1)
    return Workload("sdxl_turbo_unet_b4_T4", layers, T, had_block, k, np.zeros_like(k))


def c5_cogvideox(had_block: int = 32) -> Workload:
    """CogVideoX-2B-shaped video DiT: 30 blocks, hidden 1920, 17550+226 tokens, 50 steps.

    fmt = MXFP4 with probability 0.6 per (layer, step), seed 50; INT8 layer-steps
    use k = 0.  Block Hadamard b = 32 on every layer.
    """
    shapes = [("qkv", (5760, 1920)), ("out", (1920, 1920)),
              ("mlp_up", (7680, 1920)), ("mlp_down", (1920, 7680))]
    layers = _blocks(17550 + 226, shapes, 30, "blk")
    T, L = 50, len(layers)
    fmt = (_rng(50).random((T, L)) < 0.6).astype(np.uint8)
    return Workload("cogvideox2b_30x1920_tok17776_T50", layers, T, had_block,
                    np.zeros((T, L), dtype=np.uint8), fmt)


# Block input/output pairs for the online INT8 / 4-bit selector: out = in +
# delta * noise * mean|in| per row.  A small pool of deltas stands for stable
# (small) and unstable (large) blocks; each (step, block) draws one pair.
DMPQ_DELTAS = (0.02, 0.05, 0.4, 0.8)
DMPQ_POOL_P = (0.3, 0.3, 0.2, 0.2)


def gen_block_io(M: int, H: int, seed: int, delta: float) -> Tuple[torch.Tensor, torch.Tensor]:
    """Seeded bf16 block input and output [M][H]."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, H, generator=g)
    y = x + delta * torch.randn(M, H, generator=g) * x.abs().mean(dim=1, keepdim=True)
    return x.to(torch.bfloat16), y.to(torch.bfloat16)


def dmpq_pool_draws(steps: int, blocks: int, seed: int = 70) -> np.ndarray:
    """Index into DMPQ_DELTAS per (step, block), int [steps][blocks]."""
    return _rng(seed).choice(len(DMPQ_DELTAS), size=(steps, blocks), p=DMPQ_POOL_P)


WORKLOADS = {
    "c1": c1_single_linear,
    "c2": c2_pixart_sigma,
    "c3": c3_sana,
    "c4": c4_sdxl_turbo,
    "c5": c5_cogvideox,
}


def activation_seed(step: int, K: int) -> int:
    """One activation tensor per distinct (M, K) per step."""
    return 1000 * step + K

"""CPU oracle for the timestep-adaptive-bit quantized linear.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
module.  The product path (the C-ABI library and its Python binding) never
calls it and shares no code with it.

Plain, slow, obviously-correct numpy.  Integer work is exact (int64).  The
quantizers take their rounding decisions in IEEE fp32, the precision the
kernels decide codes in, so codes and scales are expected bit-exact; the
dequantized outputs are evaluated in fp64 and compared within a tolerance.
Two next-row steps are plain definitions evaluated more precisely than any
kernel does: the GELU folded into the down projection's quantizer (fp64,
rounded once to bf16) and DMPQ's relative L1 change (exactly rounded sums);
the tests compare the kernels with them within stated error bounds.

Sources (web pages; section names as the pages print them):
  * TASQ: Temporal-Adaptive Bit Sparsification Quantization for Diffusion
    Models -- gist.science technical summary, section 2 "Metodologia"
    (shared weight buffer, LSB mask, truncation equation, Temporal-Precision
    Engine) and the newx.sg abstract.
  * HQ-DM: Single Hadamard Transformation-Based QAT -- gist.science technical
    summary, section 2.1 (block-diagonal Hadamard on activations, recovery by
    orthogonality, normalization folded into the fp scales) and 2.2
    (symmetric quantization).
  * 6Bit-Diffusion -- gist.science technical summary, section 2A (DMPQ:
    INT8 vs 4-bit per layer-step, local block Hadamard before quantization).
  * The 4-bit format is OCP Microscaling (MX) v1.0 MXFP4 (E2M1 elements,
    E8M0 shared scale per 32 elements) -- the public OCP specification, the
    gfx950-native stand-in for the NVFP4 format the 6Bit-Diffusion page names.

Every function says which passage it follows.  Readings where the pages are
silent or garbled are stated inline.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

# --------------------------------------------------------------------------
# bf16 <-> fp32 (plumbing for bf16 inputs and outputs)
# --------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs).

    Keeps the upper 16 bits of the fp32 pattern and rounds on the 16 dropped
    bits: up if they exceed half, and on an exact half only if the kept part
    is odd.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == 1))
    return (upper + round_up.astype(np.uint64)).astype(np.uint16)


# --------------------------------------------------------------------------
# O1, O2: Sylvester Hadamard and the block fast Walsh-Hadamard transform
# --------------------------------------------------------------------------


def sylvester_hadamard(n: int) -> np.ndarray:
    """Standard (Sylvester) Hadamard matrix H_n with entries +-1, n a power of two.

    HQ-DM (gist.science summary, section 2.1, "Mecanismo"): the rotation is a
    block-diagonal matrix built from standard Hadamard matrices H_k.  Built by
    the doubling recursion H_{2n} = [[H_n, H_n], [H_n, -H_n]] starting from
    H_1 = [1].  Unnormalized: H H^T = n I.
    """
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard size must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def block_fwht_f32(v: np.ndarray, b: int) -> np.ndarray:
    """Unnormalized block Walsh-Hadamard transform along the last axis, in fp32.

    HQ-DM section 2.1: activations are multiplied by a block-diagonal H built
    from H_b; the normalization 2^{-k/2} is taken out of the transform and
    folded into the floating-point scales, so the transform itself uses +-1
    entries only.  6Bit-Diffusion section 2A applies the same local block
    transform before 4-bit quantization.

    Each contiguous block of b elements is transformed independently.  Stages
    run with half-width h = 1, 2, 4, ..., b/2; a stage replaces every pair
    (v[i+j], v[i+j+h]) inside each group of 2h elements by their sum and
    difference.  All additions are fp32 (numpy float32 arithmetic is IEEE
    round-to-nearest-even), and this stage order is the contract that makes
    the result reproducible bit-for-bit.  b = 0 means no rotation.
    """
    x = np.array(v, dtype=np.float32, copy=True)
    if b == 0:
        return x
    if b & (b - 1) or b < 2:
        raise ValueError("block size must be a power of two >= 2 (or 0)")
    shape = x.shape
    K = shape[-1]
    if K % b:
        raise ValueError("row length must be a multiple of the block size")
    rows = int(np.prod(shape[:-1], dtype=np.int64)) if len(shape) > 1 else 1
    y = x.reshape(rows, K // b, b)
    h = 1
    while h < b:
        g = y.reshape(rows, K // b, b // (2 * h), 2, h)
        first = g[:, :, :, 0, :]
        second = g[:, :, :, 1, :]
        s = first + second          # fp32 add
        d = first - second          # fp32 subtract
        y = np.stack([s, d], axis=3).reshape(rows, K // b, b)
        h *= 2
    return y.reshape(shape)


# --------------------------------------------------------------------------
# O3, O4: per-row symmetric INT8 quantization
# --------------------------------------------------------------------------


def _absmax_int8_codes(y: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row absmax INT8 codes of fp32 rows y.

    Reading (the pages fix neither the scale nor the rounding): the row's
    largest magnitude a maps to 127; one fp32 division r = 127/a per row,
    then each element is multiplied by r in fp32, rounded half-to-even to an
    integer and clamped to [-127, 127].  The scale returned is a/127 (fp32).
    A zero row gives zero codes and scale 0.  HQ-DM section 2.2: symmetric
    quantization.
    """
    y = np.asarray(y, dtype=np.float32)
    M = y.shape[0]
    a = np.max(np.abs(y), axis=1).astype(np.float32) if y.shape[1] else np.zeros(M, np.float32)
    q = np.zeros(y.shape, dtype=np.int8)
    s = np.zeros(M, dtype=np.float32)
    nz = a > 0
    if np.any(nz):
        r = (np.float32(127.0) / a[nz]).astype(np.float32)             # one division per row
        t = (y[nz] * r[:, None]).astype(np.float32)                     # fp32 multiply
        q[nz] = np.clip(np.rint(t), -127, 127).astype(np.int8)          # half-to-even
        s[nz] = (a[nz] / np.float32(127.0)).astype(np.float32)
    return q, s


def quantize_act_int8(x_bits: np.ndarray, had_block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Activation quantizer: block Hadamard rotation, then per-token INT8.

    HQ-DM section 2.1 (X is multiplied by the block Hadamard H, then (XH) is
    quantized) and 6Bit-Diffusion section 2A (local block Hadamard before
    quantization).  Per-token dynamic scales stand in for HQ-DM's learned
    per-timestep LSQ scales (section 2.2), which need training.

    x_bits: uint16 bf16 patterns [M, K].  Returns (codes int8 [M, K], s_a fp32 [M]).
    """
    x = bf16_to_f32(x_bits)
    y = block_fwht_f32(x, had_block)
    return _absmax_int8_codes(y)


def quantize_weights_int8(w_bits: np.ndarray, had_block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Offline weight quantization into the single shared INT8 buffer.

    TASQ section 2 ("Representação de Peso Compartilhada"): one shared
    maximum-precision (8-bit) buffer is stored; no per-stage copies.
    Per-output-channel symmetric absmax codes.

    Reading: an int8 x int8 matrix core needs both operands as int8 codes, so
    the weights are rotated by the same block Hadamard as the activations
    before quantization.  Since H_b H_b^T = b I blockwise,
    (X H)(W H)^T = b X W^T, so the weight scale carries the exact 1/b:
    s_w = (a/127) / max(b, 1).

    w_bits: uint16 bf16 [N, K].  Returns (W_q int8 [N, K], s_w fp32 [N]).
    """
    w = bf16_to_f32(w_bits)
    y = block_fwht_f32(w, had_block)
    q, s = _absmax_int8_codes(y)
    s = (s / np.float32(max(had_block, 1))).astype(np.float32)
    return q, s


# --------------------------------------------------------------------------
# O5: the TASQ LSB mask
# --------------------------------------------------------------------------


def lsb_truncate(w_q: np.ndarray, k: int) -> np.ndarray:
    """Operational weight at (step t, layer l): drop the k least-significant bits.

    TASQ section 2: the stored n-bit weight Q_n becomes Q_M = Q_n minus its
    LSB part selected by the mask M_{t,l}; the page describes this as
    bit-plane truncation or right-shifting.  Reading of the garbled equation:
    the "LSB" term is the value of the k low bits of the two's-complement code
    (w mod 2^k, always >= 0), so Q_M = w - (w mod 2^k) = (w >> k) << k, a
    floor towards -inf.  k = 0 keeps every bit; effective precision is 8 - k.
    """
    if not 0 <= k <= 7:
        raise ValueError("k must be in [0, 7]")
    w = np.asarray(w_q, dtype=np.int64)
    return (w - np.mod(w, 1 << k)).astype(np.int8)


# --------------------------------------------------------------------------
# O6, O7: masked GEMM and bit-plane GEMM (plain definitions, exact integers)
# --------------------------------------------------------------------------

INT32_MAX = 2**31 - 1


def masked_gemm_i32(x_q: np.ndarray, w_q: np.ndarray, k: int) -> np.ndarray:
    """acc[m, n] = sum_k Xq[m, k] * Q_M[n, k], exact, returned as int32.

    TASQ section 2: the layer runs with the truncated weights of its
    (step, layer) mask over the one shared buffer.  Computed in int64 and
    checked to fit int32 (|acc| <= 127 * 128 * K).
    """
    a = np.asarray(x_q, dtype=np.int64)
    w = lsb_truncate(w_q, k).astype(np.int64)
    acc = a @ w.T
    if acc.size and np.max(np.abs(acc)) > INT32_MAX:
        raise OverflowError("accumulator exceeds int32")
    return acc.astype(np.int32)


def bitplane_gemm_i32(x_q: np.ndarray, w_q: np.ndarray, k: int) -> np.ndarray:
    """Bit-serial form: acc = sum over retained planes b of c_b * (Xq . W_b^T).

    TASQ section 2 (Temporal-Precision Engine): in a bit-serial GEMM the
    activations stay resident and only the weight bit-planes selected for the
    layer and step are streamed, so work scales with the number of planes.
    W_b in {0, 1} is bit b of the two's-complement byte; its weight c_b is
    2^b for b < 7 and -2^7 for the sign plane b = 7.  Planes b = k..7 are the
    8 - k planes the mask keeps.
    """
    a = np.asarray(x_q, dtype=np.int64)
    u = np.asarray(w_q, dtype=np.int8).view(np.uint8).astype(np.int64)
    acc = np.zeros((a.shape[0], u.shape[0]), dtype=np.int64)
    for b in range(k, 8):
        plane = (u >> b) & 1                       # W_b in {0, 1}
        weight = -(1 << 7) if b == 7 else (1 << b)
        acc += weight * (a @ plane.T)
    if acc.size and np.max(np.abs(acc)) > INT32_MAX:
        raise OverflowError("accumulator exceeds int32")
    return acc.astype(np.int32)


# --------------------------------------------------------------------------
# Plane-major storage of the shared buffer (stream only the retained planes)
# --------------------------------------------------------------------------
#
# TASQ section 2 (Temporal-Precision Engine): activation planes stay on chip
# while only the weight bit-planes a layer-step keeps are streamed, which cuts
# plane fetches from 2LR to L + R.  The same 8 bits per weight can be stored
# plane by plane so that a step with mask k reads 8 - k planes and never
# touches the k dropped ones.  The layout is this library's own encoding (the
# pages fix none): a uint32 array P[8][S][N][4] with S = ceil(K/128); word
# P[b][s][n][j] holds bit b of the 32 weights W[n][128s + 32j + i], i = 0..31,
# with weight i = 4u + q at bit position 8q + u (u = 0..7, q = 0..3).  Words
# whose 32 weights lie past K are zero.


def planes_shape(n_rows: int, k_cols: int) -> Tuple[int, int, int, int]:
    return (8, (k_cols + 127) // 128, n_rows, 4)


def pack_weight_planes(w_q: np.ndarray) -> np.ndarray:
    """Plane-major copy of the INT8 codes: uint32 [8][ceil(K/128)][N][4] (layout above)."""
    w = np.asarray(w_q, dtype=np.int8)
    n_rows, k_cols = w.shape
    if k_cols % 32:
        raise ValueError("K must be a multiple of 32")
    shape = planes_shape(n_rows, k_cols)
    padded = np.zeros((n_rows, shape[1] * 128), dtype=np.uint64)
    padded[:, :k_cols] = w.view(np.uint8)
    groups = padded.reshape(n_rows, shape[1], 4, 32)          # [N][S][j][i]
    out = np.zeros(shape, dtype=np.uint64)
    for b in range(8):
        bits = (groups >> np.uint64(b)) & np.uint64(1)        # bit b of every weight
        word = np.zeros((n_rows, shape[1], 4), dtype=np.uint64)
        for i in range(32):
            u, q = i // 4, i % 4
            word |= bits[:, :, :, i] << np.uint64(8 * q + u)
        out[b] = word.transpose(1, 0, 2)                      # [S][N][j]
    return out.astype(np.uint32)


def unpack_weight_planes(planes: np.ndarray, k: int, k_cols: int) -> np.ndarray:
    """Operational weights rebuilt from the planes b = k..7 only: int8 [N][K].

    Each retained plane contributes c_b * bit, c_b = 2^b for b < 7 and -2^7
    for the sign plane, so the result is the sum over the planes the mask
    keeps (TASQ section 2, bit-plane truncation).  Planes below k are never
    read.
    """
    if not 0 <= k <= 7:
        raise ValueError("k must be in [0, 7]")
    p = np.asarray(planes, dtype=np.uint32).astype(np.int64)
    _, n_stages, n_rows, _ = p.shape
    w = np.zeros((n_rows, n_stages, 4, 32), dtype=np.int64)
    for b in range(k, 8):
        weight = -(1 << 7) if b == 7 else (1 << b)
        word = p[b].transpose(1, 0, 2)                         # [N][S][j]
        for i in range(32):
            u, q = i // 4, i % 4
            w[:, :, :, i] += weight * ((word >> (8 * q + u)) & 1)
    return w.reshape(n_rows, n_stages * 128)[:, :k_cols].astype(np.int8)


def plane_gemm_i32(x_q: np.ndarray, planes: np.ndarray, k: int) -> np.ndarray:
    """acc = Xq . W_k^T with W_k rebuilt from the retained planes (exact int64 -> int32)."""
    a = np.asarray(x_q, dtype=np.int64)
    w = unpack_weight_planes(planes, k, a.shape[1]).astype(np.int64)
    acc = a @ w.T
    if acc.size and np.max(np.abs(acc)) > INT32_MAX:
        raise OverflowError("accumulator exceeds int32")
    return acc.astype(np.int32)


# --------------------------------------------------------------------------
# O8: dequantization epilogue
# --------------------------------------------------------------------------


def dequant(acc: np.ndarray, s_a: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """Y[m, n] = acc[m, n] * s_a[m] * s_w[n], evaluated in fp64.

    HQ-DM section 2.1 ("Eficiência de Hardware"): the core is an integer
    matrix product and the floating-point scales are applied outside it.
    """
    return (np.asarray(acc, dtype=np.float64)
            * np.asarray(s_a, dtype=np.float64)[:, None]
            * np.asarray(s_w, dtype=np.float64)[None, :])


# --------------------------------------------------------------------------
# O9, O10, O11: MXFP4 (OCP MX v1.0) quantization and GEMM
# --------------------------------------------------------------------------

MX_BLOCK = 32
E2M1_EMAX = 2                                 # largest E2M1 exponent (value 6 = 1.5 * 2^2)
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 code -> value (bit 3 sign, bits 2..0 magnitude index)."""
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code; ties go to the code with an even mantissa bit; |v| > 6 saturates.

    Computed by distance to every representable magnitude (exact in fp64 for
    fp32 inputs).  A result of magnitude 0 is emitted as +0 (code 0).
    """
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), 6.0)
    dist = np.abs(mag[..., None] - E2M1_MAGNITUDES)
    best = np.min(dist, axis=-1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer the even code (its low bit is the mantissa bit)
    even = cand & ((np.arange(8) & 1) == 0)
    pick = np.where(np.any(even, axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    code = pick.astype(np.uint8)
    neg = (v < 0) & (code != 0)
    return (code | (neg.astype(np.uint8) << 3)).astype(np.uint8)


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for positive finite a, read from the binary exponent (no log)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))   # a = m 2^e, m in [0.5, 1)
    return e.astype(np.int64) - 1


def mx_quantize_rows(x_f32: np.ndarray, had_block: int) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP4 quantization of each row in blocks of 32 elements.

    6Bit-Diffusion section 2A: layers scheduled to 4 bits are quantized after
    a local block Hadamard transform.  Format per OCP MX v1.0: each block of 32
    shares the E8M0 scale 2^X with X = floor(log2 amax) - 2 (2 being E2M1's
    largest exponent), clamped to [-127, 127], stored as X + 127; elements are
    y * 2^-X rounded to E2M1.  An all-zero block stores scale byte 127.
    Packing: element 2i in the low nibble of byte i, element 2i+1 in the high.

    x_f32: fp32 [M, K] (K % 32 == 0).  Returns (packed u8 [M, K/2], e8m0 u8 [M, K/32]).
    """
    if had_block not in (0, MX_BLOCK):
        raise ValueError("MXFP4 path takes block Hadamard 0 or 32")
    y = block_fwht_f32(x_f32, had_block)
    M, K = y.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blk = y.reshape(M, K // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.max(np.abs(blk), axis=2)
    X = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    X[nz] = np.clip(_floor_log2(amax[nz]) - E2M1_EMAX, -127, 127)
    v = blk * np.exp2(-X.astype(np.float64))[:, :, None]      # exact power-of-two scaling
    codes = e2m1_encode(v).reshape(M, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def mx_unpack(packed: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """Decode packed MXFP4 rows to fp64 values (element * 2^(byte-127))."""
    p = np.asarray(packed, dtype=np.uint8)
    M = p.shape[0]
    codes = np.empty((M, p.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = p & 0x0F
    codes[:, 1::2] = p >> 4
    vals = e2m1_decode(codes).reshape(M, -1, MX_BLOCK)
    scale = np.exp2(np.asarray(e8m0, dtype=np.float64) - 127.0)
    return (vals * scale[:, :, None]).reshape(M, -1)


def mxfp4_gemm(x_fp4, x_e8m0, w_fp4, w_e8m0, out_scale: float) -> np.ndarray:
    """Y = out_scale * sum_k xhat[m, k] * what[n, k], in fp64.

    With both operands rotated by the same H_32, (X H)(W H)^T = 32 X W^T, so
    out_scale = 1/32 recovers X W^T (HQ-DM section 2.1 recovery by
    orthogonality, with the factor kept as a floating-point scale).
    """
    xa = mx_unpack(x_fp4, x_e8m0)
    wa = mx_unpack(w_fp4, w_e8m0)
    return (xa @ wa.T) * float(out_scale)


# --------------------------------------------------------------------------
# Producer-fused quantization: GELU folded into the MLP-down activation quantizer
# --------------------------------------------------------------------------
#
# The MLP's down projection consumes GELU(up-projection output).  Folding the
# GELU into the quantizer that feeds the down projection removes a full read and
# write of the 4H-wide activation.  The pages fix no activation function; the
# DiT convention is GELU in its tanh form,
#   gelu(x) = 0.5 x (1 + tanh(u)),  u = sqrt(2/pi) (x + 0.044715 x^3).
# Reading: the down projection's input is that value rounded to bf16 (round to
# nearest, ties to even) -- what an unfused pipeline stores -- and values of
# magnitude below 2^-100 are taken as zero (GELU is that small only for
# x < -9.2, where no fp32 evaluation keeps relative accuracy).  It is then
# quantized exactly as quantize_act_int8 does.
#
# The oracle evaluates the definition in fp64 through the identity
# 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), which avoids the cancellation of
# 1 + tanh(u) for negative u (exp is numpy's fp64 exp, a library primitive),
# and rounds the fp64 value to bf16 directly (no intermediate fp32 rounding).

GELU_FLUSH = 2.0 ** -100


def gelu_tanh_f64(x: np.ndarray) -> np.ndarray:
    """GELU (tanh form) of x in fp64, x / (1 + exp(-2u)); |result| < 2^-100 -> 0."""
    x = np.asarray(x, dtype=np.float64)
    u = np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)
    with np.errstate(over="ignore"):
        g = x / (1.0 + np.exp(-2.0 * u))      # exp overflow -> inf -> g = -0 (flushed anyway)
    return np.where(np.abs(g) < GELU_FLUSH, 0.0, g)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns, round to nearest, ties to even, in one rounding.

    bf16 keeps 8 significant bits and fp32's exponent range: a normal value
    m 2^e (m in [0.5, 1)) becomes rint(m 2^8) 2^(e-8); below 2^-126 the step
    is the subnormal quantum 2^-133.  Finite inputs within the bf16 range.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    normal = np.abs(v) >= 2.0 ** -126
    q = np.where(normal, np.ldexp(np.rint(np.ldexp(m, 8)), e - 8),
                 np.ldexp(np.rint(np.ldexp(v, 133)), -133))
    q = np.where(q == 0, np.copysign(0.0, v), q)
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def quantize_act_gelu_int8(x_bits: np.ndarray, had_block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Quantizer of the down projection's input: bf16(gelu(x)), then quantize_act_int8."""
    g = gelu_tanh_f64(bf16_to_f32(np.asarray(x_bits)))
    return quantize_act_int8(f64_to_bf16_bits(g), had_block)


def quantize_act_gelu_mx(x_bits: np.ndarray, had_block: int) -> Tuple[np.ndarray, np.ndarray]:
    """The same input for a down projection scheduled to 4 bits (6Bit-Diffusion section
    2A): bf16(gelu(x)), then mx_quantize_rows."""
    g = gelu_tanh_f64(bf16_to_f32(np.asarray(x_bits)))
    return mx_quantize_rows(bf16_to_f32(f64_to_bf16_bits(g)), had_block)


# --------------------------------------------------------------------------
# HQ-DM single Hadamard: rotate only the activations, keep the weights as they are
# --------------------------------------------------------------------------
#
# HQ-DM section 2.1: the activations are multiplied by a block-diagonal
# Hadamard H and quantized; the weights are left untransformed; inference
# recovers X through the orthogonality of H, X_hat = S_XH (XH)_int H, with the
# Hadamard normalization moved into the fp scale, so the core stays an integer
# product.  With the unnormalized +-1 H (H H = b I): X ~ (s_a / b) Z with the
# integer matrix Z = (XH)_int H, |Z| <= 127 b.  Z does not fit int8, so it is
# split Z = 128 hi + lo (hi = floor(Z / 128), lo in [0, 127]) and the product
# runs as two INT8 products against the TASQ-truncated, unrotated weights:
# Z W_k^T = 128 (hi W_k^T) + lo W_k^T.


def hqdm_quantize_act(x_bits: np.ndarray, had_block: int) -> Dict[str, np.ndarray]:
    """Per token: codes of XH (as quantize_act_int8), Z = FWHT(codes), hi/lo planes, scale s_a / b."""
    b = max(had_block, 1)
    q, s_a = quantize_act_int8(x_bits, had_block)
    z = block_fwht_f32(q.astype(np.float32), had_block).astype(np.int64)   # exact: |Z| <= 127 b < 2^24
    hi = np.floor_divide(z, 128)
    lo = z - 128 * hi
    return {"q": q, "z": z, "hi": hi.astype(np.int8), "lo": lo.astype(np.int8),
            "scale": (s_a / np.float32(b)).astype(np.float32)}


def hqdm_gemm_i64(z: np.ndarray, w_q: np.ndarray, k: int) -> np.ndarray:
    """Exact Z . W_k^T (int64), W_k the truncated, unrotated weight codes (TASQ section 2)."""
    w = lsb_truncate(w_q, k).astype(np.int64)
    return np.asarray(z, dtype=np.int64) @ w.T


# --------------------------------------------------------------------------
# DMPQ: the online INT8 / 4-bit selector (6Bit-Diffusion section 2A)
# --------------------------------------------------------------------------
#
# The page: the input-output relative L1 difference of a block at step t-1
# predicts, linearly, how sensitive that block's inner linear layers are to
# quantization at step t; unstable (high-variation) blocks keep INT8, stable
# ones go to 4 bits.  It prints neither the predictor's coefficients nor the
# threshold, so a linear predictor compared with a threshold is a threshold
# theta_l on Gamma per layer: INT8 when Gamma > theta_l, else 4-bit.
#
# Gamma = sum |out - in| / sum |in| over the block's hidden states.  The page
# fixes no summation order; the oracle takes each sum exactly rounded
# (math.fsum of the fp64 terms), then one fp64 division.


def dmpq_gamma(x_in_bits: np.ndarray, x_out_bits: np.ndarray) -> Tuple[float, float, float]:
    """(Gamma, sum |out - in|, sum |in|) of one block.

    Terms are fp64: |in| exactly, |out - in| by one fp64 subtraction (exact for
    bf16 operands whose binary exponents differ by less than 45).  Each sum is
    the correctly rounded value of the exact sum of its terms (math.fsum).
    Gamma = 0 when both sums are 0, +inf when only sum |in| is 0.
    """
    a = bf16_to_f32(np.asarray(x_in_bits)).astype(np.float64)
    b = bf16_to_f32(np.asarray(x_out_bits)).astype(np.float64)
    if a.shape != b.shape:
        raise ValueError("in and out must have the same shape")
    num = math.fsum(np.abs(b - a).ravel().tolist())
    den = math.fsum(np.abs(a).ravel().tolist())
    if den == 0.0:
        return (0.0 if num == 0.0 else float("inf")), num, den
    return num / den, num, den


def dmpq_select(gamma: float, thetas) -> np.ndarray:
    """fmt per layer of the block for the next step: INT8 (0) if Gamma > theta_l, else MXFP4 (1)."""
    th = np.asarray(thetas, dtype=np.float32).astype(np.float64)
    return np.where(gamma > th, 0, 1).astype(np.uint8)


# --------------------------------------------------------------------------
# O12: the per-(step, layer) schedule and the full linear at one step
# --------------------------------------------------------------------------


def schedule_lookup(k_table: np.ndarray, fmt_table: np.ndarray, step: int, layer: int) -> Tuple[int, int]:
    """(k, fmt) for one (step, layer).

    TASQ section 2: the LSB mask M_{t,l} is learned per layer and denoising
    stage; a stage is a run of steps written out step by step.  6Bit-Diffusion
    section 2A: INT8 or 4-bit is chosen per layer and step.
    """
    return int(k_table[step, layer]), int(fmt_table[step, layer])


def linear_int8(x_bits, w_bits, had_block: int, k: int) -> Dict[str, np.ndarray]:
    """One quantized linear at a step with mask k: quantize, masked GEMM, dequant."""
    xq, s_a = quantize_act_int8(x_bits, had_block)
    wq, s_w = quantize_weights_int8(w_bits, had_block)
    acc = masked_gemm_i32(xq, wq, k)
    return {"x_q": xq, "s_a": s_a, "w_q": wq, "s_w": s_w, "acc": acc,
            "y": dequant(acc, s_a, s_w)}


def linear_mxfp4(x_bits, w_bits, had_block: int) -> Dict[str, np.ndarray]:
    """One 4-bit linear: MX-quantize both operands after the block-32 rotation, GEMM."""
    xp, xe = mx_quantize_rows(bf16_to_f32(x_bits), had_block)
    wp, we = mx_quantize_rows(bf16_to_f32(w_bits), had_block)
    scale = 1.0 / max(had_block, 1)
    return {"x_fp4": xp, "x_e8m0": xe, "w_fp4": wp, "w_e8m0": we,
            "y": mxfp4_gemm(xp, xe, wp, we, scale)}

"""Pins for the CPU oracle: each check ties it to something other than itself.

Pins used: hand-worked fixtures under tests/golden (each cites its source),
closed forms, exhaustive enumeration, brute-force loops over Python integers
or Fractions on tiny inputs, and library routines where the oracle's step is a
special case of one (the torch bf16 cast).
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import tabit_oracle as O
import tabit_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def _bits(vals):
    """fp32-exact values -> bf16 bit patterns (the values are bf16-exact)."""
    t = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.tensor(vals, dtype=torch.float32))
    return S.bf16_bits(t)


def _fp32_round(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of a positive rational (exact, via neighbours)."""
    f = np.float32(float(fr))            # within one ulp
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


# ---------------------------------------------------------------- Hadamard
def test_hadamard_golden_small():
    mats, cur = {}, None
    for line in _lines("hadamard_sylvester.txt"):
        if line.startswith("H"):
            cur = line
            mats[cur] = []
        else:
            mats[cur].append([int(v) for v in line.split()])
    for name, rows in mats.items():
        n = int(name[1:])
        assert np.array_equal(O.sylvester_hadamard(n), np.array(rows))


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_closed_form_and_orthogonality(n):
    H = O.sylvester_hadamard(n)
    closed = np.array([[(-1) ** bin(i & j).count("1") for j in range(n)] for i in range(n)])
    assert np.array_equal(H, closed)
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64))   # H H^T = n I
    assert np.array_equal(H, H.T)


# ---------------------------------------------------------------- FWHT
@pytest.mark.parametrize("b", [2, 4, 32, 64, 128])
def test_fwht_equals_blockdiag_matrix_on_small_integers(b):
    rng = np.random.default_rng(b)
    K = 4 * b
    x = rng.integers(-8, 9, size=(5, K))
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(b)] for i in range(b)])
    ref = np.concatenate([x[:, j * b:(j + 1) * b] @ H for j in range(K // b)], axis=1)
    got = O.block_fwht_f32(x.astype(np.float32), b)
    assert np.array_equal(got.astype(np.int64), ref)


@pytest.mark.parametrize("b", [32, 64, 128])
def test_fwht_round_trip_and_block_independence(b):
    rng = np.random.default_rng(7 + b)
    x = rng.integers(-100, 101, size=(3, 3 * b)).astype(np.float32)
    y = O.block_fwht_f32(O.block_fwht_f32(x, b), b)
    assert np.array_equal(y, b * x)               # H H = b I: recovery by orthogonality
    x2 = x.copy()
    x2[:, :b] += 1                                # perturb only block 0
    d = O.block_fwht_f32(x2, b) - O.block_fwht_f32(x, b)
    assert np.all(d[:, b:] == 0) and np.any(d[:, :b] != 0)


def test_fwht_identity_for_block_zero():
    x = np.random.default_rng(0).standard_normal((2, 64)).astype(np.float32)
    assert np.array_equal(O.block_fwht_f32(x, 0), x)


def test_fwht_stage_order_golden():
    lines = dict(l.split(" ", 1) for l in _lines("fwht_stage_order.txt"))

    def parse(s):
        return np.array([math.ldexp(float(m), int(e)) for m, e in
                         (p.split() for p in s.split("|"))], dtype=np.float32)
    got = O.block_fwht_f32(parse(lines["input"])[None, :], 4)[0]
    assert np.array_equal(got.view(np.uint32), parse(lines["output"]).view(np.uint32))


def test_rotated_product_identity():
    """(X H)(W H)^T = b X W^T blockwise (exact on small integers)."""
    rng = np.random.default_rng(3)
    for b in (32, 64):
        X = rng.integers(-5, 6, size=(4, 2 * b))
        W = rng.integers(-5, 6, size=(6, 2 * b))
        XH = O.block_fwht_f32(X.astype(np.float32), b).astype(np.int64)
        WH = O.block_fwht_f32(W.astype(np.float32), b).astype(np.int64)
        assert np.array_equal(XH @ WH.T, b * (X @ W.T))


# ---------------------------------------------------------------- INT8 quantizer
def test_int8_quant_golden():
    for line in _lines("int8_quant_worked.txt"):
        head, xs, qs, sc = [p.strip() for p in line.split("|")]
        _, b = head.split()
        x = [float(v) for v in xs.split()]
        q_ref = np.array([int(v) for v in qs.split()], dtype=np.int8)
        num, den = (int(v) for v in sc.split())
        q, s = O.quantize_act_int8(_bits(x)[None, :], int(b))
        assert np.array_equal(q[0], q_ref), line
        assert s[0] == _fp32_round(Fraction(num, den)), line


def test_int8_quant_properties():
    rng = np.random.default_rng(11)
    x = S.gen_activation(37, 256, seed=5)
    bits = S.bf16_bits(x)
    for b in (0, 32, 64, 128):
        q, s = O.quantize_act_int8(bits, b)
        y = O.block_fwht_f32(O.bf16_to_f32(bits), b)
        a = np.max(np.abs(y), axis=1)
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        # the element of largest magnitude maps to +-127
        idx = np.argmax(np.abs(y), axis=1)
        assert np.all(np.abs(q[np.arange(37), idx].astype(np.int32)) == 127)
        # every code is within half a step of y * r
        r = (np.float32(127.0) / a).astype(np.float32)
        assert np.all(np.abs(y * r[:, None] - q) <= 0.5 + 1e-6)
        assert np.array_equal(s, (a / np.float32(127)).astype(np.float32))
    del rng


def test_int8_quant_zero_row_and_zero_block():
    bits = np.zeros((2, 64), dtype=np.uint16)
    bits[1] = S.bf16_bits(torch.ones(64, dtype=torch.bfloat16))
    q, s = O.quantize_act_int8(bits, 32)
    assert np.all(q[0] == 0) and s[0] == 0
    assert s[1] > 0


@pytest.mark.parametrize("b", [4, 16, 64])
def test_normalization_folds_into_scale(b):
    """Extracting the 1/sqrt(b) normalization into the fp scale changes no code.

    HQ-DM section 2.1: the normalization leaves the integer core.  For these b,
    sqrt(b) is a power of two, so the normalized transform is an exact scaling.
    """
    x = O.bf16_to_f32(S.bf16_bits(S.gen_activation(9, 4 * b, seed=b)))
    y = O.block_fwht_f32(x, b)
    q1, s1 = O._absmax_int8_codes(y)
    q2, s2 = O._absmax_int8_codes(y / np.float32(math.sqrt(b)))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s1, s2 * np.float32(math.sqrt(b)))


def test_weight_scale_carries_inverse_block():
    w = S.bf16_bits(S.gen_weight(8, 128, seed=1))
    for b in (0, 32, 64):
        q, s = O.quantize_weights_int8(w, b)
        qa, sa = O.quantize_act_int8(w, b)
        assert np.array_equal(q, qa)
        assert np.array_equal(s, (sa / np.float32(max(b, 1))).astype(np.float32))


# ---------------------------------------------------------------- LSB mask
def test_lsb_golden():
    for line in _lines("lsb_truncation.txt"):
        w, k, exp = (int(v) for v in line.split())
        assert int(O.lsb_truncate(np.array([w], np.int8), k)[0]) == exp, line


def test_lsb_exhaustive():
    w = np.arange(-128, 128, dtype=np.int64)
    for k in range(8):
        got = O.lsb_truncate(w.astype(np.int8), k).astype(np.int64)
        for wi, gi in zip(w.tolist(), got.tolist()):
            assert gi == (wi >> k) << k                      # arithmetic shift (Python int)
            byte = (wi & 0xFF) & ((0xFF << k) & 0xFF)         # clear the k low bits of the byte
            assert gi == (byte - 256 if byte & 0x80 else byte)
    with pytest.raises(ValueError):
        O.lsb_truncate(w.astype(np.int8), 8)


# ---------------------------------------------------------------- GEMMs
def _brute_gemm(X, W):
    return [[sum(int(X[m][k]) * int(W[n][k]) for k in range(len(X[0]))) for n in range(len(W))]
            for m in range(len(X))]


@pytest.mark.parametrize("k", range(8))
def test_masked_gemm_brute_force(k):
    X = S.gen_int8((3, 40), seed=1, lo=-127, hi=127)
    Wq = S.gen_int8((5, 40), seed=2, lo=-127, hi=127)
    Wt = [[(int(w) >> k) << k for w in row] for row in Wq]
    ref = _brute_gemm(X, Wt)
    assert O.masked_gemm_i32(X, Wq, k).tolist() == ref
    # bit-serial definition over the retained planes, brute force
    ref_bp = [[sum(int(X[m][kk]) * sum(((int(Wq[n][kk]) & 0xFF) >> b & 1) * (-(1 << 7) if b == 7 else (1 << b))
                                      for b in range(k, 8)) for kk in range(40)) for n in range(5)]
              for m in range(3)]
    assert O.bitplane_gemm_i32(X, Wq, k).tolist() == ref_bp


def test_masked_k0_is_plain_int8_gemm():
    X = S.gen_int8((4, 64), seed=3)
    W = S.gen_int8((6, 64), seed=4, lo=-128, hi=127)
    assert O.masked_gemm_i32(X, W, 0).tolist() == _brute_gemm(X, W)


def test_bitplane_byte_identity_exhaustive():
    for w in range(-128, 128):
        for k in range(8):
            planes = sum(((w & 0xFF) >> b & 1) * (-(1 << 7) if b == 7 else (1 << b)) for b in range(k, 8))
            assert planes == (w >> k) << k


@pytest.mark.parametrize("k", [0, 3, 5, 7])
def test_bitplane_equals_masked_random(k):
    X = S.gen_int8((33, 96), seed=10 + k)
    W = S.gen_int8((17, 96), seed=20 + k, lo=-128, hi=127)
    assert np.array_equal(O.bitplane_gemm_i32(X, W, k), O.masked_gemm_i32(X, W, k))


def test_accumulator_bound_extreme():
    K = 7680
    X = np.full((1, K), -127, np.int8)
    W = np.full((1, K), -128, np.int8)
    assert int(O.masked_gemm_i32(X, W, 0)[0, 0]) == 127 * 128 * K


# ---------------------------------------------------------------- plane-major storage
# Layout (this library's encoding): word P[b][s][n][j] holds bit b of the
# weights W[n][128s + 32j + i]; weight i = 4u + q sits at bit 8q + u; words
# past K are zero.


def test_plane_layout_hand_examples():
    w = np.zeros((2, 160), np.int8)   # two K-stages, the second holds one group
    w[0, 0] = 1            # s 0, j 0, i 0 (u 0, q 0): plane 0, bit 0
    w[0, 5] = -128         # 0x80, i = 5 (u 1, q 1): plane 7, bit 9
    w[0, 31] = 3           # i = 31 (u 7, q 3): planes 0 and 1, bit 31
    w[1, 32 + 6] = 64      # j 1, i = 6 (u 1, q 2): plane 6, bit 17
    w[1, 128 + 12] = -1    # 0xFF, s 1, j 0, i = 12 (u 3, q 0): every plane, bit 3
    P = O.pack_weight_planes(w)
    assert P.shape == (8, 2, 2, 4) and P.dtype == np.uint32
    expect = np.zeros((8, 2, 2, 4), np.uint64)
    expect[0, 0, 0, 0] = 0x00000001 | 0x80000000
    expect[1, 0, 0, 0] = 0x80000000
    expect[7, 0, 0, 0] = 0x00000200
    expect[6, 0, 1, 1] = 0x00020000
    for b in range(8):
        expect[b, 1, 1, 0] |= 0x00000008
    assert np.array_equal(P.astype(np.uint64), expect)   # words past K (s 1, j 1..3) stay 0


def test_plane_round_trip_every_byte_value():
    w = np.arange(-128, 128, dtype=np.int64).astype(np.int8).reshape(1, 256)
    w = np.concatenate([w, w[:, ::-1]], axis=0)[:, :224]           # K = 224: a ragged last stage
    P = O.pack_weight_planes(w)
    for k in range(8):
        rebuilt = O.unpack_weight_planes(P, k, 224)
        assert rebuilt.tolist() == [[(int(v) >> k) << k for v in row] for row in w]


def test_plane_unpack_reads_only_retained_planes():
    w = S.gen_int8((7, 96), seed=5, lo=-128, hi=127)
    P = O.pack_weight_planes(w)
    rng = np.random.default_rng(9)
    for k in range(1, 8):
        junk = P.copy()
        junk[:k] = rng.integers(0, 2**32, size=junk[:k].shape, dtype=np.uint64).astype(np.uint32)
        assert np.array_equal(O.unpack_weight_planes(junk, k, 96), O.lsb_truncate(w, k))


@pytest.mark.parametrize("k", range(8))
def test_plane_gemm_brute_force(k):
    X = S.gen_int8((3, 64), seed=31, lo=-127, hi=127)
    Wq = S.gen_int8((4, 64), seed=32, lo=-128, hi=127)
    Wt = [[(int(w) >> k) << k for w in row] for row in Wq]
    assert O.plane_gemm_i32(X, O.pack_weight_planes(Wq), k).tolist() == _brute_gemm(X, Wt)


# ---------------------------------------------------------------- fused GELU quantizer
def _pi_decimal():
    """pi to ~70 digits by Machin's formula, pi = 16 atan(1/5) - 4 atan(1/239)."""
    getcontext().prec = 80

    def atan_inv(n):
        x = Decimal(1) / n
        s = t = x
        k = 1
        while True:
            t = -t * x * x
            k += 2
            if abs(t / k) < Decimal(10) ** -75:
                return s
            s += t / k
    return 16 * atan_inv(5) - 4 * atan_inv(239)


def _gelu_decimal_fn():
    """The closed form 0.5 x (1 + tanh(u)) in 80-digit decimal arithmetic."""
    getcontext().prec = 80
    c = (Decimal(2) / _pi_decimal()).sqrt()
    a = Decimal("0.044715")

    def g(x):
        x = Decimal(float(x))
        e = (2 * c * (x + a * x * x * x)).exp()
        return Decimal("0.5") * x * (1 + (e - 1) / (e + 1))
    return g


def _bf16_of_decimal(g: Decimal) -> int:
    """bf16 bits of g rounded to nearest (ties to the even code), decided exactly
    by comparing g with the neighbours of the fp64 estimate."""
    b = int(O.f64_to_bf16_bits(np.array([float(g)]))[0])
    best = None
    for d in (-1, 0, 1):
        bb = (b & 0x8000) | min(0x7F7F, max(0, (b & 0x7FFF) + d))
        v = Decimal(float(O.bf16_to_f32(np.array([bb], np.uint16))[0]))
        key = (abs(v - g), bb & 1)
        if best is None or key < best[0]:
            best = (key, bb)
    return best[1]


def test_pi_and_constants():
    assert str(_pi_decimal())[:32] == "3.141592653589793238462643383279"
    assert abs(float((Decimal(2) / _pi_decimal()).sqrt()) - math.sqrt(2 / math.pi)) < 1e-16


def test_gelu_bf16_every_input_against_decimal_closed_form():
    """For every finite bf16 input with |x| <= 16 (33538 values), the oracle's bf16
    GELU equals the exactly rounded bf16 of the literal closed form 0.5 x (1 + tanh(u))
    evaluated with 80 decimal digits; values below 2^-100 are 0.  Beyond |x| = 16
    GELU(x) is x for x > 0 (1 - sigma < e^-400) and below the flush for x < 0."""
    gd = _gelu_decimal_fn()
    bits = np.arange(65536, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        x = O.bf16_to_f32(bits).astype(np.float64)
    fin = np.isfinite(x)
    sel = fin & (np.abs(x) <= 16)
    got = O.f64_to_bf16_bits(O.gelu_tanh_f64(x[sel]))
    flush = Decimal(2) ** -100
    checked = 0
    for xi, gi in zip(x[sel], got):
        g = gd(xi)
        if abs(g) < flush * Decimal("0.999999"):
            assert gi in (0x0000, 0x8000), xi
        elif abs(g) > flush * Decimal("1.000001"):
            assert int(gi) == _bf16_of_decimal(g), (xi, g, hex(gi))
            checked += 1
    assert checked > 25000                       # the rest lie below the flush (tiny |x| too)
    big = x[fin & (x > 16)]
    assert np.array_equal(O.f64_to_bf16_bits(O.gelu_tanh_f64(big)), O.f64_to_bf16_bits(big))
    neg = x[fin & (x < -16)]
    assert np.all(O.gelu_tanh_f64(neg) == 0.0)


def test_gelu_odd_part_identity():
    """gelu(x) - gelu(-x) = x exactly for the tanh form (tanh is odd); in fp64 within
    a few ulp of the larger term, on both sides of the origin and deep in the tails."""
    x = np.concatenate([np.linspace(-8, 8, 4001), [1e-25, 3e-5, 0.7, 5.0]])
    d = O.gelu_tanh_f64(x) - O.gelu_tanh_f64(-x)
    assert np.all(np.abs(d - x) <= 8 * 2.0 ** -53 * np.maximum(np.abs(x), 1e-300) + 1e-300)
    assert O.gelu_tanh_f64(np.array([0.0]))[0] == 0.0


def test_f64_to_bf16_single_rounding():
    """Direct fp64 -> bf16 rounding: a value just above a bf16 midpoint whose fp32
    rounding lands exactly on the midpoint must round up (fp32 first would round to
    even, down); exact ties go to the even code; the subnormal quantum is 2^-133."""
    mid = 1.0 + 2.0 ** -8                         # midpoint between 1 and 1 + 2^-7
    above = mid + 2.0 ** -40                      # fp32(above) == mid
    assert np.float32(above) == np.float32(mid)
    assert O.f64_to_bf16_bits(np.array([above]))[0] == 0x3F81
    assert O.f64_to_bf16_bits(np.array([mid]))[0] == 0x3F80          # tie -> even
    assert O.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82   # tie -> even (up)
    assert O.f64_to_bf16_bits(np.array([-2.0 ** -133]))[0] == 0x8001
    assert O.f64_to_bf16_bits(np.array([2.0 ** -134]))[0] == 0x0000   # tie -> even (zero)
    assert O.f64_to_bf16_bits(np.array([1.5 * 2.0 ** -133]))[0] == 0x0002
    # agrees with torch's fp32 -> bf16 cast on fp32-exact values
    v = torch.randn(4096, generator=torch.Generator().manual_seed(9))
    assert np.array_equal(O.f64_to_bf16_bits(v.double().numpy()), S.bf16_bits(v.to(torch.bfloat16)))


def test_gelu_golden_values_and_row():
    """Hand-worked GELU values (negative inputs and the flush) and a quantized row."""
    for line in _lines("gelu_bf16_worked.txt"):
        tag, rest = line.split(" ", 1)
        parts = [p.strip() for p in rest.split("|")]
        if tag == "value":
            x, gv, bits = float(parts[0]), float(parts[1]), int(parts[2], 16)
            g = O.gelu_tanh_f64(np.array([x]))[0]
            assert g == 0.0 if bits == 0 else abs(g - gv) <= 1e-12 * abs(gv), x
            assert O.f64_to_bf16_bits(np.array([g]))[0] & 0x7FFF == bits & 0x7FFF
            assert bits == 0 or O.f64_to_bf16_bits(np.array([g]))[0] == bits
        elif tag == "row":
            b = int(parts[0])
            lead = [int(c) for c in parts[1].split()]
            num, den = (int(t) for t in parts[2].split())
    xs = [-0.5, -1, -1.5, -2, -3, -4, -6, -9, -9.5, 0.5, 2] + [0.0] * 21
    q, s = O.quantize_act_gelu_int8(_bits([xs]), b)
    assert q[0, :11].tolist() == lead and not q[0, 11:].any()
    assert s[0] == _fp32_round(Fraction(num, den))


def test_gelu_mx_golden_block():
    """Hand-worked MXFP4 codes of the golden row's GELU values (the 4-bit format of
    6Bit-Diffusion section 2A, OCP MX v1.0 encoding)."""
    for line in _lines("gelu_bf16_worked.txt"):
        if line.startswith("mx "):
            parts = [p.strip() for p in line.split(" ", 1)[1].split("|")]
            b = int(parts[0])
            lead = [int(v, 16) for v in parts[1].split()]
            e8 = int(parts[2])
    xs = [-0.5, -1, -1.5, -2, -3, -4, -6, -9, -9.5, 0.5, 2] + [0.0] * 21
    p, e = O.quantize_act_gelu_mx(_bits([xs]), b)
    assert p[0, :6].tolist() == lead and not p[0, 6:].any()
    assert e[0].tolist() == [e8]


def test_gelu_quant_is_identity_quant_on_large_inputs():
    """For x >= 10 the GELU is the identity in bf16, so the codes equal the plain quantizer's."""
    x = (torch.rand(7, 128, generator=torch.Generator().manual_seed(3)) * 50 + 10).to(torch.bfloat16)
    xb = S.bf16_bits(x)
    for b in (0, 64):
        q1, s1 = O.quantize_act_gelu_int8(xb, b)
        q2, s2 = O.quantize_act_int8(xb, b)
        assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    for b in (0, 32):
        p1, e1 = O.quantize_act_gelu_mx(xb, b)
        p2, e2 = O.mx_quantize_rows(O.bf16_to_f32(xb), b)
        assert np.array_equal(p1, p2) and np.array_equal(e1, e2)


# ---------------------------------------------------------------- HQ-DM single Hadamard
@pytest.mark.parametrize("b", [32, 64, 128])
def test_hqdm_codes_unrotate_by_matrix(b):
    """Z equals the codes times the explicit block-diagonal Sylvester matrix (exact integers)."""
    x = S.gen_activation(5, 2 * b, seed=b)
    r = O.hqdm_quantize_act(S.bf16_bits(x), b)
    h = O.sylvester_hadamard(b).astype(np.int64)
    blk = np.kron(np.eye(2, dtype=np.int64), h)
    assert np.array_equal(r["z"], r["q"].astype(np.int64) @ blk)
    assert np.array_equal(r["q"], O.quantize_act_int8(S.bf16_bits(x), b)[0])


def test_hqdm_hi_lo_split_exhaustive():
    z = np.arange(-127 * 128, 127 * 128 + 1, dtype=np.int64)
    hi = np.floor_divide(z, 128)
    lo = z - 128 * hi
    assert hi.min() == -127 and hi.max() == 127 and lo.min() == 0 and lo.max() == 127   # both fit int8
    assert np.array_equal(128 * hi + lo, z)
    # the oracle's planes reproduce Z on real codes
    r = O.hqdm_quantize_act(S.bf16_bits(S.gen_activation(9, 256, seed=2)), 128)
    assert np.array_equal(128 * r["hi"].astype(np.int64) + r["lo"].astype(np.int64), r["z"])
    assert r["lo"].min() >= 0


@pytest.mark.parametrize("b", [32, 64, 128])
def test_hqdm_recovers_activation_within_half_step(b):
    """HQ-DM section 2.1 recovery: X_hat = (s_a / b) Z; each element is within s_a / 2 of X,
    because the per-block code error (<= s_a/2 each) is mixed by H / b."""
    x = S.gen_activation(6, 4 * b, seed=7 + b)
    xf = O.bf16_to_f32(S.bf16_bits(x)).astype(np.float64)
    r = O.hqdm_quantize_act(S.bf16_bits(x), b)
    s_a = r["scale"].astype(np.float64) * b
    xhat = r["scale"].astype(np.float64)[:, None] * r["z"]
    assert np.all(np.abs(xf - xhat) <= s_a[:, None] * 0.5 * (1 + 1e-5) + 1e-30)


@pytest.mark.parametrize("k", [0, 3, 7])
def test_hqdm_gemm_brute_force(k):
    z = S.gen_int8((3, 32), seed=41).astype(np.int64) * 97       # int14-range values
    wq = S.gen_int8((4, 32), seed=42, lo=-128, hi=127)
    ref = [[sum(int(z[m][j]) * ((int(wq[n][j]) >> k) << k) for j in range(32)) for n in range(4)]
           for m in range(3)]
    assert O.hqdm_gemm_i64(z, wq, k).tolist() == ref


def test_hqdm_without_rotation_is_the_masked_gemm():
    x = S.gen_activation(8, 96, seed=12)
    wq = S.gen_int8((16, 96), seed=13, lo=-128, hi=127)
    r = O.hqdm_quantize_act(S.bf16_bits(x), 0)
    assert np.array_equal(r["z"], r["q"].astype(np.int64))
    assert np.array_equal(O.hqdm_gemm_i64(r["z"], wq, 2), O.masked_gemm_i32(r["q"], wq, 2))


# ---------------------------------------------------------------- DMPQ selector
def _bf(vals):
    return S.bf16_bits(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16))


def test_dmpq_gamma_closed_forms():
    x = S.gen_activation(5, 96, seed=3)
    xb = S.bf16_bits(x)
    two = S.bf16_bits((x.float() * 2).to(torch.bfloat16))            # exact doubling
    zero = np.zeros_like(xb)
    assert O.dmpq_gamma(xb, xb)[0] == 0.0
    assert O.dmpq_gamma(xb, two)[0] == 1.0
    assert O.dmpq_gamma(xb, zero)[0] == 1.0
    assert O.dmpq_gamma(zero, xb)[0] == float("inf")
    assert O.dmpq_gamma(zero, zero)[0] == 0.0


def test_dmpq_gamma_exact_on_small_integers():
    rng = np.random.default_rng(4)
    a = rng.integers(-50, 51, size=(7, 48)).astype(np.float32)
    b = rng.integers(-50, 51, size=(7, 48)).astype(np.float32)
    g, num, den = O.dmpq_gamma(_bf(a), _bf(b))
    exact_num = sum(abs(int(p) - int(q)) for p, q in zip(b.ravel(), a.ravel()))
    exact_den = sum(abs(int(q)) for q in a.ravel())
    assert num == exact_num and den == exact_den                     # every partial is an exact integer
    assert g == float(Fraction(exact_num, exact_den))                # one correctly rounded division


def test_dmpq_gamma_against_exact_rationals_wide_range():
    """Sums equal the correctly rounded exact rational sums (Fraction arithmetic on the
    bf16 values) over rows spanning 2^-40 .. 2^40; Gamma is within 2 ulp of the exact
    quotient."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn(24, 64, generator=g) * torch.exp2(torch.randint(-40, 41, (24, 1), generator=g).float())
    y = x + 0.3 * torch.randn(24, 64, generator=g) * x.abs()
    xb, yb = S.bf16_bits(x.to(torch.bfloat16)), S.bf16_bits(y.to(torch.bfloat16))
    gam, num, den = O.dmpq_gamma(xb, yb)
    a = [Fraction(float(v)) for v in O.bf16_to_f32(xb).ravel()]
    o = [Fraction(float(v)) for v in O.bf16_to_f32(yb).ravel()]
    en = sum(abs(q - p) for p, q in zip(a, o))
    ed = sum(abs(p) for p in a)
    assert num == float(en) and den == float(ed)                     # float(Fraction) rounds correctly
    exact = en / ed
    assert abs(Fraction(gam) - exact) <= 2 * Fraction(2) ** -52 * exact


def test_dmpq_sum_is_exactly_rounded_golden():
    """Terms 2^53, 1, 1, 2: the exact sum 2^53 + 4 is representable and is the result;
    a left-to-right fp64 sum gives 2^53 + 2 (2^53 + 1 rounds to 2^53 twice)."""
    row = np.zeros((1, 64), np.float32)
    row[0, 0], row[0, 16], row[0, 32], row[0, 48] = 2.0 ** 53, 1.0, 1.0, 2.0
    _, num, den = O.dmpq_gamma(_bf(np.zeros_like(row)), _bf(row))
    assert num == 2.0 ** 53 + 4 and den == 0.0
    seq = 0.0
    for v in row.ravel().astype(np.float64):
        seq += v
    assert seq == 2.0 ** 53 + 2


def test_dmpq_select_threshold_rule():
    th = np.array([0.25, 0.5, 0.75], np.float32)
    assert O.dmpq_select(0.5, th).tolist() == [0, 1, 1]              # equal to theta -> 4-bit
    assert O.dmpq_select(0.0, th).tolist() == [1, 1, 1]
    assert O.dmpq_select(float("inf"), th).tolist() == [0, 0, 0]
    assert O.dmpq_select(np.nextafter(0.5, 1.0), th).tolist() == [0, 0, 1]


# ---------------------------------------------------------------- epilogue
def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32) * np.float32(1e3),
        # exact ties: low 16 bits = 0x8000, with odd and even kept parts
        (np.arange(1000, dtype=np.uint32) * np.uint32(0x10000) + np.uint32(0x3F808000)).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38], dtype=np.float32),
    ])
    ref = S.bf16_bits(torch.from_numpy(v).to(torch.bfloat16))
    assert np.array_equal(O.f32_to_bf16_bits(v), ref)


def test_dequant_definition():
    acc = np.array([[3, -5]], np.int32)
    y = O.dequant(acc, np.array([0.5], np.float32), np.array([2.0, 0.25], np.float32))
    assert y.tolist() == [[3.0, -0.625]]


# ---------------------------------------------------------------- MXFP4
def _e2m1_table():
    dec, rnd = {}, []
    for line in _lines("e2m1_table.txt"):
        p = line.split()
        if p[0] == "ROUND":
            rnd.append((float(p[1]), int(p[2])))
        else:
            dec[int(p[0])] = float(p[1])
    return dec, rnd


def test_e2m1_decode_and_rounding_golden():
    dec, rnd = _e2m1_table()
    codes = np.arange(16)
    assert O.e2m1_decode(codes).tolist() == [dec[c] for c in range(16)]
    for v, c in rnd:
        assert int(O.e2m1_encode(np.array([v]))[0]) == c, (v, c)


def test_e2m1_encode_is_nearest_exhaustive_grid():
    dec, _ = _e2m1_table()
    vals = np.arange(-8.0, 8.0, 1 / 64)
    codes = O.e2m1_encode(vals)
    for v, c in zip(vals.tolist(), codes.tolist()):
        d = abs(min(abs(v), 6.0) * (1 if v >= 0 else -1) - dec[c])
        best = min(abs(min(abs(v), 6.0) * (1 if v >= 0 else -1) - x) for x in dec.values())
        assert d == best


def test_mx_block_golden():
    lines = {l.split(" ", 1)[0]: l.split(" ", 1)[1] for l in _lines("mx_block_worked.txt")}
    x = np.zeros((1, 32), np.float32)
    vals = [float(v) for v in lines["x"].split()]
    x[0, :len(vals)] = vals
    packed, e8 = O.mx_quantize_rows(x, 0)
    assert int(e8[0, 0]) == int(lines["e8m0"])
    pk = [int(v) for v in lines["packed"].split()]
    assert packed[0, :len(pk)].tolist() == pk and np.all(packed[0, len(pk):] == 0)


def test_mx_scale_range_property():
    """amax * 2^-X lies in [4, 8) for every nonzero block (OCP MX scale rule)."""
    x = O.bf16_to_f32(S.bf16_bits(S.gen_activation(16, 256, seed=9)))
    y = O.block_fwht_f32(x, 32).reshape(16, 8, 32).astype(np.float64)
    _, e8 = O.mx_quantize_rows(x, 32)
    amax = np.max(np.abs(y), axis=2)
    r = amax * np.exp2(-(e8.astype(np.float64) - 127))
    assert np.all((r >= 4) & (r < 8))


def test_mx_zero_block():
    packed, e8 = O.mx_quantize_rows(np.zeros((1, 64), np.float32), 32)
    assert np.all(packed == 0) and np.all(e8 == 127)


def test_mxfp4_gemm_brute_force_fractions():
    dec, _ = _e2m1_table()
    rng = np.random.default_rng(4)
    xp = rng.integers(0, 256, size=(2, 32), dtype=np.uint8)
    wp = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)
    xe = rng.integers(120, 135, size=(2, 2), dtype=np.uint8)
    we = rng.integers(120, 135, size=(3, 2), dtype=np.uint8)

    def elem(p, e, r, i):
        byte = int(p[r, i // 2])
        code = byte & 15 if i % 2 == 0 else byte >> 4
        return Fraction(dec[code]) * Fraction(2) ** (int(e[r, i // 32]) - 127)
    got = O.mxfp4_gemm(xp, xe, wp, we, 1 / 32)
    for m in range(2):
        for n in range(3):
            ref = sum(elem(xp, xe, m, i) * elem(wp, we, n, i) for i in range(64)) / 32
            assert Fraction(got[m, n]) == ref


# ---------------------------------------------------------------- schedule + inputs
def test_schedule_tables_deterministic():
    for name, fn in S.WORKLOADS.items():
        a, b = fn(), fn()
        assert np.array_equal(a.k_bits, b.k_bits) and np.array_equal(a.fmt, b.fmt)
        assert a.k_bits.shape == (a.steps, a.num_layers)
        assert a.k_bits.max() <= 7
    c2 = S.c2_pixart_sigma()
    # early steps are biased to full precision
    assert (c2.k_bits[0] == 0).mean() > (c2.k_bits[-1] == 0).mean()
    c5 = S.c5_cogvideox()
    assert 0.5 < c5.fmt.mean() < 0.7
    assert O.schedule_lookup(c2.k_bits, c2.fmt, 3, 7) == (int(c2.k_bits[3, 7]), 0)


def test_linear_int8_sanity_unpinned():
    """Approximation quality vs the fp64 product: sanity only (parity unpinned)."""
    x = S.gen_activation(16, 256, seed=1)
    w = S.gen_weight(32, 256, seed=2)
    ref = x.double().numpy() @ w.double().numpy().T
    errs = []
    for k in (0, 2, 4):
        out = O.linear_int8(S.bf16_bits(x), S.bf16_bits(w), 64, k)
        errs.append(np.linalg.norm(out["y"] - ref) / np.linalg.norm(ref))
    assert errs[0] < 0.03 and errs[0] <= errs[1] <= errs[2]
    out = O.linear_mxfp4(S.bf16_bits(x), S.bf16_bits(w), 32)
    assert np.linalg.norm(out["y"] - ref) / np.linalg.norm(ref) < 0.3

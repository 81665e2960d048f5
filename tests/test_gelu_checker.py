"""CPU tests of the fused-GELU validity checker used by the GPU parity tests.

The checker must accept every admissible result (the oracle's own codes, and
codes from any choice of bf16 neighbour for an element whose exact GELU lies
within the kernel's error bound of a rounding boundary), and must reject a
planted mistake: a code off by one, a wrong scale, a different GELU form.
"""
import numpy as np
import pytest
import torch

from oracle import tabit_oracle as O
import tabit_synth as S
from tests import gelu_validity as V


def _inputs(M, K, seed):
    x = S.gen_activation(M, K, seed=seed).float() * 3.0
    x[0] = torch.linspace(-12, 12, K)
    if M > 2:
        x[1] = torch.linspace(-9.6, -7.0, K)          # every GELU tiny: the all-tail row
    return S.bf16_bits(x.to(torch.bfloat16))


def _fp32_model(x_bits):
    """An fp32 evaluation in the kernel's steps (numpy fp32, exp2 and divide correctly
    rounded) -- within the stated bound, so it must pass."""
    x = O.bf16_to_f32(x_bits)
    f = np.float32
    k1 = f(2.0 * np.sqrt(2.0 / np.pi))
    k3 = f(0.044715 * 2.0 * np.sqrt(2.0 / np.pi))
    z = (x * (k1 + k3 * (x * x))).astype(np.float32)
    t = np.exp2((-np.abs(z) * f(1.4426950408889634)).astype(np.float32)).astype(np.float32)
    s = (f(1.0) / (f(1.0) + t)).astype(np.float32)
    sig = np.where(z >= 0, s, (t * s).astype(np.float32))
    g = (x * sig).astype(np.float32)
    g = np.where(np.abs(g) < f(2.0 ** -100), f(0.0), g)
    return O.f32_to_bf16_bits(g)


@pytest.mark.parametrize("b", [0, 64])
def test_checker_accepts_oracle_and_fp32_model(b):
    xb = _inputs(24, 1024, seed=3 + b)
    q, s = O.quantize_act_gelu_int8(xb, b)
    V.check_gelu_quant(xb, b, q, s)
    qm, sm = O.quantize_act_int8(_fp32_model(xb), b)
    info = V.check_gelu_quant(xb, b, qm, sm)
    assert info["ambiguous_elements"] > 0


@pytest.mark.parametrize("b", [0, 64])
def test_checker_accepts_other_admissible_neighbour(b):
    xb = _inputs(16, 512, seed=5)
    ref, amb = V.admissible_bf16(xb)
    assert amb
    alt = ref.copy()
    for m, k, c in amb:
        others = [v for v in c if v != ref[m, k]]
        if others:
            alt[m, k] = others[0]
    q, s = O.quantize_act_int8(alt, b)
    V.check_gelu_quant(xb, b, q, s)


@pytest.mark.parametrize("b", [0, 64])
def test_checker_rejects_planted_mistakes(b):
    xb = _inputs(16, 512, seed=7)
    q, s = O.quantize_act_gelu_int8(xb, b)
    bad = q.copy()
    m, k = 5, 100
    bad[m, k] = bad[m, k] + 1 if bad[m, k] < 127 else bad[m, k] - 1
    with pytest.raises(AssertionError):
        V.check_gelu_quant(xb, b, bad, s)
    s2 = s.copy()
    s2[3] = np.nextafter(s2[3], np.float32(1.0))
    with pytest.raises(AssertionError):
        V.check_gelu_quant(xb, b, q, s2)
    # the erf form of GELU differs by up to ~1e-3 relative: not admissible
    from scipy.special import erf
    x = O.bf16_to_f32(xb).astype(np.float64)
    ge = 0.5 * x * (1 + erf(x / np.sqrt(2.0)))
    qe, se = O.quantize_act_int8(O.f64_to_bf16_bits(np.where(np.abs(ge) < 2.0 ** -100, 0.0, ge)), b)
    with pytest.raises(AssertionError):
        V.check_gelu_quant(xb, b, qe, se)


@pytest.mark.parametrize("b", [0, 32])
def test_mx_checker_accepts_admissible_and_rejects_mistakes(b):
    xb = _inputs(16, 512, seed=13 + b)
    p, e = O.quantize_act_gelu_mx(xb, b)
    V.check_gelu_quant_mx(xb, b, p, e)
    pm, em = O.mx_quantize_rows(O.bf16_to_f32(_fp32_model(xb)), b)
    info = V.check_gelu_quant_mx(xb, b, pm, em)
    assert info["ambiguous_elements"] > 0
    bad = p.copy()
    bad[4, 37] ^= 0x01                                    # one E2M1 code off
    with pytest.raises(AssertionError):
        V.check_gelu_quant_mx(xb, b, bad, e)
    e2 = e.copy()
    e2[2, 3] += 1                                         # one block scale off
    with pytest.raises(AssertionError):
        V.check_gelu_quant_mx(xb, b, p, e2)

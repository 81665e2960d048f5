"""GPU parity of HQ-DM's single-Hadamard path (activations rotated, weights not).

Bars: the two int8 planes and the scale bit-exact against the oracle; the
int64 accumulator (128 acc_hi + acc_lo, combined exactly) bit-exact against
the oracle's Z . W_k^T on every tile configuration and several k; bf16 within
1e-2 relative of the oracle's fp64 dequantization.
"""
import numpy as np
import pytest
import torch

from oracle import tabit_oracle as O
import tabit_synth as S
import timestep_adaptive_bit_amd as T

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ctx():
    c = T.Context()
    yield c
    c.close()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _edge_x(M, K, seed):
    x = S.gen_activation(M, K, seed).float()
    if M >= 3:
        x[0] = 0.0
        x[1] *= 1e30
        x[2] *= 1e-30
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("M,K", [(1, 128), (17, 256), (300, 1152), (129, 2304)])
@pytest.mark.parametrize("b", [0, 32, 64, 128])
def test_hqdm_quant_bit_exact(ctx, M, K, b):
    x = _edge_x(M, K, seed=M + K + b)
    ref = O.hqdm_quantize_act(S.bf16_bits(x), b)
    hi, lo, sc = ctx.hqdm_quant_act(x.to(DEV), b)
    np.testing.assert_array_equal(_np(hi), ref["hi"])
    np.testing.assert_array_equal(_np(lo), ref["lo"])
    np.testing.assert_array_equal(_np(sc).view(np.uint32), ref["scale"].view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(1, 32, 128), (70, 96, 256), (300, 160, 1152), (513, 288, 384)])
def test_hqdm_gemm_every_config(ctx, M, N, K):
    b = 128 if K % 128 == 0 else 64
    x = _edge_x(M, K, seed=3 * M + N)
    ref = O.hqdm_quantize_act(S.bf16_bits(x), b)
    wq = S.gen_int8((N, K), seed=N + K, lo=-128, hi=127)
    wq[0, :] = -128
    sw = S.gen_scales(N, seed=5)
    hi, lo, sc = ctx.hqdm_quant_act(x.to(DEV), b)
    dw, dsw = torch.from_numpy(wq).to(DEV), torch.from_numpy(sw).to(DEV)
    try:
        for cfg in range(T.hqdm_config_info()):
            ctx.set_option(T.OPT_HQDM_CONFIG, cfg)
            for k in (0, 3, 7):
                print(f"hqdm {M}x{N}x{K} cfg {cfg} k {k}", flush=True)
                y, acc = ctx.hqdm_qgemm(hi, lo, sc, dw, dsw, k, want_acc=True)
                acc_ref = O.hqdm_gemm_i64(ref["z"], wq, k)
                np.testing.assert_array_equal(_np(acc), acc_ref, err_msg=f"cfg {cfg} k {k}")
                y_ref = acc_ref.astype(np.float64) * ref["scale"].astype(np.float64)[:, None] \
                    * sw.astype(np.float64)[None, :]
                yy = y.float().cpu().numpy().astype(np.float64)
                assert np.all(np.abs(yy - y_ref) <= 1e-2 * np.abs(y_ref) + 1e-30)
    finally:
        ctx.set_option(T.OPT_HQDM_CONFIG, -1)


def test_hqdm_scheduled_linear_and_full_size(ctx):
    """The scheduled path (quantizer + GEMM in the library) on a PixArt-sized linear,
    b = 64, k from the schedule; sampled rows against the oracle, int64-exact via acc."""
    M, N, K, b = 4096, 1152, 1152, 64
    x = S.gen_activation(M, K, seed=S.activation_seed(0, K))
    w = S.gen_weight(N, K, seed=3)
    wts = ctx.quantize_weights(w.to(DEV), 0)                 # unrotated weights
    ws = torch.empty(T.act_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    ctx.set_step_schedule(np.array([[2]], np.uint8))
    y = ctx.scheduled_linear(0, 0, x.to(DEV), wts, b, ws, path=T.PATH_HQDM)
    ref = O.hqdm_quantize_act(S.bf16_bits(x), b)
    wq_ref, sw_ref = O.quantize_weights_int8(S.bf16_bits(w), 0)
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(1).choice(M, 64, replace=False)])
    acc_ref = O.hqdm_gemm_i64(ref["z"][rows], wq_ref, 2)
    y_ref = acc_ref.astype(np.float64) * ref["scale"].astype(np.float64)[rows, None] \
        * sw_ref.astype(np.float64)[None, :]
    yy = y.float().cpu().numpy().astype(np.float64)[rows]
    assert np.all(np.abs(yy - y_ref) <= 1e-2 * np.abs(y_ref) + 1e-30)
    hi, lo, sc = ctx.hqdm_quant_act(x.to(DEV), b)
    _, acc = ctx.hqdm_qgemm(hi, lo, sc, wts["w_q"], wts["w_scale"], 2, want_y=False, want_acc=True)
    np.testing.assert_array_equal(_np(acc)[rows], acc_ref)


# ---------------------------------------------------------------- fused GELU quantizer
def _gelu_inputs(M, K, seed):
    x = S.gen_activation(M, K, seed=seed).float() * 3.0
    if M >= 4:
        x[0] = 0.0
        x[1] = torch.linspace(-30, 30, K)
        x[2] *= 1e-4
        x[3] = torch.linspace(-9.6, -7.0, K)        # every GELU tiny (the tail), some flushed
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("M,K", [(1, 128), (37, 640), (300, 4608), (129, 2560)])
@pytest.mark.parametrize("b", [0, 64])
def test_gelu_quant_valid(ctx, M, K, b):
    """Codes and scales of the fused GELU quantizer against the oracle's exact GELU
    rounded to bf16: bit-exact on rows without an ambiguous element; on the others
    every code and the scale must come from an admissible choice of bf16 neighbour for
    the elements whose exact GELU lies within the kernel's stated error bound of a
    rounding boundary (tests/gelu_validity.py)."""
    from tests import gelu_validity as V
    x = _gelu_inputs(M, K, seed=M * 3 + K + b)
    print(f"gelu_quant {M}x{K} b={b}", flush=True)
    q, s = ctx.gelu_quant_act(x.to(DEV), b)
    info = V.check_gelu_quant(S.bf16_bits(x), b, _np(q), _np(s))
    print(f"  {info}", flush=True)


@pytest.mark.parametrize("M,K,b", [(4096, 4608, 0), (17776, 7680, 32)])
def test_gelu_quant_valid_full_size_sampled_rows(ctx, M, K, b):
    """The MLP-down input shapes of the PixArt- and CogVideoX-shaped stacks: rows are
    independent, so 96 sampled rows (first and last included) are checked."""
    from tests import gelu_validity as V
    x = _gelu_inputs(M, K, seed=M + K)
    print(f"gelu_quant full {M}x{K} b={b}", flush=True)
    q, s = ctx.gelu_quant_act(x.to(DEV), b)
    rows = np.unique(np.r_[0, 1, 2, 3, M - 1, np.random.default_rng(2).choice(M, 91, replace=False)])
    info = V.check_gelu_quant(S.bf16_bits(x)[rows], b, _np(q)[rows], _np(s)[rows])
    print(f"  {info}", flush=True)


@pytest.mark.parametrize("M,K,b", [(37, 640, 0), (37, 640, 32), (300, 4608, 32), (129, 2560, 0)])
def test_gelu_quant_mx_valid(ctx, M, K, b):
    """The MXFP4 form of the fused quantizer: every 32-element block (own E8M0 scale)
    from an admissible choice of bf16 neighbours; other blocks bit-exact."""
    from tests import gelu_validity as V
    x = _gelu_inputs(M, K, seed=M * 7 + K + b)
    print(f"gelu_quant mx {M}x{K} b={b}", flush=True)
    p, e = ctx.gelu_quant_act(x.to(DEV), b, fmt=T.FMT_MXFP4)
    info = V.check_gelu_quant_mx(S.bf16_bits(x), b, _np(p), _np(e))
    print(f"  {info}", flush=True)


def test_gelu_quant_mx_valid_full_size_sampled_rows(ctx):
    from tests import gelu_validity as V
    M, K, b = 17776, 7680, 32
    x = _gelu_inputs(M, K, seed=91)
    print(f"gelu_quant mx full {M}x{K}", flush=True)
    p, e = ctx.gelu_quant_act(x.to(DEV), b, fmt=T.FMT_MXFP4)
    rows = np.unique(np.r_[0, 1, 2, 3, M - 1, np.random.default_rng(4).choice(M, 91, replace=False)])
    info = V.check_gelu_quant_mx(S.bf16_bits(x)[rows], b, _np(p)[rows], _np(e)[rows])
    print(f"  {info}", flush=True)

"""The MLP chained through the native schedule runner: the down projection reads
the up projection's bf16 output of the same step through the GELU-fused
quantizer (tabit_layer.input_from / input_act), INT8 and MXFP4 layer-steps.

Bars: the up projection's output within 1e-2 of the oracle; the down
projection's quantized input (the same kernel run standalone on that output)
admissible against the oracle's exact GELU (tests/gelu_validity.py); the down
projection's output within the GEMM parity bars of the oracle's product of
those codes (INT8: 1e-2 relative; MXFP4: 1e-2 plus 1e-3 of the largest |y|).
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import tabit_oracle as O
import tabit_synth as S
import timestep_adaptive_bit_amd as T
from tests import gelu_validity as V

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ctx():
    c = T.Context()
    yield c
    c.close()


def _stack(ctx, M, H, F, b, fmt_table, k_table, seed):
    """Two layers: up H -> F, down F -> H chained through GELU."""
    w_up = S.gen_weight(F, H, seed=seed)
    w_dn = S.gen_weight(H, F, seed=seed + 1)
    wts = [ctx.quantize_weights(w.to(DEV), b, int8=True, mx=True) for w in (w_up, w_dn)]
    ys = [torch.empty((M, F), dtype=torch.bfloat16, device=DEV),
          torch.empty((M, H), dtype=torch.bfloat16, device=DEV)]
    layers = (T.Layer * 2)()
    for l, (n, k) in enumerate(((F, H), (H, F))):
        layers[l].M, layers[l].N, layers[l].K = M, n, k
        layers[l].w_q, layers[l].w_scale = wts[l]["w_q"].data_ptr(), wts[l]["w_scale"].data_ptr()
        layers[l].w_fp4, layers[l].w_e8m0 = wts[l]["w_fp4"].data_ptr(), wts[l]["w_e8m0"].data_ptr()
        layers[l].y_bf16 = ys[l].data_ptr()
    layers[1].input_from, layers[1].input_act = 1, T.ACT_GELU
    ctx.set_step_schedule(np.asarray(k_table, np.uint8), np.asarray(fmt_table, np.uint8))
    return (w_up, w_dn), wts, ys, layers


def _check_step(ctx, x, ws_w, wts, ys, b, k_row, f_row, rows):
    (w_up, w_dn) = ws_w
    torch.cuda.synchronize()
    xb = S.bf16_bits(x)
    # up projection against the oracle
    if f_row[0] == 0:
        ref_up = O.linear_int8(xb[rows], S.bf16_bits(w_up), b, int(k_row[0]))["y"]
        tol_up = 1e-2 * np.abs(ref_up) + 1e-30
    else:
        ref_up = O.linear_mxfp4(xb[rows], S.bf16_bits(w_up), b)["y"]
        tol_up = 1e-2 * np.abs(ref_up) + 1e-3 * np.abs(ref_up).max() + 1e-30
    y_up = ys[0].cpu()
    assert np.all(np.abs(y_up.float().numpy()[rows].astype(np.float64) - ref_up) <= tol_up)
    # the down projection's input codes: the fused quantizer on the up output
    up_bits = S.bf16_bits(y_up)
    fmt = T.FMT_INT8 if f_row[1] == 0 else T.FMT_MXFP4
    q, s = ctx.gelu_quant_act(ys[0], b, fmt=fmt)
    q, s = q.cpu().numpy(), s.cpu().numpy()
    y_dn = ys[1].float().cpu().numpy().astype(np.float64)[rows]
    if fmt == T.FMT_INT8:
        info = V.check_gelu_quant(up_bits[rows], b, q[rows], s[rows])
        wq, sw = O.quantize_weights_int8(S.bf16_bits(w_dn), b)
        acc = O.masked_gemm_i32(q[rows], wq, int(k_row[1]))
        ref = O.dequant(acc, s[rows], sw)
        assert np.all(np.abs(y_dn - ref) <= 1e-2 * np.abs(ref) + 1e-30)
    else:
        info = V.check_gelu_quant_mx(up_bits[rows], b, q[rows], s[rows])
        wf, we = O.mx_quantize_rows(O.bf16_to_f32(S.bf16_bits(w_dn)), b)
        ref = O.mxfp4_gemm(q[rows], s[rows], wf, we, 1.0 / max(b, 1))
        assert np.all(np.abs(y_dn - ref) <= 1e-2 * np.abs(ref) + 1e-3 * np.abs(ref).max() + 1e-30)
    return info


def test_chained_mlp_small_every_format(ctx):
    """Four steps covering (up, down) = (INT8, INT8), (INT8, MXFP4), (MXFP4, INT8),
    (MXFP4, MXFP4); every row checked."""
    M, H, F, b = 96, 256, 1024, 32
    fmt = [[0, 0], [0, 1], [1, 0], [1, 1]]
    kb = [[0, 2], [3, 0], [0, 5], [0, 0]]
    ws_w, wts, ys, layers = _stack(ctx, M, H, F, b, fmt, kb, seed=5)
    act_ws = torch.empty(T.act_workspace_bytes(M, F), dtype=torch.uint8, device=DEV)
    for t in range(4):
        x = (S.gen_activation(M, H, seed=100 + t).float() * 2).to(torch.bfloat16)
        xd = x.to(DEV)
        ptrs = (ctypes.c_void_p * 2)(xd.data_ptr(), None)
        print(f"chained mlp step {t}: fmt {fmt[t]} k {kb[t]}", flush=True)
        ctx.run_schedule(t, 1, layers, ptrs, b, act_ws)
        info = _check_step(ctx, x, ws_w, wts, ys, b, kb[t], fmt[t], np.arange(M))
        print(f"  {info}", flush=True)


def test_chained_mlp_pixart_size_sampled_rows(ctx):
    """The PixArt-shaped MLP (4096 tokens, 1152 -> 4608 -> 1152), INT8 with the
    schedule's masks, b = 0; 64 sampled rows checked."""
    M, H, F, b = 4096, 1152, 4608, 0
    ws_w, wts, ys, layers = _stack(ctx, M, H, F, b, [[0, 0]], [[1, 3]], seed=21)
    act_ws = torch.empty(T.act_workspace_bytes(M, F), dtype=torch.uint8, device=DEV)
    x = S.gen_activation(M, H, seed=7)
    xd = x.to(DEV)
    ptrs = (ctypes.c_void_p * 2)(xd.data_ptr(), None)
    print("chained mlp pixart size", flush=True)
    ctx.run_schedule(0, 1, layers, ptrs, b, act_ws)
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(3).choice(M, 62, replace=False)])
    info = _check_step(ctx, x, ws_w, wts, ys, b, [1, 3], [0, 0], rows)
    print(f"  {info}", flush=True)

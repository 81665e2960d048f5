"""GPU parity of the plane-major storage and the GEMM that streams only retained planes.

Bars: the packed words bit-exact against the oracle's packing; int32
accumulators bit-exact against the oracle's plane GEMM (which equals the
masked GEMM, pinned on the CPU); bf16 within 1e-2 relative of the oracle's
dequantization, and bit-identical to the masked GEMM's bf16 (same epilogue).
Shapes cover one 32-weight group, ragged K stages (K % 128 != 0), ragged M and
N tiles, and the single-linear configuration (64 x 1152 x 1152) in full.
"""
import ctypes

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


def _bf16_np(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def _close(y, ref):
    assert np.all(np.abs(y - ref) <= 1e-2 * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("N,K", [(32, 32), (96, 160), (64, 1152), (1152, 1152), (416, 2240)])
def test_pack_planes_bit_exact(ctx, N, K):
    wq = S.gen_int8((N, K), seed=N + K, lo=-128, hi=127)
    wq[0, :] = -128
    wq[-1, :] = -1
    p = ctx.pack_weight_planes(torch.from_numpy(wq).to(DEV))
    np.testing.assert_array_equal(_np(p).view(np.uint32), O.pack_weight_planes(wq))


SHAPES = [(1, 32, 32), (17, 96, 160), (64, 640, 1152), (129, 96, 1120), (300, 416, 544),
          (513, 288, 160)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_plane_gemm_every_config_every_k(ctx, M, N, K):
    xq = S.gen_int8((M, K), seed=M + K)
    wq = S.gen_int8((N, K), seed=N + K + 1, lo=-128, hi=127)
    xq[0, :] = -127
    wq[0, :] = -128
    if N >= 2:
        wq[1, :] = 127
    sa, sw = S.gen_scales(M, seed=3), S.gen_scales(N, seed=4)
    planes_ref = O.pack_weight_planes(wq)
    dx, dw = torch.from_numpy(xq).to(DEV), torch.from_numpy(wq).to(DEV)
    dsa, dsw = torch.from_numpy(sa).to(DEV), torch.from_numpy(sw).to(DEV)
    dp = ctx.pack_weight_planes(dw)
    refs = {k: O.plane_gemm_i32(xq, planes_ref, k) for k in range(8)}
    try:
        for cfg in range(T.plane_config_info()):
            ctx.set_option(T.OPT_PLANE_CONFIG, cfg)
            for k in range(8):
                print(f"plane gemm {M}x{N}x{K} cfg {cfg} k {k}", flush=True)
                y, acc = ctx.plane_qgemm(dx, dsa, dp, dsw, k, want_acc=True)
                np.testing.assert_array_equal(_np(acc), refs[k], err_msg=f"cfg {cfg} k {k}")
                _close(_bf16_np(y), O.dequant(refs[k], sa, sw))
                ym, _ = ctx.masked_qgemm(dx, dsa, dw, dsw, k)
                assert torch.equal(y, ym), f"cfg {cfg} k {k}: bf16 differs from the masked GEMM"
    finally:
        ctx.set_option(T.OPT_PLANE_CONFIG, -1)


def test_plane_gemm_single_linear_config_full(ctx):
    """64 tokens x 1152 x 1152 with the block-64 rotation, k = 0, 2, 4, 3, every output."""
    wl = S.c1_single_linear()
    layer = wl.layers[0]
    M, N, K, b = layer.M, layer.N, layer.K, wl.had_block
    w = S.gen_weight(N, K, seed=0)
    wts = ctx.quantize_weights(w.to(DEV), b)
    dp = ctx.pack_weight_planes(wts["w_q"])
    wq_ref, sw_ref = O.quantize_weights_int8(S.bf16_bits(w), b)
    np.testing.assert_array_equal(_np(dp).view(np.uint32), O.pack_weight_planes(wq_ref))
    for t in range(wl.steps):
        k = int(wl.k_bits[t, 0])
        x = S.gen_activation(M, K, seed=S.activation_seed(t, K))
        xq, sa = ctx.hadamard_quant_act(x.to(DEV), b)
        xq_ref, sa_ref = O.quantize_act_int8(S.bf16_bits(x), b)
        y, acc = ctx.plane_qgemm(xq, sa, dp, wts["w_scale"], k, want_acc=True)
        acc_ref = O.plane_gemm_i32(xq_ref, O.pack_weight_planes(wq_ref), k)
        np.testing.assert_array_equal(_np(acc), acc_ref)
        _close(_bf16_np(y), O.dequant(acc_ref, sa_ref, sw_ref))


def test_run_schedule_on_planes(ctx):
    """The native driver on TABIT_PATH_PLANES equals the oracle's linear at every step."""
    shapes = [(96, 256, 384), (96, 384, 256)]
    steps = 3
    k_tab = np.array([[0, 5], [7, 1], [3, 3]], dtype=np.uint8)
    ctx.set_step_schedule(k_tab)
    layers = (T.Layer * len(shapes))()
    keep, refs = [], []
    for li, (M, N, K) in enumerate(shapes):
        w = S.gen_weight(N, K, seed=40 + li)
        wts = ctx.quantize_weights(w.to(DEV), 0)
        dp = ctx.pack_weight_planes(wts["w_q"])
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        layers[li].M, layers[li].N, layers[li].K = M, N, K
        layers[li].w_q = dp.data_ptr()
        layers[li].w_scale = wts["w_scale"].data_ptr()
        layers[li].y_bf16 = y.data_ptr()
        keep += [wts, dp, y]
        refs.append(O.quantize_weights_int8(S.bf16_bits(w), 0))
    ws = torch.empty(max(T.act_workspace_bytes(M, K) for M, _, K in shapes), dtype=torch.uint8,
                     device=DEV)
    for t in range(steps):
        xs = [S.gen_activation(M, K, seed=100 * t + li) for li, (M, _, K) in enumerate(shapes)]
        dxs = [x.to(DEV) for x in xs]
        ptrs = (ctypes.c_void_p * len(shapes))(*[x.data_ptr() for x in dxs])
        ctx.run_schedule(t, 1, layers, ptrs, 0, ws, path=T.PATH_PLANES)
        torch.cuda.synchronize()
        for li, (M, N, K) in enumerate(shapes):
            xq_ref, sa_ref = O.quantize_act_int8(S.bf16_bits(xs[li]), 0)
            wq_ref, sw_ref = refs[li]
            acc_ref = O.masked_gemm_i32(xq_ref, wq_ref, int(k_tab[t, li]))
            y = keep[3 * li + 2]
            _close(_bf16_np(y), O.dequant(acc_ref, sa_ref, sw_ref))

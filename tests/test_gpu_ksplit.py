"""GPU parity of the K-split tiles (few tokens, long K) under the automatic choice.

The library's chooser replaces a tile that leaves half of the CUs idle with a
variant whose K stages are split over wave groups inside the workgroup; the
groups' int32 sums are added exactly, so the bars are the unsplit ones:
accumulators bit-exact against the oracle (masked, bit-plane and plane-major
forms), bf16 within 1e-2 relative and identical across the three forms.
Shapes: one token; K with a ragged last stage; more groups than stages (some
groups walk none); a stage count the groups do not divide; 216 tiles of 64 x 64
(most of one round over 256 CUs, where the split still pays).
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


SHAPES = [(1, 32, 8192), (3, 64, 4160), (64, 1152, 4608), (17, 96, 160), (40, 320, 1120),
          (768, 1152, 1152)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_auto_ksplit_bit_exact(ctx, M, N, K):
    cfg = T.gemm_config_choose(M, N, K)
    pcfg = T.plane_config_choose(M, N, K)
    print(f"ksplit {M}x{N}x{K}: int8 cfg {cfg} {T.gemm_config_info(cfg)}, "
          f"plane cfg {pcfg} {T.plane_config_info(pcfg)}", flush=True)
    if (K + 127) // 128 > 1:                    # more than one stage: a split tile is chosen
        assert T.gemm_config_info(cfg)[2] > 1
        assert T.plane_config_info(pcfg)[2] > 1
    xq = S.gen_int8((M, K), seed=M + K)
    wq = S.gen_int8((N, K), seed=N + K, lo=-128, hi=127)
    xq[0, :] = -127
    wq[0, :] = -128
    sa, sw = S.gen_scales(M, seed=5), S.gen_scales(N, seed=6)
    dx, dw = torch.from_numpy(xq).to(DEV), torch.from_numpy(wq).to(DEV)
    dsa, dsw = torch.from_numpy(sa).to(DEV), torch.from_numpy(sw).to(DEV)
    dp = ctx.pack_weight_planes(dw)
    for k in (0, 3, 7):
        ref = O.masked_gemm_i32(xq, wq, k)
        y_ref = O.dequant(ref, sa, sw)
        ym, am = ctx.masked_qgemm(dx, dsa, dw, dsw, k, want_acc=True)
        yb, ab = ctx.qgemm_bitserial(dx, dsa, dw, dsw, k, want_acc=True)
        yp, ap = ctx.plane_qgemm(dx, dsa, dp, dsw, k, want_acc=True)
        torch.cuda.synchronize()
        for name, acc in (("masked", am), ("bit-plane", ab), ("plane-major", ap)):
            np.testing.assert_array_equal(acc.cpu().numpy(), ref, err_msg=f"{name} k {k}")
        yy = ym.float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(yy - y_ref) <= 1e-2 * np.abs(y_ref) + 1e-30), f"k {k}"
        assert torch.equal(ym, yb) and torch.equal(ym, yp), f"k {k}: bf16 differs between forms"


def test_long_k_split_of_the_128x192_tile(ctx):
    """Two six-wave groups on the 128 x 192 tile, chosen from 32 K stages on:
    ragged M, N and K; int32 equal to the one-group tile's everywhere and to
    the oracle on sampled rows (the full oracle product is too slow here)."""
    M, N, K = 3900, 1120, 4192
    cfg = T.gemm_config_choose(M, N, K)
    assert T.gemm_config_info(cfg) == (128, 192, 2)
    one = next(i for i in range(T.gemm_config_info()) if T.gemm_config_info(i) == (128, 192, 1))
    xq = S.gen_int8((M, K), seed=11)
    wq = S.gen_int8((N, K), seed=12, lo=-128, hi=127)
    sa, sw = S.gen_scales(M, seed=13), S.gen_scales(N, seed=14)
    dx, dw = torch.from_numpy(xq).to(DEV), torch.from_numpy(wq).to(DEV)
    dsa, dsw = torch.from_numpy(sa).to(DEV), torch.from_numpy(sw).to(DEV)
    rows = np.array([0, 1, 127, 128, 1919, 3840, 3899])
    try:
        for k in (0, 5):
            ys, accs = ctx.masked_qgemm(dx, dsa, dw, dsw, k, want_acc=True)
            ctx.set_option(T.OPT_GEMM_CONFIG, one)
            y1, acc1 = ctx.masked_qgemm(dx, dsa, dw, dsw, k, want_acc=True)
            ctx.set_option(T.OPT_GEMM_CONFIG, -1)
            torch.cuda.synchronize()
            assert torch.equal(accs, acc1), f"k {k}: split and one-group sums differ"
            assert torch.equal(ys, y1), f"k {k}: split and one-group bf16 differ"
            ref = O.masked_gemm_i32(xq[rows], wq, k)
            np.testing.assert_array_equal(accs.cpu().numpy()[rows], ref, err_msg=f"k {k}")
    finally:
        ctx.set_option(T.OPT_GEMM_CONFIG, -1)

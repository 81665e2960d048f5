"""GPU parity of the three-stage 128 x 192 and 128 x 96 tiles under the automatic
choice, on seeded shapes the chooser sends to them (one round of tiles, 16 to 31
K stages) and on ragged ones forced onto them.

The ring depth changes only when a stage's copies are waited for, so the bars
are the two-stage tile's: int32 accumulators bit-exact against the oracle on
sampled rows (masked and bit-plane forms) and equal to the two-stage tile's
everywhere, bf16 identical to it.
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


def _entries(shape):
    n = T.gemm_config_info()
    return [i for i in range(n) if T.gemm_config_info(i) == shape]


# (M, N, K): the SANA MLP-up and out-projection shapes, then ragged M and N
# with a ragged last stage (17 stages), 31 stages and exactly 16
AUTO = [(1024, 5600, 2240), (1024, 2240, 2240), (900, 2208, 2080), (900, 4480, 3968),
        (700, 3040, 2048)]
FORCED = [(1, 32, 2048), (130, 96, 2016), (257, 224, 2976), (333, 416, 4064)]


def _check(ctx, M, N, K, cfg_deep, cfg_two, seed):
    xq = S.gen_int8((M, K), seed=seed)
    wq = S.gen_int8((N, K), seed=seed + 1, lo=-128, hi=127)
    sa, sw = S.gen_scales(M, seed=seed + 2), S.gen_scales(N, seed=seed + 3)
    dx, dw = torch.from_numpy(xq).to(DEV), torch.from_numpy(wq).to(DEV)
    dsa, dsw = torch.from_numpy(sa).to(DEV), torch.from_numpy(sw).to(DEV)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    try:
        for k in (0, 3, 7):
            out = {}
            for name, cfg in (("deep", cfg_deep), ("two", cfg_two)):
                ctx.set_option(T.OPT_GEMM_CONFIG, cfg)
                out[name] = ctx.masked_qgemm(dx, dsa, dw, dsw, k, want_acc=True)
                out[name + "_bp"] = ctx.qgemm_bitserial(dx, dsa, dw, dsw, k, want_acc=True)
            torch.cuda.synchronize()
            for form in ("", "_bp"):
                y3, a3 = out["deep" + form]
                y2, a2 = out["two" + form]
                assert torch.equal(a3, a2), f"{M}x{N}x{K} k {k}{form}: sums differ from the two-stage tile"
                assert torch.equal(y3, y2), f"{M}x{N}x{K} k {k}{form}: bf16 differs from the two-stage tile"
            ref = O.masked_gemm_i32(xq[rows], wq, k)
            np.testing.assert_array_equal(out["deep"][1].cpu().numpy()[rows], ref,
                                          err_msg=f"{M}x{N}x{K} k {k}")
            np.testing.assert_array_equal(out["deep_bp"][1].cpu().numpy()[rows],
                                          O.bitplane_gemm_i32(xq[rows], wq, k),
                                          err_msg=f"bit-plane {M}x{N}x{K} k {k}")
    finally:
        ctx.set_option(T.OPT_GEMM_CONFIG, -1)


@pytest.mark.parametrize("M,N,K", AUTO)
def test_auto_deep_ring_bit_exact(ctx, M, N, K):
    cfg = T.gemm_config_choose(M, N, K)
    bm, bn, kg = T.gemm_config_info(cfg)
    print(f"deep ring {M}x{N}x{K}: cfg {cfg} {(bm, bn, kg)}", flush=True)
    same = _entries((bm, bn, kg))
    assert kg == 1 and len(same) == 2 and cfg == same[1], "the chooser takes the three-stage tile here"
    _check(ctx, M, N, K, same[1], same[0], seed=M + N + K)


@pytest.mark.parametrize("M,N,K", FORCED)
@pytest.mark.parametrize("shape", [(128, 192, 1), (128, 96, 1)])
def test_forced_deep_ring_bit_exact(ctx, M, N, K, shape):
    two, deep = _entries(shape)
    print(f"deep ring forced {M}x{N}x{K} {shape}: cfg {deep} vs {two}", flush=True)
    _check(ctx, M, N, K, deep, two, seed=3 * M + N + K)

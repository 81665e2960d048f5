"""The scheduled linear that allocates nothing (static device scratch) against
tabit_scheduled_linear with a caller workspace: identical bf16 outputs, bit for
bit, on two calls in a row (the second smaller, so it runs on scratch that still
holds the first call's data), on the masked INT8, HQ-DM and MXFP4 paths; a call
whose activations exceed the scratch is rejected before anything runs."""
import numpy as np
import pytest
import torch

import tabit_synth as S
import timestep_adaptive_bit_amd as T

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ctx():
    c = T.Context()
    yield c
    c.close()


def _pair(ctx, M, N, K, b, path, fmt, k, seed):
    x = S.gen_activation(M, K, seed=seed).to(DEV)
    w = S.gen_weight(N, K, seed=seed + 1).to(DEV)
    wts = ctx.quantize_weights(w, 0 if path == T.PATH_HQDM else b,
                               int8=fmt == T.FMT_INT8, mx=fmt == T.FMT_MXFP4)
    ctx.set_step_schedule(np.array([[k]], np.uint8), np.array([[fmt]], np.uint8))
    y0 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    y0 = ctx.scheduled_linear_noalloc(0, 0, x, wts, b, y0, path=path)
    ws = torch.empty(T.act_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y1 = ctx.scheduled_linear(0, 0, x, wts, b, ws, path=path)
    torch.cuda.synchronize()
    return y0, y1


@pytest.mark.parametrize("path,fmt,b,big,small", [
    (T.PATH_MASKED, T.FMT_INT8, 0, (4096, 1152, 4608), (300, 640, 1152)),
    (T.PATH_MASKED, T.FMT_INT8, 64, (2048, 3456, 1152), (17, 96, 256)),
    (T.PATH_HQDM, T.FMT_INT8, 64, (1024, 1152, 1152), (64, 256, 512)),
    (T.PATH_MASKED, T.FMT_MXFP4, 32, (4096, 1920, 1920), (96, 256, 384)),
])
def test_noalloc_equals_workspace_linear_twice(ctx, path, fmt, b, big, small):
    for i, (M, N, K) in enumerate((big, small)):
        print(f"noalloc path {path} fmt {fmt} b {b} call {i}: {M}x{N}x{K}", flush=True)
        y0, y1 = _pair(ctx, M, N, K, b, path, fmt, k=3 if fmt == T.FMT_INT8 else 0, seed=10 * i + 3)
        assert not torch.isnan(y0.float()).any()
        assert torch.equal(y0, y1), f"call {i}: no-alloc output differs"


def test_noalloc_rejects_oversize_before_launch(ctx):
    M, N, K = 17776, 1920, 7680                    # 136 MB of INT8 codes > 64 MiB of scratch
    assert T.noalloc_scratch_bytes() == 64 << 20
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((M, N), dtype=torch.bfloat16, device=DEV)
    wts = {"w_q": torch.zeros((N, K), dtype=torch.int8, device=DEV),
           "w_scale": torch.zeros((N,), dtype=torch.float32, device=DEV)}
    ctx.set_step_schedule(np.array([[0]], np.uint8))
    with pytest.raises(T.TabitError) as e:
        ctx.scheduled_linear_noalloc(0, 0, x, wts, 0, y)
    assert e.value.status == T.ESHAPE
    torch.cuda.synchronize()
    assert not y.any()                             # nothing ran

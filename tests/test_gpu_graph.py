"""The schedule runner captured into a HIP graph: every replay matches the eager run.

The library enqueues only kernels on the caller's stream (no allocation, no
memset, no synchronization), so a whole denoising schedule can be captured
once and replayed.  Each replay is checked, with unrelated eager work and
synchronizations between replays.
"""
import ctypes

import numpy as np
import pytest
import torch

import tabit_synth as S
import timestep_adaptive_bit_amd as T

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_schedule_graph_replays_match_eager():
    ctx = T.Context()
    shapes = [(256, 384, 512), (256, 512, 384), (256, 256, 512)]   # (M, N, K) per layer
    steps, b = 3, 32
    k_tab = np.array([[0, 3, 5], [2, 0, 7], [4, 1, 0]], dtype=np.uint8)
    fmt = np.array([[0, 1, 0], [1, 0, 0], [0, 0, 1]], dtype=np.uint8)
    ctx.set_step_schedule(k_tab, fmt)
    weights, ys, layers = [], [], (T.Layer * len(shapes))()
    for li, (M, N, K) in enumerate(shapes):
        wts = ctx.quantize_weights(S.gen_weight(N, K, seed=li).to(DEV), b, int8=True, mx=True)
        weights.append(wts)
        ys.append(torch.empty((M, N), dtype=torch.bfloat16, device=DEV))
        layers[li].M, layers[li].N, layers[li].K = M, N, K
        layers[li].w_q, layers[li].w_scale = wts["w_q"].data_ptr(), wts["w_scale"].data_ptr()
        layers[li].w_fp4, layers[li].w_e8m0 = wts["w_fp4"].data_ptr(), wts["w_e8m0"].data_ptr()
        layers[li].y_bf16 = ys[li].data_ptr()
    xs = [[S.gen_activation(M, K, seed=10 * t + li).to(DEV) for li, (M, _, K) in enumerate(shapes)]
          for t in range(steps)]
    x_ptrs = (ctypes.c_void_p * (steps * len(shapes)))()
    for t in range(steps):
        for li in range(len(shapes)):
            x_ptrs[t * len(shapes) + li] = xs[t][li].data_ptr()
    ws = torch.empty(max(T.act_workspace_bytes(M, K) for M, _, K in shapes), dtype=torch.uint8,
                     device=DEV)

    def run():
        ctx.run_schedule(0, steps, layers, x_ptrs, b, ws)

    run()                                   # eager reference (also warms up)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for y in ys:
            y.fill_(0)                      # eager work between replays
        junk = torch.randn(1024, 1024, device=DEV) @ torch.randn(1024, 1024, device=DEV)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li, (y, r) in enumerate(zip(ys, ref)):
            assert torch.equal(y, r), f"replay {rep}: layer {li} differs from the eager run"
        del junk
    ctx.close()

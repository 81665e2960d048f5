"""GPU parity of the DMPQ selector and the device-gated linear.

Bars: Gamma within the reordering bound of the oracle's exactly rounded sums
(any fp64 summation order of n non-negative terms is within (n - 1) 2^-53 of
the exact sum, relative; Gamma within twice that plus the roundings of the
division), and the per-layer INT8 / 4-bit decisions exact wherever Gamma is
farther than that bound from the threshold; the gated linear identical
(bit for bit) to the host-scheduled linear of the same format, and within the
parity bars of test_gpu_parity against the oracle; a captured step (selector +
gated linears) follows the data-dependent decision on every replay.
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


def _block_io(M, H, seed, delta):
    """Synthetic block input and output: out = in + delta * noise, with a wide
    dynamic range (rows scaled 1e-3 .. 1e4) so the summation order matters."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, H, generator=g)
    x *= torch.logspace(-3, 4, M).reshape(M, 1)[torch.randperm(M, generator=g)]
    y = x + delta * torch.randn(M, H, generator=g) * x.abs().mean(dim=1, keepdim=True)
    return x.to(torch.bfloat16), y.to(torch.bfloat16)


def gamma_rel_bound(n_terms: int) -> float:
    """Relative bound on |Gamma_device - Gamma_oracle|: each sum of n non-negative fp64
    terms, in any order, within (n - 1) 2^-53 / (1 - (n - 1) 2^-53) of the exact sum; the
    oracle's sums are exactly rounded (2^-53 each); one division on each side."""
    u = 2.0 ** -53
    g = (n_terms - 1) * u / (1 - (n_terms - 1) * u)
    return 2 * g + 6 * u


def check_gamma_and_decisions(gamma_dev, fmt_dev, g_ref, thetas, n_terms):
    bound = gamma_rel_bound(n_terms)
    if np.isinf(g_ref) or g_ref == 0.0:
        assert gamma_dev == g_ref
    else:
        assert abs(gamma_dev - g_ref) <= bound * g_ref, (gamma_dev, g_ref, bound)
    want = O.dmpq_select(g_ref, thetas)
    decided = 0
    for l, th in enumerate(np.asarray(thetas, np.float32).astype(np.float64)):
        if np.isinf(g_ref) or abs(g_ref - th) > bound * g_ref:
            assert fmt_dev[l] == want[l], (l, th, g_ref)
            decided += 1
        else:
            assert fmt_dev[l] in (0, 1)
    return decided


@pytest.mark.parametrize("M,H", [(1, 16), (7, 48), (300, 1920), (2500, 5600), (33, 20480),
                                 (17776, 1920)])
def test_dmpq_gamma_within_reordering_bound(ctx, M, H):
    x, y = _block_io(M, H, seed=M + H, delta=0.3)
    g_ref, _, _ = O.dmpq_gamma(S.bf16_bits(x), S.bf16_bits(y))
    # thresholds below, at (the fp32 nearest) and above Gamma, and one ulp-scale offsets
    thetas = np.array([g_ref * 0.5, np.float32(g_ref), g_ref * 2.0,
                       np.nextafter(np.float32(g_ref), np.float32(0)),
                       np.nextafter(np.float32(g_ref), np.float32(np.inf))], np.float32)
    th = torch.from_numpy(thetas).to(DEV)
    fmt = torch.full((len(thetas),), 7, dtype=torch.uint8, device=DEV)
    gamma = torch.zeros(1, dtype=torch.float64, device=DEV)
    print(f"dmpq {M}x{H}", flush=True)
    ctx.dmpq_select(x.to(DEV), y.to(DEV), th, fmt, gamma)
    torch.cuda.synchronize()
    decided = check_gamma_and_decisions(gamma.item(), fmt.cpu().numpy(), g_ref, thetas, M * H)
    assert decided >= 2


def test_dmpq_closed_forms_on_device(ctx):
    x, _ = _block_io(64, 128, seed=5, delta=0.0)
    two = (x.float() * 2).to(torch.bfloat16)
    zero = torch.zeros_like(x)
    gamma = torch.zeros(1, dtype=torch.float64, device=DEV)
    th = torch.tensor([0.5, 1.0, 2.0], device=DEV)
    fmt = torch.empty(3, dtype=torch.uint8, device=DEV)
    for a, b, want in ((x, two, 1.0), (x, x, 0.0), (x, zero, 1.0), (zero, x, float("inf")),
                       (zero, zero, 0.0)):
        ctx.dmpq_select(a.to(DEV), b.to(DEV), th, fmt, gamma)
        torch.cuda.synchronize()
        assert gamma.item() == want
        assert fmt.cpu().numpy().tolist() == O.dmpq_select(want, [0.5, 1.0, 2.0]).tolist()


def _weights(ctx, N, K, b, seed):
    w = S.gen_weight(N, K, seed=seed)
    wts = ctx.quantize_weights(w.to(DEV), b, int8=True, mx=True)
    return w, wts


@pytest.mark.parametrize("path", [T.PATH_MASKED, T.PATH_PLANES])
def test_gated_linear_equals_scheduled_linear(ctx, path):
    M, N, K, b, k = 96, 256, 384, 32, 3
    w, wts = _weights(ctx, N, K, b, seed=2)
    if path == T.PATH_PLANES:
        wts["w_planes"] = ctx.pack_weight_planes(wts["w_q"])
    x = S.gen_activation(M, K, seed=4)
    dx = x.to(DEV)
    ws = torch.empty(T.act_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    ctx.set_step_schedule(np.array([[k], [k]], np.uint8), np.array([[0], [1]], np.uint8))
    for f in (0, 1):
        fmt = torch.tensor([f], dtype=torch.uint8, device=DEV)
        y = ctx.gated_linear(fmt, k, dx, wts, b, ws, path=path)
        y_host = ctx.scheduled_linear(f, 0, dx, wts, b, ws, path=path)
        assert torch.equal(y, y_host), f"fmt {f}: gated differs from the host-scheduled linear"
        yy = y.float().cpu().numpy().astype(np.float64)
        if f == 0:
            ref = O.linear_int8(S.bf16_bits(x), S.bf16_bits(w), b, k)["y"]
            assert np.all(np.abs(yy - ref) <= 1e-2 * np.abs(ref) + 1e-30)
        else:
            ref = O.linear_mxfp4(S.bf16_bits(x), S.bf16_bits(w), b)["y"]
            assert np.all(np.abs(yy - ref) <= 1e-2 * np.abs(ref) + 1e-3 * np.abs(ref).max() + 1e-30)


def test_captured_step_follows_device_decision(ctx):
    """Selector + two gated linears captured once; replays with a stable and an
    unstable block switch the linears between MXFP4 and INT8 on the device."""
    M, H, b, k = 128, 256, 32, 2
    shapes = [(M, 384, H), (M, H, 384)]                    # (M, N, K) of two linears
    thetas = torch.tensor([0.2, 0.2], device=DEV)
    fmt = torch.zeros(2, dtype=torch.uint8, device=DEV)
    gamma = torch.zeros(1, dtype=torch.float64, device=DEV)
    dws = torch.empty(T.dmpq_workspace_bytes(M), dtype=torch.uint8, device=DEV)
    ws = torch.empty(max(T.act_workspace_bytes(m, kk) for m, _, kk in shapes), dtype=torch.uint8,
                     device=DEV)
    wl = [_weights(ctx, n, kk, b, seed=10 + i) for i, (_, n, kk) in enumerate(shapes)]
    xin = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
    xout = torch.empty_like(xin)
    xs = [torch.empty((m, kk), dtype=torch.bfloat16, device=DEV) for m, _, kk in shapes]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device=DEV) for m, n, _ in shapes]

    def step():
        ctx.dmpq_select(xin, xout, thetas, fmt, gamma, dws)
        for i in range(2):
            ctx.gated_linear(fmt[i:i + 1], k, xs[i], wl[i][1], b, ws, y=ys[i])

    cases = [(0.05, 1), (0.6, 0), (0.01, 1)]               # (delta, expected format)
    inputs = []
    for c, (delta, _) in enumerate(cases):
        a, o = _block_io(M, H, seed=50 + c, delta=delta)
        lin = [S.gen_activation(m, kk, seed=60 + 2 * c + i) for i, (m, _, kk) in enumerate(shapes)]
        inputs.append((a, o, lin))

    def load(c):
        a, o, lin = inputs[c]
        xin.copy_(a.to(DEV))
        xout.copy_(o.to(DEV))
        for i in range(2):
            xs[i].copy_(lin[i].to(DEV))

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                             # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(2):
        for c, (delta, want) in enumerate(cases):
            load(c)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            a, o, lin = inputs[c]
            g_ref, _, _ = O.dmpq_gamma(S.bf16_bits(a), S.bf16_bits(o))
            assert check_gamma_and_decisions(gamma.item(), fmt.cpu().numpy(), g_ref,
                                             [0.2, 0.2], M * H) == 2
            f_ref = O.dmpq_select(g_ref, [0.2, 0.2])
            assert f_ref.tolist() == [want, want]
            assert fmt.cpu().numpy().tolist() == f_ref.tolist(), f"replay {rep} case {c}"
            for i in range(2):
                w = wl[i][0]
                yy = ys[i].float().cpu().numpy().astype(np.float64)
                if want == 0:
                    ref = O.linear_int8(S.bf16_bits(lin[i]), S.bf16_bits(w), b, k)["y"]
                    assert np.all(np.abs(yy - ref) <= 1e-2 * np.abs(ref) + 1e-30)
                else:
                    ref = O.linear_mxfp4(S.bf16_bits(lin[i]), S.bf16_bits(w), b)["y"]
                    assert np.all(np.abs(yy - ref) <= 1e-2 * np.abs(ref) + 1e-3 * np.abs(ref).max()
                                  + 1e-30)

"""Full-size parity on every workload's distinct linear shapes.

Shapes, block sizes, formats and k values are the workloads' own (the
configurations bench.py times), and the kernels run in the launch
configuration bench.py uses (the library's automatic tile choice).
Activation and weight codes and scales are compared with the oracle in full,
bit-exact; GEMM outputs on a seeded sample of rows (first and last row
included) at every k the shape's layer-steps use: int32 accumulators
bit-exact, bf16 within 1e-2 relative, MXFP4 outputs within the MXFP4 bound of
test_gpu_parity.  One denoising step of the PixArt-shaped stack also runs
through the native schedule driver, every layer checked.
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
ROWS = 64


@pytest.fixture(scope="module")
def ctx():
    c = T.Context()
    yield c
    c.close()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _distinct(wl):
    """(M, N, K) -> (first layer of that shape, formats used, k values its INT8 steps use)."""
    seen = {}
    for li, layer in enumerate(wl.layers):
        key = (layer.M, layer.N, layer.K)
        fmts = set(int(f) for f in wl.fmt[:, li])
        ks = set(int(k) for k, f in zip(wl.k_bits[:, li], wl.fmt[:, li]) if f == 0)
        if key not in seen:
            seen[key] = (li, fmts, ks)
        else:
            seen[key][1].update(fmts)
            seen[key][2].update(ks)
    return {k: (li, sorted(f), sorted(ks)) for k, (li, f, ks) in seen.items()}


def _sample_rows(M, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(ROWS, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_shapes(ctx, name):
    wl = S.WORKLOADS[name]()
    b = wl.had_block
    for (M, N, K), (li, fmts, ks) in _distinct(wl).items():
        print(f"[{name}] {M}x{N}x{K} layer {li} fmts {fmts} k {ks}", flush=True)
        x = S.gen_activation(M, K, seed=S.activation_seed(0, K))
        w = S.gen_weight(N, K, seed=li)
        xb, wb = S.bf16_bits(x), S.bf16_bits(w)
        dx = x.to(DEV)
        wts = ctx.quantize_weights(w.to(DEV), b, int8=0 in fmts, mx=1 in fmts)
        rows = _sample_rows(M, seed=M + N + K)
        if 0 in fmts:
            wq_ref, sw_ref = O.quantize_weights_int8(wb, b)
            np.testing.assert_array_equal(_np(wts["w_q"]), wq_ref)
            np.testing.assert_array_equal(_np(wts["w_scale"]).view(np.uint32), sw_ref.view(np.uint32))
            xq, sa = ctx.hadamard_quant_act(dx, b)
            xq_ref, sa_ref = O.quantize_act_int8(xb, b)
            np.testing.assert_array_equal(_np(xq), xq_ref)
            np.testing.assert_array_equal(_np(sa).view(np.uint32), sa_ref.view(np.uint32))
            for i, k in enumerate(ks):       # every k this shape's INT8 layer-steps use
                r = rows if i == 0 else np.concatenate([rows[:8], rows[-8:]])
                y, acc = ctx.masked_qgemm(xq, sa, wts["w_q"], wts["w_scale"], k, want_acc=True)
                acc_ref = O.masked_gemm_i32(xq_ref[r], wq_ref, k)
                np.testing.assert_array_equal(_np(acc)[r], acc_ref, err_msg=f"k {k}")
                y_ref = O.dequant(acc_ref, sa_ref[r], sw_ref)
                yy = y.float().cpu().numpy().astype(np.float64)[r]
                assert np.all(np.abs(yy - y_ref) <= 1e-2 * np.abs(y_ref) + 1e-30), f"k {k}"
        if 1 in fmts:
            wf_ref, we_ref = O.mx_quantize_rows(O.bf16_to_f32(wb), b)
            np.testing.assert_array_equal(_np(wts["w_fp4"]), wf_ref)
            np.testing.assert_array_equal(_np(wts["w_e8m0"]), we_ref)
            xf, xe = ctx.hadamard_quant_act(dx, b, T.FMT_MXFP4)
            xf_np, xe_np = _np(xf), _np(xe)
            xf_ref, xe_ref = O.mx_quantize_rows(O.bf16_to_f32(xb[rows]), b)
            np.testing.assert_array_equal(xf_np[rows], xf_ref)
            np.testing.assert_array_equal(xe_np[rows], xe_ref)
            y, _ = ctx.mxfp4_qgemm(xf, xe, wts["w_fp4"], wts["w_e8m0"], 1.0 / max(b, 1))
            y_ref = O.mxfp4_gemm(xf_ref, xe_ref, wf_ref, we_ref, 1.0 / max(b, 1))
            yy = y.float().cpu().numpy().astype(np.float64)[rows]
            err = np.abs(yy - y_ref)
            assert np.all(err <= 1e-2 * np.abs(y_ref) + 1e-3 * np.abs(y_ref).max() + 1e-30)
        del dx, wts


def test_c3_bitplane_every_k_sampled(ctx):
    """The bit-plane path at the SANA-shaped sizes for every k, sampled rows bit-exact."""
    wl = S.c3_sana()
    for (M, N, K), (li, _, _) in _distinct(wl).items():
        x = S.gen_activation(M, K, seed=S.activation_seed(0, K))
        w = S.gen_weight(N, K, seed=li)
        wts = ctx.quantize_weights(w.to(DEV), 0)
        xq, sa = ctx.hadamard_quant_act(x.to(DEV), 0)
        xq_np = _np(xq)
        rows = _sample_rows(M, seed=li)
        wq_np = _np(wts["w_q"])
        for k in range(8):
            _, acc = ctx.qgemm_bitserial(xq, sa, wts["w_q"], wts["w_scale"], k, want_y=False,
                                         want_acc=True)
            np.testing.assert_array_equal(_np(acc)[rows], O.bitplane_gemm_i32(xq_np[rows], wq_np, k))


@pytest.mark.parametrize("step", [0, 19])
def test_pixart_schedule_step_every_layer(ctx, step):
    """One denoising step of the PixArt-Sigma-shaped stack through the native
    driver (tabit_run_schedule, as bench.py runs it): all 112 linears, each with
    its own weights and its (layer, step) k from the installed table; every
    layer's output checked on sampled rows against the oracle's linear."""
    wl = S.c2_pixart_sigma()
    L, b = len(wl.layers), wl.had_block
    ctx.set_step_schedule(wl.k_bits, wl.fmt)
    layers = (T.Layer * L)()
    keep, w_refs = [], []
    for li, layer in enumerate(wl.layers):
        w = S.gen_weight(layer.N, layer.K, seed=li)
        wts = ctx.quantize_weights(w.to(DEV), b)
        y = torch.empty((layer.M, layer.N), dtype=torch.bfloat16, device=DEV)
        layers[li].M, layers[li].N, layers[li].K = layer.M, layer.N, layer.K
        layers[li].w_q, layers[li].w_scale = wts["w_q"].data_ptr(), wts["w_scale"].data_ptr()
        layers[li].y_bf16 = y.data_ptr()
        keep.append((wts, y))
        w_refs.append(O.quantize_weights_int8(S.bf16_bits(w), b))
    xs = {}
    for layer in wl.layers:
        if (layer.M, layer.K) not in xs:
            xs[(layer.M, layer.K)] = S.gen_activation(layer.M, layer.K,
                                                      seed=S.activation_seed(step, layer.K))
    dxs = {key: x.to(DEV) for key, x in xs.items()}
    x_ptrs = (ctypes.c_void_p * L)(*[dxs[(l.M, l.K)].data_ptr() for l in wl.layers])
    ws = torch.empty(max(T.act_workspace_bytes(l.M, l.K) for l in wl.layers), dtype=torch.uint8,
                     device=DEV)
    print(f"pixart step {step}: run_schedule over {L} layers", flush=True)
    ctx.run_schedule(step, 1, layers, x_ptrs, b, ws)
    torch.cuda.synchronize()
    rows = _sample_rows(wl.layers[0].M, seed=100 + step)[:12]
    acts = {key: O.quantize_act_int8(S.bf16_bits(x[rows]), b) for key, x in xs.items()}
    for li, layer in enumerate(wl.layers):
        k = int(wl.k_bits[step, li])
        xq_ref, sa_ref = acts[(layer.M, layer.K)]
        wq_ref, sw_ref = w_refs[li]
        y_ref = O.dequant(O.masked_gemm_i32(xq_ref, wq_ref, k), sa_ref, sw_ref)
        yy = keep[li][1].float().cpu().numpy().astype(np.float64)[rows]
        assert np.all(np.abs(yy - y_ref) <= 1e-2 * np.abs(y_ref) + 1e-30), f"layer {li} k {k}"


# ------------------------------------------------------------ the library's size limits
MAX_M, MAX_K = 65535, 32768      # an operand of 2^31 - 32768 bytes: the largest the ABI accepts
MAX_ROWS = np.array([0, 1, 30001, MAX_M - 2, MAX_M - 1])


def _device_int8(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(-127, 128, shape, dtype=torch.int8, device=DEV, generator=g)


def test_gemm_at_the_size_limits(ctx):
    """K = 32768 (256 stages) and an activation operand just under 2 GiB, so
    every byte offset the kernels form is near the top of the 31-bit range:
    sampled rows (the last ones included) bit-exact against the oracle."""
    N = 96
    xq = _device_int8((MAX_M, MAX_K), seed=21)
    wq_h = S.gen_int8((N, MAX_K), seed=22, lo=-128, hi=127)
    wq = torch.from_numpy(wq_h).to(DEV)
    sa = torch.from_numpy(S.gen_scales(MAX_M, seed=23)).to(DEV)
    sw = torch.from_numpy(S.gen_scales(N, seed=24)).to(DEV)
    x_rows = xq[torch.from_numpy(MAX_ROWS).to(DEV)].cpu().numpy()
    for k in (0, 5):
        _, acc = ctx.masked_qgemm(xq, sa, wq, sw, k, want_y=False, want_acc=True)
        got = acc[torch.from_numpy(MAX_ROWS).to(DEV)].cpu().numpy()
        np.testing.assert_array_equal(got, O.masked_gemm_i32(x_rows, wq_h, k), err_msg=f"k {k}")
        del acc
    del xq
    torch.cuda.empty_cache()


def test_int8_quantizer_at_the_size_limits(ctx):
    """Rows of 32768 elements (two 16-element chunks per thread) over an input
    of 2^31 - 32768 elements: codes and scales of sampled rows bit-exact."""
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    x = torch.randn((MAX_M, MAX_K), dtype=torch.float32, device=DEV, generator=g).to(torch.bfloat16)
    q, s = ctx.hadamard_quant_act(x, 32)
    rows = torch.from_numpy(MAX_ROWS).to(DEV)
    x_bits = x[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    q_ref, s_ref = O.quantize_act_int8(x_bits, 32)
    np.testing.assert_array_equal(q[rows].cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s[rows].cpu().numpy(), s_ref)
    del x, q, s
    torch.cuda.empty_cache()

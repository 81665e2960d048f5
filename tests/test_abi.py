"""C-ABI library: loads, exports every declared symbol, host logic and argument validation.

No test here launches a kernel: every call either touches host state only or
fails validation before its first HIP call, so the suite runs without a GPU.
"""
import ctypes

import numpy as np
import pytest

import tabit_synth as S
import timestep_adaptive_bit_amd as T

FAKE = 0x10000            # 16-byte aligned, never dereferenced (validation fails first)
MISALIGNED = 0x10001


@pytest.fixture(scope="module")
def lib():
    return T.load()


@pytest.fixture
def ctx():
    c = T.Context()
    yield c
    c.close()


def test_every_header_symbol_is_exported(lib):
    names = T.header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
        assert n in T._lib._SIGNATURES, f"binding lacks {n}"


def test_version_and_last_error(lib, ctx):
    assert "gfx950" in T.version()
    assert ctx.last_error() == ""
    assert lib.tabit_last_error(None) == b"null tabit_ctx"
    assert lib.tabit_create(None) == T.EINVAL


def test_schedule_round_trip_all_workloads(ctx):
    for fn in S.WORKLOADS.values():
        w = fn()
        ctx.set_step_schedule(w.k_bits, w.fmt)
        for t in range(w.steps):
            for l in range(0, w.num_layers, 7):
                assert ctx.schedule_lookup(t, l) == (int(w.k_bits[t, l]), int(w.fmt[t, l]))


def test_schedule_errors(ctx):
    with pytest.raises(T.TabitError) as e:
        ctx.schedule_lookup(0, 0)
    assert e.value.status == T.ENOSCHED
    with pytest.raises(T.TabitError) as e:
        ctx.set_step_schedule(np.full((2, 3), 8))
    assert e.value.status == T.ERANGE
    with pytest.raises(T.TabitError) as e:
        ctx.set_step_schedule(np.zeros((2, 3)), np.full((2, 3), 2))
    assert e.value.status == T.EINVAL
    ctx.set_step_schedule(np.zeros((2, 3)))
    assert ctx.schedule_lookup(1, 2) == (0, 0)          # fmt NULL means all INT8
    for t, l in ((-1, 0), (2, 0), (0, 3), (0, -1)):
        with pytest.raises(T.TabitError) as e:
            ctx.schedule_lookup(t, l)
        assert e.value.status == T.ENOSCHED
    st = T.load().tabit_set_step_schedule(ctx.handle, 0, 3, FAKE, None)
    assert st == T.ESHAPE


def _gemm(lib, ctx, fn, **kw):
    a = dict(xq=FAKE, xs=FAKE, wq=FAKE, ws=FAKE, M=64, N=64, K=64, k=0, y=FAKE, acc=None)
    a.update(kw)
    return getattr(lib, fn)(ctx.handle, a["xq"], a["xs"], a["wq"], a["ws"], a["M"], a["N"], a["K"],
                            a["k"], a["y"], a["acc"], None)


@pytest.mark.parametrize("fn", ["tabit_masked_qgemm", "tabit_qgemm_bitserial", "tabit_plane_qgemm"])
def test_gemm_validation(lib, ctx, fn):
    cases = [
        (dict(k=8), T.ERANGE), (dict(k=-1), T.ERANGE),
        (dict(K=33), T.ESHAPE), (dict(K=0), T.ESHAPE), (dict(K=65536), T.ESHAPE),
        (dict(N=48), T.ESHAPE), (dict(N=-32), T.ESHAPE), (dict(M=-1), T.ESHAPE),
        (dict(xq=None), T.EINVAL), (dict(ws=None), T.EINVAL), (dict(y=None, acc=None), T.EINVAL),
        (dict(xq=MISALIGNED), T.EALIGN), (dict(y=FAKE + 8), T.EALIGN),
        (dict(xs=FAKE + 2), T.EALIGN),
        (dict(M=0), T.OK), (dict(N=0), T.OK),        # empty problems are no-ops
        (dict(M=1 << 16, K=32768), T.ESHAPE),         # an operand of 2 GiB
        (dict(N=65536, K=32768), T.ESHAPE),
    ]
    for kw, want in cases:
        assert _gemm(lib, ctx, fn, **kw) == want, (kw, ctx.last_error())
    assert lib.tabit_masked_qgemm(None, FAKE, FAKE, FAKE, FAKE, 1, 32, 32, 0, FAKE, None, None) == T.EINVAL


def test_pack_planes_validation(lib, ctx):
    def p(N=64, K=64, w=FAKE, out=FAKE):
        return lib.tabit_pack_weight_planes(ctx.handle, w, N, K, out, None)
    assert p(w=None) == T.EINVAL
    assert p(out=None) == T.EINVAL
    assert p(N=48) == T.ESHAPE
    assert p(K=48) == T.ESHAPE
    assert p(K=65536) == T.ESHAPE
    assert p(N=65536, K=32768) == T.ESHAPE
    assert p(out=FAKE + 4) == T.EALIGN
    assert p(N=0) == T.OK
    assert lib.tabit_pack_weight_planes(None, FAKE, 32, 32, FAKE, None) == T.EINVAL
    assert T.weight_planes_bytes(1152, 1152) == 1152 * 1152
    assert T.weight_planes_bytes(64, 160) == 64 * 256          # K padded to whole 128-code stages
    assert T.weight_planes_bytes(0, 64) == 0


def test_dmpq_validation(lib, ctx):
    def d(M=4, H=64, th=FAKE, n=2, fmt=FAKE, g=FAKE, ws=FAKE, nb=1 << 20, xi=FAKE):
        return lib.tabit_dmpq_select(ctx.handle, xi, FAKE, M, H, th, n, fmt, g, ws, nb, None)
    assert d(xi=None) == T.EINVAL
    assert d(th=None) == T.EINVAL                      # n_layers > 0 needs theta and fmt
    assert d(n=0, g=None) == T.EINVAL                  # nothing to write
    assert d(n=-1) == T.EINVAL
    assert d(M=0) == T.ESHAPE
    assert d(H=40) == T.ESHAPE
    assert d(H=65536) == T.ESHAPE
    assert d(nb=16) == T.ESHAPE                        # workspace below 16 bytes per row
    assert d(g=FAKE + 4) == T.EALIGN
    assert T.dmpq_workspace_bytes(100) >= 1600 and T.dmpq_workspace_bytes(0) == 0


def test_gated_linear_validation(lib, ctx):
    def g(fmt=FAKE, k=0, path=0, M=8, N=32, K=64, b=0, wq=FAKE, wf=FAKE, ws=FAKE, nb=1 << 20):
        return lib.tabit_gated_linear(ctx.handle, fmt, k, path, FAKE, M, N, K, b, wq, FAKE, wf, FAKE,
                                      ws, nb, FAKE, None)
    assert g(fmt=None) == T.EINVAL
    assert g(wf=None) == T.EINVAL                      # both weight formats are required
    assert g(path=1) == T.EINVAL
    assert g(k=8) == T.ERANGE
    assert g(b=64) == T.ERANGE                         # the MXFP4 branch needs b in {0, 32}
    assert g(N=48) == T.ESHAPE
    assert g(nb=8) == T.ESHAPE
    assert g(ws=MISALIGNED) == T.EALIGN
    assert g(M=0) == T.OK


def test_gelu_quant_validation(lib, ctx):
    def q(M=4, K=64, b=0, fmt=0, xq=FAKE, sc=FAKE):
        return lib.tabit_gelu_quant_act(ctx.handle, FAKE, M, K, b, fmt, xq, sc, None)
    assert q(xq=None) == T.EINVAL
    assert q(fmt=2) == T.EINVAL
    assert q(b=16) == T.ERANGE
    assert q(fmt=1, b=64) == T.ERANGE                  # MXFP4 takes b in {0, 32}
    assert q(K=48) == T.ESHAPE
    assert q(xq=MISALIGNED) == T.EALIGN
    assert q(M=0) == T.OK


def test_run_schedule_chain_validation(lib, ctx):
    """Chained inputs (MLP up -> GELU -> down) are validated before any launch."""
    ctx.set_step_schedule(np.zeros((1, 2), np.uint8))

    def run(from1=1, act1=T.ACT_GELU, k1=256, path=0, m1=8):
        layers = (T.Layer * 2)()
        layers[0].M, layers[0].N, layers[0].K = 8, 256, 64
        layers[1].M, layers[1].N, layers[1].K = m1, 64, k1
        for l in layers:
            l.w_q, l.w_scale, l.y_bf16 = FAKE, FAKE, FAKE
        layers[1].input_from, layers[1].input_act = from1, act1
        x_ptrs = (ctypes.c_void_p * 2)(FAKE, None)
        return lib.tabit_run_schedule(ctx.handle, 0, 1, layers, 2, x_ptrs, 0, path, FAKE, 1 << 30,
                                      None, None)
    assert run(from1=2) == T.EINVAL                    # not an earlier layer
    assert run(from1=-1) == T.EINVAL
    assert run(act1=7) == T.EINVAL
    assert run(k1=128) == T.ESHAPE                     # layer 0's output is 8 x 256
    assert run(m1=16) == T.ESHAPE
    assert run(path=4) == T.EINVAL                     # no GELU-fused HQ-DM quantizer
    assert run(from1=0) == T.EINVAL                    # external input missing (NULL)


def test_hqdm_validation(lib, ctx):
    def q(M=4, K=64, b=32, hi=FAKE, lo=FAKE, sc=FAKE):
        return lib.tabit_hqdm_quant_act(ctx.handle, FAKE, M, K, b, hi, lo, sc, None)
    assert q(lo=None) == T.EINVAL
    assert q(b=16) == T.ERANGE
    assert q(K=48) == T.ESHAPE
    assert q(hi=MISALIGNED) == T.EALIGN
    assert q(M=0) == T.OK

    def g(M=8, N=32, K=64, k=0, lo=FAKE, y=FAKE, acc=None):
        return lib.tabit_hqdm_qgemm(ctx.handle, FAKE, lo, FAKE, FAKE, FAKE, M, N, K, k, y, acc, None)
    assert g(lo=None) == T.EINVAL
    assert g(y=None) == T.EINVAL
    assert g(k=8) == T.ERANGE
    assert g(N=40) == T.ESHAPE
    assert g(lo=MISALIGNED) == T.EALIGN
    assert g(M=0) == T.OK
    assert T.hqdm_config_info() >= 1


def test_quant_act_validation(lib, ctx):
    def q(M=4, K=64, b=0, fmt=0, x=FAKE, xq=FAKE, xs=FAKE):
        return lib.tabit_hadamard_quant_act(ctx.handle, x, M, K, b, fmt, xq, xs, None)
    assert q(b=16) == T.ERANGE
    assert q(b=256, K=512) == T.ERANGE
    assert q(b=64, K=96) == T.ESHAPE
    assert q(K=48) == T.ESHAPE
    assert q(K=65536) == T.ESHAPE
    assert q(fmt=2) == T.EINVAL
    assert q(fmt=1, b=64) == T.ERANGE
    assert q(x=None) == T.EINVAL
    assert q(xq=MISALIGNED) == T.EALIGN
    assert q(M=0) == T.OK


def test_quantize_weights_validation(lib, ctx):
    def w(N=32, K=64, b=0, wq=FAKE, ws=FAKE, wf=None, we=None):
        return lib.tabit_quantize_weights(ctx.handle, FAKE, N, K, b, wq, ws, wf, we, None)
    assert w(wq=None) == T.EINVAL                       # pair given half
    assert w(wq=None, ws=None) == T.EINVAL              # nothing requested
    assert w(wf=FAKE) == T.EINVAL
    assert w(wf=FAKE, we=FAKE, b=64) == T.ERANGE        # MX copy needs b in {0, 32}
    assert w(b=128, K=64) == T.ESHAPE
    assert w(N=0) == T.OK


def test_mxfp4_validation(lib, ctx):
    def m(M=32, N=32, K=64, y=FAKE, acc=None, s=1.0):
        return lib.tabit_mxfp4_qgemm(ctx.handle, FAKE, FAKE, FAKE, FAKE, M, N, K, s, y, acc, None)
    assert m(K=40) == T.ESHAPE
    assert m(N=40) == T.ESHAPE
    assert m(y=None) == T.EINVAL
    assert m(s=float("nan")) == T.EINVAL
    assert m(M=0) == T.OK


def test_scheduled_linear_validation(lib, ctx):
    def s(step=0, layer=0, path=0, M=8, N=32, K=64, b=0, wq=FAKE, ws_=FAKE, wf=None, we=None,
          ws=FAKE, nbytes=1 << 20):
        return lib.tabit_scheduled_linear(ctx.handle, step, layer, path, FAKE, M, N, K, b, wq, ws_,
                                          wf, we, ws, nbytes, FAKE, None)
    assert s() == T.ENOSCHED
    ctx.set_step_schedule(np.array([[0, 3]]), np.array([[0, 1]]))
    assert s(path=5) == T.EINVAL
    assert s(path=2) == T.EINVAL                         # 2 names the MXFP4 GEMM only in autotune
    assert s(step=1) == T.ENOSCHED
    assert s(nbytes=10) == T.ESHAPE
    assert s(wq=None) == T.EINVAL                        # INT8 step without INT8 weights
    assert s(layer=1) == T.EINVAL                        # MXFP4 step without the MX copy
    assert s(layer=1, wf=FAKE, we=FAKE, b=64) == T.ERANGE
    assert s(ws=MISALIGNED) == T.EALIGN
    # every operand is checked before the quantizer is enqueued (these calls would
    # otherwise launch it on the fake pointers)
    assert s(wq=MISALIGNED) == T.EALIGN
    assert s(ws_=FAKE + 2) == T.EALIGN
    assert s(layer=1, wf=MISALIGNED, we=FAKE) == T.EALIGN
    assert s(M=1 << 16, K=1 << 15, nbytes=1 << 40) == T.ESHAPE        # M*K = 2^31: over 2 GiB
    assert s(path=3, N=1 << 24, K=32, nbytes=1 << 20) == T.ESHAPE     # plane-major copy over 2 GiB
    assert s(M=0) == T.OK


def test_noalloc_validation(lib, ctx):
    """The no-alloc linear validates like the workspace one and rejects activations
    larger than its static scratch, all before any HIP call."""
    def s(step=0, layer=0, path=0, M=8, N=32, K=64, b=0, wq=FAKE, ws_=FAKE, wf=None, we=None):
        return lib.tabit_scheduled_linear_noalloc(ctx.handle, step, layer, path, FAKE, M, N, K, b,
                                                  wq, ws_, wf, we, FAKE, None)
    assert lib.tabit_noalloc_scratch_bytes() == 64 << 20
    assert s() == T.ENOSCHED
    ctx.set_step_schedule(np.array([[0, 3]]), np.array([[0, 1]]))
    assert s(path=5) == T.EINVAL
    assert s(wq=None) == T.EINVAL
    assert s(wq=MISALIGNED) == T.EALIGN
    assert s(layer=1) == T.EINVAL
    assert s(M=8192, K=8192) == T.ESHAPE                              # 64 MiB of codes + scales
    assert s(M=4096, K=8192, path=4) == T.ESHAPE                      # HQ-DM: two planes
    assert s(layer=1, wf=FAKE, we=FAKE, b=32, M=16384, K=8192) == T.ESHAPE   # MX: 64 + 4 MiB
    assert s(M=0) == T.OK


def test_workspace_bytes():
    for M, K in ((1, 32), (64, 1152), (17776, 7680)):
        n = T.act_workspace_bytes(M, K)
        assert n >= M * K + 4 * M and n % 256 == 0
    assert T.act_workspace_bytes(0, 64) == 0


def test_mfma_probe_validation(ctx, lib):
    """Argument errors come back before any HIP call."""
    out = ctypes.c_double()
    fake = ctypes.c_void_p(4096)
    assert lib.tabit_mfma_peak_probe(ctx._h, 2, 10, fake, 1 << 20, ctypes.byref(out), None) == T.EINVAL
    assert lib.tabit_mfma_peak_probe(ctx._h, 0, 0, fake, 1 << 20, ctypes.byref(out), None) == T.ERANGE
    assert lib.tabit_mfma_peak_probe(ctx._h, 0, 10, None, 1 << 20, ctypes.byref(out), None) == T.EINVAL
    assert lib.tabit_mfma_peak_probe(ctx._h, 0, 10, fake, 1 << 20, None, None) == T.EINVAL
    assert lib.tabit_mfma_peak_probe(None, 0, 10, fake, 1 << 20, ctypes.byref(out), None) == T.EINVAL
    assert lib.tabit_mfma_probe_sink_ints(256) >= 256 * 64


def test_options_and_configs(ctx):
    n = T.gemm_config_info()
    assert n >= 1
    for i in range(n):
        bm, bn, sk = T.gemm_config_info(i)
        assert bm % 16 == 0 and bn % 16 == 0 and sk >= 1
        ctx.set_option(T.OPT_GEMM_CONFIG, i)
    ctx.set_option(T.OPT_GEMM_CONFIG, -1)
    with pytest.raises(T.TabitError):
        ctx.set_option(T.OPT_GEMM_CONFIG, n)
    with pytest.raises(T.TabitError):
        ctx.set_option(99, 0)
    for M, N, K in ((64, 1152, 1152), (4096, 3456, 1152), (17776, 7680, 1920)):
        assert 0 <= T.gemm_config_choose(M, N, K) < n
    npl = T.plane_config_info()
    assert npl >= 1
    for i in range(npl):
        bm, bn, kg = T.plane_config_info(i)
        assert bm % 32 == 0 and bn % 32 == 0 and kg >= 1
        ctx.set_option(T.OPT_PLANE_CONFIG, i)
    # few tiles (64 tokens): a K-split tile; a full chip of tiles: none
    assert T.plane_config_info(T.plane_config_choose(64, 1152, 1152, 256))[2] > 1
    assert T.plane_config_info(T.plane_config_choose(4096, 4608, 1152, 256))[2] == 1
    with pytest.raises(T.TabitError):
        T.plane_config_choose(64, 1152, 0)
    ctx.set_option(T.OPT_PLANE_CONFIG, -1)
    with pytest.raises(T.TabitError):
        ctx.set_option(T.OPT_PLANE_CONFIG, npl)


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(T._lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(T._lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        T._lib.load()


def test_mxfp4_chooser_rules():
    """The MXFP4 chooser takes the 256x256 tile on the wide CogVideoX linears and
    256x192 where N = 1920 (K a multiple of 128), never 256x256 for K that is not
    (its byte-scale variant spills), and always a valid index; negative sizes and
    K < 1 are rejected."""
    import random
    n = T.mxfp4_config_info()
    info = [T.mxfp4_config_info(i) for i in range(n)]
    for (M, N, K) in [(17776, 7680, 1920), (17776, 5760, 1920)]:
        assert info[T.mxfp4_config_choose(M, N, K)] == (256, 256), (M, N, K)
    for (M, N, K) in [(17776, 1920, 7680), (17776, 1920, 1920)]:
        assert info[T.mxfp4_config_choose(M, N, K)] == (256, 192), (M, N, K)
    rng = random.Random(11)
    for _ in range(2000):
        M = rng.choice([1, 17, 64, 256, 1024, 4096, 17776]) + rng.randrange(0, 300)
        N = 32 * rng.randrange(1, 320)
        K = 32 * rng.randrange(1, 400)
        c = T.mxfp4_config_choose(M, N, K, rng.choice([0, 80, 256, 304]))
        assert 0 <= c < n
        if K % 128:
            assert info[c] != (256, 256), (M, N, K)
    for bad in [(-1, 32, 32), (32, -1, 32), (32, 32, 0)]:
        with pytest.raises(T.TabitError):
            T.mxfp4_config_choose(*bad)


def test_int8_chooser_split_rules():
    """Over seeded random shapes: a K-split tile only when the same tile's
    workgroups fit in one round over the CUs, two-group tiles only from 32 K
    stages on, and whenever a split is taken it walks fewer stages per group
    than the unsplit tile would."""
    import random
    rng = random.Random(5)
    n = T.gemm_config_info()
    info = [T.gemm_config_info(i) for i in range(n)]
    for _ in range(2000):
        M = rng.choice([1, 3, 17, 64, 100, 256, 512, 768, 1024, 2048, 4096, 17776]) + rng.randrange(0, 64)
        N = 32 * rng.randrange(1, 320)
        K = 32 * rng.randrange(1, 1024)
        cus = rng.choice([0, 80, 256, 304])
        c = T.gemm_config_choose(M, N, K, cus)
        assert 0 <= c < n
        bm, bn, kg = info[c]
        if kg == 1:
            continue
        tiles = -(-M // bm) * -(-N // bn)
        assert tiles <= (cus or 256), (M, N, K, cus, info[c])
        stages = -(-K // 128)
        assert -(-stages // kg) < stages or stages == 1, (M, N, K, info[c])
        if kg == 2:
            assert stages >= 32, (M, N, K, info[c])


def test_int8_chooser_deep_ring_rule():
    """The three-stage 128 x 192 and 128 x 96 tiles (the second table entry of
    each shape with one K group) replace the two-stage tile only when its
    workgroups fit in one round and K has 16 to 31 stages; from 32 stages the
    two-group split takes over, below 16 the two-stage tile stays."""
    n = T.gemm_config_info()
    info = [T.gemm_config_info(i) for i in range(n)]

    def entries(shape):
        return [i for i in range(n) if info[i] == shape]

    two192, deep192 = entries((128, 192, 1))
    two96, deep96 = entries((128, 96, 1))
    assert T.gemm_config_choose(1024, 5600, 2240, 256) == deep192    # 18 stages, 240 tiles
    assert T.gemm_config_choose(1024, 2240, 2240, 256) == deep96     # 18 stages, 192 tiles
    assert T.gemm_config_choose(4096, 1152, 1152, 256) == two192     # 9 stages
    assert T.gemm_config_choose(4096, 1280, 1280, 256) == two192     # 10 stages
    assert info[T.gemm_config_choose(4096, 1152, 4608, 256)] == (128, 192, 2)   # 36 stages
    import random
    rng = random.Random(9)
    for _ in range(2000):
        M = rng.choice([1, 64, 256, 512, 1024, 2048, 4096]) + rng.randrange(0, 64)
        N = 32 * rng.randrange(1, 320)
        K = 32 * rng.randrange(1, 1024)
        cus = rng.choice([0, 80, 256, 304])
        c = T.gemm_config_choose(M, N, K, cus)
        if c in (deep192, deep96):
            bm, bn, _ = info[c]
            stages = -(-K // 128)
            assert 16 <= stages < 32, (M, N, K, cus)
            assert -(-M // bm) * -(-N // bn) <= (cus or 256), (M, N, K, cus)

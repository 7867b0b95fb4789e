"""GPU parity of the HIP path against the CPU oracle (MI355X only).

Tolerance (floating point): max |Y_gpu - Y_ref| <= 1e-2 and
||Y_gpu - Y_ref||_F / ||Y_ref||_F <= 1e-3, with Y_ref the float64 oracle and
Y_gpu the fp16 output (fp32 accumulation, one rounding to fp16).
Integer / byte work (format expansion, exact pins) is compared bitwise.
"""
import numpy as np
import pytest

import oracle
import swm_workloads as wl

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
REL_FRO = 1e-3


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(Y_gpu, Y_ref, what=""):
    Yg = np.asarray(Y_gpu, dtype=np.float64)
    err = np.abs(Yg - Y_ref)
    assert np.all(np.isfinite(Yg)), what
    mx = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(Y_ref))
    rel = float(np.linalg.norm(Yg - Y_ref)) / den if den > 0 else float(np.linalg.norm(Yg))
    assert mx <= MAX_ABS, f"{what}: max abs err {mx}"
    assert rel <= REL_FRO, f"{what}: rel Frobenius err {rel}"


def _compress(swm, W, mask):
    return swm.sparse_compress(W, mask)


# ------------------------------------------------------------------ tiny workload
@pytest.mark.parametrize("N", [1, 3, 8])
def test_tiny_spmm(gpu_lib, N):
    swm = gpu_lib
    W, mask, X = wl.tiny()
    f = _compress(swm, W, mask)
    Y = swm.spmm(f, _t(X[:N]))
    assert_close(_np(Y), oracle.masked_matmul(W, mask, X[:N]), f"tiny N={N}")


def test_decompress_round_trip_bitwise(gpu_lib):
    swm = gpu_lib
    for (W, mask) in [wl.tiny()[:2], wl.pruned_weight(91, 0, 200, 333, 0.5)]:
        f = _compress(swm, W, mask)
        D = _np(swm.decompress(f)).view(np.uint16)
        want = np.where(mask, W.view(np.uint16), np.uint16(0))
        assert np.array_equal(D, want)


def test_export_matches_oracle_encoder(gpu_lib):
    swm = gpu_lib
    W, mask, _ = wl.tiny()
    f = _compress(swm, W, mask)
    blob = f.export()
    assert blob == oracle.tcb_encode(W, mask).blob()
    g = swm.format_import(blob)
    assert np.array_equal(_np(swm.decompress(g)).view(np.uint16), _np(swm.decompress(f)).view(np.uint16))


# ------------------------------------------------------------------ exact pins
def test_identity_weight_returns_x_bitwise(gpu_lib):
    swm = gpu_lib
    K = 200
    W = np.eye(K, dtype=np.float16)
    X = np.random.default_rng(1).standard_normal((16, K)).astype(np.float16)
    f = _compress(swm, W, np.eye(K, dtype=bool))
    Y = _np(swm.spmm(f, _t(X)))
    assert np.array_equal(Y.view(np.uint16), X.view(np.uint16))


def test_permutation_weight_bitwise(gpu_lib):
    swm = gpu_lib
    K = 130
    g = np.random.default_rng(2)
    perm = g.permutation(K)
    P = np.zeros((K, K), dtype=np.float16)
    P[np.arange(K), perm] = 1
    X = g.standard_normal((5, K)).astype(np.float16)
    f = _compress(swm, P, P != 0)
    Y = _np(swm.spmm(f, _t(X)))
    assert np.array_equal(Y.view(np.uint16), X[:, perm].view(np.uint16))


def test_one_hot_activations_pick_columns_bitwise(gpu_lib):
    swm = gpu_lib
    W, mask = wl.pruned_weight(92, 0, 128, 96, 0.5)
    f = _compress(swm, W, mask)
    ks = [0, 1, 17, 63, 64, 95]
    X = np.zeros((len(ks), 96), dtype=np.float16)
    for n, k in enumerate(ks):
        X[n, k] = 1
    Y = _np(swm.spmm(f, _t(X))).view(np.uint16)
    for n, k in enumerate(ks):
        assert np.array_equal(Y[n], np.where(mask[:, k], W[:, k].view(np.uint16), 0))


def test_all_zero_mask_gives_zero(gpu_lib):
    swm = gpu_lib
    W, _ = wl.pruned_weight(93, 0, 100, 300, 0.5)
    f = _compress(swm, W, np.zeros(W.shape, dtype=bool))
    X = np.random.default_rng(3).standard_normal((7, 300)).astype(np.float16)
    Y = _np(swm.spmm(f, _t(X)))
    assert np.all(Y == 0)


# ------------------------------------------------------------------ ragged shapes and N sweep
@pytest.mark.parametrize("M,K,N", [
    (1, 1, 1), (65, 129, 2), (300, 1000, 16), (64, 4096, 5), (130, 72, 17), (77, 333, 9), (513, 260, 33),
    (77, 333, 20), (40, 1000, 32), (17, 4100, 31),   # N = 17..32: two token groups (unaligned K: two passes)
])
def test_ragged_shapes(gpu_lib, M, K, N):
    swm = gpu_lib
    W, mask = wl.pruned_weight(94, M * 10 + K, M, K, 0.5)
    X = np.random.default_rng(M + K + N).standard_normal((N, K)).astype(np.float16)
    f = _compress(swm, W, mask)
    Y = _np(swm.spmm(f, _t(X)))
    assert_close(Y, oracle.masked_matmul(W, mask, X), f"{M}x{K}x{N}")


# Decode schedules: K sets the tiles per wave (segments of two tiles per wave:
# 1, 2, 3, 4, 6, 8; odd counts end on a one-tile segment, K % 64 != 0 ends on
# a partial tile) and the sparsity sets how many 1 KiB loads a segment needs.
@pytest.mark.parametrize("K,s,N", [
    (2048, 0.5, 1), (4096, 0.5, 16), (4104, 0.5, 3), (6144, 0.8, 7), (8192, 0.0, 16), (8192, 1.0, 2),
    (11008, 0.5, 4), (11008, 0.3, 16), (16384, 0.5, 1), (16384, 0.05, 9), (1024, 0.5, 16), (520, 0.5, 5),
    (4096, 0.5, 32), (11008, 0.5, 24), (16384, 0.5, 17), (520, 0.5, 32), (8192, 1.0, 20),
])
def test_decode_schedules(gpu_lib, K, s, N):
    swm = gpu_lib
    M = 40
    W, mask = wl.pruned_weight(96, K // 8 + int(100 * s), M, K, s)
    X = np.random.default_rng(K + N).standard_normal((N, K)).astype(np.float16)
    f = _compress(swm, W, mask)
    Y = _np(swm.spmm(f, _t(X)))
    assert_close(Y, oracle.masked_matmul(W, mask, X), f"{M}x{K}x{N} s={s}")
    if s == 1.0:
        assert np.all(Y == 0)


@pytest.mark.parametrize("N", [6, 28])
def test_strided_activations_and_outputs(gpu_lib, N):
    import torch
    swm = gpu_lib
    W, mask = wl.pruned_weight(95, 0, 192, 256, 0.5)
    X = np.random.default_rng(4).standard_normal((N, 256)).astype(np.float16)
    f = _compress(swm, W, mask)
    Xbig = torch.zeros((N, 304), dtype=torch.float16, device="cuda")
    Xbig[:, :256] = _t(X)
    Ybig = torch.full((N, 200), 7.0, dtype=torch.float16, device="cuda")
    swm.spmm(f, Xbig[:, :256], Ybig[:, :192])
    Yb = _np(Ybig)
    assert_close(Yb[:, :192], oracle.masked_matmul(W, mask, X), "strided")
    assert np.all(Yb[:, 192:] == 7.0)  # columns beyond M untouched


# ------------------------------------------------------------------ full-size decode (q_proj)
@pytest.fixture(scope="module")
def qproj(gpu_lib):
    W, mask, X = wl.decode_qproj(16)
    return W, mask, X, gpu_lib.sparse_compress(W, mask)


@pytest.mark.parametrize("N", [1, 8, 16])
def test_qproj_decode(gpu_lib, qproj, N):
    W, mask, X, f = qproj
    Y = _np(gpu_lib.spmm(f, _t(X[:N])))
    assert_close(Y, oracle.masked_matmul(W, mask, X[:N]), f"q_proj N={N}")


@pytest.mark.parametrize("N", [24, 32])
def test_qproj_decode_two_token_groups(gpu_lib, N):
    W, mask, X = wl.decode_qproj(32)
    f = gpu_lib.sparse_compress(W, mask)
    Y = _np(gpu_lib.spmm(f, _t(X[:N])))
    assert_close(Y, oracle.masked_matmul(W, mask, X[:N]), f"q_proj N={N}")


def test_qproj_deterministic(gpu_lib, qproj):
    W, mask, X, f = qproj
    a = _np(gpu_lib.spmm(f, _t(X)))
    b = _np(gpu_lib.spmm(f, _t(X)))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("N", [1, 8, 16])
def test_qproj_dense_gemm(gpu_lib, qproj, N):
    W, mask, X, _ = qproj
    Y = _np(gpu_lib.dense_gemm(_t(W), _t(X[:N])))
    assert_close(Y, oracle.masked_matmul(W, None, X[:N]), f"dense q_proj N={N}")


# ------------------------------------------------------------------ spMspV (down_proj, SiLU-gated x)
@pytest.fixture(scope="module")
def down(gpu_lib):
    W, mask, x = wl.spmspv_down(4, 0.3)
    return W, mask, x, gpu_lib.sparse_compress(W, mask)


@pytest.mark.parametrize("n", [1, 4])
def test_spmspv_down(gpu_lib, down, n):
    W, mask, x, f = down
    frac = float(np.mean(x[:n] == 0))
    assert 0.6 < frac < 0.8
    y = _np(gpu_lib.spmspv(f, _t(x[:n])))
    assert_close(y, oracle.masked_matmul_skip(W, mask, x[:n]), f"spmspv n={n}")
    y2 = _np(gpu_lib.spmm(f, _t(x[:n])))
    assert_close(y2, oracle.masked_matmul(W, mask, x[:n]), f"spmm on sparse x n={n}")


def test_spmspv_zero_and_dense_inputs(gpu_lib, down):
    W, mask, x, f = down
    z = np.zeros((2, W.shape[1]), dtype=np.float16)
    z[1, 5] = np.float16(-0.0)
    assert np.all(_np(gpu_lib.spmspv(f, _t(z))) == 0)
    xd = np.random.default_rng(5).standard_normal((3, W.shape[1])).astype(np.float16)
    a = _np(gpu_lib.spmspv(f, _t(xd))).view(np.uint16)
    b = _np(gpu_lib.spmm(f, _t(xd))).view(np.uint16)
    assert np.array_equal(a, b)  # nothing to skip: identical arithmetic


# ------------------------------------------------------------------ spMspV over the column-run encoding
@pytest.fixture(scope="module")
def down_skip(gpu_lib, down):
    W, mask, x, f = down
    g = gpu_lib.format_import(f.export())
    nbytes = g.enable_skipping()
    assert nbytes > 0 and g.enable_skipping() == nbytes  # idempotent
    return W, mask, x, g


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_spmspv_skip_down(gpu_lib, down_skip, n):
    # n <= 2: the skipping kernel; n = 3, 4: the full product on the tiled
    # format.  The skipping kernel itself serves up to four tokens through
    # spmspv_threshold with tau = 0 (the same activations, nothing dropped).
    W, mask, x, g = down_skip
    ref = oracle.masked_matmul_skip(W, mask, x[:n])
    y = _np(gpu_lib.spmspv(g, _t(x[:n])))
    assert_close(y, ref, f"spmspv n={n}")
    yc = _np(gpu_lib.spmspv_threshold(g, _t(x[:n]), 0.0))
    assert_close(yc, ref, f"column-run kernel n={n}")
    if n <= 2:
        assert np.array_equal(y.view(np.uint16), yc.view(np.uint16))
    else:
        assert np.array_equal(y.view(np.uint16), _np(gpu_lib.spmm(g, _t(x[:n]))).view(np.uint16))


def test_compress_with_skipping_flag(gpu_lib, down):
    # SWM_CFG_SKIPPING at compress time gives the same handle as
    # enable_skipping afterwards: same encoding size, bitwise the same results
    W, mask, x, f = down
    h = gpu_lib.sparse_compress(W, mask, skipping=True)
    g = gpu_lib.sparse_compress(W, mask)
    nb = g.enable_skipping()
    assert h.enable_skipping() == nb  # already attached: idempotent, same size
    for n in (1, 2):
        a = _np(gpu_lib.spmspv(h, _t(x[:n]))).view(np.uint16)
        b = _np(gpu_lib.spmspv(g, _t(x[:n]))).view(np.uint16)
        assert np.array_equal(a, b)
        assert_close(a.view(np.float16), oracle.masked_matmul_skip(W, mask, x[:n]), f"flag n={n}")
    assert h.export() == f.export()  # the tiled format is unchanged


def test_spmspv_skip_repeatable_and_deterministic(gpu_lib, down_skip):
    # every sum runs in a fixed order: calls in a row agree bitwise
    W, mask, x, g = down_skip
    xs = _t(x[:4])
    ys = [_np(gpu_lib.spmspv_threshold(g, xs, 0.0)).view(np.uint16) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
    y2 = [_np(gpu_lib.spmspv(g, _t(x[:2]))).view(np.uint16) for _ in range(2)]
    assert np.array_equal(y2[0], y2[1])
    y1 = _np(gpu_lib.spmspv(g, _t(x[:1])))  # n changes between calls on one handle
    assert_close(y1, oracle.masked_matmul_skip(W, mask, x[:1]), "after n=4")


def test_spmspv_skip_graph_replays(gpu_lib, down_skip):
    # the captured launches replay with new activations (x changes between
    # replays) and eager calls in between; every replay equals the eager call
    import torch
    W, mask, x, g = down_skip
    n = 2
    xb = _t(x[:n])
    yb = torch.empty((n, W.shape[0]), dtype=torch.float16, device="cuda")
    gpu_lib.spmspv(g, xb, yb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu_lib.spmspv(g, xb, yb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    for rep in range(4):
        xr = x[:n].copy()
        xr[:, rng.random(W.shape[1]) < 0.3] = 0
        xb.copy_(_t(xr))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_graph = yb.cpu().numpy().copy()
        y_eager = _np(gpu_lib.spmspv(g, _t(xr)))  # eager call between replays
        assert np.array_equal(y_graph.view(np.uint16), y_eager.view(np.uint16)), f"replay {rep}"
        assert_close(y_graph, oracle.masked_matmul_skip(W, mask, xr), f"replay {rep}")


def test_spmspv_skip_zero_dense_and_fallback(gpu_lib, down_skip):
    W, mask, x, g = down_skip
    z = np.zeros((3, W.shape[1]), dtype=np.float16)
    z[1, 7] = np.float16(-0.0)
    # nothing active: +0 everywhere, through the skipping kernel (n = 2, and
    # n = 3 via the threshold call) and the full product (n = 3)
    assert np.all(_np(gpu_lib.spmspv(g, _t(z[:2]))).view(np.uint16) == 0)
    assert np.all(_np(gpu_lib.spmspv_threshold(g, _t(z), 0.0)).view(np.uint16) == 0)
    assert np.all(_np(gpu_lib.spmspv(g, _t(z))) == 0)
    xd = np.random.default_rng(6).standard_normal((4, W.shape[1])).astype(np.float16)
    assert_close(_np(gpu_lib.spmspv(g, _t(xd))), oracle.masked_matmul(W, mask, xd), "all columns active")
    x5 = x[:4].copy()
    x5 = np.concatenate([x5, x[:1]], axis=0)  # n = 5: the full-product path
    assert_close(_np(gpu_lib.spmspv(g, _t(x5))), oracle.masked_matmul_skip(W, mask, x5), "n=5 fallback")
    assert_close(_np(gpu_lib.spmm(g, _t(x[:4]))), oracle.masked_matmul(W, mask, x[:4]), "spmm unaffected")


@pytest.mark.parametrize("n", [1, 2, 4])
def test_spmspv_threshold_down(gpu_lib, down_skip, n):
    # raw x = SiLU(g)*u with no zeroing; the kernel drops |x| < 0.3 itself
    W, mask, x_zeroed, g = down_skip
    x_raw = wl.silu_gated_sparse(wl.CFG_SPMSPV, 0, 4, W.shape[1], 0.0)[:n]
    y = _np(gpu_lib.spmspv_threshold(g, _t(x_raw), 0.3))
    assert_close(y, oracle.masked_matmul_threshold(W, mask, x_raw, 0.3), f"threshold n={n}")
    # same active list and values as zeroing x first: bitwise the same result
    # (through the same kernel; swm_spmspv takes it for n <= 2)
    y0 = _np(gpu_lib.spmspv_threshold(g, _t(x_zeroed[:n]), 0.0))
    assert np.array_equal(y.view(np.uint16), y0.view(np.uint16))
    if n <= 2:
        assert np.array_equal(y.view(np.uint16), _np(gpu_lib.spmspv(g, _t(x_zeroed[:n]))).view(np.uint16))
    # tau = 0 is the plain call (bitwise where swm_spmspv runs the same
    # kernel); tau above every |x| gives zeros
    ya = _np(gpu_lib.spmspv_threshold(g, _t(x_raw), 0.0))
    yb = _np(gpu_lib.spmspv(g, _t(x_raw)))
    if n <= 2:
        assert np.array_equal(ya.view(np.uint16), yb.view(np.uint16))
    assert_close(ya, oracle.masked_matmul(W, mask, x_raw), f"threshold 0 n={n}")
    assert_close(yb, oracle.masked_matmul(W, mask, x_raw), f"spmspv n={n}")
    assert np.all(_np(gpu_lib.spmspv_threshold(g, _t(x_raw), 1e4)).view(np.uint16) == 0)


def test_spmspv_threshold_errors(gpu_lib, down, down_skip):
    import ctypes
    import torch
    W, mask, x, f = down                     # skipping not enabled on f
    g = down_skip[3]
    lib = gpu_lib.load()
    xd = _t(x)
    y = torch.empty((4, W.shape[0]), dtype=torch.float16, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp, yp = ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(y.data_ptr())
    K, M = W.shape[1], W.shape[0]
    assert lib.swm_spmspv_threshold(f._h, xp, K, yp, M, 1, ctypes.c_float(0.3), s) == 8    # not enabled
    assert lib.swm_spmspv_threshold(g._h, xp, K, yp, M, 5, ctypes.c_float(0.3), s) == 8    # n > 4
    assert lib.swm_spmspv_threshold(g._h, xp, K, yp, M, 1, ctypes.c_float(-1.0), s) == 1   # tau < 0
    assert lib.swm_spmspv_threshold(g._h, xp, K, yp, M, 1, ctypes.c_float(float("nan")), s) == 1
    assert lib.swm_spmspv_threshold(g._h, xp, K - 1, yp, M, 1, ctypes.c_float(0.3), s) == 1  # ldx < K
    assert lib.swm_spmspv_threshold(g._h, xp, K, yp, M, 0, ctypes.c_float(0.3), s) == 1      # n < 1


@pytest.mark.parametrize("M,K,density,n,zero_frac", [
    (1, 1, 1.0, 1, 0.0), (300, 70, 0.5, 3, 0.5), (257, 1000, 0.3, 4, 0.7), (513, 2049, 0.5, 2, 0.9),
    (100, 513, 1.0, 1, 0.0), (4096, 64, 0.5, 4, 0.5), (4096, 5, 0.5, 2, 0.4), (40, 11008, 0.5, 1, 0.7),
])
def test_spmspv_skip_ragged(gpu_lib, M, K, density, n, zero_frac):
    g = np.random.default_rng(M * 31 + K)
    W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    mask = g.random((M, K)) < density
    x = g.standard_normal((n, K)).astype(np.float16)
    x[:, g.random(K) < zero_frac] = 0  # whole input channels off, as after an activation threshold
    f = gpu_lib.sparse_compress(W, mask, skipping=True)
    ref = oracle.masked_matmul_skip(W, mask, x)
    assert_close(_np(gpu_lib.spmspv(f, _t(x))), ref, f"{M}x{K} n={n}")
    assert_close(_np(gpu_lib.spmspv_threshold(f, _t(x), 0.0)), ref, f"column-run kernel {M}x{K} n={n}")


def test_spmspv_skip_strided(gpu_lib):
    import torch
    g = np.random.default_rng(8)
    M, K, n = 300, 700, 3
    W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    mask = g.random((M, K)) < 0.5
    x = g.standard_normal((n, K)).astype(np.float16)
    x[:, g.random(K) < 0.6] = 0
    f = gpu_lib.sparse_compress(W, mask)
    f.enable_skipping()
    xb = torch.zeros((n, K + 37), dtype=torch.float16, device="cuda")
    xb[:, :K] = _t(x)
    yb = torch.full((n, M + 11), 7.0, dtype=torch.float16, device="cuda")
    gpu_lib.spmspv(f, xb[:, :K], yb[:, :M])
    out = _np(yb)
    assert_close(out[:, :M], oracle.masked_matmul_skip(W, mask, x), "strided")
    assert np.all(out[:, M:] == 7.0)  # outside the output view untouched


# ------------------------------------------------------------------ dense baseline, ragged
@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (65, 129, 3), (300, 1000, 16), (100, 64, 20), (1000, 512, 32),
                                   (3000, 256, 30), (20000, 64, 32), (257, 4104, 17),
                                   # 5-16 tokens: activations staged through LDS, ragged K per wave
                                   (300, 1000, 5), (77, 2056, 8), (513, 4104, 9), (40, 8, 12), (1040, 11008, 15)])
def test_dense_gemm_ragged(gpu_lib, M, K, N):
    g = np.random.default_rng(M * K)
    W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    X = g.standard_normal((N, K)).astype(np.float16)
    Y = _np(gpu_lib.dense_gemm(_t(W), _t(X)))
    assert_close(Y, oracle.masked_matmul(W, None, X), f"dense {M}x{K}x{N}")


@pytest.mark.parametrize("block", ["1", "2", "3"])    # 256x256 (eight waves), 256x128, 128x128
@pytest.mark.parametrize("M,K,N", [(300, 72, 40), (1000, 1032, 300), (257, 4104, 513), (4096, 256, 1024)])
def test_dense_gemm_each_block_shape(gpu_lib, block, M, K, N, monkeypatch):
    """Every block shape of the tiled dense kernel on ragged M, N and K
    (K % 64 != 0 included); SWM_DENSE_BLOCK is read on every call."""
    monkeypatch.setenv("SWM_DENSE_BLOCK", block)
    g = np.random.default_rng(M + K + N)
    W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    X = g.standard_normal((N, K)).astype(np.float16)
    Y = _np(gpu_lib.dense_gemm(_t(W), _t(X)))
    assert_close(Y, oracle.masked_matmul(W, None, X), f"dense block {block} {M}x{K}x{N}")


_REG_STAGED_CHECK = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[2])
import torch
import sparse_weight_matmul_amd as swm
import oracle
for M, K, N in [(100, 64, 20), (1000, 512, 32), (257, 4104, 17), (3000, 256, 300), (4096, 4096, 512)]:
    g = np.random.default_rng(M * K + N)
    W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    X = g.standard_normal((N, K)).astype(np.float16)
    Y = swm.dense_gemm(torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()).float().cpu().numpy()
    ref = oracle.masked_matmul(W, None, X)
    mx = float(np.abs(Y - ref).max())
    rel = float(np.linalg.norm(Y - ref) / np.linalg.norm(ref))
    print(M, K, N, mx, rel, flush=True)
    assert np.all(np.isfinite(Y)) and mx <= MAX_ABS and rel <= REL_FRO, (M, K, N, mx, rel)
print("ok")
"""


def test_dense_gemm_register_staged_kernel():
    """The register-staged MFMA kernel (taken for operands past 4 GiB, or
    with SWM_DENSE_DMA=0, read once per process: hence a child process)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SWM_DENSE_DMA="0")
    code = f"MAX_ABS = {MAX_ABS}\nREL_FRO = {REL_FRO}\n" + _REG_STAGED_CHECK
    r = subprocess.run([sys.executable, "-c", code, root, os.path.join(root, "tests")], env=env,
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]


_LOG_SKIP_CHECK = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[2])
import torch
import sparse_weight_matmul_amd as swm
import oracle
import swm_workloads as wl
W, mask, x = wl.spmspv_down(4, 0.3)
f = swm.sparse_compress(W, mask, skipping=True)
X = torch.from_numpy(x).cuda()
for n in (1, 4):
    y = swm.spmspv(f, X[:n]).float().cpu().numpy()
    ref = oracle.masked_matmul_skip(W, mask, x[:n])
    assert np.abs(y - ref).max() <= 1e-2, n
    if sys.argv[3] == "off":
        assert np.array_equal(y, swm.spmm(f, X[:n]).float().cpu().numpy()), n
swm.dense_gemm(torch.from_numpy(W).cuda(), X[:1])
torch.cuda.synchronize()
print("ok", flush=True)
"""


_DIRECT_B_CHECK = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[2])
import torch
import sparse_weight_matmul_amd as swm
import oracle
g = np.random.default_rng(8208)
M, K = 8208, 4040                      # 513 slabs, 64 tiles per slab row (the last one 8 columns wide)
W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
mask = g.random((M, K)) < 0.5
Wu = (0.02 * g.standard_normal((M, K))).astype(np.float16)
mu = g.random((M, K)) < 0.5
X = g.standard_normal((16, K)).astype(np.float16)
f, fu = swm.sparse_compress(W, mask), swm.sparse_compress(Wu, mu)
Xd = torch.from_numpy(X).cuda()
for n in (9, 13, 16):
    y = swm.spmm(f, Xd[:n]).float().cpu().numpy()
    ref = oracle.masked_matmul(W, mask, X[:n])
    err = np.abs(y - ref).max()
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert err <= 1e-2 and rel <= 1e-3, (n, err, rel)
h = swm.gate_up_silu(f, fu, Xd[:16], 0.0).float().cpu().numpy()
want = oracle.gate_up_silu(W, mask, Wu, mu, X[:16], 0.0)
assert np.abs(h - want).max() <= 1e-2, np.abs(h - want).max()
torch.cuda.synchronize()
print("ok", flush=True)
"""


def test_decode_b_operands_from_memory_tall_ragged():
    """A tall matrix (513 slabs, a ragged last tile column) makes the decode
    plan load the B operands straight into registers at 9-16 tokens (the
    dispatch log says so); spmm at N = 9, 13, 16 and the gated step at 16
    tokens match the oracle.  A child process, because SWM_LOG is read once."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SWM_LOG="1")
    r = subprocess.run([sys.executable, "-c", _DIRECT_B_CHECK, root, os.path.join(root, "tests")], env=env,
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]
    log = [ln for ln in r.stderr.splitlines() if ln.startswith("[swm] sparse_compress M=8208")]
    assert log and all("B operands from memory" in ln for ln in log), log


@pytest.mark.parametrize("mode", ["off", "on"])
def test_dispatch_log_and_skip_switch(mode):
    """SWM_LOG=1 names every dispatch decision on stderr; SWM_SKIP forces the
    skipping kernel off (then spmspv equals spmm bitwise) or on for n <= 4.
    Both are read once per process: hence a child process."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SWM_LOG="1", SWM_SKIP=mode)
    r = subprocess.run([sys.executable, "-c", _LOG_SKIP_CHECK, root, os.path.join(root, "tests"), mode], env=env,
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]
    log = [ln for ln in r.stderr.splitlines() if ln.startswith("[swm] ")]
    assert any(ln.startswith("[swm] sparse_compress M=4096 K=11008") for ln in log), log
    assert any(ln.startswith("[swm] dense_gemm M=4096 K=11008 N=1: streaming") for ln in log), log
    cr = [ln for ln in log if "column-run skipping kernel" in ln]
    dec = [ln for ln in log if ln.startswith("[swm] spmspv") and ": decode" in ln]
    if mode == "off":
        assert not cr and len(dec) == 2, log
    else:
        assert len(cr) == 2 and not dec, log


def test_dense_gemm_graph_replay_after_larger_k(gpu_lib):
    """The streaming dense kernel allocates nothing: a captured small-K call
    still replays correctly after an eager call with a much larger K (the
    loads past a wave's columns read the library's own zero constant)."""
    import torch
    swm = gpu_lib
    g = np.random.default_rng(77)
    Ws = (0.02 * g.standard_normal((300, 520))).astype(np.float16)
    Wb = (0.02 * g.standard_normal((64, 20000))).astype(np.float16)
    xb = torch.empty((5, 520), dtype=torch.float16, device="cuda")
    yb = torch.empty((5, 300), dtype=torch.float16, device="cuda")
    Wsd = _t(Ws)
    xb.copy_(_t(g.standard_normal((5, 520)).astype(np.float16)))
    swm.dense_gemm(Wsd, xb, yb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swm.dense_gemm(Wsd, xb, yb)
    torch.cuda.synchronize()
    for rep in range(3):
        Xb = g.standard_normal((9, 20000)).astype(np.float16)
        assert_close(_np(swm.dense_gemm(_t(Wb), _t(Xb))), oracle.masked_matmul(Wb, None, Xb), f"large K {rep}")
        X = g.standard_normal((5, 520)).astype(np.float16)
        xb.copy_(_t(X))
        torch.cuda.synchronize()
        graph.replay()
        assert_close(_np(yb), oracle.masked_matmul(Ws, None, X), f"replay {rep}")


# ------------------------------------------------------------------ error paths through the ABI
def test_error_codes(gpu_lib):
    import ctypes
    import torch
    swm = gpu_lib
    lib = swm.load()
    W, mask, X = wl.tiny()
    f = swm.sparse_compress(W, mask)
    x = _t(X)
    y = torch.empty((8, 256), dtype=torch.float16, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp, yp = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr())
    assert lib.swm_spmm(f._h, xp, 512, yp, 256, 0, s) == 1        # N <= 0
    assert lib.swm_spmm(f._h, xp, 100, yp, 256, 8, s) == 1        # ldx < K
    assert lib.swm_spmm(f._h, xp, 512, yp, 100, 8, s) == 1        # ldy < M
    assert lib.swm_spmspv(f._h, xp, 512, yp, 256, 17, s) == 1     # n > 16
    assert lib.swm_spmspv(f._h, xp, 512, yp, 256, 0, s) == 1      # n < 1
    assert lib.swm_dense_gemm(xp, 512, xp, 512, yp, 256, 256, 512, -1, s) == 1
    g = swm.sparse_compress(W, mask, tile=(16, 32))
    assert lib.swm_spmm(g._h, xp, 512, yp, 256, 8, s) == 8        # no kernel for tk=32


# ------------------------------------------------------------------ prefill (N > 16)
@pytest.mark.parametrize("M,K,N", [(256, 64, 256), (300, 512, 300), (1000, 1024, 257), (257, 4104, 513),
                                   (64, 128, 17), (520, 200, 40)])
def test_prefill_ragged(gpu_lib, M, K, N):
    swm = gpu_lib
    W, mask = wl.pruned_weight(96, M + K, M, K, 0.5)
    X = np.random.default_rng(M * 3 + N).standard_normal((N, K)).astype(np.float16)
    f = _compress(swm, W, mask)
    ref = oracle.masked_matmul(W, mask, X)
    assert_close(_np(swm.spmm(f, _t(X))), ref, f"prefill sparse {M}x{K}x{N}")
    assert_close(_np(swm.dense_gemm(_t(W), _t(X))), ref, f"prefill dense {M}x{K}x{N}")


def test_prefill_sparse_equals_dense_bitwise(gpu_lib):
    """Same MFMA sequence on the same (exactly expanded) operands: identical bits."""
    swm = gpu_lib
    W, mask = wl.pruned_weight(97, 0, 512, 1024, 0.5)
    X = np.random.default_rng(6).standard_normal((300, 1024)).astype(np.float16)
    f = _compress(swm, W, mask)
    a = _np(swm.spmm(f, _t(X))).view(np.uint16)
    b = _np(swm.dense_gemm(_t(W), _t(X))).view(np.uint16)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ prefill up/gate, every (sparsity, N) point, full outputs
@pytest.fixture(scope="module", params=[0.5, 0.6, 0.7], ids=lambda s: f"s{s}")
def upgate(gpu_lib, request):
    """up/gate 11008x4096 at one sparsity: the fp64 oracle over all 4096
    tokens once, sliced by N (each token's output depends on that token only)."""
    s = request.param
    W, mask, X = wl.prefill_upgate(s, 4096)
    f = gpu_lib.sparse_compress(W, mask)
    ref = oracle.masked_matmul(W, mask, X)
    ws = _workspace(gpu_lib, f, 4096)[0]
    yield s, W, mask, X, f, ref, ws
    del f, ws


@pytest.mark.parametrize("route", ["spmm", "spmm_ws"])
@pytest.mark.parametrize("N", [512, 2048, 4096])
def test_prefill_upgate_full(gpu_lib, upgate, N, route):
    swm = gpu_lib
    s, W, mask, X, f, ref, ws = upgate
    Xd = _t(X[:N])
    Y = _np(swm.spmm(f, Xd) if route == "spmm" else swm.spmm_ws(f, Xd, ws))
    assert_close(Y, ref[:N], f"up/gate s={s} N={N} {route}")
    if route == "spmm_ws" and N == 4096:
        # on-chip expansion and the workspace route run the same MFMA order on
        # the same (exactly expanded) operands
        Yo = _np(swm.spmm(f, Xd))
        assert np.array_equal(Yo.view(np.uint16), Y.view(np.uint16))
    if s == 0.5 and N == 512 and route == "spmm":
        Yd = _np(swm.dense_gemm(_t(W), Xd))
        assert np.array_equal(Yd.view(np.uint16), Y.view(np.uint16))


# ------------------------------------------------------------------ prefill through the workspace (expand once, dense MFMA)
def _workspace(swm, f, N, extra=0):
    import torch
    nb = swm.spmm_workspace_bytes(f, N)
    return torch.empty(nb + extra, dtype=torch.uint8, device="cuda"), nb


@pytest.mark.parametrize("M,K,N", [(520, 392, 1100), (256, 4096, 1024), (1000, 1024, 1031)])
def test_spmm_ws_expand_route(gpu_lib, M, K, N):
    """N >= 1024: W is expanded into the workspace and multiplied by the dense
    kernel.  Checked against the oracle, and bitwise against dense_gemm on
    the exactly expanded W (same kernel, same operands)."""
    swm = gpu_lib
    W, mask = wl.pruned_weight(98, M + K + N, M, K, 0.5)
    X = np.random.default_rng(M + 7 * N).standard_normal((N, K)).astype(np.float16)
    f = _compress(swm, W, mask)
    ws, nb = _workspace(swm, f, N)
    assert nb >= 2 * M * K and nb % 256 == 0
    Xd = _t(X)
    Y = _np(swm.spmm_ws(f, Xd, ws))
    assert_close(Y, oracle.masked_matmul(W, mask, X), f"spmm_ws {M}x{K}x{N}")
    Yd = _np(swm.dense_gemm(_t(np.where(mask, W, np.float16(0))), Xd))
    assert np.array_equal(Y.view(np.uint16), Yd.view(np.uint16))
    # the workspace holds the expanded W afterwards (row-major, ld = K)
    got = _np(ws[:2 * M * K]).view(np.uint16).reshape(M, K)
    assert np.array_equal(got, np.where(mask, W.view(np.uint16), np.uint16(0)))


def test_spmm_ws_degenerate_cases(gpu_lib):
    """Through the expansion route: an all-pruned W and zero activations give
    exact +0; a single kept entry per row gives that entry times x."""
    import torch
    swm = gpu_lib
    M, K, N = 100, 200, 1024
    W, _ = wl.pruned_weight(104, 0, M, K, 0.5)
    X = wl.activations(104, 0, N, K)
    f0 = swm.sparse_compress(W, np.zeros((M, K), dtype=bool))
    f = swm.sparse_compress(W, np.ones((M, K), dtype=bool))
    nb0, nbf = swm.spmm_workspace_bytes(f0, N), swm.spmm_workspace_bytes(f, N)
    assert 0 < nb0 == nbf
    ws = torch.empty(nbf, dtype=torch.uint8, device="cuda")
    assert np.all(_np(swm.spmm_ws(f0, _t(X), ws)).view(np.uint16) == 0)
    assert np.all(_np(swm.spmm_ws(f, _t(np.zeros((N, K), dtype=np.float16)), ws)).view(np.uint16) == 0)
    one = np.zeros((M, K), dtype=bool)
    cols = np.arange(M) % K
    one[np.arange(M), cols] = True
    f1 = swm.sparse_compress(W, one)
    Y = _np(swm.spmm_ws(f1, _t(X), ws))
    want = (X[:, cols].astype(np.float32) * W[np.arange(M), cols].astype(np.float32)).astype(np.float16)
    # exact values; a zero product may carry either sign (the accumulator starts at +0)
    assert np.array_equal(Y.astype(np.float32), want.astype(np.float32))


def test_spmm_ws_route_rule(gpu_lib):
    """The expansion route: always from 1024 tokens; from 256 when the on-chip
    kernel's ceil(M/128)*ceil(N/256) blocks fill at most half of the 256 CUs or
    spill past one round; never below 256."""
    import torch
    swm = gpu_lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Ws, ms = wl.pruned_weight(99, 3, 300, 64, 0.5)     # 3 row blocks: always under-filled
    Wb, mb = wl.pruned_weight(99, 4, 11008, 64, 0.5)   # 86 row blocks
    fs, fb = swm.sparse_compress(Ws, ms), swm.sparse_compress(Wb, mb)
    need_s, need_b = (2 * 300 * 64 + 255) // 256 * 256, (2 * 11008 * 64 + 255) // 256 * 256
    assert [swm.spmm_workspace_bytes(fs, n) for n in (33, 255, 256, 700, 1024)] == [0, 0, need_s, need_s, need_s]

    def expect(n):  # the rule written out for the 86-row-block matrix
        blocks = 86 * -(-n // 256)
        return need_b if n >= 1024 or (n >= 256 and (2 * blocks <= cus or blocks > cus)) else 0
    Ns = (255, 256, 512, 640, 1024, 4096)
    assert [swm.spmm_workspace_bytes(fb, n) for n in Ns] == [expect(n) for n in Ns]
    if cus == 256:  # MI355X: 86 blocks at most half, 172 on chip, 258 a second round
        assert [expect(n) for n in Ns] == [0, need_b, 0, need_b, need_b, need_b]


def test_spmm_ws_below_threshold_and_fallbacks(gpu_lib):
    """Below the route's threshold, without a workspace, or with unaligned X
    the call runs spmm's kernels (identical bits) and leaves the workspace
    untouched."""
    import torch
    swm = gpu_lib
    M, K = 300, 512
    W, mask = wl.pruned_weight(99, 0, M, K, 0.5)
    f = _compress(swm, W, mask)
    assert swm.spmm_workspace_bytes(f, 255) == 0
    assert swm.spmm_workspace_bytes(f, 1024) == (2 * M * K + 255) // 256 * 256
    for N in (16, 100, 255):
        X = _t(np.random.default_rng(N).standard_normal((N, K)).astype(np.float16))
        ws = torch.full((4096,), 0xA5, dtype=torch.uint8, device="cuda")
        a = _np(swm.spmm_ws(f, X, ws)).view(np.uint16)
        b = _np(swm.spmm(f, X)).view(np.uint16)
        assert np.array_equal(a, b), N
        assert bool((ws == 0xA5).all())
        c = _np(swm.spmm_ws(f, X, None)).view(np.uint16)
        assert np.array_equal(c, b), N
    # N above the threshold, X with ldx % 8 != 0: spmm's path, workspace untouched
    N = 1030
    Xs = np.random.default_rng(5).standard_normal((N, K + 4)).astype(np.float16)
    Xv = _t(Xs)[:, :K]
    ws = torch.full((swm.spmm_workspace_bytes(f, N),), 0x5A, dtype=torch.uint8, device="cuda")
    a = _np(swm.spmm_ws(f, Xv, ws))
    assert bool((ws == 0x5A).all())
    assert np.array_equal(a.view(np.uint16), _np(swm.spmm(f, Xv)).view(np.uint16))
    assert_close(a, oracle.masked_matmul(W, mask, Xs[:, :K]), "spmm_ws unaligned fallback")


# ------------------------------------------------------------------ prefill on the sparse matrix cores (2:4 layer + residual)
def _layer24_bytes(M, K, residual):
    kp = -(-K // 64) * 64
    vb = -(-(M * kp) // 256) * 256              # values: M x kp/2 fp16
    mb = -(-(M * (kp // 16) * 2) // 256) * 256  # indices: M x kp/16 uint16
    return 2 * (vb + mb) if residual else vb + mb


@pytest.mark.parametrize("N", [1024, 2048, 4096])
def test_smfmac_route_2_4_qproj(gpu_lib, N):
    """q_proj 4096x4096 with a 2:4 magnitude mask on the sparse-matrix-core
    route: no residual layer; the handle keeps the 2:4 layer compacted at
    compress time, so spmm_ws needs no workspace and spmm takes the same
    kernel (bitwise equal); full outputs against the oracle.  Without the
    option the handle expands."""
    swm = gpu_lib
    W, mask, _ = wl.decode_qproj_2_4(1)
    X = wl.activations(wl.CFG_WIDE, 13, N, 4096)
    assert swm.spmm_workspace_bytes(swm.sparse_compress(W, mask), N) == 2 * 4096 * 4096
    f = swm.sparse_compress(W, mask, smfmac=True)
    ws, nb = _workspace(swm, f, N, extra=256)
    assert nb == 0
    Xd = _t(X)
    Y = _np(swm.spmm_ws(f, Xd, ws))
    assert_close(Y, oracle.masked_matmul(W, mask, X), f"2:4 q_proj N={N}")
    assert np.array_equal(Y.view(np.uint16), _np(swm.spmm(f, Xd)).view(np.uint16))


@pytest.mark.parametrize("M,K,N,s", [(520, 392, 1100, 0.5), (300, 4104, 1024, 0.7), (1000, 1024, 1031, 0.6),
                                     (256, 64, 1024, 0.0), (64, 200, 1500, 1.0)])
def test_smfmac_route_with_residual(gpu_lib, M, K, N, s):
    """Unstructured masks through the sparse-matrix-core route (forced per
    handle): the 2:4 layer and the residual layer add up to the exact masked
    product (ragged M, K not a multiple of 64, N not a multiple of 256; a
    dense mask, where every group keeps 4, and an all-pruned one)."""
    swm = gpu_lib
    W, mask = wl.pruned_weight(105, M + K + N, M, K, s)
    X = wl.activations(105, M + N, N, K)
    f = swm.sparse_compress(W, mask, smfmac=True)
    assert swm.spmm_workspace_bytes(f, N) == 0
    Y = _np(swm.spmm(f, _t(X)))
    assert_close(Y, oracle.masked_matmul(W, mask, X), f"smfmac {M}x{K}x{N} s={s}")
    if s == 1.0:
        assert np.all(Y.view(np.uint16) == 0)


def test_smfmac_route_upgate_70_full(gpu_lib):
    """up/gate 11008x4096 at 70% (the config's highest sparsity) forced onto
    the sparse matrix cores with its residual layer, N = 2048, full outputs;
    below the route's token counts the same handle decodes as usual."""
    swm = gpu_lib
    W, mask, X = wl.prefill_upgate(0.7, 2048)
    f = swm.sparse_compress(W, mask, smfmac=True)
    assert_close(_np(swm.spmm(f, _t(X))), oracle.masked_matmul(W, mask, X), "up/gate 70% smfmac")
    assert_close(_np(swm.spmm(f, _t(X[:16]))), oracle.masked_matmul(W, mask, X[:16]), "up/gate 70% decode")


@pytest.mark.parametrize("i", [4, 6])   # gate_proj 11008x4096 (688 blocks), down_proj 4096x11008
def test_smfmac_layer_2_4_as_benchmarked(gpu_lib, i):
    """The layer's 2:4-pruned linears as the layer bench runs them: a handle
    imported from the export blob gets its layers by enable_smfmac and gives
    the compressed handle's bits; full outputs at N = 4096 against the oracle."""
    swm = gpu_lib
    W, mask, X = wl.layer_linear_2_4(i, 4096)
    f = swm.sparse_compress(W, mask, smfmac=True)
    g = swm.format_import(f.export())
    nb = g.enable_smfmac()
    assert nb == f.enable_smfmac() > 0       # idempotent, same layers
    Xd = _t(X)
    Y = _np(swm.spmm(f, Xd))
    assert_close(Y, oracle.masked_matmul(W, mask, X), f"2:4 linear {i}")
    assert np.array_equal(Y.view(np.uint16), _np(swm.spmm(g, Xd)).view(np.uint16))


def test_spmm_ws_errors(gpu_lib):
    import ctypes
    import torch
    swm = gpu_lib
    lib = swm.load()
    M, K, N = 256, 512, 1024
    W, mask = wl.pruned_weight(99, 1, M, K, 0.5)
    f = _compress(swm, W, mask)
    X = torch.zeros((N, K), dtype=torch.float16, device="cuda")
    Y = torch.empty((N, M), dtype=torch.float16, device="cuda")
    need = swm.spmm_workspace_bytes(f, N)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    xp, yp, wp = ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(Y.data_ptr()), ctypes.c_void_p(ws.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.swm_spmm_ws(f._h, xp, K, yp, M, N, wp, need - 1, s) == 1           # too small
    assert lib.swm_spmm_ws(f._h, xp, K, yp, M, N, None, need, s) == 1             # NULL with bytes
    assert lib.swm_spmm_ws(f._h, xp, K, yp, M, N, ctypes.c_void_p(ws.data_ptr() + 8), need, s) == 3  # misaligned
    assert lib.swm_spmm_ws(f._h, xp, K - 8, yp, M, N, wp, need, s) == 1           # ldx < K
    assert lib.swm_spmm_ws(f._h, xp, K, yp, M, N, wp, need, s) == 0
    torch.cuda.synchronize()


# ------------------------------------------------------------------ gated FFN hidden activation (decode)
def assert_glu_close(H_gpu, H_full, tau, what):
    """H_gpu: the kernel's fp16 output; H_full: the oracle's H without the
    threshold (float64).  The bound is the product's: max |err| <= 1e-2 and
    relative Frobenius <= 1e-3 (h is rounded once to fp16, half an ulp is
    below 0.0078 for |h| < 32, and the workloads' max |h| is about 17).  The
    threshold decision is taken on the fp16-rounded h on both sides; where the
    oracle's |h| lies within 1e-2 of tau both decisions are valid, so such an
    entry must be +0 or within the bound; every other entry must take the
    oracle's decision."""
    Hg = np.asarray(H_gpu, dtype=np.float64)
    assert np.all(np.isfinite(Hg)), what
    assert float(np.abs(H_full).max()) < 32, what  # the bound's premise
    tol = MAX_ABS
    mag = np.abs(H_full.astype(np.float16).astype(np.float64))
    band = np.abs(mag - tau) <= tol
    kept = mag >= tau
    want = np.where(kept, H_full, 0.0)
    ok = np.abs(Hg - want) <= tol
    ok_band = (Hg == 0) | (np.abs(Hg - H_full) <= tol)
    bad = ~np.where(band, ok_band, ok)
    assert not bad.any(), f"{what}: {int(bad.sum())} entries off, first at {np.argwhere(bad)[0]}"
    out = ~band
    den = float(np.linalg.norm(want[out]))
    if den > 0:
        rel = float(np.linalg.norm(Hg[out] - want[out])) / den
        assert rel <= REL_FRO, f"{what}: rel Frobenius err {rel}"
    if tau > 0:  # the threshold must have dropped something clear of the band
        assert np.any((Hg == 0) & ~band & (H_full != 0)), what


@pytest.fixture(scope="module")
def gate_up(gpu_lib):
    Wg, mg, X = wl.layer_linear(4, 32)
    Wu, mu, _ = wl.layer_linear(5, 32)
    fg, fu = gpu_lib.sparse_compress(Wg, mg), gpu_lib.sparse_compress(Wu, mu)
    full = oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0)
    return Wg, mg, Wu, mu, X, fg, fu, full


@pytest.mark.parametrize("N", [1, 4, 16, 24])
@pytest.mark.parametrize("tau", [0.0, 0.3])
def test_gate_up_silu_llama_shape(gpu_lib, gate_up, N, tau):
    """gate/up 11008x4096 at 50%, one launch for both products."""
    Wg, mg, Wu, mu, X, fg, fu, full = gate_up
    H = _np(gpu_lib.gate_up_silu(fg, fu, _t(X[:N]), tau))
    assert_glu_close(H, full[:N], tau, f"gate/up N={N} tau={tau}")


@pytest.mark.parametrize("M,K,N,tau", [(1000, 1032, 3, 0.1), (40, 64, 16, 0.0), (300, 8192, 5, 0.2),
                                       (17, 136, 1, 0.05), (4096, 4096, 8, 0.3), (520, 392, 31, 0.1)])
def test_gate_up_silu_ragged(gpu_lib, M, K, N, tau):
    swm = gpu_lib
    Wg, mg = wl.pruned_weight(100, M + K, M, K, 0.5)
    Wu, mu = wl.pruned_weight(100, M + K + 1, M, K, 0.6)
    X = wl.activations(100, M + N, N, K)
    H = _np(swm.gate_up_silu(swm.sparse_compress(Wg, mg), swm.sparse_compress(Wu, mu), _t(X), tau))
    assert_glu_close(H, oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0), tau, f"glu {M}x{K} N={N} tau={tau}")


def test_gate_up_silu_degenerate_cases(gpu_lib):
    """Zero activations give exact +0; the largest tau drops every entry; the
    same handle as gate and up gives SiLU(g) * g; an all-pruned gate gives
    SiLU(0) * u = 0."""
    swm = gpu_lib
    M, K = 520, 392
    Wg, mg = wl.pruned_weight(103, 0, M, K, 0.5)
    Wu, mu = wl.pruned_weight(103, 1, M, K, 0.5)
    fg, fu = swm.sparse_compress(Wg, mg), swm.sparse_compress(Wu, mu)
    X = wl.activations(103, 0, 5, K)
    Z = np.zeros((5, K), dtype=np.float16)
    assert np.all(_np(swm.gate_up_silu(fg, fu, _t(Z), 0.0)).view(np.uint16) == 0)
    assert np.all(_np(swm.gate_up_silu(fg, fu, _t(X), 65504.0)).view(np.uint16) == 0)
    H = _np(swm.gate_up_silu(fg, fg, _t(X), 0.0))
    assert_glu_close(H, oracle.gate_up_silu(Wg, mg, Wg, mg, X, 0.0), 0.0, "gate == up")
    f0 = swm.sparse_compress(Wg, np.zeros_like(mg))
    assert np.all(_np(swm.gate_up_silu(f0, fu, _t(X), 0.0)) == 0)


def test_gate_up_silu_feeds_skipping_down(gpu_lib, gate_up):
    """The fused activation, thresholded, drives the skipping down projection:
    y = W_down H over the channels H keeps (checked with the GPU's own H)."""
    swm = gpu_lib
    Wg, mg, Wu, mu, X, fg, fu, full = gate_up
    Wd, md, _ = wl.layer_linear(6, 1)
    fd = swm.sparse_compress(Wd, md)
    fd.enable_skipping()
    for n in (1, 4):
        Hd = swm.gate_up_silu(fg, fu, _t(X[:n]), 0.3)
        y = _np(swm.spmspv(fd, Hd))
        Hh = _np(Hd)
        assert (Hh == 0).mean() > 0.3
        assert_close(y, oracle.masked_matmul_skip(Wd, md, Hh), f"down after glu n={n}")


def test_gate_up_silu_chain_graph_replays(gpu_lib, gate_up):
    """The fused FFN step and the skipping down product captured in one HIP
    graph: every replay, with new activations and eager calls in between,
    equals the eager chain bit for bit."""
    import torch
    swm = gpu_lib
    Wg, mg, Wu, mu, X, fg, fu, full = gate_up
    Wd, md, _ = wl.layer_linear(6, 1)
    fd = swm.sparse_compress(Wd, md)
    fd.enable_skipping()
    n, tau = 2, 0.3
    xb = _t(X[:n])
    hb = torch.empty((n, Wg.shape[0]), dtype=torch.float16, device="cuda")
    yb = torch.empty((n, Wd.shape[0]), dtype=torch.float16, device="cuda")
    swm.gate_up_silu(fg, fu, xb, tau, hb)
    swm.spmspv(fd, hb, yb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swm.gate_up_silu(fg, fu, xb, tau, hb)
        swm.spmspv(fd, hb, yb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    for rep in range(3):
        xr = (X[:n].astype(np.float32) * (0.5 + rng.random(X.shape[1]))).astype(np.float16)
        xb.copy_(_t(xr))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        h_graph, y_graph = hb.cpu().numpy().copy(), yb.cpu().numpy().copy()
        h_eager = swm.gate_up_silu(fg, fu, _t(xr), tau)
        y_eager = _np(swm.spmspv(fd, h_eager))
        assert np.array_equal(h_graph.view(np.uint16), _np(h_eager).view(np.uint16)), f"replay {rep}"
        assert np.array_equal(y_graph.view(np.uint16), y_eager.view(np.uint16)), f"replay {rep}"
    assert_glu_close(h_graph, oracle.gate_up_silu(Wg, mg, Wu, mu, xr, 0.0), tau, "graph replay")


def test_spmm_ws_graph_replays(gpu_lib):
    """Expansion and dense product captured in one graph; replays with new
    activations equal eager calls bit for bit."""
    import torch
    swm = gpu_lib
    M, K, N = 520, 392, 1100
    W, mask = wl.pruned_weight(102, 0, M, K, 0.5)
    f = _compress(swm, W, mask)
    ws, _ = _workspace(swm, f, N)
    xb = torch.empty((N, K), dtype=torch.float16, device="cuda")
    yb = torch.empty((N, M), dtype=torch.float16, device="cuda")
    xb.copy_(_t(wl.activations(102, 0, N, K)))
    swm.spmm_ws(f, xb, ws, yb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swm.spmm_ws(f, xb, ws, yb)
    torch.cuda.synchronize()
    for rep in range(3):
        X = wl.activations(102, rep + 1, N, K)
        xb.copy_(_t(X))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_graph = yb.cpu().numpy().copy()
        y_eager = _np(swm.spmm_ws(f, _t(X), ws))
        assert np.array_equal(y_graph.view(np.uint16), y_eager.view(np.uint16)), f"replay {rep}"
        assert_close(y_graph, oracle.masked_matmul(W, mask, X), f"replay {rep}")


def test_gate_up_silu_errors(gpu_lib):
    import ctypes
    import torch
    swm = gpu_lib
    lib = swm.load()
    M, K = 64, 128
    Wg, mg = wl.pruned_weight(101, 0, M, K, 0.5)
    fg, fu = swm.sparse_compress(Wg, mg), swm.sparse_compress(Wg, mg)
    fo = swm.sparse_compress(*wl.pruned_weight(101, 1, M + 16, K, 0.5))
    X = torch.zeros((16, K + 8), dtype=torch.float16, device="cuda")
    H = torch.empty((16, M), dtype=torch.float16, device="cuda")
    xp, hp = ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(H.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = lambda a, b, ldx, n, tau, x=xp: lib.swm_gate_up_silu(a, b, x, ldx, hp, M, n, tau, s)
    assert f(fg._h, fu._h, K, 4, 0.0) == 0
    assert f(fg._h, fo._h, K, 4, 0.0) == 1               # shapes differ
    assert f(fg._h, None, K, 4, 0.0) == 1
    assert f(fg._h, fu._h, K, 0, 0.0) == 1               # n < 1
    assert f(fg._h, fu._h, K, 33, 0.0) == 1              # n > 32
    assert f(fg._h, fu._h, K, 4, float("nan")) == 1
    assert f(fg._h, fu._h, K, 4, -1.0) == 1
    assert f(fg._h, fu._h, K - 8, 4, 0.0) == 1           # ldx < K
    assert f(fg._h, fu._h, K + 4, 4, 0.0) == 3           # ldx % 8 != 0: SWM_ERR_ALIGN
    assert f(fg._h, fu._h, K, 4, 0.0, ctypes.c_void_p(X.data_ptr() + 2)) == 3  # misaligned X: SWM_ERR_ALIGN
    Wb, mb = wl.pruned_weight(101, 2, 32, 8256, 0.5)     # 129 tiles per row
    fb = swm.sparse_compress(Wb, mb)
    Xb = torch.zeros((1, 8256), dtype=torch.float16, device="cuda")
    assert lib.swm_gate_up_silu(fb._h, fb._h, ctypes.c_void_p(Xb.data_ptr()), 8256, hp, 32, 1, 0.0, s) == 8
    torch.cuda.synchronize()


# ------------------------------------------------------------------ gated FFN hidden activation (prefill)
def _glu_ws(swm, fg, fu, X, tau, extra=0):
    """gate_up_silu_ws with a fresh workspace of exactly the bytes it asks for (+ extra)."""
    import torch
    n = X.shape[0]
    nb = swm.gate_up_silu_workspace_bytes(fg, fu, n)
    ws = torch.empty(nb + extra, dtype=torch.uint8, device="cuda") if nb + extra > 0 else None
    return swm.gate_up_silu_ws(fg, fu, _t(X), ws, tau), nb


@pytest.fixture(scope="module")
def gate_up_prefill(gpu_lib):
    """gate/up 11008x4096 at 50% (the Llama-2-7B layer's), 640 prefill tokens."""
    Wg, mg, X = wl.layer_linear(4, 640)
    Wu, mu, _ = wl.layer_linear(5, 640)
    fg, fu = gpu_lib.sparse_compress(Wg, mg), gpu_lib.sparse_compress(Wu, mu)
    full = oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0)
    return Wg, mg, Wu, mu, X, fg, fu, full


@pytest.mark.parametrize("N", [33, 640])
@pytest.mark.parametrize("tau", [0.0, 0.3])
def test_gate_up_silu_ws_llama_shape(gpu_lib, gate_up_prefill, N, tau):
    """The prefill route (both weights expanded as interleaved rows, one dense
    MFMA product with the gated epilogue) against the oracle, every output;
    640 tokens span three 256-token blocks with a ragged last one."""
    Wg, mg, Wu, mu, X, fg, fu, full = gate_up_prefill
    H, nb = _glu_ws(gpu_lib, fg, fu, X[:N], tau)
    assert nb == 2 * Wg.shape[0] * Wg.shape[1] * 2
    assert_glu_close(_np(H), full[:N], tau, f"gate/up prefill N={N} tau={tau}")


def test_gate_up_silu_ws_full_size(gpu_lib):
    """gate/up 11008x4096 at 50% and N = 4096, the size the FFN bench times:
    every output against the oracle (tau = 0.3), and the dense gated step on
    W (.) mask returns the same bits."""
    Wg, mg, X = wl.layer_linear(4, 4096)
    Wu, mu, _ = wl.layer_linear(5, 4096)
    fg, fu = gpu_lib.sparse_compress(Wg, mg), gpu_lib.sparse_compress(Wu, mu)
    H = _np(_glu_ws(gpu_lib, fg, fu, X, 0.3)[0])
    Hd = _np(gpu_lib.dense_gate_up_silu(_t(_interleave(Wg, Wu)), _t(X), 0.3))
    assert np.array_equal(H.view(np.uint16), Hd.view(np.uint16))
    assert_glu_close(H, oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0), 0.3, "gate/up prefill N=4096")


@pytest.mark.parametrize("M,K,N,tau", [(1000, 1032, 33, 0.1), (520, 392, 300, 0.0), (300, 8192, 100, 0.2),
                                       (17, 136, 257, 0.05), (4096, 4096, 1100, 0.3), (131, 520, 70, 0.0)])
def test_gate_up_silu_ws_ragged(gpu_lib, M, K, N, tau):
    """Ragged channel and token counts (partial row and token blocks, the 128-
    and 256-row block shapes) against the oracle."""
    swm = gpu_lib
    Wg, mg = wl.pruned_weight(104, M + K, M, K, 0.5)
    Wu, mu = wl.pruned_weight(104, M + K + 1, M, K, 0.6)
    X = wl.activations(104, M + N, N, K)
    fg, fu = swm.sparse_compress(Wg, mg), swm.sparse_compress(Wu, mu)
    H, _ = _glu_ws(swm, fg, fu, X, tau, extra=256)
    assert_glu_close(_np(H), oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0), tau, f"glu ws {M}x{K} N={N} tau={tau}")


def test_gate_up_silu_ws_small_n_is_decode_path(gpu_lib, gate_up_prefill):
    """Below 33 tokens the call is swm_gate_up_silu (no workspace): bit for bit."""
    Wg, mg, Wu, mu, X, fg, fu, full = gate_up_prefill
    for n in (1, 16, 32):
        assert gpu_lib.gate_up_silu_workspace_bytes(fg, fu, n) == 0
        H = gpu_lib.gate_up_silu_ws(fg, fu, _t(X[:n]), None, 0.3)
        ref = gpu_lib.gate_up_silu(fg, fu, _t(X[:n]), 0.3)
        assert np.array_equal(_np(H).view(np.uint16), _np(ref).view(np.uint16)), n


def test_gate_up_silu_ws_degenerate_cases(gpu_lib):
    """Zero activations give exact +0; the largest tau drops every entry; the
    same handle as gate and up gives SiLU(g) * g; an all-pruned gate gives
    SiLU(0) * u = 0."""
    swm = gpu_lib
    M, K, N = 520, 392, 96
    Wg, mg = wl.pruned_weight(105, 0, M, K, 0.5)
    Wu, mu = wl.pruned_weight(105, 1, M, K, 0.5)
    fg, fu = swm.sparse_compress(Wg, mg), swm.sparse_compress(Wu, mu)
    X = wl.activations(105, 0, N, K)
    Z = np.zeros((N, K), dtype=np.float16)
    assert np.all(_np(_glu_ws(swm, fg, fu, Z, 0.0)[0]).view(np.uint16) == 0)
    assert np.all(_np(_glu_ws(swm, fg, fu, X, 65504.0)[0]).view(np.uint16) == 0)
    H = _np(_glu_ws(swm, fg, fg, X, 0.0)[0])
    assert_glu_close(H, oracle.gate_up_silu(Wg, mg, Wg, mg, X, 0.0), 0.0, "gate == up")
    f0 = swm.sparse_compress(Wg, np.zeros_like(mg))
    assert np.all(_np(_glu_ws(swm, f0, fu, X, 0.0)[0]) == 0)


def test_gate_up_silu_ws_graph_replays(gpu_lib):
    """Both expansions and the gated product captured in one graph: replays
    with new activations (eager calls in between) equal eager calls bit for bit."""
    import torch
    swm = gpu_lib
    M, K, N, tau = 520, 392, 300, 0.1
    Wg, mg = wl.pruned_weight(106, 0, M, K, 0.5)
    Wu, mu = wl.pruned_weight(106, 1, M, K, 0.5)
    fg, fu = swm.sparse_compress(Wg, mg), swm.sparse_compress(Wu, mu)
    ws = torch.empty(swm.gate_up_silu_workspace_bytes(fg, fu, N), dtype=torch.uint8, device="cuda")
    xb = torch.empty((N, K), dtype=torch.float16, device="cuda")
    hb = torch.empty((N, M), dtype=torch.float16, device="cuda")
    xb.copy_(_t(wl.activations(106, 0, N, K)))
    swm.gate_up_silu_ws(fg, fu, xb, ws, tau, hb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swm.gate_up_silu_ws(fg, fu, xb, ws, tau, hb)
    torch.cuda.synchronize()
    for rep in range(3):
        X = wl.activations(106, rep + 1, N, K)
        xb.copy_(_t(X))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        h_graph = hb.cpu().numpy().copy()
        h_eager = _np(_glu_ws(swm, fg, fu, X, tau)[0])
        assert np.array_equal(h_graph.view(np.uint16), h_eager.view(np.uint16)), f"replay {rep}"
        assert_glu_close(h_graph, oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0), tau, f"replay {rep}")


def test_gate_up_silu_ws_errors(gpu_lib):
    import ctypes
    import torch
    swm = gpu_lib
    lib = swm.load()
    M, K, N = 64, 128, 40
    Wg, mg = wl.pruned_weight(107, 0, M, K, 0.5)
    fg, fu = swm.sparse_compress(Wg, mg), swm.sparse_compress(Wg, mg)
    fo = swm.sparse_compress(*wl.pruned_weight(107, 1, M + 16, K, 0.5))
    need = swm.gate_up_silu_workspace_bytes(fg, fu, N)
    assert need == 2 * M * K * 2 and swm.gate_up_silu_workspace_bytes(fg, fo, N) == 0
    X = torch.zeros((N, K + 8), dtype=torch.float16, device="cuda")
    H = torch.empty((N, M), dtype=torch.float16, device="cuda")
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    xp, hp, wp = ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(H.data_ptr()), ctypes.c_void_p(ws.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = lambda a, b, ldx, n, tau, w=wp, nb=need, x=xp: lib.swm_gate_up_silu_ws(a, b, x, ldx, hp, M, n, tau, w, nb, s)
    assert f(fg._h, fu._h, K, N, 0.0) == 0
    assert f(fg._h, fo._h, K, N, 0.0) == 1                # shapes differ
    assert f(fg._h, None, K, N, 0.0) == 1
    assert f(fg._h, fu._h, K, 0, 0.0) == 1                # n < 1
    assert f(fg._h, fu._h, K, N, float("nan")) == 1
    assert f(fg._h, fu._h, K, N, -1.0) == 1
    assert f(fg._h, fu._h, K - 8, N, 0.0) == 1            # ldx < K
    assert f(fg._h, fu._h, K, N, 0.0, nb=need - 1) == 1   # workspace too small
    assert f(fg._h, fu._h, K, N, 0.0, w=None) == 1        # NULL workspace
    assert f(fg._h, fu._h, K, N, 0.0, w=ctypes.c_void_p(ws.data_ptr() + 8)) == 3  # misaligned workspace
    assert f(fg._h, fu._h, K + 4, N, 0.0) == 3            # ldx % 8 != 0: SWM_ERR_ALIGN
    assert f(fg._h, fu._h, K, N, 0.0, x=ctypes.c_void_p(X.data_ptr() + 2)) == 3  # misaligned X
    assert f(fg._h, fu._h, K, 4, 0.0, w=None, nb=0) == 0  # decode path: no workspace needed
    torch.cuda.synchronize()


def _interleave(Wg, Wu):
    """2M x K: gate row m at 2m, up row m at 2m + 1."""
    W2 = np.empty((2 * Wg.shape[0], Wg.shape[1]), dtype=np.float16)
    W2[0::2], W2[1::2] = Wg, Wu
    return W2


def test_dense_gate_up_silu_equals_sparse_route_bitwise(gpu_lib, gate_up_prefill):
    """The dense gated product on W (.) mask returns the bits of the sparse
    prefill route (the expansion reproduces W (.) mask exactly, and both run
    one kernel), and both match the oracle."""
    Wg, mg, Wu, mu, X, fg, fu, full = gate_up_prefill
    W2 = _t(_interleave(Wg, Wu))  # the workload's W has +0 at every pruned entry
    for n, tau in ((640, 0.3), (100, 0.0)):
        Hd = _np(gpu_lib.dense_gate_up_silu(W2, _t(X[:n]), tau))
        Hs = _np(_glu_ws(gpu_lib, fg, fu, X[:n], tau)[0])
        assert np.array_equal(Hd.view(np.uint16), Hs.view(np.uint16)), n
        assert_glu_close(Hd, full[:n], tau, f"dense gate/up n={n}")


@pytest.mark.parametrize("M,K,N,tau", [(520, 392, 5, 0.1), (17, 136, 40, 0.0), (1000, 1032, 300, 0.2)])
def test_dense_gate_up_silu_ragged(gpu_lib, M, K, N, tau):
    swm = gpu_lib
    Wg, mg = wl.pruned_weight(108, M + K, M, K, 0.5)
    Wu, mu = wl.pruned_weight(108, M + K + 1, M, K, 0.6)
    X = wl.activations(108, M + N, N, K)
    H = _np(swm.dense_gate_up_silu(_t(_interleave(Wg, Wu)), _t(X), tau))
    assert_glu_close(H, oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0), tau, f"dense glu {M}x{K} N={N} tau={tau}")


def test_dense_gate_up_silu_errors(gpu_lib):
    import ctypes
    import torch
    lib = gpu_lib.load()
    M, K, N = 64, 128, 40
    W2 = torch.zeros((2 * M, K + 8), dtype=torch.float16, device="cuda")
    X = torch.zeros((N, K + 8), dtype=torch.float16, device="cuda")
    H = torch.empty((N, M), dtype=torch.float16, device="cuda")
    wp, xp, hp = (ctypes.c_void_p(t.data_ptr()) for t in (W2, X, H))
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = lambda ldw, ldx, m, k, n, tau, w=wp, x=xp: lib.swm_dense_gate_up_silu(w, ldw, x, ldx, hp, M, m, k, n, tau, s)
    assert f(K, K, M, K, N, 0.0) == 0
    assert f(K, K, M, K, 0, 0.0) == 1                     # N <= 0
    assert f(K - 8, K, M, K, N, 0.0) == 1                 # ldw < K
    assert f(K, K, M, K, N, float("nan")) == 1
    assert f(K + 4, K, M, K, N, 0.0) == 3                 # ldw % 8 != 0
    assert f(K, K, M, K, N, 0.0, w=ctypes.c_void_p(W2.data_ptr() + 2)) == 3
    assert f(K, K, M, K, N, 0.0, x=ctypes.c_void_p(X.data_ptr() + 2)) == 3
    assert f(K, K, M, 12, N, 0.0) == 8                    # K % 8 != 0
    assert f(K, K, 0, K, N, 0.0) == 0                     # M == 0: nothing to do
    torch.cuda.synchronize()


# ------------------------------------------------------------------ wider workloads
@pytest.mark.parametrize("s", [0.6, 0.7])
@pytest.mark.parametrize("N", [1, 16])
def test_qproj_decode_higher_sparsity(gpu_lib, s, N):
    W, mask, X = wl.decode_qproj_sparsity(s, N)
    f = gpu_lib.sparse_compress(W, mask)
    assert_close(_np(gpu_lib.spmm(f, _t(X))), oracle.masked_matmul(W, mask, X), f"q_proj s={s} N={N}")


@pytest.mark.parametrize("N", [1, 16])
def test_qproj_decode_2_4_mask(gpu_lib, N):
    W, mask, X = wl.decode_qproj_2_4(N)
    f = gpu_lib.sparse_compress(W, mask)
    assert_close(_np(gpu_lib.spmm(f, _t(X))), oracle.masked_matmul(W, mask, X), f"q_proj 2:4 N={N}")


def test_fig1_shape_full(gpu_lib):
    # M/K/N = 65536/16384/32 at 50%: every output of the sparse and the dense
    # kernel against the oracle, computed in row blocks of 8192 (the fp64
    # masked weight of one block is 1 GiB)
    swm = gpu_lib
    W, mask, X = wl.fig1_shape()
    f = swm.sparse_compress(W, mask)
    Y = _np(swm.spmm(f, _t(X)))
    del f
    Yd = _np(swm.dense_gemm(_t(W), _t(X)))
    for r in range(0, W.shape[0], 8192):
        ref = oracle.masked_matmul(W[r:r + 8192], mask[r:r + 8192], X)
        assert_close(Y[:, r:r + 8192], ref, f"fig1 spmm rows {r}..")
        assert_close(Yd[:, r:r + 8192], ref, f"fig1 dense rows {r}..")


# ------------------------------------------------------------------ the layer's stacked projections, as benchmarked
@pytest.mark.parametrize("g,N", [(0, 16), (2, 16), (0, 4096)])   # qkv 12288x4096, gate_up 22016x4096
def test_layer_stacked_projections_as_benchmarked(gpu_lib, g, N):
    # row-stacked q;k;v and gate;up through spmm_ws, full outputs; each row
    # range must equal its own linear's product with the group's input
    swm = gpu_lib
    W, mask, X = wl.layer_fused(g, N)
    f = swm.sparse_compress(W, mask)
    ref = oracle.masked_matmul(W, mask, X)
    ws, nb = _workspace(swm, f, N)
    assert (nb > 0) == (N == 4096)
    Y = _np(swm.spmm_ws(f, _t(X), ws))
    assert_close(Y, ref, f"stacked group {g} N={N}")
    r0 = 0
    for i in wl.LAYER_FUSED[g][1]:
        Wi, mi, _ = wl.layer_linear(i, N)
        assert_close(Y[:, r0:r0 + Wi.shape[0]], oracle.masked_matmul(Wi, mi, X), f"linear {i} inside group {g}")
        r0 += Wi.shape[0]


# ------------------------------------------------------------------ layer shapes in the bench's launch configuration
@pytest.mark.parametrize("i", [0, 4, 6])   # q_proj 4096x4096, gate_proj 11008x4096, down_proj 4096x11008
@pytest.mark.parametrize("N", [16, 4096])
def test_layer_linears_as_benchmarked(gpu_lib, i, N):
    # the layer workload's own seeded inputs, full outputs; at N = 4096 through
    # both prefill routes (on chip, and W expanded once into a workspace)
    swm = gpu_lib
    W, mask, X = wl.layer_linear(i, N)
    f = swm.sparse_compress(W, mask)
    ref = oracle.masked_matmul(W, mask, X)
    Xd = _t(X)
    assert_close(_np(swm.spmm(f, Xd)), ref, f"linear {i} N={N} spmm")
    if N == 4096:
        ws, nb = _workspace(swm, f, N)
        assert nb > 0
        assert_close(_np(swm.spmm_ws(f, Xd, ws)), ref, f"linear {i} N={N} spmm_ws")


# ------------------------------------------------------------------ guard bands and run-twice determinism
def _guarded(torch, rows, cols, pad_rows=2, pad_cols=64):
    """An fp16 buffer with guard bands around a (rows, cols) view; the view
    starts 16-byte aligned and its leading dimension is a multiple of 8."""
    buf = torch.full((rows + pad_rows, cols + pad_cols), 7.0, dtype=torch.float16, device="cuda")
    view = buf[1:rows + 1, 32:32 + cols]
    return buf, view


def _guard_ok(buf, rows, cols):
    b = _np(buf)
    inside = np.zeros(b.shape, dtype=bool)
    inside[1:rows + 1, 32:32 + cols] = True
    return bool(np.all(b[~inside] == 7.0))


@pytest.mark.parametrize("route,N", [("spmm", 5), ("spmm", 24), ("spmm", 300), ("spmm_ws", 1100),
                                     ("dense", 7), ("dense", 300), ("spmspv_skip", 1), ("spmspv_skip", 2),
                                     ("spmspv_tiled", 3), ("glu", 5), ("glu", 20)])
def test_outputs_stay_in_their_view_and_repeat_bitwise(gpu_lib, route, N):
    """Every product writes exactly its strided output view (a guard band of
    7.0 around it stays intact) and a second call gives the same bits: the
    reductions have a fixed order, so a difference would show a race."""
    import torch
    swm = gpu_lib
    M, K = 1000, 1032
    g = np.random.default_rng(N * 31 + len(route))
    W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    mask = g.random((M, K)) < 0.5
    X = g.standard_normal((N, K)).astype(np.float16)
    if route.startswith("spmspv"):
        X[:, g.random(K) < 0.7] = 0
    f = swm.sparse_compress(W, mask, skipping=route == "spmspv_skip")
    fu = swm.sparse_compress((0.02 * g.standard_normal((M, K))).astype(np.float16), mask) if route == "glu" else None
    Xd = _t(X)
    outs = []
    for _ in range(2):
        buf, view = _guarded(torch, N, M)
        if route == "spmm":
            swm.spmm(f, Xd, view)
            ref = oracle.masked_matmul(W, mask, X)
        elif route == "spmm_ws":
            ws, nb = _workspace(swm, f, N)
            assert nb > 0
            swm.spmm_ws(f, Xd, ws, view)
            ref = oracle.masked_matmul(W, mask, X)
        elif route == "dense":
            swm.dense_gemm(_t(np.where(mask, W, np.float16(0))), Xd, view)
            ref = oracle.masked_matmul(W, mask, X)
        elif route.startswith("spmspv"):
            swm.spmspv(f, Xd, view)
            ref = oracle.masked_matmul_skip(W, mask, X)
        else:
            swm.gate_up_silu(f, fu, Xd, 0.0, view)
            ref = None   # values: the gate/up parity tests
        torch.cuda.synchronize()
        assert _guard_ok(buf, N, M), f"{route} N={N} wrote outside its view"
        if ref is not None:
            assert_close(_np(view), ref, f"{route} N={N}")
        outs.append(_np(view).copy())
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16)), f"{route} N={N} not repeatable"

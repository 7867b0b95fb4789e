"""swm_spmspv_noalloc: the skipping product with its partial sums in the
library's fixed device array, against swm_spmspv (whose partials live in the
handle's workspace) -- same kernels, so the results must agree bitwise, and
both must meet the oracle's bound."""
import numpy as np
import pytest

import oracle
import swm_workloads as wl

pytestmark = pytest.mark.gpu


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _close(Y, ref, what):
    Yg = np.asarray(Y, dtype=np.float64)
    assert np.all(np.isfinite(Yg)), what
    assert float(np.abs(Yg - ref).max()) <= 1e-2, what
    assert float(np.linalg.norm(Yg - ref)) <= 1e-3 * float(np.linalg.norm(ref)), what


def test_noalloc_matches_spmspv_two_calls_second_smaller(gpu_lib):
    swm = gpu_lib
    # first call: down_proj 4096x11008 at 50%, SiLU-gated x (about 70% zeros),
    # n = 2 (the skipping kernel serves up to two tokens)
    W, mask, x = wl.spmspv_down(2, 0.3)
    f = swm.sparse_compress(W, mask, skipping=True)
    xd = _t(x)
    a = _np(swm.spmspv(f, xd)).view(np.uint16)
    b = _np(swm.spmspv_noalloc(f, xd)).view(np.uint16)
    assert np.array_equal(a, b)
    _close(b.view(np.float16), oracle.masked_matmul_skip(W, mask, x), "down n=2")
    # second call, smaller: 300 x 700 weight, n = 1 (fewer row blocks and
    # splits: the array keeps the first call's partials beyond this call's)
    g = np.random.default_rng(41)
    W2 = (0.02 * g.standard_normal((300, 700))).astype(np.float16)
    m2 = g.random((300, 700)) < 0.5
    x2 = g.standard_normal((1, 700)).astype(np.float16)
    x2[:, g.random(700) < 0.6] = 0
    f2 = swm.sparse_compress(W2, m2)
    f2.enable_skipping()
    x2d = _t(x2)
    a2 = _np(swm.spmspv(f2, x2d)).view(np.uint16)
    b2 = _np(swm.spmspv_noalloc(f2, x2d)).view(np.uint16)
    assert np.array_equal(a2, b2)
    _close(b2.view(np.float16), oracle.masked_matmul_skip(W2, m2, x2), "300x700 n=1")
    # the tiled path (no column-run encoding, or n > 2) is swm_spmspv's too
    h = swm.sparse_compress(W2, m2)
    assert np.array_equal(_np(swm.spmspv_noalloc(h, x2d)).view(np.uint16), _np(swm.spmspv(h, x2d)).view(np.uint16))


def test_noalloc_rejects_partials_beyond_the_array(gpu_lib):
    import ctypes
    import torch
    swm = gpu_lib
    lib = swm.load()
    # 65536 rows x 5120 columns: 256 row blocks x 5 splits x 4 x 256 floats
    # = 5 MiB of partials, above the 4 MiB array -> SWM_ERR_UNSUPPORTED
    M, K = 65536, 5120
    W = np.zeros((M, K), dtype=np.float16)
    mask = np.zeros((M, K), dtype=bool)
    W[::97, ::5] = np.float16(0.5)
    mask[::97, ::5] = True
    f = swm.sparse_compress(W, mask)
    f.enable_skipping()
    x = torch.zeros((1, K), dtype=torch.float16, device="cuda")
    y = torch.full((1, M), 3.0, dtype=torch.float16, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = lib.swm_spmspv_noalloc(f._h, ctypes.c_void_p(x.data_ptr()), K, ctypes.c_void_p(y.data_ptr()), M, 1, s)
    assert code == 8
    assert bool((y == 3.0).all())  # nothing launched, output untouched
    # the allocating call serves the same handle
    assert bool((swm.spmspv(f, x) == 0).all())

"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* exact integer brute force (every fp16 product is an integer multiple of
  2**-48) with a deterministic float64 error bound;
* special cases with exact answers (identity, permutation, one-hot, all-zero
  mask, hand-worked 3x10 example);
* a hand-worked byte image of the format (tests/golden/tcb_hand_example.json);
* format invariants and a round trip;
* planted mistakes: mutated copies of the oracle must fail these pins.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.exact import exact_masked_matmul, exact_to_float, fp64_error_bound
import swm_workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_against_exact(fn, W, mask, X):
    Y = fn(W, mask, X)
    exact = exact_to_float(exact_masked_matmul(W, mask, X))
    bound = fp64_error_bound(W, mask, X) + np.abs(exact) * 2.0 ** -52
    return np.all(np.abs(Y - exact) <= bound), Y, exact


def _rand_case(seed, M, K, N, density, ties=False, signed_zero=False):
    g = np.random.default_rng(seed)
    if ties:
        W = g.choice(np.array([-0.5, -0.25, 0.25, 0.5, 1.0], dtype=np.float16), size=(M, K))
    else:
        W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    if signed_zero:
        z = g.random((M, K)) < 0.1
        W[z] = np.float16(-0.0)
    mask = g.random((M, K)) < density
    X = g.standard_normal((N, K)).astype(np.float16)
    return W, mask, X


# ---------------------------------------------------------------- brute force
def test_oracle_matches_exact_brute_force_on_tiny_workload():
    W, mask, X = wl.tiny()
    ok, Y, exact = _check_against_exact(oracle.masked_matmul, W, mask, X)
    assert ok
    assert Y.shape == (8, 256)


@pytest.mark.parametrize("seed,M,K,N,density", [
    (1, 1, 1, 1, 1.0), (2, 3, 7, 2, 0.5), (3, 65, 130, 3, 0.5), (4, 17, 300, 5, 0.01),
    (5, 40, 33, 17, 0.99), (6, 129, 9, 1, 0.3),
])
def test_oracle_matches_exact_on_random_shapes(seed, M, K, N, density):
    W, mask, X = _rand_case(seed, M, K, N, density, ties=seed % 2 == 0, signed_zero=True)
    ok, _, _ = _check_against_exact(oracle.masked_matmul, W, mask, X)
    assert ok
    ok, _, _ = _check_against_exact(oracle.masked_matmul_skip, W, mask, X)
    assert ok


# ---------------------------------------------------------------- exact special cases
def test_all_zero_mask_gives_zero():
    W, _, X = _rand_case(7, 70, 90, 4, 0.5)
    mask = np.zeros(W.shape, dtype=bool)
    assert np.all(oracle.masked_matmul(W, mask, X) == 0)
    assert np.all(oracle.masked_matmul_skip(W, mask, X) == 0)


def test_dense_mask_is_the_plain_product_brute_force():
    W, _, X = _rand_case(8, 20, 50, 3, 1.0)
    ok, _, _ = _check_against_exact(oracle.masked_matmul, W, np.ones(W.shape, bool), X)
    assert ok


def test_identity_and_permutation_are_exact():
    K, N = 96, 5
    g = np.random.default_rng(9)
    X = g.standard_normal((N, K)).astype(np.float16)
    W = np.eye(K, dtype=np.float16)
    assert np.array_equal(oracle.to_fp16(oracle.masked_matmul(W, np.eye(K, dtype=bool), X)).view(np.uint16),
                          X.view(np.uint16) & np.uint16(0xFFFF))
    perm = g.permutation(K)
    P = np.zeros((K, K), dtype=np.float16)
    P[np.arange(K), perm] = 1
    Y = oracle.masked_matmul(P, P != 0, X)
    assert np.array_equal(Y, X[:, perm].astype(np.float64))


def test_one_hot_activations_pick_a_weight_column():
    W, mask, _ = _rand_case(10, 33, 40, 1, 0.5)
    for k in (0, 17, 39):
        X = np.zeros((1, 40), dtype=np.float16)
        X[0, k] = 1
        Y = oracle.masked_matmul(W, mask, X)
        assert np.array_equal(Y[0], np.where(mask[:, k], W[:, k].astype(np.float64), 0.0))


def test_power_of_two_scaling_is_exact():
    W, mask, X = _rand_case(11, 30, 64, 2, 0.5)
    Y1 = oracle.masked_matmul(W, mask, X)
    Y2 = oracle.masked_matmul(W, mask, (X.astype(np.float64) * 0.25).astype(np.float16))
    # scaling by 2**-2 keeps every fp16 normal value exact at this magnitude
    assert np.allclose(Y2 * 4.0, Y1, rtol=0, atol=1e-12)


def test_hand_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "tcb_hand_example.json")))
    W = np.array(d["W_rows_fp16"], dtype=np.float16)
    X = np.array([d["x"]], dtype=np.float16)
    assert list(oracle.masked_matmul(W, None, X)[0]) == d["y"]
    assert list(oracle.masked_matmul_skip(W, None, X)[0]) == d["y"]


def test_skip_ignores_all_zero_channels_only():
    W, mask, X = _rand_case(12, 50, 80, 4, 0.5)
    X[:, ::3] = 0
    X[1, 1] = np.float16(-0.0)
    X[0, 2] = 0
    act = oracle.active_inputs(X)
    assert not act[0] and act[4]
    assert not act[1] or np.any(X[:, 1] != 0)
    assert np.all(oracle.masked_matmul_skip(W, mask, np.zeros_like(X)) == 0)
    ok, _, _ = _check_against_exact(oracle.masked_matmul_skip, W, mask, X)
    assert ok


# ---------------------------------------------------------------- format
def test_format_hand_worked_bytes():
    d = json.load(open(os.path.join(GOLDEN, "tcb_hand_example.json")))
    W = np.array(d["W_rows_fp16"], dtype=np.float16)
    f = oracle.tcb_encode(W, None, TK=d["TK"])
    assert f.TM == d["TM"]
    assert (f.Mt, f.Kt, f.nnz, f.padded_len, f.max_tile) == (d["Mt"], d["Kt"], d["nnz"], d["padded_len"], d["max_tile"])
    assert list(f.tile_ptr) == d["tile_ptr"]
    assert [int(b) for b in f.bits] == d["bits"]
    assert [format(int(v), "04x") for v in f.values] == d["values_hex"]
    assert f.header() == bytes.fromhex(d["header_hex"].replace(" ", ""))
    blob = f.blob()
    assert len(blob) == 64 + 4 * 2 + 8 * 8 + 2 * 8
    g = oracle.tcb_parse(blob)
    assert np.array_equal(oracle.tcb_decode(g), W.view(np.uint16))


@pytest.mark.parametrize("M,K,TK,density", [
    (1, 1, 32, 1.0), (16, 64, 64, 0.5), (100, 70, 64, 0.5), (130, 300, 96, 0.3),
    (65, 257, 256, 0.01), (200, 40, 32, 0.99), (64, 64, 64, 0.0),
])
def test_format_round_trip_and_invariants(M, K, TK, density):
    W, mask, _ = _rand_case(M * 1000 + K, M, K, 1, density, signed_zero=True)
    f = oracle.tcb_encode(W, mask, TK=TK)
    dec = oracle.tcb_decode(oracle.tcb_parse(f.blob()))
    want = np.where(mask, W.view(np.uint16), np.uint16(0))
    assert np.array_equal(dec, want)  # bit-exact, -0 kept where the mask keeps it
    assert f.nnz == int(mask.sum())
    pc = np.array([bin(int(b)).count("1") for b in f.bits])
    assert pc.sum() == f.nnz
    per_tile = pc.reshape(f.Mt * f.Kt, TK // 4).sum(axis=1)
    lens = np.diff(f.tile_ptr.astype(np.int64))
    assert np.all(lens % 8 == 0) and np.all(lens >= per_tile) and np.all(lens - per_tile < 8)
    for t in range(f.Mt * f.Kt):
        pad = f.values[f.tile_ptr[t] + per_tile[t]:f.tile_ptr[t + 1]]
        assert np.all(pad == 0)
    assert f.max_tile == (lens.max() if lens.size else 0)


def test_null_mask_keeps_nonzeros():
    W, _, _ = _rand_case(13, 70, 70, 1, 1.0, signed_zero=True)
    W[3, 3] = 0
    f = oracle.tcb_encode(W, None, TK=64)
    keep = (W.view(np.uint16) & 0x7FFF) != 0
    assert f.nnz == int(keep.sum())
    dec = oracle.tcb_decode(f)
    assert np.array_equal(dec, np.where(keep, W.view(np.uint16), 0))


# ---------------------------------------------------------------- column-run encoding (skipping)
def test_threshold_hand_worked():
    # values worked by hand from the rule (keep |x| >= tau); the tau = 0.5 case
    # sits on the boundary, so a strict comparison fails it, and thresholding W
    # instead of x or dropping the sign of x fails the others
    d = json.load(open(os.path.join(GOLDEN, "threshold_hand_example.json")))
    W = np.array(d["W"], dtype=np.float16)
    x = np.array([d["x"]], dtype=np.float16)
    for c in d["cases"]:
        xk = oracle.threshold_activations(x, c["tau"])
        assert np.array_equal(xk.astype(np.float64)[0], np.array(c["x_kept"])), c["tau"]
        y = oracle.masked_matmul_threshold(W, None, x, c["tau"])
        assert np.array_equal(y[0], np.array(c["y"])), c["tau"]


def test_threshold_invariants():
    g = np.random.default_rng(21)
    W = (0.1 * g.standard_normal((40, 300))).astype(np.float16)
    mask = g.random((40, 300)) < 0.5
    x = g.standard_normal((3, 300)).astype(np.float16)
    # tau = 0 is the plain product; tau above every |x| gives exact zeros
    assert np.allclose(oracle.masked_matmul_threshold(W, mask, x, 0.0), oracle.masked_matmul(W, mask, x), atol=1e-12)
    assert np.all(oracle.masked_matmul_threshold(W, mask, x, 1e4) == 0)
    # the kept set only shrinks as tau grows, and kept values are untouched
    prev = np.ones(x.shape, dtype=bool)
    for tau in (0.0, 0.1, 0.5, 1.0, 2.0):
        xk = oracle.threshold_activations(x, tau)
        kept = xk != 0
        assert np.all(kept <= prev) and np.array_equal(xk[kept], x[kept])
        prev = kept
    # a channel whose every token is below tau takes no part: changing its
    # weights changes nothing
    tau = 0.8
    dead = ~np.any(np.abs(x.astype(np.float32)) >= tau, axis=0)
    W2 = W.copy()
    W2[:, dead] = np.float16(7.0)
    assert np.array_equal(oracle.masked_matmul_threshold(W2, mask, x, tau), oracle.masked_matmul_threshold(W, mask, x, tau))


def test_threshold_keeps_nan_like_the_plain_product():
    # A NaN activation is not below any tau: it is kept, so the thresholded
    # product agrees with the plain skipping product at tau = 0 (NaN reaches
    # exactly the outputs whose kept weight in that column is nonzero or zero:
    # 0 * NaN is NaN), and an Inf stays too.  Infinities and NaNs in the same
    # column would make a dropped-versus-kept mistake visible as a NaN or as a
    # finite value.
    W = np.array([[1.0, 0.5, 0.0], [0.0, 2.0, 1.0]], dtype=np.float16)
    x = np.array([[np.nan, 0.25, np.inf]], dtype=np.float16)
    for tau in (0.0, 0.3, 1e4):
        xk = oracle.threshold_activations(x, tau)
        assert np.isnan(xk[0, 0]) and np.isinf(xk[0, 2])
    assert xk[0, 1] == 0  # 0.25 < 1e4 is dropped
    with np.errstate(invalid="ignore"):
        y0 = oracle.masked_matmul_threshold(W, None, x, 0.0)
        ys = oracle.masked_matmul_skip(W, None, x)
        y1 = oracle.masked_matmul_threshold(W, None, x, 0.3)
    assert np.array_equal(np.isnan(y0), np.isnan(ys)) and np.all(np.isnan(y0))
    assert np.all(np.isnan(y1))  # row 0: 1*NaN; row 1: 0*NaN + 2*0 + 1*Inf


def test_colruns_hand_worked_bytes():
    d = json.load(open(os.path.join(GOLDEN, "colruns_hand_example.json")))
    W = np.array(d["W_rows_fp16"], dtype=np.float16)
    c = oracle.colruns_encode(W, None)
    assert c.Mb == d["Mb"]
    assert list(c.ptr) == d["ptr"]
    assert [int(b) for b in c.bits] == d["bits"]
    assert [format(int(v), "04x") for v in c.values] == d["values_hex"]
    blob = c.blob()
    assert blob[:32] == bytes.fromhex(d["header_hex"].replace(" ", ""))
    Wd, keep = oracle.colruns_decode(oracle.colruns_parse(blob))
    assert np.array_equal(Wd, W.view(np.uint16)) and np.array_equal(keep, W != 0)
    # a row-major value order (the tiled format's is column by column in 16-row
    # slabs) must not reproduce the hand bytes
    Wb = W.view(np.uint16)
    assert [format(int(v), "04x") for v in Wb[Wb != 0]] != [v for v in d["values_hex"] if v != "0000"]


def test_colruns_group_order_hand_worked():
    # 1024 x 2 (four 256-row blocks, one group); kept: (row 700, column 0) and
    # (row 5, column 1).  Row 700 is block 2, word 2 ((700 - 512) // 64), bit
    # 60; its entry is (0*2 + 0)*4 + 2 = 2.  Row 5 is block 0, word 0, bit 5;
    # its entry is (0*2 + 1)*4 + 0 = 4.  Each run is one value padded to 4.
    W = np.zeros((1024, 2), dtype=np.float16)
    W[700, 0] = np.float16(1.5)
    W[5, 1] = np.float16(-2.0)
    c = oracle.colruns_encode(W, None)
    expect_bits = [0] * 32
    expect_bits[2 * 4 + 2] = 1 << 60
    expect_bits[4 * 4 + 0] = 1 << 5
    assert [int(v) for v in c.bits] == expect_bits
    assert list(c.ptr) == [0, 0, 0, 4, 4, 8, 8, 8, 8]
    assert [format(int(v), "04x") for v in c.values] == ["3e00", "0000", "0000", "0000", "c000", "0000", "0000", "0000"]


@pytest.mark.parametrize("M,K,density", [(1, 1, 1.0), (256, 64, 0.5), (257, 70, 0.3), (600, 40, 0.0),
                                         (513, 130, 1.0), (64, 300, 0.05), (1100, 40, 0.5)])
def test_colruns_round_trip_and_invariants(M, K, density):
    W, mask, _ = _rand_case(M * 977 + K, M, K, 1, density, signed_zero=True)
    c = oracle.colruns_encode(W, mask)
    Wd, keep = oracle.colruns_decode(oracle.colruns_parse(c.blob()))
    assert np.array_equal(keep, mask)
    assert np.array_equal(Wd, np.where(mask, W.view(np.uint16), np.uint16(0)))  # -0 kept where the mask keeps it
    pc = np.array([bin(int(b)).count("1") for b in c.bits]).reshape(-1, 4).sum(axis=1)
    assert pc.sum() == int(mask.sum())
    lens = np.diff(c.ptr.astype(np.int64))
    assert np.all(lens % 4 == 0) and np.all(lens >= pc) and np.all(lens - pc < 4)
    for e in range(len(lens)):
        assert np.all(c.values[c.ptr[e] + pc[e]:c.ptr[e + 1]] == 0)
    # same kept entries as the tiled format
    t = oracle.tcb_encode(W, mask, TK=64)
    assert np.array_equal(oracle.tcb_decode(t), Wd)


# ---------------------------------------------------------------- planted mistakes
def _mut_dropped_last_term(W, mask, X):
    return oracle.masked_matmul(W[:, :-1], None if mask is None else mask[:, :-1], X[:, :-1])


def _mut_mask_ignored(W, mask, X):
    return oracle.masked_matmul(W, None, X)


def _mut_sign(W, mask, X):
    Y = oracle.masked_matmul(W, mask, X)
    Y[:, 0] = -Y[:, 0]
    return Y


def _mut_transposed_weight(W, mask, X):
    Wt = np.ascontiguousarray(W.T)
    return oracle.masked_matmul(Wt, None if mask is None else mask.T, X[:, :Wt.shape[1]])


@pytest.mark.parametrize("mut", [_mut_dropped_last_term, _mut_mask_ignored, _mut_sign, _mut_transposed_weight])
def test_planted_mistakes_fail_the_pins(mut):
    W, mask, X = _rand_case(14, 24, 24, 3, 0.5)
    try:
        ok, _, _ = _check_against_exact(mut, W, mask, X)
    except Exception:
        ok = False
    assert not ok


def test_planted_format_mistakes_fail_hand_bytes():
    # plain row-major or plain column-major value orders must not reproduce the hand bytes
    d = json.load(open(os.path.join(GOLDEN, "tcb_hand_example.json")))
    W = np.array(d["W_rows_fp16"], dtype=np.float16)
    Wb = W.view(np.uint16)
    rowmajor = [format(int(v), "04x") for v in Wb[Wb != 0]]
    colmajor = [format(int(v), "04x") for v in Wb.T[Wb.T != 0]]
    assert rowmajor != d["values_hex"][:7]
    assert colmajor != d["values_hex"][:7]
    # a word layout with one column per 16-bit group in plain order (no interleave) differs
    f = oracle.tcb_encode(W, None, TK=32)
    assert [int(b) for b in f.bits] == d["bits"]
    assert int(f.bits[0]) != (1 | 4 | (1 << 17))


# ------------------------------------------------------------------ gated FFN hidden activation
def test_silu_closed_forms():
    """SiLU(z) = z / (1 + e^-z): values worked by hand, its odd-part identity
    SiLU(z) - SiLU(-z) = z, and its limits."""
    z = np.array([0.0, 1.0, -1.0, 2.0, -2.0])
    want = [0.0, 0.7310585786300049, -0.2689414213699951, 1.7615941559557649, -0.2384058440442351]
    assert np.allclose(oracle.silu(z), want, rtol=0, atol=1e-15)
    g = np.random.default_rng(31).standard_normal(1000) * 5
    assert np.allclose(oracle.silu(g) - oracle.silu(-g), g, rtol=0, atol=1e-12)
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-15
    assert 0 > oracle.silu(np.array([-40.0]))[0] > -1e-15
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0  # exp overflow handled


def test_gate_up_silu_hand_example():
    d = json.load(open(os.path.join(GOLDEN, "gate_up_silu_hand_example.json")))
    Wg, Wu = np.array(d["Wg"], dtype=np.float16), np.array(d["Wu"], dtype=np.float16)
    mg, mu = np.array(d["mask_g"], dtype=bool), np.array(d["mask_u"], dtype=bool)
    X = np.array(d["X"], dtype=np.float16)
    H = np.array(d["H"])
    for c in d["cases"]:
        got = oracle.gate_up_silu(Wg, mg, Wu, mu, X, c["tau"])
        want = np.where(np.array(c["kept"]), H, 0.0)
        assert np.allclose(got, want, rtol=0, atol=1e-15), c["tau"]
    # gate and up are not interchangeable, and the gate mask is applied
    assert not np.allclose(oracle.gate_up_silu(Wu, mu, Wg, mg, X), H, atol=1e-3)
    assert not np.allclose(oracle.gate_up_silu(Wg, None, Wu, mu, X), H, atol=1e-3)


def test_gate_up_silu_brute_force():
    """Pure-Python loops with math.exp on a small random case."""
    import math
    g = np.random.default_rng(32)
    M, K, N = 7, 13, 3
    Wg = (0.3 * g.standard_normal((M, K))).astype(np.float16)
    Wu = (0.3 * g.standard_normal((M, K))).astype(np.float16)
    mg, mu = g.random((M, K)) < 0.5, g.random((M, K)) < 0.6
    X = g.standard_normal((N, K)).astype(np.float16)
    got = oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0)
    for t in range(N):
        for m in range(M):
            gs = sum(float(Wg[m, k]) * float(X[t, k]) for k in range(K) if mg[m, k])
            us = sum(float(Wu[m, k]) * float(X[t, k]) for k in range(K) if mu[m, k])
            h = gs / (1.0 + math.exp(-gs)) * us
            assert abs(got[t, m] - h) <= 1e-12 * max(1.0, abs(h)), (t, m)


def test_gate_up_silu_threshold_invariants():
    g = np.random.default_rng(33)
    M, K, N = 40, 64, 4
    Wg = (0.1 * g.standard_normal((M, K))).astype(np.float16)
    Wu = (0.1 * g.standard_normal((M, K))).astype(np.float16)
    mg, mu = g.random((M, K)) < 0.5, g.random((M, K)) < 0.5
    X = g.standard_normal((N, K)).astype(np.float16)
    full = oracle.gate_up_silu(Wg, mg, Wu, mu, X, 0.0)
    assert np.all(oracle.gate_up_silu(Wg, mg, Wu, mu, X, 1e4) == 0)
    prev = np.ones(full.shape, dtype=bool)
    for tau in (0.0, 0.05, 0.1, 0.3):
        h = oracle.gate_up_silu(Wg, mg, Wu, mu, X, tau)
        kept = h != 0
        assert np.all(kept <= prev) and np.array_equal(h[kept], full[kept])
        # the decision is taken on the fp16-rounded value
        dec = np.abs(full.astype(np.float16).astype(np.float32)) >= np.float32(tau)
        assert np.array_equal(kept, dec & (full != 0))
        prev = kept
    # an all-pruned gate gives SiLU(0) = 0 everywhere
    assert np.all(oracle.gate_up_silu(Wg, np.zeros_like(mg), Wu, mu, X) == 0)

"""Pins of the seeded input generator (shared by both sides; no method arithmetic)."""
import numpy as np
import pytest
from scipy import integrate, stats

import swm_workloads as wl


def test_keep_count_round_half_even():
    assert wl.keep_count(4096, 0.5) == 2048
    assert wl.keep_count(4096, 0.6) == 1638
    assert wl.keep_count(4096, 0.7) == 1229
    assert wl.keep_count(11008, 0.5) == 5504
    assert wl.keep_count(5, 0.5) == 3  # round(2.5) = 2 (half to even)


def test_magnitude_prune_ties_go_to_lower_column():
    W = np.array([[0.5, -0.5, 0.25, 0.5, -0.25, 1.0]], dtype=np.float16)
    m = wl.magnitude_prune_mask(W, 0.5)  # keep 3: 1.0 at col 5, then 0.5s at cols 0, 1
    assert m.tolist() == [[True, True, False, False, False, True]]


def test_magnitude_prune_against_sort_definition():
    g = np.random.default_rng(0)
    W = g.choice(np.array([0.0, 0.25, -0.25, 0.5, 1.0, -1.0], dtype=np.float16), size=(40, 37))
    for s in (0.0, 0.3, 0.5, 0.7, 1.0):
        m = wl.magnitude_prune_mask(W, s)
        keep = wl.keep_count(37, s)
        for r in range(40):
            order = sorted(range(37), key=lambda c: (-abs(float(W[r, c])), c))
            assert set(np.nonzero(m[r])[0]) == set(order[:keep])


def test_pruned_weight_is_zero_where_pruned():
    W, mask = wl.pruned_weight(99, 0, 64, 128, 0.5)
    assert np.all(mask.sum(axis=1) == 64)
    assert np.all(W.view(np.uint16)[~mask] == 0)


def test_generators_are_deterministic():
    a = wl.activations(2, 0, 4, 100)
    b = wl.activations(2, 0, 4, 100)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    c = wl.activations(2, 1, 4, 100)
    assert not np.array_equal(a, c)


def test_tiny_mask_is_bernoulli_half():
    W, mask, X = wl.tiny()
    assert W.shape == (256, 512) and X.shape == (8, 512)
    assert abs(mask.mean() - 0.5) < 0.01
    assert np.all(W.view(np.uint16)[~mask] == 0)


def test_silu_threshold_zero_fraction_matches_distribution():
    """P(|SiLU(g) u| < tau) for g, u ~ N(0,1), by 1-D quadrature over g.

    For fixed g, |SiLU(g) u| < tau iff |u| < tau/|SiLU(g)|, probability
    2 Phi(tau/|s|) - 1.  The generator's empirical zero fraction must agree.
    """
    tau = 0.3

    def inner(gv):
        s = abs(gv / (1 + np.exp(-gv)))
        return stats.norm.pdf(gv) * (1.0 if s == 0 else (2 * stats.norm.cdf(tau / s) - 1))

    p, _ = integrate.quad(inner, -12, 12, points=[0.0], limit=200)
    x = wl.silu_gated_sparse(77, 0, 4, 50000, tau)
    frac = np.mean(x == 0)
    assert 0.69 < p < 0.72  # roughly 70% of entries fall below 0.3
    assert abs(frac - p) < 0.01
    assert np.all(np.abs(x[x != 0].astype(np.float64)) >= tau)


def test_prune_2_4_mask_rule():
    # every full group of 4 along K keeps exactly its 2 largest |w| (lower column
    # on ties); a short trailing group keeps its first half, rounded up
    g = np.random.default_rng(5)
    W = (g.standard_normal((50, 27)) * 0.02).astype(np.float16)
    W[0, :4] = np.float16(0.5)                     # all tied: columns 0, 1
    W[1, :4] = np.array([1, -3, 2, 2], dtype=np.float16)  # -3 then the first 2
    m = wl.prune_2_4_mask(W)
    assert m[0, :4].tolist() == [True, True, False, False]
    assert m[1, :4].tolist() == [False, True, True, False]
    groups = m[:, :24].reshape(50, 6, 4)
    assert np.all(groups.sum(axis=2) == 2)
    a = np.abs(W[:, :24].astype(np.float32)).reshape(50, 6, 4)
    kept_min = np.where(groups, a, np.inf).min(axis=2)
    drop_max = np.where(~groups, a, -np.inf).max(axis=2)
    assert np.all(kept_min >= drop_max)
    assert np.all(m[:, 24:26]) and not np.any(m[:, 26])


def test_layer_fused_groups_cover_each_linear_once():
    idx = [i for _, g in wl.LAYER_FUSED for i in g]
    assert sorted(idx) == list(range(7))
    for _, g in wl.LAYER_FUSED:   # a group's linears share K, so their rows stack
        assert len({wl.LLAMA7B_LINEARS[i][2] for i in g}) == 1


def test_stack_linears_rows_and_input():
    g = np.random.default_rng(3)
    parts = [(g.standard_normal((m, 8)).astype(np.float16), g.random((m, 8)) < 0.5,
              g.standard_normal((2, 8)).astype(np.float16)) for m in (3, 5)]
    W, mask, X = wl.stack_linears(parts)
    assert W.shape == (8, 8) and mask.shape == (8, 8)
    assert np.array_equal(W[3:], parts[1][0]) and np.array_equal(mask[:3], parts[0][1])
    assert X is parts[0][2]

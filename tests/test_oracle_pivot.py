"""Pins for the oracle's pivot modes ("HLG sampling -- a piecewise tone curve on the logits",
section "The pivot"): the pivot mu is computed from the full normalised log-prob vector
l = log-softmax(x) over the finite entries, as

  - top-anchored:     mu = l_max - c (the curve centred c nats below the most probable token);
  - entropy-anchored: mu = sum_i p_i l_i = -H(p), p = softmax(x).

Pins: scipy's entropy and logsumexp (independent implementations), closed forms (a row of n
equal logits has mu = -log n; a single finite logit has mu = 0; with the top anchor the most
probable token sits at z = c, so its transformed value is g(c)), invariance under a common
shift of the logits, and the draws of the independent pure-Python sampler given that mu.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

from tests.test_oracle_sampling import _chi2_pvalue, _py_draw, _softmax

CURVE = dict(m=1.5, w=1.0, beta_t=1.0, beta_h=2.0)


def _rows(seed=5):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 3, size=(6, 500))
    x[1, rng.choice(500, 200, replace=False)] = -np.inf
    x[2] *= 20.0                      # wide range
    x[3, :] = 1.25                    # flat
    x[4, :] = -np.inf
    x[4, 17] = 3.0                    # a single finite logit
    x[5, :] = -np.inf                 # no finite logit
    return x


def test_entropy_pivot_is_minus_entropy(oracle_mod):
    x = _rows()
    mu = oracle_mod.pivot(x, "entropy")
    for r in range(4):
        fin = np.isfinite(x[r])
        p = special.softmax(x[r][fin])
        assert mu[r] == pytest.approx(-stats.entropy(p), rel=1e-12, abs=1e-12), r
    assert mu[3] == pytest.approx(-math.log(500), rel=1e-14)
    assert mu[4] == 0.0
    assert math.isnan(mu[5])


@pytest.mark.parametrize("c", [0.0, 2.5, 6.0])
def test_top_pivot(oracle_mod, c):
    x = _rows()
    mu = oracle_mod.pivot(x, "top", c)
    for r in range(5):
        fin = np.isfinite(x[r])
        lse = special.logsumexp(x[r][fin])
        assert mu[r] == pytest.approx(x[r][fin].max() - lse - c, abs=1e-12), r
    assert math.isnan(mu[5])


@pytest.mark.parametrize("c", [0.5, 4.0])
def test_top_anchor_places_argmax_at_c(oracle_mod, c):
    x = _rows()[:5]
    lp = oracle_mod.hlg_transform(x, None, CURVE["m"], CURVE["w"], CURVE["beta_t"],
                                  CURVE["beta_h"], pivot="top", pivot_offset=c)
    want = oracle_mod.hlg_g(np.array([c]), CURVE["m"], CURVE["w"], CURVE["beta_t"],
                            CURVE["beta_h"])[0]
    for r in range(5):
        j = int(np.argmax(x[r]))
        assert lp[r, j] == pytest.approx(want, rel=1e-12, abs=1e-12), r
        assert np.all(lp[r] <= want + 1e-12)
    assert np.all(np.isneginf(lp[1][np.isneginf(x[1])]))


@pytest.mark.parametrize("mode", ["top", "entropy"])
def test_pivot_shift_invariant(oracle_mod, mode):
    x = _rows()[:5]
    a = oracle_mod.hlg_transform(x, None, 1.5, 1.0, 1.0, 2.0, pivot=mode, pivot_offset=3.0)
    b = oracle_mod.hlg_transform(x + 7.25, None, 1.5, 1.0, 1.0, 2.0, pivot=mode,
                                 pivot_offset=3.0)
    fin = np.isfinite(a)
    np.testing.assert_allclose(b[fin], a[fin], rtol=1e-9, atol=1e-9)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))


def test_bad_pivot_arguments(oracle_mod):
    x = _rows()[:1]
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.pivot(x, 4)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.pivot(x, "top", float("inf"))
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.sample(x, [1.0], [1], [0], hlg=dict(CURVE, pivot="top",
                                                          pivot_offset=float("nan")))


def _median_brute(x):
    """The mass median of one row by sorting in float64: the log-prob of the first group of
    equal logits (from the top) at which the probability mass reaches one half, and how far
    the running total before and after that group lies from one half."""
    fin = x[np.isfinite(x)]
    lse = special.logsumexp(fin)
    p = np.exp(fin - lse)
    cum = 0.0
    for v in np.unique(fin)[::-1]:
        before = cum
        cum += p[fin == v].sum()
        if cum >= 0.5:
            return v - lse, min(0.5 - before, cum - 0.5)
    raise AssertionError("mass never reached one half")


def test_median_pivot_closed_forms(oracle_mod):
    # a flat row: every token is the median, mu = -log(n)
    for n in (1, 7, 500):
        mu = oracle_mod.pivot(np.full((1, n), 2.5), "median")[0]
        assert abs(mu + math.log(n)) < 1e-12
    # one token of logit 5 over n - 1 of logit 0: it alone holds e^5 / (e^5 + n - 1) of the
    # mass, over one half for n = 100 (median at 5), under it for n = 1000 (median at 0)
    for n, top in ((100, True), (1000, False)):
        x = np.zeros((1, n))
        x[0, 3] = 5.0
        lse = math.log(math.exp(5.0) + (n - 1))
        want = (5.0 if top else 0.0) - lse
        assert abs(oracle_mod.pivot(x, "median")[0] - want) < 1e-12
    # -0 and +0 are one logit; masked entries take no part
    x = np.array([[0.0, -0.0, -np.inf, -3.0]])
    lse = math.log(2.0 + math.exp(-3.0))
    assert abs(oracle_mod.pivot(x, "median")[0] - (0.0 - lse)) < 1e-12


def test_median_pivot_matches_sorting(oracle_mod):
    rng = np.random.default_rng(67)
    x = rng.normal(0, 1.5, size=(40, 300))
    x[::3] = np.round(x[::3] * 2.0) / 2.0           # coarse grid: long runs of equal logits
    x[1::4, ::5] = -np.inf
    mu = oracle_mod.pivot(x, "median")
    checked = 0
    for r in range(x.shape[0]):
        want, margin = _median_brute(x[r])
        if margin < 1e-9:
            continue
        assert abs(mu[r] - want) < 1e-12, r
        checked += 1
    assert checked >= 35
    # a row with no finite logit has no pivot
    assert np.isnan(oracle_mod.pivot(np.full((1, 4), -np.inf), "median")[0])


@pytest.mark.parametrize("mode", ["top", "entropy", "median"])
def test_pivot_draws_match_brute_force(oracle_mod, mode):
    """The sampler with a pivot mode draws exactly what the independent pure-Python sampler
    draws given the mu of that mode (mu computed here with scipy, in float64)."""
    rng = np.random.default_rng(61)
    B, V, K = 4, 13, 5
    x = rng.normal(0, 1.2, size=(B, V))
    x[2, [1, 7]] = -np.inf
    T = np.array([1.0, 0.6, 1.4, 0.9], dtype=np.float32)
    seed = rng.integers(0, 2**64, size=B, dtype=np.uint64)
    offset = rng.integers(0, 2**40, size=B, dtype=np.uint64)
    c = 2.0
    hlg = dict(CURVE, pivot=mode, pivot_offset=c)
    idx, _, _ = oracle_mod.sample(x, T, seed, offset, K=K, hlg=hlg)
    for b in range(B):
        fin = np.isfinite(x[b])
        ell = x[b][fin] - special.logsumexp(x[b][fin])
        if mode == "top":
            mu = ell.max() - c
        elif mode == "entropy":
            mu = float(np.dot(np.exp(ell), ell))
        else:
            mu = _median_brute(x[b])[0]
        for k in range(K):
            off = (int(offset[b]) + k) % 2**64
            want = _py_draw(list(x[b]), b, float(T[b]), int(seed[b]), off,
                            tuple(CURVE[k_] for k_ in ("m", "w", "beta_t", "beta_h")), mu)
            assert idx[b, k] == want, (mode, b, k)


@pytest.mark.parametrize("mode", ["top", "entropy"])
def test_pivot_chi_square(oracle_mod, mode):
    rng = np.random.default_rng(71)
    x = np.concatenate([rng.normal(0, 2, 15), [-np.inf]])
    hlg = dict(CURVE, pivot=mode, pivot_offset=3.0)
    lp = oracle_mod.hlg_transform(x[None, :], None, CURVE["m"], CURVE["w"], CURVE["beta_t"],
                                  CURVE["beta_h"], pivot=mode, pivot_offset=3.0)[0]
    T = 0.8
    n = 300_000
    idx, _, _ = oracle_mod.sample(x[None, :], [T], [123], [0], K=n, hlg=hlg)
    counts = np.bincount(idx.ravel(), minlength=x.size)
    assert counts[-1] == 0
    assert _chi2_pvalue(counts, _softmax(lp / T), n) > 1e-3

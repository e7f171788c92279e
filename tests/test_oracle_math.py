"""Pins for the oracle's Gumbel map, HLG curve and log-sum-exp.

Gumbel map: high-precision values from mpmath, the endpoints, monotonicity and the moments of
the Gumbel law (mean = Euler's constant, variance = pi^2/6).

HLG curve ("HLG sampling -- a piecewise tone curve on the logits", section "The transfer
function" and its list "Properties that matter", section "The degeneracies are the safety
anchors"): g(0) = 0, g(+-w) = +-m w, slope m at the pivot and m*beta/(beta+d) at a distance d
past a knot (so C1 at the knots), monotone, -inf -> -inf without NaN, the rolloff-off
degeneracies, and ranking / argmax invariance.

Log-sum-exp: scipy's implementation, closed forms and shift invariance.
"""
import math

import numpy as np
import pytest

mpmath = pytest.importorskip("mpmath")


# --------------------------------------------------------------------------- Gumbel map
def _mp_gumbel(r):
    mpmath.mp.dps = 50
    u = (mpmath.mpf(int(r)) + mpmath.mpf(1) / 2) / mpmath.mpf(2) ** 32
    return float(-mpmath.log(-mpmath.log(u)))


def test_gumbel_high_precision(oracle_mod):
    rng = np.random.default_rng(3)
    words = np.concatenate([
        np.array([0, 1, 2, 3, 2**31 - 1, 2**31, 2**31 + 1, 2**32 - 3, 2**32 - 2, 2**32 - 1],
                 dtype=np.uint64),
        rng.integers(0, 2**32, size=300, dtype=np.uint64),
        (2**32 - 1 - rng.integers(0, 2**20, size=100, dtype=np.uint64)),
    ]).astype(np.uint32)
    got = oracle_mod.gumbel(words)
    for r, g in zip(words, got):
        want = _mp_gumbel(r)
        assert abs(g - want) <= 4e-15 * max(1.0, abs(want)), (int(r), g, want)


def test_gumbel_endpoints(oracle_mod):
    g = oracle_mod.gumbel(np.array([0, 2**32 - 1], dtype=np.uint32))
    # r = 0: u = 2^-33, -log u = 33 ln 2;  r = 2^32-1: u = 1 - 2^-33, -log u ~ 2^-33
    assert g[0] == pytest.approx(-math.log(33 * math.log(2)), rel=1e-14)
    assert g[1] == pytest.approx(33 * math.log(2), rel=1e-9)
    assert -3.131 < g[0] < -3.129 and 22.87 < g[1] < 22.88


def test_gumbel_monotone(oracle_mod):
    rng = np.random.default_rng(4)
    w = np.unique(rng.integers(0, 2**32, size=20000, dtype=np.uint64)).astype(np.uint32)
    g = oracle_mod.gumbel(w)
    assert np.all(np.diff(g) > 0)


def test_gumbel_law_moments(oracle_mod):
    w = oracle_mod.stream_words(2024, 0, 0, 1 << 20)
    g = oracle_mod.gumbel(w)
    n = g.size
    euler_gamma = 0.57721566490153286
    assert abs(g.mean() - euler_gamma) < 5 * math.pi / math.sqrt(6 * n)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    # P(G <= 0) = exp(-1) for the standard Gumbel law
    p0 = (g <= 0).mean()
    assert abs(p0 - math.exp(-1)) < 5 * math.sqrt(p0 * (1 - p0) / n)


# --------------------------------------------------------------------------- HLG curve
PARAMS = [
    (1.5, 2.0, 1.0, 2.0),
    (1.25, 1.5, 0.5, 1.0),
    (1.0 / 0.7, 4.0, 6.0, 4.0),   # exploration point of the design doc with T = 0.7
    (0.8, 0.25, 3.0, 0.1),
]


@pytest.mark.parametrize("m,w,bt,bh", PARAMS)
def test_curve_knots_and_pivot(oracle_mod, m, w, bt, bh):
    g = oracle_mod.hlg_g([0.0, w, -w], m, w, bt, bh)
    assert g[0] == 0.0
    assert g[1] == pytest.approx(m * w, rel=1e-15)
    assert g[2] == pytest.approx(-m * w, rel=1e-15)


@pytest.mark.parametrize("m,w,bt,bh", PARAMS)
def test_curve_slopes(oracle_mod, m, w, bt, bh):
    """Slope m inside the mid band, m*beta/(beta+d) a distance d past each knot; both
    one-sided slopes at the knots equal m (C1)."""
    h = 1e-6
    for z in [0.0, 0.3 * w, -0.7 * w]:
        d = oracle_mod.hlg_g([z - h, z + h], m, w, bt, bh)
        assert (d[1] - d[0]) / (2 * h) == pytest.approx(m, rel=1e-6)
    for dist in [1e-3, 0.5, 2.0, 17.0]:
        zs = w + dist
        d = oracle_mod.hlg_g([zs - h, zs + h], m, w, bt, bh)
        assert (d[1] - d[0]) / (2 * h) == pytest.approx(m * bh / (bh + dist), rel=1e-5)
        zt = -w - dist
        d = oracle_mod.hlg_g([zt - h, zt + h], m, w, bt, bh)
        assert (d[1] - d[0]) / (2 * h) == pytest.approx(m * bt / (bt + dist), rel=1e-5)
    # one-sided slopes at the knots
    for knot in (w, -w):
        gk = oracle_mod.hlg_g([knot - 1e-7, knot, knot + 1e-7], m, w, bt, bh)
        left = (gk[1] - gk[0]) / 1e-7
        right = (gk[2] - gk[1]) / 1e-7
        assert left == pytest.approx(m, rel=1e-5)
        assert right == pytest.approx(m, rel=1e-5)


@pytest.mark.parametrize("m,w,bt,bh", PARAMS)
def test_curve_monotone_and_ranking(oracle_mod, m, w, bt, bh):
    rng = np.random.default_rng(5)
    z = np.sort(rng.normal(0, 3 * w + 1, size=20000))
    g = oracle_mod.hlg_g(z, m, w, bt, bh)
    assert np.all(np.diff(g) >= 0)
    strict = np.diff(z) > 1e-9 * (1 + np.abs(z[1:]))
    assert np.all(np.diff(g)[strict] > 0)
    x = rng.normal(0, 3, size=(50, 1000))
    for row in x:
        gr = oracle_mod.hlg_g(row, m, w, bt, bh)
        assert np.argmax(gr) == np.argmax(row)
        np.testing.assert_array_equal(np.argsort(gr, kind="stable"), np.argsort(row, kind="stable"))


@pytest.mark.parametrize("m,w,bt,bh", PARAMS)
def test_curve_masks_survive(oracle_mod, m, w, bt, bh):
    g = oracle_mod.hlg_g([-np.inf], m, w, bt, bh)
    assert g[0] == -np.inf
    g = oracle_mod.hlg_g([-np.inf], m, np.inf, bt, bh)
    assert g[0] == -np.inf


def test_curve_odd_when_rolloffs_equal(oracle_mod):
    z = np.linspace(-20, 20, 4001)
    g = oracle_mod.hlg_g(z, 1.3, 1.7, 2.5, 2.5)
    np.testing.assert_allclose(g, -g[::-1], rtol=0, atol=1e-13)


def test_curve_tails_are_logarithmic(oracle_mod):
    """Far past the knots the curve grows like m*beta*ln|z| (shoulder) and falls like
    -m*beta*ln|z| (toe): the increments over a decade of z approach m*beta*ln 10."""
    m, w, bt, bh = 1.5, 2.0, 1.0, 2.0
    g = oracle_mod.hlg_g([1e6, 1e7, -1e6, -1e7], m, w, bt, bh)
    assert g[1] - g[0] == pytest.approx(m * bh * math.log(10), rel=1e-5)
    assert g[2] - g[3] == pytest.approx(m * bt * math.log(10), rel=1e-5)


def test_curve_degeneracies(oracle_mod):
    """Rolloff off (w = inf) gives g = m z bit-exactly; m = 1 with rolloff off is the
    identity; a huge rolloff constant tends to m z."""
    rng = np.random.default_rng(6)
    z = rng.normal(0, 10, size=5000)
    np.testing.assert_array_equal(oracle_mod.hlg_g(z, 1.0, np.inf, 1.0, 1.0), z)
    m = 1.0 / 0.7
    np.testing.assert_array_equal(oracle_mod.hlg_g(z, m, np.inf, 3.0, 4.0), m * z)
    np.testing.assert_allclose(oracle_mod.hlg_g(z, m, 0.5, 1e300, 1e300), m * z, rtol=1e-12)


# --------------------------------------------------------------------------- LSE
def test_logsumexp_against_scipy(oracle_mod):
    from scipy.special import logsumexp
    rng = np.random.default_rng(7)
    x = rng.normal(0, 4, size=(8, 5000))
    x[2, rng.choice(5000, 1000, replace=False)] = -np.inf
    got = oracle_mod.logsumexp(x)
    for b in range(8):
        row = x[b][np.isfinite(x[b])]
        assert got[b] == pytest.approx(logsumexp(row), rel=1e-14, abs=1e-13)


def test_logsumexp_closed_forms(oracle_mod):
    x = np.full((1, 1000), 3.25)
    assert oracle_mod.logsumexp(x)[0] == pytest.approx(3.25 + math.log(1000), rel=1e-15)
    y = np.full((1, 10), -np.inf)
    assert oracle_mod.logsumexp(y)[0] == -np.inf
    z = np.full((1, 10), -np.inf)
    z[0, 4] = -7.5
    assert oracle_mod.logsumexp(z)[0] == -7.5
    rng = np.random.default_rng(8)
    r = rng.normal(0, 2, size=(1, 777))
    assert oracle_mod.logsumexp(r + 100.0)[0] == pytest.approx(oracle_mod.logsumexp(r)[0] + 100.0,
                                                               rel=1e-14)


def test_logsumexp_is_compensated(oracle_mod):
    """One term of 1 beside 10^6 terms of exp(-40) ~ 4.25e-18: each tiny term is below half an
    ulp of the running sum, so a plain double sum stays exactly 1 and gives LSE = 0. The
    compensated sum keeps them: LSE = log1p(10^6 exp(-40)) (closed form)."""
    n = 1_000_000
    x = np.full((1, n + 1), -40.0)
    x[0, 0] = 0.0
    want = math.log1p(n * math.exp(-40.0))
    got = oracle_mod.logsumexp(x)[0]
    assert got == pytest.approx(want, rel=1e-9)
    assert got > 0.0


def test_transform_is_curve_of_centred_logprob(oracle_mod):
    """l' = g(l - mu), l = x - LSE(x): checked against scipy's log-softmax and the
    pivot/knot identities; masked entries stay -inf."""
    from scipy.special import log_softmax
    rng = np.random.default_rng(9)
    x = rng.normal(0, 3, size=(3, 4000))
    x[1, :100] = -np.inf
    mu = np.array([-8.0, -9.5, -7.25], dtype=np.float32)
    m, w, bt, bh = 1.5, 2.0, 1.0, 2.0
    out = oracle_mod.hlg_transform(x, mu, m, w, bt, bh)
    for b in range(3):
        fin = np.isfinite(x[b])
        ls = np.full(x.shape[1], -np.inf)
        ls[fin] = log_softmax(x[b][fin])
        z = ls - float(mu[b])
        mid = np.abs(z) <= w
        np.testing.assert_allclose(out[b][mid], m * z[mid], rtol=1e-12, atol=1e-12)
        assert np.all(out[b][~fin] == -np.inf)
        assert np.all(out[b][fin & (z > w)] > m * w)
        assert np.all(out[b][fin & (z < -w)] < -m * w)


def test_oracle_rejects_nan_and_posinf(oracle_mod):
    x = np.zeros((1, 8))
    x[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle_mod.logsumexp(x)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle_mod.sample(x, [1.0], [1], [0])
    with pytest.raises(ValueError):
        oracle_mod.hlg_transform(np.zeros((1, 4)), [0.0], 0.0, 1.0, 1.0, 1.0)

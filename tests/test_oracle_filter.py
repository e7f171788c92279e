"""Pins for the oracle's top-k / top-p filters on the Gumbel path (curve off).

"Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (mlxcel issue #900) names
rejection-based top-k / top-p as the follow-on without giving an algorithm. Reading, as
documented in the oracle: temperature first, then top-k, then top-p on the tempered
probabilities of the tokens top-k keeps; each filter is a threshold on the logit and every
token at or above it is kept (ties included); the draw is the Gumbel-max of x / T over the
kept tokens (section Background: an exact sample of softmax(x / T), here renormalised over the
kept set).

Pins: an independent numpy implementation of the kept set (np.unique groups and np.cumsum),
closed cases (k = 1 and a tiny p keep only the largest logit; k >= n with p = 1 is the
unfiltered sampler, ids and scores), the pure-Python brute-force sampler on the kept set, and
chi-square tests of the draws against the renormalised softmax (threshold as in
test_oracle_sampling: expected counts below 5 pooled, p-value above 1e-3).
"""
import math

import numpy as np
import pytest

from tests.test_oracle_sampling import _chi2_pvalue, _py_word


def _np_tau(x, T, k, p):
    """Independent kept-set threshold: distinct finite logits in descending order with their
    multiplicities, top-k by counting, top-p by a cumulative sum of group masses."""
    fin = x[np.isfinite(x)]
    if T == 0 or fin.size == 0:
        return -np.inf
    vals, counts = np.unique(fin, return_counts=True)
    vals, counts = vals[::-1], counts[::-1]
    tau = -np.inf
    keep_groups = len(vals)
    if 0 < k < fin.size:
        covered = np.cumsum(counts)
        g = int(np.searchsorted(covered, k))      # group holding the k-th largest
        tau = vals[g]
        keep_groups = g + 1
    if p < 1:
        mass = counts[:keep_groups] * np.exp((vals[:keep_groups] - vals[0]) / T)
        cum = np.cumsum(mass)
        g = int(np.argmax(cum >= p * cum[-1]))
        tau = max(tau, vals[g])
    return tau


def _rows(seed=3):
    rng = np.random.default_rng(seed)
    rows = [rng.normal(0, 2, 300),
            np.round(rng.normal(0, 1, 200) * 4) / 4,          # many ties
            np.where(rng.random(250) < 0.3, -np.inf, rng.normal(1, 3, 250)),
            np.concatenate([[8.0], rng.normal(0, 0.5, 99)]),   # one dominant token
            rng.normal(0, 0.05, 120)]                        # nearly flat
    V = max(len(r) for r in rows)
    x = np.full((len(rows), V), -np.inf)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    return x


@pytest.mark.parametrize("k,p", [(1, 1.0), (5, 1.0), (50, 1.0), (0, 0.5), (0, 0.9),
                                 (0, 0.999), (20, 0.8), (3, 0.3), (1000, 0.95)])
@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_threshold_matches_numpy(oracle_mod, k, p, T):
    x = _rows()
    n = x.shape[0]
    tau, amb = oracle_mod.filter_threshold(x, [T] * n, top_k=[k] * n, top_p=[p] * n)
    for r in range(n):
        want = _np_tau(x[r], T, k, p)
        if amb[r]:
            continue
        assert tau[r] == want, (r, tau[r], want)


def test_kept_set_properties(oracle_mod):
    x = _rows(7)
    n = x.shape[0]
    for k, p in [(7, 1.0), (0, 0.6), (15, 0.5)]:
        tau, _ = oracle_mod.filter_threshold(x, [1.0] * n, top_k=[k] * n, top_p=[p] * n)
        for r in range(n):
            fin = x[r][np.isfinite(x[r])]
            kept = fin[fin >= tau[r]]
            assert fin.max() in kept                            # the argmax is always kept
            if k > 0:
                # at least min(k, n) tokens when only top-k acts; ties may add more
                if p >= 1:
                    assert kept.size >= min(k, fin.size)
                    assert (fin > tau[r]).sum() < k or kept.size == fin.size
            if p < 1:
                # the kept tokens carry at least p of the mass top-k keeps
                w = np.exp(fin - fin.max())
                base = w[fin >= _np_tau(x[r], 1.0, k, 1.0)].sum()
                assert w[fin >= tau[r]].sum() >= p * base * (1 - 1e-12)


def test_closed_cases(oracle_mod):
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1.5, size=(6, 400))
    x[:, ::7] = -np.inf
    T = np.full(6, 0.8, dtype=np.float32)
    seed = rng.integers(0, 2**64, size=6, dtype=np.uint64)
    off = rng.integers(0, 2**40, size=6, dtype=np.uint64)
    K = 40
    top = np.nanargmax(np.where(np.isfinite(x), x, -np.inf), axis=1)
    for k, p in [(1, 1.0), (0, 1e-6), (1, 1e-6)]:
        ids = oracle_mod.sample_filtered(x, T, seed, off, K=K, top_k=[k] * 6, top_p=[p] * 6)[0]
        assert np.all(ids == top[:, None])
    # nothing filtered: the unfiltered sampler, ids and both scores
    a = oracle_mod.sample_filtered(x, T, seed, off, K=K, top_k=[400] * 6, top_p=[1.0] * 6)
    b = oracle_mod.sample(x, T, seed, off, K=K)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])
    assert np.all(np.isneginf(a[3]))


def test_invalid_and_special_rows(oracle_mod):
    x = np.zeros((6, 5))
    x[0, :] = -np.inf
    x[5] = [0.0, 2.0, 1.0, 2.0, -1.0]
    T = np.array([1.0, 1.0, 1.0, -1.0, np.nan, 0.0], dtype=np.float32)
    p = np.array([0.5, 0.0, np.nan, 0.5, 0.5, 0.01], dtype=np.float32)
    ids = oracle_mod.sample_filtered(x, T, np.arange(6, dtype=np.uint64),
                                     np.zeros(6, dtype=np.uint64), K=2, top_k=[0] * 6,
                                     top_p=p)[0]
    assert ids[0].tolist() == [-1, -1]                      # no finite logit
    assert ids[1].tolist() == [-2, -2] and ids[2].tolist() == [-2, -2]   # p <= 0, NaN
    assert ids[3].tolist() == [-2, -2] and ids[4].tolist() == [-2, -2]   # bad T
    assert ids[5].tolist() == [1, 1]                        # greedy: the first argmax


def _py_draw_filtered(x, row, T, seed, off, k, p):
    """Pure Python: the kept set by sorting, then the Gumbel-max over it."""
    fin = sorted((v for v in x if v > -math.inf), reverse=True)
    if not fin:
        return -1
    if T == 0:
        return max(range(len(x)), key=lambda i: (x[i], -i))
    tau = -math.inf
    kept = fin
    if 0 < k < len(fin):
        tau = fin[k - 1]
        kept = [v for v in fin if v >= tau]
    if p < 1:
        w = [math.exp((v - fin[0]) / T) for v in kept]
        S, cum = math.fsum(w), 0.0
        for i, v in enumerate(kept):
            cum += w[i]
            # all logits equal to v are in the prefix before the test
            if i + 1 < len(kept) and kept[i + 1] == v:
                continue
            if cum >= p * S:
                tau = max(tau, v)
                break
    best, j = -math.inf, -1
    for i, v in enumerate(x):
        if not v > -math.inf or v < tau:
            continue
        u = (_py_word(seed, row, off, i) + 0.5) / 2.0 ** 32
        s = v / T - math.log(-math.log(u))
        if j < 0 or s > best:
            best, j = s, i
    return j


def test_brute_force_tiny(oracle_mod):
    rng = np.random.default_rng(19)
    B, V, K = 6, 13, 5
    x = np.round(rng.normal(0, 1, size=(B, V)) * 8) / 8      # ties
    x[2, [1, 4]] = -np.inf
    T = np.array([1.0, 0.6, 1.4, 1.0, 0.9, 0.0], dtype=np.float32)
    k = np.array([3, 0, 5, 13, 1, 2], dtype=np.int32)
    p = np.array([1.0, 0.7, 0.9, 0.5, 1.0, 0.3], dtype=np.float32)
    seed = np.array([1, 2**64 - 1, 77, 5, 6, 9], dtype=np.uint64)
    off = np.array([0, 2**32 - 2, 3, 2**63, 1, 0], dtype=np.uint64)
    rid = np.array([0, 1, 40, 3, 4, 5], dtype=np.int64)
    ids, _, _, _, amb = oracle_mod.sample_filtered(x, T, seed, off, K=K, top_k=k, top_p=p,
                                                   row_id=rid)
    for b in range(B):
        if amb[b]:
            continue
        for d in range(K):
            want = _py_draw_filtered(list(x[b]), int(rid[b]), float(T[b]), int(seed[b]),
                                     (int(off[b]) + d) % 2**64, int(k[b]), float(p[b]))
            assert ids[b, d] == want, (b, d)


def _restricted_softmax(x, T, tau):
    w = np.where(x >= tau, np.exp((x - x.max()) / T), 0.0)
    return w / w.sum()


@pytest.mark.parametrize("k,p", [(5, 1.0), (0, 0.7), (6, 0.8)])
@pytest.mark.parametrize("T", [0.7, 1.3])
def test_chi_square_filtered(oracle_mod, k, p, T):
    rng = np.random.default_rng(int(T * 10) + k)
    x = rng.normal(0, 1.2, 12)
    n = 200_000
    ids, _, _, tau, amb = oracle_mod.sample_filtered(x[None, :], [T], [123], [0], K=n,
                                                     top_k=[k], top_p=[p])
    assert not amb[0]
    probs = _restricted_softmax(x, T, tau[0])
    counts = np.bincount(ids.ravel(), minlength=x.size)
    assert np.all(counts[probs == 0] == 0)
    assert _chi2_pvalue(counts, probs, n) > 1e-3

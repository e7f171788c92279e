"""The curve set per row in one launch (hs_sample_rows) against the oracle, row by row: each
row is sampled as the oracle samples that row alone with its own setting (the curve off, or
its own knobs and pivot mode), keyed by its global row index ("HLG sampling -- a piecewise
tone curve on the logits", sections Knobs and The pivot: settings arrive per request; mlxcel
issue "Softmax-free GPU sampling", section Background: the draw of a row depends on (seed,
row, element, offset) only).

A row whose setting is invalid gives -2, as the per-call entry points reject the same
setting. Rows that share one setting give bit-identical ids and scores to the per-call path
with that setting."""
import math

import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import assert_parity, on_device, require_gpu

pytestmark = pytest.mark.gpu

A = {"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0}
B_ = {"m": 0.8, "w": 0.5, "beta_t": 3.0, "beta_h": 0.5}
SETTINGS = [
    None,
    dict(A),
    dict(A, pivot="top", pivot_offset=2.0),
    dict(A, pivot="entropy"),
    dict(B_),
    dict(B_, pivot="top", pivot_offset=-1.0),
    dict(B_, pivot="entropy"),
    {"m": 1.25, "w": math.inf, "beta_t": 0.5, "beta_h": 1.0},
]


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _oracle_rows(O, w, settings, bad=(), layout="plain"):
    """Per-row oracle results: ids, best and second-best scores [B, K]; rows in bad give -2."""
    B, K = w.B, w.K
    idx = np.zeros((B, K), dtype=np.int64)
    s1 = np.full((B, K), np.nan)
    s2 = np.full((B, K), np.nan)
    for r in range(B):
        if r in bad:
            idx[r] = -2
            continue
        h = settings[r]
        mu = None
        if h is not None:
            mu = w.mu[r:r + 1] if h.get("pivot", "input") == "input" else None
        o, a1, a2 = O.sample(w.logits[r:r + 1], w.T[r:r + 1], w.seed[r:r + 1],
                             w.offset[r:r + 1], K=K, mu=mu, hlg=h,
                             row_id=np.array([r], dtype=np.int64), layout=layout)
        idx[r], s1[r], s2[r] = o[0], a1[0], a2[0]
    return idx, s1, s2


def _cycle(B):
    return [SETTINGS[r % len(SETTINGS)] for r in range(B)]


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 151936), (torch.float32, 50001),
                                     (torch.float16, 4099)])
def test_mixed_rows_match_oracle(hs, oracle_mod, dtype, V):
    B, K = 16, 3
    w = W.generic(B, V, dtype, seed=V % 1000 + 3, scale=1.0, mask_frac=0.05, hlg=dict(A), K=K)
    w.T[[5, 13]] = 0.0                       # greedy rows, curve on and off
    w.T[8] = 0.0
    settings = _cycle(B)
    d = on_device(w)
    o, s1, s2 = _oracle_rows(oracle_mod, w, settings)
    x64 = w.logits.double().numpy()
    rows = hs.hlg_rows(settings)
    for name, opts in [("auto", None), ("one-block", hs.SampleOpts(variant=1)),
                       ("split7", hs.SampleOpts(variant=2, nchunk=7)),
                       ("split5-groups2", hs.SampleOpts(variant=2, nchunk=5, draw_groups=2)),
                       ("split7-exchange", hs.SampleOpts(variant=2, nchunk=7, draw_groups=1,
                                                         split_lse=2)),
                       ("split7-exchange-nowait", hs.SampleOpts(variant=2, nchunk=7,
                                                                draw_groups=1, split_lse=2,
                                                                exchange_wait=-1))]:
        g = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], rows, mu=d["mu"], k=K,
                           opts=opts).cpu().numpy()
        assert_parity(g, o, s1, s2, x64, "mixed rows %s %s" % (dtype, name))


def test_invalid_and_empty_rows(hs, oracle_mod):
    B, V, K = 12, 3001, 2
    w = W.generic(B, V, torch.float32, seed=17, hlg=dict(A), K=K)
    w.logits[10, :] = float("-inf")          # no finite logit: -1 (curve on, given pivot)
    w.logits[11, :] = float("-inf")          # the same with the curve off
    w.mu[6] = np.nan                         # given pivot with a NaN mu: -2
    settings = [dict(A), {"m": 0.0, "w": 1.0, "beta_t": 1.0, "beta_h": 1.0},
                {"m": 1.0, "w": -1.0, "beta_t": 1.0, "beta_h": 1.0},
                {"m": 1.0, "w": 1.0, "beta_t": math.inf, "beta_h": 1.0},
                {"m": 1.0, "w": 1.0, "beta_t": 1.0, "beta_h": float("nan")},
                dict(A, pivot="top", pivot_offset=float("nan")),
                dict(A), None, dict(A, pivot="entropy"), dict(A, pivot=7), dict(A), None]
    bad = {1, 2, 3, 4, 5, 6, 9}
    d = on_device(w)
    rows = hs.hlg_rows(settings)
    # a reserved field that is not zero makes a row with its curve on invalid too (row 8)
    rows8 = rows.clone()
    rows8[8, 28:32] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device=rows.device)
    g = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], rows, mu=d["mu"],
                       k=K).cpu().numpy()
    o, s1, s2 = _oracle_rows(oracle_mod, w, settings, bad=bad)
    assert_parity(g, o, s1, s2, w.logits.double().numpy(), "invalid rows")
    assert all(g[r].tolist() == [-2] * K for r in bad)
    assert g[10].tolist() == [-1] * K and g[11].tolist() == [-1] * K
    g8 = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], rows8, mu=d["mu"],
                        k=K).cpu().numpy()
    assert g8[8].tolist() == [-2] * K
    np.testing.assert_array_equal(np.delete(g8, 8, 0), np.delete(g, 8, 0))
    # without a mu array only the given-pivot rows fail
    gn = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], rows, k=K).cpu().numpy()
    given = {0, 6, 10}   # row 10 has no finite logit, but an invalid setting takes precedence
    for r in range(B):
        if r in given | bad:
            assert gn[r].tolist() == [-2] * K, r
        else:
            np.testing.assert_array_equal(gn[r], g[r])


@pytest.mark.parametrize("setting", [None, dict(A), dict(A, pivot="top", pivot_offset=2.0),
                                     dict(A, pivot="entropy"), dict(B_),
                                     dict(A, pivot="median")],
                         ids=["off", "given", "top", "entropy", "given-B", "median"])
@pytest.mark.parametrize("variant", ["one-block", "split7"])
def test_uniform_rows_equal_per_call(hs, setting, variant):
    """All rows sharing one setting: bit-identical ids and winning scores to hs_sample_ex with
    that setting (the curve off: hlg = NULL)."""
    B, V, K = 8, 60000, 4
    w = W.generic(B, V, torch.bfloat16, seed=29, scale=1.2, mask_frac=0.02, hlg=dict(A), K=K)
    w.T[3] = 0.0
    d = on_device(w)
    median = setting is not None and setting.get("pivot") == "median"
    opts = hs.SampleOpts(variant=1) if variant == "one-block" else hs.SampleOpts(variant=2,
                                                                                 nchunk=7)
    opts.median_rows = int(median)   # the caller says whether any row asks for the median
    rows = hs.hlg_rows([setting] * B)
    g, gb = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], rows, mu=d["mu"], k=K,
                           opts=opts, want_best=True)
    ref, rb = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"],
                           mu=d["mu"] if setting is not None else None, hlg=setting, k=K,
                           opts=opts, want_best=True)
    np.testing.assert_array_equal(g.cpu().numpy(), ref.cpu().numpy())
    np.testing.assert_array_equal(gb.cpu().numpy(), rb.cpu().numpy())


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 151936), (torch.float32, 50001)])
def test_mixed_rows_with_median(hs, oracle_mod, dtype, V):
    """Median-pivot rows among the others: their shifts come from a first kernel that skips
    every other row. Compared with the oracle on the rows whose mass boundary is decided away
    from one half (the median rows) and on every other row."""
    from tests.test_gpu_pivot import _median_sure
    B, K = 12, 3
    w = W.generic(B, V, dtype, seed=V % 997 + 11, scale=1.0, mask_frac=0.05, hlg=dict(A), K=K)
    w.T[7] = 0.0
    settings = [None, dict(A, pivot="median"), dict(A), dict(B_, pivot="median"),
                dict(A, pivot="top", pivot_offset=1.0), dict(A, pivot="entropy")] * 2
    d = on_device(w)
    o, s1, s2 = _oracle_rows(oracle_mod, w, settings)
    med = np.array([h is not None and h.get("pivot") == "median" for h in settings])
    sure = ~med | _median_sure(oracle_mod, w)
    x64 = w.logits.double().numpy()
    rows = hs.hlg_rows(settings)
    assert (~sure).sum() <= 1, (~sure).sum()
    for name, opts in [("auto", hs.SampleOpts(median_rows=1)),
                       ("split7", hs.SampleOpts(variant=2, nchunk=7, median_rows=1))]:
        g = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], rows, mu=d["mu"], k=K,
                           opts=opts).cpu().numpy()
        assert_parity(g[sure], o[sure], s1[sure], s2[sure], x64[sure],
                      "rows with median %s %s" % (dtype, name))
        assert np.all(g >= 0)
    # without median_rows no shift launch runs: the median rows give -2, the others the same
    gn = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], rows, mu=d["mu"],
                        k=K).cpu().numpy()
    assert np.all(gn[med] == -2)
    np.testing.assert_array_equal(gn[~med], g[~med])


@pytest.mark.parametrize("layout", ["plain", "screened"])
def test_mixed_rows_headline_shape(hs, oracle_mod, layout):
    """256 x 151936 bf16, the headline shape, with the eight settings cycled over the rows."""
    w = W.config4()
    settings = _cycle(w.B)
    d = on_device(w)
    g = hs.sample_rows(d["logits"], d["T"], d["seed"], d["offset"], hs.hlg_rows(settings),
                       mu=d["mu"], k=1,
                       opts=hs.SampleOpts(layout=hs.LAYOUTS[layout])).cpu().numpy()
    o, s1, s2 = _oracle_rows(oracle_mod, w, settings, layout=layout)
    print(assert_parity(g, o, s1, s2, w.logits.double().numpy(), "mixed 256x151936 " + layout))

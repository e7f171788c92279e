"""The curve's pivot modes on the HIP path against the oracle [HLG, The pivot]: the pivot
given per row, top-anchored (mu = l_max - c, so z = x - (x_max - c)), entropy-anchored
(mu = sum p l, so z = x - E_p[x]) and the mass median (z = x - x_med).

Tolerances. The kernels form the shift c of z = x - c in fp32 from fp32 sums: c = LSE + mu
(given pivot, LSE within 4e-6 max(1, |LSE|)), c = x_max - offset (top; one rounding), or
c = M + ln2 U/S with U = sum 2^t t, S = sum 2^t (entropy; two fp32 sums, each within a few
1e-7 relative per partial, the mean t-value within 4e-6 max(1, |M|, |c|)). The pivot
mu = c - LSE carries both errors: it is checked within 1e-5 max(1, |LSE|, |mu|). A transformed
logit g(x - c) moves by at most m |dc| (the curve's slope is at most m) beyond its own fp32
rounding, so it is checked within 1e-5 max(1, |g|) + m 1e-5 max(1, |c|). Sampled ids follow
the near-tie rule of the other parity tests."""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import assert_parity, gpu_sample, on_device, oracle_sample, require_gpu

pytestmark = pytest.mark.gpu

CURVE = {"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0}
MODES = [("input", 0.0), ("top", 2.0), ("top", -1.5), ("entropy", 0.0), ("median", 0.0)]
ANCHORED = [("top", 2.0), ("top", 0.0), ("entropy", 0.0)]


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _curve(mode, off, base=CURVE):
    h = dict(base)
    h["pivot"] = mode
    h["pivot_offset"] = off
    return h


def _tiny_with_empty_row():
    w = W.generic(4, 7, torch.float32, seed=10, mask_frac=0.3,
                  hlg={"m": 0.8, "w": 0.25, "beta_t": 3.0, "beta_h": 0.1})
    w.logits[2, :] = float("-inf")
    return w


CASES = [
    ("fp32 bimodal 8x151936", lambda: W.config3()),
    ("bf16 flat 16x151936", lambda: W.config4(B=16)),
    ("f16 ragged 5x4099", lambda: W.generic(5, 4099, torch.float16, seed=9, scale=1.5,
                                            mask_frac=0.2, hlg=dict(CURVE))),
    ("fp32 tiny 4x7 empty row", _tiny_with_empty_row),
]


@pytest.mark.parametrize("mode,off", MODES, ids=["%s%g" % m for m in MODES])
@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_pivot_values_and_transform(hs, oracle_mod, name, make, mode, off):
    w = make()
    x = w.logits.cuda()
    h = _curve(mode, off, w.hlg)
    mu = torch.from_numpy(w.mu).cuda()
    lse = oracle_mod.logsumexp(w.logits)
    ref_mu = oracle_mod.pivot(w.logits, mode, off, mu=w.mu)
    got_mu = hs.hlg_pivot(x, h, mu=mu).cpu().numpy().astype(np.float64)
    # the median: rows whose boundary is decided away from one half (see _median_sure)
    sel = _median_sure(oracle_mod, w) if mode == "median" else np.ones(w.B, dtype=bool)
    empty = ~np.isfinite(lse)
    assert np.all(np.isnan(got_mu[empty])) and np.all(np.isnan(ref_mu[empty]))
    f = ~empty & sel
    tol = 1e-5 * np.maximum.reduce([np.ones(f.sum()), np.abs(lse[f]), np.abs(ref_mu[f])])
    assert np.all(np.abs(got_mu[f] - ref_mu[f]) <= tol), np.abs(got_mu[f] - ref_mu[f]).max()

    lp = hs.hlg_transform(x, mu, h).cpu().numpy().astype(np.float64)
    ref = oracle_mod.hlg_transform(w.logits, w.mu, h["m"], h["w"], h["beta_t"], h["beta_h"],
                                   pivot=mode, pivot_offset=off)
    masked = ~np.isfinite(w.logits.double().numpy())
    assert np.all(lp[masked] == -np.inf)
    fin = ~masked & sel[:, None]
    c = (lse + ref_mu)[:, None] * np.ones_like(ref)      # the shift of z = x - c per row
    tol = 1e-5 * np.maximum(1.0, np.abs(ref[fin])) + h["m"] * 1e-5 * np.maximum(1.0, np.abs(c[fin]))
    err = np.abs(lp[fin] - ref[fin])
    assert np.all(err <= tol), (err / tol).max()


@pytest.mark.parametrize("mode,off", ANCHORED, ids=["%s%g" % m for m in ANCHORED])
@pytest.mark.parametrize("dtype,V", [(torch.float32, 70001), (torch.bfloat16, 151936)])
def test_pivot_sampling_variants(hs, oracle_mod, mode, off, dtype, V):
    """Every kernel decomposition draws the same ids: one block per row, rows split over 2, 7
    and 64 blocks (the pivot then comes from the split pre-pass's per-chunk partials),
    screened against exhaustive scoring (bit-identical), and draws spread over blocks. (One
    block holds at most 19456 16-byte vectors: fp32 rows stay below 77824 logits.)"""
    w = W.generic(6, V, dtype, seed=63, scale=0.8, mask_frac=0.05,
                  hlg=_curve(mode, off), K=3)
    d = on_device(w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    x64 = w.logits.double().numpy()
    res = {}
    for name, opts in [("auto", None),
                       ("one-block", hs.SampleOpts(variant=1)),
                       ("split2", hs.SampleOpts(variant=2, nchunk=2)),
                       ("split7", hs.SampleOpts(variant=2, nchunk=7)),
                       ("split64", hs.SampleOpts(variant=2, nchunk=64)),
                       ("one-block-exhaustive", hs.SampleOpts(variant=1, no_screen=1)),
                       ("split7-exhaustive", hs.SampleOpts(variant=2, nchunk=7, no_screen=1)),
                       ("draw-groups", hs.SampleOpts(variant=1, draw_groups=3)),
                       ("split5-draw-groups", hs.SampleOpts(variant=2, nchunk=5, draw_groups=2)),
                       ("split7-exchange", hs.SampleOpts(variant=2, nchunk=7, draw_groups=1,
                                                         split_lse=2)),
                       ("split7-exchange-nowait", hs.SampleOpts(variant=2, nchunk=7,
                                                                draw_groups=1, split_lse=2,
                                                                exchange_wait=-1))]:
        idx, best = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], hlg=w.hlg, k=3,
                                 opts=opts, want_best=True)
        idx = idx.cpu().numpy()
        res[name] = (idx, best.cpu().numpy())
        assert_parity(idx, o, s1, s2, x64, "%s %s %s" % (mode, dtype, name))
    for a, b in [("one-block", "one-block-exhaustive"), ("split7", "split7-exhaustive"),
                 ("split7-exchange", "split7-exchange-nowait")]:
        np.testing.assert_array_equal(res[a][0], res[b][0])
        np.testing.assert_array_equal(res[a][1], res[b][1])


@pytest.mark.parametrize("V", [1, 3, 9, 1000, 65537])
@pytest.mark.parametrize("mode,off", ANCHORED, ids=["%s%g" % m for m in ANCHORED])
def test_pivot_ragged_vocab(hs, oracle_mod, V, mode, off):
    w = W.generic(3, V, torch.bfloat16, seed=V + 5, mask_frac=0.1 if V > 4 else 0.0,
                  hlg=_curve(mode, off), K=3, offset_max=2**33)
    g = gpu_sample(hs, w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    assert_parity(g, o, s1, s2, w.logits.double().numpy(), "V=%d %s" % (V, mode))


@pytest.mark.parametrize("mode,off", ANCHORED, ids=["%s%g" % m for m in ANCHORED])
def test_pivot_special_rows(hs, oracle_mod, mode, off):
    """An anchored pivot needs no mu: a NaN in mu is ignored (it gives -2 only with the pivot
    given); empty rows give -1, bad temperatures -2, greedy rows the argmax of x."""
    V = 777
    rng = np.random.default_rng(37)
    x = rng.normal(0, 1, size=(8, V)).astype(np.float32)
    x[0, :] = -np.inf
    x[1, :] = -np.inf
    x[1, 400] = 2.5
    x[2, [3, 50, 600]] = 9.0
    T = np.array([1.0, 0.7, 0.0, 1.0, -1.0, np.nan, np.inf, 1.2], dtype=np.float32)
    mu = np.full(8, np.nan, dtype=np.float32)
    seed = rng.integers(0, 2**64, size=8, dtype=np.uint64)
    off_ = np.array([0, 2**32 - 1, 5, 5, 0, 0, 0, 9], dtype=np.uint64)
    w = W.Workload("special", torch.from_numpy(x), T, seed, off_, K=3, hlg=_curve(mode, off),
                   mu=mu)
    g = gpu_sample(hs, w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    assert_parity(g, o, s1, s2, x.astype(np.float64), "special rows %s" % mode)
    assert g[0].tolist() == [-1] * 3
    assert g[1].tolist() == [400] * 3
    assert g[2].tolist() == [3] * 3
    assert g[4].tolist() == [-2] * 3 and g[5].tolist() == [-2] * 3 and g[6].tolist() == [-2] * 3
    assert np.all(g[[3, 7]] >= 0)


def test_top_anchor_shift_invariance(hs):
    """With the top anchor, z = x - (x_max - c) does not depend on the row's LSE, so adding a
    constant to a row leaves every draw unchanged (up to the rounding of x + a, exact here:
    the shift is a power of two and the logits are multiples of 2^-10)."""
    rng = np.random.default_rng(71)
    x = (np.round(rng.normal(0, 2, size=(8, 50000)) * 1024) / 1024).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    T = torch.full((8,), 0.9, device="cuda")
    seed = torch.arange(8, device="cuda", dtype=torch.int64) * 977 + 5
    off = torch.zeros(8, device="cuda", dtype=torch.int64)
    h = _curve("top", 1.0)
    a = hs.sample(t, T, seed, off, hlg=h, k=8).cpu().numpy()
    b = hs.sample(t + 64.0, T, seed, off, hlg=h, k=8).cpu().numpy()
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("layout", ["plain", "screened"])
@pytest.mark.parametrize("mode,off", [("top", 2.0), ("entropy", 0.0)])
def test_pivot_headline_shape(hs, oracle_mod, mode, off, layout):
    """256 x 151936 bf16 logits, the headline sampling shape, with an anchored pivot."""
    w = W.config4()
    w.hlg = _curve(mode, off, w.hlg)
    g = gpu_sample(hs, w, layout=layout)
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(g, o, s1, s2, w.logits.double().numpy(),
                        "256x151936 %s %s" % (mode, layout)))


@pytest.mark.parametrize("layout", ["plain", "screened"])
def test_pivot_many_draws_split_rows(hs, oracle_mod, layout):
    """64 x 262144 fp32, 16 draws per row, entropy anchor: rows split over blocks, every row
    against the oracle."""
    w = W.config5(B=64)
    w.hlg = _curve("entropy", 0.0, w.hlg)
    d = on_device(w)
    g = gpu_sample(hs, w, dev=d, layout=layout)
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(g, o, s1, s2, w.logits.double().numpy(), "entropy 16 draws " + layout))


# ---- the mass-median pivot: mu = the log-prob at which the mass from the top first reaches
# one half, so z = x - x_med with x_med the top-p boundary at p = 0.5 and T = 1. The GPU sums
# fp32 terms exp2((x - x_max) log2(e)), each within a few 1e-7 relative, in fp64: its running
# totals lie within ~3e-7 of the total mass of the oracle's. A row whose boundary moves when
# the target moves by 1e-6 of the total (p = 0.5 (1 +- 2e-6)) may therefore take a
# neighbouring logit; its draws are only checked for validity.
def _median_sure(oracle_mod, w, rel=2e-6):
    B = w.B
    x64 = w.logits.double().numpy()
    one = np.ones(B, np.float32)
    lo = oracle_mod.filter_threshold(x64, one, top_p=np.full(B, 0.5 * (1 - rel), np.float32))[0]
    hi = oracle_mod.filter_threshold(x64, one, top_p=np.full(B, 0.5 * (1 + rel), np.float32))[0]
    return np.asarray(lo == hi)


@pytest.mark.parametrize("dtype,V", [(torch.float32, 70001), (torch.bfloat16, 151936),
                                     (torch.float16, 32000)])
def test_median_pivot_sampling_variants(hs, oracle_mod, dtype, V):
    """The median shift is worked out once per row before the sampling kernel, so every
    kernel decomposition gives the same ids and scores bit for bit."""
    w = W.generic(6, V, dtype, seed=65, scale=0.8, mask_frac=0.05, hlg=_curve("median", 0.0),
                  K=3)
    d = on_device(w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    sure = _median_sure(oracle_mod, w)
    # rows left out of the id comparison (their boundary is not decided): at most one
    assert (~sure).sum() <= 1, (~sure).sum()
    x64 = w.logits.double().numpy()
    res = {}
    for name, opts in [("auto", None),
                       ("one-block", hs.SampleOpts(variant=1)),
                       ("split7", hs.SampleOpts(variant=2, nchunk=7)),
                       ("split64", hs.SampleOpts(variant=2, nchunk=64)),
                       ("one-block-exhaustive", hs.SampleOpts(variant=1, no_screen=1)),
                       ("draw-groups", hs.SampleOpts(variant=1, draw_groups=3)),
                       ("split5-draw-groups", hs.SampleOpts(variant=2, nchunk=5, draw_groups=2))]:
        idx, best = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], hlg=w.hlg, k=3,
                                 opts=opts, want_best=True)
        idx = idx.cpu().numpy()
        res[name] = (idx, best.cpu().numpy())
        assert_parity(idx[sure], o[sure], s1[sure], s2[sure], x64[sure],
                      "median %s %s" % (dtype, name))
        assert np.all(idx >= 0) and np.all(np.isfinite(x64[np.arange(6)[:, None], idx]))
    for name in res:
        np.testing.assert_array_equal(res[name][0], res["auto"][0])
        np.testing.assert_array_equal(res[name][1], res["auto"][1])


def test_median_pivot_special_rows(hs, oracle_mod):
    """Tiny and ragged rows, an empty row (-1), a bad temperature (-2), a greedy row, a flat
    row (every token is the median) and a row with one dominant token."""
    V = 777
    w = W.generic(7, V, torch.bfloat16, seed=66, scale=1.5, mask_frac=0.1,
                  hlg=_curve("median", 0.0), K=4, offset_max=2**35)
    x = w.logits.float().numpy().copy()
    x[0, :] = -np.inf
    x[3, :] = 0.75
    x[4, :] = 0.0
    x[4, 11] = 9.0
    w.logits = torch.from_numpy(x).to(torch.bfloat16)
    w.T[1] = -1.0
    w.T[2] = 0.0
    g = gpu_sample(hs, w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    sure = _median_sure(oracle_mod, w)
    assert sure.all()
    x64 = w.logits.double().numpy()
    assert g[0].tolist() == [-1] * 4 and g[1].tolist() == [-2] * 4
    assert g[2].tolist() == [int(np.argmax(x64[2]))] * 4
    assert_parity(g[sure], o[sure], s1[sure], s2[sure], x64[sure], "median special rows")
    for V in (1, 3, 9, 1000):
        wv = W.generic(3, V, torch.float16, seed=V + 70, mask_frac=0.1 if V > 4 else 0.0,
                       hlg=_curve("median", 0.0), K=3)
        gv = gpu_sample(hs, wv)
        ov, t1, t2 = oracle_sample(oracle_mod, wv)
        sv = _median_sure(oracle_mod, wv)
        assert sv.all()
        assert_parity(gv[sv], ov[sv], t1[sv], t2[sv], wv.logits.double().numpy()[sv],
                      "median V=%d" % V)


def test_median_pivot_headline_shape(hs, oracle_mod):
    """Every row of the 256 x 151936 bf16 shape; a row whose median boundary is not decided
    (none at this shape) would be left out of the id comparison, and at most one may be."""
    w = W.config4()
    w.hlg = _curve("median", 0.0, w.hlg)
    g = gpu_sample(hs, w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    sure = _median_sure(oracle_mod, w)
    assert (~sure).sum() <= 1, (~sure).sum()
    x64 = w.logits.double().numpy()
    assert np.all(np.isfinite(x64[np.arange(w.B)[:, None], g]))
    print(assert_parity(g[sure], o[sure], s1[sure], s2[sure], x64[sure], "median 256x151936"),
          "rows left out:", int((~sure).sum()))

"""Sampled token ids of the HIP path against the oracle on the workloads of the pages
(mlxcel issue "Softmax-free GPU sampling", sections Performance validation and Regression
guard; mlx-bun HLG design document), every size in the launch configuration the library
picks. Every row of every workload is compared with the oracle, the 1024 x 262144 x 16-draw
workload included (its oracle run takes tens of seconds on all host cores)."""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import (LAYOUTS, assert_parity, gpu_sample, on_device, oracle_sample,
                            require_gpu)
from tests.test_oracle_sampling import _chi2_pvalue

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _x64(w, rows=None):
    x = w.logits if rows is None else w.logits[rows]
    return x.double().numpy()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config1_32k_fp32_1000_draws(hs, oracle_mod, layout):
    w = W.config1()
    g = gpu_sample(hs, w, layout=layout)
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(g, o, s1, s2, _x64(w), "config1 %s" % layout))


def test_config1_single_draw_launches_match(hs):
    """Draw k of the 1000-draw call equals a one-draw call at offset k."""
    w = W.config1()
    d = on_device(w)
    allk = gpu_sample(hs, w, dev=d)
    for k in (0, 1, 2, 17, 500, 999):
        one = hs.sample(d["logits"], d["T"], d["seed"], d["offset"] + k, k=1)
        assert int(one.item()) == int(allk[0, k])


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("T", [0.5, 1.0, 1.5])
def test_chi_square_v16(hs, oracle_mod, T, layout):
    """1e6 draws of linspace(-4, 4) on the GPU: chi-square against exact softmax (cells with
    expected count < 5 pooled, reject at p < 1e-3) and index-exact against the oracle."""
    x = W.chi_square_rows()
    K = 1_000_000
    seed = np.array([0xC0FFEE + int(10 * T)], dtype=np.uint64)
    xt = torch.tensor(x, dtype=torch.float32)[None, :]
    g = hs.sample_ex(xt.cuda(), torch.tensor([T]).cuda(), seed, np.zeros(1, np.uint64), k=K,
                     opts=hs.SampleOpts(layout=hs.LAYOUTS[layout]))
    g = g.cpu().numpy()
    counts = np.bincount(g.ravel(), minlength=16)
    p = np.exp(x / T - (x / T).max())
    p /= p.sum()
    pval = _chi2_pvalue(counts, p, K)
    assert pval > 1e-3, pval
    o, s1, s2 = oracle_mod.sample(xt, [T], seed, [0], K=K, layout=layout)
    print(assert_parity(g, o, s1, s2, xt.double().numpy(), "chi2 T=%g %s" % (T, layout)))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("B", [1, 4, 8])
@pytest.mark.parametrize("T", [0.5, 1.5])
def test_config2_peaked_bf16(hs, oracle_mod, B, T, layout):
    w = W.config2(B=B, T=T)
    g = gpu_sample(hs, w, layout=layout)
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(g, o, s1, s2, _x64(w), "config2 B=%d T=%g %s" % (B, T, layout)))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config3_bimodal_fp32_hlg(hs, oracle_mod, layout):
    w = W.config3()
    g = gpu_sample(hs, w, layout=layout)
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(g, o, s1, s2, _x64(w), "config3 %s" % layout))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config4_headline_bf16_hlg(hs, oracle_mod, layout):
    w = W.config4()
    g = gpu_sample(hs, w, layout=layout)
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(g, o, s1, s2, _x64(w), "config4 %s" % layout))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config5_262k_fp32_hlg_16_draws(hs, oracle_mod, layout):
    """All 1024 rows x 16 draws against the oracle."""
    w = W.config5()
    d = on_device(w)
    g = gpu_sample(hs, w, dev=d, layout=layout)
    del d
    torch.cuda.empty_cache()
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(g, o, s1, s2, _x64(w), "config5 all rows %s" % layout))

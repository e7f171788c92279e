"""Combinations of the features on the HIP path against the oracle: padded and misaligned
rows (ld > V, rows not 16-byte aligned) with the top-k / top-p filters, per-row curve settings
and the anchored pivots; fp16 logits in every mode; a one-token vocabulary; a batch of 4096
short rows; many draws on split rows with the in-kernel exchange; large temperatures. The
comparison rule is the one of the other parity tests (near-ties exempt)."""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import assert_parity, on_device, oracle_sample, require_gpu

pytestmark = pytest.mark.gpu
A = {"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0}


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _padded(x, pad, dtype):
    """x [B, V] as a view of a [B, V + pad] tensor: row stride V + pad (odd pads misalign)."""
    B, V = x.shape
    big = torch.full((B, V + pad), float("-inf"), dtype=dtype)
    big[:, :V] = x
    return big.cuda()[:, :V]


@pytest.mark.parametrize("dtype,pad", [(torch.bfloat16, 3), (torch.float32, 1),
                                       (torch.float16, 8), (torch.bfloat16, 0)])
def test_filters_on_strided_rows(hs, oracle_mod, dtype, pad):
    w = W.generic(5, 20011, dtype, seed=pad + 3, scale=1.2, mask_frac=0.05, K=3)
    x = _padded(w.logits, pad, dtype)
    d = on_device(w)
    k = np.array([0, 7, 100, 1, 20011], dtype=np.int32)
    p = np.array([0.8, 1.0, 0.95, 0.5, 0.3], dtype=np.float32)
    g = hs.sample_filtered(x, d["T"], d["seed"], d["offset"], top_k=torch.from_numpy(k).cuda(),
                           top_p=torch.from_numpy(p).cuda(), k=3).cpu().numpy()
    o, s1, s2, tau, amb = oracle_mod.sample_filtered(w.logits, w.T, w.seed, w.offset, K=3,
                                                     top_k=k, top_p=p)
    sure = ~amb
    assert_parity(g[sure], o[sure], s1[sure], s2[sure], w.logits.double().numpy()[sure],
                  "filters %s pad %d" % (dtype, pad))


@pytest.mark.parametrize("dtype,pad", [(torch.bfloat16, 5), (torch.float32, 2), (torch.float16, 0)])
def test_rows_and_pivots_on_strided_rows(hs, oracle_mod, dtype, pad):
    B, V, K = 8, 30001, 2
    w = W.generic(B, V, dtype, seed=pad + 11, scale=1.0, mask_frac=0.05, hlg=dict(A), K=K)
    x = _padded(w.logits, pad, dtype)
    d = on_device(w)
    settings = [None, dict(A), dict(A, pivot="top", pivot_offset=3.0), dict(A, pivot="entropy")] * 2
    g = hs.sample_rows(x, d["T"], d["seed"], d["offset"], hs.hlg_rows(settings), mu=d["mu"],
                       k=K).cpu().numpy()
    for r in range(B):
        h = settings[r]
        mu = w.mu[r:r + 1] if h is not None and "pivot" not in h else None
        o, s1, s2 = oracle_mod.sample(w.logits[r:r + 1], w.T[r:r + 1], w.seed[r:r + 1],
                                      w.offset[r:r + 1], K=K, mu=mu, hlg=h,
                                      row_id=np.array([r], dtype=np.int64))
        assert_parity(g[r:r + 1], o, s1, s2, w.logits[r:r + 1].double().numpy(),
                      "rows %s pad %d row %d" % (dtype, pad, r))
    for mode in ("top", "entropy"):
        h = dict(A, pivot=mode, pivot_offset=1.0)
        gp = hs.sample(x, d["T"], d["seed"], d["offset"], hlg=h, k=K).cpu().numpy()
        o, s1, s2 = oracle_mod.sample(w.logits, w.T, w.seed, w.offset, K=K, hlg=h)
        assert_parity(gp, o, s1, s2, w.logits.double().numpy(), "%s %s pad %d" % (mode, dtype, pad))


def test_one_token_vocabulary(hs):
    x = torch.tensor([[0.5], [-np.inf], [3.0]], dtype=torch.float32).cuda()
    T = torch.tensor([1.0, 1.0, 0.0]).cuda()
    seed = torch.tensor([1, 2, 3], dtype=torch.int64).cuda()
    off = torch.zeros(3, dtype=torch.int64).cuda()
    assert hs.sample(x, T, seed, off, k=4).cpu().tolist() == [[0] * 4, [-1] * 4, [0] * 4]
    assert hs.sample(x, T, seed, off, hlg=dict(A, pivot="entropy"), k=2).cpu().tolist() == \
        [[0] * 2, [-1] * 2, [0] * 2]
    assert hs.sample_filtered(x, T, seed, off, top_k=1, top_p=0.5, k=2).cpu().tolist() == \
        [[0] * 2, [-1] * 2, [0] * 2]


def test_large_batch_short_rows(hs, oracle_mod):
    w = W.generic(4096, 300, torch.bfloat16, seed=5, scale=1.5, mask_frac=0.1, hlg=dict(A), K=2)
    g = hs.sample(w.logits.cuda(), torch.from_numpy(w.T).cuda(), w.seed, w.offset,
                  mu=torch.from_numpy(w.mu).cuda(), hlg=w.hlg, k=2).cpu().numpy()
    rows = np.sort(np.random.default_rng(3).choice(4096, size=256, replace=False))
    o, s1, s2 = oracle_sample(oracle_mod, w, rows=rows)
    assert_parity(g[rows], o, s1, s2, w.logits[rows].double().numpy(), "4096 x 300")


def test_many_draws_on_split_rows_with_exchange(hs, oracle_mod):
    """Two 151936-logit fp32 rows (split: two chunks at least), 300 draws each, one draw group
    per row, partials exchanged in the kernel: draws are flushed in batches of 64."""
    w = W.generic(2, 151936, torch.float32, seed=9, scale=1.0, mask_frac=0.05, hlg=dict(A),
                  K=300)
    d = on_device(w)
    for opts in (hs.SampleOpts(variant=2, nchunk=8, draw_groups=1, split_lse=2),
                 hs.SampleOpts(variant=2, nchunk=8, draw_groups=1, split_lse=1)):
        g = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], mu=d["mu"], hlg=w.hlg,
                         k=300, opts=opts).cpu().numpy()
        o, s1, s2 = oracle_sample(oracle_mod, w)
        assert_parity(g, o, s1, s2, w.logits.double().numpy(), "300 draws split")


@pytest.mark.parametrize("T", [50.0, 1e4])
def test_large_temperatures(hs, oracle_mod, T):
    """Nearly uniform draws: the screen's bounds stay valid when l'/T is tiny next to G."""
    w = W.generic(4, 50000, torch.bfloat16, seed=13, scale=2.0, hlg=dict(A), K=4)
    w.T[:] = T
    d = on_device(w)
    for hlg in (None, w.hlg):
        g = hs.sample(d["logits"], d["T"], d["seed"], d["offset"], mu=d["mu"] if hlg else None,
                      hlg=hlg, k=4).cpu().numpy()
        o, s1, s2 = oracle_mod.sample(w.logits, w.T, w.seed, w.offset, K=4,
                                      mu=w.mu if hlg else None, hlg=hlg)
        assert_parity(g, o, s1, s2, w.logits.double().numpy(), "T=%g hlg=%s" % (T, bool(hlg)))

"""A seeded sweep of random configurations on the HIP path against the oracle: dtype, batch,
vocabulary (from one token to rows that must be split), draws, curve and pivot mode (given,
top, entropy, median), word layout, masking, padded rows, large counter offsets, greedy and
invalid rows, the top-k / top-p filters, and now and then one block per row (long chunks) or
one draw group per row (a block's later draws). Each case is small enough for the oracle; the
comparison rule is the other parity tests'. HS_SWEEP_SEED and HS_SWEEP_CASES select a longer
or different sweep (defaults: the seed below, 48 cases)."""
import os

import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import assert_parity, require_gpu
from tests.test_gpu_filter import _check_rows
from tests.test_gpu_pivot import _median_sure

pytestmark = pytest.mark.gpu

CURVE = {"m": 1.25, "w": 1.5, "beta_t": 0.5, "beta_h": 1.0}
DTYPES = (torch.float32, torch.bfloat16, torch.float16)
VOCABS = (1, 3, 64, 1000, 4099, 30011, 100003)


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _case(rng, i):
    dtype = DTYPES[int(rng.integers(len(DTYPES)))]
    V = int(VOCABS[int(rng.integers(len(VOCABS)))])
    B = int(rng.integers(1, 7))
    K = int((1, 2, 7)[int(rng.integers(3))])
    mode = ("off", "given", "top", "entropy", "median", "filter")[int(rng.integers(6))]
    hlg = dict(CURVE) if mode in ("given", "top", "entropy", "median") else None
    if mode in ("top", "entropy", "median"):
        hlg["pivot"] = mode
        if mode == "top":
            hlg["pivot_offset"] = float(rng.uniform(0.0, 6.0))
    w = W.generic(B, V, dtype, seed=1000 + i, scale=float(rng.choice([0.5, 2.0])),
                  mask_frac=float(rng.choice([0.0, 0.1, 0.5])) if V > 3 else 0.0,
                  hlg=dict(CURVE) if mode == "given" else None, K=K,
                  offset_max=int(rng.choice([0, 2**40])))
    w.hlg = hlg
    if B > 2 and rng.random() < 0.5:
        w.T[0] = 0.0                      # a greedy row
    if B > 3 and rng.random() < 0.3:
        w.T[1] = -1.0                     # an invalid temperature
    pad = int(rng.choice([0, 0, 1, 8]))
    return w, mode, pad


def _device_rows(w, pad):
    """The logits on the GPU, as a view of a [B, V + pad] tensor when pad > 0."""
    if pad == 0:
        return w.logits.cuda()
    B, V = w.logits.shape
    big = torch.full((B, V + pad), float("-inf"), dtype=w.logits.dtype)
    big[:, :V] = w.logits
    return big.cuda()[:, :V]


def test_random_configurations(hs, oracle_mod):
    rng = np.random.default_rng(int(os.environ.get("HS_SWEEP_SEED", "20261202")))
    for i in range(int(os.environ.get("HS_SWEEP_CASES", "48"))):
        w, mode, pad = _case(rng, i)
        layout = ("plain", "screened")[int(rng.integers(2))]
        variant = int(rng.choice([0, 0, 1]))   # 1: one block per row where it fits
        epv = 4 if w.logits.dtype == torch.float32 else 8
        if (w.V + epv - 1) // epv > 19 * 1024:   # more vectors than one block holds
            variant = 0
        groups = int(rng.choice([0, 0, 1]))    # 1: one draw group per row
        label = "case %d: %s B=%d V=%d K=%d %s pad %d %s variant %d groups %d" % (
            i, w.logits.dtype, w.B, w.V, w.K, mode, pad, layout, variant, groups)
        print(label, flush=True)
        if mode == "filter":
            k = rng.choice([0, 1, 5, 50, w.V + 1], size=w.B).astype(np.int32)
            p = rng.choice([1.0, 0.3, 0.9, 0.999], size=w.B).astype(np.float32)
            _check_rows(hs, oracle_mod, w, k, p, label)
            continue
        x = _device_rows(w, pad)
        T = torch.from_numpy(np.ascontiguousarray(w.T)).cuda()
        seed = torch.from_numpy(np.ascontiguousarray(w.seed).view(np.int64)).cuda()
        off = torch.from_numpy(np.ascontiguousarray(w.offset).view(np.int64)).cuda()
        mu = torch.from_numpy(w.mu).cuda() if mode == "given" else None
        opts = hs.SampleOpts(layout=hs.LAYOUTS[layout], variant=variant, draw_groups=groups)
        g = hs.sample_ex(x, T, seed, off, mu=mu, hlg=w.hlg, k=w.K, opts=opts).cpu().numpy()
        o, s1, s2 = oracle_mod.sample(w.logits, w.T, w.seed, w.offset, K=w.K,
                                      mu=w.mu if mode == "given" else None, hlg=w.hlg,
                                      layout=layout)
        x64 = w.logits.double().numpy()
        # the median: rows whose mass boundary is decided away from one half
        sure = _median_sure(oracle_mod, w) if mode == "median" else np.ones(w.B, dtype=bool)
        assert_parity(g[sure], o[sure], s1[sure], s2[sure], x64[sure], label)
        ok = g >= 0
        assert np.all(np.isfinite(x64[np.nonzero(ok)[0], g[ok]]))

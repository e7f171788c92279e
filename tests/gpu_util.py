"""Helpers shared by the GPU parity tests: device placement of a synthetic workload, the
oracle run on the same inputs, and the comparison rule.

Comparison rule for sampled token ids (both sides draw from the same Philox words):
  - every index must equal the oracle's, except draws whose oracle best and second-best
    scores differ by less than 1e-6 of the larger magnitude (near-ties); such exempt draws
    are counted and may be at most 0.01% of the draws compared;
  - no index may point at a -inf logit;
  - -1 (no finite logit) and -2 (invalid temperature / pivot) must match exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

NEAR_TIE_REL = 1e-6
MAX_EXEMPT_FRAC = 1e-4


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import logit_transform_amd as hs
    hs.load()   # no fallback: with a GPU present, a missing library is a failure
    return hs


def on_device(w):
    d = torch.device("cuda")
    out = dict(logits=w.logits.to(d), T=torch.from_numpy(np.ascontiguousarray(w.T)).to(d),
               seed=torch.from_numpy(np.ascontiguousarray(w.seed).view(np.int64)).to(d),
               offset=torch.from_numpy(np.ascontiguousarray(w.offset).view(np.int64)).to(d))
    if w.hlg is not None:
        out["mu"] = torch.from_numpy(np.ascontiguousarray(w.mu)).to(d)
    return out


LAYOUTS = ("plain", "screened")


def gpu_sample(hs, w, dev=None, layout="plain", **kw) -> np.ndarray:
    """hs_sample (plain word layout) or hs_sample_ex with the given word layout."""
    dev = dev or on_device(w)
    if layout == "plain" and "opts" not in kw:
        out = hs.sample(dev["logits"], dev["T"], dev["seed"], dev["offset"], mu=dev.get("mu"),
                        hlg=w.hlg, k=w.K, **kw)
    else:
        opts = kw.pop("opts", None) or hs.SampleOpts()
        opts.layout = hs.LAYOUTS[layout]
        out = hs.sample_ex(dev["logits"], dev["T"], dev["seed"], dev["offset"],
                           mu=dev.get("mu"), hlg=w.hlg, k=w.K, opts=opts, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_sample(O, w, rows=None, layout="plain"):
    x = w.logits if rows is None else w.logits[rows]
    rsel = np.arange(w.B) if rows is None else np.asarray(rows)
    mu = None if w.hlg is None else w.mu[rsel]
    return O.sample(x, w.T[rsel], w.seed[rsel], w.offset[rsel], K=w.K, mu=mu, hlg=w.hlg,
                    row_id=rsel.astype(np.int64), layout=layout)


def assert_parity(gpu_idx, or_idx, s1, s2, x64, label: str, max_exempt_frac=MAX_EXEMPT_FRAC):
    """gpu_idx, or_idx, s1, s2: [n, K]; x64: the n rows' logits as float64 [n, V]."""
    gpu_idx = np.asarray(gpu_idx)
    or_idx = np.asarray(or_idx)
    assert gpu_idx.shape == or_idx.shape, (gpu_idx.shape, or_idx.shape)
    n, K = gpu_idx.shape
    # indices that point at a token must point at a finite logit
    valid = gpu_idx >= 0
    rows = np.repeat(np.arange(n)[:, None], K, axis=1)
    picked = x64[rows[valid], gpu_idx[valid]]
    assert np.all(np.isfinite(picked)), "%s: a masked token was sampled" % label
    assert np.all(gpu_idx < x64.shape[1])
    # special codes must agree exactly
    special = (or_idx < 0) | (gpu_idx < 0)
    assert np.array_equal(gpu_idx[special], or_idx[special]), "%s: -1/-2 codes differ" % label
    mism = gpu_idx != or_idx
    with np.errstate(invalid="ignore"):
        scale = np.maximum(np.abs(s1), np.abs(s2))
        near = np.isfinite(s1) & np.isfinite(s2) & (np.abs(s1 - s2) < NEAR_TIE_REL * scale)
    exempt = mism & near
    bad = mism & ~near
    if bad.any():
        r, k = np.argwhere(bad)[0]
        raise AssertionError(
            "%s: %d non-exempt mismatches of %d draws; first at row %d draw %d: gpu %d oracle %d "
            "(oracle best %.9g second %.9g, gap %.3g)" % (label, bad.sum(), n * K, r, k,
                                                          gpu_idx[r, k], or_idx[r, k], s1[r, k],
                                                          s2[r, k], s1[r, k] - s2[r, k]))
    allowed = int(np.floor(max_exempt_frac * n * K))
    assert exempt.sum() <= allowed, "%s: %d near-tie mismatches > %d allowed" % (
        label, exempt.sum(), allowed)
    return dict(draws=n * K, exempt=int(exempt.sum()), near_ties=int(near.sum()))

"""The allocation-free entry point (hs_sample_noalloc) against hs_sample_ex: the same kernels,
the workspace taken from the library's static device array instead of the caller's. Two calls
in a row through the C ABI, the second with a smaller input (the array keeps the first call's
contents); and a pair whose second call keeps its keys where the first call's split pre-pass
left its partials (the array is zero-filled again when the shape changes)."""
import ctypes as C

import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import assert_parity, on_device, oracle_sample, require_gpu

pytestmark = pytest.mark.gpu
HLG_A = {"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0}


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _both(hs, w, opts_kw):
    d = on_device(w)
    ref, rb = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], mu=d.get("mu"),
                           hlg=w.hlg, k=w.K, opts=hs.SampleOpts(**opts_kw), want_best=True)
    L = hs.load()
    x = hs._logits_struct(d["logits"])
    out = torch.full((w.B, w.K), -7, dtype=torch.int32, device="cuda")
    best = torch.empty((w.B, w.K), dtype=torch.float32, device="cuda")
    hp = hs._hlg_struct(w.hlg)
    opts = hs.SampleOpts(**opts_kw)
    rc = L.hs_sample_noalloc(C.byref(x), d["T"].data_ptr(),
                             d["mu"].data_ptr() if "mu" in d else None,
                             C.byref(hp) if hp is not None else None, d["seed"].data_ptr(),
                             d["offset"].data_ptr(), w.K, out.data_ptr(), best.data_ptr(),
                             C.byref(opts), hs._stream(torch.device("cuda")))
    assert rc == 0, hs.load().hs_status_str(rc)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), rb.cpu().numpy(), out.cpu().numpy(), best.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    # split rows with the curve on (the in-kernel exchange), then a smaller split shape
    (dict(B=8, V=151936, dtype=torch.float32, hlg=HLG_A, K=3, layout=1, seed=5),
     dict(B=3, V=40000, dtype=torch.bfloat16, hlg=None, K=2, layout=0, seed=6)),
    # many draws spread over blocks with the pre-pass, then one small row
    (dict(B=4, V=100000, dtype=torch.bfloat16, hlg=HLG_A, K=16, layout=0, seed=7),
     dict(B=1, V=5000, dtype=torch.float32, hlg=HLG_A, K=3, layout=1, seed=8)),
    # one row, 16 chunks and 4 draw groups with the pre-pass (its partials at [512, 768) of
    # the array), then 16 split rows without the curve, whose keys lie at [256, 768)
    (dict(B=1, V=100000, dtype=torch.bfloat16, hlg=HLG_A, K=4, layout=1, seed=11),
     dict(B=16, V=65536, dtype=torch.bfloat16, hlg=None, K=3, layout=0, seed=12)),
])
def test_noalloc_matches_sample_ex(hs, oracle_mod, first, second):
    for case in (first, second):
        w = W.generic(case["B"], case["V"], case["dtype"], seed=case["seed"], hlg=case["hlg"],
                      K=case["K"], mask_frac=0.05)
        kw = dict(layout=case["layout"])
        ref, rb, got, gb = _both(hs, w, kw)
        np.testing.assert_array_equal(got, ref)
        np.testing.assert_array_equal(gb, rb)
        o, s1, s2 = oracle_sample(oracle_mod, w, layout=("plain", "screened")[case["layout"]])
        print(assert_parity(got, o, s1, s2, w.logits.double().numpy(), "noalloc %s" % case))

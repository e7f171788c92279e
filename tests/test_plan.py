"""The host-side launch planner (hs_sample_plan), without a GPU (256 CUs assumed): the plans
chosen for the pages' workloads, and the invariants every plan keeps (chunks cover the row and
none is empty, each block holds its chunk, draw groups cover the K draws, split rows only with
a workspace, explicit choices honoured)."""
import itertools

import pytest
import torch

hs = pytest.importorskip("logit_transform_amd")

HS_ERR_WORKSPACE, HS_ERR_UNSUPPORTED = -3, -5
NV_BUCKETS = (1, 2, 4, 6, 8, 12, 16, 19)


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(hs.library_path()):
        pytest.skip("libhs.so not built")
    return hs.load()


def _epv(dtype):
    return 4 if dtype == torch.float32 else 8


def _check_invariants(p, B, V, K, dtype):
    nvec = -(-V // _epv(dtype))
    assert 1 <= p["nchunk"] <= 64
    assert p["cv"] * p["nchunk"] >= nvec and (p["nchunk"] - 1) * p["cv"] < nvec
    assert p["bs"] in (256, 512, 1024) and p["nv"] in NV_BUCKETS
    assert p["nv"] * p["bs"] >= p["cv"]
    g, kpg = p["draw_groups"], p["draws_per_group"]
    assert g * kpg >= K and (g - 1) * kpg < K
    assert p["grid"] == B * p["nchunk"] * g


def test_plans_of_the_workloads():
    f32, bf16 = torch.float32, torch.bfloat16
    # one 32768-logit row, 1000 draws: the draws spread over ~one block per CU, no split
    p = hs.sample_plan(1, 32768, 1000, f32, False)
    assert (p["nchunk"], p["draw_groups"], p["draws_per_group"]) == (1, 250, 4)
    # 8 x 65536 bf16, curve off: split so that the batch fills about half the CUs
    assert hs.sample_plan(8, 65536, 1, bf16, False)["nchunk"] == 16
    # 8 x 151936 fp32 with the curve: at most 16 chunks (their partials are exchanged)
    p = hs.sample_plan(8, 151936, 1, f32, True)
    assert p["nchunk"] == 16 and p["grid"] == 128
    # ... which 16 rows fill one block per CU
    p = hs.sample_plan(16, 151936, 1, f32, True)
    assert p["nchunk"] == 16 and p["grid"] == 256
    # the 256 x 151936 bf16 headline: one block of 1024 threads per row, 19 slots each
    p = hs.sample_plan(256, 151936, 1, bf16, True)
    assert (p["nchunk"], p["bs"], p["nv"], p["grid"]) == (1, 1024, 19, 256)
    # 1024 x 262144 fp32: rows longer than one block holds are split (4 chunks)
    p = hs.sample_plan(1024, 262144, 16, f32, True)
    assert (p["nchunk"], p["draw_groups"]) == (4, 1)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_invariants_over_shapes(dtype):
    for B, V, K, hlg in itertools.product((1, 3, 8, 64, 256, 1024), (1, 7, 1000, 32768, 151936,
                                                                      262144),
                                          (1, 4, 1000), (False, True)):
        if B * K >= 2**31:
            continue
        p = hs.sample_plan(B, V, K, dtype, hlg)
        _check_invariants(p, B, V, K, dtype)
        # without a workspace rows are never split; rows too long for one block are refused
        fits = -(-V // _epv(dtype)) <= 19 * 1024
        if fits:
            q = hs.sample_plan(B, V, K, dtype, hlg, have_ws=False)
            assert q["nchunk"] == 1
            _check_invariants(q, B, V, K, dtype)
        else:
            with pytest.raises(hs.HsError) as e:
                hs.sample_plan(B, V, K, dtype, hlg, have_ws=False)
            assert e.value.status == HS_ERR_WORKSPACE


def test_explicit_choices():
    f32 = torch.float32
    p = hs.sample_plan(2, 100000, 3, f32, True, opts=hs.SampleOpts(variant=2, nchunk=7,
                                                                   draw_groups=3))
    assert (p["nchunk"], p["draw_groups"], p["draws_per_group"]) == (7, 3, 1)
    p = hs.sample_plan(2, 50000, 3, f32, True, opts=hs.SampleOpts(variant=1))
    assert p["nchunk"] == 1
    with pytest.raises(hs.HsError) as e:      # one block cannot hold 100000 fp32 logits
        hs.sample_plan(2, 100000, 3, f32, True, opts=hs.SampleOpts(variant=1))
    assert e.value.status == HS_ERR_UNSUPPORTED
    # variant 2 without an explicit count still splits
    assert hs.sample_plan(256, 32768, 1, f32, False, opts=hs.SampleOpts(variant=2))["nchunk"] >= 2

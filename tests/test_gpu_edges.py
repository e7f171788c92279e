"""Edge cases, kernel-variant invariance and determinism of the HIP path, against the oracle.

Edge cases: tiny and ragged vocabularies, rows with no finite logit (-1), invalid
temperatures and pivots (-2), greedy rows with ties (T = 0, curve on or off), rolloff off
(w = inf), fp16 input, rows that are not 16-byte aligned, offsets that carry across 2^32 and
wrap at 2^64, and rows split over many blocks.

Invariance: the index of every draw is a function of (seed, row, element, offset) only, so
one-block-per-row, split rows, screened and exhaustive scoring, and any spreading of draws
over blocks must agree (mlxcel issue "Softmax-free GPU sampling", section Background:
stateless and reproducible; section Regression guard: determinism)."""
import math

import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import (LAYOUTS, assert_parity, gpu_sample, on_device, oracle_sample,
                            require_gpu)

pytestmark = pytest.mark.gpu
HLG_A = {"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0}


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _check(hs, O, w, label, layout="plain", **kw):
    g = gpu_sample(hs, w, layout=layout, **kw)
    o, s1, s2 = oracle_sample(O, w, layout=layout)
    return assert_parity(g, o, s1, s2, w.logits.double().numpy(), label + " " + layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("V", [1, 2, 3, 5, 8, 9, 31, 33, 1000, 4097, 65537])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("hlg", [None, HLG_A])
def test_ragged_vocab(hs, oracle_mod, V, dtype, hlg, layout):
    w = W.generic(3, V, dtype, seed=V, mask_frac=0.1 if V > 4 else 0.0, hlg=hlg, K=3,
                  offset_max=2**33)
    _check(hs, oracle_mod, w, "V=%d %s hlg=%s" % (V, dtype, hlg is not None), layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fp16_and_misaligned_rows(hs, oracle_mod, layout):
    w = W.generic(6, 3001, torch.float16, seed=21, mask_frac=0.25, hlg=HLG_A, K=2)
    _check(hs, oracle_mod, w, "f16", layout=layout)
    big = torch.full((6, 3004), float("-inf"), dtype=torch.float16)
    big[:, :3001] = w.logits
    d = on_device(w)
    x = big.cuda()[:, :3001]
    g = hs.sample_ex(x, d["T"], d["seed"], d["offset"], mu=d["mu"], hlg=w.hlg, k=2,
                     opts=hs.SampleOpts(layout=hs.LAYOUTS[layout])).cpu().numpy()
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    assert_parity(g, o, s1, s2, w.logits.double().numpy(), "f16 misaligned " + layout)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_special_rows(hs, oracle_mod, layout):
    V = 777
    rng = np.random.default_rng(31)
    x = rng.normal(0, 1, size=(8, V)).astype(np.float32)
    x[0, :] = -np.inf                                  # no finite logit -> -1
    x[1, :] = -np.inf
    x[1, 400] = 2.5                                    # a single finite logit
    x[2, [3, 50, 600]] = 9.0                           # greedy with a three-way tie
    x[3, [10, 11]] = 4.0
    T = np.array([1.0, 0.7, 0.0, 0.0, -1.0, np.nan, np.inf, 1.2], dtype=np.float32)
    mu = np.array([-5, -5, -5, -5, -5, -5, -5, np.nan], dtype=np.float32)
    seed = rng.integers(0, 2**64, size=8, dtype=np.uint64)
    off = np.array([0, 2**32 - 1, 5, 5, 0, 0, 0, 0], dtype=np.uint64)
    for hlg in (None, HLG_A):
        w = W.Workload("special", torch.from_numpy(x), T, seed, off, K=3, hlg=hlg,
                       mu=mu if hlg else None)
        g = gpu_sample(hs, w, layout=layout)
        o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
        assert_parity(g, o, s1, s2, x.astype(np.float64), "special rows hlg=%s %s"
                      % (bool(hlg), layout))
        assert g[0].tolist() == [-1] * 3
        assert g[1].tolist() == [400] * 3
        assert g[2].tolist() == [3] * 3 and g[3].tolist() == [10] * 3
        assert g[4].tolist() == [-2] * 3 and g[5].tolist() == [-2] * 3 and g[6].tolist() == [-2] * 3
        if hlg:
            assert g[7].tolist() == [-2] * 3


@pytest.mark.parametrize("groups", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype,V", [(torch.float32, 32768), (torch.bfloat16, 151936),
                                     (torch.bfloat16, 151937)])
def test_special_rows_one_block_per_row(hs, oracle_mod, layout, dtype, V, groups):
    """The special rows again with one block per row over long rows (8 and 19 vectors per
    thread: the first draw's bootstrap candidates are then drawn and scored by one wave for
    the whole block), plus rows whose few finite logits leave most lanes without a valid
    champion; V = 151937 also gives rows that are not 16-byte aligned and a ragged tail. With
    one draw group per row a block's later draws follow its first."""
    rng = np.random.default_rng(37)
    B = 11
    x = rng.normal(0, 1, size=(B, V)).astype(np.float32)
    x[0, :] = -np.inf                                  # no finite logit -> -1
    x[1, :] = -np.inf
    x[1, V // 3] = 2.5                                 # a single finite logit
    x[2, [3, V // 2, V - 1]] = 9.0                     # greedy with a three-way tie
    x[3] = np.minimum(x[3], 3.5)                       # (long rows reach 4 by chance)
    x[3, [10, 11]] = 4.0
    for r in (8, 9):                                   # about 1% finite, scattered
        keep = rng.random(V) < 0.01
        x[r, ~keep] = -np.inf
    x[10, : V - 100] = -np.inf                         # finite logits only in the tail
    x = torch.from_numpy(x).to(dtype).float().numpy()  # values on the input grid
    T = np.array([1.0, 0.7, 0.0, 0.0, -1.0, np.nan, np.inf, 1.2, 0.8, 1.3, 1.0],
                 dtype=np.float32)
    mu = np.full(B, -5.0, dtype=np.float32)
    mu[7] = np.nan
    seed = rng.integers(0, 2**64, size=B, dtype=np.uint64)
    off = rng.integers(0, 2**40, size=B, dtype=np.uint64)
    for hlg in (None, HLG_A):
        opts = hs.SampleOpts(variant=1, draw_groups=groups)
        w = W.Workload("special long", torch.from_numpy(x).to(dtype), T, seed, off, K=3,
                       hlg=hlg, mu=mu if hlg else None)
        plan = hs.sample_plan(B, V, 3, dtype, hlg is not None, True, opts)
        assert plan["nchunk"] == 1 and plan["nv"] >= 8, plan
        assert groups == 0 or plan["draws_per_group"] == 3, plan
        g = gpu_sample(hs, w, layout=layout, opts=opts)
        o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
        assert_parity(g, o, s1, s2, x.astype(np.float64), "special long rows %s V=%d hlg=%s %s"
                      % (dtype, V, bool(hlg), layout))
        assert g[0].tolist() == [-1] * 3
        assert g[1].tolist() == [V // 3] * 3
        assert g[2].tolist() == [3] * 3 and g[3].tolist() == [10] * 3
        assert g[4].tolist() == [-2] * 3 and g[5].tolist() == [-2] * 3 and g[6].tolist() == [-2] * 3
        if hlg:
            assert g[7].tolist() == [-2] * 3
        assert (g[10] >= V - 100).all()


@pytest.mark.parametrize("hlg", [None, HLG_A])
def test_subnormal_temperature_is_invalid(hs, oracle_mod, hlg):
    """A subnormal temperature (1/T overflows fp32) is invalid (-2) on the GPU and in the oracle,
    also on rows holding an exact 0 logit (0 * inf would be NaN); the smallest normal T is a
    valid, near-greedy temperature."""
    V = 500
    # |l'| / FLT_MIN stays inside the fp32 range: |x| < 1.9, no ties at the top
    x = (1.9 * np.tanh(np.random.default_rng(33).normal(0, 1, size=(4, V)))).astype(np.float32)
    x[:, 7] = 0.0
    T = np.array([1e-39, 1e-45, np.float32(2.0 ** -126), 1.0], dtype=np.float32)
    rng = np.random.default_rng(34)
    seed = rng.integers(0, 2**64, size=4, dtype=np.uint64)
    off = np.zeros(4, dtype=np.uint64)
    mu = np.full(4, -6.0, dtype=np.float32) if hlg else None
    w = W.Workload("tiny T", torch.from_numpy(x), T, seed, off, K=2, hlg=hlg, mu=mu)
    g = gpu_sample(hs, w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    assert g[0].tolist() == [-2, -2] and g[1].tolist() == [-2, -2]
    assert o[0].tolist() == [-2, -2] and o[1].tolist() == [-2, -2]
    assert_parity(g, o, s1, s2, x.astype(np.float64), "tiny T hlg=%s" % bool(hlg))
    assert g[2].tolist() == [int(np.argmax(x[2]))] * 2


def test_rolloff_off_equals_temperature(hs, oracle_mod):
    """Rolloff off (w = inf) with gain m is temperature 1/m (HLG design document, section
    "The degeneracies are the safety anchors"): the same draws as the curve-off path at
    temperature T/m, the log-softmax shift being common to all tokens. Each path is checked
    against the oracle's own run of it; where the two paths' ids differ, both oracle runs must
    call the draw a near-tie."""
    w = W.generic(16, 20000, torch.float32, seed=41, K=4)
    d = on_device(w)
    m = 1.0 / 0.7
    hlg = {"m": m, "w": math.inf, "beta_t": 1.0, "beta_h": 1.0}
    mu = np.zeros(16, dtype=np.float32)
    a = hs.sample(d["logits"], d["T"], d["seed"], d["offset"], mu=torch.from_numpy(mu).cuda(),
                  hlg=hlg, k=4).cpu().numpy()
    Tm = (d["T"] / m)
    b = hs.sample(d["logits"], Tm, d["seed"], d["offset"], k=4).cpu().numpy()
    x64 = w.logits.double().numpy()
    rows = np.arange(16, dtype=np.int64)
    oa, a1, a2 = oracle_mod.sample(w.logits, w.T, w.seed, w.offset, K=4, mu=mu, hlg=hlg,
                                   row_id=rows)
    ob, b1, b2 = oracle_mod.sample(w.logits, Tm.cpu().numpy(), w.seed, w.offset, K=4,
                                   row_id=rows)
    print(assert_parity(a, oa, a1, a2, x64, "rolloff off"))
    print(assert_parity(b, ob, b1, b2, x64, "temperature T/m"))

    def near(s1, s2):
        return np.abs(s1 - s2) < 1e-6 * np.maximum(np.abs(s1), np.abs(s2))
    diff = a != b
    assert np.all(near(a1, a2)[diff] & near(b1, b2)[diff]), np.argwhere(diff)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_offsets_wrap(hs, oracle_mod, layout):
    w = W.generic(4, 5000, torch.float32, seed=51, K=5)
    w.offset = np.array([2**64 - 2, 2**32 - 3, 0, 2**63], dtype=np.uint64)
    _check(hs, oracle_mod, w, "offset wrap", layout=layout)


@pytest.mark.parametrize("layout,dtype,V", [("plain", torch.bfloat16, 151936),
                                            ("screened", torch.bfloat16, 151936),
                                            ("screened", torch.float32, 70001),
                                            ("screened", torch.float16, 33331)])
@pytest.mark.parametrize("hlg", [None, HLG_A])
def test_variant_invariance(hs, oracle_mod, hlg, layout, dtype, V):
    w = W.generic(6, V, dtype, seed=61, scale=0.8, mask_frac=0.05, hlg=hlg, K=3)
    d = on_device(w)
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    x64 = w.logits.double().numpy()
    results = {}
    for name, opts in [("auto", None),
                       ("one-block", hs.SampleOpts(variant=1)),
                       ("split2", hs.SampleOpts(variant=2, nchunk=2)),
                       ("split7", hs.SampleOpts(variant=2, nchunk=7)),
                       ("split64", hs.SampleOpts(variant=2, nchunk=64)),
                       ("one-block-exhaustive", hs.SampleOpts(variant=1, no_screen=1)),
                       ("split7-exhaustive", hs.SampleOpts(variant=2, nchunk=7, no_screen=1)),
                       ("draw-groups", hs.SampleOpts(variant=1, draw_groups=3)),
                       ("split5-draw-groups", hs.SampleOpts(variant=2, nchunk=5, draw_groups=2)),
                       ("split7-prepass", hs.SampleOpts(variant=2, nchunk=7, draw_groups=1,
                                                        split_lse=1)),
                       ("split7-exchange", hs.SampleOpts(variant=2, nchunk=7, draw_groups=1,
                                                         split_lse=2)),
                       ("split7-exchange-nowait", hs.SampleOpts(variant=2, nchunk=7,
                                                                draw_groups=1, split_lse=2,
                                                                exchange_wait=-1)),
                       ("split64-exchange", hs.SampleOpts(variant=2, nchunk=64, draw_groups=1,
                                                          split_lse=2))]:
        opts = opts or hs.SampleOpts()
        opts.layout = hs.LAYOUTS[layout]
        idx, best = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], mu=d.get("mu"),
                                 hlg=hlg, k=3, opts=opts, want_best=True)
        idx = idx.cpu().numpy()
        results[name] = (idx, best.cpu().numpy())
        assert_parity(idx, o, s1, s2, x64, "%s %s" % (name, layout))
    # screening never changes a result: same variant, screened vs exhaustive, bit-identical;
    # nor does which block works out a chunk's log-sum-exp partial in the exchange
    for a, b in [("one-block", "one-block-exhaustive"), ("split7", "split7-exhaustive"),
                 ("split7-exchange", "split7-exchange-nowait")]:
        np.testing.assert_array_equal(results[a][0], results[b][0])
        np.testing.assert_array_equal(results[a][1], results[b][1])
    # without the curve nothing depends on the decomposition at all
    if hlg is None:
        for name in results:
            np.testing.assert_array_equal(results[name][1], results["one-block"][1])


def test_determinism(hs):
    w = W.config4(B=32)
    d = on_device(w)
    a = gpu_sample(hs, w, dev=d)
    for _ in range(3):
        np.testing.assert_array_equal(gpu_sample(hs, w, dev=d), a)


def test_k_draws_equal_single_draws(hs):
    w = W.generic(5, 30000, torch.bfloat16, seed=71, hlg=HLG_A, K=8)
    d = on_device(w)
    allk = gpu_sample(hs, w, dev=d)
    for k in range(8):
        one = hs.sample(d["logits"], d["T"], d["seed"], d["offset"] + k, mu=d["mu"], hlg=HLG_A, k=1)
        np.testing.assert_array_equal(one.cpu().numpy()[:, 0], allk[:, k])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_resident_grid_work_queue(hs, oracle_mod, layout):
    """More (row, chunk) items than resident blocks, one draw group per row: the automatic
    plan runs a resident grid that takes items from a counter and exchanges the chunks'
    partials in the kernel (no pre-pass). Ids agree with the oracle's; two calls in a row on one
    workspace give the same result and leave the counters zero. Ids and scores equal the
    one-block-per-item exchange's bit for bit (every block working the other chunks' partials
    out itself, which gives the owner's values exactly), and the pre-pass route's up to the
    rounding of the row's log-sum-exp."""
    B, V, K = 600, 100000, 2
    w = W.generic(B, V, torch.float32, seed=83, mask_frac=0.05, hlg=HLG_A, K=K)
    plan = hs.sample_plan(B, V, K, torch.float32, True)
    assert plan["nchunk"] > 1 and plan["draw_groups"] == 1 and plan["grid"] > plan["cus"]
    assert plan["nv"] == 16   # a chunk size with a work-queue kernel
    d = on_device(w)
    lay = hs.LAYOUTS[layout]
    ws = hs.workspace(B, V, K, torch.float32, True)
    runs = [hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], mu=d["mu"], hlg=HLG_A,
                         k=K, ws=ws, opts=hs.SampleOpts(layout=lay), want_best=True)
            for _ in range(2)]
    exch = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], mu=d["mu"], hlg=HLG_A,
                        k=K, opts=hs.SampleOpts(layout=lay, split_lse=2, exchange_wait=-1),
                        want_best=True)
    pre = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], mu=d["mu"], hlg=HLG_A, k=K,
                       opts=hs.SampleOpts(layout=lay, split_lse=1), want_best=True)
    torch.cuda.synchronize()
    for idx, best in runs:
        np.testing.assert_array_equal(idx.cpu().numpy(), exch[0].cpu().numpy())
        np.testing.assert_array_equal(best.cpu().numpy(), exch[1].cpu().numpy())
    np.testing.assert_allclose(runs[0][1].cpu().numpy(), pre[1].cpu().numpy(), rtol=1e-6)
    # workspace layout for B = 600, K = 2 (256-byte aligned regions): counters [0, 4864),
    # keys [4864, 14592), pre-pass partials (left as written) [14592, 628992), exchange slots
    # [628992, 1243392), thresholds and row marks, then the work queue (the last 256 bytes)
    assert int(ws[:14592].to(torch.int32).abs().sum()) == 0
    assert int(ws[628992:1243392].to(torch.int32).abs().sum()) == 0
    assert int(ws[-256:].to(torch.int32).abs().sum()) == 0
    o, s1, s2 = oracle_sample(oracle_mod, w, layout=layout)
    print(assert_parity(runs[0][0].cpu().numpy(), o, s1, s2, w.logits.double().numpy(),
                        "work queue " + layout))


@pytest.mark.parametrize("dtype,V,nv,pivot", [(torch.bfloat16, 196608, 12, "top"),
                                               (torch.float16, 250000, 16, "entropy")])
def test_work_queue_other_kernels(hs, oracle_mod, dtype, V, nv, pivot):
    """The work-queue grid's other instantiations: 16-bit rows in chunks of 12 and 16 slots per
    lane, with the top and entropy anchors (screened layout). Ids agree with the oracle's, and
    ids and scores equal the one-block-per-item exchange's bit for bit."""
    B, K = 300, 1
    hlg = dict(HLG_A, pivot=pivot, pivot_offset=2.0 if pivot == "top" else 0.0)
    w = W.generic(B, V, dtype, seed=87, scale=1.0, mask_frac=0.1, hlg=hlg, K=K)
    plan = hs.sample_plan(B, V, K, dtype, True)
    assert plan["nchunk"] > 1 and plan["draw_groups"] == 1 and plan["grid"] > plan["cus"]
    assert plan["nv"] == nv
    d = on_device(w)
    opts = hs.SampleOpts(layout=hs.LAYOUTS["screened"])
    ws = hs.workspace(B, V, K, dtype, True)
    q = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], hlg=hlg, k=K, ws=ws,
                     opts=opts, want_best=True)
    exch = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], hlg=hlg, k=K,
                        opts=hs.SampleOpts(layout=opts.layout, split_lse=2, exchange_wait=-1),
                        want_best=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q[0].cpu().numpy(), exch[0].cpu().numpy())
    np.testing.assert_array_equal(q[1].cpu().numpy(), exch[1].cpu().numpy())
    assert int(ws[:256].to(torch.int32).abs().sum()) == 0
    assert int(ws[-256:].to(torch.int32).abs().sum()) == 0
    o, s1, s2 = oracle_sample(oracle_mod, w, layout="screened")
    print(assert_parity(q[0].cpu().numpy(), o, s1, s2, w.logits.double().numpy(),
                        "work queue %s %s" % (dtype, pivot)))


def test_workspace_left_clean(hs):
    """A split call leaves its workspace's counters, keys and exchange slots zero-filled, so
    calls can reuse it (with draw groups and the pre-pass, with the in-kernel exchange, and
    without the curve)."""
    w = W.generic(2, 100000, torch.float32, seed=81, hlg=HLG_A, K=4)
    d = on_device(w)
    ws = hs.workspace(2, 100000, 4, torch.float32, True)
    # layout for B = 2, K = 4: counters [0, 256), keys [256, 512), pre-pass partials
    # [512, 2560), exchange slots [2560, 4608)
    for hlg, opts in ((HLG_A, hs.SampleOpts(variant=2, nchunk=9)),
                      (HLG_A, hs.SampleOpts(variant=2, nchunk=9, draw_groups=1, split_lse=2)),
                      (None, hs.SampleOpts(variant=2, nchunk=9)),
                      (None, hs.SampleOpts(variant=2, nchunk=9, draw_groups=2))):
        outs = [hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"],
                             mu=d["mu"] if hlg else None, hlg=hlg, k=4, ws=ws,
                             opts=opts).cpu().numpy()
                for _ in range(3)]
        torch.cuda.synchronize()
        assert int(ws[:512].to(torch.int32).abs().sum()) == 0
        assert int(ws[2560:4608].to(torch.int32).abs().sum()) == 0
        for o in outs[1:]:
            np.testing.assert_array_equal(o, outs[0])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("hlg", [None, HLG_A])
def test_wide_range_rows(hs, oracle_mod, dtype, hlg):
    """Logits spanning hundreds of nats inside each lane's share of a row. The one-block kernel
    streams the log-sum-exp per lane against the lane's first vector maximum; lanes whose
    largest logit lies far from it sum again against that maximum, and the screen's bounds
    must hold at any scale. One block per row (forced) and the automatic split plan."""
    B, V = 4, 65536
    epv = 4 if dtype == torch.float32 else 8
    rng = np.random.default_rng(91)
    x = rng.normal(0, 2, size=(B, V)).astype(np.float32)
    first = 1024 * epv                    # the first vector of every lane (blocks of 1024)
    x[0, :first] -= 300.0                 # first vectors far below the rest
    x[1, :first] += 300.0                 # first vectors far above the rest
    x[2, 5 * first:] += 250.0             # later vectors far above the first ones
    x[3] *= 60.0                          # wide spread everywhere
    t = torch.from_numpy(x).to(dtype)
    T = rng.uniform(0.5, 1.5, size=B).astype(np.float32)
    seed = rng.integers(0, 2**64, size=B, dtype=np.uint64)
    off = rng.integers(0, 2**32, size=B, dtype=np.uint64)
    mu = W.mean_finite_logprob(t) if hlg is not None else None
    w = W.Workload("wide range", t, T, seed, off, K=4, hlg=hlg, mu=mu)
    d = on_device(w)
    o, s1, s2 = oracle_sample(oracle_mod, w)
    x64 = t.double().numpy()
    for name, opts in [("one-block", hs.SampleOpts(variant=1)), ("auto", None)]:
        idx = hs.sample_ex(d["logits"], d["T"], d["seed"], d["offset"], mu=d.get("mu"),
                           hlg=hlg, k=4, opts=opts).cpu().numpy()
        assert_parity(idx, o, s1, s2, x64, "wide range %s %s" % (name, dtype))
    if hlg is not None:
        lse = hs.logsumexp(d["logits"]).cpu().numpy().astype(np.float64)
        ref = np.array([np.logaddexp.reduce(x64[b]) for b in range(B)])
        np.testing.assert_allclose(lse, ref, rtol=2e-6, atol=0)

"""Top-k / top-p on the Gumbel path (curve off) on the HIP path against the oracle.

Reading (the Gumbel-max issue, "Softmax-free GPU sampling", names the filters as its follow-on
without an algorithm): temperature first, then top-k, then top-p on the tempered probabilities
of the tokens top-k keeps; row b keeps every token with x >= tau_b; the draw is the Gumbel-max
of x / T over the kept tokens.

Thresholds: a top-k threshold is a logit of the row and must equal the oracle's exactly. A
top-p threshold is decided by a mass sum: rows where the oracle's crossing lies within 1e-5 of
the target (flagged by the oracle) may take a neighbouring logit, so there the GPU threshold
must lie between the oracle's for p (1 + 2e-5) and p (1 - 2e-5), and its draws are checked
against that threshold only (a kept token, never a masked one). Elsewhere ids follow the
near-tie rule of the other parity tests."""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import assert_parity, on_device, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _case(B, V, dtype, seed, mask_frac=0.05, K=3):
    w = W.generic(B, V, dtype, seed=seed, scale=1.5, mask_frac=mask_frac, K=K)
    rng = np.random.default_rng(seed + 1)
    k = rng.choice([0, 1, 5, 50, 1000, V + 3], size=B).astype(np.int32)
    p = rng.choice([1.0, 0.5, 0.9, 0.95, 0.3, 0.999], size=B).astype(np.float32)
    return w, k, p


def _check_rows(hs, O, w, k, p, label, opts=None, want_best=False):
    d = on_device(w)
    kt = torch.from_numpy(k).cuda()
    pt = torch.from_numpy(p).cuda()
    tau_g = hs.filter_threshold(d["logits"], d["T"], top_k=kt, top_p=pt).cpu().numpy()
    layout = "screened" if (opts is not None and opts.layout == 1) else "plain"
    o, s1, s2, tau_o, amb = O.sample_filtered(w.logits, w.T, w.seed, w.offset, K=w.K, top_k=k,
                                              top_p=p, layout=layout)
    x64 = w.logits.double().numpy()
    # thresholds
    for r in range(w.B):
        if np.isnan(tau_o[r]):
            assert np.isnan(tau_g[r]), (label, r)
        elif not amb[r]:
            assert tau_g[r] == tau_o[r], (label, r, tau_g[r], tau_o[r])
        else:
            hi = O.filter_threshold(x64[r:r + 1], w.T[r:r + 1], top_k=k[r:r + 1],
                                    top_p=np.float32(min(1.0, p[r] * (1 - 2e-5))))[0][0]
            lo = O.filter_threshold(x64[r:r + 1], w.T[r:r + 1], top_k=k[r:r + 1],
                                    top_p=np.float32(min(1.0, p[r] * (1 + 2e-5))))[0][0]
            assert lo <= tau_g[r] <= hi, (label, r, lo, tau_g[r], hi)
    res = hs.sample_filtered(d["logits"], d["T"], d["seed"], d["offset"], top_k=kt, top_p=pt,
                             k=w.K, opts=opts, want_best=want_best)
    g = (res[0] if want_best else res).cpu().numpy()
    sure = ~amb
    assert_parity(g[sure], o[sure], s1[sure], s2[sure], x64[sure], label)
    for r in np.nonzero(amb)[0]:
        assert np.all(g[r] >= 0) and np.all(x64[r, g[r]] >= tau_g[r]), (label, r)
    return (g, res[1].cpu().numpy()) if want_best else g


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 151936), (torch.float32, 50001),
                                     (torch.float16, 32000), (torch.bfloat16, 1000),
                                     (torch.float32, 7)])
def test_filters_match_oracle(hs, oracle_mod, dtype, V):
    w, k, p = _case(12, V, dtype, seed=V % 977 + 1, mask_frac=0.05 if V > 10 else 0.0)
    _check_rows(hs, oracle_mod, w, k, p, "filters %s V=%d" % (dtype, V))


def test_filter_kernel_choices(hs, oracle_mod):
    """One block per row, split rows and draw groups, screened and exhaustive: the same ids;
    screened and exhaustive scoring bit-identical."""
    w, k, p = _case(6, 70001, torch.bfloat16, seed=5, K=4)
    res = {}
    for name, opts in [("one-block", hs.SampleOpts(variant=1)),
                       ("split7", hs.SampleOpts(variant=2, nchunk=7)),
                       ("split3-groups2", hs.SampleOpts(variant=2, nchunk=3, draw_groups=2)),
                       ("one-block-exhaustive", hs.SampleOpts(variant=1, no_screen=1)),
                       ("split7-exhaustive", hs.SampleOpts(variant=2, nchunk=7, no_screen=1))]:
        res[name] = _check_rows(hs, oracle_mod, w, k, p, name, opts=opts, want_best=True)
    for a, b in [("one-block", "one-block-exhaustive"), ("split7", "split7-exhaustive")]:
        np.testing.assert_array_equal(res[a][0], res[b][0])
        np.testing.assert_array_equal(res[a][1], res[b][1])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_filters_on_heavily_tied_rows(hs, oracle_mod, dtype):
    """16-bit rows with long runs of equal logits: more than 65535 copies of one value (a
    16-bit counter of the exact-value histogram overflows, and the radix selection takes
    over), signed zeros (-0 and +0 are one value, merged or not past 65535), values on a coarse
    grid, more than 65535 masked entries (never counted), and a constant row."""
    B, V = 6, 151936
    w = W.generic(B, V, dtype, seed=21, scale=1.0, K=3)
    x = w.logits.float().numpy().copy()
    rng = np.random.default_rng(22)
    x[0, rng.choice(V, 70000, replace=False)] = 0.5
    z = rng.choice(V, 80000, replace=False)
    x[1, z] = np.where(rng.random(80000) < 0.5, 0.0, -0.0)
    z = rng.choice(V, 60000, replace=False)
    x[2, z] = np.where(rng.random(60000) < 0.5, 0.0, -0.0)
    x[3] = np.round(x[3] * 4.0) / 4.0
    x[4, rng.choice(V, 100000, replace=False)] = -np.inf
    x[5] = 1.0
    w.logits = torch.from_numpy(x).to(dtype)
    # k lands inside the tie runs (row 0: below the 70000 copies of 0.5; row 2: in the zeros)
    n_above0 = int((x[0] > 0.5).sum())
    n_above2 = int((x[2] > 0.0).sum())
    k = np.array([n_above0 + 100, 0, n_above2 + 10, 50, 1000, 5], dtype=np.int32)
    p = np.array([0.9, 0.5, 0.95, 0.8, 0.3, 0.7], dtype=np.float32)
    _check_rows(hs, oracle_mod, w, k, p, "tied rows %s" % dtype)
    k2 = np.array([1, 70001, 0, 0, 200000, 0], dtype=np.int32)
    p2 = np.array([0.999, 1.0, 0.6, 0.99, 0.95, 0.5], dtype=np.float32)
    _check_rows(hs, oracle_mod, w, k2, p2, "tied rows (2) %s" % dtype)


def _row_marks(hs, ws, B, V, K, dtype):
    """The per-row marks of rows the threshold kernel drew itself: the workspace region (B int32,
    256-byte aligned) before the last 256 bytes (the resident grid's work counters)."""
    n = hs.workspace_bytes(B, V, K, dtype, False)
    off = n - 256 - (B * 4 + 255) // 256 * 256
    return ws[off:off + 4 * B].view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("layout", ["plain", "screened"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_fused_draws_match_the_sampler(hs, oracle_mod, dtype, layout):
    """Rows that keep few tokens are drawn by the threshold kernel (automatic plan); the
    sampling kernel on every row (an explicit variant) gives the same ids and scores."""
    B, V, K = 8, 60001, 7
    w = W.generic(B, V, dtype, seed=77, scale=1.5, mask_frac=0.05, K=K)
    k = np.array([1, 5, 50, 2048, 2049, 0, 100, 1000], dtype=np.int32)
    p = np.array([1.0, 1.0, 0.9, 1.0, 1.0, 0.3, 0.5, 1.0], dtype=np.float32)
    d = on_device(w)
    kt, pt = torch.from_numpy(k).cuda(), torch.from_numpy(p).cuda()
    lay = hs.LAYOUTS[layout]
    ws = hs.workspace(B, V, K, dtype, False)
    g, bs = hs.sample_filtered(d["logits"], d["T"], d["seed"], d["offset"], top_k=kt, top_p=pt,
                               k=K, ws=ws, want_best=True, opts=hs.SampleOpts(layout=lay))
    marks = _row_marks(hs, ws, B, V, K, dtype)
    assert marks[0] == 1 and marks[1] == 1 and marks[2] == 1, marks   # a few dozen kept tokens
    assert marks[4] == 0, marks                                         # over 2048 kept
    r, rb = hs.sample_filtered(d["logits"], d["T"], d["seed"], d["offset"], top_k=kt,
                               top_p=pt, k=K, opts=hs.SampleOpts(variant=1, layout=lay),
                               want_best=True)
    np.testing.assert_array_equal(g.cpu().numpy(), r.cpu().numpy())
    np.testing.assert_array_equal(bs.cpu().numpy(), rb.cpu().numpy())
    _check_rows(hs, oracle_mod, w, k, p, "fused %s %s" % (dtype, layout),
                opts=hs.SampleOpts(layout=lay))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fused_draw_limits(hs, oracle_mod, dtype):
    """(kept tokens) x draws at the limit (32 x 2048 = 65536: drawn in the threshold kernel)
    and just past it (33 x 2048: left to the sampler); the same ids either way."""
    B, V, K = 2, 4096, 2048
    w = W.generic(B, V, dtype, seed=79, scale=1.0, K=K)
    x = w.logits.float().numpy().copy()
    for r in range(B):
        x[r, np.random.default_rng(r).choice(V, 40, replace=False)] = 10.0 + 0.25 * np.arange(40)
    w.logits = torch.from_numpy(x).to(dtype)
    d = on_device(w)
    for kk, fused in ((32, 1), (33, 0)):
        k = np.full(B, kk, dtype=np.int32)
        ws = hs.workspace(B, V, K, dtype, False)
        g = hs.sample_filtered(d["logits"], d["T"], d["seed"], d["offset"],
                               top_k=torch.from_numpy(k).cuda(), k=K, ws=ws)
        assert (_row_marks(hs, ws, B, V, K, dtype) == fused).all()
        r = hs.sample_filtered(d["logits"], d["T"], d["seed"], d["offset"],
                               top_k=torch.from_numpy(k).cuda(), k=K,
                               opts=hs.SampleOpts(variant=1))
        np.testing.assert_array_equal(g.cpu().numpy(), r.cpu().numpy())
        _check_rows(hs, oracle_mod, w, k, np.ones(B, dtype=np.float32), "limit k=%d" % kk)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_special_rows_and_closed_cases(hs, dtype):
    """fp32 rows take the radix selection and the sampler; bf16 rows the histogram and, where
    few tokens are kept, the threshold kernel's own draw."""
    V = 500
    rng = np.random.default_rng(41)
    x = rng.normal(0, 1, size=(8, V)).astype(np.float32)
    x = torch.from_numpy(x).to(dtype).float().numpy()   # values exact in both dtypes
    x[0, :] = -np.inf                                   # no finite logit: -1
    x[1, [7, 9]] = 6.0                                  # tied maximum
    T = np.array([1.0, 1.0, 0.7, 1.0, 1.0, -1.0, 0.0, 1.0], dtype=np.float32)
    k = np.array([3, 1, 1, 0, 0, 5, 2, V], dtype=np.int32)
    p = np.array([0.9, 1.0, 1.0, 0.0, np.nan, 0.5, 0.1, 1.0], dtype=np.float32)
    t = torch.from_numpy(x).to(dtype).cuda()
    Tt = torch.from_numpy(T).cuda()
    seed = torch.arange(8, dtype=torch.int64, device="cuda") * 31 + 7
    off = torch.zeros(8, dtype=torch.int64, device="cuda")
    kt, pt = torch.from_numpy(k).cuda(), torch.from_numpy(p).cuda()
    g = hs.sample_filtered(t, Tt, seed, off, top_k=kt, top_p=pt, k=6).cpu().numpy()
    assert g[0].tolist() == [-1] * 6
    assert set(g[1].tolist()) <= {7, 9}                 # top-1 with a tie keeps both
    assert g[2].tolist() == [int(np.argmax(x[2]))] * 6  # k = 1
    assert g[3].tolist() == [-2] * 6 and g[4].tolist() == [-2] * 6   # p <= 0, NaN
    assert g[5].tolist() == [-2] * 6                    # bad T
    assert g[6].tolist() == [int(np.argmax(x[6]))] * 6  # greedy ignores the filters
    # nothing filtered (k >= V, p = 1): the unfiltered sampler
    ref = hs.gumbel_argmax(t, Tt, seed, off, k=6).cpu().numpy()
    np.testing.assert_array_equal(g[7], ref[7])
    tau = hs.filter_threshold(t, Tt, top_k=kt, top_p=pt).cpu().numpy()
    assert np.isneginf(tau[7]) and np.isneginf(tau[6]) and np.isnan(tau[3])


def test_no_filter_arrays_is_unfiltered(hs):
    w = W.generic(4, 20000, torch.bfloat16, seed=3, K=5)
    d = on_device(w)
    a = hs.sample_filtered(d["logits"], d["T"], d["seed"], d["offset"], k=5).cpu().numpy()
    b = hs.gumbel_argmax(d["logits"], d["T"], d["seed"], d["offset"], k=5).cpu().numpy()
    np.testing.assert_array_equal(a, b)


def test_filters_headline_shape(hs, oracle_mod):
    """256 x 151936 bf16 logits, curve off, top-k 50 and top-p 0.9 on every row."""
    w = W.config4()
    w.hlg = None
    w.mu = None
    B = w.B
    k = np.full(B, 50, dtype=np.int32)
    p = np.full(B, 0.9, dtype=np.float32)
    print(_check_rows(hs, oracle_mod, w, k, p, "256x151936 top-k 50 top-p 0.9").shape)

"""GPU building blocks against the oracle, through the C ABI: Philox words (bit-exact), the
fp32 Gumbel map (bounded error, exhaustive over all 2^32 words), log-sum-exp and the HLG
transform (within 1e-5 * max(1, |l'|), masks exactly -inf)."""
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def hs():
    return require_gpu()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.uint32)).view(np.int32))


def test_philox_kat_and_random(hs, oracle_mod):
    from tests.test_oracle_philox import load_kat
    kat = load_kat()
    ctr = np.array([c for c, _, _ in kat], dtype=np.uint32)
    key = np.array([k for _, k, _ in kat], dtype=np.uint32)
    got = hs.philox4x32_10(_i32(ctr).cuda(), _i32(key).cuda()).cpu().numpy().view(np.uint32)
    assert got.tolist() == [w for _, _, w in kat]
    rng = np.random.default_rng(101)
    ctr = rng.integers(0, 2**32, size=(1 << 16, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(1 << 16, 2), dtype=np.uint64).astype(np.uint32)
    got = hs.philox4x32_10(_i32(ctr).cuda(), _i32(key).cuda()).cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, oracle_mod.philox4x32_10(ctr, key))


@pytest.mark.parametrize("layout", ["plain", "screened"])
@pytest.mark.parametrize("V", [1, 5, 37, 4096, 151936])
def test_stream_words_bit_exact(hs, oracle_mod, V, layout):
    seeds = np.array([0, 2**64 - 1, 0x0123456789ABCDEF], dtype=np.uint64)
    offs = np.array([0, 2**32 - 1, 2**64 - 3], dtype=np.uint64)
    for k in (0, 1, 5):
        got = hs.stream_words(seeds, offs, 3, V, k, layout=layout).cpu().numpy().view(np.uint32)
        for b in range(3):
            want = oracle_mod.stream_words(int(seeds[b]), b, (int(offs[b]) + k) % 2**64, V,
                                           layout=layout)
            np.testing.assert_array_equal(got[b], want)


# Error bound of the fp32 Gumbel map: G is formed from E = -log(u) kept to a few ulps of
# relative error (log1p on the upper half), then G = -log(E) rounds once more; the absolute
# error is then below 3e-7 + 2 ulp(|G|) (ulp(22) = 1.9e-6).
def _gumbel_tol(g64):
    return 3e-7 + 2.0 * np.spacing(np.abs(g64).astype(np.float32)).astype(np.float64)


def test_gumbel_map_sampled(hs, oracle_mod):
    rng = np.random.default_rng(102)
    words = np.concatenate([
        np.array([0, 1, 2, 2**24, 2**31 - 1, 2**31, 2**31 + 1, 2**32 - 2, 2**32 - 1],
                 dtype=np.uint64),
        rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64),
        2**32 - 1 - rng.integers(0, 2**24, size=1 << 16, dtype=np.uint64),
        rng.integers(0, 2**24, size=1 << 16, dtype=np.uint64),
        2**31 + rng.integers(-2**20, 2**20, size=1 << 16).astype(np.int64).astype(np.uint64),
    ]).astype(np.uint32)
    g32 = hs.gumbel_f32(_i32(words).cuda()).cpu().numpy().astype(np.float64)
    g64 = oracle_mod.gumbel(words)
    err = np.abs(g32 - g64)
    assert np.all(err <= _gumbel_tol(g64)), float((err / _gumbel_tol(g64)).max())
    # monotone in the word up to that rounding
    order = np.argsort(words)
    assert np.all(np.diff(g32[order]) >= -2 * _gumbel_tol(g64[order][1:]))


def test_gumbel_map_exhaustive(hs):
    """All 2^32 words: the fp32 map against float64 -log(-log(u)) evaluated by torch on the
    GPU (an independent library routine), and against its screening bound
    G <= (clz(~r) + 1) ln 2."""
    worst = 0.0
    chunk = 1 << 28
    ln2 = np.log(2.0)
    for c in range(1 << 4):
        r = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda")
        w32 = r.to(torch.int32)                              # wraps to the uint32 bit pattern
        g = hs.gumbel_f32(w32).double()
        u = (r.double() + 0.5) * 2.0 ** -32
        g64 = -torch.log(-torch.log(u))
        tol = 3e-7 + 2.0 * torch.abs(g64).float().nextafter(torch.tensor(float("inf"), device="cuda")).sub(
            torch.abs(g64).float()).double()
        err = (g - g64).abs()
        worst = max(worst, float((err / tol).max()))
        assert bool((err <= tol).all()), "chunk %d: worst err/tol %.3f" % (c, float((err / tol).max()))
        notr = (2**32 - 1) - r
        nlz = torch.where(notr == 0, torch.full_like(notr, 32),
                          31 - torch.floor(torch.log2(notr.clamp(min=1).double())).long())
        assert bool((g <= (nlz + 1).double() * ln2 + 1e-6).all())
    print("exhaustive Gumbel map: worst err/tol = %.3f" % worst)


def _rows64(x):
    return x.double().cpu().numpy()


LSE_CASES = [
    ("fp32 bimodal 8x151936", lambda: __import__("synth.workloads", fromlist=["x"]).config3()),
    ("bf16 flat 16x151936", lambda: __import__("synth.workloads", fromlist=["x"]).config4(B=16)),
    ("f16 ragged 5x4099", lambda: __import__("synth.workloads", fromlist=["x"]).generic(
        5, 4099, torch.float16, seed=9, scale=1.5, mask_frac=0.2,
        hlg={"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0})),
    ("fp32 tiny 3x7", lambda: __import__("synth.workloads", fromlist=["x"]).generic(
        3, 7, torch.float32, seed=10, mask_frac=0.3,
        hlg={"m": 0.8, "w": 0.25, "beta_t": 3.0, "beta_h": 0.1})),
]


@pytest.mark.parametrize("name,make", LSE_CASES, ids=[c[0] for c in LSE_CASES])
def test_logsumexp_and_transform(hs, oracle_mod, name, make):
    w = make()
    x = w.logits.cuda()
    lse = hs.logsumexp(x).cpu().numpy().astype(np.float64)
    want = oracle_mod.logsumexp(w.logits)
    np.testing.assert_allclose(lse, want, rtol=0, atol=4e-6 * max(1.0, np.abs(want).max()))
    lp = hs.hlg_transform(x, torch.from_numpy(w.mu).cuda(), w.hlg).cpu().numpy().astype(np.float64)
    ref = oracle_mod.hlg_transform(w.logits, w.mu, w.hlg["m"], w.hlg["w"], w.hlg["beta_t"],
                                   w.hlg["beta_h"])
    masked = ~np.isfinite(_rows64(w.logits))
    assert np.all(lp[masked] == -np.inf)
    fin = ~masked
    err = np.abs(lp[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
    assert err.max() <= 1e-5, err.max()


def test_transform_misaligned_rows(hs, oracle_mod):
    """Rows that are not 16-byte aligned (ld = V + 1) take the element-wise load path."""
    from synth.workloads import generic
    w = generic(4, 1001, torch.bfloat16, seed=11, mask_frac=0.1,
                hlg={"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0})
    big = torch.full((4, 1002), float("-inf"), dtype=torch.bfloat16)
    big[:, :1001] = w.logits
    x = big.cuda()[:, :1001]
    assert x.stride(0) == 1002
    lp = hs.hlg_transform(x, torch.from_numpy(w.mu).cuda(), w.hlg).cpu().numpy()
    ref = oracle_mod.hlg_transform(w.logits, w.mu, 1.5, 2.0, 1.0, 2.0)
    fin = np.isfinite(ref)
    assert np.all(lp[~fin] == -np.inf)
    assert (np.abs(lp[fin] - ref[fin]) / np.maximum(1, np.abs(ref[fin]))).max() <= 1e-5

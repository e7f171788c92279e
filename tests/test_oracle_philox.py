"""Pins for the oracle's Philox4x32-10 and its per-element counter layout.

- published known-answer vectors (Random123, Salmon et al. SC'11), stored in tests/golden;
- an independent pure-Python Philox written here from the published definition;
- differential runs against two open-source implementations compiled here from their
  headers (PyTorch's PhiloxRNGEngine and rocRAND's philox4x32_10_engine);
- the element -> (counter, key, word) layout read for "(seed, row, i, offset)" in the mlxcel
  issue "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel", section Task.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
M32 = 0xFFFFFFFF


def py_philox(ctr, key, rounds=10):
    """Philox4x32 from the SC'11 definition: S-box = 32x32->64 multiplies of words 0 and 2
    by 0xD2511F53 / 0xCD9E8D57, permutation (hi1^c1^k0, lo1, hi0^c3^k1, lo0), key schedule
    by the Weyl increments 0x9E3779B9 / 0xBB67AE85 between rounds."""
    c0, c1, c2, c3 = [int(v) & M32 for v in ctr]
    k0, k1 = [int(v) & M32 for v in key]
    for r in range(rounds):
        if r:
            k0 = (k0 + 0x9E3779B9) & M32
            k1 = (k1 + 0xBB67AE85) & M32
        p0 = 0xD2511F53 * c0
        p1 = 0xCD9E8D57 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & M32, p1 & M32, ((p0 >> 32) ^ c3 ^ k1) & M32, p0 & M32
    return [c0, c1, c2, c3]


def load_kat():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v = [int(t, 16) for t in line.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


def test_kat_vectors_oracle(oracle_mod):
    kat = load_kat()
    assert len(kat) == 3
    for ctr, key, want in kat:
        got = oracle_mod.philox4x32_10(ctr, key)[0]
        assert [int(v) for v in got] == want


def test_kat_vectors_pure_python():
    for ctr, key, want in load_kat():
        assert py_philox(ctr, key) == want


def test_random_inputs_match_pure_python(oracle_mod):
    rng = np.random.default_rng(11)
    ctr = rng.integers(0, 2**32, size=(2000, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(2000, 2), dtype=np.uint64).astype(np.uint32)
    got = oracle_mod.philox4x32_10(ctr, key)
    for j in range(ctr.shape[0]):
        assert [int(v) for v in got[j]] == py_philox(ctr[j], key[j])


def _build_helper(kind, tmp):
    src = os.path.join(HERE, "philox_diff", kind + "_philox.cpp")
    exe = os.path.join(tmp, kind)
    if kind == "aten":
        torch = pytest.importorskip("torch")
        inc = os.path.join(os.path.dirname(torch.__file__), "include")
        cmd = ["g++", "-O1", "-std=c++17", "-I" + inc, "-o", exe, src]
    else:
        hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
        if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
            pytest.skip("rocRAND headers / hipcc not available")
        cmd = [hipcc, "-O1", "-o", exe, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("could not build %s helper: %s" % (kind, r.stderr[-400:]))
    return exe


@pytest.mark.parametrize("kind", ["aten", "rocrand"])
def test_differential_against_open_source_engines(oracle_mod, kind):
    rng = np.random.default_rng(12 if kind == "aten" else 13)
    n = 500
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[0] = 0
    key[0] = 0
    ctr[1] = 0xFFFFFFFF
    key[1] = 0xFFFFFFFF
    with tempfile.TemporaryDirectory() as tmp:
        exe = _build_helper(kind, tmp)
        inp = "\n".join("%08x %08x %08x %08x %08x %08x" % (*c, *k) for c, k in zip(ctr, key)) + "\n"
        r = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
    ref = np.array([[int(t, 16) for t in line.split()] for line in r.stdout.strip().splitlines()],
                   dtype=np.uint64).astype(np.uint32)
    got = oracle_mod.philox4x32_10(ctr, key)
    np.testing.assert_array_equal(got, ref)


def test_element_word_layout(oracle_mod):
    """word(seed, row, off, i) = Philox(ctr=(i>>2, row, off lo, off hi),
    key=(seed lo, seed hi))[i & 3], including 64-bit seeds and offsets that carry."""
    cases = [
        (0, 0, 0, 0), (0, 0, 0, 3), (0, 0, 0, 4), (1, 2, 3, 5),
        (0xDEADBEEFCAFEF00D, 7, 0xFFFFFFFF, 151935),
        (0x0123456789ABCDEF, 255, 0x100000000, 262143),
        (2**64 - 1, 1023, 2**64 - 1, 17),
    ]
    for seed, row, off, i in cases:
        want = py_philox((i >> 2, row, off & M32, off >> 32), (seed & M32, seed >> 32))[i & 3]
        assert oracle_mod.element_word(seed, row, off, i) == want


def test_stream_words_vector(oracle_mod):
    seed, row, off, V = 0x9E3779B97F4A7C15, 5, 2**32 - 2, 37
    w = oracle_mod.stream_words(seed, row, off, V)
    for i in range(V):
        assert int(w[i]) == oracle_mod.element_word(seed, row, off, i)
    # neighbouring streams differ: row, offset and seed all enter the counter / key
    assert not np.array_equal(w, oracle_mod.stream_words(seed, row + 1, off, V))
    assert not np.array_equal(w, oracle_mod.stream_words(seed, row, off + 1, V))
    assert not np.array_equal(w, oracle_mod.stream_words(seed ^ 1, row, off, V))
    assert not np.array_equal(w, oracle_mod.stream_words(seed ^ (1 << 40), row, off, V))


def _py_screened(seed, row, off, i):
    """Element i = 8q + e of the screened layout, from the pure-Python Philox: the high half of
    its word is the 16-bit half e of the call at counter word 2q, the low half that of the call
    at 2q + 1 (half e of an output = word e // 2, low bits for even e, high bits for odd e)."""
    q, e = i // 8, i % 8
    key = (seed & M32, seed >> 32)
    hi = py_philox((2 * q, row, off & M32, off >> 32), key)
    lo = py_philox((2 * q + 1, row, off & M32, off >> 32), key)

    def half(words):
        return (words[e // 2] >> (16 * (e % 2))) & 0xFFFF
    return (half(hi) << 16) | half(lo)


SCREENED_CASES = [
    (0, 0, 0, 0), (0, 0, 0, 7), (0, 0, 0, 8), (1, 2, 3, 13),
    (0xDEADBEEFCAFEF00D, 7, 0xFFFFFFFF, 151935),
    (0x0123456789ABCDEF, 255, 0x100000000, 262143),
    (2**64 - 1, 1023, 2**64 - 1, 17),
]


@pytest.mark.parametrize("seed,row,off,i", SCREENED_CASES)
def test_screened_layout_pure_python(oracle_mod, seed, row, off, i):
    assert oracle_mod.element_word(seed, row, off, i, "screened") == \
        _py_screened(seed, row, off, i)


def test_screened_layout_recombines_plain_words(oracle_mod):
    """The screened layout draws on the same Philox calls as the plain one and only hands their
    bits out differently: with P the plain words of a stream, element 8q + e of the screened
    layout is (half e%2 of P[8q + e//2]) << 16 | (half e%2 of P[8q + 4 + e//2]). Checked on
    whole streams, ragged tails included."""
    for seed, row, off, V in [(42, 0, 0, 4096), (0x9E3779B97F4A7C15, 5, 2**32 - 2, 1003),
                              (7, 1023, 2**63 + 5, 27)]:
        plain = oracle_mod.stream_words(seed, row, off, (V + 7) // 8 * 8).astype(np.uint64)
        scr = oracle_mod.stream_words(seed, row, off, V, "screened").astype(np.uint64)
        i = np.arange(V)
        q, e = i // 8, i % 8
        shift = (16 * (e % 2)).astype(np.uint64)
        hi = (plain[8 * q + e // 2] >> shift) & 0xFFFF
        lo = (plain[8 * q + 4 + e // 2] >> shift) & 0xFFFF
        np.testing.assert_array_equal(scr, (hi << 16) | lo)


def test_screened_words_look_uniform(oracle_mod):
    """Every bit of the screened words is set about half the time, and their leading bytes
    fill 256 buckets evenly."""
    w = oracle_mod.stream_words(42, 3, 9, 1 << 16, "screened")
    bits = ((w[:, None] >> np.arange(32, dtype=np.uint32)) & 1).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 0.01)   # sd of a bit's mean ~0.002
    counts = np.bincount((w >> 24).astype(np.int64), minlength=256)
    exp = (1 << 16) / 256
    assert ((counts - exp) ** 2 / exp).sum() < 400


def test_words_look_uniform(oracle_mod):
    """Coarse sanity: 2^16 words of one stream fill 256 byte-buckets evenly."""
    w = oracle_mod.stream_words(42, 0, 0, 1 << 16)
    counts = np.bincount((w >> 24).astype(np.int64), minlength=256)
    exp = (1 << 16) / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 400  # 255 dof: mean 255, sd ~22.6

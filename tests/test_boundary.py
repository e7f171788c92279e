"""The C-ABI boundary without a GPU: the library loads, exports every symbol include/hs.h
declares, and rejects every host-checkable bad argument with its status code before any
work is enqueued (no device is touched by these calls)."""
import ctypes as C
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

hs = pytest.importorskip("logit_transform_amd")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_DTYPE, HS_ERR_WORKSPACE, HS_ERR_HIP, HS_ERR_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5
FAKE = 0x10000            # never dereferenced: every case below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hs.library_path()):
        pytest.skip("libhs.so not built")
    return hs.load()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "hs.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("hs_logsumexp", "hs_hlg_transform", "hs_gumbel_argmax", "hs_sample"):
        assert name in syms
    assert sorted(hs.EXPORTED_SYMBOLS) == syms


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for code in (HS_OK, HS_ERR_INVALID_ARG, HS_ERR_DTYPE, HS_ERR_WORKSPACE, HS_ERR_HIP,
                 HS_ERR_UNSUPPORTED):
        s = lib.hs_status_str(code).decode()
        assert s.startswith("HS_")
    assert "unknown" in lib.hs_status_str(12345).decode()
    assert "gfx950" in hs.version()


def L(B=4, V=100, ld=None, dtype=0, data=FAKE):
    return hs._Logits(data, dtype, B, V, V if ld is None else ld)


def H(m=1.5, w=2.0, bt=1.0, bh=2.0, pivot=0, off=0.0):
    return hs.HlgParams(m, w, bt, bh, pivot, off)


def sample(lib, x, T=FAKE, mu=FAKE, hlg=None, seed=FAKE, off=FAKE, K=1, out=FAKE, ws=None,
           nbytes=0):
    return lib.hs_sample(C.byref(x), T, mu, C.byref(hlg) if hlg is not None else None, seed, off,
                         K, out, ws, nbytes, None)


@pytest.mark.parametrize("x,code", [
    (L(data=0), HS_ERR_INVALID_ARG),
    (L(B=0), HS_ERR_INVALID_ARG),
    (L(B=-3), HS_ERR_INVALID_ARG),
    (L(V=0), HS_ERR_INVALID_ARG),
    (L(V=100, ld=99), HS_ERR_INVALID_ARG),
    (L(dtype=7), HS_ERR_DTYPE),
    (L(dtype=-1), HS_ERR_DTYPE),
    (L(V=2**31, ld=2**31), HS_ERR_UNSUPPORTED),
    (L(V=2**30, ld=2**30, dtype=0), HS_ERR_UNSUPPORTED),   # an fp32 row of 4 GiB
])
def test_bad_logits(lib, x, code):
    assert sample(lib, x) == code
    assert lib.hs_gumbel_argmax(C.byref(x), FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == code
    assert lib.hs_logsumexp(C.byref(x), FAKE, None) == code
    h = H()
    assert lib.hs_hlg_transform(C.byref(x), FAKE, C.byref(h), FAKE, max(x.V, 1), None) == code
    assert lib.hs_hlg_pivot(C.byref(x), FAKE, C.byref(h), FAKE, None) == code


def test_row_byte_limit(lib):
    """Within-row byte offsets are 32-bit: a row must hold fewer than 2^32 bytes, so fp32 rows
    stop at 2^30 - 1 elements while 16-bit rows reach 2^31 - 1. The logits are validated
    first: a missing output then gives HS_ERR_INVALID_ARG for an accepted shape."""
    for dtype, vmax in ((0, 2**30 - 1), (1, 2**31 - 1), (2, 2**31 - 1)):
        assert lib.hs_logsumexp(C.byref(L(B=1, V=vmax, dtype=dtype)), None, None) == \
            HS_ERR_INVALID_ARG
        assert lib.hs_logsumexp(C.byref(L(B=1, V=vmax + 1, dtype=dtype)), None, None) == \
            HS_ERR_UNSUPPORTED


def test_null_logits_struct(lib):
    assert lib.hs_sample(None, FAKE, None, None, FAKE, FAKE, 1, FAKE, None, 0, None) == HS_ERR_INVALID_ARG
    assert lib.hs_logsumexp(None, FAKE, None) == HS_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(T=None), dict(seed=None), dict(off=None), dict(out=None),
                                dict(K=0), dict(K=-2)])
def test_bad_sample_args(lib, kw):
    assert sample(lib, L(), **kw) == HS_ERR_INVALID_ARG


@pytest.mark.parametrize("h", [H(m=0.0), H(m=-1.0), H(m=math.inf), H(m=math.nan), H(w=-0.5),
                               H(w=math.nan), H(bt=0.0), H(bt=math.inf), H(bh=-1.0),
                               H(bh=math.nan), H(pivot=4), H(pivot=-1),
                               H(pivot=1, off=math.inf), H(pivot=1, off=math.nan)])
def test_bad_curve(lib, h):
    assert sample(lib, L(), hlg=h) == HS_ERR_INVALID_ARG
    x = L()
    assert lib.hs_hlg_transform(C.byref(x), FAKE, C.byref(h), FAKE, 100, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_pivot(C.byref(x), FAKE, C.byref(h), FAKE, None) == HS_ERR_INVALID_ARG


def test_median_pivot_boundary(lib):
    """The mass-median pivot needs no mu; the sampler needs the workspace for it."""
    HS_ERR_WORKSPACE = -3
    h = H(pivot=3)
    assert sample(lib, L(), hlg=h, mu=None) == HS_ERR_WORKSPACE
    x = L()
    assert lib.hs_hlg_transform(C.byref(x), None, C.byref(h), FAKE, 99, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_pivot(C.byref(x), None, C.byref(h), None, None) == HS_ERR_INVALID_ARG


def test_curve_needs_mu(lib):
    assert sample(lib, L(), hlg=H(), mu=None) == HS_ERR_INVALID_ARG


@pytest.mark.parametrize("pivot,off", [(1, 0.0), (1, -3.5), (2, 0.0), (2, math.nan)])
def test_anchored_pivots_need_no_mu(lib, pivot, off):
    """Top- and entropy-anchored pivots are derived from the row [HLG, The pivot]: no mu is
    needed, and the entropy anchor ignores the offset. With a too-small workspace the call
    gets as far as the workspace check."""
    h = H(pivot=pivot, off=off)
    assert sample(lib, L(), hlg=h, mu=None, ws=FAKE, nbytes=8) == HS_ERR_WORKSPACE
    x = L()
    assert lib.hs_hlg_transform(C.byref(x), None, C.byref(h), None, 100, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_pivot(C.byref(x), None, C.byref(h), None, None) == HS_ERR_INVALID_ARG


def test_pivot_args(lib):
    x = L()
    assert lib.hs_hlg_pivot(C.byref(x), None, C.byref(H()), FAKE, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_pivot(C.byref(x), FAKE, None, FAKE, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_pivot(C.byref(x), FAKE, C.byref(H()), None, None) == HS_ERR_INVALID_ARG


def test_binding_pivot_modes():
    assert hs._hlg_struct({"m": 1.0, "w": 1.0, "beta_t": 1.0, "beta_h": 1.0,
                           "pivot": "entropy"}).pivot == 2
    h = hs._hlg_struct((1.0, 2.0, 1.0, 1.0, "top", -2.5))
    assert (h.pivot, h.pivot_offset) == (1, -2.5)
    assert hs._hlg_struct((1.0, 2.0, 1.0, 1.0)).pivot == 0
    assert hs._hlg_struct((1.0, 2.0, 1.0, 1.0, "median")).pivot == 3
    with pytest.raises(ValueError):
        hs._hlg_struct((1.0, 2.0, 1.0, 1.0, "mode"))


def test_rolloff_off_is_accepted_by_validation(lib):
    # w = +inf is valid; with a too-small workspace the call stops at the workspace check
    assert sample(lib, L(), hlg=H(w=math.inf), ws=FAKE, nbytes=8) == HS_ERR_WORKSPACE


def test_transform_args(lib):
    x = L()
    h = H()
    assert lib.hs_hlg_transform(C.byref(x), None, C.byref(h), FAKE, 100, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_transform(C.byref(x), FAKE, None, FAKE, 100, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_transform(C.byref(x), FAKE, C.byref(h), None, 100, None) == HS_ERR_INVALID_ARG
    assert lib.hs_hlg_transform(C.byref(x), FAKE, C.byref(h), FAKE, 99, None) == HS_ERR_INVALID_ARG
    assert lib.hs_logsumexp(C.byref(x), None, None) == HS_ERR_INVALID_ARG


def test_workspace_sizes(lib):
    n = lib.hs_workspace_bytes(256, 151936, 1, 1, 1)
    assert n > 0 and n % 256 == 0
    assert lib.hs_workspace_bytes(256, 151936, 16, 1, 1) > n
    assert lib.hs_workspace_bytes(0, 10, 1, 0, 0) == 0
    assert lib.hs_workspace_bytes(1, 10, 0, 0, 0) == 0
    assert lib.hs_workspace_bytes(1, 10, 1, 9, 0) == 0
    # a given-but-too-small workspace is reported, not ignored
    assert sample(lib, L(), ws=FAKE, nbytes=n // 1000 or 8) == HS_ERR_WORKSPACE
    assert lib.hs_workspace_init(None, 256, None) == HS_ERR_INVALID_ARG
    assert lib.hs_workspace_init(FAKE, 3, None) == HS_ERR_INVALID_ARG


def test_sample_ex_opts(lib):
    x = L()
    for o in (hs.SampleOpts(variant=3), hs.SampleOpts(variant=-1), hs.SampleOpts(nchunk=-1),
              hs.SampleOpts(nchunk=65), hs.SampleOpts(draw_groups=-2),
              hs.SampleOpts(split_lse=3), hs.SampleOpts(split_lse=-1),
              hs.SampleOpts(exchange_wait=-2)):
        assert lib.hs_sample_ex(C.byref(x), FAKE, None, None, FAKE, FAKE, 1, FAKE, None, None, 0,
                                C.byref(o), None) == HS_ERR_INVALID_ARG


def test_sample_rows_args(lib):
    x = L()
    # per-row settings are required; opts are checked as for hs_sample_ex
    assert lib.hs_sample_rows(C.byref(x), FAKE, None, None, FAKE, FAKE, 1, FAKE, None, None, 0,
                              None, None) == HS_ERR_INVALID_ARG
    o = hs.SampleOpts(variant=5)
    assert lib.hs_sample_rows(C.byref(x), FAKE, None, FAKE, FAKE, FAKE, 1, FAKE, None, None, 0,
                              C.byref(o), None) == HS_ERR_INVALID_ARG
    for bad, code in ((L(data=0), HS_ERR_INVALID_ARG), (L(dtype=9), HS_ERR_DTYPE)):
        assert lib.hs_sample_rows(C.byref(bad), FAKE, None, FAKE, FAKE, FAKE, 1, FAKE, None,
                                  None, 0, None, None) == code
    for kw in (dict(T=None), dict(seed=None), dict(out=None), dict(K=0)):
        a = dict(T=FAKE, seed=FAKE, out=FAKE, K=1)
        a.update(kw)
        assert lib.hs_sample_rows(C.byref(x), a["T"], None, FAKE, a["seed"], FAKE, a["K"],
                                  a["out"], None, None, 0, None, None) == HS_ERR_INVALID_ARG
    # mu is optional (rows decide in the kernel): valid arguments reach the workspace check
    assert lib.hs_sample_rows(C.byref(x), FAKE, None, FAKE, FAKE, FAKE, 1, FAKE, None, FAKE, 8,
                              None, None) == HS_ERR_WORKSPACE


def test_hlg_rows_packing():
    import struct
    rows = [None, (1.5, 2.0, 1.0, 3.0), {"m": 0.5, "w": math.inf, "beta_t": 2.0, "beta_h": 4.0,
                                         "pivot": "top", "pivot_offset": 6.0}]
    assert C.sizeof(hs.HlgRow) == 32
    raw = bytes(hs._pack_rows(rows))
    assert len(raw) == 96
    vals = [struct.unpack_from("<4fifii", raw, 32 * i) for i in range(3)]
    assert vals[0][6] == 0                                   # off
    assert vals[1] == (1.5, 2.0, 1.0, 3.0, 0, 0.0, 1, 0)
    assert vals[2][:2] == (0.5, math.inf) and vals[2][4:] == (1, 6.0, 1, 0)


def test_filter_args(lib):
    x = L()
    assert lib.hs_filter_threshold(C.byref(x), None, FAKE, FAKE, FAKE, None) == HS_ERR_INVALID_ARG
    assert lib.hs_filter_threshold(C.byref(x), FAKE, FAKE, FAKE, None, None) == HS_ERR_INVALID_ARG
    assert lib.hs_filter_threshold(C.byref(L(dtype=5)), FAKE, None, None, FAKE, None) == HS_ERR_DTYPE
    o = hs.SampleOpts(nchunk=99)
    assert lib.hs_sample_filtered(C.byref(x), FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, None,
                                  0, C.byref(o), None) == HS_ERR_INVALID_ARG
    assert lib.hs_sample_filtered(C.byref(x), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None,
                                  0, None, None) == HS_ERR_INVALID_ARG
    # filtering needs the workspace (the thresholds live in it)
    assert lib.hs_sample_filtered(C.byref(x), FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, None, None,
                                  0, None, None) == HS_ERR_WORKSPACE


def test_aux_entry_points(lib):
    assert lib.hs_philox4x32_10(None, FAKE, FAKE, 4, None) == HS_ERR_INVALID_ARG
    assert lib.hs_philox4x32_10(FAKE, FAKE, FAKE, -1, None) == HS_ERR_INVALID_ARG
    assert lib.hs_philox4x32_10(FAKE, FAKE, FAKE, 0, None) == HS_OK
    assert lib.hs_stream_words(FAKE, FAKE, 0, 10, 0, FAKE, None) == HS_ERR_INVALID_ARG
    assert lib.hs_stream_words(FAKE, FAKE, 1, 10, -1, FAKE, None) == HS_ERR_INVALID_ARG
    assert lib.hs_stream_words(FAKE, None, 1, 10, 0, FAKE, None) == HS_ERR_INVALID_ARG
    assert lib.hs_gumbel_f32(None, FAKE, 3, None) == HS_ERR_INVALID_ARG
    assert lib.hs_gumbel_f32(FAKE, FAKE, 0, None) == HS_OK
    assert lib.hs_stream_words_ex(FAKE, FAKE, 1, 10, 0, 2, FAKE, None) == HS_ERR_INVALID_ARG
    assert lib.hs_stream_words_ex(FAKE, FAKE, 1, 10, 0, -1, FAKE, None) == HS_ERR_INVALID_ARG


def test_sample_opts_layout_is_validated(lib):
    x = L()
    for lay in (-1, 2):
        o = hs.SampleOpts(layout=lay)
        assert lib.hs_sample_ex(C.byref(x), FAKE, None, None, FAKE, FAKE, 1, FAKE, None, None, 0,
                                C.byref(o), None) == HS_ERR_INVALID_ARG


def test_noalloc_arguments(lib):
    """The allocation-free entry point checks every host-side argument before it touches a
    device, and refuses shapes whose workspace exceeds its static array."""
    cap = lib.hs_sample_noalloc_max_workspace()
    assert cap == 4 << 20

    def call(x, K=1, T=FAKE, out=FAKE, hlg=None, mu=FAKE, opts=None):
        return lib.hs_sample_noalloc(C.byref(x), T, mu, C.byref(hlg) if hlg else None, FAKE,
                                     FAKE, K, out, None, C.byref(opts) if opts else None, None)
    assert call(L(data=0)) == HS_ERR_INVALID_ARG
    assert call(L(dtype=9)) == HS_ERR_DTYPE
    assert call(L(), K=0) == HS_ERR_INVALID_ARG
    assert call(L(), T=None) == HS_ERR_INVALID_ARG
    assert call(L(), out=None) == HS_ERR_INVALID_ARG
    assert call(L(), hlg=H(m=-1.0)) == HS_ERR_INVALID_ARG
    assert call(L(), hlg=H(), mu=None) == HS_ERR_INVALID_ARG
    assert call(L(), opts=hs.SampleOpts(layout=5)) == HS_ERR_INVALID_ARG
    # workspace past the static array: B = 8192 rows need 8192 * (64 * 32) bytes of partials
    # and exchange slots alone
    big = L(B=8192, V=1000)
    assert lib.hs_workspace_bytes(8192, 1000, 1, 0, 1) > cap
    assert call(big) == HS_ERR_UNSUPPORTED
    assert call(L(B=64, V=1000), K=8192) == HS_ERR_UNSUPPORTED   # 6 MiB of counters and keys


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 8)
    with pytest.raises(ValueError):
        hs.sample(x, [1.0, 1.0], [1, 2], [0, 0])
    with pytest.raises(ValueError):
        hs.logsumexp(x)


def test_micro_library_exports():
    """The benchmark's ceiling kernels (streaming read, Philox rate) build into a library of
    their own and reject bad shapes before launching anything."""
    p = os.path.join(ROOT, "logit_transform_amd", "libhs_micro.so")
    if not os.path.exists(p):
        pytest.skip("libhs_micro.so not built")
    M = C.CDLL(p)
    M.hs_micro_stream_max.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int64, C.c_int64,
                                      C.c_void_p, C.c_void_p]
    M.hs_micro_philox_max.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                      C.c_void_p, C.c_void_p]
    assert M.hs_micro_stream_max(None, 1, 4, 64, 64, FAKE, None) == -1
    assert M.hs_micro_stream_max(FAKE, 1, 4, 63, 64, FAKE, None) == -1     # not whole vectors
    assert M.hs_micro_stream_max(FAKE, 9, 4, 64, 64, FAKE, None) == -1
    M.hs_micro_stream_max_nt.argtypes = M.hs_micro_stream_max.argtypes
    assert M.hs_micro_stream_max_nt(FAKE, 1, 4, 63, 64, FAKE, None) == -1
    assert M.hs_micro_philox_max(FAKE, 4, 10, 1, 1, FAKE, None) == -1      # V % 4 != 0
    assert M.hs_micro_philox_max(None, 4, 64, 1, 1, FAKE, None) == -1
    assert M.hs_micro_philox_max(FAKE, 4, 64, 2, 3, FAKE, None) == -1      # groups > K


def test_per_row_arguments_broadcast():
    """A per-row argument given as one value applies to every row; other lengths are refused."""
    import torch
    t = hs._row_vec(0.7, 4, torch.float32, "cpu", "T")
    assert t.tolist() == pytest.approx([0.7] * 4)
    s = hs._row_vec(2**64 - 1, 3, torch.int64, "cpu", "seed")
    assert s.tolist() == [-1, -1, -1]                       # the uint64 bit pattern
    assert hs._row_vec([1, 2, 3], 3, torch.int32, "cpu", "top_k").tolist() == [1, 2, 3]
    with pytest.raises(ValueError):
        hs._row_vec([1, 2], 3, torch.int32, "cpu", "top_k")

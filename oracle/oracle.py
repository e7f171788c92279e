"""ctypes wrapper around the double-precision CPU oracle ``hs_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline
leg are the only callers. The HIP library never imports this module and this module never
imports the HIP library.

Sources: "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document,
sections "The transfer function", "Greedy is untouched") and "Softmax-free GPU sampling:
Gumbel-max categorical sampling kernel" (lablup/mlxcel issue #900, sections "Background",
"Task", "Regression guard"); Philox4x32-10 per Salmon et al., SC'11.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        # HS_ORACLE_LIBRARY: another build of the same source (the sanitized one)
        path = os.environ.get("HS_ORACLE_LIBRARY") or _build.build(force=False)
        L = C.CDLL(path)
        u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
        u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        L.or_philox4x32_10_n.argtypes = [C.c_int64, u32p, u32p, u32p]
        L.or_philox4x32_10_n.restype = None
        L.or_element_word.argtypes = [C.c_uint64] * 4
        L.or_element_word.restype = C.c_uint32
        L.or_stream_words.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_int64, u32p]
        L.or_stream_words.restype = None
        L.or_stream_words_layout.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_int64,
                                             C.c_int, u32p]
        L.or_stream_words_layout.restype = None
        L.or_element_word_layout.argtypes = [C.c_uint64] * 4 + [C.c_int]
        L.or_element_word_layout.restype = C.c_uint32
        L.or_gumbel_n.argtypes = [C.c_int64, u32p, f64p]
        L.or_gumbel_n.restype = None
        L.or_hlg_g_n.argtypes = [C.c_int64, f64p, C.c_double, C.c_double, C.c_double,
                                 C.c_double, f64p]
        L.or_hlg_g_n.restype = None
        L.or_logsumexp.argtypes = [f64p, C.c_int64, C.c_int64, C.c_int64, f64p]
        L.or_logsumexp.restype = C.c_int
        L.or_hlg_transform.argtypes = [f64p, C.c_int64, C.c_int64, C.c_int64, f32p,
                                       C.c_float, C.c_float, C.c_float, C.c_float,
                                       C.c_int, C.c_float, f64p, C.c_int64]
        L.or_hlg_transform.restype = C.c_int
        L.or_pivot.argtypes = [f64p, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_double,
                               C.c_void_p, f64p]
        L.or_pivot.restype = C.c_int
        L.or_sample.argtypes = [f64p, C.c_int64, C.c_int64, C.c_int64, i64p, f32p, f32p,
                                C.c_int, C.c_float, C.c_float, C.c_float, C.c_float,
                                C.c_int, C.c_float, u64p, u64p, C.c_int32, i32p, f64p, f64p,
                                C.c_int]
        L.or_sample.restype = C.c_int
        L.or_filter_tau.argtypes = [f64p, C.c_int64, C.c_int64, C.c_int64, f32p, i32p, f32p,
                                    f64p, i32p]
        L.or_filter_tau.restype = C.c_int
        L.or_sample_filtered.argtypes = [f64p, C.c_int64, C.c_int64, C.c_int64, i64p, f32p,
                                         i32p, f32p, u64p, u64p, C.c_int32, i32p, f64p, f64p,
                                         f64p, i32p, C.c_int]
        L.or_sample_filtered.restype = C.c_int
        _lib = L
    return _lib


class OracleError(ValueError):
    pass


def _as_f64_rows(x) -> np.ndarray:
    """Logits (torch tensor of any float dtype, or numpy) -> C-contiguous float64 [n, V].
    bf16/f16/f32 -> f64 is exact."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").double().numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if x.ndim == 1:
        x = x[None, :]
    return x


def set_threads(n: int) -> None:
    os.environ["OMP_NUM_THREADS"] = str(int(n))


def philox4x32_10(ctr, key) -> np.ndarray:
    ctr = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(-1, 4))
    key = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(-1, 2))
    assert ctr.shape[0] == key.shape[0]
    out = np.zeros_like(ctr)
    lib().or_philox4x32_10_n(ctr.shape[0], ctr, key, out)
    return out


# Word layouts of the random stream: "plain" (element i takes word i & 3 of the call at
# counter word i >> 2) and "screened" (the 16-bit halves of the calls at 2q and 2q + 1,
# q = i >> 3, make the high and low halves of element i's word).
LAYOUTS = {"plain": 0, "screened": 1}


def _layout(layout) -> int:
    return LAYOUTS[layout] if isinstance(layout, str) else int(layout)


def element_word(seed: int, row: int, off: int, i: int, layout="plain") -> int:
    return int(lib().or_element_word_layout(seed, row, off, i, _layout(layout)))


def stream_words(seed: int, row: int, off: int, V: int, layout="plain") -> np.ndarray:
    out = np.zeros(V, dtype=np.uint32)
    lib().or_stream_words_layout(int(seed) & (2**64 - 1), int(row), int(off) & (2**64 - 1), V,
                                 _layout(layout), out)
    return out


def gumbel(r) -> np.ndarray:
    r = np.ascontiguousarray(np.asarray(r, dtype=np.uint32).ravel())
    out = np.zeros(r.shape[0], dtype=np.float64)
    lib().or_gumbel_n(r.shape[0], r, out)
    return out


def hlg_g(z, m, w, beta_t, beta_h) -> np.ndarray:
    z = np.ascontiguousarray(np.asarray(z, dtype=np.float64).ravel())
    out = np.zeros_like(z)
    lib().or_hlg_g_n(z.shape[0], z, float(m), float(w), float(beta_t), float(beta_h), out)
    return out


def logsumexp(x) -> np.ndarray:
    x = _as_f64_rows(x)
    n, V = x.shape
    out = np.zeros(n, dtype=np.float64)
    if lib().or_logsumexp(x, n, V, V, out) != 0:
        raise OracleError("NaN or +inf logit")
    return out


# Pivot modes of the curve [HLG, The pivot]: the pivot given per row, top-anchored
# (mu = l_max - c), entropy-anchored (mu = sum p l) or the mass median (the log-prob at which
# the mass summed from the top first reaches one half).
PIVOTS = {"input": 0, "top": 1, "entropy": 2, "median": 3}


def _pivot_mode(p) -> int:
    return PIVOTS[p] if isinstance(p, str) else int(p)


def pivot(x, mode, offset: float = 0.0, mu=None) -> np.ndarray:
    """The pivot mu of every row (float64), NaN for a row with no finite logit."""
    x = _as_f64_rows(x)
    n, V = x.shape
    out = np.zeros(n, dtype=np.float64)
    mu_a = None if mu is None else np.ascontiguousarray(np.asarray(mu, dtype=np.float32).reshape(n))
    rc = lib().or_pivot(x, n, V, V, _pivot_mode(mode), float(offset),
                        None if mu_a is None else mu_a.ctypes.data, out)
    if rc == -2:
        raise OracleError("invalid pivot mode or offset")
    if rc != 0:
        raise OracleError("NaN or +inf logit")
    return out


def hlg_transform(x, mu, m, w, beta_t, beta_h, pivot="input", pivot_offset=0.0) -> np.ndarray:
    x = _as_f64_rows(x)
    n, V = x.shape
    mu = np.ascontiguousarray(np.asarray(0.0 if mu is None else mu, dtype=np.float32)
                              * np.ones(n, dtype=np.float32))
    out = np.zeros((n, V), dtype=np.float64)
    rc = lib().or_hlg_transform(x, n, V, V, mu, m, w, beta_t, beta_h, _pivot_mode(pivot),
                                float(pivot_offset), out, V)
    if rc == -2:
        raise OracleError("invalid curve parameters")
    if rc != 0:
        raise OracleError("NaN or +inf logit")
    return out


def sample(x, T, seed, offset, K: int = 1, mu=None, hlg=None, row_id=None, layout="plain"):
    """Token ids [n, K] plus the best and second-best score of every draw.

    hlg: None (curve off) or a mapping/tuple (m, w, beta_t, beta_h); a mapping may also
    carry "pivot" ("input", "top", "entropy", "median") and "pivot_offset" (the c of the top
    mode).
    row_id: the global row index keying each row's Philox counter (default 0..n-1).
    layout: the word layout of the random stream ("plain" or "screened")."""
    x = _as_f64_rows(x)
    n, V = x.shape
    T = np.ascontiguousarray(np.asarray(T, dtype=np.float32).reshape(n))
    seed = np.ascontiguousarray(np.asarray(seed, dtype=np.uint64).reshape(n))
    offset = np.ascontiguousarray(np.asarray(offset, dtype=np.uint64).reshape(n))
    rid = np.arange(n, dtype=np.int64) if row_id is None else \
        np.ascontiguousarray(np.asarray(row_id, dtype=np.int64).reshape(n))
    piv, poff = 0, 0.0
    if hlg is None:
        on, p = 0, (1.0, 0.0, 1.0, 1.0)
        mu_a = np.zeros(n, dtype=np.float32)
    else:
        on = 1
        if isinstance(hlg, dict):
            p = tuple(hlg[k] for k in ("m", "w", "beta_t", "beta_h"))
            piv = _pivot_mode(hlg.get("pivot", 0))
            poff = float(hlg.get("pivot_offset", 0.0))
        else:
            p = tuple(hlg)
        mu_a = np.zeros(n, dtype=np.float32) if (mu is None and piv != 0) else \
            np.ascontiguousarray(np.asarray(mu, dtype=np.float32).reshape(n))
    out = np.zeros((n, K), dtype=np.int32)
    best = np.zeros((n, K), dtype=np.float64)
    second = np.zeros((n, K), dtype=np.float64)
    rc = lib().or_sample(x, n, V, V, rid, T, mu_a, on, p[0], p[1], p[2], p[3], piv, poff,
                         seed, offset, int(K), out, best, second, _layout(layout))
    if rc == -2:
        raise OracleError("invalid curve parameters or layout")
    if rc != 0:
        raise OracleError("NaN or +inf logit")
    return out, best, second


# Top-k / top-p on the Gumbel path, curve off (see or_filter_tau in hs_oracle.c for the
# reading): every token with a logit at or above the row's threshold tau is kept.
def _filter_args(n, T, top_k, top_p):
    T = np.ascontiguousarray(np.asarray(T, dtype=np.float32).reshape(n))
    k = np.zeros(n, dtype=np.int32) if top_k is None else \
        np.ascontiguousarray(np.broadcast_to(np.asarray(top_k, dtype=np.int32), (n,)))
    p = np.ones(n, dtype=np.float32) if top_p is None else \
        np.ascontiguousarray(np.broadcast_to(np.asarray(top_p, dtype=np.float32), (n,)))
    return T, k, p


def filter_threshold(x, T, top_k=None, top_p=None):
    """(tau [n] float64, amb [n] bool): the kept set of row r is {i : x_ri >= tau_r}; tau is
    -inf when nothing is filtered and NaN for an invalid T or p; amb marks rows whose top-p
    crossing lies within 1e-5 of the mass target (an fp32 computation may take a neighbour)."""
    x = _as_f64_rows(x)
    n, V = x.shape
    T, k, p = _filter_args(n, T, top_k, top_p)
    tau = np.zeros(n, dtype=np.float64)
    amb = np.zeros(n, dtype=np.int32)
    if lib().or_filter_tau(x, n, V, V, T, k, p, tau, amb) != 0:
        raise OracleError("NaN or +inf logit")
    return tau, amb.astype(bool)


def sample_filtered(x, T, seed, offset, K: int = 1, top_k=None, top_p=None, row_id=None,
                    layout="plain"):
    """Gumbel-max draws over the tokens top-k / top-p keep (curve off): ids [n, K], the best and
    second-best scores, and the threshold and ambiguity flag of every row."""
    x = _as_f64_rows(x)
    n, V = x.shape
    T, k, p = _filter_args(n, T, top_k, top_p)
    seed = np.ascontiguousarray(np.asarray(seed, dtype=np.uint64).reshape(n))
    offset = np.ascontiguousarray(np.asarray(offset, dtype=np.uint64).reshape(n))
    rid = np.arange(n, dtype=np.int64) if row_id is None else \
        np.ascontiguousarray(np.asarray(row_id, dtype=np.int64).reshape(n))
    out = np.zeros((n, K), dtype=np.int32)
    best = np.zeros((n, K), dtype=np.float64)
    second = np.zeros((n, K), dtype=np.float64)
    tau = np.zeros(n, dtype=np.float64)
    amb = np.zeros(n, dtype=np.int32)
    rc = lib().or_sample_filtered(x, n, V, V, rid, T, k, p, seed, offset, int(K), out, best,
                                  second, tau, amb, _layout(layout))
    if rc == -2:
        raise OracleError("invalid layout")
    if rc != 0:
        raise OracleError("NaN or +inf logit")
    return out, best, second, tau, amb.astype(bool)

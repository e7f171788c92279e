"""Python binding of libhs: batched HLG tone-curve + Gumbel-max token sampling on MI355X.

Argument marshalling only. Every step of the sampling path runs in the HIP kernels of
``libhs.so`` (built in-tree by ``logit_transform_amd/build.py``); PyTorch provides device
memory and the current stream. There is no CPU fallback: if the library is missing, or no
GPU is present, the calls raise.

Sources: "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document) and
"Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (mlxcel issue #900).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Mapping, Optional, Sequence, Union

import torch

__all__ = [
    "HsError", "HlgParams", "SampleOpts", "load", "library_path", "EXPORTED_SYMBOLS",
    "sample", "sample_ex", "sample_rows", "hlg_rows", "sample_filtered", "filter_threshold",
    "gumbel_argmax", "logsumexp",
    "hlg_transform", "hlg_pivot",
    "workspace_bytes", "PIVOTS",
    "workspace", "philox4x32_10", "stream_words", "gumbel_f32", "version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# HS_LIBRARY: another build of the same sources (the host-only sanitized one, for CPU checks)
_LIB_PATH = os.environ.get("HS_LIBRARY") or os.path.join(_HERE, "libhs.so")

HS_F32, HS_BF16, HS_F16 = 0, 1, 2
_DTYPES = {torch.float32: HS_F32, torch.bfloat16: HS_BF16, torch.float16: HS_F16}

EXPORTED_SYMBOLS = (
    "hs_logsumexp", "hs_hlg_transform", "hs_hlg_pivot", "hs_gumbel_argmax", "hs_sample",
    "hs_sample_ex", "hs_sample_rows", "hs_filter_threshold", "hs_sample_filtered",
    "hs_workspace_bytes", "hs_workspace_init", "hs_sample_plan", "hs_philox4x32_10", "hs_stream_words",
    "hs_stream_words_ex", "hs_gumbel_f32", "hs_status_str", "hs_version", "hs_sample_noalloc",
    "hs_sample_noalloc_max_workspace",
)
# word layouts of the random stream (hs_layout)
LAYOUTS = {"plain": 0, "screened": 1}


class HsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib_status(status) if _lib is not None else str(status)
        super().__init__("%s: %s" % (where, msg))


class _Logits(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("B", C.c_int64),
                ("V", C.c_int64), ("ld", C.c_int64)]


class HlgParams(C.Structure):
    """Curve knobs in nats: mid gain m, mid half-width w (+inf = rolloff off), toe and
    shoulder rolloff constants beta_t, beta_h; the pivot mode (PIVOTS) and the top anchor's
    offset c."""
    _fields_ = [("m", C.c_float), ("w", C.c_float), ("beta_t", C.c_float),
                ("beta_h", C.c_float), ("pivot", C.c_int32), ("pivot_offset", C.c_float)]


class HlgRow(C.Structure):
    """One row's curve setting for sample_rows (32 bytes, device array of B)."""
    _fields_ = [("m", C.c_float), ("w", C.c_float), ("beta_t", C.c_float),
                ("beta_h", C.c_float), ("pivot", C.c_int32), ("pivot_offset", C.c_float),
                ("enabled", C.c_int32), ("reserved", C.c_int32)]


# Where the curve's pivot comes from: given per row (mu), top-anchored (mu = l_max - c),
# entropy-anchored (mu = sum p l).
PIVOTS = {"input": 0, "top": 1, "entropy": 2, "median": 3}


def _pivot_mode(p) -> int:
    if isinstance(p, str):
        if p not in PIVOTS:
            raise ValueError("unknown pivot mode %r" % (p,))
        return PIVOTS[p]
    return int(p)


class SampleOpts(C.Structure):
    """Kernel choices for sample_ex: variant 0 auto / 1 one block per row / 2 split rows;
    nchunk blocks per split row (0 auto); no_screen 1 = score every element exactly;
    draw_groups blocks sharing one row's draws (0 auto); split_lse for split rows with the
    curve on: 0 auto / 1 log-sum-exp pre-pass / 2 partials exchanged inside the kernel;
    exchange_wait polls for the other chunks' partials (0 default, -1 none); median_rows (per-row
    settings only) 1 = some row may ask for the mass-median pivot; layout the word layout of
    the random stream (0 plain, 1 screened)."""
    _fields_ = [("variant", C.c_int32), ("nchunk", C.c_int32), ("no_screen", C.c_int32),
                ("draw_groups", C.c_int32), ("split_lse", C.c_int32),
                ("exchange_wait", C.c_int32), ("median_rows", C.c_int32),
                ("layout", C.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> C.CDLL:
    """Load libhs.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libhs.so is not built: run `python -c 'import __graft_entry__ as g; "
                          "g.build()'` or `python logit_transform_amd/build.py`")
    L = C.CDLL(_LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    LP = C.POINTER(_Logits)
    HP = C.POINTER(HlgParams)
    OP = C.POINTER(SampleOpts)
    L.hs_logsumexp.argtypes = [LP, vp, vp]
    L.hs_hlg_transform.argtypes = [LP, vp, HP, vp, i64, vp]
    L.hs_hlg_pivot.argtypes = [LP, vp, HP, vp, vp]
    L.hs_gumbel_argmax.argtypes = [LP, vp, vp, vp, i32, vp, vp, sz, vp]
    L.hs_sample.argtypes = [LP, vp, vp, HP, vp, vp, i32, vp, vp, sz, vp]
    L.hs_sample_ex.argtypes = [LP, vp, vp, HP, vp, vp, i32, vp, vp, vp, sz, OP, vp]
    L.hs_sample_noalloc.argtypes = [LP, vp, vp, HP, vp, vp, i32, vp, vp, OP, vp]
    L.hs_sample_noalloc_max_workspace.argtypes = []
    L.hs_sample_noalloc_max_workspace.restype = sz
    L.hs_sample_rows.argtypes = [LP, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, OP, vp]
    L.hs_filter_threshold.argtypes = [LP, vp, vp, vp, vp, vp]
    L.hs_sample_filtered.argtypes = [LP, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, OP, vp]
    L.hs_workspace_bytes.argtypes = [i64, i64, i32, i32, i32]
    L.hs_workspace_bytes.restype = sz
    L.hs_workspace_init.argtypes = [vp, sz, vp]
    L.hs_sample_plan.argtypes = [LP, i32, i32, i32, OP, C.POINTER(C.c_int64)]
    L.hs_sample_plan.restype = C.c_int
    L.hs_philox4x32_10.argtypes = [vp, vp, vp, i64, vp]
    L.hs_stream_words.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    L.hs_stream_words_ex.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp]
    L.hs_gumbel_f32.argtypes = [vp, vp, i64, vp]
    L.hs_status_str.argtypes = [C.c_int]
    L.hs_status_str.restype = C.c_char_p
    L.hs_version.argtypes = []
    L.hs_version.restype = C.c_char_p
    for name in ("hs_logsumexp", "hs_hlg_transform", "hs_hlg_pivot", "hs_gumbel_argmax", "hs_sample",
                 "hs_sample_ex", "hs_sample_rows", "hs_filter_threshold", "hs_sample_filtered",
                 "hs_workspace_init", "hs_philox4x32_10", "hs_stream_words",
                 "hs_stream_words_ex", "hs_gumbel_f32", "hs_sample_noalloc"):
        getattr(L, name).restype = C.c_int
    _lib = L
    return L


def _lib_status(status: int) -> str:
    return load().hs_status_str(int(status)).decode()


def version() -> str:
    return load().hs_version().decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise HsError(status, where)


def _stream(device: torch.device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require_gpu(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (no CPU path exists)" % name)


def _logits_struct(x: torch.Tensor) -> _Logits:
    _require_gpu(x, "logits")
    if x.dim() != 2:
        raise ValueError("logits must be 2-D [B, V]")
    if x.dtype not in _DTYPES:
        raise ValueError("logits dtype must be float32, bfloat16 or float16")
    if x.stride(1) != 1:
        raise ValueError("logits rows must be contiguous (stride(1) == 1)")
    ld = x.stride(0) if x.shape[0] > 1 else max(x.stride(0), x.shape[1])
    return _Logits(x.data_ptr(), _DTYPES[x.dtype], x.shape[0], x.shape[1], ld)


def _row_vec(v, B: int, dtype: torch.dtype, device, name: str) -> torch.Tensor:
    if isinstance(v, torch.Tensor):
        t = v
        if t.device.type != "cuda":
            t = t.to(device)
    else:
        import numpy as np
        arr = np.asarray(v)
        if dtype == torch.int64 and arr.dtype == np.uint64:
            arr = arr.view(np.int64)
        t = torch.as_tensor(arr).to(device)
    if dtype == torch.int64 and t.dtype == torch.uint64:
        t = t.view(torch.int64)
    if t.dtype != dtype:
        t = t.to(dtype)
    t = t.reshape(-1)
    if t.numel() == 1 and B > 1:   # one value for every row
        t = t.expand(B)
    t = t.contiguous()
    if t.numel() != B:
        raise ValueError("%s must have B=%d entries (or one for every row)" % (name, B))
    return t


def _hlg_struct(hlg) -> Optional[HlgParams]:
    if hlg is None:
        return None
    if isinstance(hlg, HlgParams):
        return hlg
    if isinstance(hlg, Mapping):
        return HlgParams(float(hlg["m"]), float(hlg["w"]), float(hlg["beta_t"]),
                         float(hlg["beta_h"]), _pivot_mode(hlg.get("pivot", 0)),
                         float(hlg.get("pivot_offset", 0.0)))
    m, w, bt, bh = hlg[:4]
    piv = _pivot_mode(hlg[4]) if len(hlg) > 4 else 0
    off = float(hlg[5]) if len(hlg) > 5 else 0.0
    return HlgParams(float(m), float(w), float(bt), float(bh), piv, off)


def _mu_vec(mu, hp, B, dev):
    """The per-row pivot, needed only when the curve is on with a given pivot."""
    if hp is None:
        return None
    if hp.pivot == 0 and mu is None:
        raise ValueError("mu is required with the curve on and the pivot given")
    return _row_vec(mu, B, torch.float32, dev, "mu") if (mu is not None and hp.pivot == 0) else None


def sample_plan(B: int, V: int, K: int, dtype: torch.dtype, hlg_on: bool,
                have_ws: bool = True, opts: Optional[SampleOpts] = None) -> dict:
    """The launch plan the library picks for a shape (no device needed: 256 CUs assumed when
    none is visible)."""
    L = load()
    x = _Logits(0x10000, _DTYPES[dtype], int(B), int(V), int(V))   # never dereferenced
    out = (C.c_int64 * 8)()
    _check(L.hs_sample_plan(C.byref(x), int(K), 1 if hlg_on else 0, 1 if have_ws else 0,
                            C.byref(opts) if opts is not None else None, out), "hs_sample_plan")
    keys = ("nchunk", "cv", "bs", "nv", "draw_groups", "draws_per_group", "grid", "cus")
    return dict(zip(keys, list(out)))


def workspace_bytes(B: int, V: int, K: int, dtype: torch.dtype, hlg_on: bool) -> int:
    return int(load().hs_workspace_bytes(B, V, K, _DTYPES[dtype], 1 if hlg_on else 0))


def workspace(B: int, V: int, K: int, dtype: torch.dtype, hlg_on: bool,
              device=None) -> torch.Tensor:
    """A zero-filled workspace for hs_sample / hs_gumbel_argmax of this shape."""
    n = workspace_bytes(B, V, K, dtype, hlg_on)
    device = torch.device(device or "cuda")
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    _check(load().hs_workspace_init(ws.data_ptr(), ws.numel(), _stream(device)),
           "hs_workspace_init")
    return ws


def sample_ex(logits: torch.Tensor, T, seed, offset, *, mu=None, hlg=None, k: int = 1,
              out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
              opts: Optional[SampleOpts] = None, want_best: bool = False):
    """Token ids [B, k] (int32) and, with want_best, the winning scores [B, k] (float32)."""
    L = load()
    x = _logits_struct(logits)
    dev = logits.device
    B = logits.shape[0]
    Tt = _row_vec(T, B, torch.float32, dev, "T")
    st = _row_vec(seed, B, torch.int64, dev, "seed")
    of = _row_vec(offset, B, torch.int64, dev, "offset")
    hp = _hlg_struct(hlg)
    mut = _mu_vec(mu, hp, B, dev)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=dev)
    best = torch.empty((B, k), dtype=torch.float32, device=dev) if want_best else None
    if ws is None:
        ws = workspace(B, logits.shape[1], k, logits.dtype, hp is not None, dev)
    rc = L.hs_sample_ex(C.byref(x), Tt.data_ptr(), _ptr(mut), C.byref(hp) if hp is not None else None,
                        st.data_ptr(), of.data_ptr(), int(k), out.data_ptr(), _ptr(best),
                        ws.data_ptr(), ws.numel(), C.byref(opts) if opts is not None else None,
                        _stream(dev))
    _check(rc, "hs_sample_ex")
    return (out, best) if want_best else out


def sample_noalloc(logits: torch.Tensor, T, seed, offset, *, mu=None, hlg=None, k: int = 1,
                   out: Optional[torch.Tensor] = None, opts: Optional[SampleOpts] = None,
                   want_best: bool = False):
    """sample_ex with the library's static workspace (hs_sample_noalloc): the library allocates
    nothing. out (and the scores, with want_best) are allocated here unless out is given."""
    L = load()
    x = _logits_struct(logits)
    dev = logits.device
    B = logits.shape[0]
    Tt = _row_vec(T, B, torch.float32, dev, "T")
    st = _row_vec(seed, B, torch.int64, dev, "seed")
    of = _row_vec(offset, B, torch.int64, dev, "offset")
    hp = _hlg_struct(hlg)
    mut = _mu_vec(mu, hp, B, dev)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=dev)
    best = torch.empty((B, k), dtype=torch.float32, device=dev) if want_best else None
    rc = L.hs_sample_noalloc(C.byref(x), Tt.data_ptr(), _ptr(mut),
                             C.byref(hp) if hp is not None else None, st.data_ptr(),
                             of.data_ptr(), int(k), out.data_ptr(), _ptr(best),
                             C.byref(opts) if opts is not None else None, _stream(dev))
    _check(rc, "hs_sample_noalloc")
    return (out, best) if want_best else out


def sample(logits: torch.Tensor, T, seed, offset, *, mu=None, hlg=None, k: int = 1,
           out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The sampling step: token ids [B, k] (int32) on logits' device, asynchronously on the
    current stream. hlg=None turns the curve off; otherwise hlg = (m, w, beta_t, beta_h
    [, pivot, pivot_offset]) or a mapping with those keys, and mu is the per-row pivot when
    the pivot mode is "input" (the default; "top", "entropy" and "median" derive it on the GPU). Rows give -1 when no logit is
    finite and -2 for an invalid temperature or pivot; T = 0 is greedy."""
    L = load()
    x = _logits_struct(logits)
    dev = logits.device
    B = logits.shape[0]
    Tt = _row_vec(T, B, torch.float32, dev, "T")
    st = _row_vec(seed, B, torch.int64, dev, "seed")
    of = _row_vec(offset, B, torch.int64, dev, "offset")
    hp = _hlg_struct(hlg)
    mut = _mu_vec(mu, hp, B, dev)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(B, logits.shape[1], k, logits.dtype, hp is not None, dev)
    rc = L.hs_sample(C.byref(x), Tt.data_ptr(), _ptr(mut), C.byref(hp) if hp is not None else None,
                     st.data_ptr(), of.data_ptr(), int(k), out.data_ptr(), ws.data_ptr(),
                     ws.numel(), _stream(dev))
    _check(rc, "hs_sample")
    return out


def hlg_rows(settings: Sequence, device=None) -> torch.Tensor:
    """Packs per-row curve settings for sample_rows into a device tensor (uint8 [B, 32]).
    Each entry is None (curve off for the row) or what `hlg` accepts elsewhere: a mapping with
    m, w, beta_t, beta_h and optionally pivot, pivot_offset, or a tuple
    (m, w, beta_t, beta_h[, pivot, pivot_offset])."""
    raw = torch.frombuffer(bytearray(bytes(_pack_rows(settings))), dtype=torch.uint8)
    return raw.reshape(len(settings), 32).to(torch.device(device or "cuda"))


def _pack_rows(settings: Sequence):
    arr = (HlgRow * len(settings))()
    for i, h in enumerate(settings):
        if h is None:
            arr[i] = HlgRow(1.0, 0.0, 1.0, 1.0, 0, 0.0, 0, 0)
        else:
            p = _hlg_struct(h)
            arr[i] = HlgRow(p.m, p.w, p.beta_t, p.beta_h, p.pivot, p.pivot_offset, 1, 0)
    return arr


def sample_rows(logits: torch.Tensor, T, seed, offset, rows, *, mu=None, k: int = 1,
                out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                opts: Optional[SampleOpts] = None, want_best: bool = False):
    """The sampling step with the curve set per row: rows is a device tensor from hlg_rows (or
    a sequence it accepts). mu [B] is read only for rows whose curve is on with the pivot given
    (it may be None otherwise: such rows then give -2). Ids [B, k] (int32) and, with
    want_best, the winning scores."""
    L = load()
    x = _logits_struct(logits)
    dev = logits.device
    B = logits.shape[0]
    if not isinstance(rows, torch.Tensor):
        rows = hlg_rows(rows, dev)
    _require_gpu(rows, "rows")
    if rows.dtype != torch.uint8 or tuple(rows.shape) != (B, 32) or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous uint8 [B, 32] tensor (see hlg_rows)")
    Tt = _row_vec(T, B, torch.float32, dev, "T")
    st = _row_vec(seed, B, torch.int64, dev, "seed")
    of = _row_vec(offset, B, torch.int64, dev, "offset")
    mut = _row_vec(mu, B, torch.float32, dev, "mu") if mu is not None else None
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=dev)
    best = torch.empty((B, k), dtype=torch.float32, device=dev) if want_best else None
    if ws is None:
        ws = workspace(B, logits.shape[1], k, logits.dtype, True, dev)
    rc = L.hs_sample_rows(C.byref(x), Tt.data_ptr(), _ptr(mut), rows.data_ptr(), st.data_ptr(),
                          of.data_ptr(), int(k), out.data_ptr(), _ptr(best), ws.data_ptr(),
                          ws.numel(), C.byref(opts) if opts is not None else None, _stream(dev))
    _check(rc, "hs_sample_rows")
    return (out, best) if want_best else out


def _filter_vecs(top_k, top_p, B, dev):
    kt = _row_vec(top_k, B, torch.int32, dev, "top_k") if top_k is not None else None
    pt = _row_vec(top_p, B, torch.float32, dev, "top_p") if top_p is not None else None
    return kt, pt


def filter_threshold(logits: torch.Tensor, T, top_k=None, top_p=None) -> torch.Tensor:
    """The top-k / top-p threshold tau [B] (float32) of every row, curve off: a row keeps the
    tokens with logit >= tau; -inf keeps all, NaN marks an invalid T or top_p."""
    L = load()
    x = _logits_struct(logits)
    dev = logits.device
    B = logits.shape[0]
    Tt = _row_vec(T, B, torch.float32, dev, "T")
    kt, pt = _filter_vecs(top_k, top_p, B, dev)
    tau = torch.empty(B, dtype=torch.float32, device=dev)
    _check(L.hs_filter_threshold(C.byref(x), Tt.data_ptr(), _ptr(kt), _ptr(pt), tau.data_ptr(),
                                 _stream(dev)), "hs_filter_threshold")
    return tau


def sample_filtered(logits: torch.Tensor, T, seed, offset, *, top_k=None, top_p=None,
                    k: int = 1, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, opts: Optional[SampleOpts] = None,
                    want_best: bool = False):
    """Gumbel-max draws over the tokens top-k / top-p keep (curve off): ids [B, k] (int32)
    and, with want_best, the winning scores. top_k (int, per row) <= 0 and top_p >= 1 turn a
    filter off; rows with an invalid T or top_p give -2."""
    L = load()
    x = _logits_struct(logits)
    dev = logits.device
    B = logits.shape[0]
    Tt = _row_vec(T, B, torch.float32, dev, "T")
    st = _row_vec(seed, B, torch.int64, dev, "seed")
    of = _row_vec(offset, B, torch.int64, dev, "offset")
    kt, pt = _filter_vecs(top_k, top_p, B, dev)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=dev)
    best = torch.empty((B, k), dtype=torch.float32, device=dev) if want_best else None
    if ws is None:
        ws = workspace(B, logits.shape[1], k, logits.dtype, False, dev)
    rc = L.hs_sample_filtered(C.byref(x), Tt.data_ptr(), _ptr(kt), _ptr(pt), st.data_ptr(),
                              of.data_ptr(), int(k), out.data_ptr(), _ptr(best), ws.data_ptr(),
                              ws.numel(), C.byref(opts) if opts is not None else None,
                              _stream(dev))
    _check(rc, "hs_sample_filtered")
    return (out, best) if want_best else out


def gumbel_argmax(logits: torch.Tensor, T, seed, offset, *, k: int = 1,
                  out: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gumbel-max draws with the curve off: token ids [B, k] (int32)."""
    L = load()
    x = _logits_struct(logits)
    dev = logits.device
    B = logits.shape[0]
    Tt = _row_vec(T, B, torch.float32, dev, "T")
    st = _row_vec(seed, B, torch.int64, dev, "seed")
    of = _row_vec(offset, B, torch.int64, dev, "offset")
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(B, logits.shape[1], k, logits.dtype, False, dev)
    rc = L.hs_gumbel_argmax(C.byref(x), Tt.data_ptr(), st.data_ptr(), of.data_ptr(), int(k),
                            out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _check(rc, "hs_gumbel_argmax")
    return out


def logsumexp(logits: torch.Tensor) -> torch.Tensor:
    L = load()
    x = _logits_struct(logits)
    out = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    _check(L.hs_logsumexp(C.byref(x), out.data_ptr(), _stream(logits.device)), "hs_logsumexp")
    return out


def hlg_transform(logits: torch.Tensor, mu, hlg) -> torch.Tensor:
    """l' = g(log-softmax(x) - mu) as float32 [B, V] (before any temperature); mu is read
    only with the pivot given (mode "input")."""
    L = load()
    x = _logits_struct(logits)
    B, V = logits.shape
    hp = _hlg_struct(hlg)
    mut = _mu_vec(mu, hp, B, logits.device)
    out = torch.empty((B, V), dtype=torch.float32, device=logits.device)
    _check(L.hs_hlg_transform(C.byref(x), _ptr(mut), C.byref(hp), out.data_ptr(), V,
                              _stream(logits.device)), "hs_hlg_transform")
    return out


def hlg_pivot(logits: torch.Tensor, hlg, mu=None) -> torch.Tensor:
    """The pivot mu [B] (float32, log-prob nats) the curve uses in hlg's pivot mode; NaN for
    a row with no finite logit."""
    L = load()
    x = _logits_struct(logits)
    B = logits.shape[0]
    hp = _hlg_struct(hlg)
    mut = _mu_vec(mu, hp, B, logits.device)
    out = torch.empty(B, dtype=torch.float32, device=logits.device)
    _check(L.hs_hlg_pivot(C.byref(x), _ptr(mut), C.byref(hp), out.data_ptr(),
                          _stream(logits.device)), "hs_hlg_pivot")
    return out


def philox4x32_10(ctr: torch.Tensor, key: torch.Tensor) -> torch.Tensor:
    """ctr int32 [n, 4], key int32 [n, 2] (bit patterns of uint32) -> int32 [n, 4]."""
    L = load()
    _require_gpu(ctr, "ctr")
    ctr = ctr.contiguous().view(torch.int32)
    key = key.to(ctr.device).contiguous().view(torch.int32)
    n = ctr.numel() // 4
    if key.numel() != 2 * n:
        raise ValueError("key must hold 2 words per counter")
    out = torch.empty((n, 4), dtype=torch.int32, device=ctr.device)
    _check(L.hs_philox4x32_10(ctr.data_ptr(), key.data_ptr(), out.data_ptr(), n,
                              _stream(ctr.device)), "hs_philox4x32_10")
    return out


def stream_words(seed, offset, B: int, V: int, k: int = 0, device="cuda",
                 layout="plain") -> torch.Tensor:
    """The samplers' random words for draw k in a word layout ("plain" or "screened"): int32
    [B, V] (uint32 bit patterns)."""
    L = load()
    dev = torch.device(device)
    st = _row_vec(seed, B, torch.int64, dev, "seed")
    of = _row_vec(offset, B, torch.int64, dev, "offset")
    out = torch.empty((B, V), dtype=torch.int32, device=dev)
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    _check(L.hs_stream_words_ex(st.data_ptr(), of.data_ptr(), B, V, int(k), lay,
                                out.data_ptr(), _stream(dev)), "hs_stream_words_ex")
    return out


def gumbel_f32(words: torch.Tensor) -> torch.Tensor:
    """The samplers' fp32 Gumbel map on uint32 words held in an int32 tensor."""
    L = load()
    _require_gpu(words, "words")
    w = words.contiguous().view(torch.int32)
    g = torch.empty(w.shape, dtype=torch.float32, device=w.device)
    _check(L.hs_gumbel_f32(w.data_ptr(), g.data_ptr(), w.numel(), _stream(w.device)),
           "hs_gumbel_f32")
    return g

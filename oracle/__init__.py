"""ctypes front of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library; the two meet only in the input arrays.

All array arguments are numpy float64 (inputs are copied to C-contiguous
float64 if they are not already); outputs are freshly allocated numpy arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB_OVERRIDE lets the mutation test run the pins against a deliberately broken build.
_LIB_PATH = os.environ.get("ORACLE_LIB_OVERRIDE") or os.path.join(_HERE, "liboracle.so")
_lib = None
_override = None  # a ctypes library to use instead of the built one (mutation tests)

_dp = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def _declare(lib):
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [_i64] * 6 + [_dp] * 3 + [
        ctypes.c_int, _i64, ctypes.c_double, ctypes.c_double, _i64, _i64, _u8p,
        _dp, _u8p, _dp, _i64p, ctypes.c_int]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [_i64] * 6 + [_dp] * 3 + [
        _i32p, ctypes.c_double, ctypes.c_double, _i64, _i64, _i64, ctypes.c_int, _u8p,
        _dp, _u8p, _dp, _i64p, ctypes.c_int]
    lib.oracle_lambda_for_target.restype = ctypes.c_double
    lib.oracle_lambda_for_target.argtypes = [_dp, _i64, ctypes.c_double, _dp]
    lib.oracle_fit_a.restype = ctypes.c_double
    lib.oracle_fit_a.argtypes = [_dp, _i64p, _i64]
    lib.oracle_lambda_from_table.restype = ctypes.c_double
    lib.oracle_lambda_from_table.argtypes = [_dp, _dp, _i64, ctypes.c_double, _i64]
    return lib


def _load():
    global _lib
    if _override is not None:
        return _override
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # local build script
        _b.build()
    _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager: route every oracle call through the library at ``path``."""

    def __init__(self, path):
        self.lib = _declare(ctypes.CDLL(path))

    def __enter__(self):
        global _override
        self._prev, _override = _override, self.lib
        return self

    def __exit__(self, *exc):
        global _override
        _override = self._prev
        return False


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, t):
    return a.ctypes.data_as(t) if a is not None else None


def prefill(q, k, v, causal=True, scale=None, lam=0.0, tile_q=64, block_k=64,
            unit_mask=None, nthreads=0, want_maps=True, window=0):
    """Blockwise skip attention, prefill form (Lq = Lk = L).

    ``window`` > 0 (causal only): query i sees keys i - window < c <= i.

    q [B,Hq,L,d], k [B,Hkv,L,d], v [B,Hkv,L,dv].  Returns a dict with
    ``o`` [B,Hq,L,dv], ``skip`` uint8 [B,Hq,nQT,nKB] (0 executed, 1 skipped,
    255 not visited), ``gap`` float64 (same shape), ``visited``, ``skipped``.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, L, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nqt = -(-L // tile_q)
    nkb = -(-L // block_k)
    o = np.zeros((B, Hq, L, dv), np.float64)
    skip = np.full((B, Hq, nqt, nkb), 255, np.uint8) if want_maps else None
    gap = np.full((B, Hq, nqt, nkb), -np.inf, np.float64) if want_maps else None
    um = None if unit_mask is None else np.ascontiguousarray(unit_mask, dtype=np.uint8)
    cnt = np.zeros(2, np.int64)
    rc = lib.oracle_prefill(B, Hq, Hkv, L, d, dv, _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp),
                            int(bool(causal)), int(window), float(scale), float(lam), tile_q, block_k,
                            _ptr(um, _u8p), _ptr(o, _dp), _ptr(skip, _u8p), _ptr(gap, _dp),
                            _ptr(cnt, _i64p), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_prefill failed with code {rc}")
    return {"o": o, "skip": skip, "gap": gap, "visited": int(cnt[0]), "skipped": int(cnt[1])}


def decode(q, k, v, seq_lens, scale=None, lam=0.0, block_k=64, num_splits=1,
           unit_mask=None, nthreads=0, want_maps=True, window=0, sink_seed=False):
    """Blockwise skip attention, decode form (one query token per sequence).

    ``window`` > 0: the query (at position seq_len-1) sees the last ``window``
    keys; the splits cut the blocks from the first one holding such a key.
    ``sink_seed``: splits after the first start their running max from the
    row maxima of the first visible block instead of -inf.

    q [B,Hq,dqk], k [B,Hkv,Lmax,dqk], v [B,Hkv,Lmax,dv], seq_lens int [B].
    Returns ``o`` [B,Hq,dv], ``skip``/``gap`` [B,Hkv,nKB], ``visited``,
    ``skipped``.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, dqk = q.shape
    Hkv, Lmax, dv = k.shape[1], k.shape[2], v.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    nkb = -(-Lmax // block_k)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    o = np.zeros((B, Hq, dv), np.float64)
    skip = np.full((B, Hkv, nkb), 255, np.uint8) if want_maps else None
    gap = np.full((B, Hkv, nkb), -np.inf, np.float64) if want_maps else None
    um = None if unit_mask is None else np.ascontiguousarray(unit_mask, dtype=np.uint8)
    cnt = np.zeros(2, np.int64)
    rc = lib.oracle_decode(B, Hq, Hkv, Lmax, dqk, dv, _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp),
                           _ptr(sl, _i32p), float(scale), float(lam), block_k, int(num_splits), int(window),
                           int(bool(sink_seed)),
                           _ptr(um, _u8p), _ptr(o, _dp), _ptr(skip, _u8p), _ptr(gap, _dp),
                           _ptr(cnt, _i64p), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_decode failed with code {rc}")
    return {"o": o, "skip": skip, "gap": gap, "visited": int(cnt[0]), "skipped": int(cnt[1])}


def gather_pages(pool, page_table, seq_lens, Lmax):
    """Contiguous per-sequence cache [B, H, Lmax, d] (float64) from a paged pool.

    The paged layout of serving engines (PagedAttention, which the BLASST
    reading notes name for end-to-end serving runs, "局限与后续工作"): row r of
    sequence b is row r mod P of pool page page_table[b, r div P], for
    pool [num_pages, H, P, d].  Rows at or past seq_lens[b] are left 0 (the
    decode never reads them).  Decode over a paged cache is defined as decode
    over this gathered cache.
    """
    pool = np.asarray(pool, dtype=np.float64)
    table = np.asarray(page_table)
    num_pages, H, P, d = pool.shape
    B = table.shape[0]
    out = np.zeros((B, H, int(Lmax), d), np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        r = np.arange(n)
        pages = table[b, r // P]
        if n and (pages.min() < 0 or pages.max() >= num_pages):
            raise ValueError(f"page table row {b} names a page outside the pool")
        out[b, :, :n, :] = pool[pages, :, r % P, :].transpose(1, 0, 2)
    return out


def lambda_for_target(gaps, target):
    """lambda whose skip set is the ceil(target*N) smallest gaps; returns (lambda, reached)."""
    lib = _load()
    g = _f64(np.asarray(gaps).ravel())
    reached = ctypes.c_double(0.0)
    lam = lib.oracle_lambda_for_target(_ptr(g, _dp), g.size, float(target), ctypes.byref(reached))
    return lam, reached.value


def fit_a(lambdas, lengths):
    """ln a = mean over lengths of ln(lambda_L * L)."""
    lib = _load()
    lam = _f64(lambdas)
    ls = np.ascontiguousarray(lengths, dtype=np.int64)
    return lib.oracle_fit_a(_ptr(lam, _dp), _ptr(ls, _i64p), lam.size)


def lambda_from_table(targets, a, target, L):
    """lambda = a(target)/L, ln a interpolated linearly in the target."""
    lib = _load()
    t, aa = _f64(targets), _f64(a)
    return lib.oracle_lambda_from_table(_ptr(t, _dp), _ptr(aa, _dp), t.size, float(target), int(L))

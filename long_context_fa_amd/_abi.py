"""ctypes marshalling for libblasst.so (mirrors include/blasst.h).

Argument marshalling only: tensors become (device pointer, dtype, strides);
the library validates, plans and launches.  Nothing here computes any part of
the attention.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libblasst.so"

BLASST_OK = 0
_BF16, _FP32 = 0, 1


class BlasstError(RuntimeError):
    """A non-OK blasst_status, with the library's message."""

    def __init__(self, status, func):
        self.status = status
        lib = load_library()
        msg = lib.blasst_last_error().decode()
        name = lib.blasst_status_str(status).decode()
        super().__init__(f"{func}: {name} ({status}): {msg}")


class _Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int),
                ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("st", ctypes.c_int64)]


class _PrefillParams(ctypes.Structure):
    _fields_ = [("q", _Tensor), ("k", _Tensor), ("v", _Tensor), ("o", _Tensor),
                ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("L", ctypes.c_int64), ("d", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("causal", ctypes.c_int), ("scale", ctypes.c_double), ("lam", ctypes.c_double),
                ("tile_q", ctypes.c_int), ("block_k", ctypes.c_int),
                ("skip_map", ctypes.c_void_p), ("gap_map", ctypes.c_void_p),
                ("counters", ctypes.c_void_p), ("window", ctypes.c_int64)]


class _DecodeParams(ctypes.Structure):
    _fields_ = [("q", _Tensor), ("k_cache", _Tensor), ("v_cache", _Tensor), ("o", _Tensor),
                ("seq_lens", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("Lmax", ctypes.c_int64), ("dqk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("scale", ctypes.c_double), ("lam", ctypes.c_double),
                ("block_k", ctypes.c_int), ("num_splits", ctypes.c_int),
                ("skip_map", ctypes.c_void_p), ("gap_map", ctypes.c_void_p),
                ("counters", ctypes.c_void_p), ("window", ctypes.c_int64), ("sink_seed", ctypes.c_int)]


class _DecodePagedParams(ctypes.Structure):
    _fields_ = [("d", _DecodeParams), ("page_table", ctypes.c_void_p),
                ("page_table_stride", ctypes.c_int64), ("num_pages", ctypes.c_int64),
                ("page_size", ctypes.c_int64)]


class _CalibTable(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("target", ctypes.POINTER(ctypes.c_double)),
                ("a", ctypes.POINTER(ctypes.c_double)), ("tile_q", ctypes.c_int), ("block_k", ctypes.c_int),
                ("num_splits", ctypes.c_int)]


_lib = None

# The parameter structs above mirror include/blasst.h at this ABI version.
ABI_VERSION = 3


def library_path():
    return os.environ.get("BLASST_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libblasst.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m long_context_fa_amd.build` "
                          "(the attention has no CPU fallback)")
    lib = ctypes.CDLL(path)
    st = ctypes.c_int
    lib.blasst_prefill.restype = st
    lib.blasst_prefill.argtypes = [ctypes.POINTER(_PrefillParams), ctypes.c_void_p]
    lib.blasst_decode_plan.restype = st
    lib.blasst_decode_plan.argtypes = [ctypes.POINTER(_DecodeParams), ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.blasst_decode.restype = st
    lib.blasst_decode.argtypes = [ctypes.POINTER(_DecodeParams), ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
    lib.blasst_decode_paged_plan.restype = st
    lib.blasst_decode_paged_plan.argtypes = [ctypes.POINTER(_DecodePagedParams), ctypes.POINTER(ctypes.c_int),
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.blasst_decode_paged.restype = st
    lib.blasst_decode_paged.argtypes = [ctypes.POINTER(_DecodePagedParams), ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
    lib.blasst_prefill_gaps.restype = st
    lib.blasst_prefill_gaps.argtypes = [ctypes.POINTER(_PrefillParams), ctypes.c_void_p]
    lib.blasst_decode_gaps.restype = st
    lib.blasst_decode_gaps.argtypes = [ctypes.POINTER(_DecodeParams), ctypes.c_void_p]
    lib.blasst_decode_noalloc.restype = st
    lib.blasst_decode_noalloc.argtypes = [ctypes.POINTER(_DecodeParams), ctypes.c_void_p]
    lib.blasst_calibrate.restype = st
    lib.blasst_calibrate.argtypes = [ctypes.POINTER(_CalibTable), ctypes.c_double, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.blasst_calibrate_search.restype = st
    lib.blasst_calibrate_search.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_double,
                                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.blasst_calibrate_fit.restype = st
    lib.blasst_calibrate_fit.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.blasst_status_str.restype = ctypes.c_char_p
    lib.blasst_status_str.argtypes = [ctypes.c_int]
    lib.blasst_last_error.restype = ctypes.c_char_p
    lib.blasst_last_error.argtypes = []
    lib.blasst_abi_version.restype = ctypes.c_int
    lib.blasst_abi_version.argtypes = []
    found = lib.blasst_abi_version()
    if found != ABI_VERSION:
        raise ImportError(f"{path} implements C ABI version {found}; this binding's structs are version "
                          f"{ABI_VERSION}: rebuild the library")
    _lib = lib
    return lib


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _FP32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _tensor(t, three_d=False):
    if t is None:
        return _Tensor(None, _BF16, 0, 0, 0)
    if t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    if three_d:
        return _Tensor(t.data_ptr(), _dtype_code(t), t.stride(0), t.stride(1), 0)
    return _Tensor(t.data_ptr(), _dtype_code(t), t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device):
    """A hipStream_t: a torch stream, a raw handle (int), or None = torch's current stream."""
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, func):
    if status != BLASST_OK:
        raise BlasstError(status, func)


# Host-side argument checks.  The library validates sizes, strides and scalars
# itself, but it receives bare pointers: it cannot see a host tensor, a tensor
# on another GPU, a K/V shorter than the query length, a map or counter buffer
# of the wrong type or size, or a length array of the wrong width.  Those are
# refused here, before any launch, with ValueError.

def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_map(t, name, dtype, numel):
    if t is None:
        return
    _need(t.dtype == dtype, f"{name} must be {dtype} (got {t.dtype})")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(t.numel() >= numel, f"{name} needs at least {numel} elements (got {t.numel()})")


def _check_counters(t):
    if t is None:
        return
    _need(t.dtype in (torch.int64, getattr(torch, "uint64", torch.int64)),
          f"counters must be a 64-bit integer tensor (got {t.dtype})")
    _need(t.is_contiguous() and t.numel() >= 2, "counters needs 2 contiguous elements (visited, skipped)")


def _check_devices(ref, **tensors):
    """Every tensor that is passed must live on the GPU of ``ref``."""
    _need(ref.is_cuda, f"tensors must be on a GPU (got {ref.device})")
    for name, t in tensors.items():
        if t is not None:
            _need(t.device == ref.device, f"{name} is on {t.device}, the query on {ref.device}")


def blasst_prefill(q, k, v, *, causal=True, lam=0.0, tile_q=128, block_k=64, scale=None, out=None,
                   out_dtype=torch.float32, skip_map=None, gap_map=None, counters=None, stream=None,
                   window=0):
    """Block-skipping prefill: q [B,Hq,L,d], k [B,Hkv,L,d], v [B,Hkv,L,dv] (bf16, device).

    ``window`` > 0 (causal): sliding window, query i sees keys i - window < c <= i.

    Returns O [B,Hq,L,dv] (``out`` if given).  Optional outputs: ``skip_map``
    uint8 and ``gap_map`` float32 of shape [B,Hq,ceil(L/tile_q),ceil(L/block_k)],
    ``counters`` uint64-compatible int64 tensor of 2 elements (visited, skipped),
    accumulated (zero it first).
    """
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k and v must be 4-D [B, H, L, d]")
    B, Hq, L, _ = q.shape
    if out is None:
        out = torch.empty(B, Hq, L, v.shape[3], dtype=out_dtype, device=q.device)
    p = _prefill_params(q, k, v, out, causal, lam, tile_q, block_k, scale, skip_map, gap_map, counters, window)
    if B > 0 and L > 0:
        _check_devices(q, k=k, v=v, out=out, skip_map=skip_map, gap_map=gap_map, counters=counters)
    _check(load_library().blasst_prefill(ctypes.byref(p), _stream(stream, q.device)), "blasst_prefill")
    return out


def blasst_prefill_gaps(q, k, v, *, causal=True, lam=0.0, tile_q=128, block_k=64, scale=None, skip_map=None,
                        gap_map=None, counters=None, stream=None, window=0):
    """The gap pass of blasst_prefill (calibration): maps and counters only, no O.

    Returns the gap map float32 [B,Hq,ceil(L/tile_q),ceil(L/block_k)] (``gap_map``
    if given, else a new one); ``skip_map`` / ``counters`` as in blasst_prefill,
    for the decisions at ``lam``.
    """
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k and v must be 4-D [B, H, L, d]")
    B, Hq, L, _ = q.shape
    if gap_map is None:
        gap_map = torch.empty(B, Hq, -(-L // tile_q), -(-L // block_k), dtype=torch.float32, device=q.device)
    p = _prefill_params(q, k, v, None, causal, lam, tile_q, block_k, scale, skip_map, gap_map, counters, window)
    if B > 0 and L > 0:
        _check_devices(q, k=k, v=v, skip_map=skip_map, gap_map=gap_map, counters=counters)
    _check(load_library().blasst_prefill_gaps(ctypes.byref(p), _stream(stream, q.device)), "blasst_prefill_gaps")
    return gap_map


def _prefill_params(q, k, v, out, causal, lam, tile_q, block_k, scale, skip_map, gap_map, counters, window):
    """blasst_prefill_params for the tensors, after the host-side shape checks
    (``out`` None: no output, for the gap pass)."""
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4 and (out is None or out.dim() == 4),
          "q, k, v and out must be 4-D [B, H, L, d]")
    B, Hq, L, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    _need(k.shape[0] == B and k.shape[2] >= L and k.shape[3] == d,
          f"k must be [B={B}, Hkv, >= L={L}, d={d}] (got {list(k.shape)})")
    _need(v.shape[0] == B and v.shape[1] == Hkv and v.shape[2] >= L,
          f"v must be [B={B}, Hkv={Hkv}, >= L={L}, dv] (got {list(v.shape)})")
    if out is not None:
        _need(list(out.shape) == [B, Hq, L, dv], f"out must be [{B}, {Hq}, {L}, {dv}] (got {list(out.shape)})")
    if tile_q > 0 and block_k > 0:
        n = B * Hq * -(-L // tile_q) * -(-L // block_k)
        _check_map(skip_map, "skip_map", torch.uint8, n)
        _check_map(gap_map, "gap_map", torch.float32, n)
    _check_counters(counters)
    return _PrefillParams(_tensor(q), _tensor(k), _tensor(v), _tensor(out), B, Hq, Hkv, L, d, dv,
                          int(bool(causal)), float(scale) if scale is not None else 0.0, float(lam),
                          int(tile_q), int(block_k), _ptr(skip_map), _ptr(gap_map), _ptr(counters), int(window))


def _check_lens(seq_lens, B):
    if seq_lens is None:
        return
    _need(seq_lens.dtype == torch.int32, f"seq_lens must be int32 (got {seq_lens.dtype})")
    _need(seq_lens.is_contiguous() and seq_lens.numel() == B, f"seq_lens must hold {B} contiguous entries")


def _decode_params(q, k_cache, v_cache, seq_lens, lam, scale, block_k, num_splits, out,
                   skip_map, gap_map, counters, window=0, sink_seed=False):
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, dqk = q.shape
    _need(k_cache.dim() == 4 and k_cache.shape[0] == B and k_cache.shape[3] == dqk,
          f"k_cache must be [B={B}, Hkv, Lmax, dqk={dqk}] (got {list(k_cache.shape)})")
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if v_cache is not None:
        _need(v_cache.dim() == 4 and list(v_cache.shape[:3]) == [B, Hkv, Lmax],
              f"v_cache must be [B={B}, Hkv={Hkv}, Lmax={Lmax}, dv] (got {list(v_cache.shape)})")
    dv = out.shape[2] if out is not None else (v_cache.shape[3] if v_cache is not None else dqk)
    if out is not None:
        _need(out.dim() == 3 and list(out.shape[:2]) == [B, Hq], f"out must be [{B}, {Hq}, dv]")
        _need(v_cache is None or dv <= v_cache.shape[3], f"dv = {dv} exceeds the v_cache width")
    _check_lens(seq_lens, B)
    if block_k > 0:
        n = B * Hkv * -(-Lmax // block_k)
        _check_map(skip_map, "skip_map", torch.uint8, n)
        _check_map(gap_map, "gap_map", torch.float32, n)
    _check_counters(counters)
    return _DecodeParams(_tensor(q, True), _tensor(k_cache), _tensor(v_cache), _tensor(out, True),
                         _ptr(seq_lens), B, Hq, Hkv, Lmax, dqk, dv,
                         float(scale) if scale is not None else 0.0, float(lam), int(block_k),
                         int(num_splits), _ptr(skip_map), _ptr(gap_map), _ptr(counters), int(window),
                         int(bool(sink_seed)))


def blasst_decode_plan(q, k_cache, v_cache, seq_lens, *, lam=0.0, scale=None, block_k=64, num_splits=0,
                       dv=None, out_dtype=torch.float32, window=0):
    """(num_splits the call will use, workspace bytes it needs)."""
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, _ = q.shape
    dv = dv if dv is not None else v_cache.shape[3]
    p = _decode_params(q, k_cache, v_cache, seq_lens, lam, scale, block_k, num_splits, None,
                       None, None, None, window)
    # the planner reads no device memory: describe O [B,Hq,dv] at q's (aligned) address
    p.o = _Tensor(q.data_ptr(), _BF16 if out_dtype == torch.bfloat16 else _FP32, Hq * dv, dv, 0)
    p.dv = dv
    ns, ws = ctypes.c_int(0), ctypes.c_size_t(0)
    _check(load_library().blasst_decode_plan(ctypes.byref(p), ctypes.byref(ns), ctypes.byref(ws)),
           "blasst_decode_plan")
    return ns.value, ws.value


def blasst_decode(q, k_cache, v_cache, seq_lens, *, lam=0.0, scale=None, block_k=64, num_splits=0,
                  dv=None, out=None, out_dtype=torch.float32, workspace=None, skip_map=None,
                  gap_map=None, counters=None, stream=None, window=0, sink_seed=False):
    """Block-skipping decode: q [B,Hq,dqk], caches [B,Hkv,Lmax,*] (bf16, device), seq_lens int32 [B].

    ``window`` > 0: sliding window, the query sees the last ``window`` keys.
    ``sink_seed``: splits after the first start their running max from the
    row maxima of the first visible block.

    For the latent (MLA) form pass ``v_cache = k_cache`` and ``dv=512``.
    ``workspace`` (uint8 device tensor) is allocated here when not given.
    Returns O [B,Hq,dv].
    """
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, _ = q.shape
    dv = dv if dv is not None else v_cache.shape[3]
    if out is None:
        out = torch.empty(B, Hq, dv, dtype=out_dtype, device=q.device)
    p = _decode_params(q, k_cache, v_cache, seq_lens, lam, scale, block_k, num_splits, out,
                       skip_map, gap_map, counters, window, sink_seed)
    lib = load_library()
    if workspace is None:
        ns, ws = ctypes.c_int(0), ctypes.c_size_t(0)
        _check(lib.blasst_decode_plan(ctypes.byref(p), ctypes.byref(ns), ctypes.byref(ws)), "blasst_decode_plan")
        workspace = torch.empty(max(ws.value, 1), dtype=torch.uint8, device=q.device)
    if B > 0:
        _check_devices(q, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, out=out, workspace=workspace,
                       skip_map=skip_map, gap_map=gap_map, counters=counters)
    _check(lib.blasst_decode(ctypes.byref(p), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                             _stream(stream, q.device)), "blasst_decode")
    return out


def blasst_decode_gaps(q, k_cache, v_cache, seq_lens, *, lam=0.0, scale=None, block_k=64, num_splits=0, dv=None,
                       skip_map=None, gap_map=None, counters=None, stream=None, window=0, sink_seed=False):
    """The gap pass of blasst_decode (calibration): maps and counters only, no
    O and no workspace; the split plan is blasst_decode's.  Returns the gap map
    float32 [B,Hkv,ceil(Lmax/block_k)] (``gap_map`` if given, else a new one)."""
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, _ = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dv = dv if dv is not None else v_cache.shape[3]
    if gap_map is None:
        gap_map = torch.empty(B, Hkv, -(-Lmax // block_k), dtype=torch.float32, device=q.device)
    p = _decode_params(q, k_cache, v_cache, seq_lens, lam, scale, block_k, num_splits, None,
                       skip_map, gap_map, counters, window, sink_seed)
    p.dv = dv
    if B > 0:
        _check_devices(q, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, skip_map=skip_map,
                       gap_map=gap_map, counters=counters)
    _check(load_library().blasst_decode_gaps(ctypes.byref(p), _stream(stream, q.device)), "blasst_decode_gaps")
    return gap_map


def blasst_decode_noalloc(q, k_cache, v_cache, seq_lens, *, lam=0.0, scale=None, block_k=64, num_splits=0,
                          dv=None, out=None, out_dtype=torch.float32, skip_map=None, gap_map=None, counters=None,
                          stream=None, window=0, sink_seed=False):
    """blasst_decode without a workspace: the split partials live in the
    library's own device array (BLASST_NOALLOC_SCRATCH_BYTES per GPU).  Calls
    that overlap on one GPU race.  Returns O [B,Hq,dv]."""
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, _ = q.shape
    dv = dv if dv is not None else v_cache.shape[3]
    if out is None:
        out = torch.empty(B, Hq, dv, dtype=out_dtype, device=q.device)
    p = _decode_params(q, k_cache, v_cache, seq_lens, lam, scale, block_k, num_splits, out,
                       skip_map, gap_map, counters, window, sink_seed)
    if B > 0:
        _check_devices(q, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, out=out,
                       skip_map=skip_map, gap_map=gap_map, counters=counters)
    _check(load_library().blasst_decode_noalloc(ctypes.byref(p), _stream(stream, q.device)), "blasst_decode_noalloc")
    return out


def _paged_params(q, k_pages, v_pages, page_table, seq_lens, Lmax, lam, scale, block_k, num_splits, o,
                  skip_map, gap_map, counters, window=0, sink_seed=False):
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, dqk = q.shape
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.stride(1) != 1:
        raise ValueError("page_table must be an int32 [B, pages_per_seq] tensor with unit column stride")
    _need(page_table.shape[0] == B, f"page_table needs {B} rows (got {page_table.shape[0]})")
    _need(k_pages.dim() == 4 and k_pages.shape[3] == dqk,
          f"k_pages must be [pages, Hkv, page_size, dqk={dqk}] (got {list(k_pages.shape)})")
    _need(v_pages.dim() == 4 and list(v_pages.shape[:3]) == list(k_pages.shape[:3]),
          f"v_pages must be [pages, Hkv, page_size, dv] like k_pages (got {list(v_pages.shape)})")
    _check_lens(seq_lens, B)
    if block_k > 0:
        n = B * k_pages.shape[1] * -(-int(Lmax) // block_k)
        _check_map(skip_map, "skip_map", torch.uint8, n)
        _check_map(gap_map, "gap_map", torch.float32, n)
    _check_counters(counters)
    d = _DecodeParams(_tensor(q, True), _tensor(k_pages), _tensor(v_pages), o,
                      _ptr(seq_lens), B, Hq, k_pages.shape[1], int(Lmax), dqk, 0,
                      float(scale) if scale is not None else 0.0, float(lam), int(block_k),
                      int(num_splits), _ptr(skip_map), _ptr(gap_map), _ptr(counters), int(window),
                      int(bool(sink_seed)))
    return _DecodePagedParams(d, page_table.data_ptr(), page_table.stride(0), k_pages.shape[0],
                              k_pages.shape[2])


def blasst_decode_paged_plan(q, k_pages, v_pages, page_table, seq_lens, Lmax, *, lam=0.0, scale=None,
                             block_k=64, num_splits=0, dv=None, out_dtype=torch.float32, window=0):
    """(num_splits the paged call will use, workspace bytes it needs)."""
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, _ = q.shape
    dv = dv if dv is not None else v_pages.shape[3]
    # the planner reads no device memory: describe O [B,Hq,dv] at q's (aligned) address
    o = _Tensor(q.data_ptr(), _BF16 if out_dtype == torch.bfloat16 else _FP32, Hq * dv, dv, 0)
    p = _paged_params(q, k_pages, v_pages, page_table, seq_lens, Lmax, lam, scale, block_k, num_splits, o,
                      None, None, None, window)
    p.d.dv = dv
    ns, ws = ctypes.c_int(0), ctypes.c_size_t(0)
    _check(load_library().blasst_decode_paged_plan(ctypes.byref(p), ctypes.byref(ns), ctypes.byref(ws)),
           "blasst_decode_paged_plan")
    return ns.value, ws.value


def blasst_decode_paged(q, k_pages, v_pages, page_table, seq_lens, Lmax, *, lam=0.0, scale=None, block_k=64,
                        num_splits=0, dv=None, out=None, out_dtype=torch.float32, workspace=None, skip_map=None,
                        gap_map=None, counters=None, stream=None, window=0, sink_seed=False):
    """Block-skipping decode over a paged cache.

    q [B,Hq,dqk]; k_pages [num_pages,Hkv,page_size,dqk] and v_pages
    [num_pages,Hkv,page_size,dv] (any strides with a contiguous last dim, e.g.
    a [num_pages,page_size,Hkv,d] pool permuted to that order); page_table
    int32 [B, pages_per_seq]; seq_lens int32 [B]; Lmax the largest length (it
    sizes the skip/gap maps [B,Hkv,ceil(Lmax/64)]).  Latent form: pass
    ``v_pages = k_pages`` and ``dv=512``.  Returns O [B,Hq,dv].
    """
    _need(q.dim() == 3, "q must be 3-D [B, Hq, dqk]")
    B, Hq, _ = q.shape
    dv = dv if dv is not None else v_pages.shape[3]
    if out is None:
        out = torch.empty(B, Hq, dv, dtype=out_dtype, device=q.device)
    _need(out.dim() == 3 and list(out.shape) == [B, Hq, dv], f"out must be [{B}, {Hq}, {dv}]")
    _need(dv <= v_pages.shape[3], f"dv = {dv} exceeds the v_pages width")
    p = _paged_params(q, k_pages, v_pages, page_table, seq_lens, Lmax, lam, scale, block_k, num_splits,
                      _tensor(out, True), skip_map, gap_map, counters, window, sink_seed)
    p.d.dv = dv
    lib = load_library()
    if workspace is None:
        ns, ws = ctypes.c_int(0), ctypes.c_size_t(0)
        _check(lib.blasst_decode_paged_plan(ctypes.byref(p), ctypes.byref(ns), ctypes.byref(ws)),
               "blasst_decode_paged_plan")
        workspace = torch.empty(max(ws.value, 1), dtype=torch.uint8, device=q.device)
    if B > 0:
        _check_devices(q, k_pages=k_pages, v_pages=v_pages, page_table=page_table, seq_lens=seq_lens, out=out,
                       workspace=workspace, skip_map=skip_map, gap_map=gap_map, counters=counters)
    _check(lib.blasst_decode_paged(ctypes.byref(p), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                   _stream(stream, q.device)), "blasst_decode_paged")
    return out


def calib_table(targets, a, *, tile_q=128, block_k=64, num_splits=0):
    """A calibration table (a plain dict, JSON-serialisable): fitted a per
    target sparsity and the tiling the fit used (num_splits 0 for prefill;
    tile_q 0 for decode)."""
    return {"target": [float(x) for x in targets], "a": [float(x) for x in a], "tile_q": int(tile_q),
            "block_k": int(block_k), "num_splits": int(num_splits)}


def save_calib_table(table, path):
    """Write a calibration table as JSON (the one state the method keeps between runs)."""
    import json
    with open(path, "w") as f:
        json.dump(table, f, indent=1)


def load_calib_table(path):
    import json
    with open(path) as f:
        t = json.load(f)
    return calib_table(t["target"], t["a"], tile_q=t["tile_q"], block_k=t["block_k"], num_splits=t["num_splits"])


def blasst_calibrate(table, target, L, *, tile_q=128, block_k=64, num_splits=0):
    """lambda = a(target) / L from a calibration table (ln a linear in the
    target) for a call with the given tiling; a table fitted with another
    tiling is refused (decisions depend on it)."""
    n = len(table["target"])
    t = (ctypes.c_double * n)(*[float(x) for x in table["target"]])
    aa = (ctypes.c_double * n)(*[float(x) for x in table["a"]])
    ct = _CalibTable(n, t, aa, int(table["tile_q"]), int(table["block_k"]), int(table["num_splits"]))
    out = ctypes.c_double(0.0)
    _check(load_library().blasst_calibrate(ctypes.byref(ct), float(target), int(L), int(tile_q), int(block_k),
                                           int(num_splits), ctypes.byref(out)), "blasst_calibrate")
    return out.value


def blasst_calibrate_search(gaps, target):
    """lambda reaching ``target`` sparsity on a gap map (host float32 array-like)."""
    import numpy as np
    g = np.ascontiguousarray(np.asarray(gaps, dtype=np.float32).ravel())
    lam, reached = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(load_library().blasst_calibrate_search(g.ctypes.data, g.size, float(target), ctypes.byref(lam),
                                                  ctypes.byref(reached)), "blasst_calibrate_search")
    return lam.value, reached.value


def blasst_calibrate_fit(lambdas, lengths):
    """a of the law lambda = a / L, fitted as ln a = mean(ln(lambda_i L_i))."""
    n = len(lambdas)
    lam = (ctypes.c_double * n)(*[float(x) for x in lambdas])
    ls = (ctypes.c_int64 * n)(*[int(x) for x in lengths])
    out = ctypes.c_double(0.0)
    _check(load_library().blasst_calibrate_fit(lam, ls, n, ctypes.byref(out)), "blasst_calibrate_fit")
    return out.value


def blasst_status_str(status):
    return load_library().blasst_status_str(int(status)).decode()


def blasst_last_error():
    return load_library().blasst_last_error().decode()


def blasst_abi_version():
    return load_library().blasst_abi_version()

"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, rejects invalid arguments with the documented codes before any launch,
and its host-only calibration calls agree with the oracle."""
import ctypes
import math
import os
import re

import numpy as np
import pytest
import torch

import oracle
import long_context_fa_amd as bl
from long_context_fa_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "blasst.h")).read()
    declared = set(re.findall(r"\b(blasst_[a-z_]+)\s*\(", header))
    assert {"blasst_prefill", "blasst_decode", "blasst_decode_plan", "blasst_decode_paged",
            "blasst_decode_paged_plan", "blasst_calibrate",
            "blasst_calibrate_search", "blasst_calibrate_fit", "blasst_status_str",
            "blasst_last_error", "blasst_abi_version"} <= declared
    lib = bl.load_library()
    for name in declared:
        assert hasattr(lib, name), name
    assert bl.blasst_abi_version() == 3
    for s in range(5):
        assert bl.blasst_status_str(s) != "unknown status"
    assert bl.blasst_status_str(99) == "unknown status"


def _bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def _prefill_err(**kw):
    """Status of blasst_prefill for host tensors that pass the binding's shape
    checks: the C ABI's own validation, called directly (the library must
    refuse the call before any launch, so the host pointers are never read)."""
    q, k, v = _bf16(1, 2, 128, 128), _bf16(1, 1, 128, 128), _bf16(1, 1, 128, 128)
    args = dict(q=q, k=k, v=v, causal=True, lam=0.01, tile_q=128, block_k=64)
    args.update(kw)
    B, Hq, L, _ = args["q"].shape
    out = torch.empty(B, Hq, L, args["v"].shape[3])
    p = _abi._prefill_params(args["q"], args["k"], args["v"], out, args["causal"], args["lam"], args["tile_q"],
                             args["block_k"], None, None, None, None, 0)
    status = bl.load_library().blasst_prefill(ctypes.byref(p), None)
    assert status != 0
    return status


@pytest.mark.parametrize("lam", [-0.1, 1.0, 1.5, float("nan")])
def test_prefill_rejects_lambda(lam):
    assert _prefill_err(lam=lam) == 1


def test_prefill_rejects_shapes_and_tiles():
    assert _prefill_err(k=_bf16(1, 3, 128, 128), v=_bf16(1, 3, 128, 128)) == 1  # Hq % Hkv
    assert _prefill_err(tile_q=32) == 2
    assert _prefill_err(block_k=32) == 2
    q, k, v = _bf16(1, 2, 128, 96), _bf16(1, 1, 128, 96), _bf16(1, 1, 128, 96)
    assert _prefill_err(q=q, k=k, v=v) == 2  # d = 96 not compiled
    assert _prefill_err(q=torch.zeros(1, 2, 128, 128, dtype=torch.float32)) == 2  # fp32 q
    qs = _bf16(1, 2, 128, 136)[..., :128]  # token stride 136: fine (multiple of 8)
    qb = _bf16(1, 2, 128, 132)[..., :128]  # token stride 132: not 16-byte aligned rows
    assert _prefill_err(q=qb) == 1
    assert qs.stride(2) == 136


def test_prefill_rejects_huge_kv_token_stride():
    """The tile copies use 32-bit offsets over a 64-row block: K/V token strides
    above 2^24 elements are refused before any launch (raw ABI call, the fake
    device pointer is never touched)."""
    fake = 1 << 20  # 16-byte aligned, never dereferenced
    def t(st, sh):
        return _abi._Tensor(fake, 0, 0, sh, st)
    for kst in ((1 << 24) + 8, 1 << 26):
        p = _abi._PrefillParams()
        p.q, p.o = t(128, 128 * 128), t(128, 128 * 128)
        p.k, p.v = t(kst, 0), t(128, 128 * 128)
        p.B, p.Hq, p.Hkv, p.L, p.d, p.dv = 1, 2, 1, 128, 128, 128
        p.causal, p.scale, p.lam, p.tile_q, p.block_k = 1, 0.0, 0.01, 128, 64
        lib = bl.load_library()
        assert lib.blasst_prefill(ctypes.byref(p), None) == 2
        assert "stride" in bl.blasst_last_error()


def test_size_limits_reject_overflowing_products():
    """Absurd sizes are refused as too large, with no overflowing product of
    caller sizes on the way (raw ABI calls; the fake device pointer is never
    touched): prefill unit counts past 2^31 - 1, and a latent cache whose
    rows * token stride * 2 does not fit 32 bits (checked by the planner)."""
    fake = 1 << 20
    lib = bl.load_library()
    def t(st, sh, sb=0):
        return _abi._Tensor(fake, 0, sb, sh, st)
    # (2^32 - 1) / 256 = 16777215 workgroups of 256 threads fit one launch at tile 128; 16777216 do not
    for B, Hq, L in ((1 << 40, 1 << 40, 128), (1 << 31, 1, 64), (1 << 20, 1 << 20, 1 << 20), (1, 1 << 62, 128),
                     (1 << 24, 1, 128), (1 << 12, 1 << 12, 128), (1 << 10, 1 << 10, 128 * 16)):
        p = _abi._PrefillParams()
        p.q = p.k = p.v = p.o = t(128, 128 * 128)
        p.B, p.Hq, p.Hkv, p.L, p.d, p.dv = B, Hq, 1, L, 128, 128
        p.causal, p.scale, p.lam, p.tile_q, p.block_k = 1, 0.0, 0.01, 128, 64
        assert lib.blasst_prefill(ctypes.byref(p), None) == 2, (B, Hq, L)
        assert "too large" in bl.blasst_last_error()
    # just inside the limit the size check passes; the K token stride check,
    # which comes after it, then refuses the call, so nothing is launched
    p = _abi._PrefillParams()
    p.q = p.v = p.o = t(128, 128 * 128)
    p.k = t((1 << 24) + 8, 0)
    p.B, p.Hq, p.Hkv, p.L, p.d, p.dv = (1 << 24) - 1, 1, 1, 128, 128, 128
    p.causal, p.scale, p.lam, p.tile_q, p.block_k = 1, 0.0, 0.01, 128, 64
    assert lib.blasst_prefill(ctypes.byref(p), None) == 2 and "stride" in bl.blasst_last_error()
    for kst, lmax in ((1 << 40, 4096), (1 << 62, 1), (576, 1 << 22)):
        p = _abi._DecodeParams()
        p.q, p.o = t(0, 576, 128 * 576), t(0, 512, 128 * 512)
        p.k_cache = p.v_cache = t(kst, 0)
        p.seq_lens = fake
        p.B, p.Hq, p.Hkv, p.Lmax, p.dqk, p.dv = 1, 128, 1, lmax, 576, 512
        p.lam, p.block_k = 0.01, 64
        splits, ws = ctypes.c_int(0), ctypes.c_size_t(0)
        assert lib.blasst_decode_plan(ctypes.byref(p), ctypes.byref(splits), ctypes.byref(ws)) == 2, (kst, lmax)
        assert "2^31" in bl.blasst_last_error()


def test_prefill_error_message_names_argument():
    _prefill_err(lam=2.0)
    assert "lambda" in bl.blasst_last_error()


def _decode_err(**kw):
    """Status of blasst_decode through the C ABI for host tensors (see _prefill_err)."""
    q = _bf16(2, 8, 128)
    kc, vc = _bf16(2, 2, 256, 128), _bf16(2, 2, 256, 128)
    lens = torch.full((2,), 256, dtype=torch.int32)
    args = dict(q=q, k_cache=kc, v_cache=vc, seq_lens=lens, lam=0.01, block_k=64, num_splits=0, dv=None,
                workspace=torch.zeros(16, dtype=torch.uint8))
    args.update(kw)
    q = args["q"]
    dv = args["dv"] if args["dv"] is not None else args["v_cache"].shape[3]
    out = torch.empty(q.shape[0], q.shape[1], dv)
    p = _abi._decode_params(q, args["k_cache"], args["v_cache"], args["seq_lens"], args["lam"], None,
                            args["block_k"], args["num_splits"], out, None, None, None)
    ws = args["workspace"]
    status = bl.load_library().blasst_decode(ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert status != 0
    return status


def test_decode_rejects():
    assert _decode_err(lam=1.0) == 1
    assert _decode_err(seq_lens=None) == 1
    assert _decode_err(num_splits=9) == 1          # more splits than blocks (4)
    assert _decode_err(block_k=128) == 2
    assert _decode_err(q=_bf16(2, 6, 128), k_cache=_bf16(2, 4, 256, 128), v_cache=_bf16(2, 4, 256, 128)) == 1
    # latent form needs V to alias K
    q = _bf16(1, 128, 576)
    kc = _bf16(1, 1, 256, 576)
    assert _decode_err(q=q, k_cache=kc, v_cache=_bf16(1, 1, 256, 576), dv=512,
                       seq_lens=torch.full((1,), 256, dtype=torch.int32)) == 2
    # more splits than one: workspace too small
    assert _decode_err(num_splits=4, workspace=torch.zeros(16, dtype=torch.uint8)) == 3
    # the latent form takes 1..128 heads sharing the latent head
    q = _bf16(1, 129, 576)
    assert _decode_err(q=q, k_cache=kc, v_cache=kc, dv=512, seq_lens=torch.full((1,), 256, dtype=torch.int32)) == 2


def test_gqa_plan_accepts_wide_groups():
    """dqk = dv decode takes up to 64 query heads per KV head (MQA included); 65 is refused."""
    kc = _bf16(1, 1, 4096, 128).expand(4, 1, 4096, 128)  # plan reads no memory; shapes only
    lens = torch.full((4,), 4096, dtype=torch.int32)
    for hq in (1, 16, 17, 32, 33, 64):
        S, ws = bl.blasst_decode_plan(_bf16(4, hq, 128), kc, kc, lens, lam=0.01)
        assert S >= 1 and ws == (4 * hq * S * (128 + 2) * 4 + 4 * S * 2 * 4 + 256 if S > 1 else 0)
    assert _decode_err(q=_bf16(1, 65, 128), k_cache=_bf16(1, 1, 256, 128), v_cache=_bf16(1, 1, 256, 128),
                       seq_lens=torch.full((1,), 256, dtype=torch.int32)) == 2


def test_latent_plan_accepts_head_shards():
    kc = _bf16(1, 1, 4096, 576).expand(16, 1, 4096, 576)  # plan reads no memory; shapes only
    lens = torch.full((16,), 4096, dtype=torch.int32)
    for hq in (1, 16, 40, 64, 128):
        S, ws = bl.blasst_decode_plan(_bf16(16, hq, 576), kc, kc, lens, lam=0.01, dv=512)
        assert S >= 1 and ws == (16 * hq * S * (512 + 2) * 4 + 16 * S * 2 * 4 + 256 if S > 1 else 0)


def test_decode_plan_host_only():
    q = _bf16(148, 32, 128)
    kc = _bf16(1, 8, 64, 128).expand(148, 8, 64, 128)  # plan reads no memory; shapes only
    lens = torch.full((148,), 64, dtype=torch.int32)
    S, ws = bl.blasst_decode_plan(q, kc, kc, lens, lam=0.01)
    assert S == 1 and ws == 0
    q1 = _bf16(1, 32, 128)
    kc1 = _bf16(1, 8, 32768, 128)
    S, ws = bl.blasst_decode_plan(q1, kc1, kc1, torch.full((1,), 32768, dtype=torch.int32), lam=0.01)
    assert S > 1 and ws >= 1 * 8 * S * 4 * (128 + 2) * 4
    S2, _ = bl.blasst_decode_plan(q1, kc1, kc1, torch.full((1,), 32768, dtype=torch.int32), lam=0.01,
                                  num_splits=7)
    assert S2 == 7


def test_empty_calls_are_noops():
    """L = 0 or B = 0 check the scalars only and return OK: empty torch
    tensors arrive as null pointers and nothing is launched or written."""
    base = _bf16(2, 2, 256, 128)
    out = torch.full((2, 2, 0, 128), 7.0)
    assert bl.blasst_prefill(base[:, :, :0], base[:, :1, :0], base[:, :1, :0], out=out, lam=0.01,
                             stream=0) is out
    bl.blasst_prefill(base[:0], base[:0, :1], base[:0, :1], out=torch.empty(0, 2, 256, 128), lam=0.01, stream=0)
    with pytest.raises(bl.BlasstError):  # scalars are still checked
        bl.blasst_prefill(base[:0], base[:0, :1], base[:0, :1], lam=1.5, stream=0)
    qd, kc = _bf16(2, 8, 128), _bf16(2, 2, 256, 128)
    lens = torch.full((2,), 256, dtype=torch.int32)
    assert bl.blasst_decode_plan(qd[:0], kc[:0], kc[:0], lens[:0], lam=0.01, num_splits=4) == (4, 0)
    bl.blasst_decode(qd[:0], kc[:0], kc[:0], lens[:0], lam=0.01, stream=0)
    with pytest.raises(bl.BlasstError):
        bl.blasst_decode(qd[:0], kc[:0], kc[:0], lens[:0], lam=0.01, window=-1, stream=0)


# ------------------------------------------------------------- paged decode
def _paged_err(page_size=64, pages=8, table_cols=4, Lmax=256, **kw):
    """Status of blasst_decode_paged through the C ABI for host tensors (see _prefill_err)."""
    q = _bf16(2, 8, 128)
    pool = _bf16(max(pages, 0), 2, page_size, 128)
    table = torch.zeros(2, table_cols, dtype=torch.int32)
    lens = torch.full((2,), Lmax, dtype=torch.int32)
    args = dict(lam=0.01, num_splits=0, workspace=torch.zeros(16, dtype=torch.uint8))
    args.update(kw)
    out = torch.empty(2, 8, 128)
    p = _abi._paged_params(q, pool, pool, table, lens, Lmax, args["lam"], None, 64, args["num_splits"],
                           _abi._tensor(out, True), None, None, None)
    p.d.dv = 128
    ws = args["workspace"]
    status = bl.load_library().blasst_decode_paged(ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert status != 0
    return status


def test_decode_paged_rejects():
    assert _paged_err(page_size=24) == 1            # not a power of two
    assert _paged_err(page_size=8, table_cols=32) == 1  # below 16 rows
    assert _paged_err(table_cols=3) == 1            # table narrower than ceil(Lmax / page_size)
    assert _paged_err(pages=0) == 1                 # empty pool
    assert _paged_err(lam=1.0) == 1                 # the decode checks still apply
    assert _paged_err(num_splits=4, workspace=torch.zeros(16, dtype=torch.uint8)) == 3
    # a null table through the C ABI itself
    q, pool = _bf16(2, 8, 128), _bf16(8, 2, 64, 128)
    o = _abi._Tensor(q.data_ptr(), 1, 8 * 128, 128, 0)
    d = _abi._DecodeParams(_abi._tensor(q, True), _abi._tensor(pool), _abi._tensor(pool), o,
                           torch.zeros(2, dtype=torch.int32).data_ptr(), 2, 8, 2, 256, 128, 128,
                           0.0, 0.01, 64, 0, None, None, None)
    p = _abi._DecodePagedParams(d, None, 4, 8, 64)
    assert bl.load_library().blasst_decode_paged_plan(ctypes.byref(p), None, None) == 1
    assert "page_table" in bl.blasst_last_error()


def test_decode_paged_plan_equals_contiguous_plan():
    """Paging changes addresses only: the split plan and the workspace are
    those of the contiguous call of the same lengths."""
    q = _bf16(16, 32, 128)
    lens = torch.full((16,), 32768, dtype=torch.int32)
    kc = _bf16(1, 8, 32768, 128).expand(16, 8, 32768, 128)
    pool = _bf16(1, 8, 64, 128).expand(8192, 8, 64, 128)
    table = torch.zeros(16, 512, dtype=torch.int32)
    for lam, ns in [(0.01, 0), (0.0, 5)]:
        assert bl.blasst_decode_paged_plan(q, pool, pool, table, lens, 32768, lam=lam, num_splits=ns) == \
            bl.blasst_decode_plan(q, kc, kc, lens, lam=lam, num_splits=ns)


def test_paged_pool_builder_round_trips_through_the_oracle_gather():
    from long_context_fa_amd import inputs
    g = torch.Generator().manual_seed(3)
    kc = torch.randn(3, 2, 200, 16, generator=g).to(torch.bfloat16)
    vc = torch.randn(3, 2, 200, 8, generator=g).to(torch.bfloat16)
    lens = [200, 1, 77]
    for P, rm in [(16, False), (64, True), (256, False)]:
        (kp, vp), table = inputs.paged_pool([kc, vc], lens, P, seed=5, spare_pages=2, row_major_heads=rm)
        assert kp.shape[1:] == (2, P, 16) and table.shape == (3, -(-200 // P))
        for c, pool in [(kc, kp), (vc, vp)]:
            got = oracle.gather_pages(pool.float().numpy(), table.numpy(), lens, 200)
            for b, n in enumerate(lens):
                np.testing.assert_array_equal(got[b, :, :n], c[b, :, :n].float().numpy())
        used = table[table >= 0]
        assert used.unique().numel() == used.numel()  # no page is shared


# ------------------------------------------------------ calibration (host C)
def test_calibrate_matches_oracle():
    targets, a = [0.3, 0.5, 0.7, 0.8], [3.0, 40.0, 900.0, 4000.0]
    for target in [0.3, 0.41, 0.5, 0.66, 0.7, 0.79, 0.8]:
        for L in [4096, 8192, 32768, 65536]:
            lam = bl.blasst_calibrate(bl.calib_table(targets, a), target, L)
            ref = oracle.lambda_from_table(targets, a, target, L)
            assert abs(lam - ref) <= 1e-13 * ref


def test_calibrate_rejects():
    T = bl.calib_table
    with pytest.raises(bl.BlasstError):
        bl.blasst_calibrate(T([0.3, 0.5], [3.0, 40.0]), 0.9, 4096)   # outside the table
    with pytest.raises(bl.BlasstError):
        bl.blasst_calibrate(T([0.5, 0.3], [3.0, 40.0]), 0.4, 4096)   # not increasing
    with pytest.raises(bl.BlasstError):
        bl.blasst_calibrate(T([0.5], [5000.0]), 0.5, 4096)           # lambda >= 1
    with pytest.raises(bl.BlasstError):
        bl.blasst_calibrate_fit([0.0], [100])
    with pytest.raises(bl.BlasstError):
        bl.blasst_calibrate_search([-np.inf, -np.inf], 0.5)


def test_calibrate_search_matches_oracle_quantile():
    rng = np.random.default_rng(5)
    gaps = rng.normal(-8, 4, size=5000).astype(np.float32)
    gaps[:50] = np.inf            # first blocks
    gaps[-300:] = -np.inf         # unvisited pairs are ignored
    vis = gaps[gaps != -np.inf].astype(np.float64)
    for target in [0.0, 0.1, 0.3, 0.5, 0.7, 0.8, 0.95]:
        lam, reached = bl.blasst_calibrate_search(gaps, target)
        lam_o, reached_o = oracle.lambda_for_target(vis, target)
        assert abs(lam - lam_o) <= 1e-12 * max(lam_o, 1e-300)
        assert reached == reached_o
        assert abs(reached - target) <= 1 / vis.size + 1e-12 or target > 0.9


def test_calibrate_fit_matches_oracle():
    Ls = [4096, 8192, 16384, 32768, 65536]
    lams = [1.1e-3, 6e-4, 2.7e-4, 1.4e-4, 6.9e-5]
    assert abs(bl.blasst_calibrate_fit(lams, Ls) - oracle.fit_a(lams, Ls)) < 1e-12


def test_binding_structs_match_the_header_abi_version():
    """The ctypes structs are written for one ABI version; the binding
    refuses a library of another (checked in load_library)."""
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "blasst.h")).read()
    v = int(re.search(r"#define BLASST_ABI_VERSION (\d+)", hdr).group(1))
    assert _abi.ABI_VERSION == v
    assert _abi.load_library().blasst_abi_version() == v


# ------------------------------------------------- binding argument checks
def test_binding_refuses_host_tensors_before_any_launch():
    """The library receives bare pointers: a host tensor, or one on another
    device than the query, is refused by the binding with ValueError."""
    q, k, v = _bf16(1, 2, 128, 128), _bf16(1, 1, 128, 128), _bf16(1, 1, 128, 128)
    with pytest.raises(ValueError, match="GPU"):
        bl.blasst_prefill(q, k, v, lam=0.01, stream=0)
    qd, kc = _bf16(2, 8, 128), _bf16(2, 2, 256, 128)
    lens = torch.full((2,), 256, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        bl.blasst_decode(qd, kc, kc, lens, lam=0.01, stream=0, workspace=torch.zeros(16, dtype=torch.uint8))
    pool, table = _bf16(8, 2, 64, 128), torch.zeros(2, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        bl.blasst_decode_paged(qd, pool, pool, table, lens, 256, lam=0.01, stream=0,
                               workspace=torch.zeros(16, dtype=torch.uint8))


def test_binding_refuses_inconsistent_prefill_arguments():
    q, k, v = _bf16(1, 2, 128, 128), _bf16(1, 1, 128, 128), _bf16(1, 1, 128, 128)
    def err(**kw):
        args = dict(q=q, k=k, v=v, lam=0.01, stream=0)
        args.update(kw)
        with pytest.raises(ValueError) as ei:
            bl.blasst_prefill(**args)
        return str(ei.value)
    assert "k must be" in err(k=_bf16(1, 1, 64, 128))                      # fewer keys than queries
    assert "k must be" in err(k=_bf16(2, 1, 128, 128))                     # other batch
    assert "v must be" in err(v=_bf16(1, 2, 128, 128))                     # other KV head count
    assert "out must be" in err(out=torch.empty(1, 2, 128, 64))
    assert "4-D" in err(q=_bf16(2, 128, 128))
    n = 1 * 2 * 1 * 2  # B * Hq * nQT * nKB
    assert "skip_map" in err(skip_map=torch.zeros(n, dtype=torch.int32))
    assert "skip_map" in err(skip_map=torch.zeros(n - 1, dtype=torch.uint8))
    assert "gap_map" in err(gap_map=torch.zeros(n, dtype=torch.float64))
    assert "counters" in err(counters=torch.zeros(2, dtype=torch.int32))
    assert "counters" in err(counters=torch.zeros(1, dtype=torch.int64))


def test_binding_refuses_inconsistent_decode_arguments():
    q, kc = _bf16(2, 8, 128), _bf16(2, 2, 256, 128)
    lens = torch.full((2,), 256, dtype=torch.int32)
    ws = torch.zeros(16, dtype=torch.uint8)
    def err(**kw):
        args = dict(q=q, k_cache=kc, v_cache=kc, seq_lens=lens, lam=0.01, stream=0, workspace=ws)
        args.update(kw)
        with pytest.raises(ValueError) as ei:
            bl.blasst_decode(**args)
        return str(ei.value)
    assert "seq_lens" in err(seq_lens=lens.to(torch.int64))                 # read as int32 pairs otherwise
    assert "seq_lens" in err(seq_lens=torch.full((3,), 256, dtype=torch.int32))
    assert "v_cache" in err(v_cache=_bf16(2, 2, 128, 128))                  # shorter than k_cache
    assert "k_cache" in err(k_cache=_bf16(1, 2, 256, 128))
    assert "skip_map" in err(skip_map=torch.zeros(2 * 2 * 4 - 1, dtype=torch.uint8))
    assert "gap_map" in err(gap_map=torch.zeros(2 * 2 * 4, dtype=torch.float16))
    assert "counters" in err(counters=torch.zeros(2, dtype=torch.float32))
    assert "out must be" in err(out=torch.empty(2, 4, 128))
    pool, table = _bf16(8, 2, 64, 128), torch.zeros(2, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="page_table"):
        bl.blasst_decode_paged(q, pool, pool, torch.zeros(3, 4, dtype=torch.int32), lens, 256, lam=0.01,
                               stream=0, workspace=ws)
    with pytest.raises(ValueError, match="v_pages"):
        bl.blasst_decode_paged(q, pool, _bf16(8, 2, 32, 128), table, lens, 256, lam=0.01, stream=0, workspace=ws)
    with pytest.raises(ValueError, match="seq_lens"):
        bl.blasst_decode_paged(q, pool, pool, table, lens.to(torch.int64), 256, lam=0.01, stream=0, workspace=ws)


def test_noalloc_decode_refuses_partials_beyond_the_scratch_before_any_launch():
    """blasst_decode_noalloc plans like blasst_decode and refuses, on the host,
    a split plan whose partials exceed BLASST_NOALLOC_SCRATCH_BYTES (raw ABI
    call; the fake device pointers are never touched)."""
    hdr = open(os.path.join(ROOT, "include", "blasst.h")).read()
    cap = eval(re.search(r"#define BLASST_NOALLOC_SCRATCH_BYTES \(([^)]*)\)", hdr).group(1).replace("u", ""))
    fake = 1 << 20
    lib = bl.load_library()
    p = _abi._DecodeParams()
    B, Hq, Hkv, L, d, S = 4096, 32, 8, 8192, 128, 32
    p.q, p.o = _abi._Tensor(fake, 0, Hq * d, d, 0), _abi._Tensor(fake, 1, Hq * d, d, 0)
    p.k_cache = p.v_cache = _abi._Tensor(fake, 0, Hkv * L * d, L * d, d)
    p.seq_lens = fake
    p.B, p.Hq, p.Hkv, p.Lmax, p.dqk, p.dv = B, Hq, Hkv, L, d, d
    p.lam, p.block_k, p.num_splits = 0.01, 64, S
    ws = ctypes.c_size_t(0)
    assert lib.blasst_decode_plan(ctypes.byref(p), None, ctypes.byref(ws)) == 0 and ws.value > cap
    assert lib.blasst_decode_noalloc(ctypes.byref(p), None) == 3
    assert "scratch" in bl.blasst_last_error()


def test_gap_passes_need_an_output_and_validate_first():
    """The gap passes write only maps and counters: with none of them given the
    call is refused; other arguments are validated as for the full pass (raw
    ABI calls with host pointers, refused before any launch)."""
    lib = bl.load_library()
    q, k, v = _bf16(1, 2, 128, 128), _bf16(1, 1, 128, 128), _bf16(1, 1, 128, 128)
    p = _abi._prefill_params(q, k, v, None, True, 0.01, 128, 64, None, None, None, None, 0)
    assert lib.blasst_prefill_gaps(ctypes.byref(p), None) == 1 and "gap pass" in bl.blasst_last_error()
    gap = torch.zeros(1, 2, 1, 2)
    p = _abi._prefill_params(q, k, v, None, True, 1.5, 128, 64, None, None, gap, None, 0)
    assert lib.blasst_prefill_gaps(ctypes.byref(p), None) == 1 and "lambda" in bl.blasst_last_error()
    qd, kc = _bf16(2, 8, 128), _bf16(2, 2, 256, 128)
    lens = torch.full((2,), 256, dtype=torch.int32)
    p = _abi._decode_params(qd, kc, kc, lens, 0.01, None, 64, 0, None, None, None, None)
    assert lib.blasst_decode_gaps(ctypes.byref(p), None) == 1 and "gap pass" in bl.blasst_last_error()
    p = _abi._decode_params(qd, kc, kc, lens, 0.01, None, 128, 0, None, None, torch.zeros(2, 2, 4), None)
    assert lib.blasst_decode_gaps(ctypes.byref(p), None) == 2  # block_k 128 is not compiled


def test_calibration_table_carries_its_tiling(tmp_path):
    """A fitted a belongs to the tiling it was fitted with (decisions depend on
    the query tile and on the decode split count): blasst_calibrate refuses a
    call with another tiling; a table survives a JSON round trip."""
    pre = bl.calib_table([0.5, 0.7], [1e-6, 3e-4], tile_q=128, block_k=64, num_splits=0)
    lam = bl.blasst_calibrate(pre, 0.7, 8192, tile_q=128, block_k=64, num_splits=0)
    assert abs(lam - 3e-4 / 8192) <= 1e-15
    for kw in (dict(tile_q=64), dict(block_k=128), dict(num_splits=4)):
        args = dict(tile_q=128, block_k=64, num_splits=0)
        args.update(kw)
        with pytest.raises(bl.BlasstError) as ei:
            bl.blasst_calibrate(pre, 0.7, 8192, **args)
        assert ei.value.status == 1 and "tiling" in bl.blasst_last_error()
    dec = bl.calib_table([0.7], [2e-2], tile_q=0, block_k=64, num_splits=4)
    assert bl.blasst_calibrate(dec, 0.7, 32768, tile_q=0, num_splits=4) == pytest.approx(2e-2 / 32768, rel=1e-14)
    with pytest.raises(bl.BlasstError):
        bl.blasst_calibrate(dec, 0.7, 32768, tile_q=0, num_splits=1)
    path = tmp_path / "table.json"
    bl.save_calib_table(pre, str(path))
    assert bl.load_calib_table(str(path)) == pre

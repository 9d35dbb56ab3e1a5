"""The gap pass (blasst_prefill_gaps, blasst_decode_gaps): scores, block maxima,
running max and decisions only.  Its gap map must be bit-equal to the one the
full pass writes at lambda = 0 and at the calibrated lambda (the running max
never depends on the decisions), its skip map and counters must equal the full
pass's at that lambda, and both maps must meet the parity bar against the
oracle."""
import numpy as np
import pytest
import torch

import long_context_fa_amd as bl
import oracle
from long_context_fa_amd import inputs
from parity import check_decisions, f64, gpu_decode, gpu_prefill, lambda_for, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _same(a, b, what):
    if torch.equal(a, b):
        return
    d = (a != b)
    idx = d.nonzero()[:8].tolist()
    raise AssertionError(f"{what}: {int(d.sum())} of {a.numel()} differ; first {idx}: "
                         f"{[a[tuple(i)].item() for i in idx]} vs {[b[tuple(i)].item() for i in idx]}")


def _gap_pass_prefill(q, k, v, *, causal, lam, tile_q, window=0):
    B, Hq, L, _ = q.shape
    nqt, nkb = -(-L // tile_q), -(-L // 64)
    skip = torch.full((B, Hq, nqt, nkb), 7, dtype=torch.uint8, device=DEV)
    gap = torch.full((B, Hq, nqt, nkb), float("nan"), dtype=torch.float32, device=DEV)
    cnt = torch.zeros(2, dtype=torch.int64, device=DEV)
    bl.blasst_prefill_gaps(q, k, v, causal=causal, lam=lam, tile_q=tile_q, skip_map=skip, gap_map=gap,
                           counters=cnt, window=window)
    torch.cuda.synchronize()
    return skip, gap, cnt.cpu().numpy()


@pytest.mark.parametrize("B,Hq,Hkv,L,d,tile_q,causal,window", [
    (1, 8, 2, 2048 + 37, 128, 128, True, 0),
    (2, 4, 4, 1000, 64, 64, True, 0),
    (1, 4, 2, 777, 128, 64, False, 0),
    (1, 4, 2, 3000, 128, 128, True, 999),
])
def test_prefill_gap_pass(B, Hq, Hkv, L, d, tile_q, causal, window):
    say(f"[gaps] prefill B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} tile={tile_q} causal={causal} window={window}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, device=DEV, seed=900 + L)
    _, _, gap0, _ = gpu_prefill(q, k, v, causal=causal, lam=0.0, tile_q=tile_q, window=window)
    lam, _ = lambda_for(gap0, 0.6)
    sk_g, gap_g, cnt_g = _gap_pass_prefill(q, k, v, causal=causal, lam=lam, tile_q=tile_q, window=window)
    _, sk_f, gap_f, cnt_f = gpu_prefill(q, k, v, causal=causal, lam=lam, tile_q=tile_q, window=window)
    _same(gap_g, gap0, "gap pass vs lambda=0 gaps")
    _same(gap_g, gap_f, "gap pass vs full-pass gaps")
    _same(sk_g, sk_f, "skip maps")
    assert np.array_equal(cnt_g, cnt_f)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=causal, lam=lam, tile_q=tile_q, block_k=64, window=window)
    check_decisions(sk_g.cpu().numpy(), gap_g.cpu().numpy(), ref["skip"], ref["gap"], lam)
    assert cnt_g[0] == ref["visited"] and abs(cnt_g[1] - ref["skipped"]) <= 0.005 * ref["visited"]


def _gap_pass_decode(q, kc, vc, lens, *, lam, splits, dv=None, window=0, sink_seed=False):
    B, Hkv, Lmax = q.shape[0], kc.shape[1], kc.shape[2]
    nkb = -(-Lmax // 64)
    skip = torch.full((B, Hkv, nkb), 7, dtype=torch.uint8, device=DEV)
    gap = torch.full((B, Hkv, nkb), float("nan"), dtype=torch.float32, device=DEV)
    cnt = torch.zeros(2, dtype=torch.int64, device=DEV)
    bl.blasst_decode_gaps(q, kc, vc, lens, lam=lam, num_splits=splits, dv=dv, skip_map=skip, gap_map=gap,
                          counters=cnt, window=window, sink_seed=sink_seed)
    torch.cuda.synchronize()
    return skip, gap, cnt.cpu().numpy()


@pytest.mark.parametrize("layout,splits,window,sink_seed", [
    ("gqa", 1, 0, False), ("gqa", 3, 0, False), ("gqa", 3, 0, True), ("gqa", 2, 1000, False),
    ("gqa_d64", 2, 0, False), ("gqa_g40", 3, 0, True), ("gqa_g64_d64", 1, 700, False),
    ("latent", 1, 0, False), ("latent", 4, 0, True),
])
def test_decode_gap_pass(layout, splits, window, sink_seed):
    say(f"[gaps] decode {layout} splits={splits} window={window} sink_seed={sink_seed}")
    if layout.startswith("gqa"):
        # (query heads, KV heads, d): 4 heads per KV head, or the 2- and 4-group forms
        Hq, Hkv, d = {"gqa": (32, 8, 128), "gqa_d64": (32, 8, 64), "gqa_g40": (80, 2, 128),
                      "gqa_g64_d64": (64, 1, 64)}[layout]
        q, kc, vc, lens = inputs.decode_inputs(3, Hq, Hkv, 3000, d, device=DEV, seed=950 + splits,
                                               seq_lens=[3000, 1234, 1])
        dv, vv = None, None
    else:
        q, kc, _, lens = inputs.decode_inputs(2, 128, 1, 4096, 576, 512, n_random=16, mla=True, device=DEV,
                                              seed=960 + splits, seq_lens=[4096, 2500])
        vc, dv = kc, 512
    kw = dict(num_splits=splits, dv=dv, window=window, sink_seed=sink_seed)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, **kw)
    lam, _ = lambda_for(gap0, 0.6)
    sk_g, gap_g, cnt_g = _gap_pass_decode(q, kc, vc, lens, lam=lam, splits=splits, dv=dv, window=window,
                                          sink_seed=sink_seed)
    _, sk_f, gap_f, cnt_f = gpu_decode(q, kc, vc, lens, lam=lam, **kw)
    _same(gap_g, gap0, "gap pass vs lambda=0 gaps")
    _same(gap_g, gap_f, "gap pass vs full-pass gaps")
    _same(sk_g, sk_f, "skip maps")
    assert np.array_equal(cnt_g, cnt_f)
    kk = f64(kc)
    ref = oracle.decode(f64(q), kk, kk[..., :dv] if dv else f64(vc), lens.cpu().numpy(), lam=lam, block_k=64,
                        num_splits=splits, window=window, sink_seed=sink_seed)
    check_decisions(sk_g.cpu().numpy(), gap_g.cpu().numpy(), ref["skip"], ref["gap"], lam)
    assert cnt_g[0] == ref["visited"]

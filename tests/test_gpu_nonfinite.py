"""GPU parity on inputs holding NaN and +-inf, and with a caller-given scale.

Non-finite inputs follow the reading both sides implement (the pages say
nothing about them): block maxima and tile gaps ignore NaN; in an executed
block every key some row of the unit sees enters every row with its weight
(0 for a row that does not see it, and 0 * inf = 0 * NaN = NaN); keys no row
sees enter nothing; O = acc / l for l != 0 and exactly 0 for l = 0; the split
merge keeps every split with l != 0.  The bar: decisions identical outside the
gap band, the same set of non-finite outputs (NaN and +-inf are not told apart:
how many zero-weight copies of a value a block holds depends on the tiling),
and the finite outputs within max-abs 1e-2 / mean-abs 1e-3."""
import numpy as np
import pytest
import torch

import long_context_fa_amd as bl
import oracle
from long_context_fa_amd import inputs
from parity import check_decisions, check_output, f64, gpu_decode, gpu_prefill, lambda_for, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAN, INF = float("nan"), float("inf")


def _compare(o_gpu, o_ref, what):
    g = o_gpu.detach().to("cpu", torch.float64).numpy()
    fg, fr = np.isfinite(g), np.isfinite(o_ref)
    bad = fg != fr
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs differ in finiteness, first at {np.argwhere(bad)[:4]}"
    assert (~fr).any(), f"{what}: the case produced no non-finite output"
    check_output(g[fr], o_ref[fr], what)


def _prefill_case(B, Hq, Hkv, L, seed, window=0):
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, 128, device=DEV, seed=seed)
    return q, k, v


@pytest.mark.parametrize("target", [None, 0.6])
def test_prefill_nonfinite_inputs(target):
    L = 640 + 37
    q, k, v = _prefill_case(1, 4, 2, L, seed=1201)
    k[0, 0, 100, :] = NAN          # NaN scores for every row of heads 0, 1 that sees key 100
    k[0, 1, 400, 7] = INF          # +-inf scores in heads 2, 3
    v[0, 0, 300, 5] = -INF         # reaches every row of a tile that executes block 4
    v[0, 1, 10, 9] = NAN
    q[0, 2, 200, :] = NAN          # a row whose scores are all NaN
    q[0, 3, 33, 0] = INF           # a row whose running max becomes +inf
    lam = 0.0
    if target is not None:
        lam, _ = lambda_for(bl.blasst_prefill_gaps(q, k, v, tile_q=128), target)
    say(f"[nonfinite] prefill L={L} lam={lam:.4g}")
    o, skip, gap, cnt = gpu_prefill(q, k, v, causal=True, lam=lam, tile_q=128)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=True, lam=lam, tile_q=128, block_k=64)
    check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], lam)
    assert cnt[0] == ref["visited"]
    _compare(o, ref["o"], f"prefill nonfinite lam={lam:.3g}")


def test_prefill_window_edge_keys_seen_by_no_row_stay_out():
    """W = 100, tile 128: tile 1 visits block 0 for keys 29..63 only; a +inf at
    key 10 (seen by no row of tile 1) must not reach it."""
    L = 512
    q, k, v = _prefill_case(1, 2, 1, L, seed=1202)
    v[0, 0, 10, 0] = INF
    k[0, 0, 140, :] = NAN
    o, skip, gap, _ = gpu_prefill(q, k, v, causal=True, lam=0.0, tile_q=128, window=100)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=True, lam=0.0, tile_q=128, block_k=64, window=100)
    check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], 0.0)
    _compare(o, ref["o"], "prefill window edge")
    # rows of tile 1 that do not see the NaN key 140 stay finite: key 10 never reached them
    assert torch.isfinite(o[0, :, 128:140]).all() and torch.isfinite(o[0, :, 240:256]).all()


@pytest.mark.parametrize("splits", [1, 3])
def test_gqa_decode_nonfinite_inputs(splits):
    q, kc, vc, lens = inputs.decode_inputs(3, 32, 8, 3000, 128, device=DEV, seed=1210 + splits,
                                           seq_lens=[3000, 1234, 1])
    kc[0, 2, 1500, :] = NAN        # a NaN sum in the split holding key 1500
    vc[1, 5, 700, 3] = INF
    vc[0, 0, 2999, 0] = NAN        # the last key: the padding of its block repeats it
    q[0, 9, 5] = INF               # head 9 (KV head 2) gets a +inf running max
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=splits)
    lam, _ = lambda_for(gap0, 0.6)
    say(f"[nonfinite] gqa decode splits={splits} lam={lam:.4g}")
    o, skip, gap, cnt = gpu_decode(q, kc, vc, lens, lam=lam, num_splits=splits)
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.cpu().numpy(), lam=lam, block_k=64, num_splits=splits)
    check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], lam)
    assert cnt[0] == ref["visited"]
    _compare(o, ref["o"], f"gqa decode nonfinite splits={splits}")


def test_latent_decode_nonfinite_inputs():
    q, kc, _, lens = inputs.decode_inputs(2, 128, 1, 8192, 576, 512, n_random=16, mla=True, device=DEV,
                                          seed=1220, seq_lens=[8192, 3000])
    kc[0, 0, 5000, :] = NAN        # latent row: NaN scores and NaN values
    kc[1, 0, 100, 10] = INF        # +-inf scores and a +inf value in column 10
    _, _, gap0, _ = gpu_decode(q, kc, kc, lens, lam=0.0, num_splits=4, dv=512)
    lam, _ = lambda_for(gap0, 0.6)
    o, skip, gap, _ = gpu_decode(q, kc, kc, lens, lam=lam, num_splits=4, dv=512)
    kk = f64(kc)
    ref = oracle.decode(f64(q), kk, kk[..., :512], lens.cpu().numpy(), lam=lam, block_k=64, num_splits=4)
    check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], lam)
    _compare(o, ref["o"], "latent decode nonfinite")


# ------------------------------------------------------- caller-given scale
@pytest.mark.parametrize("scale", [0.031, 0.2])
def test_prefill_caller_scale(scale):
    q, k, v = _prefill_case(1, 4, 2, 1000, seed=1230)
    gap0 = bl.blasst_prefill_gaps(q, k, v, tile_q=64, scale=scale)
    lam, _ = lambda_for(gap0, 0.6)
    say(f"[scale] prefill scale={scale} lam={lam:.4g}")
    B, Hq, L, _ = q.shape
    skip = torch.zeros(B, Hq, -(-L // 64), -(-L // 64), dtype=torch.uint8, device=DEV)
    gap = torch.zeros(B, Hq, -(-L // 64), -(-L // 64), dtype=torch.float32, device=DEV)
    o = bl.blasst_prefill(q, k, v, lam=lam, tile_q=64, scale=scale, skip_map=skip, gap_map=gap)
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=True, scale=scale, lam=lam, tile_q=64, block_k=64)
    check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], lam)
    check_output(o.cpu().numpy(), ref["o"], f"prefill scale={scale}")
    assert 0 < (skip == 1).sum().item()


@pytest.mark.parametrize("scale", [0.02, 0.25])
def test_decode_caller_scale(scale):
    q, kc, vc, lens = inputs.decode_inputs(2, 16, 4, 2500, 128, device=DEV, seed=1240)
    gap0 = bl.blasst_decode_gaps(q, kc, vc, lens, num_splits=2, scale=scale)
    lam, _ = lambda_for(gap0, 0.6)
    B, Hkv, nkb = 2, 4, -(-2500 // 64)
    skip = torch.zeros(B, Hkv, nkb, dtype=torch.uint8, device=DEV)
    gap = torch.zeros(B, Hkv, nkb, dtype=torch.float32, device=DEV)
    o = bl.blasst_decode(q, kc, vc, lens, lam=lam, num_splits=2, scale=scale, skip_map=skip, gap_map=gap)
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.cpu().numpy(), scale=scale, lam=lam, block_k=64,
                        num_splits=2)
    check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], lam)
    check_output(o.cpu().numpy(), ref["o"], f"decode scale={scale}")

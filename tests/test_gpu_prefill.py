"""GPU parity of blasst_prefill (HIP, gfx950) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_fa_amd import inputs
from parity import (check_decisions, check_output, f64, gpu_prefill, lambda_for, say,
                    SPARSITY_ABS)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_full(q, k, v, *, causal, lam, tile_q, what, window=0):
    """GPU vs oracle over every unit."""
    say(f"[prefill] {what}: q{tuple(q.shape)} k{tuple(k.shape)} causal={causal} lam={lam:.4g} tile={tile_q}"
        f" window={window}")
    o, skip, gap, cnt = gpu_prefill(q, k, v, causal=causal, lam=lam, tile_q=tile_q, window=window)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=causal, lam=lam, tile_q=tile_q, block_k=64,
                         window=window)
    nb = check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], lam)
    check_output(o.cpu().numpy(), ref["o"], what)
    assert cnt[0] == ref["visited"]
    assert abs(cnt[1] - ref["skipped"]) <= nb
    say(f"  visited {cnt[0]} skipped gpu {cnt[1]} oracle {ref['skipped']} band {nb}")
    return ref


def test_parity_single_head_config():
    """1x1x1024x64, fp32 inputs rounded to bf16, tile 64, causal, lambda = 1e-3."""
    q, k, v = inputs.prefill_inputs(1, 1, 1, 1024, 64, n_random=2, local_window=0, dtype=torch.float32,
                                    device=DEV, seed=1000)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    ref = _run_full(q, k, v, causal=True, lam=1e-3, tile_q=64, what="1x1x1024x64")
    assert ref["skipped"] > 0


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d,tile_q", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_parity_ragged_gqa(causal, d, tile_q):
    """L not a multiple of the tile or block; GQA 4/2; lambda at the 60% gap quantile."""
    L = 1000
    q, k, v = inputs.prefill_inputs(2, 4, 2, L, d, device=DEV, seed=7 + d + tile_q)
    _, _, gap0, _ = gpu_prefill(q, k, v, causal=causal, lam=0.0, tile_q=tile_q)
    lam, _ = lambda_for(gap0, 0.6)
    _run_full(q, k, v, causal=causal, lam=lam, tile_q=tile_q, what=f"ragged d={d} tile={tile_q}")


@pytest.mark.parametrize("L", [1, 63, 64, 65, 129])
def test_parity_tiny_lengths(L):
    q, k, v = inputs.random_inputs((1, 2, L, 128), (1, 1, L, 128), (1, 1, L, 128), dtype=torch.bfloat16,
                                   device=DEV, seed=L, std=1.0)
    for lam in [0.0, 0.3]:
        _run_full(q, k, v, causal=True, lam=lam, tile_q=128, what=f"L={L}")


def test_dense_path_matches_oracle():
    """lambda = 0 dispatches the dense kernel: softmax attention over all keys."""
    q, k, v = inputs.prefill_inputs(1, 4, 1, 2048, 128, device=DEV, seed=3)
    ref = _run_full(q, k, v, causal=True, lam=0.0, tile_q=128, what="dense")
    assert ref["skipped"] == 0


def test_skip_kernel_at_unreachable_lambda_matches_dense():
    """lambda = 1e-300 runs the skip-enabled kernel (votes, decisions, predicated
    V loads) although no block can meet the test: every visited block executes,
    and O equals the lambda = 0 kernel's to rounding of the same operations."""
    q, k, v = inputs.prefill_inputs(1, 4, 2, 1000, 128, device=DEV, seed=31)
    ref = _run_full(q, k, v, causal=True, lam=1e-300, tile_q=128, what="skip kernel, unreachable lambda")
    assert ref["skipped"] == 0
    o_skip, skip, _, cnt = gpu_prefill(q, k, v, causal=True, lam=1e-300, tile_q=128)
    o_dense, _, _, _ = gpu_prefill(q, k, v, causal=True, lam=0.0, tile_q=128)
    assert cnt[1] == 0 and not (skip.cpu().numpy() == 1).any()
    assert (o_skip - o_dense).abs().max().item() <= 1e-6


def test_bf16_output_matches_fp32_output():
    q, k, v = inputs.prefill_inputs(1, 2, 1, 1024, 128, device=DEV, seed=4)
    o32, _, _, _ = gpu_prefill(q, k, v, causal=True, lam=1e-6, tile_q=128, maps=False)
    o16, _, _, _ = gpu_prefill(q, k, v, causal=True, lam=1e-6, tile_q=128, maps=False, out_dtype=torch.bfloat16)
    ref = o32.to(torch.bfloat16).float()
    assert torch.equal(o16.float(), ref)


def test_strided_inputs():
    """Non-contiguous q/k/v (token stride > d, heads interleaved) give the same result."""
    B, Hq, Hkv, L, d = 1, 4, 2, 512, 128
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, device=DEV, seed=8)
    # [B, L, H, d] storage viewed as [B, H, L, d]
    qs = q.transpose(1, 2).contiguous().transpose(1, 2)
    ks = k.transpose(1, 2).contiguous().transpose(1, 2)
    vs = v.transpose(1, 2).contiguous().transpose(1, 2)
    o1, s1, g1, _ = gpu_prefill(q, k, v, causal=True, lam=1e-4, tile_q=128)
    o2, s2, g2, _ = gpu_prefill(qs, ks, vs, causal=True, lam=1e-4, tile_q=128)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(g1, g2)


def _sampled(q, k, v, *, lam, tile_q, units, what, window=0):
    """Full-size GPU run, oracle on a set of (b, h, tile) units."""
    B, Hq, L, _ = q.shape
    nqt = -(-L // tile_q)
    say(f"[prefill] {what}: full GPU run, oracle on {len(units)} units (window {window})")
    o, skip, gap, cnt = gpu_prefill(q, k, v, causal=True, lam=lam, tile_q=tile_q, window=window)
    mask = np.zeros((B, Hq, nqt), np.uint8)
    for (b, h, t) in units:
        mask[b, h, t] = 1
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=True, lam=lam, tile_q=tile_q, block_k=64,
                         unit_mask=mask, window=window)
    sel = mask.astype(bool)
    check_decisions(skip.cpu().numpy()[sel], gap.cpu().numpy()[sel], ref["skip"][sel], ref["gap"][sel], lam)
    rows = np.zeros((B, Hq, L), bool)
    for (b, h, t) in units:
        rows[b, h, t * tile_q:(t + 1) * tile_q] = True
    check_output(o.cpu().numpy()[rows], ref["o"][rows], what)
    # sparsity of the sampled units, GPU map vs oracle
    gs = skip.cpu().numpy()[sel]
    g_frac = (gs == 1).sum() / max(1, (gs != 255).sum())
    r_frac = ref["skipped"] / max(1, ref["visited"])
    say(f"  sampled sparsity gpu {g_frac:.4f} oracle {r_frac:.4f}; whole-run {cnt[1] / cnt[0]:.4f}")
    assert abs(g_frac - r_frac) <= SPARSITY_ABS
    return cnt


@pytest.mark.parametrize("B,Hq,Hkv,L,d,tile_q,causal", [
    (1, 8, 8, 700, 64, 64, True),       # 8 KV groups: one per XCD, 11 tiles over the four phases
    (2, 16, 4, 520, 128, 128, True),    # B * Hkv = 8 with GQA 4
    (2, 16, 8, 900, 128, 128, True),    # 16 groups: two per XCD
    (1, 16, 8, 600, 128, 64, False),    # non-causal phase edges
    (1, 32, 4, 700, 64, 64, True),      # 4 KV groups, each over 2 XCDs
    (1, 16, 2, 600, 128, 128, True),    # 2 groups over 4 XCDs each
    (1, 8, 1, 500, 128, 128, True),     # MQA: one group over all 8 XCDs
    (2, 16, 1, 520, 64, 64, False),     # B * Hkv = 2, non-causal
])
def test_parity_xcd_mapped_units_full(B, Hq, Hkv, L, d, tile_q, causal):
    """When B * Hkv is a multiple or a divisor of 8 the kernel maps
    workgroups to (tile, head, batch) through the XCD-aware rotation; every
    unit is checked against the oracle, so a unit computed twice or never
    fails here."""
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, device=DEV, seed=40 + L + d)
    _, _, gap0, _ = gpu_prefill(q, k, v, causal=causal, lam=0.0, tile_q=tile_q)
    lam, _ = lambda_for(gap0, 0.6)
    _run_full(q, k, v, causal=causal, lam=lam, tile_q=tile_q, what=f"xcd-mapped {B}x{Hq}/{Hkv}x{L}x{d}")


def test_parity_gqa_prefill_8k_full_size():
    """1x32/8x8192x128, tile 128: lambda calibrated on the GPU gap map for 70%."""
    q, k, v = inputs.prefill_inputs(1, 32, 8, 8192, 128, n_random=6, local_window=1, device=DEV, seed=1001)
    _, _, gap0, _ = gpu_prefill(q, k, v, causal=True, lam=0.0, tile_q=128)
    lam, reached = lambda_for(gap0, 0.7)
    say(f"  lambda for 70%: {lam:.4g} (reaches {reached:.4f} on the gap map)")
    units = [(0, h, t) for h in range(32) for t in range(64)]  # every (head, tile): the whole launch
    cnt = _sampled(q, k, v, lam=lam, tile_q=128, units=units, what="1x32/8x8192x128")
    assert abs(cnt[1] / cnt[0] - reached) <= SPARSITY_ABS


def test_parity_long_prefill_32k_sampled():
    """2x32/8x32768x128 at the 70% lambda: oracle on sampled units."""
    q, k, v = inputs.prefill_inputs(2, 32, 8, 32768, 128, n_random=12, local_window=4, device=DEV, seed=1003)
    _, _, gap0, _ = gpu_prefill(q, k, v, causal=True, lam=0.0, tile_q=128)
    lam, reached = lambda_for(gap0, 0.7)
    say(f"  lambda for 70%: {lam:.4g} (reaches {reached:.4f})")
    units = [(1, 31, 255), (0, 0, 254), (1, 5, 128), (0, 17, 64), (1, 9, 3), (0, 30, 200)]
    rng = np.random.default_rng(5)  # plus 122 random (batch, head, tile) units: 128 of 16384
    units += [(int(b), int(h), int(t)) for b, h, t in zip(rng.integers(0, 2, 122), rng.integers(0, 32, 122),
                                                          rng.integers(0, 256, 122))]
    cnt = _sampled(q, k, v, lam=lam, tile_q=128, units=units, what="2x32/8x32768x128")
    assert abs(cnt[1] / cnt[0] - reached) <= SPARSITY_ABS


# ------------------------------------------------------------ sliding window
@pytest.mark.parametrize("W", [1, 63, 100, 257, 999])
@pytest.mark.parametrize("d,tile_q", [(128, 128), (64, 64)])
def test_parity_sliding_window(W, d, tile_q):
    """Query i sees keys i-W < c <= i; lambda at the 60% quantile of the windowed gaps."""
    q, k, v = inputs.prefill_inputs(2, 4, 2, 1000, d, device=DEV, seed=20 + W + d)
    _, _, gap0, _ = gpu_prefill(q, k, v, causal=True, lam=0.0, tile_q=tile_q, window=W)
    lam, _ = lambda_for(gap0, 0.6)
    _run_full(q, k, v, causal=True, lam=lam, tile_q=tile_q, what=f"window {W} d={d} tile={tile_q}", window=W)


def test_sliding_window_dense_and_covering_window():
    q, k, v = inputs.prefill_inputs(1, 4, 1, 1500, 128, device=DEV, seed=21)
    ref = _run_full(q, k, v, causal=True, lam=0.0, tile_q=128, what="window 300 dense", window=300)
    assert ref["skipped"] == 0
    # a window covering the sequence is plain causal attention, bit for bit
    a = gpu_prefill(q, k, v, causal=True, lam=1e-3, tile_q=128)
    b = gpu_prefill(q, k, v, causal=True, lam=1e-3, tile_q=128, window=1500)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def test_parity_sliding_window_8k_sampled():
    """1x32/8x8192x128, window 2048, lambda for 70% of the windowed pairs."""
    q, k, v = inputs.prefill_inputs(1, 32, 8, 8192, 128, n_random=6, local_window=1, device=DEV, seed=1001)
    _, _, gap0, _ = gpu_prefill(q, k, v, causal=True, lam=0.0, tile_q=128, window=2048)
    lam, reached = lambda_for(gap0, 0.7)
    units = [(0, 3, 63), (0, 31, 40), (0, 8, 16), (0, 20, 15), (0, 0, 1), (0, 12, 0)]
    cnt = _sampled(q, k, v, lam=lam, tile_q=128, units=units, what="window 2048, 1x32/8x8192x128", window=2048)
    assert abs(cnt[1] / cnt[0] - reached) <= SPARSITY_ABS

"""GPU parity of blasst_decode (HIP, gfx950) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import long_context_fa_amd as bl
import oracle
from long_context_fa_amd import inputs
from parity import (check_decisions, check_output, f64, gpu_decode, gpu_decode_paged, lambda_for, say,
                    SPARSITY_ABS)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _compare(q, kk, vv, lens, got, *, lam, S, what, window=0, sink_seed=False):
    """Whole-call parity: GPU results ``got`` = (o, skip, gap, counters)
    against the oracle over the float64 caches kk, vv [B, Hkv, Lmax, *]."""
    o, skip, gap, cnt = got
    ref = oracle.decode(f64(q), kk, vv, lens.cpu().numpy(), lam=lam, block_k=64, num_splits=S, window=window,
                        sink_seed=sink_seed)
    nb = check_decisions(skip.cpu().numpy(), gap.cpu().numpy(), ref["skip"], ref["gap"], lam)
    check_output(o.cpu().numpy(), ref["o"], what)
    gs = skip.cpu().numpy()
    g_frac = (gs == 1).sum() / max(1, (gs != 255).sum())
    r_frac = ref["skipped"] / max(1, ref["visited"])
    say(f"  splits {S}; sparsity gpu {g_frac:.4f} oracle {r_frac:.4f}; band {nb}")
    assert abs(g_frac - r_frac) <= SPARSITY_ABS
    assert cnt[0] == ref["visited"] and abs(cnt[1] - ref["skipped"]) <= nb
    return cnt, S


def _run(q, kc, vc, lens, *, lam, splits, what, unit_mask=None, dv=None, mla=False, sink_seed=False):
    B, Hq, dqk = q.shape
    Hkv = kc.shape[1]
    say(f"[decode] {what}: q{tuple(q.shape)} cache{tuple(kc.shape)} lam={lam:.4g} splits={splits}")
    o, skip, gap, cnt = gpu_decode(q, kc, vc, lens, lam=lam, num_splits=splits, dv=dv, sink_seed=sink_seed)
    S_used, _ = bl.blasst_decode_plan(q, kc, vc, lens, lam=lam, num_splits=splits, dv=dv)
    if unit_mask is None:
        kk = f64(kc)
        vv = kk[..., :dv] if mla else f64(vc)
        return _compare(q, kk, vv, lens, (o, skip, gap, cnt), lam=lam, S=S_used, what=what, sink_seed=sink_seed)
    # copy only the sampled sequences to the host
    bs = sorted({b for b, _ in unit_mask})
    sub = {b: i for i, b in enumerate(bs)}
    kk = f64(kc[bs])
    vv = kk[..., :dv] if mla else f64(vc[bs])
    m = np.zeros((len(bs), Hkv), np.uint8)
    for b, g in unit_mask:
        m[sub[b], g] = 1
    ref_sub = oracle.decode(f64(q[bs]), kk, vv, lens[bs].cpu().numpy(), lam=lam, block_k=64,
                            num_splits=S_used, unit_mask=m, sink_seed=sink_seed)
    sel_u = np.zeros((B, Hkv), bool)
    ref = {"skip": np.full(skip.shape, 255, np.uint8), "gap": np.full(gap.shape, -np.inf),
           "o": np.zeros(o.shape), "visited": ref_sub["visited"], "skipped": ref_sub["skipped"]}
    for b, g in unit_mask:
        sel_u[b, g] = True
        ref["skip"][b, g] = ref_sub["skip"][sub[b], g]
        ref["gap"][b, g] = ref_sub["gap"][sub[b], g]
    G = Hq // Hkv
    for b in bs:
        ref["o"][b] = ref_sub["o"][sub[b]]
    nb = check_decisions(skip.cpu().numpy()[sel_u], gap.cpu().numpy()[sel_u], ref["skip"][sel_u],
                         ref["gap"][sel_u], lam)
    G = Hq // Hkv
    rows = np.repeat(sel_u, G, axis=1)
    check_output(o.cpu().numpy()[rows], ref["o"][rows], what)
    gs = skip.cpu().numpy()[sel_u]
    g_frac = (gs == 1).sum() / max(1, (gs != 255).sum())
    r_frac = ref["skipped"] / max(1, ref["visited"])
    say(f"  splits {S_used}; sparsity gpu {g_frac:.4f} oracle {r_frac:.4f}; band {nb}")
    assert abs(g_frac - r_frac) <= SPARSITY_ABS
    return cnt, S_used


@pytest.mark.parametrize("splits", [1, 2, 3, 16])
@pytest.mark.parametrize("d,G", [(128, 4), (64, 4), (128, 1), (128, 16), (64, 8),
                                 (128, 32), (64, 24), (128, 40), (128, 64), (64, 64)])
def test_parity_ragged(d, G, splits):
    B, Hkv, Lmax = 3, 2, 1000
    q, kc, vc, _ = inputs.decode_inputs(B, G * Hkv, Hkv, Lmax, d, device=DEV, seed=11 + d + G + splits)
    lens = torch.tensor([1000, 1, 333], dtype=torch.int32, device=DEV)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=splits)
    lam, _ = lambda_for(gap0, 0.6)
    _run(q, kc, vc, lens, lam=lam, splits=splits, what=f"ragged d={d} G={G}")


def test_dense_decode_matches_oracle():
    q, kc, vc, lens = inputs.decode_inputs(2, 8, 2, 4096, 128, device=DEV, seed=5)
    cnt, _ = _run(q, kc, vc, lens, lam=0.0, splits=4, what="dense")
    assert cnt[1] == 0


@pytest.mark.parametrize("mla", [False, True])
def test_skip_kernel_at_unreachable_lambda_matches_dense(mla):
    """lambda = 1e-300 runs the skip-enabled decode kernels although no block can
    meet the test: nothing is skipped and O equals the lambda = 0 kernels'."""
    if mla:
        q, kc, lens = _mla(2, 3000, seed=32)
        vc, dv = kc, 512
    else:
        q, kc, vc, lens = inputs.decode_inputs(3, 8, 2, 3000, 128, device=DEV, seed=32)
        dv = None
    cnt, S = _run(q, kc, vc, lens, lam=1e-300, splits=3, dv=dv, mla=mla, what=f"unreachable lambda mla={mla}")
    assert cnt[1] == 0
    o_skip, _, _, _ = gpu_decode(q, kc, vc, lens, lam=1e-300, num_splits=3, dv=dv)
    o_dense, _, _, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=3, dv=dv)
    assert (o_skip - o_dense).abs().max().item() <= 1e-6


def test_parity_gqa_decode_full_length():
    """4 sequences of the 32K GQA decode shape (32/8 heads, d 128), every unit checked."""
    q, kc, vc, lens = inputs.decode_inputs(4, 32, 8, 32768, 128, n_random=8, device=DEV, seed=1002)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=1)
    lam, reached = lambda_for(gap0, 0.7)
    cnt, _ = _run(q, kc, vc, lens, lam=lam, splits=1, what="4x32/8x32768x128")
    assert abs(cnt[1] / cnt[0] - reached) <= SPARSITY_ABS


def test_parity_gqa_decode_148_sequences_sampled():
    """The full 148-sequence, 32K, 32/8-head decode step; oracle on sampled units."""
    q, kc, vc, lens = inputs.decode_inputs(148, 32, 8, 32768, 128, n_random=8, device=DEV, seed=1002)
    S, _ = bl.blasst_decode_plan(q, kc, vc, lens, lam=0.01)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=S)
    lam, reached = lambda_for(gap0, 0.7)
    # every KV head of 16 sequences spread over the batch (first and last included): 128 of 1184 units
    seqs = [0, 9, 17, 28, 37, 46, 55, 63, 74, 83, 92, 100, 111, 120, 133, 147]
    units = [(b, g) for b in seqs for g in range(8)]
    cnt, _ = _run(q, kc, vc, lens, lam=lam, splits=S, what="148x32/8x32768x128", unit_mask=units)
    assert abs(cnt[1] / cnt[0] - reached) <= SPARSITY_ABS


def test_bf16_output_and_determinism():
    q, kc, vc, lens = inputs.decode_inputs(3, 8, 2, 2048, 128, device=DEV, seed=9)
    o1, s1, g1, _ = gpu_decode(q, kc, vc, lens, lam=1e-3, num_splits=2)
    o2, s2, g2, _ = gpu_decode(q, kc, vc, lens, lam=1e-3, num_splits=2)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(g1, g2)
    o3, _, _, _ = gpu_decode(q, kc, vc, lens, lam=1e-3, num_splits=2, out_dtype=torch.bfloat16)
    assert torch.equal(o3.float(), o1.to(torch.bfloat16).float())


# ---------------------------------------------------------------- latent (MLA)
# 128 query heads share one latent KV head of width 576; V = first 512 columns.

def _mla(B, Lmax, *, seed, n_random=16, lens=None):
    q, kc, _, sl = inputs.decode_inputs(B, 128, 1, Lmax, 576, 512, n_random=n_random, mla=True,
                                        device=DEV, seed=seed, seq_lens=lens)
    return q, kc, sl


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_parity_mla_ragged(splits):
    q, kc, lens = _mla(3, 2000, seed=41 + splits, lens=[2000, 1, 777])
    _, _, gap0, _ = gpu_decode(q, kc, kc, lens, lam=0.0, num_splits=splits, dv=512)
    lam, _ = lambda_for(gap0, 0.6)
    _run(q, kc, kc, lens, lam=lam, splits=splits, dv=512, mla=True, what="mla ragged")


def test_dense_mla_matches_oracle():
    q, kc, lens = _mla(2, 4096, seed=43)
    cnt, _ = _run(q, kc, kc, lens, lam=0.0, splits=3, dv=512, mla=True, what="mla dense")
    assert cnt[1] == 0


def test_mla_bf16_output_and_determinism():
    q, kc, lens = _mla(2, 3000, seed=44, lens=[3000, 1234])
    o1, s1, g1, _ = gpu_decode(q, kc, kc, lens, lam=2e-3, num_splits=2, dv=512)
    o2, s2, g2, _ = gpu_decode(q, kc, kc, lens, lam=2e-3, num_splits=2, dv=512)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(g1, g2)
    o3, _, _, _ = gpu_decode(q, kc, kc, lens, lam=2e-3, num_splits=2, dv=512, out_dtype=torch.bfloat16)
    assert torch.equal(o3.float(), o1.to(torch.bfloat16).float())
    # one split writes O directly (no combine pass); same decisions as the oracle
    o4, _, _, _ = gpu_decode(q, kc, kc, lens, lam=2e-3, num_splits=1, dv=512, out_dtype=torch.bfloat16)
    assert o4.dtype == torch.bfloat16 and torch.isfinite(o4.float()).all()


@pytest.mark.parametrize("G,splits", [(16, 1), (16, 4), (40, 3), (64, 2), (127, 1)])
def test_parity_mla_head_shards(G, splits):
    """The latent form with fewer than 128 heads (a shard of a model's heads):
    waves or lanes past G hold no query and must neither vote nor write."""
    q, kc, _, lens = inputs.decode_inputs(3, G, 1, 2000, 576, 512, n_random=16, mla=True, device=DEV,
                                          seed=140 + G + splits, seq_lens=[2000, 1, 777])
    _, _, gap0, _ = gpu_decode(q, kc, kc, lens, lam=0.0, num_splits=splits, dv=512)
    lam, _ = lambda_for(gap0, 0.6)
    _run(q, kc, kc, lens, lam=lam, splits=splits, dv=512, mla=True, what=f"mla G={G}")
    # paged: the same call over a shuffled 64-row pool is bit-equal
    (kp,), table = inputs.paged_pool([kc], lens, 64, seed=5)
    got = gpu_decode_paged(q, kp, kp, table, lens, kc.shape[2], lam=lam, num_splits=splits, dv=512)
    ref = gpu_decode(q, kc, kc, lens, lam=lam, num_splits=splits, dv=512)
    _equal_calls(got, ref)


def test_parity_mla_decode_full_size_sampled():
    """The 16-sequence, 64K-token latent decode step at ~70% sparsity, in the
    split configuration the planner picks; the oracle checks two whole
    sequences (all 128 heads)."""
    q, kc, lens = _mla(16, 65536, seed=2005)
    S, _ = bl.blasst_decode_plan(q, kc, kc, lens, lam=0.01, dv=512)
    _, _, gap0, _ = gpu_decode(q, kc, kc, lens, lam=0.0, num_splits=S, dv=512)
    lam, reached = lambda_for(gap0, 0.7)
    cnt, _ = _run(q, kc, kc, lens, lam=lam, splits=S, dv=512, mla=True, what="mla 16x128x65536x576",
                  unit_mask=[(3, 0), (15, 0)])
    assert abs(cnt[1] / cnt[0] - reached) <= SPARSITY_ABS


# ---------------------------------------------------------------- paged cache
# Pools are NaN wherever no token lives (rows past a sequence's end, spare
# pages), so a stray read shows up in O.  Paging changes only the address of
# a row: results must equal the contiguous call bit for bit, and the oracle
# over the gathered pages.

def _equal_calls(a, b):
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert (a[3] == b[3]).all()


@pytest.mark.parametrize("splits", [1, 3])
def test_shard_views_equal_contiguous_copies(splits):
    """One GPU's share of a sharded decode step, passed as a strided view with
    no copy: a context slice of the GQA cache (tokens 1024..2047 of 3000) and
    a head slice of the latent queries (16 of 48 heads).  Each call equals
    the same call on contiguous copies bit for bit, and the GQA slice matches
    the oracle over that slice."""
    q, kc, vc, _ = inputs.decode_inputs(3, 8, 2, 3000, 128, n_random=8, device=DEV, seed=150 + splits)
    ks, vs = kc[:, :, 1024:2048], vc[:, :, 1024:2048]
    assert not ks.is_contiguous()
    ls = torch.full((3,), 1024, dtype=torch.int32, device=DEV)
    _, _, gap0, _ = gpu_decode(q, ks, vs, ls, lam=0.0, num_splits=splits)
    lam, _ = lambda_for(gap0, 0.6)
    got = gpu_decode(q, ks, vs, ls, lam=lam, num_splits=splits)
    _equal_calls(got, gpu_decode(q, ks.contiguous(), vs.contiguous(), ls, lam=lam, num_splits=splits))
    _run(q, ks, vs, ls, lam=lam, splits=splits, what="GQA context slice view")
    qm, km, _, lm = inputs.decode_inputs(2, 48, 1, 1500, 576, 512, n_random=16, mla=True, device=DEV,
                                         seed=160 + splits)
    qs = qm[:, 16:32]
    assert not qs.is_contiguous()
    got = gpu_decode(qs, km, km, lm, lam=lam, num_splits=splits, dv=512)
    _equal_calls(got, gpu_decode(qs.contiguous(), km, km, lm, lam=lam, num_splits=splits, dv=512))


def _gathered(pool, table, lens, Lmax):
    return oracle.gather_pages(f64(pool), table.cpu().numpy(), lens.cpu().numpy(), Lmax)


@pytest.mark.parametrize("P,row_major", [(16, False), (64, True), (256, False)])
@pytest.mark.parametrize("d,G,splits", [(128, 4, 3), (64, 8, 1), (128, 16, 16), (128, 40, 2), (64, 64, 3)])
def test_paged_gqa_matches_contiguous_and_oracle(P, row_major, d, G, splits):
    B, Hkv, Lmax = 3, 2, 1000
    q, kc, vc, _ = inputs.decode_inputs(B, G * Hkv, Hkv, Lmax, d, device=DEV, seed=61 + d + G + P)
    lens = torch.tensor([1000, 1, 333], dtype=torch.int32, device=DEV)
    (kp, vp), table = inputs.paged_pool([kc, vc], lens, P, seed=P + d, spare_pages=3, row_major_heads=row_major)
    say(f"[paged] d={d} G={G} page={P} row_major={row_major} pool{tuple(kp.shape)} splits={splits}")
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=splits)
    lam, _ = lambda_for(gap0, 0.6)
    got = gpu_decode_paged(q, kp, vp, table, lens, Lmax, lam=lam, num_splits=splits)
    _equal_calls(got, gpu_decode(q, kc, vc, lens, lam=lam, num_splits=splits))
    _compare(q, _gathered(kp, table, lens, Lmax), _gathered(vp, table, lens, Lmax), lens, got,
             lam=lam, S=splits, what=f"paged d={d} G={G} P={P}")


def test_paged_gqa_dense_and_bf16_output():
    q, kc, vc, lens = inputs.decode_inputs(2, 8, 2, 4096, 128, device=DEV, seed=66)
    (kp, vp), table = inputs.paged_pool([kc, vc], lens, 32, seed=1, spare_pages=5)
    for lam, dt in [(0.0, torch.float32), (1e-3, torch.bfloat16)]:
        got = gpu_decode_paged(q, kp, vp, table, lens, 4096, lam=lam, num_splits=4, out_dtype=dt)
        _equal_calls(got, gpu_decode(q, kc, vc, lens, lam=lam, num_splits=4, out_dtype=dt))
        assert torch.isfinite(got[0].float()).all()


@pytest.mark.parametrize("P,splits", [(64, 2), (16, 5), (1024, 1)])
def test_paged_mla_matches_contiguous_and_oracle(P, splits):
    q, kc, lens = _mla(3, 2000, seed=71 + P, lens=[2000, 1, 777])
    (kp,), table = inputs.paged_pool([kc], lens, P, seed=P, spare_pages=2)
    say(f"[paged] mla page={P} pool{tuple(kp.shape)} splits={splits}")
    _, _, gap0, _ = gpu_decode(q, kc, kc, lens, lam=0.0, num_splits=splits, dv=512)
    lam, _ = lambda_for(gap0, 0.6)
    got = gpu_decode_paged(q, kp, kp, table, lens, 2000, lam=lam, num_splits=splits, dv=512)
    _equal_calls(got, gpu_decode(q, kc, kc, lens, lam=lam, num_splits=splits, dv=512))
    kk = _gathered(kp, table, lens, 2000)
    _compare(q, kk, kk[..., :512], lens, got, lam=lam, S=splits, what=f"paged mla P={P}")


def test_paged_gqa_decode_148_sequences_equals_contiguous():
    """The full 148-sequence, 32K, 32/8-head step over 64-row pages in a
    shuffled pool equals the contiguous call (itself checked against the
    oracle on sampled units) bit for bit, at the planner's split count."""
    q, kc, vc, lens = inputs.decode_inputs(148, 32, 8, 32768, 128, n_random=8, device=DEV, seed=1002)
    (kp, vp), table = inputs.paged_pool([kc, vc], lens, 64, seed=9)
    S, _ = bl.blasst_decode_plan(q, kc, vc, lens, lam=0.01)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=S)
    lam, _ = lambda_for(gap0, 0.7)
    say(f"[paged] 148x32/8x32768x128 page=64 splits={S} lam={lam:.4g}")
    got = gpu_decode_paged(q, kp, vp, table, lens, 32768, lam=lam)
    _equal_calls(got, gpu_decode(q, kc, vc, lens, lam=lam, num_splits=S))


# ------------------------------------------------------------ sliding window
@pytest.mark.parametrize("W", [1, 64, 200, 777])
@pytest.mark.parametrize("splits", [1, 3])
def test_window_gqa_decode(W, splits):
    q, kc, vc, _ = inputs.decode_inputs(3, 8, 2, 1000, 128, device=DEV, seed=80 + W + splits)
    lens = torch.tensor([1000, 1, 333], dtype=torch.int32, device=DEV)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=splits, window=W)
    lam, _ = lambda_for(gap0, 0.5)
    say(f"[decode] window {W} splits {splits} lam {lam:.4g}")
    got = gpu_decode(q, kc, vc, lens, lam=lam, num_splits=splits, window=W)
    _compare(q, f64(kc), f64(vc), lens, got, lam=lam, S=splits, what=f"gqa window {W}", window=W)


@pytest.mark.parametrize("W,splits", [(100, 2), (1000, 1), (65, 5)])
def test_window_mla_decode(W, splits):
    q, kc, lens = _mla(3, 2000, seed=90 + W, lens=[2000, 1, 777])
    _, _, gap0, _ = gpu_decode(q, kc, kc, lens, lam=0.0, num_splits=splits, dv=512, window=W)
    lam, _ = lambda_for(gap0, 0.5)
    say(f"[decode] mla window {W} splits {splits} lam {lam:.4g}")
    got = gpu_decode(q, kc, kc, lens, lam=lam, num_splits=splits, dv=512, window=W)
    kk = f64(kc)
    _compare(q, kk, kk[..., :512], lens, got, lam=lam, S=splits, what=f"mla window {W}", window=W)


def test_window_paged_decode_ignores_pages_outside_the_window():
    """A paged cache whose pages below the window hold NaN (freed pages of a
    sliding-window server) gives the contiguous result bit for bit."""
    q, kc, vc, _ = inputs.decode_inputs(2, 8, 2, 2048, 128, device=DEV, seed=95)
    lens = torch.tensor([2048, 1500], dtype=torch.int32, device=DEV)
    W, P = 300, 16
    (kp, vp), table = inputs.paged_pool([kc, vc], lens, P, seed=3, spare_pages=2)
    for b, n in enumerate(lens.tolist()):
        dead = table[b, :max(0, n - W) // P].long()  # pages wholly below the window
        kp[dead] = float("nan")
        vp[dead] = float("nan")
    lam = 1e-3
    got = gpu_decode_paged(q, kp, vp, table, lens, 2048, lam=lam, num_splits=2, window=W)
    _equal_calls(got, gpu_decode(q, kc, vc, lens, lam=lam, num_splits=2, window=W))
    assert torch.isfinite(got[0]).all()


# -------------------------------------------------------- sink-seeded splits
@pytest.mark.parametrize("splits,W", [(2, 0), (5, 0), (16, 0), (3, 300)])
def test_sink_seed_gqa_decode(splits, W):
    q, kc, vc, _ = inputs.decode_inputs(3, 8, 2, 1000, 128, device=DEV, seed=100 + splits + W)
    lens = torch.tensor([1000, 1, 333], dtype=torch.int32, device=DEV)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=splits, window=W, sink_seed=True)
    lam, _ = lambda_for(gap0, 0.6)
    say(f"[decode] sink seed splits {splits} window {W} lam {lam:.4g}")
    got = gpu_decode(q, kc, vc, lens, lam=lam, num_splits=splits, window=W, sink_seed=True)
    _compare(q, f64(kc), f64(vc), lens, got, lam=lam, S=splits, what=f"gqa sink seed S={splits} W={W}",
             window=W, sink_seed=True)


def test_sink_seed_one_split_is_unseeded():
    q, kc, vc, lens = inputs.decode_inputs(2, 8, 2, 2048, 64, device=DEV, seed=106)
    _equal_calls(gpu_decode(q, kc, vc, lens, lam=1e-3, num_splits=1, sink_seed=True),
                 gpu_decode(q, kc, vc, lens, lam=1e-3, num_splits=1))


@pytest.mark.parametrize("splits", [2, 5])
def test_sink_seed_mla_decode(splits):
    q, kc, lens = _mla(3, 2000, seed=107 + splits, lens=[2000, 1, 777])
    _, _, gap0, _ = gpu_decode(q, kc, kc, lens, lam=0.0, num_splits=splits, dv=512, sink_seed=True)
    lam, _ = lambda_for(gap0, 0.6)
    say(f"[decode] mla sink seed splits {splits} lam {lam:.4g}")
    got = gpu_decode(q, kc, kc, lens, lam=lam, num_splits=splits, dv=512, sink_seed=True)
    kk = f64(kc)
    _compare(q, kk, kk[..., :512], lens, got, lam=lam, S=splits, what=f"mla sink seed S={splits}", sink_seed=True)


def test_sink_seed_paged_equals_contiguous():
    q, kc, vc, lens = inputs.decode_inputs(2, 8, 2, 3000, 128, device=DEV, seed=109, seq_lens=[3000, 2222])
    (kp, vp), table = inputs.paged_pool([kc, vc], lens, 16, seed=4, spare_pages=1)
    _equal_calls(gpu_decode_paged(q, kp, vp, table, lens, 3000, lam=2e-3, num_splits=4, sink_seed=True),
                 gpu_decode(q, kc, vc, lens, lam=2e-3, num_splits=4, sink_seed=True))
    q, kc, lens = _mla(2, 3000, seed=110, lens=[3000, 1500])
    (kp,), table = inputs.paged_pool([kc], lens, 64, seed=5)
    _equal_calls(gpu_decode_paged(q, kp, kp, table, lens, 3000, lam=2e-3, num_splits=3, dv=512, sink_seed=True),
                 gpu_decode(q, kc, kc, lens, lam=2e-3, num_splits=3, dv=512, sink_seed=True))


def test_sink_seed_gqa_decode_148_sequences_sampled():
    """The full 148-sequence 32K GQA step with seeded splits at the planner's
    split count, lambda for 70% of the seeded gaps; oracle on sampled units."""
    q, kc, vc, lens = inputs.decode_inputs(148, 32, 8, 32768, 128, n_random=8, device=DEV, seed=1002)
    S, _ = bl.blasst_decode_plan(q, kc, vc, lens, lam=0.01)
    _, _, gap0, _ = gpu_decode(q, kc, vc, lens, lam=0.0, num_splits=S, sink_seed=True)
    lam, reached = lambda_for(gap0, 0.7)
    units = [(b, g) for b in (0, 37, 63, 100, 147) for g in range(8)]  # 40 of 1184 units
    cnt, _ = _run(q, kc, vc, lens, lam=lam, splits=S, what="148x32/8x32768x128 sink seed", unit_mask=units,
                  sink_seed=True)
    assert abs(cnt[1] / cnt[0] - reached) <= SPARSITY_ABS


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("mla", [False, True])
def test_zero_length_sequence(mla):
    """A sequence of length 0 yields O = 0 and an all-unvisited map; the other
    sequences are unaffected (bit-equal to a call without it)."""
    if mla:
        q, kc, _ = _mla(3, 1000, seed=120, lens=[1000, 1, 333])
        vc, dv = kc, 512
    else:
        q, kc, vc, _ = inputs.decode_inputs(3, 8, 2, 1000, 128, device=DEV, seed=121)
        dv = None
    lens = torch.tensor([1000, 0, 333], dtype=torch.int32, device=DEV)
    got = gpu_decode(q, kc, vc, lens, lam=1e-3, num_splits=3, dv=dv)
    assert torch.count_nonzero(got[0][1]) == 0
    assert (got[1][1] == 255).all() and torch.isinf(got[2][1]).all() and (got[2][1] < 0).all()
    keep = torch.tensor([0, 2], device=DEV)
    kk = kc[keep]
    vk = kk if mla else vc[keep]  # the latent V must alias K
    ref = gpu_decode(q[keep], kk, vk, lens[keep], lam=1e-3, num_splits=3, dv=dv)
    for x, y in zip(got[:3], ref[:3]):
        assert torch.equal(x[keep], y)

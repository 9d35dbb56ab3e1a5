"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Each check is something other than the oracle itself: the dense softmax
attention definition evaluated with a library matmul, the skip criterion of
the BLASST pages evaluated non-incrementally (closed form of the running
max), the dropped-mass bound that follows from the criterion, a hand-worked
example with closed-form outputs, and invariants (monotonicity in lambda,
GQA = MHA with repeated KV, split merge = single pass over the kept keys).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from bruteforce import (block_decisions, dense_probs, masked_softmax_attention,
                        prefill_mask, scores)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _prefill_case(seed, B=1, Hq=2, Hkv=1, L=200, d=16, dv=12, qstd=1.5, blocky=0):
    """Gaussian q, k, v; with ``blocky`` > 0 the keys of every run of ``blocky``
    positions are scaled by one factor in [0.05, 1] (the first run by 2), which
    makes whole blocks cold or hot as the skip test needs."""
    rng = np.random.default_rng(seed)
    q = _rand(rng, B, Hq, L, d, std=qstd)
    k = _rand(rng, B, Hkv, L, d, std=qstd)
    v = _rand(rng, B, Hkv, L, dv)
    if blocky:
        nb = -(-L // blocky)
        f = rng.uniform(0.05, 1.0, size=(B, Hkv, nb))
        f[..., 0] = 2.0
        k = k * np.repeat(f, blocky, axis=2)[..., :L, None]
    return q, k, v


def _lam_at(gap, qtl):
    """A lambda that puts ln(lambda) at quantile ``qtl`` of the finite gaps."""
    fg = gap[np.isfinite(gap)]
    return float(min(0.999, math.exp(np.quantile(fg, qtl) + 1e-6)))


# ---------------------------------------------------------------- dense limit
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("L,tq,bk", [(200, 64, 64), (130, 32, 64), (64, 64, 64), (1, 64, 64), (97, 16, 8)])
def test_prefill_lambda0_is_dense_softmax(causal, L, tq, bk):
    """lambda = 0 never skips: the oracle must be plain softmax attention (<= 1e-10)."""
    q, k, v = _prefill_case(7 + L, B=2, Hq=4, Hkv=2, L=L)
    r = oracle.prefill(q, k, v, causal=causal, lam=0.0, tile_q=tq, block_k=bk)
    scale = 1 / math.sqrt(q.shape[-1])
    mask = prefill_mask(L, causal)
    for b in range(2):
        for h in range(4):
            S = scores(q[b, h], k[b, h // 2], scale)
            ref = masked_softmax_attention(S, mask, v[b, h // 2])
            np.testing.assert_allclose(r["o"][b, h], ref, rtol=0, atol=1e-10)
    assert r["skipped"] == 0
    assert np.all((r["skip"] == 0) | (r["skip"] == 255))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 40])
def test_decode_lambda0_is_dense_softmax(splits):
    rng = np.random.default_rng(11 + splits)
    B, Hq, Hkv, Lmax, d, dv = 3, 6, 2, 300, 20, 10
    q = _rand(rng, B, Hq, d, std=1.5)
    k = _rand(rng, B, Hkv, Lmax, d, std=1.5)
    v = _rand(rng, B, Hkv, Lmax, dv)
    lens = np.array([300, 1, 129])
    r = oracle.decode(q, k, v, lens, lam=0.0, block_k=64, num_splits=splits)
    scale = 1 / math.sqrt(d)
    for b in range(B):
        for h in range(Hq):
            S = scores(q[b, h][None], k[b, h // 3], scale)
            mask = np.arange(Lmax)[None] < lens[b]
            ref = masked_softmax_attention(S, mask, v[b, h // 3])[0]
            np.testing.assert_allclose(r["o"][b, h], ref, rtol=0, atol=1e-10)
    assert r["skipped"] == 0


# ------------------------------------------------------------ skip decisions
def _prefill_brute_decisions(q, k, lam, causal, tq, bk, window=0):
    B, Hq, L, d = q.shape
    G = Hq // k.shape[1]
    nqt, nkb = -(-L // tq), -(-L // bk)
    skip = np.zeros((B, Hq, nqt, nkb), np.uint8)
    gap = np.zeros((B, Hq, nqt, nkb))
    mask = prefill_mask(L, causal, window)
    scale = 1 / math.sqrt(d)
    cols = [(j * bk, min(L, (j + 1) * bk)) for j in range(nkb)]
    for b in range(B):
        for h in range(Hq):
            S = scores(q[b, h], k[b, h // G], scale)
            for t in range(nqt):
                rows = slice(t * tq, min(L, (t + 1) * tq))
                s, g = block_decisions(S[rows], mask[rows], None, cols, lam)
                skip[b, h, t] = s
                gap[b, h, t] = g
    return skip, gap


@pytest.mark.parametrize("seed", range(12))
def test_prefill_decisions_match_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(40, 260))
    tq = int(rng.choice([16, 32, 64]))
    bk = int(rng.choice([8, 16, 32]))
    causal = bool(seed % 2)
    q, k, v = _prefill_case(seed, B=1, Hq=2, Hkv=1, L=L, d=8, dv=4, qstd=2.0, blocky=bk)
    # lambda at a random quantile of the brute-force gaps, so that both outcomes occur
    _, g0 = _prefill_brute_decisions(q, k, 0.0, causal, tq, bk)
    fg = g0[np.isfinite(g0)]
    lam = float(min(0.999, math.exp(np.quantile(fg, rng.uniform(0.2, 0.8)) + 1e-6)))
    r = oracle.prefill(q, k, v, causal=causal, lam=lam, tile_q=tq, block_k=bk)
    skip, gap = _prefill_brute_decisions(q, k, lam, causal, tq, bk)
    fin = np.isfinite(gap)
    np.testing.assert_allclose(r["gap"][fin], gap[fin], rtol=0, atol=1e-9)
    assert np.array_equal(np.isfinite(r["gap"]), fin)
    assert np.array_equal(r["gap"][~fin], gap[~fin])
    near = np.abs(gap - math.log(lam)) < 1e-9
    assert np.array_equal(r["skip"][~near], skip[~near])
    assert r["skipped"] > 0  # the cases do exercise skipping
    assert r["visited"] == int((skip != 255).sum())
    assert r["skipped"] == int((skip == 1).sum())


@pytest.mark.parametrize("seed", range(8))
def test_decode_decisions_match_bruteforce(seed):
    rng = np.random.default_rng(300 + seed)
    B, Hq, Hkv, Lmax, d, dv, bk = 2, 8, 2, int(rng.integers(70, 400)), 8, 6, 16
    splits = int(rng.integers(1, 5))
    q = _rand(rng, B, Hq, d, std=2.0)
    k = _rand(rng, B, Hkv, Lmax, d, std=2.0)
    v = _rand(rng, B, Hkv, Lmax, dv)
    lens = rng.integers(1, Lmax + 1, size=B)
    lam = float(10 ** rng.uniform(-5, -0.5))
    r = oracle.decode(q, k, v, lens, lam=lam, block_k=bk, num_splits=splits)
    G = Hq // Hkv
    scale = 1 / math.sqrt(d)
    nkb = -(-Lmax // bk)
    for b in range(B):
        nkb_b = -(-int(lens[b]) // bk)
        per = -(-nkb_b // splits)
        for g in range(Hkv):
            S = scores(q[b, g * G:(g + 1) * G], k[b, g], scale)
            mask = np.broadcast_to(np.arange(Lmax)[None] < lens[b], S.shape)
            exp_skip = [255] * nkb
            exp_gap = [-math.inf] * nkb
            for s in range(splits):
                jb, je = s * per, min(nkb_b, (s + 1) * per)
                if jb >= je:
                    continue
                cols = [(j * bk, min(Lmax, (j + 1) * bk)) for j in range(jb, je)]
                sk, gp = block_decisions(S, mask, None, cols, lam)
                exp_skip[jb:je] = sk
                exp_gap[jb:je] = gp
            exp_gap = np.array(exp_gap)
            fin = np.isfinite(exp_gap)
            np.testing.assert_allclose(r["gap"][b, g][fin], exp_gap[fin], rtol=0, atol=1e-9)
            assert np.array_equal(r["gap"][b, g][~fin], exp_gap[~fin])
            near = np.abs(exp_gap - math.log(lam)) < 1e-9
            assert np.array_equal(r["skip"][b, g][~near], np.array(exp_skip, np.uint8)[~near])


# ----------------------------------------------------- outputs of kept keys
def _kept_mask_prefill(skip, L, tq, bk, causal):
    """Visible and executed entries, for each (b, h): [L, L]."""
    B, Hq, nqt, nkb = skip.shape
    base = prefill_mask(L, causal)
    out = np.zeros((B, Hq, L, L), bool)
    for t in range(nqt):
        for j in range(nkb):
            ex = skip[:, :, t, j] == 0
            out[:, :, t * tq:(t + 1) * tq, j * bk:(j + 1) * bk] = ex[:, :, None, None]
    return out & base[None, None]


@pytest.mark.parametrize("seed", range(6))
def test_prefill_output_is_softmax_over_executed_keys(seed):
    """A skipped block changes nothing: O equals softmax attention over executed keys (<= 1e-12)."""
    rng = np.random.default_rng(500 + seed)
    L, tq, bk = 192, 32, 16
    causal = seed % 2 == 0
    q, k, v = _prefill_case(seed + 50, B=1, Hq=2, Hkv=2, L=L, d=8, dv=5, qstd=2.0, blocky=bk)
    r0 = oracle.prefill(q, k, v, causal=causal, lam=0.0, tile_q=tq, block_k=bk)
    lam = _lam_at(r0["gap"], rng.uniform(0.3, 0.8))
    r = oracle.prefill(q, k, v, causal=causal, lam=lam, tile_q=tq, block_k=bk)
    assert r["skipped"] > 0
    kept = _kept_mask_prefill(r["skip"], L, tq, bk, causal)
    scale = 1 / math.sqrt(8)
    for h in range(2):
        S = scores(q[0, h], k[0, h], scale)
        ref = masked_softmax_attention(S, kept[0, h], v[0, h])
        np.testing.assert_allclose(r["o"][0, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_decode_output_is_softmax_over_executed_keys(splits):
    """Split partials merged by log-sum-exp equal one softmax over the union of executed keys."""
    rng = np.random.default_rng(700 + splits)
    B, Hq, Hkv, Lmax, d, dv, bk = 2, 4, 1, 512, 8, 7, 32
    q = _rand(rng, B, Hq, d, std=2.0)
    k = _rand(rng, B, Hkv, Lmax, d, std=2.0)
    v = _rand(rng, B, Hkv, Lmax, dv)
    lens = np.array([512, 333])
    r0 = oracle.decode(q, k, v, lens, lam=0.0, block_k=bk, num_splits=splits)
    lam = _lam_at(r0["gap"], 0.6)
    r = oracle.decode(q, k, v, lens, lam=lam, block_k=bk, num_splits=splits)
    assert r["skipped"] > 0
    scale = 1 / math.sqrt(d)
    for b in range(B):
        ex = np.repeat(r["skip"][b, 0] == 0, bk)[:Lmax] & (np.arange(Lmax) < lens[b])
        S = scores(q[b], k[b, 0], scale)
        ref = masked_softmax_attention(S, np.broadcast_to(ex, S.shape), v[b, 0])
        np.testing.assert_allclose(r["o"][b], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------- mass bound
@pytest.mark.parametrize("seed", range(6))
def test_dropped_mass_bound(seed):
    """Per row, the dense-softmax mass of skipped keys is < lambda * (number of skipped keys)."""
    rng = np.random.default_rng(900 + seed)
    L, tq, bk, d = 256, 32, 16, 8
    q, k, v = _prefill_case(seed + 90, B=1, Hq=1, Hkv=1, L=L, d=d, dv=3, qstd=2.0, blocky=bk)
    r0 = oracle.prefill(q, k, v, causal=True, lam=0.0, tile_q=tq, block_k=bk)
    lam = _lam_at(r0["gap"], rng.uniform(0.3, 0.9))
    r = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=tq, block_k=bk)
    assert r["skipped"] > 0
    S = scores(q[0, 0], k[0, 0], 1 / math.sqrt(d))
    base = prefill_mask(L, True)
    p = dense_probs(S, base)
    kept = _kept_mask_prefill(r["skip"], L, tq, bk, True)[0, 0]
    dropped = base & ~kept
    mass = (p * dropped).sum(axis=1)
    nskip = dropped.sum(axis=1)
    assert np.all(mass <= lam * nskip + 1e-15)
    # and O is within the corresponding bound of dense attention
    dense = masked_softmax_attention(S, base, v[0, 0])
    err = np.abs(r["o"][0, 0] - dense).max(axis=1)
    span = v[0, 0].max(axis=0) - v[0, 0].min(axis=0)
    assert np.all(err <= mass * span.max() + 1e-12)


# ------------------------------------------------------------- invariants
def test_skip_set_monotone_in_lambda():
    q, k, v = _prefill_case(3, B=1, Hq=2, Hkv=1, L=256, d=8, dv=4, qstd=2.0, blocky=16)
    prev = None
    for lam in [0.0, 1e-6, 1e-4, 1e-3, 1e-2, 0.1, 0.5, 0.999]:
        r = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=32, block_k=16)
        s = r["skip"] == 1
        if prev is not None:
            assert np.all(s >= prev)
        prev = s
    assert prev.any()


def test_first_block_always_executed():
    q, k, v = _prefill_case(5, B=1, Hq=1, Hkv=1, L=200, d=8, dv=4, qstd=2.0)
    r = oracle.prefill(q, k, v, causal=True, lam=0.999999, tile_q=32, block_k=16)
    assert np.all(r["skip"][..., 0] == 0)
    assert np.all(np.isposinf(r["gap"][..., 0]))
    rng = np.random.default_rng(2)
    qd = _rand(rng, 2, 2, 8, std=2)
    kd = _rand(rng, 2, 1, 300, 8, std=2)
    vd = _rand(rng, 2, 1, 300, 3)
    rd = oracle.decode(qd, kd, vd, [300, 300], lam=0.999999, block_k=16, num_splits=4)
    nkb = 19  # ceil(300/16); per split = 5 blocks
    for s in range(4):
        assert np.all(rd["skip"][:, 0, s * 5] == 0)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _prefill_case(9, B=1, Hq=4, Hkv=2, L=150, d=8, dv=6, qstd=2.0)
    r1 = oracle.prefill(q, k, v, causal=True, lam=0.01, tile_q=32, block_k=16)
    r2 = oracle.prefill(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), causal=True,
                        lam=0.01, tile_q=32, block_k=16)
    assert np.array_equal(r1["o"], r2["o"])
    assert np.array_equal(r1["skip"], r2["skip"])


def test_causal_unvisited_blocks():
    """Causal tiles never visit blocks strictly above the diagonal."""
    q, k, v = _prefill_case(4, B=1, Hq=1, Hkv=1, L=256, d=8, dv=4)
    r = oracle.prefill(q, k, v, causal=True, lam=0.01, tile_q=64, block_k=32)
    for t in range(4):
        for j in range(8):
            visited = j * 32 <= t * 64 + 63
            assert (r["skip"][0, 0, t, j] != 255) == visited


def test_input_validation():
    q, k, v = _prefill_case(1, L=16)
    for bad in [-0.1, 1.0, float("nan")]:
        with pytest.raises(ValueError):
            oracle.prefill(q, k, v, lam=bad)
    with pytest.raises(ValueError):
        oracle.decode(q[:, :, 0], k, v, [0], lam=0.1)


# ------------------------------------------------------ hand-worked example
def test_worked_example_closed_form():
    """Hand-built cases whose scores, gaps, decisions and outputs are closed forms."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        examples = json.load(f)["examples"]
    for ex in examples:
        bk = ex["block_k"]
        kv = np.array(ex["key_values"], dtype=np.float64)  # scalar keys, d = 1
        L = kv.size
        q = np.array([[[ex["query"]]]])            # [B=1, Hq=1, d=1]
        k = kv.reshape(1, 1, L, 1)
        v = np.zeros((1, 1, L, 1))
        v[0, 0, ex["value_one_at"], 0] = 1.0       # V is the indicator of one key
        for case in ex["cases"]:
            r = oracle.decode(q, k, v, [L], scale=1.0, lam=case["lambda"], block_k=bk)
            assert list(r["skip"][0, 0]) == case["skip"], case
            assert np.array_equal(r["gap"][0, 0][1:], np.array(ex["gaps_after_first"]))
            # O = e^{s*} / sum over executed keys of e^{s}, with the key scores known exactly
            s = kv * ex["query"]
            ex_keys = np.repeat(np.array(case["skip"]) == 0, bk)
            expect = math.exp(s[ex["value_one_at"]]) / np.exp(s[ex_keys]).sum()
            assert abs(r["o"][0, 0, 0] - expect) < 1e-14


# --------------------------------------------------------------- calibration
def test_lambda_for_target_hits_target_exactly():
    q, k, v = _prefill_case(21, B=1, Hq=2, Hkv=1, L=512, d=8, dv=4, qstd=2.0, blocky=16)
    r0 = oracle.prefill(q, k, v, causal=True, lam=0.0, tile_q=32, block_k=16)
    vis = r0["skip"] != 255
    gaps = r0["gap"][vis]
    N = gaps.size
    for target in [0.3, 0.5, 0.7]:
        lam, reached = oracle.lambda_for_target(gaps, target)
        assert 0 < lam < 1
        r = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=32, block_k=16)
        frac = r["skipped"] / r["visited"]
        assert r["visited"] == N
        assert abs(frac - reached) < 1e-12
        assert abs(frac - target) <= 1.0 / N + 1e-12
        # ln(lambda) separates the ceil(target*N) smallest gaps from the rest with margin on both sides
        sg = np.sort(gaps)
        kk = math.ceil(target * N)
        assert sg[kk - 1] < math.log(lam) < sg[kk]


def test_fit_a_recovers_planted_a():
    Ls = np.array([4096, 8192, 16384, 32768, 65536])
    a = 37.5
    assert abs(oracle.fit_a(a / Ls, Ls) - a) < 1e-9 * a
    noisy = a / Ls * np.exp(np.array([0.1, -0.1, 0.05, -0.05, 0.0]))
    assert abs(oracle.fit_a(noisy, Ls) - a) < 1e-9 * a  # log-noise averaging to 0


def test_lambda_from_table():
    t, a = [0.3, 0.5, 0.7], [2.0, 8.0, 32.0]
    assert abs(oracle.lambda_from_table(t, a, 0.5, 1000) - 8.0 / 1000) < 1e-15
    assert abs(oracle.lambda_from_table(t, a, 0.6, 1000) - 16.0 / 1000) < 1e-15  # geometric midpoint
    assert abs(oracle.lambda_from_table(t, a, 0.4, 2000) - 4.0 / 2000) < 1e-15


# --------------------------------------------------------------- paged cache
def test_gather_pages_inverts_a_page_scatter():
    """Writing each sequence's rows page by page into a shuffled pool (an
    explicit loop here, the inverse operation) and gathering them back
    returns the original rows; rows past a sequence's length come back 0."""
    rng = np.random.default_rng(7)
    B, H, Lmax, d, P = 3, 2, 100, 5, 16
    lens = [100, 1, 37]
    cache = rng.standard_normal((B, H, Lmax, d))
    need = [-(-n // P) for n in lens]
    order = rng.permutation(sum(need) + 4)
    pool = np.full((order.size, H, P, d), np.nan)
    table = np.full((B, -(-Lmax // P)), -1, np.int64)
    nxt = 0
    for b in range(B):
        for i in range(need[b]):
            page = order[nxt]
            nxt += 1
            table[b, i] = page
            for r in range(i * P, min((i + 1) * P, lens[b])):
                pool[page, :, r - i * P, :] = cache[b, :, r, :]
    got = oracle.gather_pages(pool, table, lens, Lmax)
    for b in range(B):
        np.testing.assert_array_equal(got[b, :, :lens[b]], cache[b, :, :lens[b]])
        assert not got[b, :, lens[b]:].any()


def test_gather_pages_single_page_per_sequence_is_the_pool():
    """One page of Lmax rows per sequence with table b -> b: the pool is the cache."""
    rng = np.random.default_rng(8)
    pool = rng.standard_normal((3, 2, 64, 4))
    got = oracle.gather_pages(pool, np.arange(3)[:, None], [64, 64, 64], 64)
    np.testing.assert_array_equal(got, pool)


def test_gather_pages_rejects_a_page_outside_the_pool():
    pool = np.zeros((2, 1, 16, 4))
    with pytest.raises(ValueError):
        oracle.gather_pages(pool, np.array([[0, 2]]), [20], 32)


# ------------------------------------------------------------ sliding window
# Reading: query i sees keys i - W < c <= i; decode's query sits at len-1 and
# its splits cut the blocks from the first one that holds a visible key.

@pytest.mark.parametrize("L,W,tq,bk", [(300, 100, 64, 64), (257, 64, 128, 64), (200, 1, 32, 16),
                                       (130, 129, 64, 32), (90, 7, 16, 8)])
def test_window_lambda0_is_band_softmax(L, W, tq, bk):
    q, k, v = _prefill_case(40 + W, B=1, Hq=2, Hkv=1, L=L)
    r = oracle.prefill(q, k, v, causal=True, lam=0.0, tile_q=tq, block_k=bk, window=W)
    mask = prefill_mask(L, True, W)
    for h in range(2):
        S = scores(q[0, h], k[0, 0], 1 / math.sqrt(q.shape[-1]))
        np.testing.assert_allclose(r["o"][0, h], masked_softmax_attention(S, mask, v[0, 0]), rtol=0, atol=1e-10)
    # a block is visited iff some row of the tile sees one of its keys
    for t in range(-(-L // tq)):
        for j in range(-(-L // bk)):
            seen = mask[t * tq:(t + 1) * tq, j * bk:(j + 1) * bk].any()
            assert (r["skip"][0, 0, t, j] != 255) == seen


@pytest.mark.parametrize("seed", range(8))
def test_window_prefill_decisions_match_bruteforce(seed):
    rng = np.random.default_rng(500 + seed)
    L = int(rng.integers(60, 260))
    tq = int(rng.choice([16, 32, 64]))
    bk = int(rng.choice([8, 16, 32]))
    W = int(rng.integers(1, L))
    q, k, v = _prefill_case(seed + 50, B=1, Hq=2, Hkv=1, L=L, d=8, dv=4, qstd=2.0, blocky=bk)
    _, g0 = _prefill_brute_decisions(q, k, 0.0, True, tq, bk, W)
    lam = _lam_at(g0, rng.uniform(0.2, 0.8))
    r = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=tq, block_k=bk, window=W)
    skip, gap = _prefill_brute_decisions(q, k, lam, True, tq, bk, W)
    fin = np.isfinite(gap)
    np.testing.assert_allclose(r["gap"][fin], gap[fin], rtol=0, atol=1e-9)
    assert np.array_equal(r["gap"][~fin], gap[~fin])
    near = np.abs(gap - math.log(lam)) < 1e-9
    assert np.array_equal(r["skip"][~near], skip[~near])
    assert r["visited"] == int((skip != 255).sum())


def test_window_of_one_returns_the_own_value():
    """W = 1: every query sees only itself, so O[i] = V[i] whatever lambda is."""
    q, k, v = _prefill_case(61, B=1, Hq=1, Hkv=1, L=150, d=8, dv=5)
    for lam in (0.0, 0.5):
        r = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=64, block_k=16, window=1)
        np.testing.assert_allclose(r["o"][0, 0], v[0, 0], rtol=0, atol=1e-15)


def test_window_covering_the_sequence_is_plain_causal():
    q, k, v = _prefill_case(62, B=1, Hq=2, Hkv=1, L=200, blocky=16)
    lam = 0.05
    a = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=32, block_k=16)
    for W in (200, 500):
        b = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=32, block_k=16, window=W)
        for key in ("o", "skip", "gap"):
            assert np.array_equal(a[key], b[key])
    rng = np.random.default_rng(63)
    qd, kd, vd = _rand(rng, 2, 4, 8, std=2.0), _rand(rng, 2, 2, 300, 8, std=2.0), _rand(rng, 2, 2, 300, 6)
    lens = np.array([300, 77])
    a = oracle.decode(qd, kd, vd, lens, lam=lam, block_k=16, num_splits=3)
    b = oracle.decode(qd, kd, vd, lens, lam=lam, block_k=16, num_splits=3, window=300)
    for key in ("o", "skip", "gap"):
        assert np.array_equal(a[key], b[key])


@pytest.mark.parametrize("W", [1, 50, 64, 65, 200])
def test_window_decode_is_the_last_prefill_row(W):
    """One split, one head per KV head: the decode unit of a sequence of length
    L is the prefill unit of its last position (tile of one row)."""
    rng = np.random.default_rng(64 + W)
    L, d, dv = 300, 8, 6
    q, k, v = _rand(rng, 1, 1, L, d, std=2.0), _rand(rng, 1, 1, L, d, std=2.0), _rand(rng, 1, 1, L, dv)
    lam = 0.02
    p = oracle.prefill(q, k, v, causal=True, lam=lam, tile_q=1, block_k=32, window=W)
    r = oracle.decode(q[:, :, -1], k, v, np.array([L]), lam=lam, block_k=32, num_splits=1, window=W)
    np.testing.assert_allclose(r["o"][0, 0], p["o"][0, 0, -1], rtol=0, atol=1e-14)
    assert np.array_equal(r["skip"][0, 0], p["skip"][0, 0, -1])
    np.testing.assert_allclose(r["gap"][0, 0], p["gap"][0, 0, -1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_window_decode_decisions_and_split_origin(seed):
    """Decisions by the closed form of the running max over the band, with
    the splits cutting the blocks that meet the window; merged output equals
    softmax over the executed keys."""
    rng = np.random.default_rng(700 + seed)
    B, Hq, Hkv, Lmax, d, dv, bk = 2, 4, 2, int(rng.integers(200, 500)), 8, 6, 16
    splits = int(rng.integers(2, 5))
    q = _rand(rng, B, Hq, d, std=2.0)
    k = _rand(rng, B, Hkv, Lmax, d, std=2.0)
    v = _rand(rng, B, Hkv, Lmax, dv)
    lens = rng.integers(Lmax // 2, Lmax + 1, size=B)
    W = int(rng.integers(bk + 1, Lmax // 2))
    lam = float(10 ** rng.uniform(-4, -1))
    r = oracle.decode(q, k, v, lens, lam=lam, block_k=bk, num_splits=splits, window=W)
    G, scale, nkb = Hq // Hkv, 1 / math.sqrt(d), -(-Lmax // bk)
    for b in range(B):
        n = int(lens[b])
        j0 = max(0, n - W) // bk
        nkb_b = -(-n // bk)
        per = -(-(nkb_b - j0) // splits)
        keys = np.arange(Lmax)
        for g in range(Hkv):
            S = scores(q[b, g * G:(g + 1) * G], k[b, g], scale)
            mask = np.broadcast_to((keys < n) & (keys >= n - W), S.shape)
            exp_skip, exp_gap = [255] * nkb, [-math.inf] * nkb
            for s in range(splits):
                jb, je = j0 + s * per, min(nkb_b, j0 + (s + 1) * per)
                if jb >= je:
                    continue
                cols = [(j * bk, min(Lmax, (j + 1) * bk)) for j in range(jb, je)]
                exp_skip[jb:je], exp_gap[jb:je] = block_decisions(S, mask, None, cols, lam)
                assert exp_gap[jb] == math.inf  # each split starts from m = -inf
            exp_gap = np.array(exp_gap)
            fin = np.isfinite(exp_gap)
            np.testing.assert_allclose(r["gap"][b, g][fin], exp_gap[fin], rtol=0, atol=1e-9)
            assert np.array_equal(r["gap"][b, g][~fin], exp_gap[~fin])
            near = np.abs(exp_gap - math.log(lam)) < 1e-9
            assert np.array_equal(r["skip"][b, g][~near], np.array(exp_skip, np.uint8)[~near])
            # output = softmax over the visible keys of executed blocks
            ex = np.repeat(r["skip"][b, g] == 0, bk)[:Lmax]
            for hh in range(G):
                ref = masked_softmax_attention(S[hh:hh + 1], (mask[hh] & ex)[None], v[b, g])[0]
                np.testing.assert_allclose(r["o"][b, g * G + hh], ref, rtol=0, atol=1e-10)


# -------------------------------------------------------- sink-seeded splits
# Reading: split s >= 1 starts its running max from the row maxima of the
# sequence's first visible block; split 0 starts from -inf.

def _seed_case(seed, Lmax=400, bk=16, W=0):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, dv = 2, 4, 2, 8, 6
    q = _rand(rng, B, Hq, d, std=2.0)
    k = _rand(rng, B, Hkv, Lmax, d, std=2.0)
    f = rng.uniform(0.05, 1.0, size=(B, Hkv, -(-Lmax // bk)))
    f[..., 0] = 2.5  # a hot sink block
    k = k * np.repeat(f, bk, axis=2)[..., :Lmax, None]
    v = _rand(rng, B, Hkv, Lmax, dv)
    lens = np.array([Lmax, int(rng.integers(Lmax // 2, Lmax))])
    return q, k, v, lens


@pytest.mark.parametrize("seed,W", [(0, 0), (1, 0), (2, 0), (3, 150), (4, 0), (5, 90)])
def test_sink_seed_decisions_and_output(seed, W):
    """Decisions by the closed form with the seeded running max, and the
    merged output equal to softmax over the executed keys."""
    q, k, v, lens = _seed_case(800 + seed, W=W)
    bk, splits = 16, 4
    B, Hq, dd = q.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    G, scale, nkb = Hq // Hkv, 1 / math.sqrt(dd), -(-Lmax // bk)
    g0 = oracle.decode(q, k, v, lens, lam=0.0, block_k=bk, num_splits=splits, window=W, sink_seed=True)["gap"]
    lam = _lam_at(g0, 0.5)
    r = oracle.decode(q, k, v, lens, lam=lam, block_k=bk, num_splits=splits, window=W, sink_seed=True)
    keys = np.arange(Lmax)
    seeded_first_skips = 0
    for b in range(B):
        n = int(lens[b])
        lo = max(0, n - W) if W else 0
        j0 = lo // bk
        nkb_b = -(-n // bk)
        per = -(-(nkb_b - j0) // splits)
        for g in range(Hkv):
            S = scores(q[b, g * G:(g + 1) * G], k[b, g], scale)
            vis = (keys < n) & (keys >= lo)
            mask = np.broadcast_to(vis, S.shape)
            blk0 = slice(j0 * bk, (j0 + 1) * bk)
            seed_max = np.where(mask[:, blk0], S[:, blk0], -np.inf).max(axis=1)
            exp_skip, exp_gap = [255] * nkb, [-math.inf] * nkb
            for s in range(splits):
                jb, je = j0 + s * per, min(nkb_b, j0 + (s + 1) * per)
                if jb >= je:
                    continue
                cols = [(j * bk, min(Lmax, (j + 1) * bk)) for j in range(jb, je)]
                init = seed_max if s > 0 else None
                exp_skip[jb:je], exp_gap[jb:je] = block_decisions(S, mask, None, cols, lam, init=init)
                if s > 0 and exp_skip[jb] == 1:
                    seeded_first_skips += 1
            exp_gap = np.array(exp_gap)
            fin = np.isfinite(exp_gap)
            np.testing.assert_allclose(r["gap"][b, g][fin], exp_gap[fin], rtol=0, atol=1e-9)
            assert np.array_equal(r["gap"][b, g][~fin], exp_gap[~fin])
            near = np.abs(exp_gap - math.log(lam)) < 1e-9
            assert np.array_equal(r["skip"][b, g][~near], np.array(exp_skip, np.uint8)[~near])
            ex = np.repeat(r["skip"][b, g] == 0, bk)[:Lmax]
            for hh in range(G):
                ref = masked_softmax_attention(S[hh:hh + 1], (vis & ex)[None], v[b, g])[0]
                np.testing.assert_allclose(r["o"][b, g * G + hh], ref, rtol=0, atol=1e-10)
    assert seeded_first_skips > 0  # the seed does let a split skip its first block


def test_sink_seed_with_one_split_changes_nothing():
    q, k, v, lens = _seed_case(810)
    a = oracle.decode(q, k, v, lens, lam=0.05, block_k=16, num_splits=1)
    b = oracle.decode(q, k, v, lens, lam=0.05, block_k=16, num_splits=1, sink_seed=True)
    for key in ("o", "skip", "gap"):
        assert np.array_equal(a[key], b[key])


@pytest.mark.parametrize("seed", range(4))
def test_sink_seed_skips_a_superset_and_keeps_the_mass_bound(seed):
    """The seed only raises the running max: gaps shrink, the skip set grows,
    and the dropped dense-softmax mass stays below lambda per skipped key."""
    q, k, v, lens = _seed_case(820 + seed)
    lam = 0.02
    a = oracle.decode(q, k, v, lens, lam=lam, block_k=16, num_splits=5)
    b = oracle.decode(q, k, v, lens, lam=lam, block_k=16, num_splits=5, sink_seed=True)
    vis = a["skip"] != 255
    assert np.array_equal(vis, b["skip"] != 255)
    assert np.all(b["gap"][vis] <= a["gap"][vis])
    assert np.all(b["skip"][a["skip"] == 1] == 1)
    assert b["skipped"] > a["skipped"]
    B, Hq, dd = q.shape
    G, scale, Lmax = Hq // k.shape[1], 1 / math.sqrt(dd), k.shape[2]
    for bb in range(B):
        n = int(lens[bb])
        for h in range(Hq):
            S = scores(q[bb, h][None], k[bb, h // G], scale)[0, :n]
            p = np.exp(S - S.max())
            p /= p.sum()
            sk = np.repeat(b["skip"][bb, h // G] == 1, 16)[:n]
            assert p[sk].sum() < lam * max(1, sk.sum())


def test_sink_seed_fully_skipped_split_contributes_nothing():
    """A split whose blocks are all far colder than the sink skips everything
    (l = 0); the merge ignores it and O is softmax over the executed keys."""
    rng = np.random.default_rng(830)
    Lmax, d, dv, bk = 256, 8, 4, 16
    q = np.ones((1, 1, d))
    k = np.zeros((1, 1, Lmax, d))
    k[0, 0, :bk] = 3.0                        # sink: score 3*8/sqrt(8)
    k[0, 0, bk:] = rng.standard_normal((Lmax - bk, d)) * 0.01
    k[0, 0, 192:] = 2.9                       # last split: scores 0.3 below the sink, executed
    v = rng.standard_normal((1, 1, Lmax, dv))
    lam = 0.05
    r = oracle.decode(q, k, v, np.array([Lmax]), lam=lam, block_k=bk, num_splits=4, sink_seed=True)
    sk = r["skip"][0, 0]
    assert np.all(sk[4:12] == 1)              # splits 1 and 2: every block skipped
    assert sk[0] == 0 and np.all(sk[12:] == 0)
    S = scores(q[0], k[0, 0], 1 / math.sqrt(d))
    ex = np.repeat(sk == 0, bk)
    ref = masked_softmax_attention(S, ex[None], v[0, 0])[0]
    np.testing.assert_allclose(r["o"][0, 0], ref, rtol=0, atol=1e-12)


# --------------------------------------------- non-finite inputs (reading R24)
# The pages say nothing about NaN or infinite inputs.  The reading both sides
# implement: block maxima and the tile gap ignore NaN; in an executed block
# every key that some row of the unit sees enters every row with weight
# p (0 for a row that does not see it, and 0 * inf = 0 * NaN = NaN); keys no
# row sees enter nothing; O = acc / l for l != 0, exactly 0 for l = 0; the
# split merge keeps every split with l != 0.  Each pin below derives the
# expected outcome from these rules and IEEE arithmetic by hand.

def _finite_case(seed, L, d=8, dv=6, Hkv=1, Hq=1):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((1, Hq, L, d)), rng.standard_normal((1, Hkv, L, d)),
            rng.standard_normal((1, Hkv, L, dv)))


def test_nan_score_makes_exactly_the_rows_that_see_it_nan():
    """K[5] = NaN: every row that sees key 5 has a NaN weight, hence a NaN sum and
    a NaN output; rows 0..4 do not see it (causal) and stay plain softmax."""
    L = 130
    q, k, v = _finite_case(31, L)
    k[0, 0, 5, :] = np.nan
    r = oracle.prefill(q, k, v, causal=True, lam=0.0, tile_q=64, block_k=64)
    o = r["o"][0, 0]
    assert np.isnan(o[5:]).all()
    S = scores(q[0, 0], k[0, 0], 1 / math.sqrt(8))
    ref = masked_softmax_attention(S[:5, :5], prefill_mask(5, True), v[0, 0, :5])
    assert np.abs(o[:5] - ref).max() <= 1e-12


def test_nonfinite_v_reaches_every_row_of_a_tile_that_executes_its_block():
    """V[5, 0] = +inf, V[70, 1] = NaN, lambda = 0 (every visited block executes).
    Tile 0 (rows 0..63): rows 0..4 do not see key 5 but it is seen by rows
    5..63, so they add 0 * inf = NaN; rows 5..63 add p * inf = +inf.  Tile 1
    (rows 64..127): all see key 5 (+inf); key 70 is seen by rows 70..127, so
    rows 64..69 add 0 * NaN and everyone is NaN at feature 1.  Later tiles see
    both keys.  Every other feature is plain causal softmax."""
    L = 200
    q, k, v = _finite_case(32, L)
    v[0, 0, 5, 0] = np.inf
    v[0, 0, 70, 1] = np.nan
    o = oracle.prefill(q, k, v, causal=True, lam=0.0, tile_q=64, block_k=64)["o"][0, 0]
    assert np.isnan(o[:5, 0]).all() and np.isposinf(o[5:, 0]).all()
    assert np.isfinite(o[:64, 1]).all() and np.isnan(o[64:, 1]).all()
    S = scores(q[0, 0], k[0, 0], 1 / math.sqrt(8))
    ref = masked_softmax_attention(S, prefill_mask(L, True), v[0, 0, :, 2:])
    assert np.abs(o[:, 2:] - ref).max() <= 1e-12
    fin = np.isfinite(v[0, 0, :, 1])
    ref1 = masked_softmax_attention(S[:64, :64], prefill_mask(64, True), v[0, 0, :64, 1:2])
    assert np.abs(o[:64, 1:2] - ref1).max() <= 1e-12 and fin[:64].all()


def test_rows_that_have_seen_no_key_gather_zero_weighted_values():
    """Window W = 1 (row i sees key i only), tile 128: in block 0 rows 64..127
    see no key yet, but keys 0..63 are seen by rows 0..63, so those rows gather
    0 * V; with V[3, 0] = NaN all 128 rows of tile 0 end NaN at feature 0
    (a later rescale by 0 keeps the NaN).  Tile 1 visits blocks 2 and 3 only.
    Every other value is V itself (W = 1)."""
    L = 256
    q, k, v = _finite_case(33, L)
    v[0, 0, 3, 0] = np.nan
    o = oracle.prefill(q, k, v, causal=True, lam=0.0, tile_q=128, block_k=64, window=1)["o"][0, 0]
    assert np.isnan(o[:128, 0]).all()
    assert np.array_equal(o[128:, 0], v[0, 0, 128:, 0])
    assert np.abs(o[:, 1:] - v[0, 0, :, 1:]).max() <= 1e-12


def test_keys_no_row_of_the_tile_sees_contribute_nothing():
    """Window W = 100, tile 128: tile 1 (rows 128..255) visits block 0 for keys
    29..63, which row 128 sees; keys 0..28 are seen by no row of tile 1, so
    V[10, 0] = +inf leaves tile 1 finite, while every row of tile 0 sees or
    shares key 10 and is non-finite at feature 0."""
    L = 256
    q, k, v = _finite_case(34, L)
    v[0, 0, 10, 0] = np.inf
    o = oracle.prefill(q, k, v, causal=True, lam=0.0, tile_q=128, block_k=64, window=100)["o"][0, 0]
    assert not np.isfinite(o[:110, 0]).any()     # rows 0..109 see key 10 or share its block with rows that do
    assert np.isfinite(o[128:, 0]).all()
    S = scores(q[0, 0], k[0, 0], 1 / math.sqrt(8))
    # rows 128..255 see keys 29..255 only
    ref = masked_softmax_attention(S[128:, 29:], prefill_mask(L, True, 100)[128:, 29:], v[0, 0, 29:])
    assert np.abs(o[128:] - ref).max() <= 1e-12


def test_nan_row_sum_propagates_through_the_split_merge():
    """Decode, 2 splits of 128 keys: K[200] = NaN makes split 1's sum NaN for
    both heads; the merge keeps splits with l != 0, so O is NaN everywhere.
    Without the NaN, the two-split merge equals plain softmax."""
    rng = np.random.default_rng(35)
    q, k, v = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 1, 256, 8)), rng.standard_normal((1, 1, 256, 5))
    lens = np.array([256])
    base = oracle.decode(q, k, v, lens, lam=0.0, block_k=64, num_splits=2)["o"]
    S = scores(q[0], k[0, 0], 1 / math.sqrt(8))
    assert np.abs(base[0] - masked_softmax_attention(S, np.ones_like(S, bool), v[0, 0])).max() <= 1e-12
    k[0, 0, 200, :] = np.nan
    o = oracle.decode(q, k, v, lens, lam=0.0, block_k=64, num_splits=2)["o"]
    assert np.isnan(o).all()


def _nan_aware_decisions(S, mask, blocks, lam):
    """Decisions by the closed form with the R24 rules: per-row block maxima
    ignore NaN, the running max is their prefix maximum, a NaN row gap never
    blocks a skip."""
    lnlam = -math.inf if lam == 0 else math.log(lam)
    R = S.shape[0]
    prev = np.full(R, -np.inf)
    skips = []
    for c0, c1 in blocks:
        mb = mask[:, c0:c1]
        if not mb.any():
            skips.append(255)
            continue
        vals = np.where(mb, S[:, c0:c1], -np.inf)
        mt = np.array([max([x for x in row if not np.isnan(x)], default=-np.inf) for row in vals])
        with np.errstate(invalid="ignore"):
            d = np.where(mt == -np.inf, -np.inf, np.where(prev == -np.inf, np.inf, mt - prev))
        d = d[~np.isnan(d)]
        g = d.max() if d.size else -np.inf
        skips.append(1 if g < lnlam else 0)
        prev = np.fmax(prev, mt)
    return skips


def test_infinite_query_row_gives_nan_output_and_never_blocks_a_skip():
    """Q[10] = (+inf, 0, ..., 0): row 10's scores are +inf or -inf by the sign
    of k[:, 0]; its running max becomes +inf at its first block, after which its
    gaps are NaN or -inf and never keep the tile from skipping.  Its output is
    NaN (weight exp(inf - inf)); decisions equal the closed form."""
    L, tq = 320, 64
    q, k, v = _prefill_case(36, B=1, Hq=1, Hkv=1, L=L, d=8, dv=6, qstd=2.5, blocky=64)
    q[0, 0, 10, :] = 0.0
    q[0, 0, 10, 0] = np.inf
    r0 = oracle.prefill(q, k, v, causal=False, lam=0.0, tile_q=tq, block_k=64)
    lam = _lam_at(r0["gap"][np.isfinite(r0["gap"])], 0.5)
    r = oracle.prefill(q, k, v, causal=False, lam=lam, tile_q=tq, block_k=64)
    assert r["skipped"] > 0
    assert np.isnan(r["o"][0, 0, 10]).all()
    assert np.isfinite(np.delete(r["o"][0, 0], 10, axis=0)).all()
    with np.errstate(invalid="ignore"):
        S = 0.0 + np.einsum("id,cd->ic", q[0, 0], k[0, 0]) / math.sqrt(8)
    mask = np.ones((L, L), bool)
    for t in range(L // tq):
        rows = slice(t * tq, (t + 1) * tq)
        want = _nan_aware_decisions(S[rows], mask[rows], [(c, c + 64) for c in range(0, L, 64)], lam)
        assert list(r["skip"][0, 0, t]) == want, t


def test_nan_scores_are_ignored_by_the_block_max():
    """A NaN key (K[191] = NaN, the last key of block 2) gives NaN scores in
    block 2 for every row; the block max and the running max ignore them, so
    the decisions are those of the closed form over the finite scores
    (non-causal, lambda at the median gap), and every row of a tile that
    executes block 2 is NaN."""
    L, tq = 320, 64
    q, k, v = _prefill_case(37, B=1, Hq=1, Hkv=1, L=L, d=8, dv=6, qstd=2.5, blocky=64)
    r0 = oracle.prefill(q, k, v, causal=False, lam=0.0, tile_q=tq, block_k=64)
    lam = _lam_at(r0["gap"][np.isfinite(r0["gap"])], 0.5)
    k[0, 0, 191, :] = np.nan
    r = oracle.prefill(q, k, v, causal=False, lam=lam, tile_q=tq, block_k=64)
    with np.errstate(invalid="ignore"):
        S = np.einsum("id,cd->ic", q[0, 0], k[0, 0]) / math.sqrt(8)
    mask = np.ones((L, L), bool)
    nskip = 0
    for t in range(L // tq):
        rows = slice(t * tq, (t + 1) * tq)
        want = _nan_aware_decisions(S[rows], mask[rows], [(c, c + 64) for c in range(0, L, 64)], lam)
        assert list(r["skip"][0, 0, t]) == want, t
        nskip += sum(x == 1 for x in want)
        if want[2] == 0:
            assert np.isnan(r["o"][0, 0, rows]).all()
    assert nskip > 0

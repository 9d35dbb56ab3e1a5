"""Seeded synthetic inputs for block-skipping attention (shared by the HIP path's
tests and benchmark and by the oracle checks).

This module only draws random tensors; it holds none of the attention
arithmetic.  The recipe imitates the structure that the BLASST pages report
for long-context attention (a "sink" block that every query attends to, the
query's local segment, and a few retrieved earlier segments), so that block
sparsity arises the way the method expects:

* keys are cut into segments of ``seg`` tokens (one segment per 64-key block);
  each segment of each KV head has a center ~ N(0, center_std^2 I), and each key
  is its segment's center plus N(0, I) noise;
* a query is the SUM of the centers of its picked segments plus N(0, I) noise,
  where the picks are: the sink segment 0, the last ``local_window`` segments
  ending at the query's own segment, and ``n_random`` segments drawn uniformly
  with replacement from the earlier segments 1 .. own-1 (own when there are
  none).  Prefill draws the random picks once per (batch, query head, 64-query
  segment); decode draws them once per sequence and shares them by all heads;
* V ~ N(0, I).

All tensors are generated in float32 with a ``torch.Generator`` seeded on the
target device and then rounded (round-to-nearest-even) to ``dtype``.
"""
from __future__ import annotations

import torch


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _picks(nseg_q, n_random, sink, local_window, shape, g, device):
    """Segment picks for every query segment: int64 [*shape, nseg_q, P]."""
    sig = torch.arange(nseg_q, device=device)
    cols = []
    if sink:
        cols.append(torch.zeros(nseg_q, dtype=torch.long, device=device))
    for i in range(local_window):
        cols.append((sig - i).clamp_min(0))
    fixed = torch.stack(cols, -1) if cols else torch.zeros(nseg_q, 0, dtype=torch.long, device=device)
    fixed = fixed.expand(*shape, nseg_q, fixed.shape[-1])
    if n_random == 0:
        return fixed.contiguous()
    u = torch.rand(*shape, nseg_q, n_random, generator=g, device=device)
    span = (sig - 1).clamp_min(1).to(torch.float32)  # number of segments 1 .. own-1
    rnd = 1 + torch.floor(u * span[:, None]).to(torch.long)
    rnd = torch.where((sig <= 1)[:, None], sig[:, None].expand_as(rnd), rnd)
    return torch.cat([fixed, rnd], -1).contiguous()


def prefill_inputs(B, Hq, Hkv, L, d, dv=None, *, seg=64, center_std=2.0, n_random=6,
                   sink=True, local_window=1, dtype=torch.bfloat16, device="cpu", seed=0):
    """Segment-center inputs for causal prefill.

    Returns (q [B,Hq,L,d], k [B,Hkv,L,d], v [B,Hkv,L,dv]) in ``dtype``.
    """
    dv = d if dv is None else dv
    assert Hq % Hkv == 0
    g = _gen(device, seed)
    nseg = -(-L // seg)
    tok_seg = torch.arange(L, device=device) // seg
    centers = torch.randn(B, Hkv, nseg, d, generator=g, device=device) * center_std
    k = centers[:, :, tok_seg, :] + torch.randn(B, Hkv, L, d, generator=g, device=device)
    picks = _picks(nseg, n_random, sink, local_window, (B, Hq), g, device)  # [B,Hq,nseg,P]
    hk = torch.arange(Hq, device=device) // (Hq // Hkv)
    cq = centers[:, hk]  # [B,Hq,nseg,d]
    P = picks.shape[-1]
    qseg = torch.zeros(B, Hq, nseg, d, device=device)
    for p in range(P):
        idx = picks[..., p:p + 1].expand(B, Hq, nseg, d)
        qseg += torch.gather(cq, 2, idx)
    q = qseg[:, :, tok_seg, :] + torch.randn(B, Hq, L, d, generator=g, device=device)
    v = torch.randn(B, Hkv, L, dv, generator=g, device=device)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def decode_inputs(B, Hq, Hkv, L, dqk, dv=None, *, seg=64, center_std=2.0, n_random=8,
                  sink=True, mla=False, dtype=torch.bfloat16, device="cpu", seed=0,
                  seq_lens=None, chunk=8):
    """Segment-center inputs for decode (one query token per sequence).

    Returns (q [B,Hq,dqk], k_cache [B,Hkv,L,dqk], v_cache, seq_lens int32 [B]).
    With ``mla=True`` there is no separate V cache (``v_cache`` is None): the
    value of a token is the first ``dv`` columns of its latent K row.
    The caches are generated ``chunk`` sequences at a time to bound the
    float32 temporaries.
    """
    dv = dqk if dv is None else dv
    assert Hq % Hkv == 0
    g = _gen(device, seed)
    nseg = -(-L // seg)
    tok_seg = torch.arange(L, device=device) // seg
    G = Hq // Hkv
    k = torch.empty(B, Hkv, L, dqk, dtype=dtype, device=device)
    v = None if mla else torch.empty(B, Hkv, L, dv, dtype=dtype, device=device)
    q = torch.empty(B, Hq, dqk, dtype=dtype, device=device)
    for b0 in range(0, B, chunk):
        nb = min(chunk, B - b0)
        centers = torch.randn(nb, Hkv, nseg, dqk, generator=g, device=device) * center_std
        kk = centers[:, :, tok_seg, :]
        kk += torch.randn(nb, Hkv, L, dqk, generator=g, device=device)
        k[b0:b0 + nb] = kk.to(dtype)
        del kk
        # picks shared by all heads of a sequence: sink + n_random uniform from 1..nseg-1
        npk = n_random + (1 if sink else 0)
        u = torch.rand(nb, n_random, generator=g, device=device)
        rnd = 1 + torch.floor(u * max(nseg - 1, 1)).to(torch.long)
        rnd = rnd.clamp_max(nseg - 1)
        picks = torch.cat([torch.zeros(nb, 1, dtype=torch.long, device=device), rnd], 1) if sink else rnd
        qs = torch.zeros(nb, Hkv, dqk, device=device)
        for p in range(npk):
            idx = picks[:, p].view(nb, 1, 1, 1).expand(nb, Hkv, 1, dqk)
            qs += torch.gather(centers, 2, idx)[:, :, 0, :]
        qq = qs.repeat_interleave(G, dim=1) + torch.randn(nb, Hq, dqk, generator=g, device=device)
        q[b0:b0 + nb] = qq.to(dtype)
        if not mla:
            v[b0:b0 + nb] = torch.randn(nb, Hkv, L, dv, generator=g, device=device).to(dtype)
    if seq_lens is None:
        seq_lens = torch.full((B,), L, dtype=torch.int32, device=device)
    else:
        seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32, device=device)
    return q, k, v, seq_lens


def random_inputs(shape_q, shape_k, shape_v, *, dtype=torch.float64, device="cpu", seed=0, std=1.0):
    """Plain N(0, std^2) tensors (edge-case and property tests)."""
    g = _gen(device, seed)
    q = (torch.randn(*shape_q, generator=g, device=device) * std).to(dtype)
    k = (torch.randn(*shape_k, generator=g, device=device) * std).to(dtype)
    v = torch.randn(*shape_v, generator=g, device=device).to(dtype)
    return q, k, v


def paged_pool(caches, seq_lens, page_size, *, seed=0, spare_pages=0, fill=float("nan"),
               row_major_heads=False):
    """Scatter contiguous caches [B, H, Lmax, d] into a shuffled page pool.

    The pages of all sequences take a seeded random order among
    ``num_pages = used + spare_pages`` pool pages; every pool row that holds
    no token of a sequence (rows past seq_len in a sequence's last page, spare
    pages) is ``fill`` (NaN by default, so a read of such a row shows up in
    the result).  All caches share one page table (a KV cache's K and V).

    Returns (pools, page_table): each pool is an [num_pages, H, page_size, d]
    tensor (with ``row_major_heads`` a permuted view of [num_pages,
    page_size, H, d] storage), and page_table is int32 [B, ceil(Lmax /
    page_size)] on the caches' device, -1 past each sequence's pages.
    """
    B, H, Lmax, _ = caches[0].shape
    dev = caches[0].device
    lens = [int(x) for x in (seq_lens.tolist() if torch.is_tensor(seq_lens) else seq_lens)]
    npg = [-(-ln // page_size) for ln in lens]
    used = sum(npg)
    total = used + spare_pages
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(total, generator=g)[:used]
    table = torch.full((B, -(-Lmax // page_size)), -1, dtype=torch.int32)
    pools = []
    for c in caches:
        d = c.shape[3]
        if row_major_heads:
            pool = torch.full((total, page_size, H, d), fill, dtype=c.dtype, device=dev).permute(0, 2, 1, 3)
        else:
            pool = torch.full((total, H, page_size, d), fill, dtype=c.dtype, device=dev)
        pools.append(pool)
    off = 0
    for b in range(B):
        ids = perm[off:off + npg[b]]
        off += npg[b]
        table[b, :npg[b]] = ids.to(torch.int32)
        if npg[b] == 0:
            continue
        idx = ids.to(dev)
        for c, pool in zip(caches, pools):
            rows = torch.full((H, npg[b] * page_size, c.shape[3]), fill, dtype=c.dtype, device=dev)
            rows[:, :lens[b]] = c[b, :, :lens[b]]
            pool[idx] = rows.view(H, npg[b], page_size, c.shape[3]).permute(1, 0, 2, 3)
    return pools, table.to(dev)

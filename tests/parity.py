"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same inputs (bf16 values upcast exactly to fp64), and
compare with the tolerances of the method's parity bar:

* O: max-abs error <= 1e-2 and mean-abs error <= 1e-3;
* skip decisions identical except where the oracle's tile gap lies within
  1e-3 of ln(lambda) (there the fp32 and fp64 sides may legitimately differ);
* block sparsity within 0.5% absolute.
"""
import math

import numpy as np
import torch

import long_context_fa_amd as bl
import oracle

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
GAP_BAND = 1e-3
SPARSITY_ABS = 5e-3


def say(*a):
    print(*a, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def lnlam(lam):
    return -math.inf if lam == 0 else math.log(lam)


def check_decisions(gpu_skip, gpu_gap, ref_skip, ref_gap, lam, mask=None):
    """Compare maps (numpy), optionally only where ``mask`` is True. Returns #band."""
    gs, gg = np.asarray(gpu_skip), np.asarray(gpu_gap, dtype=np.float64)
    rs, rg = np.asarray(ref_skip), np.asarray(ref_gap)
    if mask is not None:
        gs, gg, rs, rg = gs[mask], gg[mask], rs[mask], rg[mask]
    # visitation is exact integer work
    assert np.array_equal(gs == 255, rs == 255), "visited pairs differ"
    vis = rs != 255
    band = np.zeros(rg.shape, bool)  # the exemption band, on visited pairs only (their gaps are never -inf)
    with np.errstate(invalid="ignore"):  # -inf gaps of visited pairs (non-finite inputs) at lambda = 0
        band[vis] = np.abs(rg[vis] - lnlam(lam)) < GAP_BAND
    bad = vis & ~band & (gs != rs)
    assert not bad.any(), f"{int(bad.sum())} decisions differ outside the band"
    # gaps: same infinities, finite values close
    assert np.array_equal(np.isposinf(gg[vis]), np.isposinf(rg[vis]))
    fin = vis & np.isfinite(rg)
    if fin.any():
        err = np.abs(gg[fin] - rg[fin])
        tol = 1e-3 + 2e-5 * np.abs(rg[fin])
        assert np.all(err <= tol), f"gap error {err.max():.3g}"
    assert np.all(np.isneginf(gg[~vis]))
    return int((vis & band).sum())


def check_output(o_gpu, o_ref, what=""):
    d = np.abs(np.asarray(o_gpu, dtype=np.float64) - o_ref)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    say(f"  {what} O max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, (mx, mean)
    return mx, mean


def gpu_prefill(q, k, v, *, causal, lam, tile_q, maps=True, out_dtype=torch.float32, window=0):
    B, Hq, L, _ = q.shape
    nqt, nkb = -(-L // tile_q), -(-L // 64)
    skip = torch.full((B, Hq, nqt, nkb), 7, dtype=torch.uint8, device=q.device) if maps else None
    gap = torch.full((B, Hq, nqt, nkb), float("nan"), dtype=torch.float32, device=q.device) if maps else None
    cnt = torch.zeros(2, dtype=torch.int64, device=q.device)
    o = bl.blasst_prefill(q, k, v, causal=causal, lam=lam, tile_q=tile_q, skip_map=skip, gap_map=gap,
                          counters=cnt, out_dtype=out_dtype, window=window)
    torch.cuda.synchronize()
    return o, skip, gap, cnt.cpu().numpy()


def gpu_decode(q, kc, vc, lens, *, lam, num_splits=0, dv=None, maps=True, out_dtype=torch.float32, window=0,
               sink_seed=False):
    B = q.shape[0]
    Hkv, Lmax = kc.shape[1], kc.shape[2]
    nkb = -(-Lmax // 64)
    skip = torch.full((B, Hkv, nkb), 7, dtype=torch.uint8, device=q.device) if maps else None
    gap = torch.full((B, Hkv, nkb), float("nan"), dtype=torch.float32, device=q.device) if maps else None
    cnt = torch.zeros(2, dtype=torch.int64, device=q.device)
    o = bl.blasst_decode(q, kc, vc, lens, lam=lam, num_splits=num_splits, dv=dv, skip_map=skip, gap_map=gap,
                         counters=cnt, out_dtype=out_dtype, window=window, sink_seed=sink_seed)
    torch.cuda.synchronize()
    return o, skip, gap, cnt.cpu().numpy()


def gpu_decode_paged(q, k_pages, v_pages, table, lens, Lmax, *, lam, num_splits=0, dv=None,
                     out_dtype=torch.float32, window=0, sink_seed=False):
    """blasst_decode_paged with fresh skip/gap maps and counters (as gpu_decode)."""
    B, Hkv = q.shape[0], k_pages.shape[1]
    nkb = -(-Lmax // 64)
    skip = torch.full((B, Hkv, nkb), 7, dtype=torch.uint8, device=q.device)
    gap = torch.full((B, Hkv, nkb), float("nan"), dtype=torch.float32, device=q.device)
    cnt = torch.zeros(2, dtype=torch.int64, device=q.device)
    o = bl.blasst_decode_paged(q, k_pages, v_pages, table, lens, Lmax, lam=lam, num_splits=num_splits, dv=dv,
                               skip_map=skip, gap_map=gap, counters=cnt, out_dtype=out_dtype, window=window,
                               sink_seed=sink_seed)
    torch.cuda.synchronize()
    return o, skip, gap, cnt.cpu().numpy()


def lambda_for(gap_map_gpu, target):
    """Calibrate lambda on a GPU gap map with the library's host search."""
    g = gap_map_gpu.cpu().numpy().ravel()
    return bl.blasst_calibrate_search(g, target)

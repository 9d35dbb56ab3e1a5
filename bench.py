"""Benchmark of the BLASST block-skipping attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Step = one blasst_prefill call on the GQA causal prefill workload
(B=1, Hq=32, Hkv=8, L=8192, d=128, bf16, query tile 128, key block 64) at the
lambda that the library's own calibration search gives for 70% block
sparsity on that input.  ``value`` is the dense-equivalent throughput
4*B*Hq*L^2*d/2 / time, in TFLOP/s.  The same run also measures
  * the same prefill at the 50% lambda and with lambda = 0 (the dense kernel),
    for speedups over the library's own dense path, and the gap pass that
    calibration runs (scores, block maxima and decisions only);
  * the GQA decode workload (148 sequences, Hq=32, Hkv=8, 32768 cached tokens,
    d=128, bf16 cache, block 64) at the 70% and 50% lambdas and lambda = 0:
    microseconds per decode step and HBM GB/s on the bytes actually loaded;
    then the same step over a paged cache (64-row pages of a shuffled pool;
    likewise for the latent decode below), with a 4096-key sliding window,
    and with sink-seeded splits (likewise for the latent decode);
  * the latent (MLA) decode workload (16 sequences, 128 query heads sharing one
    576-wide latent KV head, V = its first 512 columns, 65536 cached tokens)
    at the 70% lambda and lambda = 0: microseconds per step, GB/s on the
    loaded bytes and MFMA utilisation (the workload sits near the ridge);
  * one GPU's share of each decode step sharded over 8 GPUs, at its real
    shape: a 4096-token context slice of the GQA step, 16 of the latent
    step's 128 heads;
  * the long causal prefill (B=2, Hq=32, Hkv=8, L=32768, d=128) over the
    target sparsities 30/50/70/80% and dense (with its own MFMA roofline at
    70%), and with a 4096-key sliding window at 70% and dense;
  * the calibration law lambda = a/L: a fitted on calibration inputs at
    L = 4K..128K (a table that records its tiling), then the sparsity
    lambda = a/L achieves on fresh inputs;
  * the fp64 CPU oracle on a bounded sample of the prefill workload.
Every timed call passes a counters buffer (each call returns its skip counts).
Inputs are seeded synthetic segment-center tensors generated on the device.
Prints ONE JSON line.  ``--only NAME`` runs one measurement (for profilers).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import long_context_fa_amd as bl  # noqa: E402
from long_context_fa_amd import inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


MIN_WARM_MS = 100.0  # --min-warm-ms


def time_calls(fn, steps, warmup, min_warm_ms=None):
    """ms per call: at least ``warmup`` untimed calls and at least ``min_warm_ms`` of
    untimed work (the clocks settle), then ``steps`` calls enqueued back to back between
    two events on the launch stream, bracketed by device synchronisation."""
    min_warm_ms = MIN_WARM_MS if min_warm_ms is None else min_warm_ms
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < min_warm_ms:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return ms, ms, None


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CSRC = os.path.join(ROOT, "long_context_fa_amd", "csrc")


def measured_traffic(workload):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE passes, or None when
    the record is missing or the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for line in lines:
        if not line.startswith("traffic " + workload + " "):
            continue
        f = dict(kv.split("=", 1) for kv in line.split()[2:])
        h = hashlib.sha256()
        for src in f["sources"].split(","):
            h.update(open(os.path.join(CSRC, src), "rb").read())
        if h.hexdigest()[:16] != f["sha"]:
            return None
        return float(f["bytes_per_launch"])
    return None


def prefill_workload(seed=1001):
    B, Hq, Hkv, L, d = 1, 32, 8, 8192, 128
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, n_random=6, local_window=1, device="cuda", seed=seed)
    return (B, Hq, Hkv, L, d), (q, k, v)


def decode_workload(seed=1002):
    B, Hq, Hkv, L, d = 148, 32, 8, 32768, 128
    q, kc, vc, lens = inputs.decode_inputs(B, Hq, Hkv, L, d, n_random=8, device="cuda", seed=seed)
    return (B, Hq, Hkv, L, d), (q, kc, vc, lens)


def mla_workload(seed=2005):
    B, Hq, L, dqk, dv = 16, 128, 65536, 576, 512
    q, kc, _, lens = inputs.decode_inputs(B, Hq, 1, L, dqk, dv, n_random=16, mla=True, device="cuda", seed=seed)
    return (B, Hq, L, dqk, dv), (q, kc, lens)


def long_prefill_workload(seed=1004):
    B, Hq, Hkv, L, d = 2, 32, 8, 32768, 128
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, n_random=12, local_window=4, device="cuda", seed=seed)
    return (B, Hq, Hkv, L, d), (q, k, v)


def calibrate_prefill(q, k, v, targets, window=0, causal=True, tile_q=128):
    """lambda for each target sparsity: the gap pass (no O), then the exact quantile."""
    gap = bl.blasst_prefill_gaps(q, k, v, causal=causal, lam=0.0, tile_q=tile_q, window=window)
    g = gap.cpu().numpy().ravel()
    return {t: bl.blasst_calibrate_search(g, t) for t in targets}


def calibrate_decode(q, kc, vc, lens, S, targets, dv=None, window=0, sink_seed=False):
    """lambda for each target sparsity: the decode gap pass (no O), then the exact quantile."""
    gap = bl.blasst_decode_gaps(q, kc, vc, lens, lam=0.0, num_splits=S, dv=dv, window=window, sink_seed=sink_seed)
    g = gap.cpu().numpy().ravel()
    return {t: bl.blasst_calibrate_search(g, t) for t in targets}


def seed_leg(q, kc, vc, lens, S, lam70, steps, warmup, dv=None):
    """Sink-seeded splits against unseeded ones on one decode workload: time
    and sparsity at the unseeded 70% lambda, time at the seeded 70% lambda,
    and at equal (70%) sparsity the mean |O - O_dense| of both (fp32 O)."""
    ws = max(bl.blasst_decode_plan(q, kc, vc, lens, lam=1e-3, num_splits=S, dv=dv)[1], 1)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    lam_s = calibrate_decode(q, kc, vc, lens, S, [0.7], dv=dv, sink_seed=True)[0.7][0]

    def call(lam, seed, cnt=None, out_dtype=torch.bfloat16):
        return bl.blasst_decode(q, kc, vc, lens, lam=lam, num_splits=S, dv=dv, workspace=work, counters=cnt,
                                sink_seed=seed, out_dtype=out_dtype)

    res = {"num_splits": S, "lambda70_unseeded": lam70, "lambda70_seeded": lam_s}
    for name, lam in (("at_unseeded_lambda70", lam70), ("s70", lam_s)):
        mean_ms, _, _ = time_calls(lambda lam=lam: call(lam, True), steps, warmup)
        vis, skp = counts(lambda c, lam=lam: call(lam, True, c))
        res[name] = {"us": mean_ms * 1e3, "sparsity": skp / vis}
        log(f"  seeded splits, {name}: {mean_ms * 1e3:.1f} us, sparsity {skp / vis:.4f}")
    o_dense = call(0.0, False, out_dtype=torch.float32)
    e_u = (call(lam70, False, out_dtype=torch.float32) - o_dense).abs().mean().item()
    e_s = (call(lam_s, True, out_dtype=torch.float32) - o_dense).abs().mean().item()
    torch.cuda.synchronize()
    res["mean_abs_err_vs_dense70"] = {"unseeded": e_u, "seeded": e_s}
    log(f"  mean |O - O_dense| at 70%: unseeded {e_u:.3e}, seeded {e_s:.3e}")
    return res


def counts(fn_with_counters):
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    fn_with_counters(cnt)
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    return int(c[0]), int(c[1])


def cpu_baseline_prefill(q, k, v, lam, budget_s=20.0):
    """The fp64 oracle on a bounded sample of query tiles of the prefill workload."""
    import oracle

    B, Hq, L, d = q.shape
    tile = 128
    nqt = L // tile
    threads = min(16, len(os.sched_getaffinity(0)))
    f = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    qh, kh, vh = f(q), f(k), f(v)
    rng = np.random.default_rng(7)
    all_units = [(b, h, t) for b in range(B) for h in range(Hq) for t in range(nqt)]
    order = rng.permutation(len(all_units))
    done_flops, done_s, n_units = 0.0, 0.0, 0
    batch = threads
    while done_s < budget_s * 0.5 and n_units < len(all_units):
        mask = np.zeros((B, Hq, nqt), np.uint8)
        picks = [all_units[i] for i in order[n_units:n_units + batch]]
        batch = len(picks)
        flops = 0.0
        for (b, h, t) in picks:
            mask[b, h, t] = 1
            r0 = t * tile
            flops += 4.0 * d * sum(r + 1 for r in range(r0, r0 + tile))  # dense-equivalent
        t0 = time.perf_counter()
        oracle.prefill(qh, kh, vh, causal=True, lam=lam, tile_q=tile, block_k=64, unit_mask=mask,
                       nthreads=threads, want_maps=False)
        dt = time.perf_counter() - t0
        done_flops += flops
        done_s += dt
        n_units += batch
        log(f"  cpu oracle: {n_units} units, {done_s:.1f} s")
        if done_s + 2 * dt > budget_s:
            break
        batch *= 2
    what = (f"all {n_units} query tiles (the whole workload)" if n_units == len(all_units)
            else f"{n_units} random query tiles of {len(all_units)}")
    return {"value": done_flops / done_s / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": threads,
            "kind": "oracle",
            "sample": f"{what}, 128 rows each, of the 1x32/8x8192x128 causal prefill at the 70% lambda: "
                      f"{done_s:.1f} s of fp64 work on {threads} threads"}


def cpu_oracle_decode(q, kc, vc, lens, lam, S, *, dv=None, n_seq=2, seed=8):
    """The fp64 oracle on every (sequence, KV head) unit of n_seq random
    sequences of a decode step; the step time is extrapolated from the wall
    time per wave of `threads` units to all units."""
    import oracle

    B, Hq, _ = q.shape
    Hkv = kc.shape[1]
    threads = min(16, len(os.sched_getaffinity(0)))
    bs = sorted(np.random.default_rng(seed).choice(B, size=min(n_seq, B), replace=False).tolist())
    f = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    qh, kh = f(q[bs]), f(kc[bs])
    vh = kh[..., :dv] if dv is not None else f(vc[bs])
    t0 = time.perf_counter()
    oracle.decode(qh, kh, vh, lens[bs].cpu().numpy(), lam=lam, block_k=64, num_splits=S, nthreads=threads,
                  want_maps=False)
    wall = time.perf_counter() - t0
    units, total = len(bs) * Hkv, B * Hkv
    waves = lambda n: -(-n // threads)  # noqa: E731
    us = wall / waves(units) * waves(total) * 1e6
    log(f"  cpu oracle decode: {units} units in {wall:.2f} s -> {us:.4g} us/step extrapolated")
    return {"value": us, "unit": "us/step (extrapolated)", "cores": threads, "kind": "oracle",
            "sample": f"all {units} (sequence, KV head) units of {len(bs)} random sequences of {B} at the 70% "
                      f"lambda, {wall:.2f} s on {threads} threads; step time = wall time per wave of {threads} "
                      f"units x the {waves(total)} waves of the {total} units"}


def cpu_oracle_long_prefill(q, k, v, lam, budget_s=6.0, seed=9):
    """The fp64 oracle on random query tiles of two query heads (one KV head)
    of the long prefill; dense-equivalent throughput and the extrapolated
    time of the whole launch."""
    import oracle

    B, Hq, L, d = q.shape
    G = Hq // k.shape[1]
    threads = min(16, len(os.sched_getaffinity(0)))
    f = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    qh, kh, vh = f(q[:1, :2]), f(k[:1, :1]), f(v[:1, :1])
    assert G >= 2
    tile, nqt = 128, L // 128
    units = [(h, t) for h in range(2) for t in range(nqt)]
    order = np.random.default_rng(seed).permutation(len(units))
    done_flops, done_s, n, batch = 0.0, 0.0, 0, threads
    while n < len(units):
        mask = np.zeros((1, 2, nqt), np.uint8)
        picks = [units[i] for i in order[n:n + batch]]
        flops = 0.0
        for h, t in picks:
            mask[0, h, t] = 1
            r0 = t * tile
            flops += 4.0 * d * (tile * r0 + tile * (tile + 1) / 2)  # dense-equivalent
        t0 = time.perf_counter()
        oracle.prefill(qh, kh, vh, causal=True, lam=lam, tile_q=tile, block_k=64, unit_mask=mask,
                       nthreads=threads, want_maps=False)
        dt = time.perf_counter() - t0
        done_flops, done_s, n = done_flops + flops, done_s + dt, n + len(picks)
        if done_s + 2 * dt > budget_s:
            break
        batch *= 2
    tflops = done_flops / done_s / 1e12
    full_ms = 4.0 * B * Hq * L * L * d / 2 / (tflops * 1e12) * 1e3
    log(f"  cpu oracle long prefill: {n} tiles in {done_s:.1f} s -> {tflops:.4f} TFLOP/s, {full_ms:.4g} ms extrapolated")
    return {"value": tflops, "unit": "TFLOP/s (dense-equivalent)", "ms_extrapolated": full_ms, "cores": threads,
            "kind": "oracle",
            "sample": f"{n} random query tiles (128 rows) of 2 query heads sharing one KV head, of "
                      f"{B * Hq * nqt} tiles, at the 70% lambda: {done_s:.1f} s on {threads} threads"}


def measured_peaks(reps=20):
    """Attainable rates on this GPU, for reading the roofline fractions beside
    the spec peaks: a 2 GiB device-to-device copy (bytes read + written per
    second) and a 16384^3 bf16 GEMM through torch (the vendor GEMM library)."""
    src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    n = 16384
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(8):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps // 2):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 * (reps // 2) / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    log(f"measured peaks: device copy {copy_gbps:.0f} GB/s (read + write), bf16 GEMM 16384^3 {gemm_tflops:.0f} TFLOP/s")
    return {"device_copy_gbps": copy_gbps, "bf16_gemm_16384_tflops": gemm_tflops,
            "spec_hbm_gbps": PEAK_HBM_GBS, "spec_bf16_tflops": PEAK_BF16_TFLOPS,
            "note": "attainable rates measured in this run; the roofline fractions use the spec peaks"}


# A lambda so small that no visited block can meet the test (log2 of it is
# about -997, far below any score gap), but above 0, so the call runs the
# skip-enabled kernels: their time against the lambda = 0 kernels is the cost
# of the skip logic itself.
LAM_TINY = 1e-300


def bench_prefill(steps, warmup, names=("s70", "s50", "dense", "skip0", "gaps")):
    (B, Hq, Hkv, L, d), (q, k, v) = prefill_workload()
    cal = calibrate_prefill(q, k, v, [0.5, 0.7])
    lam70, reach70 = cal[0.7]
    lam50, reach50 = cal[0.5]
    log(f"prefill lambda70={lam70:.4g} (gap-map sparsity {reach70:.4f}) lambda50={lam50:.4g} ({reach50:.4f})")
    out = torch.empty(B, Hq, L, d, dtype=torch.bfloat16, device="cuda")
    gap = torch.empty(B, Hq, L // 128, L // 64, dtype=torch.float32, device="cuda")
    run_cnt = torch.zeros(2, dtype=torch.int64, device="cuda")  # every timed call returns its skip counts

    def pf(lam, cnt=None):
        return lambda: bl.blasst_prefill(q, k, v, causal=True, lam=lam, tile_q=128, out=out, counters=cnt)

    def gp(lam, cnt=None):  # the gap pass (calibration): maps and counters only, no O
        return lambda: bl.blasst_prefill_gaps(q, k, v, causal=True, lam=lam, tile_q=128, gap_map=gap, counters=cnt)

    dense_flops = 4.0 * B * Hq * L * L * d / 2
    lams = {"s70": lam70, "s50": lam50, "dense": 0.0, "skip0": LAM_TINY, "gaps": lam70}
    res = {}
    for name in names:
        lam = lams[name]
        call = gp if name == "gaps" else pf
        mean_ms, _, _ = time_calls(call(lam, run_cnt), steps, warmup)
        vis, skp = counts(lambda c: call(lam, c)())
        res[name] = {"lambda": lam, "ms": mean_ms, "visited": vis, "skipped": skp,
                     "sparsity": skp / vis if vis else 0.0,
                     "dense_equiv_tflops": dense_flops / (mean_ms * 1e-3) / 1e12}
        log(f"prefill {name}: {mean_ms:.4f} ms, sparsity {res[name]['sparsity']:.4f}, "
            f"{res[name]['dense_equiv_tflops']:.1f} dense-equiv TFLOP/s")
    return (q, k, v, lam70), res, dense_flops


def bench_decode(steps, warmup, names=("s70", "s50", "dense", "skip0", "gaps"), paged_names=(), window=0,
                 seed=False, oracle_cpu=False):
    (DB, DHq, DHkv, DL, Dd), (dq, kc, vc, lens) = decode_workload()
    S, ws = bl.blasst_decode_plan(dq, kc, vc, lens, lam=1e-3)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    dout = torch.empty(DB, DHq, Dd, dtype=torch.bfloat16, device="cuda")
    dgap = torch.empty(DB, DHkv, DL // 64, dtype=torch.float32, device="cuda")
    run_cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    dcal = calibrate_decode(dq, kc, vc, lens, S, [0.5, 0.7])

    def dc(lam, cnt=None, gaps=False):
        if gaps:
            return lambda: bl.blasst_decode_gaps(dq, kc, vc, lens, lam=lam, num_splits=S, gap_map=dgap, counters=cnt)
        return lambda: bl.blasst_decode(dq, kc, vc, lens, lam=lam, num_splits=S, out=dout,
                                        workspace=work, counters=cnt)

    lams = {"s70": dcal[0.7][0], "s50": dcal[0.5][0], "dense": 0.0, "skip0": LAM_TINY, "gaps": dcal[0.7][0]}
    dres = {}
    for name in names:
        lam = lams[name]
        mean_ms, _, _ = time_calls(dc(lam, run_cnt, name == "gaps"), steps, warmup)
        vis, skp = counts(lambda c: dc(lam, c, name == "gaps")())
        blk = 64 * Dd * 2
        if name == "gaps":  # K of every visited block; no V, no partials, no O
            loaded = vis * blk + dq.numel() * 2
        else:
            loaded = vis * blk + (vis - skp) * blk + dq.numel() * 2 + dout.numel() * 2
            if S > 1:
                loaded += 2 * DB * DHq * S * (Dd + 2) * 4
        dres[name] = {"lambda": lam, "us": mean_ms * 1e3, "sparsity": skp / vis, "bytes": loaded,
                      "gbps": loaded / (mean_ms * 1e-3) / 1e9}
        log(f"decode {name}: {mean_ms * 1e3:.1f} us, sparsity {skp / vis:.4f}, "
            f"{dres[name]['gbps']:.0f} GB/s on loaded bytes")
    if paged_names:
        # The same step over a paged cache: 64-row pages in a shuffled pool
        # (the layout of serving engines), same lambda and split count.
        (kp, vp), table = inputs.paged_pool([kc, vc], lens, 64, seed=9)
        for name in paged_names:
            lam = lams[name.replace("paged_", "")]

            def pg(cnt=None, lam=lam):
                return bl.blasst_decode_paged(dq, kp, vp, table, lens, DL, lam=lam, num_splits=S, out=dout,
                                              workspace=work, counters=cnt)

            mean_ms, _, _ = time_calls(pg, steps, warmup)
            vis, skp = counts(lambda c: pg(c))
            dres[name] = {"lambda": lam, "us": mean_ms * 1e3, "sparsity": skp / vis}
            log(f"decode {name} (64-row pages): {mean_ms * 1e3:.1f} us, sparsity {skp / vis:.4f}")
        del kp, vp, table
    if window:
        # The same step with a sliding window of `window` keys (its own lambda).
        Sw, wsw = bl.blasst_decode_plan(dq, kc, vc, lens, lam=1e-3, window=window)
        wwork = torch.empty(max(wsw, 1), dtype=torch.uint8, device="cuda")
        lamw = calibrate_decode(dq, kc, vc, lens, Sw, [0.7], window=window)[0.7][0]
        for name, lam in (("window_s70", lamw), ("window_dense", 0.0)):

            def wd(cnt=None, lam=lam):
                return bl.blasst_decode(dq, kc, vc, lens, lam=lam, num_splits=Sw, out=dout, workspace=wwork,
                                        counters=cnt, window=window)

            mean_ms, _, _ = time_calls(wd, steps, warmup)
            vis, skp = counts(lambda c: wd(c))
            blk = 64 * Dd * 2
            loaded = vis * blk + (vis - skp) * blk + dq.numel() * 2 + dout.numel() * 2
            if Sw > 1:
                loaded += 2 * DB * DHq * Sw * (Dd + 2) * 4
            dres[name] = {"lambda": lam, "us": mean_ms * 1e3, "sparsity": skp / vis, "splits": Sw,
                          "gbps": loaded / (mean_ms * 1e-3) / 1e9}
            log(f"decode {name} (window {window}): {mean_ms * 1e3:.1f} us, sparsity {skp / vis:.4f}, "
                f"{dres[name]['gbps']:.0f} GB/s, splits {Sw}")
    if seed:
        dres["sink_seed"] = seed_leg(dq, kc, vc, lens, S, lams["s70"], steps, warmup)
    if oracle_cpu:
        dres["cpu_oracle"] = cpu_oracle_decode(dq, kc, vc, lens, lams["s70"], S)
    return S, dres


def bench_paged_layouts(steps, warmup, rounds=4):
    """Where the paged GQA decode's extra time goes, at the 70% lambda: the
    contiguous cache against three page pools holding the same rows, timed in
    alternating rounds (median per layout):
      shuffled  64-row pages [pages, Hkv, 64, d] in seeded random order (the bench's paged leg);
      in_order  the same pool layout with the pages in sequence order;
      whole     the contiguous cache itself passed as one page per sequence (page = Lmax rows):
                the addresses of the contiguous call, through the paged kernel's code.
    whole - contiguous is the cost of the paged code path; in_order - whole that of the pool's
    address pattern (16 KB per head and block, 128 KB apart); shuffled - in_order that of the
    random page order."""
    (B, Hq, Hkv, L, d), (q, kc, vc, lens) = decode_workload()
    S, ws = bl.blasst_decode_plan(q, kc, vc, lens, lam=1e-3)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    lam = calibrate_decode(q, kc, vc, lens, S, [0.7])[0.7][0]
    (kp, vp), table = inputs.paged_pool([kc, vc], lens, 64, seed=9)
    npb = L // 64

    def in_order(c):  # page b * npb + i holds rows 64 i .. 64 i + 63 of sequence b
        return c.view(B, Hkv, npb, 64, d).permute(0, 2, 1, 3, 4).reshape(B * npb, Hkv, 64, d)

    ko, vo = in_order(kc), in_order(vc)
    t_in = (torch.arange(B, device="cuda", dtype=torch.int32)[:, None] * npb
            + torch.arange(npb, device="cuda", dtype=torch.int32)[None, :]).contiguous()
    t_whole = torch.arange(B, device="cuda", dtype=torch.int32)[:, None].contiguous()
    calls = {
        "contiguous": lambda: bl.blasst_decode(q, kc, vc, lens, lam=lam, num_splits=S, out=out, workspace=work),
        "whole": lambda: bl.blasst_decode_paged(q, kc, vc, t_whole, lens, L, lam=lam, num_splits=S, out=out,
                                                workspace=work),
        "in_order": lambda: bl.blasst_decode_paged(q, ko, vo, t_in, lens, L, lam=lam, num_splits=S, out=out,
                                                   workspace=work),
        "shuffled": lambda: bl.blasst_decode_paged(q, kp, vp, table, lens, L, lam=lam, num_splits=S, out=out,
                                                   workspace=work),
    }
    ref = None
    for name, fn in calls.items():  # every layout gives the contiguous call's O, bit for bit
        fn()
        torch.cuda.synchronize()
        if ref is None:
            ref = out.clone()
        elif not torch.equal(out, ref):
            raise RuntimeError(f"paged layout {name} differs from the contiguous call")
    times = {name: [] for name in calls}
    for _ in range(rounds):
        for name, fn in calls.items():
            times[name].append(time_calls(fn, steps, warmup, min_warm_ms=20.0)[0] * 1e3)
    med = {name: float(np.median(v)) for name, v in times.items()}
    c = med["contiguous"]
    res = {"num_splits": S, "lambda70": lam, "us": med, "rounds": rounds,
           "overhead_vs_contiguous": {k: v / c - 1.0 for k, v in med.items() if k != "contiguous"},
           "split": {"paged_code": med["whole"] / c - 1.0, "pool_address_pattern": (med["in_order"] - med["whole"]) / c,
                     "random_page_order": (med["shuffled"] - med["in_order"]) / c}}
    for name in calls:
        log(f"decode 70% {name}: {med[name]:.1f} us ({med[name] / c - 1.0:+.2%})")
    return res


def bench_mla(steps, warmup, names=("s70", "s50", "dense", "skip0", "gaps"), paged_names=(), seed=False,
              oracle_cpu=False):
    (B, Hq, L, dqk, dv), (q, kc, lens) = mla_workload()
    S, ws = bl.blasst_decode_plan(q, kc, kc, lens, lam=1e-3, dv=dv)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, dv, dtype=torch.bfloat16, device="cuda")
    mgap = torch.empty(B, 1, L // 64, dtype=torch.float32, device="cuda")
    run_cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    cal = calibrate_decode(q, kc, kc, lens, S, [0.5, 0.7], dv=dv)

    def dc(lam, cnt=None, gaps=False):
        if gaps:
            return lambda: bl.blasst_decode_gaps(q, kc, kc, lens, lam=lam, num_splits=S, dv=dv, gap_map=mgap,
                                                 counters=cnt)
        return lambda: bl.blasst_decode(q, kc, kc, lens, lam=lam, num_splits=S, out=out, dv=dv,
                                        workspace=work, counters=cnt)

    lams = {"s70": cal[0.7][0], "s50": cal[0.5][0], "dense": 0.0, "skip0": LAM_TINY, "gaps": cal[0.7][0]}
    res = {}
    for name in names:
        lam = lams[name]
        gaps = name == "gaps"
        mean_ms, _, _ = time_calls(dc(lam, run_cnt, gaps), steps, warmup)
        vis, skp = counts(lambda c: dc(lam, c, gaps)())
        # V aliases the K tile: a visited block loads its 64 x 576 latent rows once
        loaded = vis * 64 * dqk * 2 + q.numel() * 2 + (0 if gaps else out.numel() * 2)
        if S > 1 and not gaps:
            loaded += 2 * B * Hq * S * (dv + 2) * 4
        flops = vis * 2.0 * Hq * 64 * dqk + (0 if gaps else (vis - skp) * 2.0 * Hq * 64 * dv)
        sec = mean_ms * 1e-3
        res[name] = {"lambda": lam, "us": mean_ms * 1e3, "sparsity": skp / vis, "bytes": loaded,
                     "gbps": loaded / sec / 1e9, "tflops": flops / sec / 1e12}
        log(f"mla decode {name}: {mean_ms * 1e3:.1f} us, sparsity {skp / vis:.4f}, "
            f"{res[name]['gbps']:.0f} GB/s, {res[name]['tflops']:.0f} TFLOP/s")
    if paged_names:
        # The same step over a paged latent cache: 64-row pages in a shuffled pool.
        (kp,), table = inputs.paged_pool([kc], lens, 64, seed=9)
        for name in paged_names:
            lam = lams[name.replace("paged_", "")]

            def pg(cnt=None, lam=lam):
                return bl.blasst_decode_paged(q, kp, kp, table, lens, L, lam=lam, num_splits=S, out=out, dv=dv,
                                              workspace=work, counters=cnt)

            mean_ms, _, _ = time_calls(pg, steps, warmup)
            vis, skp = counts(lambda c: pg(c))
            res[name] = {"lambda": lam, "us": mean_ms * 1e3, "sparsity": skp / vis}
            log(f"mla decode {name} (64-row pages): {mean_ms * 1e3:.1f} us, sparsity {skp / vis:.4f}")
        del kp, table
    if seed:
        res["sink_seed"] = seed_leg(q, kc, kc, lens, S, lams["s70"], steps, warmup, dv=dv)
    if oracle_cpu:
        res["cpu_oracle"] = cpu_oracle_decode(q, kc, kc, lens, lams["s70"], S, dv=dv, n_seq=1)
    return S, res


def bench_long_prefill(steps, warmup, targets=(0.3, 0.5, 0.7, 0.8), oracle_cpu=False, window_leg=True):
    (B, Hq, Hkv, L, d), (q, k, v) = long_prefill_workload()
    cal = calibrate_prefill(q, k, v, list(targets))
    out = torch.empty(B, Hq, L, d, dtype=torch.bfloat16, device="cuda")
    dense_flops = 4.0 * B * Hq * L * L * d / 2

    def pf(lam, cnt=None):
        return lambda: bl.blasst_prefill(q, k, v, causal=True, lam=lam, tile_q=128, out=out, counters=cnt)

    run_cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    rows = []
    for t in list(targets) + [None]:
        lam = 0.0 if t is None else cal[t][0]
        mean_ms, _, _ = time_calls(pf(lam, run_cnt), steps, warmup)
        vis, skp = counts(lambda c: pf(lam, c)())
        mfma = (2 * vis - skp) * 2.0 * 128 * 64 * d  # QK of every visited pair, PV of the executed ones
        rows.append({"target": t, "lambda": lam, "ms": mean_ms, "sparsity": skp / vis,
                     "dense_equiv_tflops": dense_flops / (mean_ms * 1e-3) / 1e12,
                     "mfma_flops": mfma, "mfma_util_executed": mfma / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
        log(f"long prefill target {t}: {mean_ms:.3f} ms, sparsity {skp / vis:.4f}")
    dense_ms = rows[-1]["ms"]
    for r in rows:
        r["speedup_vs_dense"] = dense_ms / r["ms"]
    cpu = cpu_oracle_long_prefill(q, k, v, cal[0.7][0]) if oracle_cpu and 0.7 in cal else None
    win = window_prefill(q, k, v, out, 4096, steps, warmup) if window_leg else None
    return rows, win, cpu


def bench_prefill_lengths(steps, warmup, lengths=(2048, 4096, 8192, 16384, 32768), tokens=65536):
    """The 70% speedup over dense as a function of sequence length: causal GQA
    prefill (32 query / 8 KV heads, d = 128, the 8K workload's input recipe)
    at a fixed 65536 tokens per launch (B = tokens / L), lambda calibrated to
    70% block sparsity at each length."""
    rows = []
    for L in lengths:
        B, Hq, Hkv, d = tokens // L, 32, 8, 128
        q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, n_random=6, local_window=1, device="cuda",
                                        seed=1100 + L // 1024)
        lam70, _ = calibrate_prefill(q, k, v, [0.7])[0.7]
        out = torch.empty(B, Hq, L, d, dtype=torch.bfloat16, device="cuda")
        dense_flops = 4.0 * B * Hq * L * L * d / 2
        row = {"L": L, "B": B, "lambda70": lam70}
        for name, lam in (("s70", lam70), ("dense", 0.0)):
            def pf(cnt=None, lam=lam):
                return bl.blasst_prefill(q, k, v, causal=True, lam=lam, tile_q=128, out=out, counters=cnt)
            mean_ms, _, _ = time_calls(pf, steps, warmup)
            vis, skp = counts(lambda c: pf(c))
            mfma = (vis + (vis - skp)) * 2.0 * 128 * 64 * d
            row[name] = {"ms": mean_ms, "sparsity": skp / vis,
                         "dense_equiv_tflops": dense_flops / (mean_ms * 1e-3) / 1e12,
                         "mfma_util_executed": mfma / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        row["speedup70_vs_dense"] = row["dense"]["ms"] / row["s70"]["ms"]
        log(f"prefill L={L} B={B}: dense {row['dense']['ms']:.3f} ms, 70% {row['s70']['ms']:.3f} ms "
            f"(sparsity {row['s70']['sparsity']:.4f}), speedup {row['speedup70_vs_dense']:.3f}")
        rows.append(row)
        del q, k, v, out
        torch.cuda.empty_cache()
    return rows


def bench_prefill_variants(steps, warmup):
    """The prefill kernels off the headline shape, on the 8K workload's input
    recipe (B = 1, 32 query / 8 KV heads, L = 8192): non-causal, d = 64, and a
    64-row query tile, each at its own 70% lambda and at lambda = 0.  Executed
    MFMA work counts QK of every visited (tile, block) pair and P.V of every
    executed one."""
    cases = [("causal_d128_tile128", True, 128, 128), ("noncausal_d128_tile128", False, 128, 128),
             ("causal_d64_tile128", True, 64, 128), ("causal_d128_tile64", True, 128, 64),
             ("causal_d64_tile64", True, 64, 64)]
    B, Hq, Hkv, L = 1, 32, 8, 8192
    rows = []
    for name, causal, d, tile in cases:
        q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, n_random=6, local_window=1, device="cuda", seed=1001)
        lam70, _ = calibrate_prefill(q, k, v, [0.7], causal=causal, tile_q=tile)[0.7]
        out = torch.empty(B, Hq, L, d, dtype=torch.bfloat16, device="cuda")
        dense_flops = 4.0 * B * Hq * L * L * d / (2 if causal else 1)
        row = {"case": name, "causal": causal, "d": d, "tile_q": tile, "lambda70": lam70}
        for leg, lam in (("s70", lam70), ("dense", 0.0)):
            def pf(cnt=None, lam=lam):
                return bl.blasst_prefill(q, k, v, causal=causal, lam=lam, tile_q=tile, out=out, counters=cnt)
            mean_ms, _, _ = time_calls(pf, steps, warmup)
            vis, skp = counts(lambda c: pf(c))
            mfma = (vis + (vis - skp)) * 2.0 * tile * 64 * d
            row[leg] = {"ms": mean_ms, "sparsity": skp / vis,
                        "dense_equiv_tflops": dense_flops / (mean_ms * 1e-3) / 1e12,
                        "mfma_util_executed": mfma / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        row["speedup70_vs_dense"] = row["dense"]["ms"] / row["s70"]["ms"]
        log(f"prefill {name}: dense {row['dense']['ms']:.3f} ms ({row['dense']['mfma_util_executed']:.3f} MFMA), "
            f"70% {row['s70']['ms']:.3f} ms ({row['s70']['mfma_util_executed']:.3f}), "
            f"speedup {row['speedup70_vs_dense']:.3f}")
        rows.append(row)
        del q, k, v, out
        torch.cuda.empty_cache()
    return rows


def bench_decode_wide(steps, warmup):
    """GQA/MQA decode with 17..64 query heads per KV head (the kernel's 2- and
    4-group forms) on the decode workload's input recipe, at the planner's
    split count, at the 70% lambda and at lambda = 0.  Loaded bytes: K of
    every visited block and V of every executed one."""
    cases = [(64, 64, 1, 32768, 128), (64, 32, 1, 32768, 128), (32, 64, 2, 32768, 128),
             (16, 48, 1, 65536, 128), (64, 64, 1, 32768, 64)]
    rows = []
    for B, Hq, Hkv, L, d in cases:
        q, kc, vc, lens = inputs.decode_inputs(B, Hq, Hkv, L, d, n_random=8, device="cuda", seed=1002)
        S, ws = bl.blasst_decode_plan(q, kc, vc, lens, lam=1e-3)
        work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
        lam70 = calibrate_decode(q, kc, vc, lens, S, [0.7])[0.7][0]
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        row = {"B": B, "Hq": Hq, "Hkv": Hkv, "L": L, "d": d, "num_splits": S}
        for leg, lam in (("s70", lam70), ("dense", 0.0)):
            def dc(cnt=None, lam=lam):
                return bl.blasst_decode(q, kc, vc, lens, lam=lam, num_splits=S, out=out, workspace=work,
                                        counters=cnt)
            tc = torch.zeros(2, dtype=torch.int64, device="cuda")  # timed calls return their counts too
            mean_ms, _, _ = time_calls(lambda: dc(tc), steps, warmup)
            vis, skp = counts(lambda c: dc(c))
            loaded = (vis + (vis - skp)) * 64 * d * 2
            row[leg] = {"us": mean_ms * 1e3, "sparsity": skp / vis, "hbm_gbps": loaded / (mean_ms * 1e-3) / 1e9}
        log(f"decode wide {B}x{Hq}/{Hkv}x{L}x{d} S={S}: 70% {row['s70']['us']:.1f} us "
            f"({row['s70']['hbm_gbps']:.0f} GB/s), dense {row['dense']['us']:.1f} us "
            f"({row['dense']['hbm_gbps']:.0f} GB/s)")
        rows.append(row)
        del q, kc, vc, work, out
        torch.cuda.empty_cache()
    return rows


def bench_shards(steps, warmup, n_gpus=8):
    """One GPU's share of a decode step sharded over n_gpus, at its real shape
    (nothing runs on a second GPU):
      * context-parallel GQA decode: the 148 x 32/8 x 32K x 128 step's cache cut
        into n_gpus contiguous slices of 32768/n_gpus tokens; one GPU holds the
        third slice (a strided view of the full cache, no copy) and runs the
        split kernel and combine on it, its slice being one split of the whole
        step (lambda calibrated to 70% on that slice).  The partials that GPU
        would all-gather are B * Hq * (d + 2) fp32 values;
      * head-parallel latent decode: the 16 x 128/1 x 64K step's 128 query
        heads split n_gpus ways, each GPU taking 128/n_gpus heads with the
        whole latent cache.
    Microseconds per step at the 70% lambda and at lambda = 0, and GB/s on
    the loaded bytes (K of every visited block, V of every executed one)."""
    res = {}
    (B, Hq, Hkv, L, d), (q, kc, vc, lens) = decode_workload()
    Ls = L // n_gpus
    ks, vs = kc[:, :, 2 * Ls:3 * Ls], vc[:, :, 2 * Ls:3 * Ls]
    ls = torch.full_like(lens, Ls)
    S, ws = bl.blasst_decode_plan(q, ks, vs, ls, lam=1e-3)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    lam70 = calibrate_decode(q, ks, vs, ls, S, [0.7])[0.7][0]
    row = {"shape": f"{B}x{Hq}/{Hkv}x{Ls}x{d}: tokens {2 * Ls}..{3 * Ls - 1} of the {L}-token cache",
           "num_splits": S, "allgather_bytes_per_gpu": B * Hq * (d + 2) * 4}
    for leg, lam in (("s70", lam70), ("dense", 0.0)):
        def dc(cnt=None, lam=lam):
            return bl.blasst_decode(q, ks, vs, ls, lam=lam, num_splits=S, out=out, workspace=work, counters=cnt)
        tc = torch.zeros(2, dtype=torch.int64, device="cuda")
        mean_ms, _, _ = time_calls(lambda: dc(tc), steps, warmup)
        vis, skp = counts(lambda c: dc(c))
        loaded = (vis + (vis - skp)) * 64 * d * 2
        row[leg] = {"lambda": lam, "us": mean_ms * 1e3, "sparsity": skp / vis,
                    "hbm_gbps": loaded / (mean_ms * 1e-3) / 1e9}
    log(f"decode context shard 1/{n_gpus} ({row['shape']}, S={S}): 70% {row['s70']['us']:.1f} us "
        f"({row['s70']['hbm_gbps']:.0f} GB/s), dense {row['dense']['us']:.1f} us ({row['dense']['hbm_gbps']:.0f} GB/s)")
    res["gqa_context_shard"] = row
    del q, kc, vc, ks, vs, work, out
    torch.cuda.empty_cache()

    (B, Hq, L, dqk, dv), (q, kc, lens) = mla_workload()
    Hs = Hq // n_gpus
    qs = q[:, :Hs]
    S, ws = bl.blasst_decode_plan(qs, kc, kc, lens, lam=1e-3, dv=dv)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hs, dv, dtype=torch.bfloat16, device="cuda")
    lam70 = calibrate_decode(qs, kc, kc, lens, S, [0.7], dv=dv)[0.7][0]
    row = {"shape": f"{B}x{Hs}/1x{L}, dqk={dqk} dv={dv}: heads 0..{Hs - 1} of {Hq}", "num_splits": S}
    for leg, lam in (("s70", lam70), ("dense", 0.0)):
        def mc(cnt=None, lam=lam):
            return bl.blasst_decode(qs, kc, kc, lens, lam=lam, num_splits=S, out=out, dv=dv, workspace=work,
                                    counters=cnt)
        tc = torch.zeros(2, dtype=torch.int64, device="cuda")
        mean_ms, _, _ = time_calls(lambda: mc(tc), steps, warmup)
        vis, skp = counts(lambda c: mc(c))
        loaded = vis * 64 * dqk * 2
        row[leg] = {"lambda": lam, "us": mean_ms * 1e3, "sparsity": skp / vis,
                    "hbm_gbps": loaded / (mean_ms * 1e-3) / 1e9}
    log(f"latent decode head shard 1/{n_gpus} ({row['shape']}, S={S}): 70% {row['s70']['us']:.1f} us "
        f"({row['s70']['hbm_gbps']:.0f} GB/s), dense {row['dense']['us']:.1f} us")
    res["latent_head_shard"] = row
    del q, kc, work, out
    torch.cuda.empty_cache()
    return res


def window_prefill(q, k, v, out, W, steps, warmup):
    """The same prefill with a sliding window of W keys, at the 70% lambda of
    the windowed gaps and at lambda = 0."""
    B, Hq, L, d = q.shape
    lam70, _ = calibrate_prefill(q, k, v, [0.7], window=W)[0.7]
    # dense-equivalent work of windowed attention: row i sees min(i+1, W) keys
    keys = W * (W + 1) // 2 + (L - W) * W if L > W else L * (L + 1) // 2
    dense_flops = 4.0 * B * Hq * d * keys

    def pf(lam, cnt=None):
        return lambda: bl.blasst_prefill(q, k, v, causal=True, lam=lam, tile_q=128, out=out, counters=cnt,
                                         window=W)

    res = {"window": W, "dense_equiv_flops": dense_flops}
    for name, lam in (("s70", lam70), ("dense", 0.0)):
        mean_ms, _, _ = time_calls(pf(lam), steps, warmup)
        vis, skp = counts(lambda c: pf(lam, c)())
        mfma = (vis + (vis - skp)) * 2.0 * 128 * 64 * d
        res[name] = {"lambda": lam, "ms": mean_ms, "sparsity": skp / vis,
                     "dense_equiv_tflops": dense_flops / (mean_ms * 1e-3) / 1e12,
                     "mfma_util_executed": mfma / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        log(f"windowed prefill W={W} {name}: {mean_ms:.3f} ms, sparsity {skp / vis:.4f}")
    res["speedup70_vs_dense"] = res["dense"]["ms"] / res["s70"]["ms"]
    return res


def bench_calibration(lengths=(4096, 8192, 16384, 32768, 65536, 131072), targets=(0.5, 0.7)):
    """The calibration law lambda = a(target) / L on the GQA prefill generator,
    over L = 4K .. 128K (one sequence of 32 query / 8 KV heads, d = 128).

    For each L, lambda_L is the exact quantile of the gap map (gap pass) of a
    calibration input (seed 2000 + L/1024); a is fitted as ln a = mean(ln(lambda_L * L))
    over all the lengths and stored as a table with its tiling (query tile 128,
    key block 64).
    Fresh evaluation inputs (seed 1000 + L/1024) are then run with
    lambda = a / L from the fitted table, and the achieved block sparsity is
    compared with the target; so is the sparsity that the per-length lambda_L
    itself reaches on the evaluation input (how well a calibration transfers
    between inputs of one length, apart from the 1/L law)."""
    B, Hq, Hkv, d = 1, 32, 8, 128
    lam_at = {t: [] for t in targets}
    for L in lengths:
        q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, n_random=6, local_window=1, device="cuda",
                                        seed=2000 + L // 1024)
        cal = calibrate_prefill(q, k, v, list(targets))
        for t in targets:
            lam_at[t].append(cal[t][0])
        del q, k, v
    a_fit = [bl.blasst_calibrate_fit(lam_at[t], lengths) for t in targets]
    table = bl.calib_table(list(targets), a_fit, tile_q=128, block_k=64, num_splits=0)
    rows = []
    for L in lengths:
        q, k, v = inputs.prefill_inputs(B, Hq, Hkv, L, d, n_random=6, local_window=1, device="cuda",
                                        seed=1000 + L // 1024)
        def sparsity(lam):  # the gap pass counts the skips at lam (decisions as the full pass)
            cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
            bl.blasst_prefill_gaps(q, k, v, causal=True, lam=lam, tile_q=128, counters=cnt)
            torch.cuda.synchronize()
            vis, skp = (int(x) for x in cnt.cpu())
            return skp / vis

        for t in targets:
            lam = bl.blasst_calibrate(table, t, L, tile_q=128, block_k=64, num_splits=0)
            lam_l = lam_at[t][list(lengths).index(L)]
            got, got_l = sparsity(lam), sparsity(lam_l)
            rows.append({"L": L, "target": t, "lambda_L_calibrated": lam_l, "lambda_L_times_L": lam_l * L,
                         "lambda_from_fit": lam, "achieved": got, "deviation": got - t,
                         "achieved_with_lambda_L": got_l})
            log(f"calibration L={L} target {t}: lambda(a/L)={lam:.4g} achieved {got:.4f}; "
                f"lambda_L={lam_l:.4g} (lambda_L*L={lam_l * L:.4g}) achieves {got_l:.4f}")
        del q, k, v
    torch.cuda.empty_cache()
    return {"workload": "GQA causal prefill B=1 Hq=32 Hkv=8 d=128, tile 128, block 64; calibration seeds "
                        "2000+L/1024, evaluation seeds 1000+L/1024",
            "a_fit": dict(zip([str(t) for t in targets], a_fit)),
            "table": table,
            "mean_abs_deviation": {str(t): float(np.mean([abs(r["deviation"]) for r in rows if r["target"] == t]))
                                   for t in targets},
            "rows": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode and long-prefill sections")
    ap.add_argument("--no-calibration", action="store_true", help="skip the calibration-law study")
    ap.add_argument("--only", choices=["prefill70", "prefill_dense", "prefill_gaps", "decode70", "decode_dense",
                                       "decode_gaps", "mla70", "mla_dense", "mla_gaps", "decode_paged70",
                                       "decode_paged_layouts", "prefill_variants", "decode_wide", "decode_shards",
                                       "mla_paged70", "long_prefill70", "long_prefill_dense", "prefill_lengths"],
                    help="run one measurement only and print its numbers (profiling runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--min-warm-ms", type=float, default=100.0,
                    help="least untimed work before each timed run (profiling runs pass 0 so that the trace "
                         "averages cover mostly timed calls)")
    args = ap.parse_args()
    global MIN_WARM_MS
    MIN_WARM_MS = args.min_warm_ms
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the method has no multi-GPU path here; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    steps, warmup = args.steps, args.warmup

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only == "prefill_lengths":
        print(json.dumps({"only": args.only, "result": bench_prefill_lengths(steps, warmup)}, default=str),
              flush=True)
        return
    if args.only in ("long_prefill70", "long_prefill_dense"):
        t = (0.7,) if args.only == "long_prefill70" else ()
        rows, _, _ = bench_long_prefill(steps, warmup, targets=t, window_leg=False)
        print(json.dumps({"only": args.only, "result": rows}, default=str), flush=True)
        return
    if args.only == "prefill_variants":
        print(json.dumps({"only": args.only, "result": bench_prefill_variants(steps, warmup)}, default=str),
              flush=True)
        return
    if args.only == "decode_shards":
        print(json.dumps({"only": args.only, "result": bench_shards(steps, warmup)}, default=str), flush=True)
        return
    if args.only == "decode_wide":
        print(json.dumps({"only": args.only, "result": bench_decode_wide(steps, warmup)}, default=str), flush=True)
        return
    if args.only == "decode_paged_layouts":
        print(json.dumps({"only": args.only, "result": bench_paged_layouts(steps, warmup)}, default=str), flush=True)
        return
    if args.only in ("decode_paged70", "mla_paged70"):
        fn = bench_decode if args.only == "decode_paged70" else bench_mla
        r = fn(steps, warmup, names=(), paged_names=("paged_s70",))
        print(json.dumps({"only": args.only, "result": r}, default=str), flush=True)
        return
    if args.only:
        which = args.only.split("70")[0].split("_dense")[0].split("_gaps")[0]
        name = "dense" if "dense" in args.only else ("gaps" if "gaps" in args.only else "s70")
        fn = {"prefill": bench_prefill, "decode": bench_decode, "mla": bench_mla}[which]
        r = fn(steps, warmup, names=(name,))
        print(json.dumps({"only": args.only, "result": r[1] if which == "prefill" else r}, default=str), flush=True)
        return

    # ------------------------------------------------------------ prefill
    (q, k, v, lam70), res, dense_flops = bench_prefill(steps, warmup)
    B, Hq, L, d = q.shape
    bc, br = 64, 128
    tile_flops = 2.0 * br * bc * d  # one (query tile, key block) product, QK or PV
    exec70 = res["s70"]["visited"] - res["s70"]["skipped"]
    mfma_flops70 = res["s70"]["visited"] * tile_flops + exec70 * tile_flops
    achieved = mfma_flops70 / (res["s70"]["ms"] * 1e-3) / 1e12
    mfma_flops_dense = 2 * res["dense"]["visited"] * tile_flops  # executed work of the dense kernel
    prefill = {
        "lambda70": lam70, "sparsity70": res["s70"]["sparsity"], "ms70": res["s70"]["ms"],
        "lambda50": res["s50"]["lambda"], "sparsity50": res["s50"]["sparsity"], "ms50": res["s50"]["ms"],
        "ms_dense": res["dense"]["ms"],
        "dense_equiv_tflops_dense_path": res["dense"]["dense_equiv_tflops"],
        "speedup70_vs_dense": res["dense"]["ms"] / res["s70"]["ms"],
        "speedup50_vs_dense": res["dense"]["ms"] / res["s50"]["ms"],
        "mfma_util_executed70": achieved / PEAK_BF16_TFLOPS,
        "mfma_util_dense": mfma_flops_dense / (res["dense"]["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "ms_skip_logic_nothing_skipped": res["skip0"]["ms"],
        "skip_logic_overhead_vs_dense": res["skip0"]["ms"] / res["dense"]["ms"] - 1.0,
        "gap_pass": {"ms": res["gaps"]["ms"], "vs_dense": res["gaps"]["ms"] / res["dense"]["ms"],
                     "note": "calibration pass: scores, block maxima, running max and decisions; no exp, V or P.V"},
        "timed_calls_return_counts": True,
    }

    # ------------------------------------------------------------- decode
    decode = mla = long_prefill = shards = None
    if not args.no_decode:
        oc = not args.no_cpu_baseline
        S, dres = bench_decode(steps, warmup, paged_names=("paged_s70", "paged_dense"), window=4096, seed=True,
                               oracle_cpu=oc)
        decode = {
            "workload": "GQA decode B=148 Hq=32 Hkv=8 L=32768 d=128 bf16, block 64, one query token per sequence",
            "num_splits": S,
            "us_per_step70": dres["s70"]["us"], "sparsity70": dres["s70"]["sparsity"],
            "us_per_step50": dres["s50"]["us"], "sparsity50": dres["s50"]["sparsity"],
            "us_per_step_dense": dres["dense"]["us"],
            "speedup70_vs_dense": dres["dense"]["us"] / dres["s70"]["us"],
            "speedup50_vs_dense": dres["dense"]["us"] / dres["s50"]["us"],
            "us_skip_logic_nothing_skipped": dres["skip0"]["us"],
            "skip_logic_overhead_vs_dense": dres["skip0"]["us"] / dres["dense"]["us"] - 1.0,
            "roofline": {"bound": "hbm", "achieved": dres["s70"]["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": dres["s70"]["gbps"] / PEAK_HBM_GBS, "traffic": measured_traffic("decode70"),
                         "algorithmic_bytes": dres["s70"]["bytes"]},
            "paged": {"page_size": 64, "layout": "pool [pages, Hkv, 64, d] in shuffled order, int32 page table",
                      "us_per_step70": dres["paged_s70"]["us"], "sparsity70": dres["paged_s70"]["sparsity"],
                      "us_per_step_dense": dres["paged_dense"]["us"],
                      "overhead70_vs_contiguous": dres["paged_s70"]["us"] / dres["s70"]["us"] - 1.0,
                      "overhead_dense_vs_contiguous": dres["paged_dense"]["us"] / dres["dense"]["us"] - 1.0},
            "window": {"window": 4096, "num_splits": dres["window_s70"]["splits"],
                       "us_per_step70": dres["window_s70"]["us"], "sparsity70": dres["window_s70"]["sparsity"],
                       "us_per_step_dense": dres["window_dense"]["us"],
                       "speedup70_vs_dense": dres["window_dense"]["us"] / dres["window_s70"]["us"],
                       "hbm_gbps70": dres["window_s70"]["gbps"], "hbm_gbps_dense": dres["window_dense"]["gbps"]},
            "sink_seed": dres["sink_seed"],
            "gap_pass": {"us": dres["gaps"]["us"], "vs_dense": dres["gaps"]["us"] / dres["dense"]["us"],
                         "hbm_gbps": dres["gaps"]["gbps"]},
            "cpu_oracle": dres.get("cpu_oracle"),
        }
        torch.cuda.empty_cache()
        S, mres = bench_mla(steps, warmup, paged_names=("paged_s70", "paged_dense"), seed=True, oracle_cpu=oc)
        m70 = mres["s70"]
        mla = {
            "workload": "latent (MLA) decode B=16 Hq=128 sharing one KV head, dqk=576 dv=512 (V = K[..., :512]), "
                        "L=65536, bf16 cache, block 64",
            "num_splits": S,
            "us_per_step70": m70["us"], "sparsity70": m70["sparsity"],
            "us_per_step50": mres["s50"]["us"], "sparsity50": mres["s50"]["sparsity"],
            "us_per_step_dense": mres["dense"]["us"],
            "speedup70_vs_dense": mres["dense"]["us"] / m70["us"],
            "us_skip_logic_nothing_skipped": mres["skip0"]["us"],
            "skip_logic_overhead_vs_dense": mres["skip0"]["us"] / mres["dense"]["us"] - 1.0,
            "hbm_gbps70": m70["gbps"], "mfma_tflops70": m70["tflops"],
            "mfma_tflops_dense": mres["dense"]["tflops"], "hbm_gbps_dense": mres["dense"]["gbps"],
            "roofline": {"bound": "hbm", "achieved": m70["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": m70["gbps"] / PEAK_HBM_GBS, "traffic": measured_traffic("mla70"),
                         "algorithmic_bytes": m70["bytes"], "mfma_frac": m70["tflops"] / PEAK_BF16_TFLOPS},
            "paged": {"page_size": 64, "layout": "pool [pages, 1, 64, 576] in shuffled order, int32 page table",
                      "us_per_step70": mres["paged_s70"]["us"], "sparsity70": mres["paged_s70"]["sparsity"],
                      "us_per_step_dense": mres["paged_dense"]["us"],
                      "overhead70_vs_contiguous": mres["paged_s70"]["us"] / m70["us"] - 1.0,
                      "overhead_dense_vs_contiguous": mres["paged_dense"]["us"] / mres["dense"]["us"] - 1.0},
            "sink_seed": mres["sink_seed"],
            "gap_pass": {"us": mres["gaps"]["us"], "vs_dense": mres["gaps"]["us"] / mres["dense"]["us"],
                         "hbm_gbps": mres["gaps"]["gbps"]},
            "cpu_oracle": mres.get("cpu_oracle"),
        }
        torch.cuda.empty_cache()
        shards = bench_shards(steps, warmup)
        sweep, wres, lcpu = bench_long_prefill(max(2, steps // 4), max(1, warmup // 2), oracle_cpu=oc)
        r70 = next((r for r in sweep if r["target"] == 0.7), None)
        long_prefill = {
            "workload": "GQA causal prefill B=2 Hq=32 Hkv=8 L=32768 d=128 bf16, query tile 128, key block 64",
            "roofline": None if r70 is None else {
                "bound": "mfma", "achieved": r70["mfma_flops"] / (r70["ms"] * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": r70["mfma_util_executed"], "traffic": measured_traffic("long_prefill70"),
                "algorithmic_flops": r70["mfma_flops"]},
            "speedup70_vs_dense": None if r70 is None else r70["speedup_vs_dense"],
            "sweep": sweep,
            "window": wres,
            "cpu_oracle": lcpu,
        }
        torch.cuda.empty_cache()

    peaks = measured_peaks()

    calibration = None
    if not args.no_calibration:
        calibration = bench_calibration()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(q, k, v, lam70)
        log(f"cpu oracle: {cpu['value']:.4f} TFLOP/s dense-equivalent on {cpu['cores']} threads")

    line = {
        "metric": "prefill dense-equiv TFLOP/s + decode us/step at ~70% block skip vs lambda=0",
        "value": res["s70"]["dense_equiv_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": res["s70"]["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "GQA causal prefill B=1 Hq=32 Hkv=8 L=8192 d=128 bf16, query tile 128, "
                               "key block 64, lambda calibrated for 70% block sparsity",
                   "global_batch": B, "seq_len": L, "parallelism": "none (1 GPU)"},
        "prefill": prefill,
        "decode": decode,
        "mla_decode": mla,
        "decode_shard_of_8_gpus": shards,
        "long_prefill": long_prefill,
        "calibration": calibration,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill70"),
                     "algorithmic_flops": mfma_flops70},
        "cpu_baseline": cpu,
        "measured_peaks": peaks,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

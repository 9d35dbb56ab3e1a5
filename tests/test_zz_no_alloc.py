"""The no-allocation decode entry point against blasst_decode (same kernels,
caller workspace): two calls in a row, the second smaller, for the GQA and the
latent head layouts; outputs, skip maps and counters must be identical, and the
outputs must meet the parity bar against the oracle."""
import numpy as np
import pytest
import torch

import long_context_fa_amd as bl
import oracle
from long_context_fa_amd import inputs
from parity import check_output

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _both(q, kc, vc, lens, lam, splits, dv=None):
    B, Hkv, L = q.shape[0], kc.shape[1], kc.shape[2]
    nkb = -(-L // 64)
    out = {}
    for name in ("ws", "noalloc"):
        sk = torch.full((B, Hkv, nkb), 77, dtype=torch.uint8, device=DEV)
        cnt = torch.zeros(2, dtype=torch.int64, device=DEV)
        fn = bl.blasst_decode if name == "ws" else bl.blasst_decode_noalloc
        o = fn(q, kc, vc, lens, lam=lam, num_splits=splits, dv=dv, skip_map=sk, counters=cnt)
        torch.cuda.synchronize()
        out[name] = (o.cpu(), sk.cpu(), cnt.cpu())
    for a, b in zip(out["ws"], out["noalloc"]):
        assert torch.equal(a, b)
    return out["noalloc"][0]


@pytest.mark.parametrize("layout", ["gqa", "latent"])
def test_noalloc_matches_workspace_call_twice_second_smaller(layout):
    cases = ([(6, 32, 8, 4096, 4), (2, 16, 4, 1536, 3)] if layout == "gqa"
             else [(3, 128, 1, 8192, 16), (1, 128, 1, 2048, 5)])
    for i, (B, Hq, Hkv, L, S) in enumerate(cases):
        print(f"noalloc {layout} call {i}: B={B} Hq={Hq} Hkv={Hkv} L={L} splits={S}", flush=True)
        if layout == "gqa":
            q, kc, vc, lens = inputs.decode_inputs(B, Hq, Hkv, L, 128, device=DEV, seed=700 + i)
            dv = None
        else:
            q, kc, _, lens = inputs.decode_inputs(B, Hq, 1, L, 576, 512, n_random=16, mla=True, device=DEV,
                                                  seed=710 + i)
            vc, dv = kc, 512
        lens[0] = L - 37  # a ragged length
        lam = 1e-3
        o = _both(q, kc, vc, lens, lam, S, dv)
        kk = _f64(kc)
        ref = oracle.decode(_f64(q), kk, kk[..., :dv] if dv else _f64(vc), lens.cpu().numpy(),
                            lam=lam, block_k=64, num_splits=S)
        check_output(o.numpy(), ref["o"], f"noalloc {layout} call {i}")


def test_noalloc_refuses_partials_beyond_the_scratch():
    q, kc, vc, lens = inputs.decode_inputs(1, 4, 1, 64 * 64, 64, device=DEV, seed=9)
    qb = q.expand(60000, 4, 64)   # many sequences, shapes only: refused before any launch
    kb = kc.expand(60000, 1, 4096, 64)
    lb = lens.expand(60000).contiguous()
    with pytest.raises(bl.BlasstError) as ei:
        bl.blasst_decode_noalloc(qb, kb, kb, lb, lam=1e-3, num_splits=64)
    assert ei.value.status == 3 and "scratch" in bl.blasst_last_error()

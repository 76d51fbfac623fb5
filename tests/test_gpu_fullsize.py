"""GPU parity at the five workloads' full sizes, through moe_forward as bench.py calls it.

Routing ids and the aligned slot order are compared in full (bit-exact).  The
layer output is compared on sampled tokens the float64 oracle computes one by
one (a token's output does not depend on the batch it is in), and checked for
finiteness everywhere; a second run must be bitwise identical.
"""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import moe as O

pytestmark = pytest.mark.gpu

M = pytest.importorskip("bit_weight_expert_amd")
from gpu_util import assert_rows_close, gpu_forward, host_bf16, upload  # noqa: E402

SAMPLE = (0, 1, 7, 63, 511, 2047, 4095, 8191)
_cache = {}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    _cache.clear()


def _config(cfg):
    if cfg not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        L = S.make_config(cfg)
        D = upload(L)
        toks = [t for t in SAMPLE if t < L.T]
        ref = O.forward_tokens(L, toks)
        _cache[cfg] = (L, D, toks, ref)
    return _cache[cfg]


CASES = [(1, 32)] + [(2, t) for t in S.CONFIGS[2]["T"]] + [(3, 2048)] + \
        [(4, t) for t in S.CONFIGS[4]["T"]] + [(5, 2048)]


@pytest.mark.parametrize("cfg,T", CASES)
def test_forward_full_size(cfg, T):
    L, D, toks, ref = _config(cfg)
    Lt = L.take(T)
    Dt = dict(D, x=D["x"][:T], logits=D["logits"][:T])
    print(f"config {cfg} T={T} E={L.E} k={L.top_k} H={L.H} I={L.I} {L.w13.fmt}", flush=True)
    out = gpu_forward(Lt, Dt)
    # routing and align, bit-exact, at the tile size moe_forward uses
    ids_ref, w_ref = O.route(Lt)
    ids, w = M.moe_route(Dt["logits"], L.top_k, L.route, Dt["expert_bias"], L.renormalize)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=2e-6)
    bm = M.moe_forward_block_m(T, L.top_k, L.E)
    si, ei, npp = M.moe_align(ids, L.E, bm)
    si_ref, ei_ref, npp_ref = O.align(ids_ref, L.E, bm)
    np.testing.assert_array_equal(si.cpu().numpy(), si_ref)
    np.testing.assert_array_equal(ei.cpu().numpy(), ei_ref)
    assert int(npp.item()) == int(npp_ref)
    # output: finite everywhere, oracle rows on the sampled tokens
    got = host_bf16(out)
    assert np.isfinite(got).all()
    rows = [i for i, t in enumerate(toks) if t < T]
    err = assert_rows_close(got[[toks[i] for i in rows]], ref[rows], what=f"config {cfg} T={T}")
    print(f"config {cfg} T={T}: max per-row rel err {err:.2e} over {len(rows)} sampled tokens", flush=True)
    # determinism
    out2 = gpu_forward(Lt, Dt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))

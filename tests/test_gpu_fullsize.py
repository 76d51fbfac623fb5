"""GPU parity at the five workloads' full sizes, through moe_forward as bench.py calls it.

Routing ids and the aligned slot order are compared in full (bit-exact).  The
workspace and the output start as 0xFF bytes (bf16 NaN), so a tile that is
skipped, or that reads a workspace region before it is written, shows: every
output row must come back finite.  The layer output is compared with the
float64 oracle on a sample of tokens chosen so that every aligned block that
moe_forward forms at the batch's tile size holds at least one compared slot
(each expert's last, partial block included; every compared row spans all
column tiles of both GEMMs).  A token's output does not depend on the batch
it is in, so one oracle pass per workload serves every token count.  A second
run must be bitwise identical.
"""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import moe as O

pytestmark = pytest.mark.gpu

M = pytest.importorskip("bit_weight_expert_amd")
from gpu_util import (assert_rows_close, block_covering_tokens, gpu_forward,  # noqa: E402
                      host_bf16, upload)

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
    """Inputs at the config's largest T, the compared tokens of each T and the
    oracle's rows for their union."""
    if cfg not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        L = S.make_config(cfg)
        D = upload(L)
        ids_ref, _ = O.route(L)
        per_t = {}
        for T in S.CONFIGS[cfg]["T"]:
            bm = M.moe_forward_block_m(T, L.top_k, L.E)
            per_t[T] = block_covering_tokens(ids_ref[:T], L.E, bm, extra=SAMPLE)
        toks = sorted(set().union(*per_t.values()))
        print(f"config {cfg}: oracle on {len(toks)} tokens", flush=True)
        ref = dict(zip(toks, O.forward_tokens(L, toks)))
        _cache[cfg] = (L, D, per_t, ref)
    return _cache[cfg]


CASES = [(1, 32)] + [(2, t) for t in S.CONFIGS[2]["T"]] + [(3, 2048)] + \
        [(4, t) for t in S.CONFIGS[4]["T"]] + [(5, 2048)]


@pytest.mark.parametrize("cfg,T", CASES)
def test_forward_full_size(cfg, T):
    print(f"config {cfg} T={T}: preparing", flush=True)
    L, D, per_t, ref = _config(cfg)
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
    # output: finite everywhere (it started as NaN), oracle rows on tokens
    # that cover every aligned block
    got = host_bf16(out)
    assert np.isfinite(got).all(), f"config {cfg} T={T}: non-finite output rows"
    toks = per_t[T]
    err = assert_rows_close(got[toks], np.stack([ref[t] for t in toks]), what=f"config {cfg} T={T}")
    print(f"config {cfg} T={T}: max per-row rel err {err:.3e} over {len(toks)} tokens covering "
          f"all {int(npp_ref) // bm} blocks of {bm} rows", flush=True)
    # determinism
    out2 = gpu_forward(Lt, Dt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))

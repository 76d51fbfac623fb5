"""moe_forward_noalloc: the layer on the library's fixed per-GPU scratch.

Compared through the C-ABI with moe_forward (which takes the same kernels on a
caller workspace): bit-identical outputs, and within the tolerance of the
float64 oracle on tokens covering every aligned block; two calls in a row,
the second with a smaller batch (the scratch keeps the first call's
contents); a call that needs more than the scratch fails on the host.
"""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import moe as O

pytestmark = pytest.mark.gpu

M = pytest.importorskip("bit_weight_expert_amd")
from gpu_util import (assert_rows_close, block_covering_tokens, gpu_forward,  # noqa: E402
                      host_bf16, poisoned, upload)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _noalloc(L, D, T):
    out = poisoned((T, L.H))
    return M.moe_forward_noalloc(D["x"][:T], D["logits"][:T], L.top_k, L.I, D["w13"], D["w2"],
                                 out, act=L.act, route=L.route, expert_bias=D["expert_bias"],
                                 renormalize=L.renormalize, alpha=L.alpha, beta=L.beta,
                                 limit=L.limit, mul_topk_weights=L.mul_topk_weights)


@pytest.mark.parametrize("cfg,Ts", [(2, (1024, 40)), (5, (700, 3)), (3, (96, 1))])
def test_noalloc_matches_forward(cfg, Ts):
    L = S.make_config(cfg)
    D = upload(L)
    ids_all, _ = O.route(L)
    for T in Ts:                                   # the second call is smaller
        print(f"noalloc config {cfg} T={T}", flush=True)
        Lt = L.take(T)
        Dt = dict(D, x=D["x"][:T], logits=D["logits"][:T])
        got = _noalloc(L, D, T)
        ref_gpu = gpu_forward(Lt, Dt)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref_gpu.view(torch.int16)), \
            f"config {cfg} T={T}: moe_forward_noalloc differs from moe_forward"
        bm = M.moe_forward_block_m(T, L.top_k, L.E)
        toks = block_covering_tokens(ids_all[:T], L.E, bm, extra=(0, T - 1))
        g = host_bf16(got)
        assert np.isfinite(g).all()
        err = assert_rows_close(g[toks], O.forward_tokens(Lt, toks), what=f"noalloc config {cfg} T={T}")
        print(f"noalloc config {cfg} T={T}: bitwise equal to moe_forward, max rel err {err:.3e}",
              flush=True)


def test_noalloc_rejects_beyond_scratch():
    L = S.make_config(2)
    T = 2048                                         # needs ~133 MB of workspace
    need = M.moe_forward_workspace_bytes(T, L.E, L.top_k, L.H, L.I)
    assert need > M.NOALLOC_SCRATCH_BYTES
    D = upload(L)
    out = poisoned((T, L.H))
    with pytest.raises(M.MoeError) as ei:
        M.moe_forward_noalloc(D["x"][:T], D["logits"][:T], L.top_k, L.I, D["w13"], D["w2"], out)
    assert ei.value.status == 7
    torch.cuda.synchronize()
    assert (out.view(torch.int16) == -1).all()      # nothing was enqueued

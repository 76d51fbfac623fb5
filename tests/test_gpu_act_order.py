"""GPU parity of GPTQ act-order: the weight-prep sort, the per-slot gather and the layer.

The sort and the gather only move bits, so they are compared bit-exact (with
the oracle's act_order_sort and a numpy gather).  The layer runs through
moe_forward with the group-ordered families and their k_perm, and is compared
with the float64 oracle reading the original rows through g_idx, within the
layer tolerance.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import formats as F
from oracle import moe as O

pytestmark = pytest.mark.gpu

M = pytest.importorskip("bit_weight_expert_amd")
from gpu_util import (assert_rows_close, gpu_forward, host_bf16,  # noqa: E402
                      upload)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def prepare(w, Dw):
    """Group-ordered device family with k_perm, from act-order host weights w."""
    qs, kp, st = M.moe_gptq_act_order_sort(Dw.qweight, torch.from_numpy(w.g_idx).cuda(), w.group)
    torch.cuda.synchronize()
    assert not st.any().item(), st.cpu().numpy()
    return dataclasses.replace(Dw, qweight=qs, k_perm=kp)


@pytest.mark.parametrize("K,N,G", [(2880, 256, 64), (256, 40, 32), (8192, 16, 128), (2688, 264, 64)])
def test_sort_bitexact(K, N, G):
    E = 5
    w = S.make_weights("gptq", E=E, N=N, K=K, group=G, bias=False, seed=K + N, act_order=True)
    g_idx = w.g_idx.copy()
    g = np.flatnonzero(g_idx[1] == 0)[0]
    g_idx[1, g] = 1                                   # expert 1: group 0 short, group 1 long
    g_idx[3, 7] = K // G                              # expert 3: a group id out of range
    print(f"sort K={K} N={N} G={G}", flush=True)
    qw = torch.from_numpy(w.qweight).cuda()
    qs, kp, st = M.moe_gptq_act_order_sort(qw, torch.from_numpy(g_idx).cuda(), G)
    torch.cuda.synchronize()
    qs, kp, st = qs.cpu().numpy(), kp.cpu().numpy(), st.cpu().numpy()
    for e in range(E):
        ref_q, ref_p, ok = F.act_order_sort(w.qweight[e], g_idx[e], G)
        assert st[e] == (0 if ok else 1), (e, st)
        assert ok == (e not in (1, 3))
        np.testing.assert_array_equal(kp[e], ref_p)
        if ok:
            np.testing.assert_array_equal(qs[e], ref_q)


@pytest.mark.parametrize("top_k,inplace", [(4, False), (1, False), (1, True), (6, False)])
def test_permute_slots_bitexact(top_k, inplace):
    rng = np.random.default_rng(top_k + 10 * inplace)
    m, K, E = 37, 2880 if top_k != 6 else 2688, 9
    src = rng.integers(-32768, 32767, size=(m, K), dtype=np.int64).astype(np.int16)
    perm = np.stack([rng.permutation(K) for _ in range(E)]).astype(np.int32)
    ids = rng.integers(-1, E + 1, size=(m * top_k,), dtype=np.int64).astype(np.int32)  # some invalid
    fill = np.full((m * top_k, K), 0x1234, dtype=np.int16)
    print(f"permute top_k={top_k} inplace={inplace}", flush=True)
    d_src = torch.from_numpy(src).cuda().view(torch.bfloat16)
    if inplace:
        out = d_src
    else:
        out = torch.from_numpy(fill).cuda().view(torch.bfloat16)
    M.moe_permute_slots(d_src, top_k, torch.from_numpy(perm).cuda(), torch.from_numpy(ids).cuda(),
                        out=out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy()
    ref = (src.copy() if inplace else fill.copy())
    for f in range(m * top_k):
        e = ids[f]
        if 0 <= e < E:
            ref[f] = src[f // top_k][perm[e]]
    np.testing.assert_array_equal(got, ref)


def _layer(act="swigluoai", E=4, k=2, H=320, I=192, T=13, G=64, seed=31, **kw):
    # unit-scale inputs, as in the other layer tests: GPTQ weights are rounded
    # to bf16 once for the matrix cores, and at x_std = 4 that rounding alone
    # brings rows of the plain (identity g_idx) GPTQ layer to the tolerance
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    return S.make_layer(E=E, top_k=k, H=H, I=I, fmt="gptq", act=act, route=route, T=T,
                        seed=seed, group=G, act_order=True,
                        router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw)


def _plain(w, seed):
    """A family of the same shape without act-order (for one-sided cases)."""
    return S.make_weights("gptq", E=w.qweight.shape[0], N=w.N, K=w.K, group=w.group, seed=seed)


@pytest.mark.parametrize("act", ["swigluoai", "relu2"])
@pytest.mark.parametrize("T", [1, 13, 200])
@pytest.mark.parametrize("which", ["both", "w13", "w2"])
@pytest.mark.parametrize("policy", ["auto", "wide"])
def test_forward_act_order(act, T, which, policy):
    L = _layer(act, T=T, G=32 if act == "relu2" else 64)
    if which == "w13":
        L = dataclasses.replace(L, w2=_plain(L.w2, 5))
    elif which == "w2":
        L = dataclasses.replace(L, w13=_plain(L.w13, 6))
    D = upload(L)
    if L.w13.g_idx is not None:
        D["w13"] = prepare(L.w13, D["w13"])
    if L.w2.g_idx is not None:
        D["w2"] = prepare(L.w2, D["w2"])
    print(f"act-order forward {act} T={T} {which} {policy}", flush=True)
    out = gpu_forward(L, D, kernel=policy)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"act-order {act} T{T} {which}")


def test_forward_act_order_weight_on_input():
    L = dataclasses.replace(_layer(E=6, k=1, T=40, renormalize=False), weight_on_input=True)
    D = upload(L)
    D["w13"], D["w2"] = prepare(L.w13, D["w13"]), prepare(L.w2, D["w2"])
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what="act-order weight on input")


@pytest.mark.parametrize("T", [64, 2048])
def test_forward_act_order_full_size(T):
    """The INT4-GPTQ g64 gpt-oss-20b layer shape (E=32, top-4, 2880/2880)
    quantised in activation order; sampled tokens against the oracle."""
    c = dict(S.CONFIGS[3])
    c.pop("name")
    c.pop("T")
    L = S.make_layer(T=2048, seed=S.config_seed(3) + 1, act_order=True, **c).take(T)
    D = upload(L)
    D["w13"], D["w2"] = prepare(L.w13, D["w13"]), prepare(L.w2, D["w2"])
    print(f"act-order full size T={T}", flush=True)
    out = gpu_forward(L, D)
    toks = [t for t in (0, 1, 7, 63, 511, 2047) if t < T]
    ref = O.forward_tokens(L, toks)
    got = host_bf16(out)
    assert np.isfinite(got).all()
    assert_rows_close(got[toks], ref, what=f"act-order full size T{T}")


def test_forward_act_order_empty_batch():
    L = _layer(T=4)
    D = upload(L)
    D["w13"], D["w2"] = prepare(L.w13, D["w13"]), prepare(L.w2, D["w2"])
    out = M.moe_forward(D["x"][:0], D["logits"][:0], L.top_k, L.I, D["w13"], D["w2"])
    assert out.shape == (0, L.H)

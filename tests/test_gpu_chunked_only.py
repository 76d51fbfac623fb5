"""GPU parity of chunked-only NVFP4/MXFP4 families: the codes and scales by K
chunk alone on the device (QuantWeights.chunked_only, qweight = scales = NULL
at the C-ABI), so every kernel -- split-K, wide, streaming, MX -- reads them.

Each path is compared with the float64 oracle (per-row 5e-3, as everywhere)
and, where the same kernel runs on the checkpoint layout, bit for bit with
that run: the two layouts hold the same bytes in another order, and the
kernels do the same arithmetic in the same order on both.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import moe as O

pytestmark = pytest.mark.gpu

M = pytest.importorskip("bit_weight_expert_amd")
from gpu_util import (assert_rows_close, assert_untouched, block_covering_tokens,  # noqa: E402
                      dev_bf16, gpu_forward, host_bf16, poisoned, upload)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _layer(fmt, act="swigluoai", E=4, k=2, H=320, I=192, T=13, seed=71, **kw):
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    return S.make_layer(E=E, top_k=k, H=H, I=I, fmt=fmt, act=act, route=route, T=T, seed=seed,
                        router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw)


def _align(L, B):
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    dev = tuple(torch.from_numpy(a).cuda() for a in (si, ei, np.array([npp], np.int32)))
    return ids, w, (si, ei, npp), dev


def _same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{what}: layouts differ"


# (block_m, kernel): split-K and wide kernels on 16/32-row blocks, the
# streaming kernel on 64/128-row blocks (its checkpoint-layout form is
# another kernel, so those cases compare with the oracle only)
PATHS = [(16, "splitk"), (16, "wide"), (32, "wide"), (32, "splitk"), (64, "auto"), (128, "auto")]


@pytest.mark.parametrize("fmt,H", [("nvfp4", 320), ("nvfp4", 2880), ("mxfp4", 352),
                                   ("mxfp4", 2880)])
@pytest.mark.parametrize("B,kernel", PATHS)
def test_gemm1_chunked_only(fmt, H, B, kernel):
    L = _layer(fmt, H=H, T=40, x_std=4.0)
    D = upload(L)
    wkc = D["w13"].chunked_only()
    assert wkc.qweight is None and wkc.scales is None
    ids, w, (si, ei, npp), da = _align(L, B)
    n_out = L.w13.N // 2
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, "swigluoai", L.alpha, L.beta, L.limit, si, ei,
                       npp, B)
    print(f"gemm1 chunked-only {fmt} H={H} B={B} {kernel}", flush=True)
    outs = []
    for wq in (wkc, D["w13"]):
        out = poisoned((L.T * L.top_k, n_out))
        M.moe_w4a16_gemm1(D["x"], L.top_k, wq, "swigluoai", L.alpha, L.beta, L.limit, *da, B,
                          out=out, kernel=kernel)
        outs.append(out)
    assert_rows_close(host_bf16(outs[0]), ref, rows=cov, what=f"gemm1 chunked-only {fmt} B{B}")
    assert_untouched(outs[0], cov, "gemm1 chunked-only")
    if B <= 32:
        _same_bits(outs[0], outs[1], f"gemm1 {fmt} H{H} B{B} {kernel}")


@pytest.mark.parametrize("fmt,I", [("nvfp4", 192), ("nvfp4", 2880), ("mxfp4", 224),
                                   ("mxfp4", 2880)])
@pytest.mark.parametrize("B,kernel", PATHS)
def test_gemm2_chunked_only(fmt, I, B, kernel):
    L = _layer(fmt, I=I, E=5, k=3, T=23)
    D = upload(L)
    wkc = D["w2"].chunked_only()
    ids, w, (si, ei, npp), da = _align(L, B)
    n = L.T * L.top_k
    rng = np.random.default_rng(I + B)
    a_bits = S.f32_to_bf16_bits(rng.standard_normal((n, I)).astype(np.float32))
    tw = w.reshape(-1).astype(np.float32)
    ref, cov = O.gemm2(a_bits, n, L.w2, tw, True, si, ei, npp, B)
    print(f"gemm2 chunked-only {fmt} I={I} B={B} {kernel}", flush=True)
    outs = []
    for wq in (wkc, D["w2"]):
        out = poisoned((n, L.H))
        M.moe_w4a16_gemm2(dev_bf16(a_bits), wq, torch.from_numpy(tw).cuda(), True, *da, B,
                          out=out, kernel=kernel)
        outs.append(out)
    assert_rows_close(host_bf16(outs[0]), ref, rows=cov, what=f"gemm2 chunked-only {fmt} B{B}")
    assert_untouched(outs[0], cov, "gemm2 chunked-only")
    if B <= 32:
        _same_bits(outs[0], outs[1], f"gemm2 {fmt} I{I} B{B} {kernel}")


@pytest.mark.parametrize("fmt,act", [("nvfp4", "swigluoai"), ("nvfp4", "relu2"),
                                     ("mxfp4", "swigluoai")])
@pytest.mark.parametrize("T", [1, 13, 200, 600])
def test_forward_chunked_only(fmt, act, T):
    """1 and 13 tokens: 16-row blocks; 200 and 600: 64/128-row blocks."""
    L = _layer(fmt, act, E=6, T=T)
    D = upload(L)
    D["w13"], D["w2"] = D["w13"].chunked_only(), D["w2"].chunked_only()
    print(f"forward chunked-only {fmt} {act} T={T}", flush=True)
    got = host_bf16(gpu_forward(L, D))
    assert np.isfinite(got).all()
    assert_rows_close(got, O.forward(L)["out"], what=f"forward chunked-only {fmt} {act} T{T}")


@pytest.mark.parametrize("cfg,T", [(2, 1), (2, 64), (2, 4096), (4, 8), (4, 1024)])
def test_forward_chunked_only_full_size(cfg, T):
    """gpt-oss-20b NVFP4 (1, 64 and 4096 tokens) and gpt-oss-120b MXFP4 (8 and
    1024 tokens, skewed: the mixed tiling) held chunked-only; tokens covering
    every aligned block against the oracle, and the same output bit for bit
    as the family holding both layouts."""
    L = S.make_config(cfg, T)
    D = upload(L)
    both = {}
    for name in ("w13", "w2"):
        kc = D[name].chunked_only()
        both[name] = dataclasses.replace(D[name], scales_kc=kc.scales_kc, qweight_kc=kc.qweight_kc)
        D[name] = kc
    print(f"forward chunked-only full size cfg{cfg} T={T}", flush=True)
    out = gpu_forward(L, D)
    ref_both = gpu_forward(L, {**D, **both})
    _same_bits(out, ref_both, f"forward cfg{cfg} T{T}")
    ids, _ = O.route(L)
    toks = block_covering_tokens(ids, L.E, M.moe_forward_block_m(T, L.top_k, L.E),
                                 extra=(0, T - 1))
    got = host_bf16(out)
    assert np.isfinite(got).all()
    err = assert_rows_close(got[toks], O.forward_tokens(L, toks),
                            what=f"forward chunked-only cfg{cfg} T{T}")
    print(f"chunked-only cfg{cfg} T={T}: max per-row rel err {err:.3e} over {len(toks)} tokens",
          flush=True)


@pytest.mark.parametrize("T", [1, 200])
def test_forward_mxfp8_chunked_only(T):
    """The MXFP8-activation layer (MX kernels) on a chunked-only MXFP4 family:
    the same bits as with the checkpoint scales beside the codes by chunk."""
    L = _layer("mxfp4", E=6, T=T, H=352, I=224)
    D = upload(L)
    outs = []
    for mk in (lambda w: w.chunked_only(),
               lambda w: dataclasses.replace(w, qweight_kc=M.moe_mxfp4_codes_by_chunk(w))):
        w13, w2 = mk(D["w13"]), mk(D["w2"])
        out = poisoned((T, L.H))
        M.moe_forward_mxfp8(D["x"], D["logits"], L.top_k, L.I, w13, w2, act=L.act, route=L.route,
                            alpha=L.alpha, beta=L.beta, limit=L.limit, out=out)
        outs.append(out)
    _same_bits(outs[0], outs[1], f"mxfp8 forward T{T}")
    assert np.isfinite(host_bf16(outs[0])).all()

"""GPU parity of the NVFP4 weights with their scales (and codes) laid out by K chunk.

The re-layouts move bytes only and are compared bit-exact with NumPy; the
64/128-row GEMM kernel that streams the chunk scales (scales only, or scales
and codes by chunk) is compared with the float64 oracle (which reads the
checkpoint layout) like the other GEMM paths.
"""
import dataclasses

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


def with_kc(Dw, codes=False):
    return dataclasses.replace(Dw, scales_kc=M.moe_nvfp4_scales_by_chunk(Dw),
                               qweight_kc=M.moe_nvfp4_codes_by_chunk(Dw) if codes else None)


CODES = pytest.mark.parametrize("codes", [False, True], ids=["scales", "scales+codes"])


@pytest.mark.parametrize("E,N,K", [(3, 384, 320), (2, 2880, 2880), (5, 16, 64)])
def test_scales_by_chunk_bitexact(E, N, K):
    w = S.make_weights("nvfp4", E=E, N=N, K=K, bias=False, seed=N + K)
    Dw = upload_w = M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales,
                                                None, w.global_scale, None)
    got = M.moe_nvfp4_scales_by_chunk(upload_w).cpu().numpy()
    ref = w.scales.reshape(E, N, K // 64, 4).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(got, ref)
    assert Dw.scales.shape == (E, N, K // 16)


@pytest.mark.parametrize("E,N,K", [(3, 384, 320), (2, 2880, 2880), (5, 16, 64)])
def test_codes_by_chunk_bitexact(E, N, K):
    w = S.make_weights("nvfp4", E=E, N=N, K=K, bias=False, seed=N + K + 1)
    Dw = M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales, None,
                                    w.global_scale, None)
    got = M.moe_nvfp4_codes_by_chunk(Dw).cpu().numpy()
    ref = w.qweight.reshape(E, N, K // 64, 32).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(got, ref)
    assert got.shape == (E, K // 64, N, 32)


def _small(act="swigluoai", E=4, k=2, H=320, I=192, T=300, seed=51, **kw):
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    return S.make_layer(E=E, top_k=k, H=H, I=I, fmt="nvfp4", act=act, route=route, T=T, seed=seed,
                        router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw)


@CODES
@pytest.mark.parametrize("act", ["none", "swigluoai", "relu2"])
@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("H", [320, 2880])
def test_gemm1_scales_by_chunk(act, B, H, codes):
    L = _small("relu2" if act == "relu2" else "swigluoai", H=H, T=300 if H < 2880 else 150,
               x_std=12.0)
    D = upload(L)
    w13 = with_kc(D["w13"], codes)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    print(f"gemm1 by chunk act={act} B={B} H={H} codes={codes}", flush=True)
    out = M.moe_w4a16_gemm1(D["x"], L.top_k, w13, act, L.alpha, L.beta, L.limit, t(si), t(ei),
                            t(np.array([npp], np.int32)), B)
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, act, L.alpha, L.beta, L.limit, si, ei, npp, B)
    assert_rows_close(host_bf16(out), ref, rows=cov, what=f"gemm1 scales by chunk {act} B{B} H{H}")


@CODES
@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("I", [192, 2880])
def test_gemm2_scales_by_chunk(B, I, codes):
    L = _small(I=I, T=300 if I < 2880 else 150)
    D = upload(L)
    w2 = with_kc(D["w2"], codes)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    n = L.T * L.top_k
    a_bits = S.f32_to_bf16_bits(np.random.default_rng(I + B).standard_normal((n, I)).astype(np.float32))
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    print(f"gemm2 by chunk B={B} I={I} codes={codes}", flush=True)
    y = M.moe_w4a16_gemm2(t(a_bits.view(np.int16)).view(torch.bfloat16), w2,
                          t(w.reshape(-1).astype(np.float32)), True, t(si), t(ei),
                          t(np.array([npp], np.int32)), B)
    ref, cov = O.gemm2(a_bits, n, L.w2, w.reshape(-1), True, si, ei, npp, B)
    assert_rows_close(host_bf16(y), ref, rows=cov, what=f"gemm2 scales by chunk B{B} I{I}")


@CODES
@pytest.mark.parametrize("T", [13, 200, 600])
def test_forward_scales_by_chunk(T, codes):
    """T = 13: 16-row blocks (the decode kernels ignore the re-laid copies);
    T = 200, 600: 128-row blocks on the streaming kernel."""
    L = _small(T=T, E=6)
    D = upload(L)
    D["w13"], D["w2"] = with_kc(D["w13"], codes), with_kc(D["w2"], codes)
    print(f"forward by chunk T={T} codes={codes}", flush=True)
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"forward scales by chunk T{T}")


@CODES
def test_forward_scales_by_chunk_full_size(codes):
    """The gpt-oss-20b NVFP4 layer at T = 4096 (the benchmark's headline
    configuration); sampled tokens against the oracle, bitwise repeatable."""
    L = S.make_config(2, 4096)
    D = upload(L)
    D["w13"], D["w2"] = with_kc(D["w13"], codes), with_kc(D["w2"], codes)
    print(f"forward by chunk full size codes={codes}", flush=True)
    out = gpu_forward(L, D)
    out2 = gpu_forward(L, D)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    ids, _ = O.route(L)
    toks = block_covering_tokens(ids, L.E, M.moe_forward_block_m(4096, L.top_k, L.E),
                                 extra=(0, 1, 7, 63, 511, 2047, 4095))
    got = host_bf16(out)
    assert np.isfinite(got).all()
    assert_rows_close(got[toks], O.forward_tokens(L, toks), what="forward scales by chunk full size")


# ------------------------------------------------------------ MXFP4 by chunk --
# MXFP4 on the streaming kernel: scales by 128-deep chunk (moe_mxfp4_scales_by_chunk)
# and, optionally, the codes by 128-deep chunk that the MX kernels read too.

def with_kc_mx(Dw, codes=False):
    return dataclasses.replace(Dw, scales_kc=M.moe_mxfp4_scales_by_chunk(Dw),
                               qweight_kc=M.moe_mxfp4_codes_by_chunk(Dw) if codes else None)


@pytest.mark.parametrize("E,N,K", [(3, 384, 320), (2, 2880, 2880), (5, 16, 352), (2, 48, 96)])
def test_mxfp4_scales_by_chunk_bitexact(E, N, K):
    w = S.make_weights("mxfp4", E=E, N=N, K=K, bias=False, seed=N + K + 5)
    Dw = M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales, None, None, None)
    got = M.moe_mxfp4_scales_by_chunk(Dw).cpu().numpy()
    kc = (K + 127) // 128
    padded = np.zeros((E, N, kc * 4), np.uint8)
    padded[:, :, :K // 32] = w.scales
    np.testing.assert_array_equal(got, padded.reshape(E, N, kc, 4).transpose(0, 2, 1, 3))


def _small_mx(act="swigluoai", E=4, k=2, H=320, I=192, T=300, seed=53, **kw):
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    return S.make_layer(E=E, top_k=k, H=H, I=I, fmt="mxfp4", act=act, route=route, T=T, seed=seed,
                        router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw)


@CODES
@pytest.mark.parametrize("act", ["none", "swigluoai", "relu2"])
@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("H", [320, 352, 2880])
def test_mxfp4_gemm1_by_chunk(act, B, H, codes):
    """K = 352: a 64-deep chunk ends the 128-deep layout's last, partial chunk,
    then the 32-wide tail (checkpoint layout)."""
    L = _small_mx("relu2" if act == "relu2" else "swigluoai", H=H, T=300 if H < 2880 else 150,
                  x_std=12.0)
    D = upload(L)
    w13 = with_kc_mx(D["w13"], codes)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    print(f"mxfp4 gemm1 by chunk act={act} B={B} H={H} codes={codes}", flush=True)
    n_out = L.w13.N // 2 if act == "swigluoai" else L.w13.N
    out = M.moe_w4a16_gemm1(D["x"], L.top_k, w13, act, L.alpha, L.beta, L.limit, t(si), t(ei),
                            t(np.array([npp], np.int32)), B, out=poisoned((L.T * L.top_k, n_out)))
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, act, L.alpha, L.beta, L.limit, si, ei, npp, B)
    assert_rows_close(host_bf16(out), ref, rows=cov, what=f"mxfp4 gemm1 by chunk {act} B{B} H{H}")


@CODES
@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("I", [192, 224, 2880])
def test_mxfp4_gemm2_by_chunk(B, I, codes):
    L = _small_mx(I=I, T=300 if I < 2880 else 150)
    D = upload(L)
    w2 = with_kc_mx(D["w2"], codes)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    n = L.T * L.top_k
    a_bits = S.f32_to_bf16_bits(np.random.default_rng(I + B).standard_normal((n, I)).astype(np.float32))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    print(f"mxfp4 gemm2 by chunk B={B} I={I} codes={codes}", flush=True)
    y = M.moe_w4a16_gemm2(t(a_bits.view(np.int16)).view(torch.bfloat16), w2,
                          t(w.reshape(-1).astype(np.float32)), True, t(si), t(ei),
                          t(np.array([npp], np.int32)), B, out=poisoned((n, L.H)))
    ref, cov = O.gemm2(a_bits, n, L.w2, w.reshape(-1), True, si, ei, npp, B)
    assert_rows_close(host_bf16(y), ref, rows=cov, what=f"mxfp4 gemm2 by chunk B{B} I{I}")


@pytest.mark.parametrize("T", [13, 600])
def test_mxfp4_forward_by_chunk(T):
    """T = 13: 16-row blocks (the decode kernels read the checkpoint copy);
    T = 600: 128-row blocks on the streaming kernel reading the chunked copies."""
    L = _small_mx(T=T, E=6)
    D = upload(L)
    D["w13"], D["w2"] = with_kc_mx(D["w13"], True), with_kc_mx(D["w2"], True)
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"mxfp4 forward by chunk T{T}")


def test_mxfp4_forward_by_chunk_full_size():
    """The gpt-oss-120b MXFP4 layer at T = 8192 with the chunked copies, as
    bench.py loads it: tokens covering every aligned block against the oracle."""
    L = S.make_config(4, 8192)
    D = upload(L)
    D["w13"], D["w2"] = with_kc_mx(D["w13"], True), with_kc_mx(D["w2"], True)
    print("mxfp4 forward by chunk full size", flush=True)
    out = gpu_forward(L, D)
    ids, _ = O.route(L)
    toks = block_covering_tokens(ids, L.E, M.moe_forward_block_m(8192, L.top_k, L.E),
                                 extra=(0, 1, 7, 63, 511, 4095, 8191))
    got = host_bf16(out)
    assert np.isfinite(got).all()
    err = assert_rows_close(got[toks], O.forward_tokens(L, toks), what="mxfp4 by chunk full size")
    print(f"mxfp4 by chunk full size: max rel err {err:.3e} over {len(toks)} tokens", flush=True)


# ------------------------------------------------------------ uneven loads --
# 128-row blocks on the streamed-scale kernels with experts of 1 to 5 blocks.

@pytest.mark.parametrize("fmt,act", [("nvfp4", "swigluoai"), ("nvfp4", "relu2"),
                                     ("mxfp4", "swigluoai"), ("gptq", "swigluoai"),
                                     ("gptq", "relu2")])
@pytest.mark.parametrize("H,I", [(320, 192), (2880, 384)])
def test_forward_uneven_loads(fmt, act, H, I):
    """Uneven loads over 5 experts (from one 128-row block to five, odd and
    even counts); every output row against the oracle."""
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    L = S.make_layer(E=5, top_k=2, H=H, I=I, fmt=fmt, act=act, route=route, T=700, seed=61,
                     skew_std=0.8, router_bias_std=0.1 if route == "sigmoid_bias" else 0.0)
    ids, _ = O.route(L)
    blocks = -(-np.bincount(ids.reshape(-1), minlength=L.E) // 128)
    assert M.moe_forward_block_m(L.T, L.top_k, L.E) == 128
    assert (blocks % 2 == 1).any() and (blocks >= 4).any(), blocks
    D = upload(L)
    if fmt == "nvfp4":
        D["w13"], D["w2"] = with_kc(D["w13"], True), with_kc(D["w2"], True)
    elif fmt == "mxfp4":
        D["w13"], D["w2"] = with_kc_mx(D["w13"], True), with_kc_mx(D["w2"], True)
    print(f"uneven loads {fmt} {act} H={H} I={I} blocks={blocks.tolist()}", flush=True)
    out = gpu_forward(L, D)
    got = host_bf16(out)
    assert np.isfinite(got).all()
    assert_rows_close(got, O.forward(L)["out"], what=f"uneven loads {fmt} {act} H{H} I{I}")

"""GPU parity of the MXFP8-activation layer (MXFP4 weights x MXFP8 activations).

The quantiser's bytes are compared bit-exact with the oracle's (every
decision is taken on exact bf16 inputs on both sides).  The MX-scaled GEMMs
get the oracle's own MXFP8 operands and are compared with the oracle's
GEMMs in the same mode; the layer (both the MX-scaled kernels at 64/128-row
blocks and the dequantised path at smaller blocks) with the oracle's layer.
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
from gpu_util import assert_rows_close, dev_bf16, host_bf16, upload  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _bf16_rows(rows, K, seed):
    """bf16 bits with per-block magnitudes from 2^-30 to 2^30, zero blocks,
    negative zeros and exact ties of the e4m3 grid."""
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.integers(-30, 30, size=(rows, K // 32, 1)))
    v = (rng.standard_normal((rows, K // 32, 32)) * mag).reshape(rows, K)
    v[0, :32] = 0.0
    v[0, 32:64] = -0.0
    if K >= 128:
        v[1, 64:96] = np.array([448, 460, 464, 1.0625, 1.1875, -3.25] + [0.5] * 26) * 2.0 ** 3
    return S.f32_to_bf16_bits(v.astype(np.float32))


def _pad(codes, scales, K):
    rows = codes.shape[0]
    c = np.zeros((rows, M.mxfp8_lda(K)), np.uint8)
    s = np.zeros((rows, M.mxfp8_lds(K)), np.uint8)
    c[:, :K] = codes
    s[:, :K // 32] = scales
    return c, s


@pytest.mark.parametrize("rows,K", [(7, 32), (33, 96), (300, 2880), (65, 2688), (16, 352)])
def test_quantize_bitexact(rows, K):
    bits = _bf16_rows(rows, K, rows + K)
    print(f"mxfp8 quantize rows={rows} K={K}", flush=True)
    x = dev_bf16(bits)
    c, s, d = M.moe_mxfp8_quantize(x, codes=True, dequant=True)
    torch.cuda.synchronize()
    ref_c, ref_s = F.quantize_mxfp8(F.bf16_to_f64(bits))
    rc, rs = _pad(ref_c, ref_s, K)
    np.testing.assert_array_equal(c.cpu().numpy(), rc)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    deq = F.dequantize_mxfp8(ref_c, ref_s)
    np.testing.assert_array_equal(host_bf16(d), F.bf16_round(deq))


def test_quantize_nonfinite_block_and_in_place_dequant():
    bits = _bf16_rows(4, 128, 3)
    bits[2, 40] = 0x7F80          # +inf in block 1 of row 2
    bits[3, 100] = 0x7FC0         # NaN in block 3 of row 3
    x = dev_bf16(bits)
    c, s, _ = M.moe_mxfp8_quantize(x, codes=True)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    c = c.cpu().numpy()
    assert s[2, 1] == 255 and s[3, 3] == 255 and np.all(c[2, 32:64] == 0x7F)
    ref_c, ref_s = F.quantize_mxfp8(F.bf16_to_f64(bits))
    np.testing.assert_array_equal(c[:, :128], ref_c)
    np.testing.assert_array_equal(s[:, :4], ref_s)
    # dequantised values written over the input
    y = dev_bf16(_bf16_rows(9, 2880, 8))
    ref = F.bf16_round(F.mxfp8_round_trip(host_bf16(y)))
    M._binding._check(M.lib().moe_mxfp8_quantize(y.data_ptr(), 9, 2880, None, None, y.data_ptr(),
                                                   M._binding._stream()), "in place")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bf16(y), ref)


def _layer(act="swigluoai", E=4, k=2, H=320, I=192, T=300, seed=41, **kw):
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    return dataclasses.replace(
        S.make_layer(E=E, top_k=k, H=H, I=I, fmt="mxfp4", act=act, route=route, T=T, seed=seed,
                     router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw),
        act_fmt="mxfp8")


def _up_mx(codes, scales, K):
    c, s = _pad(codes, scales, K)
    return torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()


@pytest.mark.parametrize("act", ["none", "swigluoai", "relu2"])
@pytest.mark.parametrize("H", [320, 352, 2880])
@pytest.mark.parametrize("B", [64, 128])
def test_mx_gemm1_parity(act, H, B):
    L = _layer("relu2" if act == "relu2" else "swigluoai", H=H, T=300 if H < 2880 else 150)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    xc, xs = F.quantize_mxfp8(F.bf16_to_f64(L.x))
    dc, ds = _up_mx(xc, xs, H)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    print(f"mx gemm1 act={act} H={H} B={B}", flush=True)
    out = M.moe_mx_gemm1(dc, ds, L.top_k, H, D["w13"], act, L.alpha, L.beta, L.limit, t(si), t(ei),
                         t(np.array([npp], np.int32)), B)
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, act, L.alpha, L.beta, L.limit, si, ei, npp, B,
                       act_fmt="mxfp8")
    assert_rows_close(host_bf16(out), ref, rows=cov, what=f"mx gemm1 {act} H{H} B{B}")


@pytest.mark.parametrize("I", [192, 224, 2880])
@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("mul", [True, False])
def test_mx_gemm2_parity(I, B, mul):
    L = _layer(I=I, T=300 if I < 2880 else 150)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    n = L.T * L.top_k
    rng = np.random.default_rng(I + B)
    a = F.bf16_round(rng.standard_normal((n, I)) * np.exp2(rng.integers(-4, 4, (n, 1))))
    ac, as_ = F.quantize_mxfp8(a)
    dc, ds = _up_mx(ac, as_, I)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    print(f"mx gemm2 I={I} B={B} mul={mul}", flush=True)
    y = M.moe_mx_gemm2(dc, ds, I, D["w2"], t(w.reshape(-1).astype(np.float32)), mul, t(si), t(ei),
                       t(np.array([npp], np.int32)), B)
    ref, cov = O.gemm2(a, n, L.w2, w.reshape(-1), mul, si, ei, npp, B, act_fmt="mxfp8")
    assert_rows_close(host_bf16(y), ref, rows=cov, what=f"mx gemm2 I{I} B{B}")


def gpu_forward_mx(L, D):
    return M.moe_forward_mxfp8(D["x"], D["logits"], L.top_k, L.I, D["w13"], D["w2"], act=L.act,
                               route=L.route, expert_bias=D["expert_bias"],
                               renormalize=L.renormalize, alpha=L.alpha, beta=L.beta,
                               limit=L.limit, mul_topk_weights=L.mul_topk_weights)


def gpu_act(L, D):
    """GEMM1's bf16 output as moe_forward_mxfp8 computes it, from the same
    public steps: MX-scaled GEMM1 at 64/128-row blocks, else the bf16 GEMM1 on
    the dequantised MXFP8 input."""
    T = D["x"].shape[0]
    bm = M.moe_forward_block_m(T, L.top_k, L.E)
    ids, tw, si, ei, npp = M.moe_route_align(D["logits"], L.top_k, bm, L.route, D["expert_bias"],
                                             L.renormalize)
    if bm >= 64:
        c, s, _ = M.moe_mxfp8_quantize(D["x"])
        act = M.moe_mx_gemm1(c, s, L.top_k, L.H, D["w13"], L.act, L.alpha, L.beta, L.limit,
                             si, ei, npp, bm)
    else:
        _, _, xd = M.moe_mxfp8_quantize(D["x"], codes=False, dequant=True)
        act = M.moe_w4a16_gemm1(xd, L.top_k, D["w13"], L.act, L.alpha, L.beta, L.limit,
                                si, ei, npp, bm)
    torch.cuda.synchronize()
    return act, bm


def _check_layer(L, D, got, act_bits, tokens=None):
    """Stage 1: GEMM1's output against the oracle's.  Stage 2: the layer output
    against the oracle's GEMM2 + sum applied to the GPU's own GEMM1 output --
    GEMM2's MXFP8 input is an integer decision taken from bf16 values, which
    the GPU rounds from fp32 sums and the oracle from fp64 sums; a value on a
    rounding edge can land one e4m3 step (or one shared exponent) apart, so
    the stage is compared from identical bf16 values, as the pieces are."""
    ids, w = O.route(L)
    k = L.top_k
    toks = list(range(L.T)) if tokens is None else list(tokens)
    xq = F.mxfp8_round_trip(F.bf16_to_f64(L.x[toks]))
    a_gpu = F.bf16_to_f64(act_bits)
    ref_act = np.zeros((len(toks) * k, a_gpu.shape[1]))
    ref_out = np.zeros((len(toks), L.H))
    rows = []
    for e in sorted(set(int(v) for v in ids[toks].reshape(-1)) & set(range(L.E))):
        W13 = F.decode_expert(L.w13, e)
        W2 = F.decode_expert(L.w2, e)
        for i, t in enumerate(toks):
            for j in range(k):
                if ids[t, j] != e:
                    continue
                h = W13 @ xq[i] + O._bias_f64(L.w13, e)
                ref_act[i * k + j] = O.activation(h, L.act, L.alpha, L.beta, L.limit)
                rows.append(i * k + j)
                y = W2 @ F.mxfp8_round_trip(a_gpu[t * k + j]) + O._bias_f64(L.w2, e)
                if L.mul_topk_weights:
                    y = y * float(w[t, j])
                ref_out[i] += y
    sel = np.array([t * k + j for t in toks for j in range(k)])
    assert_rows_close(a_gpu[sel][rows], ref_act[rows], what="GEMM1 output")
    assert_rows_close(got[toks], ref_out, what="layer output given the GPU's GEMM1 output")


@pytest.mark.parametrize("act", ["swigluoai", "relu2"])
@pytest.mark.parametrize("T", [1, 13, 200, 600])
def test_forward_mxfp8(act, T):
    """T = 1, 13: 16/32-row blocks (dequantised MXFP8 values on the bf16
    kernels); T = 200, 600: 64/128-row blocks (MX-scaled kernels)."""
    L = _layer(act, T=T, E=6, k=2 if act == "swigluoai" else 3)
    D = upload(L)
    print(f"forward mxfp8 {act} T={T} block_m={M.moe_forward_block_m(T, L.top_k, L.E)}", flush=True)
    out = gpu_forward_mx(L, D)
    out2 = gpu_forward_mx(L, D)
    act_gpu, _ = gpu_act(L, D)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    bits = act_gpu.view(torch.int16).cpu().numpy().view(np.uint16)
    _check_layer(L, D, host_bf16(out), bits)
    # the whole layer against the oracle alone: close, within the effect of
    # the few intermediate codes that can differ
    rel = O.row_rel_err(host_bf16(out), O.forward(L)["out"])
    assert np.median(rel) < 5e-3 and rel.max() < 3e-2


@pytest.mark.parametrize("T", [1024, 8192])
def test_forward_mxfp8_full_size(T):
    """The gpt-oss-120b MXFP4 layer (E=128, top-4, 2880/2880, skewed routing)
    with MXFP8 activations; sampled tokens against the oracle."""
    L = dataclasses.replace(S.make_config(4, T), act_fmt="mxfp8")
    D = upload(L)
    print(f"forward mxfp8 full size T={T} block_m={M.moe_forward_block_m(T, 4, 128)}", flush=True)
    out = gpu_forward_mx(L, D)
    act_gpu, _ = gpu_act(L, D)
    toks = [t for t in (0, 1, 7, 63, 511, 1023, 4095, 8191) if t < T]
    got = host_bf16(out)
    assert np.isfinite(got).all()
    bits = act_gpu.view(torch.int16).cpu().numpy().view(np.uint16)
    _check_layer(L, D, got, bits, toks)


def test_mx_gemm1_longest_k_that_fits():
    """K = 4608: both scale tiles just fit the kernel's LDS and the A scale
    tile takes 18 of its 24 DMA instructions."""
    L = _layer("swigluoai", E=3, H=4608, I=64, T=100)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, 64)
    xc, xs = F.quantize_mxfp8(F.bf16_to_f64(L.x))
    dc, ds = _up_mx(xc, xs, L.H)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = M.moe_mx_gemm1(dc, ds, L.top_k, L.H, D["w13"], "swigluoai", L.alpha, L.beta, L.limit,
                         t(si), t(ei), t(np.array([npp], np.int32)), 64)
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, "swigluoai", L.alpha, L.beta, L.limit, si, ei,
                       npp, 64, act_fmt="mxfp8")
    assert_rows_close(host_bf16(out), ref, rows=cov, what="mx gemm1 K=4608")


def test_forward_mxfp8_empty_batch():
    L = _layer(T=4)
    D = upload(L)
    out = M.moe_forward_mxfp8(D["x"][:0], D["logits"][:0], L.top_k, L.I, D["w13"], D["w2"])
    assert out.shape == (0, L.H)


# ------------------------------------------------- MXFP4 codes by K chunk --

@pytest.mark.parametrize("E,N,K", [(3, 384, 320), (2, 2880, 2880), (5, 16, 352), (2, 48, 128)])
def test_mxfp4_codes_by_chunk_bitexact(E, N, K):
    w = S.make_weights("mxfp4", E=E, N=N, K=K, bias=False, seed=N + K + 3)
    Dw = M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales, None, None, None)
    got = M.moe_mxfp4_codes_by_chunk(Dw).cpu().numpy()
    kc = (K + 127) // 128
    padded = np.zeros((E, N, kc * 64), np.uint8)
    padded[:, :, : K // 2] = w.qweight
    np.testing.assert_array_equal(got, padded.reshape(E, N, kc, 64).transpose(0, 2, 1, 3))


@pytest.mark.parametrize("K", [320, 352, 2880])
@pytest.mark.parametrize("B", [64, 128])
def test_mx_gemms_codes_by_chunk(K, B):
    """The MX kernels reading the chunked copy: bit for bit what they give on
    the checkpoint codes (only the copy source differs), and the oracle's
    values; K % 128 = 64 and 96 cover a partial last chunk."""
    L = _layer(H=K, I=K, T=300 if K < 2880 else 150)
    D = upload(L)
    w13c = dataclasses.replace(D["w13"], qweight_kc=M.moe_mxfp4_codes_by_chunk(D["w13"]))
    w2c = dataclasses.replace(D["w2"], qweight_kc=M.moe_mxfp4_codes_by_chunk(D["w2"]))
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xc, xs = F.quantize_mxfp8(F.bf16_to_f64(L.x))
    dc, ds = _up_mx(xc, xs, K)
    print(f"mx gemms codes by chunk K={K} B={B}", flush=True)
    args = (L.act, L.alpha, L.beta, L.limit, t(si), t(ei), t(np.array([npp], np.int32)), B)
    o1 = M.moe_mx_gemm1(dc, ds, L.top_k, K, D["w13"], *args)
    o1c = M.moe_mx_gemm1(dc, ds, L.top_k, K, w13c, *args)
    assert torch.equal(o1.view(torch.int16), o1c.view(torch.int16))
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, L.act, L.alpha, L.beta, L.limit, si, ei, npp, B,
                       act_fmt="mxfp8")
    assert_rows_close(host_bf16(o1c), ref, rows=cov, what=f"mx gemm1 codes by chunk K{K} B{B}")
    n = L.T * L.top_k
    rng = np.random.default_rng(K + B)
    a = F.bf16_round(rng.standard_normal((n, K)))
    ac, as_ = F.quantize_mxfp8(a)
    dc2, ds2 = _up_mx(ac, as_, K)
    args2 = (t(w.reshape(-1).astype(np.float32)), True, t(si), t(ei), t(np.array([npp], np.int32)), B)
    y = M.moe_mx_gemm2(dc2, ds2, K, D["w2"], *args2)
    yc = M.moe_mx_gemm2(dc2, ds2, K, w2c, *args2)
    assert torch.equal(y.view(torch.int16), yc.view(torch.int16))
    ref2, cov2 = O.gemm2(a, n, L.w2, w.reshape(-1), True, si, ei, npp, B, act_fmt="mxfp8")
    assert_rows_close(host_bf16(yc), ref2, rows=cov2, what=f"mx gemm2 codes by chunk K{K} B{B}")


def test_forward_mxfp8_codes_by_chunk_full_size():
    """gpt-oss-120b shape, T = 8192: the chunked copies change no output bit."""
    L = dataclasses.replace(S.make_config(4, 8192), act_fmt="mxfp8")
    D = upload(L)
    out = gpu_forward_mx(L, D)
    D["w13"] = dataclasses.replace(D["w13"], qweight_kc=M.moe_mxfp4_codes_by_chunk(D["w13"]))
    D["w2"] = dataclasses.replace(D["w2"], qweight_kc=M.moe_mxfp4_codes_by_chunk(D["w2"]))
    print("forward mxfp8 codes by chunk full size", flush=True)
    outc = gpu_forward_mx(L, D)
    assert torch.equal(out.view(torch.int16), outc.view(torch.int16))

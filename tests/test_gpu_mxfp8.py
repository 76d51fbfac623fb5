"""GPU parity of the MXFP8-activation layer (MXFP4 weights x MXFP8 activations).

The quantiser's bytes are compared bit-exact with the oracle's (every
decision is taken on exact bf16 inputs on both sides).  The MX-scaled GEMMs
get the oracle's own MXFP8 operands and are compared with the oracle's
GEMMs in the same mode.  The layer (both the MX-scaled kernels at 64/128-row
blocks and the dequantised path at smaller blocks) is held to a validity
rule on its intermediate MXFP8 operand (GPU and oracle take that integer
decision from differently rounded sums; see _check_mxfp8_act) and then to
the tolerance.
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
from gpu_util import (assert_rows_close, block_covering_tokens, dev_bf16, host_bf16,  # noqa: E402
                      poisoned, upload)


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
    # scales by K chunk: the streamed-scale kernel, the same bits
    outs = M.moe_mx_gemm1(dc, ds, L.top_k, H, D["w13"].chunked_only(), act, L.alpha, L.beta,
                          L.limit, t(si), t(ei), t(np.array([npp], np.int32)), B)
    assert torch.equal(out.view(torch.int16), outs.view(torch.int16)), "streamed scales"


def _live_tile_ids(counts, seed):
    """top_k = 1 routing with the given slot count per expert, tokens shuffled."""
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    return np.random.default_rng(seed).permutation(ids).reshape(-1, 1)


@pytest.mark.parametrize("act", ["swigluoai", "relu2"])
def test_mx_gemm1_live_row_tiles(act):
    """128-row blocks holding 1, 33, 65, 97 and 129 slots: one to four live 32-row
    tiles (the kernel multiplies only those) and a full block followed by a
    one-row block; every row (the output starts as NaN bytes) matches the
    oracle, and the streamed-scale kernel gives the same bits."""
    counts = [1, 33, 65, 97, 129]
    T = sum(counts)
    L = _layer(act, E=len(counts), k=1, H=352, T=T, seed=7)
    D = upload(L)
    ids = _live_tile_ids(counts, 5)
    si, ei, npp = O.align(ids, L.E, 128)
    xc, xs = F.quantize_mxfp8(F.bf16_to_f64(L.x))
    dc, ds = _up_mx(xc, xs, L.H)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = (L.alpha, L.beta, L.limit, t(si), t(ei), t(np.array([npp], np.int32)), 128)
    n_out = L.w13.N // 2 if act == "swigluoai" else L.w13.N
    out = M.moe_mx_gemm1(dc, ds, 1, L.H, D["w13"], act, *args, out=poisoned((T, n_out)))
    ref, cov = O.gemm1(L.x, T, 1, L.w13, act, L.alpha, L.beta, L.limit, si, ei, npp, 128,
                       act_fmt="mxfp8")
    assert cov.all()
    assert_rows_close(host_bf16(out), ref, what=f"mx gemm1 live tiles {act}")
    outs = M.moe_mx_gemm1(dc, ds, 1, L.H, D["w13"].chunked_only(), act, *args)
    assert torch.equal(out.view(torch.int16), outs.view(torch.int16)), "streamed scales"


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
    ys = M.moe_mx_gemm2(dc, ds, I, D["w2"].chunked_only(), t(w.reshape(-1).astype(np.float32)),
                        mul, t(si), t(ei), t(np.array([npp], np.int32)), B)
    assert torch.equal(y.view(torch.int16), ys.view(torch.int16)), "streamed scales"


def gpu_forward_mx(L, D):
    """moe_forward_mxfp8 on a workspace and output poisoned with 0xFF bytes."""
    T = D["x"].shape[0]
    ws = poisoned((max(M.moe_forward_mxfp8_workspace_bytes(T, L.E, L.top_k, L.H, L.I), 1),),
                  torch.uint8)
    return M.moe_forward_mxfp8(D["x"], D["logits"], L.top_k, L.I, D["w13"], D["w2"], act=L.act,
                               route=L.route, expert_bias=D["expert_bias"],
                               renormalize=L.renormalize, alpha=L.alpha, beta=L.beta,
                               limit=L.limit, mul_topk_weights=L.mul_topk_weights, workspace=ws,
                               out=poisoned((T, L.H)))


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


U32 = 2.0 ** -24   # unit roundoff of fp32


def _act_bound(h, habs, K, act, alpha, beta, limit):
    """Elementwise bound on |GPU activation before its bf16 rounding - exact
    activation of h|.  The GEMM sums K exact products in fp32: within
    K*u*sum|terms| of the exact sum, plus 2u|h| for the scale multiply and
    the bias add.  The activation propagates that error with its derivative
    (first order, doubled for margin; the clamps only lower the derivative)
    and adds the error of the hardware exp2 and reciprocal in the sigmoid
    (a few ulp: 8u of the value)."""
    dh = K * U32 * habs + 2 * U32 * np.abs(h)
    if act == "relu2":
        r = np.maximum(h, 0.0)
        return 2.0 * (2 * r * dh + dh * dh) + 8 * U32 * r * r
    g = np.minimum(h[..., 0::2], limit)
    u = np.clip(h[..., 1::2], -limit, limit)
    sg = 1.0 / (1.0 + np.exp(-alpha * g))
    da_dg = np.abs(sg * (1.0 + alpha * g * (1.0 - sg)) * (u + beta))
    da_du = np.abs(g * sg)
    a = g * sg * (u + beta)
    return 2.0 * (da_dg * dh[..., 0::2] + da_du * dh[..., 1::2]) + 8 * U32 * np.abs(a)


def _ulp_bf16(v):
    """Spacing of bf16 values at |v| (8 significant bits; subnormal step 2^-133)."""
    m = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(m)) - 7)


def _check_mxfp8_act(a64, bound, a_gpu, gpu_codes, gpu_scales):
    """The GPU's bf16 activation and its MXFP8 encoding are results the exact
    activation a64 admits:
      1. |a_gpu - a64| <= bound + half a bf16 step, element by element;
      2. (checked by the caller) the GPU quantiser's bytes of a_gpu are the
         oracle's quantize_mxfp8 of a_gpu, bit for bit;
      3. every block exponent the GPU chose is one that the block maximum
         reaches inside the interval, and every element code is the e4m3 code,
         at that exponent, of a bf16 value inside [a64 - bound, a64 + bound]
         (the encode is monotone in the value), so each code that differs from
         the oracle's encoding of its own bf16 rounding of a64 sits on a
         rounding edge the oracle exhibits.
    Returns the number of codes and exponents that differ from the oracle's."""
    half = 0.5 * _ulp_bf16(np.abs(a64) + bound)
    err = np.abs(a_gpu - a64)
    assert (err <= bound + half * (1 + 2.0 ** -8)).all(), (
        f"GPU activation outside the fp32 bound: worst excess "
        f"{np.max(err - bound - half):.3e} at {np.unravel_index(np.argmax(err - bound - half), err.shape)}")
    lo = F.bf16_round(a64 - bound)
    hi = F.bf16_round(a64 + bound)
    rows, K = a64.shape
    blk = lambda v: np.abs(v).reshape(rows, K // 32, 32)
    amax_lo = np.max(np.minimum(blk(lo), blk(hi)) * (np.sign(lo) == np.sign(hi)).reshape(rows, K // 32, 32),
                     axis=-1)
    amax_hi = np.max(np.maximum(blk(lo), blk(hi)), axis=-1)
    _, e_lo = F.quantize_mxfp8(np.repeat(amax_lo, 32, axis=-1))
    _, e_hi = F.quantize_mxfp8(np.repeat(amax_hi, 32, axis=-1))
    e_lo, e_hi = e_lo.astype(np.int64), e_hi.astype(np.int64)
    # an all-zero block (amax 0) takes byte 0: below every nonzero exponent
    gs = gpu_scales.astype(np.int64)
    ok_e = ((e_lo <= gs) | (amax_lo == 0)) & (gs <= e_hi)
    assert ok_e.all(), f"block exponent out of the admissible range at {np.argwhere(~ok_e)[:4]}"
    scale = np.repeat(F.E8M0_TABLE[gpu_scales], 32, axis=-1)
    v_lo = F.E4M3FN_TABLE[F.e4m3_encode(lo / scale)]
    v_hi = F.E4M3FN_TABLE[F.e4m3_encode(hi / scale)]
    v_gpu = F.E4M3FN_TABLE[gpu_codes]
    ok_c = (v_lo <= v_gpu) & (v_gpu <= v_hi)
    assert ok_c.all(), f"MXFP8 code not admissible at {np.argwhere(~ok_c)[:4]}"
    oc, os_ = F.quantize_mxfp8(F.bf16_round(a64))
    return int((oc != gpu_codes).sum()), int((os_ != gpu_scales).sum())


def _check_layer(L, D, got, act_gpu, tokens=None):
    """The MXFP8 layer against the oracle.

    GEMM2's MXFP8 input is an integer decision taken from bf16 values that
    the GPU rounds from fp32 sums and the oracle from exact sums: on a
    rounding edge both results are correct, so the check is a validity rule
    (see _check_mxfp8_act) on the GPU's activation and its encoding, and the
    layer output is then held to the tolerance against the oracle's GEMM2 and
    sum applied to the validated MXFP8 operand."""
    ids, w = O.route(L)
    k = L.top_k
    toks = list(range(L.T)) if tokens is None else list(tokens)
    xq = F.mxfp8_round_trip(F.bf16_to_f64(L.x[toks]))
    a_bits = act_gpu.view(torch.int16).cpu().numpy().view(np.uint16)
    a_all = F.bf16_to_f64(a_bits)
    sel = np.array([t * k + j for t in toks for j in range(k)])
    # 2. the GPU quantiser's bytes of the GPU's activation (the kernel the layer runs)
    gc, gsc, _ = M.moe_mxfp8_quantize(act_gpu[torch.from_numpy(sel).cuda()].contiguous())
    gc = gc.cpu().numpy()[:, :L.I]
    gsc = gsc.cpu().numpy()[:, :L.I // 32]
    rc, rs = F.quantize_mxfp8(a_all[sel])
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_array_equal(gsc, rs)
    a64 = np.zeros((len(sel), L.I))
    bound = np.zeros((len(sel), L.I))
    ref_out = np.zeros((len(toks), L.H))
    for e in sorted(set(int(v) for v in ids[toks].reshape(-1)) & set(range(L.E))):
        W13 = F.decode_expert(L.w13, e)
        W2 = F.decode_expert(L.w2, e)
        b13 = O._bias_f64(L.w13, e)
        for i, t in enumerate(toks):
            for j in range(k):
                if ids[t, j] != e:
                    continue
                r = i * k + j
                h = W13 @ xq[i] + b13
                habs = np.abs(W13) @ np.abs(xq[i]) + np.abs(b13)
                a64[r] = O.activation(h, L.act, L.alpha, L.beta, L.limit)
                bound[r] = _act_bound(h, habs, L.H, L.act, L.alpha, L.beta, L.limit)
                y = W2 @ F.dequantize_mxfp8(gc[r], gsc[r]) + O._bias_f64(L.w2, e)
                if L.mul_topk_weights:
                    y = y * float(w[t, j])
                ref_out[i] += y
    # 1 and 3
    n_codes, n_exp = _check_mxfp8_act(a64, bound, a_all[sel], gc, gsc)
    # 4. the layer output
    err = assert_rows_close(got[toks], ref_out, what="layer output")
    whole = O.row_rel_err(got[toks], O.forward_tokens(L, toks)).max()
    print(f"mxfp8 layer: {n_codes} codes and {n_exp} block exponents of {gc.size} on a rounding "
          f"edge; layer max rel err {err:.3e} (against the oracle's own encoding: {whole:.3e})",
          flush=True)


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
    got = host_bf16(out)
    assert np.isfinite(got).all()
    _check_layer(L, D, got, act_gpu)


def _steps_mx_small(L, D, policy="auto"):
    """moe_forward_mxfp8's result at 16/32-row blocks from the public steps:
    route and sort, the quantiser's dequantised MXFP8 values of x, the bf16
    GEMM1, the same for its output, the bf16 GEMM2, and each token's k-row sum
    in float32 (j ascending, one bf16 rounding) on the host."""
    T, k = D["x"].shape[0], L.top_k
    bm = M.moe_forward_block_m(T, k, L.E)
    assert bm <= 32
    _, tw, si, ei, npp = M.moe_route_align(D["logits"], k, bm, L.route, D["expert_bias"],
                                           L.renormalize)
    _, _, xd = M.moe_mxfp8_quantize(D["x"], codes=False, dequant=True)
    act = M.moe_w4a16_gemm1(xd, k, D["w13"], L.act, L.alpha, L.beta, L.limit, si, ei, npp, bm,
                            kernel=policy)
    _, _, ad = M.moe_mxfp8_quantize(act, codes=False, dequant=True)
    y = M.moe_w4a16_gemm2(ad, D["w2"], tw.reshape(-1), L.mul_topk_weights, si, ei, npp, bm,
                          kernel=policy)
    yh = y.float().cpu().numpy().reshape(T, k, L.H)
    acc = np.zeros((T, L.H), np.float32)
    for j in range(k):
        acc += yh[:, j]
    return torch.from_numpy(acc).to(torch.bfloat16)


@pytest.mark.parametrize("case", ["E6_T1", "E6_T13_nan", "cfg4_T1", "cfg4_T16"])
def test_forward_mxfp8_small_blocks_equal_steps(case):
    """At 16/32-row blocks the layer equals its public steps -- the quantiser's
    dequantised MXFP8 values of x and of the activation around the bf16 GEMMs
    -- bit for bit.  cfg4_T16 runs the 128-column kernel (enough column
    tiles), the others the split-K one; a NaN in one 32-block of x makes that
    token's rows NaN on both sides."""
    if case.startswith("cfg4"):
        T = int(case.split("_T")[1])
        L = dataclasses.replace(S.make_config(4, T), act_fmt="mxfp8")
    else:
        T = 13 if "T13" in case else 1
        L = _layer("relu2" if "nan" in case else "swigluoai", T=T, E=6, k=3 if "nan" in case else 2)
    D = upload(L)
    if "nan" in case:
        xb = D["x"].clone()
        xb[2, 40] = float("nan")
        D = dict(D, x=xb)
    print(f"mxfp8 small blocks {case} block_m={M.moe_forward_block_m(T, L.top_k, L.E)}", flush=True)
    out = gpu_forward_mx(L, D)
    ref = _steps_mx_small(L, D)
    # bit for bit, except the payload of a NaN (the steps' sum runs on the host)
    a, b = out.cpu().float().numpy(), ref.float().numpy()
    nan = np.isnan(a)
    assert (nan == np.isnan(b)).all(), "NaN positions differ"
    diff = out.cpu().view(torch.int16).numpy()[~nan] != ref.view(torch.int16).numpy()[~nan]
    assert not diff.any(), f"{int(diff.sum())} of {int((~nan).sum())} values differ"
    got = host_bf16(out)
    if "nan" in case:
        assert np.isnan(got[2]).all() and np.isfinite(np.delete(got, 2, axis=0)).all()
    else:
        assert np.isfinite(got).all()


@pytest.mark.parametrize("T", [1024, 8192])
def test_forward_mxfp8_full_size(T):
    """The gpt-oss-120b MXFP4 layer (E=128, top-4, 2880/2880, skewed routing)
    with MXFP8 activations, on tokens covering every aligned block."""
    L = dataclasses.replace(S.make_config(4, T), act_fmt="mxfp8")
    D = upload(L)
    bm = M.moe_forward_block_m(T, 4, 128)
    print(f"forward mxfp8 full size T={T} block_m={bm}", flush=True)
    out = gpu_forward_mx(L, D)
    act_gpu, _ = gpu_act(L, D)
    ids, _ = O.route(L)
    toks = block_covering_tokens(ids, L.E, bm, extra=(0, 1, 7, 63, 511, 1023, 4095, 8191))
    got = host_bf16(out)
    assert np.isfinite(got).all()
    _check_layer(L, D, got, act_gpu, toks)


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


def test_mx_gemm1_long_k_streamed_scales():
    """K = 6144: beyond the resident scale tiles (the checkpoint family is
    refused); the chunked-only family streams them with the chunks."""
    L = _layer("swigluoai", E=3, H=6144, I=64, T=100)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, 128)
    xc, xs = F.quantize_mxfp8(F.bf16_to_f64(L.x))
    dc, ds = _up_mx(xc, xs, L.H)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = ("swigluoai", L.alpha, L.beta, L.limit, t(si), t(ei), t(np.array([npp], np.int32)), 128)
    with pytest.raises(RuntimeError):
        M.moe_mx_gemm1(dc, ds, L.top_k, L.H, D["w13"], *args)
    out = M.moe_mx_gemm1(dc, ds, L.top_k, L.H, D["w13"].chunked_only(), *args)
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, "swigluoai", L.alpha, L.beta, L.limit, si, ei,
                       npp, 128, act_fmt="mxfp8")
    assert_rows_close(host_bf16(out), ref, rows=cov, what="mx gemm1 K=6144 streamed scales")


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
    values; K % 128 = 64 and 96 cover a partial last chunk.  The chunked-only
    family (scales by K chunk too) runs the kernel whose scale tiles stream
    with the chunks: bit for bit the same again."""
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
    o1s = M.moe_mx_gemm1(dc, ds, L.top_k, K, D["w13"].chunked_only(), *args)
    assert torch.equal(o1.view(torch.int16), o1s.view(torch.int16)), "streamed scales"
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
    ys = M.moe_mx_gemm2(dc2, ds2, K, D["w2"].chunked_only(), *args2)
    assert torch.equal(y.view(torch.int16), ys.view(torch.int16)), "streamed scales"
    ref2, cov2 = O.gemm2(a, n, L.w2, w.reshape(-1), True, si, ei, npp, B, act_fmt="mxfp8")
    assert_rows_close(host_bf16(yc), ref2, rows=cov2, what=f"mx gemm2 codes by chunk K{K} B{B}")


def test_forward_mxfp8_codes_by_chunk_full_size():
    """gpt-oss-120b shape, T = 8192: the chunked copies (codes, then codes and
    scales) change no output bit."""
    L = dataclasses.replace(S.make_config(4, 8192), act_fmt="mxfp8")
    D = upload(L)
    out = gpu_forward_mx(L, D)
    D["w13"] = dataclasses.replace(D["w13"], qweight_kc=M.moe_mxfp4_codes_by_chunk(D["w13"]))
    D["w2"] = dataclasses.replace(D["w2"], qweight_kc=M.moe_mxfp4_codes_by_chunk(D["w2"]))
    print("forward mxfp8 codes by chunk full size", flush=True)
    outc = gpu_forward_mx(L, D)
    assert torch.equal(out.view(torch.int16), outc.view(torch.int16))
    # chunked-only families: the MX kernels stream both scale tiles
    D["w13"], D["w2"] = D["w13"].chunked_only(), D["w2"].chunked_only()
    outs = gpu_forward_mx(L, D)
    assert torch.equal(out.view(torch.int16), outs.view(torch.int16)), "streamed scales"

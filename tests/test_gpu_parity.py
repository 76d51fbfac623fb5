"""GPU parity: every step of the HIP path against the float64 oracle, through the C-ABI.

Integer results (routing ids, sorted ids, expert ids, padded length) must be
bit-exact; float results within 5e-3 per-row relative error with no NaN/Inf.
Shapes here are small enough for the oracle to finish in seconds but span
several tiles and ragged K / N tails (K = 320 = 2*128 + 64).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import moe as O

pytestmark = pytest.mark.gpu

M = pytest.importorskip("bit_weight_expert_amd")
from gpu_util import (TOL, assert_rows_close, assert_untouched, dev_bf16, gpu_forward,  # noqa: E402
                      host_bf16, poisoned, upload, upload_weights)

# The kernel for 16/32-row blocks ("auto" takes the split-K kernel at these
# small sizes, "wide" forces the 128-column kernel).
POLICIES = ["auto", "wide"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()  # the HIP library must load; no fallback exists


# ------------------------------------------------------------------ routing --

@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_route_bitexact_full_size(cfg):
    logits, bias = S.make_router_inputs(cfg)
    c = S.CONFIGS[cfg]
    ids_ref, w_ref = O.route(logits, c["top_k"], c["route"], bias, True)
    ids, w = M.moe_route(torch.from_numpy(logits).cuda(), c["top_k"], c["route"],
                         None if bias is None else torch.from_numpy(bias).cuda(), True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=2e-6, atol=0)


@pytest.mark.parametrize("E,k,kind,renorm", [(8, 2, "softmax", False), (130, 5, "sigmoid_bias", True),
                                             (1024, 16, "softmax", True), (3, 3, "softmax", True),
                                             (1, 1, "softmax", True), (2, 2, "sigmoid_bias", False),
                                             (64, 8, "softmax", True), (65, 7, "sigmoid_bias", True),
                                             (127, 16, "softmax", False), (128, 1, "softmax", True)])
def test_route_shapes(E, k, kind, renorm):
    """Ties, one and two scores per lane (E = 64 / 65 / 127 / 128), k up to 16,
    the single-expert layer; row 1 ties experts 5 and 69 (the two entries of
    one lane) at the top, which the lower id must win."""
    rng = np.random.default_rng(E)
    T = 37
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = 0.25                       # all tied: lowest ids win
    if E > 64 + 5:
        logits[1, 5] = logits[1, 64 + 5] = 9.0  # one lane's two entries tied at the top
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if kind == "sigmoid_bias" else None
    if bias is not None and E > 64 + 5:
        bias[5] = bias[64 + 5] = 0.0
    ids_ref, w_ref = O.route(logits, k, kind, bias, renorm)
    ids, w = M.moe_route(torch.from_numpy(logits).cuda(), k, kind,
                         None if bias is None else torch.from_numpy(bias).cuda(), renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=2e-6)


@pytest.mark.parametrize("T,E,k,kind,B", [(1, 128, 8, "sigmoid_bias", 16), (8, 32, 4, "softmax", 16), (16, 32, 4, "softmax", 16),
                                           (64, 128, 6, "softmax", 32), (256, 64, 16, "sigmoid_bias", 64),
                                           (37, 130, 5, "softmax", 16), (5, 1024, 16, "softmax", 16),
                                           (300, 128, 4, "softmax", 64), (1, 3, 3, "softmax", 16)])
def test_route_align_fused(T, E, k, kind, B):
    """route + align in one call equals the oracle's route then align (one
    launch up to 16 tokens, the two kernels above)."""
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, : min(E, 40)] = 0.5             # ties among the top scores
    if T > 2 and kind == "sigmoid_bias":
        logits[2, 1] = np.nan                 # a NaN score is never selected
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if kind == "sigmoid_bias" else None
    ids_ref, w_ref = O.route(logits, k, kind, bias, True)
    ref = O.align(ids_ref, E, B)
    got = M.moe_route_align(torch.from_numpy(logits).cuda(), k, B, kind,
                            None if bias is None else torch.from_numpy(bias).cuda(), True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[0].cpu().numpy(), ids_ref)
    np.testing.assert_allclose(got[1].cpu().numpy(), w_ref, rtol=2e-6)
    np.testing.assert_array_equal(got[2].cpu().numpy(), ref[0])
    np.testing.assert_array_equal(got[3].cpu().numpy(), ref[1])
    assert int(got[4].item()) == int(ref[2])


# -------------------------------------------------------------------- align --

@pytest.mark.parametrize("T,k,E,B", [(1, 4, 32, 16), (13, 2, 8, 16), (64, 4, 32, 64), (511, 6, 128, 32),
                                      (4096, 4, 32, 128), (8192, 4, 128, 64), (3, 3, 1024, 16),
                                      (3001, 7, 1000, 32), (2000, 1, 1, 16), (700, 8, 2, 64)])
def test_align_bitexact(T, k, E, B):
    """Ragged per-wave runs (3001 x 7 slots), a single expert, two experts."""
    rng = np.random.default_rng(T + E + B)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 3:
        ids[2, 0] = E + 7          # not routed
        ids[3, k - 1] = -2
    ref = O.align(ids, E, B)
    got = M.moe_align(torch.from_numpy(ids).cuda(), E, B)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[0].cpu().numpy(), ref[0])
    np.testing.assert_array_equal(got[1].cpu().numpy(), ref[1])
    assert int(got[2].item()) == int(ref[2])


@pytest.mark.parametrize("T,k,E,B", [(1, 4, 32, 16), (13, 2, 8, 16), (511, 6, 128, 32),
                                      (4096, 4, 32, 128), (8192, 4, 128, 64), (3, 3, 1024, 16),
                                      (3001, 7, 1000, 32), (2000, 1, 1, 16), (700, 8, 2, 64),
                                      (16383, 4, 64, 128)])
def test_align_large_bitexact(T, k, E, B):
    """The 16-workgroup sort: the same outputs as the oracle (and so as the
    single workgroup), ragged ranges and runs included; counts start dirty."""
    rng = np.random.default_rng(T + E + B + 1)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 3:
        ids[2, 0] = E + 7
        ids[3, k - 1] = -2
    ref = O.align(ids, E, B)
    counts = torch.full((16 * E,), 12345, dtype=torch.int32, device="cuda")
    got = M.moe_align_large(torch.from_numpy(ids).cuda(), E, B, counts=counts)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[0].cpu().numpy(), ref[0])
    np.testing.assert_array_equal(got[1].cpu().numpy(), ref[1])
    assert int(got[2].item()) == int(ref[2])


def test_align_skewed_routing_full_size():
    logits, _ = S.make_router_inputs(4)          # E=128, T=8192, per-expert offsets
    ids_ref, _ = O.route(logits, 4, "softmax", None, True)
    for B in (16, 64, 128):
        ref = O.align(ids_ref, 128, B)
        for sort in (M.moe_align, M.moe_align_large):
            got = sort(torch.from_numpy(ids_ref).cuda(), 128, B)
            np.testing.assert_array_equal(got[0].cpu().numpy(), ref[0])
            np.testing.assert_array_equal(got[1].cpu().numpy(), ref[1])
            assert int(got[2].item()) == int(ref[2])


# -------------------------------------------------------------------- GEMMs --
# Every GEMM output starts as 0xFF bytes (bf16 NaN): covered rows must come
# back finite and within tolerance, rows no block covers must stay untouched.

def _small(fmt, act="swigluoai", E=4, k=2, H=320, I=192, T=13, seed=21, **kw):
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    return S.make_layer(E=E, top_k=k, H=H, I=I, fmt=fmt, act=act, route=route, T=T, seed=seed,
                        router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw)


def _dev_align(si, ei, npp):
    return tuple(torch.from_numpy(a).cuda() for a in (si, ei, np.array([npp], np.int32)))


def _gemm1(D, L, act, dsi, dei, dnpp, B, kernel, n_rows, topk_w=None, w13=None):
    n_out = L.w13.N // 2 if act == "swigluoai" else L.w13.N
    out = poisoned((n_rows, n_out))
    return M.moe_w4a16_gemm1(D["x"], L.top_k, D["w13"] if w13 is None else w13, act, L.alpha,
                             L.beta, L.limit, dsi, dei, dnpp, B, out=out, topk_w=topk_w,
                             kernel=kernel)


def _gemm2(a, w2, tw, mul, dsi, dei, dnpp, B, kernel, top_k=1):
    out = poisoned((a.shape[0] * top_k, w2.N))
    return M.moe_w4a16_gemm2(a, w2, tw, mul, dsi, dei, dnpp, B, out=out, top_k=top_k,
                             kernel=kernel)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "gptq"])
@pytest.mark.parametrize("act", ["none", "swigluoai", "relu2"])
@pytest.mark.parametrize("B,policy", [(16, "auto"), (16, "wide"), (32, "wide"), (64, "auto")])
def test_gemm1_parity(fmt, act, B, policy):
    L = _small(fmt, "relu2" if act == "relu2" else "swigluoai", x_std=12.0)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, act, L.alpha, L.beta, L.limit, si, ei, npp, B)
    out = _gemm1(D, L, act, *_dev_align(si, ei, npp), B, policy, L.T * L.top_k)
    assert_rows_close(host_bf16(out), ref, rows=cov, what=f"gemm1 {fmt} {act} B{B} {policy}")
    assert_untouched(out, cov, "gemm1")


@pytest.mark.parametrize("fmt,act", [("nvfp4", "swigluoai"), ("mxfp4", "relu2"), ("gptq", "swigluoai")])
@pytest.mark.parametrize("B", [64, 128])
def test_gemm1_live_row_tiles(fmt, act, B):
    """Streaming-kernel blocks with one to four live 32-row tiles (slot counts
    1, 33, 65, 97 and 129 per expert, top_k = 1, tokens shuffled): the kernel
    multiplies only the live tiles; every row (the output starts as NaN bytes)
    matches the oracle."""
    counts = [1, 33, 65, 97, 129]
    T = sum(counts)
    L = _small(fmt, act, E=len(counts), k=1, T=T, seed=8)
    D = upload(L)
    ids = np.random.default_rng(6).permutation(
        np.repeat(np.arange(len(counts), dtype=np.int32), counts)).reshape(-1, 1)
    si, ei, npp = O.align(ids, L.E, B)
    ref, cov = O.gemm1(L.x, T, 1, L.w13, act, L.alpha, L.beta, L.limit, si, ei, npp, B)
    assert cov.all()
    out = _gemm1(D, L, act, *_dev_align(si, ei, npp), B, "auto", T)
    assert_rows_close(host_bf16(out), ref, what=f"gemm1 live tiles {fmt} {act} B{B}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "gptq"])
@pytest.mark.parametrize("B,policy", [(16, "auto"), (32, "auto"), (16, "wide"), (32, "wide"),
                                      (128, "auto")])
def test_gemm2_parity_and_mul_flag(fmt, B, policy):
    L = _small(fmt, E=5, k=3, T=11)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    n = L.T * L.top_k
    rng = np.random.default_rng(3)
    a_bits = S.f32_to_bf16_bits(rng.standard_normal((n, L.I)).astype(np.float32))
    tw = w.reshape(-1).astype(np.float32)
    ref1, cov = O.gemm2(a_bits, n, L.w2, tw, True, si, ei, npp, B)
    da = _dev_align(si, ei, npp)
    a = dev_bf16(a_bits)
    dtw = torch.from_numpy(tw).cuda()
    y1 = _gemm2(a, D["w2"], dtw, True, *da, B, policy)
    y0 = _gemm2(a, D["w2"], dtw, False, *da, B, policy)
    assert_rows_close(host_bf16(y1), ref1, rows=cov, what=f"gemm2 {fmt} B{B} {policy}")
    assert_untouched(y1, cov, "gemm2")
    # forensic check: the multiplier each row received is its own weight
    g1, g0 = host_bf16(y1), host_bf16(y0)
    ratio = (g1[cov] * g0[cov]).sum(1) / np.maximum((g0[cov] * g0[cov]).sum(1), 1e-30)
    np.testing.assert_allclose(ratio, tw[cov], rtol=5e-3)


@pytest.mark.parametrize("fmt", ["nvfp4", "gptq"])
@pytest.mark.parametrize("B,policy", [(16, "splitk"), (16, "wide"), (64, "auto")])
def test_gemm2_top_k_shares_rows(fmt, B, policy):
    """GEMM2 with top_k > 1: row f reads A row f // top_k (as GEMM1 does) and
    takes its own slot's routing weight; equal to the top_k = 1 view on the
    repeated rows."""
    L = _small(fmt, E=5, k=3, T=17)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    rng = np.random.default_rng(13)
    a_bits = S.f32_to_bf16_bits(rng.standard_normal((L.T, L.I)).astype(np.float32))
    tw = w.reshape(-1).astype(np.float32)
    n = L.T * L.top_k
    ref, cov = O.gemm2(np.repeat(a_bits, L.top_k, axis=0), n, L.w2, tw, True, si, ei, npp, B)
    y = _gemm2(dev_bf16(a_bits), D["w2"], torch.from_numpy(tw).cuda(), True,
               *_dev_align(si, ei, npp), B, policy, top_k=L.top_k)
    assert_rows_close(host_bf16(y), ref, rows=cov, what=f"gemm2 top_k={L.top_k} {fmt} B{B} {policy}")
    assert_untouched(y, cov, "gemm2 top_k")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_gemm2_power_of_two_weights_bitwise(fmt):
    """With routing weights 2^-m the in-kernel multiply equals the external one bit for bit."""
    L = _small(fmt, E=4, k=4, T=9)
    D = upload(L)
    ids, _ = O.route(L)
    si, ei, npp = O.align(ids, L.E, 16)
    n = L.T * L.top_k
    tw = np.ldexp(np.ones(n, np.float32), -(np.arange(n) % 5)).astype(np.float32)
    rng = np.random.default_rng(4)
    a = dev_bf16(S.f32_to_bf16_bits(rng.standard_normal((n, L.I)).astype(np.float32)))
    da = _dev_align(si, ei, npp)
    dtw = torch.from_numpy(tw).cuda()
    y1 = _gemm2(a, D["w2"], dtw, True, *da, 16, "auto")
    y0 = _gemm2(a, D["w2"], dtw, False, *da, 16, "auto")
    ext = (y0.float() * dtw[:, None]).to(torch.bfloat16)
    assert torch.equal(y1.view(torch.int16), ext.view(torch.int16))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "gptq"])
@pytest.mark.parametrize("B,policy", [(16, "auto"), (16, "wide"), (64, "auto")])
def test_gemm1_weight_on_input(fmt, B, policy):
    """GEMM1 with each input row scaled by its slot's routing weight, in all three kernels."""
    L = _small(fmt, "swigluoai", x_std=12.0)
    D = upload(L)
    ids, _ = O.route(L)
    tw = np.random.default_rng(7).uniform(0.05, 1.5, size=L.T * L.top_k).astype(np.float32)
    si, ei, npp = O.align(ids, L.E, B)
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, "swigluoai", L.alpha, L.beta, L.limit, si, ei,
                       npp, B, topk_w_flat=tw)
    out = _gemm1(D, L, "swigluoai", *_dev_align(si, ei, npp), B, policy, L.T * L.top_k,
                 topk_w=torch.from_numpy(tw).cuda())
    assert_rows_close(host_bf16(out), ref, rows=cov, what=f"gemm1 weight on input {fmt} B{B} {policy}")


# ------------------------------------------------------------------ forward --

@pytest.mark.parametrize("fmt,act", [("nvfp4", "swigluoai"), ("mxfp4", "swigluoai"),
                                     ("gptq", "swigluoai"), ("nvfp4", "relu2")])
@pytest.mark.parametrize("T", [1, 13, 100])
@pytest.mark.parametrize("policy", POLICIES)
def test_forward_parity_small(fmt, act, T, policy):
    L = _small(fmt, act, E=6, k=3, T=T, skew_std=1.0)
    D = upload(L)
    out = gpu_forward(L, D, kernel=policy)
    ref = O.forward(L)["out"]
    assert_rows_close(host_bf16(out), ref, what=f"forward {fmt} {act} T{T}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("T", [1, 13, 100])
def test_forward_weight_on_input(fmt, T):
    """top_k = 1 with the routing weight on GEMM1's input (weights not renormalised)."""
    L = dataclasses.replace(_small(fmt, E=6, k=1, T=T, renormalize=False), weight_on_input=True)
    D = upload(L)
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"forward weight on input {fmt} T{T}")


def test_forward_config1_full():
    L = S.make_config(1)
    D = upload(L)
    out = gpu_forward(L, D)
    ref = O.forward(L)["out"]
    err = assert_rows_close(host_bf16(out), ref, what=S.CONFIGS[1]["name"])
    print(f"config 1: max per-row rel err {err:.3e} over all {L.T} tokens", flush=True)


def test_forward_deterministic_bitwise():
    L = _small("nvfp4", E=6, k=3, T=100)
    D = upload(L)
    a = gpu_forward(L, D)
    b = gpu_forward(L, D)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("fmt,act,E,k", [("nvfp4", "swigluoai", 6, 3), ("gptq", "swigluoai", 32, 4),
                                         ("mxfp4", "relu2", 9, 1), ("nvfp4", "relu2", 40, 6)])
@pytest.mark.parametrize("T", [1, 2, 16, 64, 65])
@pytest.mark.parametrize("policy", POLICIES)
def test_forward_sum_equals_steps_bitwise(fmt, act, E, k, T, policy):
    """moe_forward equals its steps through the public entry points -- route and
    sort, GEMM1, GEMM2 -- followed by each token's k-row sum in float32, j
    ascending, rounded once to bf16, bit for bit, on 16-, 32- and 64-row blocks
    and both decode kernels.  Two more calls on one workspace (poisoned once,
    then left with the previous call's contents) give the same bits."""
    L = _small(fmt, act, E=E, k=k, T=T, skew_std=1.0)
    D = upload(L)
    out = gpu_forward(L, D, kernel=policy)
    B = M.moe_forward_block_m(T, k, E)
    _, tw, si, ei, npp = M.moe_route_align(D["logits"], k, B, L.route, D["expert_bias"],
                                           L.renormalize)
    act_rows = _gemm1(D, L, act, si, ei, npp, B, policy, T * k)
    y = _gemm2(act_rows, D["w2"], tw.reshape(-1), L.mul_topk_weights, si, ei, npp, B, policy)
    yh = y.float().cpu().numpy().reshape(T, k, L.H)
    acc = np.zeros((T, L.H), np.float32)
    for j in range(k):
        acc += yh[:, j]
    ref = torch.from_numpy(acc).to(torch.bfloat16)
    assert torch.equal(out.cpu().view(torch.int16), ref.view(torch.int16)), (
        f"forward {fmt} {act} E{E} k{k} T{T} B{B} {policy}: differs from its steps")
    ws = poisoned((M.moe_forward_workspace_bytes(T, E, k, L.H, L.I),), torch.uint8)
    kw = dict(act=L.act, route=L.route, expert_bias=D["expert_bias"], renormalize=L.renormalize,
              alpha=L.alpha, beta=L.beta, limit=L.limit, mul_topk_weights=L.mul_topk_weights,
              workspace=ws, kernel=policy)
    for _ in range(2):
        again = M.moe_forward(D["x"], D["logits"], k, L.I, D["w13"], D["w2"], out=poisoned((T, L.H)),
                              **kw)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("fmt", ["nvfp4", "gptq"])
@pytest.mark.parametrize("T", [5, 300, 600])
def test_forward_max_experts_and_top_k(fmt, T):
    """The largest routing the ABI takes, E = 1024 and top_k = 16, through the
    whole layer: one launch for route and sort (T = 5), the routing kernel and
    the one-workgroup sort with mixed-tiling planning (T = 300), the
    16-workgroup sort into 64-row streaming tiles (T = 600)."""
    L = _small(fmt, E=1024, k=16, H=128, I=64, T=T, seed=31)
    D = upload(L)
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"forward E1024 k16 {fmt} T{T}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("E,k,H,I,T", [(1, 1, 128, 64, 1), (1, 1, 128, 64, 200),
                                       (4, 2, 32, 32, 3), (4, 2, 32, 32, 150)])
def test_forward_degenerate_shapes(fmt, E, k, H, I, T):
    """One expert taking every token (the dense layer), and hidden = intermediate =
    32: both GEMMs are a single 32-deep K tail with no full chunk, over one or
    two 16/32-column weight fragments; decode and streaming kernels."""
    L = _small(fmt, E=E, k=k, H=H, I=I, T=T, seed=33)
    D = upload(L)
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"forward E{E} k{k} H{H} I{I} T{T}")


@pytest.mark.parametrize("fmt", ["nvfp4", "gptq"])
@pytest.mark.parametrize("T", [1, 13, 300])
def test_forward_without_routing_weights(fmt, T):
    """mul_topk_weights = False: the k rows are summed unweighted (16-row decode
    blocks and 64/128-row streaming tiles)."""
    L = _small(fmt, E=6, k=3, T=T, seed=35, mul_topk_weights=False)
    D = upload(L)
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"forward unweighted {fmt} T{T}")


def test_forward_t0_is_noop():
    L = _small("nvfp4", T=4)
    D = upload(L)
    x0 = D["x"][:0]
    out = M.moe_forward(x0, D["logits"][:0], L.top_k, L.I, D["w13"], D["w2"])
    assert out.shape == (0, L.H)


def test_forward_top_k_equals_e():
    L = _small("mxfp4", E=3, k=3, T=7)
    D = upload(L)
    out = gpu_forward(L, D)
    assert_rows_close(host_bf16(out), O.forward(L)["out"], what="top_k = E")


@pytest.mark.parametrize("K", [32, 96, 224, 256, 288, 480, 544, 4128])
@pytest.mark.parametrize("B,policy", [(16, "auto"), (32, "auto"), (64, "auto"), (128, "auto"),
                                      (16, "wide"), (32, "wide")])
def test_gemm2_k_tails(K, B, policy):
    """Every K tail decomposition (256-chunks + 128/64/32 pieces) in both kernels."""
    fmt = "mxfp4" if K % 64 else "nvfp4"
    L = _small(fmt, E=3, k=2, H=96, I=K, T=40)
    D = upload(L)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    n = L.T * L.top_k
    rng = np.random.default_rng(K)
    a_bits = S.f32_to_bf16_bits(rng.standard_normal((n, K)).astype(np.float32))
    tw = w.reshape(-1).astype(np.float32)
    ref, cov = O.gemm2(a_bits, n, L.w2, tw, True, si, ei, npp, B)
    y = _gemm2(dev_bf16(a_bits), D["w2"], torch.from_numpy(tw).cuda(), True,
               *_dev_align(si, ei, npp), B, policy)
    assert_rows_close(host_bf16(y), ref, rows=cov, what=f"gemm2 K={K} B{B} {policy}")
    assert_untouched(y, cov, "gemm2 K tail")


@pytest.mark.parametrize("fmt,K,N,group,B", [
    ("nvfp4", 12320, 96, None, 64),    # scales too long for LDS: split-K kernel on 32-row sub-blocks
    ("gptq", 2560, 128, 32, 128),      # GPTQ group 32: scales resident in LDS, K split over 8 waves
    ("gptq", 2560, 96, 128, 128),      # group 128: scale rows streamed, one per two chunks; ragged N
    ("gptq", 12288, 64, 128, 64),      # K too long for resident scales: streamed
    ("gptq", 256, 80, 64, 64),         # N % 32 != 0: split-K kernel on 32-row sub-blocks
    ("mxfp4", 2880, 320, None, 128),   # MXFP4 at the gpt-oss K, ragged last column tile
])
@pytest.mark.parametrize("policy", POLICIES)
def test_gemm2_tile_fallbacks(fmt, K, N, group, B, policy):
    """The prefill kernel's tile choices and fallbacks (scale tile size, zero-point alignment)."""
    E, k, T = 3, 2, 40
    w2 = S.make_weights(fmt, E=E, N=N, K=K, group=group, seed=K + N)
    rng = np.random.default_rng(K + N)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, size=T * k).astype(np.float32)
    si, ei, npp = O.align(ids, E, B)
    n = T * k
    a_bits = S.f32_to_bf16_bits(rng.standard_normal((n, K)).astype(np.float32))
    ref, cov = O.gemm2(a_bits, n, w2, tw, True, si, ei, npp, B)
    y = _gemm2(dev_bf16(a_bits), upload_weights(w2), torch.from_numpy(tw).cuda(), True,
               *_dev_align(si, ei, npp), B, policy)
    assert_rows_close(host_bf16(y), ref, rows=cov, what=f"gemm2 {fmt} K={K} N={N} B{B} {policy}")


@pytest.mark.parametrize("fmt,act", [("nvfp4", "swigluoai"), ("mxfp4", "swigluoai"),
                                     ("gptq", "swigluoai"), ("nvfp4", "relu2")])
@pytest.mark.parametrize("policy", ["auto", "splitk", "wide"])
def test_forward_mixed_tiling(fmt, act, policy):
    """Few slots per expert on average (16-row blocks: 8 per expert over 128
    experts) with a few experts holding hundreds: moe_forward sends those
    experts' full 128-row runs to the streaming kernel (a tile list built on
    the device) and the rest to the decode kernels; the whole output against
    the oracle, every row."""
    L = _small(fmt, act, E=128, k=2, T=512, skew_std=2.5, seed=77)
    ids, _ = O.route(L)
    cnt = np.bincount(ids.reshape(-1), minlength=L.E)
    bm = M.moe_forward_block_m(L.T, L.top_k, L.E)
    assert bm <= 32 and (cnt >= 128).sum() >= 2, (bm, np.sort(cnt)[-4:])
    D = upload(L)
    out = gpu_forward(L, D, kernel=policy)
    err = assert_rows_close(host_bf16(out), O.forward(L)["out"], what=f"mixed tiling {fmt} {act}")
    print(f"mixed tiling {fmt} {act} {policy}: {int((cnt // 128).sum())} tiles of 128 rows, "
          f"max rel err {err:.3e}", flush=True)


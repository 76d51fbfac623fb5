"""Pins for the oracle's routing, align, GEMMs, activation and sum (CPU only)."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import brute, formats as F, moe as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- routing --

def test_softmax_route_matches_torch_topk():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((50, 32)).astype(np.float32)
    ids, w = O.route_softmax(logits, 4, renormalize=False)
    tw, ti = torch.topk(torch.softmax(torch.from_numpy(logits).double(), -1), 4, dim=-1)
    np.testing.assert_array_equal(ids, ti.numpy())
    np.testing.assert_allclose(w, tw.numpy(), rtol=1e-12)
    ids_r, w_r = O.route_softmax(logits, 4, renormalize=True)
    np.testing.assert_array_equal(ids_r, ids)
    np.testing.assert_allclose(w_r, tw.numpy() / tw.numpy().sum(1, keepdims=True), rtol=1e-12)


def test_softmax_route_full_k_is_softmax():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((5, 8)).astype(np.float32)
    ids, w = O.route_softmax(logits, 8, renormalize=True)
    p = torch.softmax(torch.from_numpy(logits).double(), -1).numpy()
    np.testing.assert_allclose(np.take_along_axis(p, ids.astype(np.int64), 1), w, rtol=1e-12)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-12)


def test_route_ties_go_to_lower_id():
    logits = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]], dtype=np.float32)
    ids, w = O.route_softmax(logits, 2)
    assert ids.tolist() == [[1, 2]]
    np.testing.assert_allclose(w, [[0.5, 0.5]])


def test_sigmoid_bias_route_n_group_1_is_plain_topk():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((40, 128)).astype(np.float32)
    bias = (rng.standard_normal(128) * 0.1).astype(np.float32)
    ids, w = O.route_sigmoid_bias(logits, bias, 6)
    s = torch.sigmoid(torch.from_numpy(logits).double()).float()
    score = s + torch.from_numpy(bias)
    _, ti = torch.topk(score, 6, dim=-1)
    np.testing.assert_array_equal(ids, ti.numpy())
    sel = torch.gather(s.double(), 1, ti).numpy()
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-7)
    # the bias changes selection but never enters the weights
    ids0, _ = O.route_sigmoid_bias(logits, np.zeros(128, np.float32), 6)
    assert (ids0 != ids).any()


# ------------------------------------------------------------------- align --

def _brute_align(ids, E, B):
    flat = list(np.asarray(ids).reshape(-1))
    n = len(flat)
    order = sorted((int(e), f) for f, e in enumerate(flat) if 0 <= e < E)
    sorted_ids, expert_ids = [], []
    for e in range(E):
        fs = [f for (ee, f) in order if ee == e]
        if not fs:
            continue
        pad = -(-len(fs) // B) * B
        sorted_ids += fs + [n] * (pad - len(fs))
        expert_ids += [e] * (pad // B)
    return sorted_ids, expert_ids


@pytest.mark.parametrize("T,k,E,B", [(1, 4, 32, 16), (7, 2, 8, 16), (33, 4, 32, 64), (64, 6, 128, 32),
                                      (5, 3, 4, 128), (0, 4, 32, 16)])
def test_align_matches_brute_force_and_invariants(T, k, E, B):
    rng = np.random.default_rng(T * 100 + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 2:
        ids[1, 0] = E + 3          # out-of-range ids are not placed
        ids[2, 1] = -1
    sorted_ids, expert_ids, npp = O.align(ids, E, B)
    cap = O.align_capacity(T, k, E, B)
    assert sorted_ids.shape == (cap,) and expert_ids.shape == (cap // B,)
    bs, be = _brute_align(ids, E, B)
    assert int(npp) == len(bs)
    np.testing.assert_array_equal(sorted_ids[:npp], bs)
    np.testing.assert_array_equal(expert_ids[:npp // B], be)
    assert np.all(sorted_ids[npp:] == T * k) and np.all(expert_ids[npp // B:] == -1)
    # each valid slot exactly once; blocks expert-homogeneous
    valid = [f for f in range(T * k) if 0 <= ids.reshape(-1)[f] < E]
    placed = sorted_ids[:npp][sorted_ids[:npp] < T * k]
    assert sorted(placed.tolist()) == valid
    for b in range(npp // B):
        blk = sorted_ids[b * B:(b + 1) * B]
        assert np.all(ids.reshape(-1)[blk[blk < T * k]] == expert_ids[b])
    assert cap >= npp


# -------------------------------------------------------------- activation --

def test_swigluoai_special_cases():
    a, b, lim = 1.702, 1.0, 7.0
    # gate well above the limit: clamped to 7, sigmoid(alpha*7) ~ 1 - 6.6e-6
    g = np.array([50.0]); u = np.array([2.0])
    np.testing.assert_allclose(O.swigluoai(g, u, a, b, lim), 7.0 * 3.0 / (1 + np.exp(-a * 7)))
    # up clamped on both sides
    np.testing.assert_allclose(O.swigluoai(np.array([1.0]), np.array([-20.0]), a, b, lim),
                               1.0 / (1 + np.exp(-a)) * (-7.0 + 1.0))
    np.testing.assert_allclose(O.swigluoai(np.array([1.0]), np.array([20.0]), a, b, lim),
                               1.0 / (1 + np.exp(-a)) * (7.0 + 1.0))
    # gate is not clamped from below: a very negative gate gives ~0 (x*sigmoid(x) -> 0)
    assert abs(O.swigluoai(np.array([-30.0]), np.array([1.0]), a, b, lim)[0]) < 1e-20
    # gate 0 gives 0; up = -beta gives 0
    assert O.swigluoai(np.array([0.0]), np.array([3.0]), a, b, lim)[0] == 0.0
    assert O.swigluoai(np.array([2.0]), np.array([-1.0]), a, b, lim)[0] == 0.0
    # alpha -> large makes sigmoid a step: g*(u+1) for g>0
    np.testing.assert_allclose(O.swigluoai(np.array([0.5]), np.array([0.25]), 1e4, 1.0, lim), 0.5 * 1.25)


def test_relu2_special_cases():
    h = np.array([-3.0, -0.0, 0.0, 0.5, 2.0])
    np.testing.assert_array_equal(O.relu2(h), [0.0, 0.0, 0.0, 0.25, 4.0])


# --------------------------------------------------------- gemms + forward --

def _tiny_layer(fmt, act="swigluoai", route="softmax", E=3, k=2, H=64, I=64, T=3, seed=5, **kw):
    return S.make_layer(E=E, top_k=k, H=H, I=I, fmt=fmt, act=act, route=route, T=T, seed=seed,
                        router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw)


@pytest.mark.parametrize("fmt,act,route", [("nvfp4", "swigluoai", "softmax"),
                                           ("mxfp4", "swigluoai", "softmax"),
                                           ("gptq", "swigluoai", "softmax"),
                                           ("nvfp4", "relu2", "sigmoid_bias")])
def test_forward_matches_pure_python_brute_force(fmt, act, route):
    L = _tiny_layer(fmt, act, route, x_std=4.0)   # x_std=4 drives some gates past the clamp
    ref = O.forward(L, block_m=16)
    out = np.array(brute.forward(L, ref["topk_ids"], ref["topk_w"]))
    np.testing.assert_allclose(ref["out"], out, rtol=1e-10, atol=1e-12)


def test_forward_matches_brute_force_at_e8_n512_k512():
    """The page's small passing shape (E=8, N=K=512), with 2 routed slots."""
    L = S.make_layer(E=8, top_k=2, H=512, I=256, fmt="nvfp4", T=1, seed=11)
    ref = O.forward(L, block_m=16)
    out = np.array(brute.forward(L, ref["topk_ids"], ref["topk_w"]))
    np.testing.assert_allclose(ref["out"], out, rtol=1e-10, atol=1e-12)


def test_dense_special_case_e1_k1():
    """E = 1, top_k = 1: the layer is a dense two-layer MLP (np.matmul of the decoded weights)."""
    L = _tiny_layer("mxfp4", E=1, k=1, T=5, H=64, I=32)
    ref = O.forward(L)
    x = F.bf16_to_f64(L.x)
    W13 = F.decode_expert(L.w13, 0)
    W2 = F.decode_expert(L.w2, 0)
    h = np.matmul(x, W13.T) + F.bf16_to_f64(L.w13.bias[0])
    g, u = np.minimum(h[:, 0::2], 7.0), np.clip(h[:, 1::2], -7.0, 7.0)
    a = g / (1 + np.exp(-1.702 * g)) * (u + 1.0)
    y = np.matmul(a, W2.T) + F.bf16_to_f64(L.w2.bias[0])
    np.testing.assert_allclose(ref["out"], y, rtol=1e-12)    # routing weight is 1 with k = 1


def test_all_ones_codes_give_row_sums():
    """Codes all 1.0 with unit scales: gemm1 (act none) is the row sum of x plus bias."""
    L = _tiny_layer("nvfp4", H=64, I=32, T=4)
    L.w13.qweight[:] = 0x22                         # e2m1 1.0 in both nibbles
    L.w13.scales[:] = 0x38                          # e4m3 1.0
    L.w13.global_scale[:] = 1.0
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, 16)
    h, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, "none", 0, 0, 0, si, ei, npp, 16)
    x = F.bf16_to_f64(L.x)
    for f in range(L.T * L.top_k):
        e = ids.reshape(-1)[f]
        np.testing.assert_allclose(h[f], x[f // L.top_k].sum() + F.bf16_to_f64(L.w13.bias[e]), rtol=1e-13)


def test_mul_topk_weights_equals_external_multiply_and_forensic_ratio():
    """gemm2(mul=1) == gemm2(mul=0) * w per row; the recovered ratio is the row's own weight.

    The golden rows are the page's buggy observations: each applied ratio
    there differs from the row's own weight, and the same ratio check rejects it.
    """
    L = _tiny_layer("nvfp4", E=4, k=4, H=64, I=32, T=6)
    ids, w = O.route(L)
    si, ei, npp = O.align(ids, L.E, 16)
    rng = np.random.default_rng(0)
    a = S.f32_to_bf16_bits(rng.standard_normal((L.T * L.top_k, L.I)).astype(np.float32))
    y1, _ = O.gemm2(a, L.T * L.top_k, L.w2, w.reshape(-1), True, si, ei, npp, 16)
    y0, _ = O.gemm2(a, L.T * L.top_k, L.w2, w.reshape(-1), False, si, ei, npp, 16)
    np.testing.assert_allclose(y1, y0 * w.reshape(-1, 1), rtol=1e-14)
    ratio = (y1 * y0).sum(1) / (y0 * y0).sum(1)
    np.testing.assert_allclose(ratio, w.reshape(-1), rtol=1e-12)
    for row in open(os.path.join(GOLDEN, "mul_topk_forensic.txt")):
        row = row.split("#", 1)[0].split()
        if row:
            applied, own = float(row[1]), float(row[2])
            assert abs(applied / own - 1) > 0.01       # the check flags every buggy row


def test_weight_on_input_is_linear_in_the_weight_and_matches_brute_force():
    """Routing weight applied on GEMM1's input: with the activation left out,
    h_w - b = w (h - b) row by row; the whole layer (top_k = 1, weights not
    renormalised, so they differ from 1) equals the pure-Python brute force."""
    L = _tiny_layer("nvfp4", E=4, k=1, H=64, I=32, T=9, renormalize=False)
    ids, w = O.route(L)
    assert np.all(w < 1.0)
    si, ei, npp = O.align(ids, L.E, 16)
    h1, _ = O.gemm1(L.x, L.T, 1, L.w13, "none", 0, 0, 0, si, ei, npp, 16, topk_w_flat=w.reshape(-1))
    h0, _ = O.gemm1(L.x, L.T, 1, L.w13, "none", 0, 0, 0, si, ei, npp, 16)
    b = np.stack([F.bf16_to_f64(L.w13.bias[e]) for e in ids.reshape(-1)])
    np.testing.assert_allclose(h1 - b, (h0 - b) * w.reshape(-1, 1), rtol=1e-12, atol=1e-12)
    Lw = dataclasses.replace(L, weight_on_input=True)
    ref = O.forward(Lw, block_m=16)
    out = np.array(brute.forward(Lw, ref["topk_ids"], ref["topk_w"]))
    np.testing.assert_allclose(ref["out"], out, rtol=1e-10, atol=1e-12)
    assert not np.allclose(ref["out"], O.forward(L, block_m=16)["out"], rtol=1e-3)


def test_tail_scale_group_is_applied_at_true_k():
    """A distinctive last scale group (x4) at K = 2880, 2688, 1856 shows in the decoded tail."""
    for K in (2880, 2688, 1856):
        codes = np.full((2, K // 2), 0x22, dtype=np.uint8)
        sc = np.full((2, K // 16), 0x38, dtype=np.uint8)
        sc[:, -1] = 0x48                              # e4m3 4.0
        W = F.decode_nvfp4(codes, sc, 1.0, 16)
        assert np.all(W[:, :K - 16] == 1.0) and np.all(W[:, K - 16:] == 4.0)


def test_sum_skips_invalid_ids_and_keeps_j_order():
    y = np.arange(6 * 3, dtype=np.float64).reshape(6, 3)
    ids = np.array([[0, 1], [5, 1], [2, -1]])
    out = O.moe_sum(y, ids, E=4)
    np.testing.assert_array_equal(out[0], y[0] + y[1])
    np.testing.assert_array_equal(out[1], y[3])
    np.testing.assert_array_equal(out[2], y[4])


def test_forward_tokens_matches_forward():
    """The sampled-token path used at full sizes equals the whole-batch definition."""
    L = _tiny_layer("nvfp4", E=5, k=3, T=9, H=64, I=64)
    full = O.forward(L)["out"]
    rows = [0, 3, 8]
    np.testing.assert_allclose(O.forward_tokens(L, rows), full[rows], rtol=1e-12, atol=1e-15)


def test_act_order_layer_matches_brute_force():
    """GPTQ weights quantised in activation order (random channel order per
    expert, both families): the vectorised layer equals the pure-Python
    brute force, which reads each element's group from g_idx by hand."""
    L = _tiny_layer("gptq", E=3, k=2, H=128, I=64, T=4, group=32, act_order=True, x_std=2.0)
    assert L.w13.g_idx is not None and L.w2.g_idx is not None
    assert not np.array_equal(L.w13.g_idx[0], np.arange(128) // 32)
    ref = O.forward(L, block_m=16)
    out = np.array(brute.forward(L, ref["topk_ids"], ref["topk_w"]))
    np.testing.assert_allclose(ref["out"], out, rtol=1e-10, atol=1e-12)
    plain = dataclasses.replace(L, w13=dataclasses.replace(L.w13, g_idx=None))
    assert not np.allclose(O.forward(plain, block_m=16)["out"], ref["out"], rtol=1e-3)


def test_mxfp8_layer_matches_brute_force_and_differs_from_bf16():
    """MXFP8 activations: the vectorised layer equals the pure-Python brute
    force (its e4m3 rounding a search over all codes); the result is close to
    the bf16-activation layer (e4m3 keeps 4 significant bits) but not equal."""
    L = dataclasses.replace(_tiny_layer("mxfp4", E=3, k=2, H=64, I=64, T=4, x_std=2.0),
                            act_fmt="mxfp8")
    ref = O.forward(L, block_m=16)
    out = np.array(brute.forward(L, ref["topk_ids"], ref["topk_w"]))
    np.testing.assert_allclose(ref["out"], out, rtol=1e-10, atol=1e-12)
    b16 = O.forward(dataclasses.replace(L, act_fmt="bf16"), block_m=16)["out"]
    rel = O.row_rel_err(ref["out"], b16)
    assert np.all(rel < 0.1) and np.all(rel > 1e-4)
    tok = O.forward_tokens(L, [0, 3])
    np.testing.assert_allclose(tok, ref["out"][[0, 3]], rtol=1e-12, atol=1e-12)

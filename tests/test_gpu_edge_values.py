"""GPU parity at the edges of the number formats, through the C-ABI.

* Extreme scale bytes: NVFP4 e4m3 {0x00, 0x01, 0x7E, 0x7F}, MXFP4 e8m0 {0x00,
  0x01, 0xFE, 0xFF} and GPTQ fp16 NaN / zero scales, each the only non-zero
  contribution to some weight rows (the other groups of those rows hold zero
  codes), so the output of those rows is decided by the byte's decode.  NaN
  bytes must give NaN exactly where the oracle has NaN; every other output
  within the per-row tolerance (over its finite columns).
* NaN activations: a NaN in one token's input makes every output of that
  token NaN through the swigluoai and ReLU^2 clamps (a clamp must not turn
  NaN into the limit), and leaves every other token untouched.
* GPTQ group maps: the identity g_idx gives bit-identical results to none;
  any other map poisons the outputs of that expert only.
All outputs start as 0xFF bytes (NaN), every kernel family is exercised
(split-K and wide for 16-row blocks, the streaming kernel for 64-row blocks).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import moe as O

pytestmark = pytest.mark.gpu

M = pytest.importorskip("bit_weight_expert_amd")
from gpu_util import (TOL, assert_untouched, dev_bf16, gpu_forward, host_bf16,  # noqa: E402
                      poisoned, upload, upload_weights)

KERNELS = [(16, "splitk"), (16, "wide"), (64, "auto")]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _routing(E, k, T, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, size=T * k).astype(np.float32)
    return ids, tw


def _dev(*a):
    return tuple(torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in a)


def _compare_with_nan(got, ref, cov, what):
    """NaN exactly where the oracle has NaN; the finite part of each row within TOL."""
    got, ref = got[cov], ref[cov]
    nan_ref = np.isnan(ref)
    assert (np.isnan(got) == nan_ref).all(), f"{what}: NaN placement differs from the oracle"
    assert np.isfinite(got[~nan_ref]).all(), f"{what}: infinities"
    g = np.where(nan_ref, 0.0, got)
    r = np.where(nan_ref, 0.0, ref)
    rel = O.row_rel_err(g, r)
    assert rel.max() <= TOL, f"{what}: max per-row rel err {rel.max():.3e}"
    return float(rel.max()), int(nan_ref.any(axis=1).sum())


def _run_gemm2(w, a_bits, ids, tw, B, kernel, E):
    n = a_bits.shape[0]
    si, ei, npp = O.align(ids, E, B)
    ref, cov = O.gemm2(a_bits, n, w, tw, True, si, ei, npp, B)
    dsi, dei, dnpp = _dev(si, ei, np.array([npp], np.int32))
    Dw = upload_weights(w)
    y = poisoned((n, w.N))
    y = M.moe_w4a16_gemm2(dev_bf16(a_bits), Dw, torch.from_numpy(tw).cuda(), True, dsi, dei, dnpp,
                          B, out=y, kernel=kernel)
    assert_untouched(y, cov)
    return host_bf16(y), ref, cov


def _nvfp4_probe_family(E, N, K, seed):
    """NVFP4 weights whose row n has one live 16-group, g = n % (K/16), with
    scale byte PROBE[(n // G) % 4]; the other groups hold zero codes."""
    w = S.make_weights("nvfp4", E=E, N=N, K=K, bias=False, seed=seed)
    probes = np.array([0x00, 0x01, 0x7E, 0x7F], np.uint8)
    q = w.qweight.copy()
    sc = w.scales.copy()
    ng = K // 16
    for n in range(N):
        g = n % ng
        live = np.zeros(K // 2, bool)
        live[g * 8:(g + 1) * 8] = True
        q[:, n, ~live] = 0
        sc[:, n, :] = 0x38                       # 1.0: no effect on zero codes
        sc[:, n, g] = probes[(n // ng) % 4]
    return dataclasses.replace(w, qweight=q, scales=sc)


def _mxfp4_probe_family(E, N, K, seed):
    """MXFP4 weights (K = 128: four 32-groups) whose row n has one live group
    g = n % 4 with e8m0 byte {0xFE, 0x00, 0x01, 0xFF}[g]; the other groups
    hold zero codes under scale 2^0.  Codes of the 0xFE group are limited to
    |v| <= 1.5, so the dequantised weight (1.5 * 2^127) stays in bf16 range."""
    assert K == 128
    w = S.make_weights("mxfp4", E=E, N=N, K=K, bias=False, seed=seed)
    probes = np.array([0xFE, 0x00, 0x01, 0xFF], np.uint8)
    q = w.qweight.copy()
    sc = np.full_like(w.scales, 127)
    small = np.array([0, 1, 2, 3, 8, 9, 10, 11], np.uint8)      # e2m1 codes of 0, 0.5, 1, 1.5
    rng = np.random.default_rng(seed)
    for n in range(N):
        g = n % 4
        live = np.zeros(K // 2, bool)
        live[g * 16:(g + 1) * 16] = True
        q[:, n, ~live] = 0
        if g == 0:
            lo = rng.choice(small, size=(E, 16))
            hi = rng.choice(small, size=(E, 16))
            q[:, n, live] = (lo | (hi << 4)).astype(np.uint8)
        sc[:, n, g] = probes[g]
    return dataclasses.replace(w, qweight=q, scales=sc)


def _mx_inputs(n, K, seed):
    """Inputs whose 32-groups are scaled so every live product stays in fp32
    range: group 0 (the 2^127 weights) by 2^-100, groups 1 and 2 (2^-127 and
    2^-126) by 2^100, group 3 by 1."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, K)).astype(np.float32)
    a[:, 0:32] *= np.float32(2.0 ** -100)
    a[:, 32:96] *= np.float32(2.0 ** 100)
    return S.f32_to_bf16_bits(a)


@pytest.mark.parametrize("B,kernel", KERNELS)
def test_nvfp4_extreme_scale_bytes(B, kernel):
    E, k, T, N, K = 3, 2, 40, 128, 128
    w = _nvfp4_probe_family(E, N, K, seed=5)
    ids, tw = _routing(E, k, T, 6)
    a = S.f32_to_bf16_bits(np.random.default_rng(7).standard_normal((T * k, K)).astype(np.float32))
    got, ref, cov = _run_gemm2(w, a, ids, tw, B, kernel, E)
    err, nan_rows = _compare_with_nan(got, ref, cov, f"nvfp4 e4m3 edges B{B} {kernel}")
    assert nan_rows == cov.sum()        # every covered row has the 0x7F columns
    print(f"nvfp4 e4m3 edge bytes B{B} {kernel}: max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("B,kernel", KERNELS)
def test_mxfp4_extreme_scale_bytes(B, kernel):
    E, k, T, N, K = 3, 2, 40, 128, 128
    w = _mxfp4_probe_family(E, N, K, seed=8)
    ids, tw = _routing(E, k, T, 9)
    a = _mx_inputs(T * k, K, 10)
    got, ref, cov = _run_gemm2(w, a, ids, tw, B, kernel, E)
    # the oracle's 2^127 rows hold ~2^27, the 2^-127 rows ~2^-27: both finite
    assert np.isfinite(ref[cov][:, 0::4]).all() and np.isfinite(ref[cov][:, 1::4]).all()
    err, nan_rows = _compare_with_nan(got, ref, cov, f"mxfp4 e8m0 edges B{B} {kernel}")
    assert nan_rows == cov.sum()
    # each probe column class on its own (a wrong decode of one byte cannot
    # hide behind larger columns of the same row)
    for g in range(3):
        rel = O.row_rel_err(got[cov][:, g::4], ref[cov][:, g::4])
        assert rel.max() <= TOL, f"e8m0 byte class {g}: {rel.max():.3e}"
    print(f"mxfp4 e8m0 edge bytes B{B} {kernel}: max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("B,kernel", KERNELS)
def test_gptq_nan_and_zero_scales(B, kernel):
    E, k, T, N, K, G = 3, 2, 40, 128, 256, 64
    w = S.make_weights("gptq", E=E, N=N, K=K, group=G, bias=False, seed=11)
    sc = w.scales.copy()                         # fp16 [E][K/G][N]
    sc[1, 2, 5] = np.float16(np.nan)            # expert 1, group 2, column 5
    sc[:, 0, 7] = np.float16(0.0)               # a zero scale everywhere in group 0 of column 7
    w = dataclasses.replace(w, scales=sc)
    ids, tw = _routing(E, k, T, 12)
    a = S.f32_to_bf16_bits(np.random.default_rng(13).standard_normal((T * k, K)).astype(np.float32))
    got, ref, cov = _run_gemm2(w, a, ids, tw, B, kernel, E)
    err, nan_rows = _compare_with_nan(got, ref, cov, f"gptq NaN scale B{B} {kernel}")
    assert nan_rows > 0
    print(f"gptq NaN / zero scales B{B} {kernel}: max rel err {err:.2e}, {nan_rows} NaN rows", flush=True)


def _small(fmt, act, T=13, **kw):
    route = "sigmoid_bias" if act == "relu2" else "softmax"
    return S.make_layer(E=4, top_k=2, H=320, I=192, fmt=fmt, act=act, route=route, T=T, seed=23,
                        router_bias_std=0.1 if route == "sigmoid_bias" else 0.0, **kw)


@pytest.mark.parametrize("act", ["swigluoai", "relu2"])
@pytest.mark.parametrize("B,kernel", KERNELS)
def test_nan_activation_propagates(act, B, kernel):
    """GEMM1: a NaN in token 3's input gives NaN in all its slots' outputs."""
    L = _small("nvfp4", act, T=40)
    x = L.x.copy()
    x[3, 17] = 0x7FC0                            # bf16 NaN
    L = dataclasses.replace(L, x=x)
    D = upload(L)
    ids, _ = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    ref, cov = O.gemm1(L.x, L.T, L.top_k, L.w13, act, L.alpha, L.beta, L.limit, si, ei, npp, B)
    dsi, dei, dnpp = _dev(si, ei, np.array([npp], np.int32))
    n_out = L.w13.N // 2 if act == "swigluoai" else L.w13.N
    out = M.moe_w4a16_gemm1(D["x"], L.top_k, D["w13"], act, L.alpha, L.beta, L.limit, dsi, dei,
                            dnpp, B, out=poisoned((L.T * L.top_k, n_out)), kernel=kernel)
    got = host_bf16(out)
    assert np.isnan(ref[3 * L.top_k:4 * L.top_k]).all()
    _compare_with_nan(got, ref, cov, f"NaN activation {act} B{B} {kernel}")


def test_nan_token_forward():
    """moe_forward: the NaN token's output row is NaN, every other row matches."""
    L = _small("mxfp4", "swigluoai", T=100)
    x = L.x.copy()
    x[41, 0] = 0x7FC0
    L = dataclasses.replace(L, x=x)
    D = upload(L)
    got = host_bf16(gpu_forward(L, D))
    ref = O.forward(L)["out"]
    assert np.isnan(got[41]).all() and np.isnan(ref[41]).all()
    keep = np.arange(L.T) != 41
    rel = O.row_rel_err(got[keep], ref[keep])
    assert np.isfinite(got[keep]).all() and rel.max() <= TOL


@pytest.mark.parametrize("B,kernel", KERNELS)
def test_gptq_g_idx_identity_and_poison(B, kernel):
    """g_idx = k // G is the same weights as no map (bit-identical outputs);
    a map that differs in one row of expert 2 turns exactly the rows of
    expert 2's slots into NaN and leaves the others bit-identical."""
    L = _small("gptq", "swigluoai", T=40)
    D = upload(L)
    ids, tw = O.route(L)
    si, ei, npp = O.align(ids, L.E, B)
    dsi, dei, dnpp = _dev(si, ei, np.array([npp], np.int32))
    n = L.T * L.top_k
    rows_e = O.slot_experts(si, ei, npp, B, n)

    def g1(w13):
        return M.moe_w4a16_gemm1(D["x"], L.top_k, w13, "swigluoai", L.alpha, L.beta, L.limit,
                                 dsi, dei, dnpp, B, out=poisoned((n, L.I)), kernel=kernel)

    ident = torch.arange(L.H, dtype=torch.int32, device="cuda").div(L.w13.group, rounding_mode="floor")
    ident = ident.repeat(L.E, 1).contiguous()
    base = g1(D["w13"])
    same = g1(dataclasses.replace(D["w13"], g_idx=ident))
    assert torch.equal(base.view(torch.int16), same.view(torch.int16))
    bad = ident.clone()
    bad[2, 70] = 0                               # row 70 sits in group 1
    poison = host_bf16(g1(dataclasses.replace(D["w13"], g_idx=bad)))
    b = host_bf16(base)
    hit = rows_e == 2
    assert hit.any()
    assert np.isnan(poison[hit]).all()
    ok = (rows_e >= 0) & ~hit
    assert np.array_equal(poison[ok], b[ok])
    # GEMM2 and the layer take the identity map too
    a = dev_bf16(S.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((n, L.I)).astype(np.float32)))
    dtw = torch.from_numpy(tw.reshape(-1).astype(np.float32)).cuda()
    identk = torch.arange(L.I, dtype=torch.int32, device="cuda").div(L.w2.group, rounding_mode="floor")
    identk = identk.repeat(L.E, 1).contiguous()
    y0 = M.moe_w4a16_gemm2(a, D["w2"], dtw, True, dsi, dei, dnpp, B, out=poisoned((n, L.H)),
                           kernel=kernel)
    y1 = M.moe_w4a16_gemm2(a, dataclasses.replace(D["w2"], g_idx=identk), dtw, True, dsi, dei, dnpp,
                           B, out=poisoned((n, L.H)), kernel=kernel)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    D2 = dict(D, w13=dataclasses.replace(D["w13"], g_idx=ident),
              w2=dataclasses.replace(D["w2"], g_idx=identk))
    f0 = gpu_forward(L, D, kernel=kernel)
    f1 = gpu_forward(L, D2, kernel=kernel)
    assert torch.equal(f0.view(torch.int16), f1.view(torch.int16))

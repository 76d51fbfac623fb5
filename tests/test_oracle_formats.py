"""Pins for the oracle's format decoders (CPU only).

Each check ties oracle.formats to something other than itself: the table the
NVFP4 page prints, the closed form of e2m1, torch's float8_e4m3fn decode,
ldexp, hand-built GPTQ words, and the group counts the pages state.
"""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    for ln in open(os.path.join(GOLDEN, name)):
        ln = ln.split("#", 1)[0].strip()
        if ln:
            rows.append(ln.split())
    return rows


def test_e2m1_table_matches_page():
    printed = np.array([float(v) for v in _golden_rows("e2m1_table.txt")[0]])
    assert printed.shape == (16,)
    np.testing.assert_array_equal(F.E2M1_TABLE, printed)
    # signed zero at code 8 as printed
    assert np.signbit(F.E2M1_TABLE[8]) and not np.signbit(F.E2M1_TABLE[0])


def test_e2m1_table_matches_closed_form():
    # e2m1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; e = 0 is subnormal.
    for code in range(16):
        s = -1.0 if code & 8 else 1.0
        e, m = (code >> 1) & 3, code & 1
        v = s * (m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
        assert F.E2M1_TABLE[code] == v, code


def test_e4m3fn_all_bytes_match_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(np.isnan(F.E4M3FN_TABLE), nan)
    np.testing.assert_array_equal(F.E4M3FN_TABLE[~nan], ref[~nan])
    assert F.E4M3FN_TABLE[0x7E] == 448.0 and F.E4M3FN_TABLE[0x01] == 2.0 ** -9


def test_e8m0_is_power_of_two():
    for b in range(255):
        assert F.E8M0_TABLE[b] == np.ldexp(1.0, b - 127)
    assert np.isnan(F.E8M0_TABLE[255])


def test_bf16_and_fp16_decode():
    vals = np.array([0.0, 1.0, -2.5, 3.140625, 1e-3], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    got = F.bf16_to_f64(bits)
    ref = torch.from_numpy(vals).to(torch.bfloat16).double().numpy()
    # the chosen values are exact in bf16 except 1e-3, which truncation and RNE
    # round the same way here
    np.testing.assert_array_equal(got[:4], ref[:4])
    h = np.array([1.0, 0.0999755859375, -65504.0], dtype=np.float16)
    np.testing.assert_array_equal(F.fp16_to_f64(h), h.astype(np.float64))


def test_nvfp4_decode_nibble_order_and_scales():
    # one row, K = 32: byte j holds codes for k = 2j (low) and 2j+1 (high)
    codes = np.array([(k * 5 + 3) % 16 for k in range(32)], dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[0x38, 0x40]], dtype=np.uint8)   # e4m3 1.0 and 2.0
    W = F.decode_nvfp4(packed, scales, 0.5, 16)
    for k in range(32):
        s = 1.0 if k < 16 else 2.0
        assert W[0, k] == F.E2M1_TABLE[codes[k]] * s * 0.5


def test_mxfp4_decode():
    codes = np.arange(32, dtype=np.uint8) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    W = F.decode_mxfp4(packed, np.array([[127 - 3]], dtype=np.uint8), 32)
    np.testing.assert_array_equal(W[0], F.E2M1_TABLE[codes] / 8.0)


def test_gptq_decode_hand_built_words():
    # K = 64 (one group), N = 8: q[k, n] = (k + n) % 16, z[n] = n, s[n] = 0.5 * (n + 1)
    K, N, G = 64, 8, 64
    q = np.array([[(k + n) % 16 for n in range(N)] for k in range(K)], dtype=np.int64)
    qw = np.zeros((K // 8, N), dtype=np.int64)
    for k in range(K):
        qw[k // 8] |= q[k] << (4 * (k % 8))
    zw = np.zeros((1, 1), dtype=np.int64)
    for n in range(N):
        zw[0, 0] |= n << (4 * n)
    s = np.array([[0.5 * (n + 1) for n in range(N)]], dtype=np.float16)
    W = F.decode_gptq(qw.astype(np.uint32).view(np.int32), zw.astype(np.uint32).view(np.int32), s, G)
    assert W.shape == (N, K)
    for n in range(N):
        for k in range(K):
            assert W[n, k] == (q[k, n] - n) * 0.5 * (n + 1)
    # an all-ones word (nibble 15 everywhere) with zero point 15 decodes to 0
    W0 = F.decode_gptq(np.full((8, 8), -1, dtype=np.int32), np.full((1, 1), -1, dtype=np.int32),
                       np.ones((1, 8), dtype=np.float16), 64)
    assert not W0.any()


@pytest.mark.parametrize("row", _golden_rows("group_counts.txt"))
def test_group_counts_from_pages(row):
    """Each stated group count is the number of distinct scale groups decode uses.

    Every scale group gets a distinctive power-of-two scale; decoding an all-
    ones code row must show exactly the stated number of distinct groups, the
    last one covering the tail, with nothing read past the real groups.
    """
    K, G, ngroups = int(row[0]), int(row[1]), int(row[2])
    assert K // G == ngroups and K % G == 0
    if G == 16:   # NVFP4
        codes = np.full((1, K // 2), 0x22, dtype=np.uint8)       # both nibbles = 1.0
        sc = np.array([[0x38 + 8 * (g % 4) for g in range(ngroups)]], dtype=np.uint8)  # 1,2,4,8
        W = F.decode_nvfp4(codes, sc, 1.0, G)
        for g in range(ngroups):
            assert np.all(W[0, g * G:(g + 1) * G] == 2.0 ** (g % 4))
        with pytest.raises(AssertionError):
            F.decode_nvfp4(codes, np.concatenate([sc, sc[:, :8]], axis=1), 1.0, G)  # padded groups
    else:         # GPTQ
        N = 8
        qw = np.full((K // 8, N), 0x11111111, dtype=np.int64).astype(np.uint32).view(np.int32)
        zw = np.zeros((ngroups, 1), dtype=np.int32)
        s = np.array([[2.0 ** (g % 5)] * N for g in range(ngroups)], dtype=np.float16)
        W = F.decode_gptq(qw, zw, s, G)
        for g in range(ngroups):
            assert np.all(W[:, g * G:(g + 1) * G] == 2.0 ** (g % 5))


# ------------------------------------------------------------- act-order --

def _act_order_expert(N=24, K=256, G=32, seed=3):
    import synthetic as S
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    perm = rng.permutation(K)
    qw, zz, s16, g_idx = S.quantize_gptq_act_order(w, perm, G)
    return w, perm, qw, zz, s16, g_idx


def test_gptq_act_order_decode_equals_group_ordered_quantisation():
    """Quantising in activation order is quantising the column-permuted matrix.

    Channel perm[j] belongs to group j // G, so column j of the decode of
    quantize_gptq(W[:, perm]) (identity groups, pinned above by hand-built
    words) must equal column perm[j] of the act-order decode, exactly.  A
    decode that used k // G instead of g_idx[k] fails this."""
    import synthetic as S
    G = 32
    w, perm, qw, zz, s16, g_idx = _act_order_expert(G=G)
    W_act = F.decode_gptq(qw, zz, s16, G, g_idx)
    qw_p, zz_p, s_p = S.quantize_gptq(np.ascontiguousarray(w[:, perm]), G)
    W_grp = F.decode_gptq(qw_p, zz_p, s_p, G)
    np.testing.assert_array_equal(W_act[:, perm], W_grp)
    assert not np.array_equal(F.decode_gptq(qw, zz, s16, G), W_act)   # g_idx matters here


def test_gptq_act_order_decode_is_within_one_step_of_the_float_weight():
    """Round-to-nearest quantisation keeps each decoded weight within one step
    (the scale of the element's own group, with the clip at 15 allowed for)
    of the float weight it came from; decoding with the identity groups does
    not."""
    G = 32
    w, perm, qw, zz, s16, g_idx = _act_order_expert(G=G)
    s_own = s16.astype(np.float64)[g_idx, :].T          # [N, K]: scale of (n, k)'s group
    err = np.abs(F.decode_gptq(qw, zz, s16, G, g_idx) - w)
    assert np.all(err <= s_own * 1.01)
    err_id = np.abs(F.decode_gptq(qw, zz, s16, G) - w)
    assert np.any(err_id > s_own * 1.01)


def test_act_order_sort_decodes_to_the_permuted_weight():
    """Rows in group order decode (identity groups) to the act-order weight's
    columns taken in perm order; perm is the stable sort of g_idx."""
    G = 32
    w, perm0, qw, zz, s16, g_idx = _act_order_expert(G=G, seed=8)
    qs, perm, ok = F.act_order_sort(qw, g_idx, G)
    assert ok
    assert np.all(np.diff(g_idx[perm]) >= 0)                       # groups ascending
    for g in range(256 // G):                                     # ascending k inside a group
        run = perm[g * G:(g + 1) * G]
        assert np.all(np.diff(run) > 0) and np.all(g_idx[run] == g)
    np.testing.assert_array_equal(F.decode_gptq(qs, zz, s16, G),
                                  F.decode_gptq(qw, zz, s16, G, g_idx)[:, perm])


def test_act_order_sort_rejects_maps_that_are_not_act_order():
    G = 32
    _, _, qw, zz, s16, g_idx = _act_order_expert(G=G)
    uneven = g_idx.copy()
    uneven[np.flatnonzero(uneven == 0)[0]] = 1                    # group 0 short, group 1 long
    out_of_range = g_idx.copy()
    out_of_range[5] = 256 // G
    for bad in (uneven, out_of_range):
        qs, perm, ok = F.act_order_sort(qw, bad, G)
        assert not ok
        np.testing.assert_array_equal(perm, np.arange(256))
        np.testing.assert_array_equal(qs, qw)


# ------------------------------------------------------------------ MXFP8 --

def test_e4m3_encode_matches_torch_in_range():
    """Every finite e4m3 value, every midpoint between neighbours (ties go to
    the even code) and random float32 values in [-448, 448] encode as torch's
    float8_e4m3fn cast of the same float32 values does."""
    vals = F.E4M3FN_TABLE[np.isfinite(F.E4M3FN_TABLE)]
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2
    rnd = np.random.default_rng(4).uniform(-448, 448, 20000)
    x = np.concatenate([pos, -pos, mids, -mids, rnd, rnd * 1e-3]).astype(np.float32)
    got = F.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)
    # the tie cases really are ties: each midpoint lands on an even code
    assert np.all(F.e4m3_encode(mids) % 2 == 0)


def test_e4m3_encode_saturates_and_keeps_nan():
    big = np.array([448.0, 460.0, 464.0, 500.0, 511.9, 1e6, np.inf])
    assert np.all(F.e4m3_encode(big) == 0x7E)
    assert np.all(F.e4m3_encode(-big) == 0xFE)
    assert F.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_mxfp8_block_rules():
    """Shared exponent floor(log2 amax) - 8 puts each block's largest element
    in e4m3's top binade [256, 512); every element is within half an e4m3 step
    of its value (saturated ones: within 64 units); zero blocks are zero;
    quantising the dequantised values gives the same bytes back."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    v[3, 32:64] = 0.0
    codes, scales = F.quantize_mxfp8(v)
    blk = v.reshape(64, 8, 32)
    amax = np.abs(blk).max(-1)
    unit = F.E8M0_TABLE[scales]
    nz = amax > 0
    assert np.all((amax[nz] / unit[nz] >= 256) & (amax[nz] / unit[nz] < 512))
    assert scales[3, 1] == 0 and not codes[3, 32:64].any()
    deq = F.dequantize_mxfp8(codes, scales)
    s = np.abs(v) / np.repeat(unit, 32, axis=1)                  # element in units of the scale
    _, ex = np.frexp(np.where(s > 0, s, 1.0))
    half_step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 4)       # half of 2**(E-3)
    err = np.abs(deq - v) / np.repeat(unit, 32, axis=1)
    assert np.all(np.where(s < 448, err <= half_step, err <= 64))
    c2, s2 = F.quantize_mxfp8(deq)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)


def test_mxfp8_hand_examples():
    one = np.zeros(32); one[0] = 1.0                # amax 1 -> exponent -8, 1 = 256 * 2**-8
    c, s = F.quantize_mxfp8(one)
    assert s[0] == 127 - 8 and c[0] == 0x78 and not c[1:].any()
    top = np.zeros(32); top[5] = -448.0; top[6] = 3.0   # amax 448 -> exponent 0, values kept
    c, s = F.quantize_mxfp8(top)
    assert s[0] == 127 and c[5] == 0xFE and F.E4M3FN_TABLE[c[6]] == 3.0
    tiny = np.full(32, 2.0 ** -134)                  # exponent clamped at -127: e4m3 subnormal 2**-7
    c, s = F.quantize_mxfp8(tiny)
    assert s[0] == 0 and np.all(c == 0x04)
    c, s = F.quantize_mxfp8(np.full(32, 2.0 ** -140))  # below half the smallest subnormal: zero
    assert s[0] == 0 and not c.any()


def test_bf16_round_is_one_rounding():
    """Nearest bf16 in one step: agrees with torch's cast on float32 inputs
    (no double rounding possible), and picks the nearer neighbour where a
    float64 value sits just below a bf16 midpoint."""
    x = (np.random.default_rng(5).standard_normal(50000) * 10.0).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(F.bf16_round(x.astype(np.float64)), ref)
    mid = 1.0 + 2.0 ** -8                            # midpoint of 1 and 1 + 2**-7
    assert F.bf16_round(np.array([mid - 2.0 ** -40]))[0] == 1.0
    assert F.bf16_round(np.array([mid]))[0] == 1.0   # tie -> even
    assert F.bf16_round(np.array([mid + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7

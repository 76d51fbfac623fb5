"""Oracle: decoding of the 4-bit weight formats, in float64.

Test infrastructure only.  Nothing in the product path imports this module;
only tests/, the smoke check and the CPU-baseline leg of the benchmark do.

Every decode here is exact: the decoded values are small dyadic rationals (or
fp16-scaled integers) that float64 holds without rounding.

Sources
-------
* NVFP4: e2m1 codes, two per byte along K with the even index in the low
  nibble, fp8-e4m3fn block scale per 16 along K and a float32 global scale
  per expert, dequantised as code value x block scale x global scale --
  "moe_wna16_marlin_gemm applies wrong per-row topk weights", minimal repro
  (random NVFP4 weights in ModelOpt layout and its fp32 dequantised
  reference).  The 16-entry e2m1 table is the one printed in that repro.
* MXFP4: e2m1 codes with one e8m0 shared exponent per 32 along K (named on
  "gpt-oss-120b MXFP4 + --enable-expert-parallel crashes"; the per-32 e8m0
  block is the OCP microscaling definition).
* INT4 GPTQ: qweight / qzeros / scales / g_idx per expert, group_size 64
  because 2880 is not a multiple of 128 (OneCompression "GPT-OSS
  (mixed_gptq)", sections "Why GPT-OSS needs special handling" and
  "1. Quantize with 4-bit MoE experts").  Packing: 8 nibbles per int32,
  low nibble first; zeros packed along N; w = (q - z) * s with no +1
  zero offset.  g_idx gives the group of each row: k // G when absent
  (identity), any map for weights quantised in activation order (the page
  lists g_idx beside qweight, qzeros and scales; its meaning is GPTQ's).

Pinned by tests/test_oracle_formats.py: the table equals the page's printed
table and the closed form of e2m1; e4m3fn against torch's float8 decode for
all 256 bytes; e8m0 against ldexp; GPTQ against hand-built words; group
counts 2880/64 = 45 and 2688/16 = 168 (the "168 real + 8 padded scale
groups" of the Nemotron page) via distinctive per-group scales; act-order
decode against the float weights it was quantised from (error within half a
step of the row's own group) and against the group-sorted form.
"""
from __future__ import annotations

import numpy as np

# e2m1 value of each 4-bit code, as printed in the NVFP4 repro.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def e4m3fn_value(byte: int) -> float:
    """OCP fp8 e4m3fn: bias 7, no infinities, S.1111.111 is NaN."""
    b = int(byte) & 0xFF
    sign = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def e8m0_value(byte: int) -> float:
    """OCP e8m0 shared exponent: 2**(byte-127); 0xFF is NaN."""
    b = int(byte) & 0xFF
    if b == 0xFF:
        return float("nan")
    return 2.0 ** (b - 127)


E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def fp16_to_f64(vals: np.ndarray) -> np.ndarray:
    return np.asarray(vals, dtype=np.float16).astype(np.float64)


def _nibbles_along_k(packed: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> codes [N, K]; code k sits in byte k//2, low nibble if k is even."""
    n, kh = packed.shape
    out = np.empty((n, 2 * kh), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def decode_nvfp4(qweight_e: np.ndarray, scales_e: np.ndarray, gscale_e: float,
                 group: int = 16) -> np.ndarray:
    """One expert's NVFP4 weight -> float64 W[N, K] = e2m1 * e4m3(scale[n, k//G]) * gs."""
    codes = _nibbles_along_k(qweight_e)
    n, k = codes.shape
    assert scales_e.shape == (n, k // group), (scales_e.shape, n, k, group)
    blk = E4M3FN_TABLE[scales_e]                       # [N, K/G]
    return E2M1_TABLE[codes] * np.repeat(blk, group, axis=1) * float(gscale_e)


def decode_mxfp4(qweight_e: np.ndarray, scales_e: np.ndarray, group: int = 32) -> np.ndarray:
    """One expert's MXFP4 weight -> float64 W[N, K] = e2m1 * 2**(scale[n, k//G] - 127)."""
    codes = _nibbles_along_k(qweight_e)
    n, k = codes.shape
    assert scales_e.shape == (n, k // group), (scales_e.shape, n, k, group)
    return E2M1_TABLE[codes] * np.repeat(E8M0_TABLE[scales_e], group, axis=1)


def decode_gptq(qweight_e: np.ndarray, zeros_e: np.ndarray, scales_e: np.ndarray,
                group: int = 64, g_idx_e: np.ndarray | None = None) -> np.ndarray:
    """One expert's GPTQ weight -> float64 W[N, K] (note: transposed from storage).

    Storage is qweight int32 [K/8, N], zeros int32 [K/G, N/8], scales fp16
    [K/G, N]; W^T[k, n] = (q[k, n] - z[g(k), n]) * s[g(k), n] with
    g(k) = g_idx[k] (identity g_idx gives k // G).
    """
    kq, n = qweight_e.shape
    k = 8 * kq
    ngroups = k // group
    assert scales_e.shape == (ngroups, n) and zeros_e.shape == (ngroups, n // 8)
    qw = qweight_e.view(np.uint32).astype(np.int64)
    q = np.empty((k, n), dtype=np.int64)
    for i in range(8):
        q[i::8, :] = (qw >> (4 * i)) & 0xF
    zw = zeros_e.view(np.uint32).astype(np.int64)
    z = np.empty((ngroups, n), dtype=np.int64)
    for i in range(8):
        z[:, i::8] = (zw >> (4 * i)) & 0xF
    g = (np.arange(k) // group) if g_idx_e is None else np.asarray(g_idx_e, dtype=np.int64)
    wt = (q - z[g, :]).astype(np.float64) * fp16_to_f64(scales_e)[g, :]
    return np.ascontiguousarray(wt.T)


def act_order_sort(qweight_e: np.ndarray, g_idx_e: np.ndarray, group: int):
    """One act-order GPTQ expert with its rows in group order.

    Returns (qweight_sorted int32 [K/8, N], perm int32 [K], ok).  perm is the
    stable sort of the rows by g_idx (ascending k inside a group) and row j
    of qweight_sorted is row perm[j] of qweight; the groups then sit in runs
    of `group` rows, so the sorted weight decodes with the identity g_idx,
    its column k of W multiplying input channel perm[k].  ok is False when
    g_idx is not an act-order map (a value outside [0, K/G), or a group
    without exactly `group` rows); perm is then the identity and qweight is
    returned unchanged.
    """
    kq, n = qweight_e.shape
    k = 8 * kq
    g = np.asarray(g_idx_e, dtype=np.int64)
    ngroups = k // group
    ok = bool(g.shape == (k,) and g.min() >= 0 and g.max() < ngroups and
              np.all(np.bincount(g, minlength=ngroups) == group))
    if not ok:
        return qweight_e.copy(), np.arange(k, dtype=np.int32), False
    perm = np.argsort(g, kind="stable")
    qw = qweight_e.view(np.uint32).astype(np.int64)
    q = np.empty((k, n), dtype=np.int64)
    for i in range(8):
        q[i::8, :] = (qw >> (4 * i)) & 0xF
    qs = q[perm, :]
    out = np.zeros((kq, n), dtype=np.int64)
    for i in range(8):
        out |= qs[i::8, :] << (4 * i)
    return out.astype(np.uint32).view(np.int32), perm.astype(np.int32), True


# ---------------------------------------------------------------------------
# MXFP8 activations (e4m3 elements, one e8m0 shared exponent per 32 along K)
# ---------------------------------------------------------------------------
#
# The MXFP4 x MXFP8 variant of the layer ("gpt-oss-120b MXFP4 +
# --enable-expert-parallel crashes", sections "Actual behavior" and "Why the
# mxfp8 workaround is not a fix": the activation option switches the MoE to
# MXFP8 activations).  The page names the format only; the encoding is the OCP
# microscaling one: per block of 32 the shared exponent is
# floor(log2(amax)) - 8 (8 = the exponent of e4m3's largest normal, 448 =
# 1.75 * 2**8), the elements are value / 2**exponent rounded to the nearest
# e4m3 value (ties to even), and magnitudes past 448 saturate to 448.
# Readings: an all-zero block takes the smallest exponent (byte 0); the
# exponent is clamped to the e8m0 range [-127, 127]; a block holding a NaN or
# an infinity gets the NaN exponent 0xFF and NaN elements.


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float64 -> e4m3fn byte: round to nearest, ties to even, saturating at
    +-448; NaN -> 0x7F (sign kept)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    fin = np.isfinite(a)
    a0 = np.where(fin, a, 0.0)
    # normal range: a = q * 2**(E-3) with q in [8, 16) after rounding
    _, ex = np.frexp(np.where(a0 > 0, a0, 1.0))
    E = np.maximum(ex.astype(np.int64) - 1, -6)          # below 2**-6: the subnormal step 2**-9
    q = np.rint(np.ldexp(a0, -(E - 3))).astype(np.int64)  # exact scaling, then ties-to-even
    up = q == 16
    E = np.where(up, E + 1, E)
    q = np.where(up, 8, q)
    sub = q < 8                                           # only when E == -6: subnormal code q
    mag = np.where(sub, q, ((E + 7) << 3) | (q - 8))
    mag = np.minimum(mag, 0x7E)                           # 448 is the largest finite value
    mag = np.where(np.isnan(a), 0x7F, np.where(np.isinf(a), 0x7E, mag))
    return (mag.astype(np.uint8) | sign).astype(np.uint8)


def quantize_mxfp8(v: np.ndarray, block: int = 32):
    """float64 [..., K] -> (codes uint8 [..., K], scales uint8 e8m0 [..., K/block])."""
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    assert k % block == 0, k
    blk = v.reshape(v.shape[:-1] + (k // block, block))
    amax = np.max(np.abs(blk), axis=-1)
    bad = ~np.isfinite(amax)
    _, ex = np.frexp(np.where((amax > 0) & ~bad, amax, 1.0))
    e = np.where((amax > 0) & ~bad, ex.astype(np.int64) - 1 - 8, -127)
    e = np.clip(e, -127, 127)
    codes = e4m3_encode(np.ldexp(blk, -e[..., None]))
    codes = np.where(bad[..., None], np.uint8(0x7F), codes).astype(np.uint8)
    scales = np.where(bad, 255, e + 127).astype(np.uint8)
    return codes.reshape(v.shape), scales


def dequantize_mxfp8(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """(codes [..., K], e8m0 scales [..., K/block]) -> float64 [..., K], exactly."""
    return E4M3FN_TABLE[codes] * np.repeat(E8M0_TABLE[scales], block, axis=-1)


def mxfp8_round_trip(v: np.ndarray, block: int = 32) -> np.ndarray:
    """The values an MXFP8 operand holds for float64 input v."""
    return dequantize_mxfp8(*quantize_mxfp8(v, block), block)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float64 -> the nearest bf16 value (ties to even), as float64, in one
    rounding: 8 significant bits, exponent >= -126 (below that the subnormal
    step 2**-133), past the largest finite bf16 -> infinity."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(np.where(np.isfinite(v) & (v != 0), v, 1.0))
    step = np.maximum(ex.astype(np.int64) - 8, -133)      # |v| in [2**(ex-1), 2**ex)
    r = np.ldexp(np.rint(np.ldexp(v, -step)), step)
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)
    return np.where(np.isfinite(v), r, v)


def decode_expert(w, e: int) -> np.ndarray:
    """Decode expert e of a weight family (synthetic.Weights-like object)."""
    if w.fmt == "nvfp4":
        return decode_nvfp4(w.qweight[e], w.scales[e], float(w.global_scale[e]), w.group)
    if w.fmt == "mxfp4":
        return decode_mxfp4(w.qweight[e], w.scales[e], w.group)
    if w.fmt == "gptq":
        g_idx = getattr(w, "g_idx", None)
        return decode_gptq(w.qweight[e], w.zeros[e], w.scales[e], w.group,
                           None if g_idx is None else g_idx[e])
    raise ValueError(w.fmt)

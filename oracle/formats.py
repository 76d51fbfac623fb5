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

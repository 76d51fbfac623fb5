"""Oracle cross-check: the layer by pure-Python loops, for tiny shapes only.

Test infrastructure only (never used by the product path).  It shares no
decode table with oracle.formats: e2m1 is evaluated from its bit fields
(sign * 2**(e-1) * (1 + m/2), or sign * m/2 when e = 0), fp8 scales through
torch's float8_e4m3fn conversion, and every weight element is pulled out of
its packed word by hand.  Its job is to catch indexing mistakes in the
vectorised oracle (a transposed operand, a wrong nibble, a wrong group, the
gate/up interleave, the row a routing weight lands on).
"""
from __future__ import annotations

import math


def _e2m1(code: int) -> float:
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * 0.5 * m
    return s * 2.0 ** (e - 1) * (1.0 + 0.5 * m)


def _e4m3(byte: int) -> float:
    import torch
    return float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def _bf16(bits: int) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def weight(w, e: int, n: int, k: int, _cache={}) -> float:
    """Element W_e[n][k] of a weight family, decoded by hand."""
    if w.fmt in ("nvfp4", "mxfp4"):
        byte = int(w.qweight[e, n, k // 2])
        code = (byte >> 4) if (k & 1) else (byte & 0xF)
        sb = int(w.scales[e, n, k // w.group])
        if w.fmt == "nvfp4":
            key = ("e4m3", sb)
            if key not in _cache:
                _cache[key] = _e4m3(sb)
            return _e2m1(code) * _cache[key] * float(w.global_scale[e])
        return _e2m1(code) * (math.nan if sb == 255 else 2.0 ** (sb - 127))
    # gptq: storage is [K/8][N] words, zeros [K/G][N/8] words, scales [K/G][N]
    word = int(w.qweight[e, k // 8, n]) & 0xFFFFFFFF
    q = (word >> (4 * (k % 8))) & 0xF
    g_idx = getattr(w, "g_idx", None)      # act-order: the row's own group
    g = k // w.group if g_idx is None else int(g_idx[e, k])
    zword = int(w.zeros[e, g, n // 8]) & 0xFFFFFFFF
    z = (zword >> (4 * (n % 8))) & 0xF
    return (q - z) * float(w.scales[e, g, n])


_E4M3_POS = None


def _e4m3_nearest(v: float) -> float:
    """Nearest finite e4m3 value by search over all codes (ties to the even
    code), saturating at 448."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = [(_e4m3(c), c) for c in range(0x7F)]      # 0 .. 448, codes 0x00 .. 0x7E
    a = abs(v)
    if a >= 448.0:
        r = 448.0
    else:
        best = min(_E4M3_POS, key=lambda vc: (abs(a - vc[0]), vc[1] & 1))
        r = best[0]
    return -r if v < 0 else r


def _bf16_nearest(v: float) -> float:
    """Nearest bf16 value (8 significant bits, ties to even) of a normal float."""
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)            # v = m * 2**e, 0.5 <= |m| < 1
    s = abs(m) * 256.0
    lo = math.floor(s)
    d = s - lo
    q = lo + 1 if (d > 0.5 or (d == 0.5 and lo % 2 == 1)) else lo
    return math.copysign(q * 2.0 ** (e - 8), v)


def _mxfp8(vals):
    """MXFP8 value of a row, block by block of 32 (shared exponent
    floor(log2 amax) - 8, elements rounded to e4m3)."""
    out = []
    for b0 in range(0, len(vals), 32):
        blk = vals[b0:b0 + 32]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            out.extend([0.0] * len(blk))
            continue
        ex = math.frexp(amax)[1] - 1 - 8
        ex = max(ex, -127)
        out.extend(_e4m3_nearest(v / 2.0 ** ex) * 2.0 ** ex for v in blk)
    return out


def forward(layer, ids, tw):
    """out[t][h] for every token, given routing (ids[t][j], tw[t][j])."""
    L = layer
    T = L.x.shape[0]
    out = [[0.0] * L.H for _ in range(T)]
    on_input = getattr(L, "weight_on_input", False)   # routing weight scales the input row
    mx = getattr(L, "act_fmt", "bf16") == "mxfp8"      # GEMM inputs at their MXFP8 values
    for t in range(T):
        xt = [_bf16(v) for v in L.x[t]]
        if mx:
            xt = _mxfp8(xt)
        for j in range(L.top_k):
            e = int(ids[t][j])
            if not (0 <= e < L.E):
                continue
            xin = [v * float(tw[t][j]) for v in xt] if on_input else xt
            h = []
            for n in range(L.w13.N):
                acc = 0.0
                for k in range(L.H):
                    acc += weight(L.w13, e, n, k) * xin[k]
                if L.w13.bias is not None:
                    acc += _bf16(L.w13.bias[e, n])
                h.append(acc)
            if L.act == "swigluoai":
                a = []
                for i in range(L.I):
                    g, u = h[2 * i], h[2 * i + 1]
                    g = g if g < L.limit else L.limit
                    u = max(-L.limit, min(L.limit, u))
                    a.append(g / (1.0 + math.exp(-L.alpha * g)) * (u + L.beta))
            else:
                a = [max(v, 0.0) ** 2 for v in h]
            if mx:
                a = _mxfp8([_bf16_nearest(v) for v in a])
            for n in range(L.H):
                acc = 0.0
                for k in range(L.I):
                    acc += weight(L.w2, e, n, k) * a[k]
                if L.w2.bias is not None:
                    acc += _bf16(L.w2.bias[e, n])
                if L.mul_topk_weights and not on_input:
                    acc *= float(tw[t][j])
                out[t][n] += acc
    return out

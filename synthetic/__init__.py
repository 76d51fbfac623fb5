"""Seeded synthetic inputs for the fused W4A16 Mixture-of-Experts layer.

This module is shared by the oracle side (tests, CPU baseline) and the GPU
side (tests, bench).  It only *produces bytes*: router logits, bf16
activations, and 4-bit expert weights in the three storage formats the
pages discuss.  It holds none of the layer's arithmetic (no decode, no
routing, no GEMM); quantisation here is a way to draw realistic weight
bytes, and both sides then consume exactly the same bytes.

Workload shapes follow the pages:
  * gpt-oss-20b MoE call: E=32, top_k=4, hidden=intermediate=2880, NVFP4
    group 16 ("moe_wna16_marlin_gemm applies wrong per-row topk weights",
    environment and repro sections);
  * the same shape as INT4 GPTQ, group 64 (OneCompression "GPT-OSS
    (mixed_gptq)", "Why GPT-OSS needs special handling");
  * gpt-oss-120b, E=128, MXFP4 ("gpt-oss-120b MXFP4 + --enable-expert-parallel
    crashes", environment section);
  * Nemotron-3-Nano, E=128, top-6, hidden 2688, non-gated ReLU^2,
    sigmoid+bias grouped top-k with n_group=1 ("NVFP4 MoE monolithic backend
    ... Nemotron-3-Nano", environment section).

Recipe (applies to every config): NumPy PCG64 streams spawned from
SeedSequence(1000*cfg+7) -- child 0 draws the logits, then the per-expert
logit offsets or router bias; child 1 draws x; children 2 and 3 draw W13 and
W2, one grandchild stream per expert plus one for the bias.  x and logits are
drawn at the largest token count and smaller T take the leading rows.  Weights are
N(0, 0.02) float32 (0.02 is the standard deviation) and quantised as below;
biases N(0, 0.02) rounded to bf16; activations N(0, 1) rounded to bf16;
logits N(0, 1) float32.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses

import numpy as np

# --------------------------------------------------------------------------
# bf16 / fp16 byte helpers (rounding of *inputs* only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Weight-byte generators.  Each takes float32 W[N, K] (output x reduce) of one
# expert and returns its storage bytes.
# --------------------------------------------------------------------------

# e2m1 magnitudes in code order; used only to pick the nearest code.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _e2m1_nearest_code(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (ties to the even code), saturating at +-6."""
    m = np.abs(v)
    # midpoints between neighbouring magnitudes; at a tie the even code wins,
    # so the comparison is '>' when the lower neighbour is even, else '>='.
    code = ((m > 0.25).astype(np.uint8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75)
            + (m > 2.5) + (m >= 3.5) + (m > 5.0))
    code = code.astype(np.uint8)
    code |= np.where(v < 0, np.uint8(8), np.uint8(0))
    return code


def _pack_nibbles_along_k(codes: np.ndarray) -> np.ndarray:
    """[N, K] nibbles -> [N, K/2] bytes, even k in the low nibble."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _to_e4m3_bits(s: np.ndarray) -> np.ndarray:
    import torch  # CPU only: RNE conversion to float8_e4m3fn
    t = torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_nvfp4(w: np.ndarray, group: int = 16):
    """NVFP4 bytes for one expert: (codes u8 [N,K/2], scales e4m3 u8 [N,K/G], gscale f32).

    Global scale gs = amax/(6*448); block scale s = e4m3(amax_blk/6/gs);
    code = nearest e2m1 of w/(s*gs).
    """
    n, k = w.shape
    amax = float(np.max(np.abs(w)))
    gs = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    blk = w.reshape(n, k // group, group)
    bmax = np.max(np.abs(blk), axis=2)
    s_bits = _to_e4m3_bits(bmax / np.float32(6.0) / gs)
    import torch
    s_val = torch.from_numpy(s_bits).view(torch.float8_e4m3fn).float().numpy()
    denom = (s_val * gs)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(denom > 0, blk / np.where(denom > 0, denom, 1), 0).astype(np.float32)
    codes = _e2m1_nearest_code(q.reshape(n, k))
    return _pack_nibbles_along_k(codes), s_bits, gs


def quantize_mxfp4(w: np.ndarray, group: int = 32):
    """MXFP4 bytes for one expert: (codes u8 [N,K/2], scales e8m0 u8 [N,K/G]).

    Shared exponent e = floor(log2(amax_blk)) - 2, stored as e+127; code =
    nearest e2m1 of w / 2**e.
    """
    n, k = w.shape
    blk = w.reshape(n, k // group, group)
    bmax = np.max(np.abs(blk), axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(bmax > 0, np.floor(np.log2(np.where(bmax > 0, bmax, 1))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    s_bits = (e + 127).astype(np.uint8)
    q = (blk / np.ldexp(np.float32(1.0), e)[:, :, None].astype(np.float32)).astype(np.float32)
    codes = _e2m1_nearest_code(q.reshape(n, k))
    return _pack_nibbles_along_k(codes), s_bits


def quantize_gptq(w: np.ndarray, group: int = 64):
    """INT4 GPTQ-format bytes (round to nearest, asymmetric) for one expert.

    Returns qweight int32 [K/8, N] (nibble i holds k%8==i), zeros int32
    [K/G, N/8] (nibble i holds n%8==i), scales fp16 [K/G, N].  Per group and
    column: s = fp16((max-min)/15), z = clip(round(-min/s), 0, 15),
    q = clip(round(w/s) + z, 0, 15).
    """
    n, k = w.shape
    wt = np.ascontiguousarray(w.T)                     # [K, N]
    g = wt.reshape(k // group, group, n)
    mn = g.min(axis=1)
    mx = g.max(axis=1)
    s16 = ((mx - mn) / np.float32(15.0)).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16).astype(np.float16)
    s = s16.astype(np.float32)
    z = np.clip(np.rint(-mn / s), 0, 15).astype(np.int64)
    q = np.clip(np.rint(g / s[:, None, :]) + z[:, None, :], 0, 15).astype(np.int64)
    q = q.reshape(k, n)
    qw = np.zeros((k // 8, n), dtype=np.int64)
    for i in range(8):
        qw |= q[i::8, :] << (4 * i)
    zz = np.zeros((k // group, n // 8), dtype=np.int64)
    for i in range(8):
        zz |= z[:, i::8] << (4 * i)
    return (qw.astype(np.uint32).view(np.int32), zz.astype(np.uint32).view(np.int32), s16)


def quantize_gptq_act_order(w: np.ndarray, perm: np.ndarray, group: int = 64):
    """INT4 GPTQ bytes quantised in activation order, for one expert.

    perm is the order in which the input channels (columns of w [N, K]) are
    quantised; channel perm[j] joins group j // G.  The columns are grouped in
    that order, quantised as quantize_gptq does, and the rows of qweight are
    put back in channel order.  Returns (qweight int32 [K/8, N], zeros int32
    [K/G, N/8], scales fp16 [K/G, N], g_idx int32 [K]) with
    g_idx[perm[j]] = j // G.
    """
    n, k = w.shape
    perm = np.asarray(perm, dtype=np.int64)
    qw_p, zz, s16 = quantize_gptq(np.ascontiguousarray(w[:, perm]), group)
    # unpack the permuted rows, put row j back at channel perm[j], repack
    qp = qw_p.view(np.uint32).astype(np.int64)
    q_perm = np.empty((k, n), dtype=np.int64)
    for i in range(8):
        q_perm[i::8, :] = (qp >> (4 * i)) & 0xF
    q = np.empty_like(q_perm)
    q[perm, :] = q_perm
    qw = np.zeros((k // 8, n), dtype=np.int64)
    for i in range(8):
        qw |= q[i::8, :] << (4 * i)
    g_idx = np.empty((k,), dtype=np.int32)
    g_idx[perm] = (np.arange(k) // group).astype(np.int32)
    return qw.astype(np.uint32).view(np.int32), zz, s16, g_idx


# --------------------------------------------------------------------------
# Layer description
# --------------------------------------------------------------------------

FORMATS = ("nvfp4", "mxfp4", "gptq")
DEFAULT_GROUP = {"nvfp4": 16, "mxfp4": 32, "gptq": 64}


@dataclasses.dataclass
class Weights:
    """One expert weight tensor family (all experts); logical W_e is [N][K]."""
    fmt: str
    group: int
    N: int
    K: int
    qweight: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray | None
    global_scale: np.ndarray | None
    bias: np.ndarray | None          # bf16 bits [E, N] or None
    g_idx: np.ndarray | None = None  # GPTQ act-order: int32 [E, K] group of each row, or None


@dataclasses.dataclass
class Layer:
    E: int
    top_k: int
    H: int
    I: int
    act: str                         # "swigluoai" | "relu2"
    route: str                       # "softmax" | "sigmoid_bias"
    renormalize: bool
    mul_topk_weights: bool
    alpha: float
    beta: float
    limit: float
    logits: np.ndarray               # f32 [T, E]
    expert_bias: np.ndarray | None   # f32 [E]
    x: np.ndarray                    # bf16 bits [T, H]
    w13: Weights
    w2: Weights
    seed: int
    weight_on_input: bool = False    # routing weight scales GEMM1's input (top_k = 1)
    act_fmt: str = "bf16"            # "mxfp8": each GEMM takes its input at its MXFP8 value

    @property
    def T(self) -> int:
        return self.x.shape[0]

    @property
    def N1(self) -> int:
        return 2 * self.I if self.act == "swigluoai" else self.I

    def take(self, T: int) -> "Layer":
        """The same layer restricted to the first T tokens."""
        return dataclasses.replace(self, logits=self.logits[:T], x=self.x[:T])


def _make_weights(ss, fmt, group, E, N, K, bias, threads=8, act_order=False):
    """Draw E experts of W[N, K] ~ N(0, 0.02), quantise each, then the bias.

    Expert e draws from its own child stream ss.spawn(E+1)[e] (the last child
    draws the bias), so experts can be generated in parallel and the bytes do
    not depend on the thread count.  act_order (GPTQ only): after W, the
    expert's stream draws a uniform random channel order and the expert is
    quantised in that order (quantize_gptq_act_order); W itself is unchanged.
    """
    assert not act_order or fmt == "gptq"
    kids = ss.spawn(E + 1)
    if fmt in ("nvfp4", "mxfp4"):
        qweight = np.empty((E, N, K // 2), dtype=np.uint8)
        scales = np.empty((E, N, K // group), dtype=np.uint8)
        zeros = None
    else:
        qweight = np.empty((E, K // 8, N), dtype=np.int32)
        scales = np.empty((E, K // group, N), dtype=np.float16)
        zeros = np.empty((E, K // group, N // 8), dtype=np.int32)
    gscale = np.empty((E,), dtype=np.float32) if fmt == "nvfp4" else None
    g_idx = np.empty((E, K), dtype=np.int32) if act_order else None

    def one(e):
        rng = np.random.Generator(np.random.PCG64(kids[e]))
        w = rng.standard_normal((N, K), dtype=np.float32)
        w *= np.float32(0.02)
        if act_order:
            qweight[e], zeros[e], scales[e], g_idx[e] = quantize_gptq_act_order(
                w, rng.permutation(K), group)
        elif fmt == "nvfp4":
            qweight[e], scales[e], gscale[e] = quantize_nvfp4(w, group)
        elif fmt == "mxfp4":
            qweight[e], scales[e] = quantize_mxfp4(w, group)
        else:
            qweight[e], zeros[e], scales[e] = quantize_gptq(w, group)

    if threads > 1 and E > 1:
        with concurrent.futures.ThreadPoolExecutor(min(threads, E)) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    b = None
    if bias:
        rb = np.random.Generator(np.random.PCG64(kids[E]))
        b = f32_to_bf16_bits(rb.standard_normal((E, N), dtype=np.float32) * np.float32(0.02))
    return Weights(fmt=fmt, group=group, N=N, K=K, qweight=qweight, scales=scales,
                   zeros=zeros, global_scale=gscale, bias=b, g_idx=g_idx)


def make_weights(fmt, *, E, N, K, group=None, bias=True, seed=0, threads=8,
                 act_order=False) -> Weights:
    """One family of synthetic 4-bit expert weights [E][N][K] (same recipe as make_layer)."""
    return _make_weights(np.random.SeedSequence(seed), fmt, group or DEFAULT_GROUP[fmt], E, N, K,
                         bias, threads, act_order)


def make_layer(*, E, top_k, H, I, fmt, act="swigluoai", route="softmax", T,
               seed, group=None, bias=True, skew_std=0.0, router_bias_std=0.0,
               renormalize=True, mul_topk_weights=True, alpha=1.702, beta=1.0,
               limit=7.0, x_std=1.0, threads=8, act_order=False) -> Layer:
    """Draw one synthetic MoE layer (see the module docstring for the recipe)."""
    group = group or DEFAULT_GROUP[fmt]
    ss_router, ss_x, ss_w13, ss_w2 = np.random.SeedSequence(seed).spawn(4)
    rng = np.random.Generator(np.random.PCG64(ss_router))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    expert_bias = None
    if skew_std > 0:
        off = rng.standard_normal((E,), dtype=np.float32) * np.float32(skew_std)
        logits = (logits + off[None, :]).astype(np.float32)
    if route == "sigmoid_bias":
        expert_bias = rng.standard_normal((E,), dtype=np.float32) * np.float32(router_bias_std)
    rx = np.random.Generator(np.random.PCG64(ss_x))
    x = f32_to_bf16_bits(rx.standard_normal((T, H), dtype=np.float32) * np.float32(x_std))
    n1 = 2 * I if act == "swigluoai" else I
    w13 = _make_weights(ss_w13, fmt, group, E, n1, H, bias, threads, act_order)
    w2 = _make_weights(ss_w2, fmt, group, E, H, I, bias, threads, act_order)
    return Layer(E=E, top_k=top_k, H=H, I=I, act=act, route=route,
                 renormalize=renormalize, mul_topk_weights=mul_topk_weights,
                 alpha=alpha, beta=beta, limit=limit, logits=logits,
                 expert_bias=expert_bias, x=x, w13=w13, w2=w2, seed=seed)


# The five workloads.  "T" lists the token counts; inputs are drawn at max(T).
CONFIGS = {
    1: dict(name="tiny E8 top2 h512 NVFP4", E=8, top_k=2, H=512, I=512, fmt="nvfp4",
            act="swigluoai", route="softmax", T=(32,)),
    2: dict(name="gpt-oss-20b E32 top4 h2880 NVFP4", E=32, top_k=4, H=2880, I=2880,
            fmt="nvfp4", act="swigluoai", route="softmax", T=(1, 8, 64, 512, 4096)),
    3: dict(name="gpt-oss-20b E32 top4 h2880 INT4-GPTQ g64", E=32, top_k=4, H=2880,
            I=2880, fmt="gptq", act="swigluoai", route="softmax", T=(2048,)),
    4: dict(name="gpt-oss-120b E128 top4 h2880 MXFP4 skewed", E=128, top_k=4, H=2880,
            I=2880, fmt="mxfp4", act="swigluoai", route="softmax", T=(1, 16, 128, 1024, 8192),
            skew_std=1.5),
    5: dict(name="Nemotron-3-Nano E128 top6 h2688 i1856 ReLU2 NVFP4", E=128, top_k=6,
            H=2688, I=1856, fmt="nvfp4", act="relu2", route="sigmoid_bias", T=(2048,),
            router_bias_std=0.1, bias=False),
}


def config_seed(cfg: int) -> int:
    return 1000 * cfg + 7


def make_config(cfg: int, T: int | None = None) -> Layer:
    """The named workload at its own seed.

    Inputs are drawn at the config's largest token count (so every T sees
    the same leading rows); T, if given, keeps the first T tokens.
    """
    c = dict(CONFIGS[cfg])
    c.pop("name")
    ts = c.pop("T")
    t_draw = max(ts)
    layer = make_layer(T=t_draw, seed=config_seed(cfg), **c)
    if T is not None:
        layer = layer.take(T)
    return layer


def make_router_inputs(cfg: int, T: int | None = None):
    """Only the router inputs of a config: (logits f32 [T, E], expert_bias f32 [E] or None).

    Same seed and draw order as make_config (logits and the per-expert
    offsets / router bias are the first draws), so the values are identical.
    """
    c = CONFIGS[cfg]
    ss_router = np.random.SeedSequence(config_seed(cfg)).spawn(4)[0]
    rng = np.random.Generator(np.random.PCG64(ss_router))
    t_draw = max(c["T"])
    E = c["E"]
    logits = rng.standard_normal((t_draw, E), dtype=np.float32)
    if c.get("skew_std", 0.0) > 0:
        off = rng.standard_normal((E,), dtype=np.float32) * np.float32(c["skew_std"])
        logits = (logits + off[None, :]).astype(np.float32)
    bias = None
    if c["route"] == "sigmoid_bias":
        bias = rng.standard_normal((E,), dtype=np.float32) * np.float32(c["router_bias_std"])
    if T is not None:
        logits = logits[:T]
    return logits, bias

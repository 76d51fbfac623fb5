"""Oracle: the fused W4A16 MoE layer written out from its definition (float64).

Test infrastructure only.  The product path never imports, links or runs
anything under oracle/; tests, the smoke check and the benchmark's CPU
baseline do.

What the layer computes (the plain definition; the GPU reaches it up to
rounding):

  route   topk(softmax(logits), k), renormalised over the selected k
          ("moe_wna16_marlin_gemm applies wrong per-row topk weights",
          repro "Routing" step), or sigmoid + per-expert bias grouped top-k
          with n_group = 1, weights renormalised ("NVFP4 MoE monolithic
          backend ... Nemotron-3-Nano", Analysis item 3).
  align   stable sort of the flat slots f = t*k + j by expert, each expert's
          segment padded to a multiple of block_m; per-block expert id, -1
          for unused blocks; sentinel id = size_m*top_k marks padding (the
          same repro: moe_align_block_size and its reference loop that skips
          blocks with expert id < 0 and ids >= M*TOPK).
  gemm1   h = W13_e x_t + b13_e for each slot, then swigluoai over the
          interleaved (gate = even row, up = odd row) pairs, or ReLU^2
          ("gpt-oss-20b NVFP4 inference is broken", Gap 3: clamped SwiGLU
          with alpha/beta/limit, biases, interleaved gate/up; Nemotron page:
          non-gated ReLU^2).
  gemm2   y = (W2_e a + b2_e) * w_slot when mul_topk_weights, per row by the
          slot's own routing weight (repro fp32 reference
          "out[row] = (act[row] @ w[e].T + 0) * topk_w[row]").
          The other mode the same page names, apply_router_weight_on_input
          (top_k = 1): the routing weight scales GEMM1's input row instead,
          h = W13_e (w_slot x_t) + b13_e, and GEMM2 multiplies nothing.
  sum     out_t = sum_j y_{t,j} at the true hidden width (the op's output is
          the unpadded 2880, "gpt-oss-120b MXFP4 ... crashes", root cause).
  mxfp8   (act_fmt = "mxfp8", the MXFP8-activation variant the same page
          names) each GEMM takes its input at its MXFP8 value: x as given,
          the activation after its bf16 rounding (formats.quantize_mxfp8).

Readings where the pages are silent (each listed in the design notes):
  * swigluoai: g' = min(g, limit), u' = clamp(u, -limit, limit),
    a = g' * sigmoid(alpha * g') * (u' + beta), beta = 1.  The pages only
    name alpha / beta / clamp_limit; the formula itself is parity unpinned
    against the pages and is pinned only by its closed-form special cases.
  * top-k order: descending, ties to the lower expert id; softmax top-k is
    selected on the raw logits (softmax is monotone).
  * sigmoid+bias: score = fp32(sigmoid computed in float64) + bias in fp32;
    the k largest scores are selected; the weights are the *unbiased*
    sigmoids renormalised (routed scale 1).  Selection is an integer
    decision taken from float32 scores on both sides.
  * bias is added before the activation (gemm1) and before the routing
    weight multiply (gemm2).
  * ids outside [0, E) are not routed anywhere: they get no slot in align
    and contribute nothing to the sum.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_round, bf16_to_f64, decode_expert, mxfp8_round_trip

# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------


def _topk_desc_lowid(score: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row; ties go to the lower index."""
    T, E = score.shape
    # stable argsort of -score keeps lower ids first among equal scores
    order = np.argsort(-score, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_softmax(logits: np.ndarray, top_k: int, renormalize: bool = True):
    """topk(softmax(logits)) -> (ids int32 [T,k], weights float64 [T,k])."""
    lg = np.asarray(logits, dtype=np.float32)
    ids = _topk_desc_lowid(lg, top_k)
    l64 = lg.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


def sigmoid_f32(logits: np.ndarray) -> np.ndarray:
    """Sigmoid evaluated in float64 and rounded once to float32."""
    l64 = np.asarray(logits, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-l64))).astype(np.float32)


def route_sigmoid_bias(logits: np.ndarray, expert_bias: np.ndarray, top_k: int,
                       renormalize: bool = True):
    """Sigmoid + bias top-k with n_group = 1 (grouped top-k over one group).

    Selection uses the float32 sum sigmoid + bias; weights use the unbiased
    sigmoid values of the selected experts.
    """
    s = sigmoid_f32(logits)
    score = (s + np.asarray(expert_bias, dtype=np.float32)[None, :]).astype(np.float32)
    ids = _topk_desc_lowid(score, top_k)
    w = np.take_along_axis(s.astype(np.float64), ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


def route(layer_or_logits, top_k=None, kind="softmax", expert_bias=None, renormalize=True):
    if hasattr(layer_or_logits, "logits"):
        L = layer_or_logits
        return route(L.logits, L.top_k, L.route, L.expert_bias, L.renormalize)
    if kind == "softmax":
        return route_softmax(layer_or_logits, top_k, renormalize)
    if kind == "sigmoid_bias":
        return route_sigmoid_bias(layer_or_logits, expert_bias, top_k, renormalize)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# align
# ---------------------------------------------------------------------------


def align_capacity(T: int, top_k: int, E: int, block_m: int) -> int:
    """Rows of sorted_ids: every expert that can be hit pads to block_m."""
    n = T * top_k
    worst = n + min(E, n) * (block_m - 1)
    return ((worst + block_m - 1) // block_m) * block_m


def align(topk_ids: np.ndarray, E: int, block_m: int):
    """Stable per-expert sort with padding -> (sorted_ids, expert_ids, num_post_pad).

    sorted_ids has align_capacity() entries, expert_ids capacity/block_m.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    n = ids.shape[0]
    sentinel = n
    cap = align_capacity(n, 1, E, block_m)   # depends on T*k only
    sorted_ids = np.full(cap, sentinel, dtype=np.int32)
    expert_ids = np.full(cap // block_m if block_m else 0, -1, dtype=np.int32)
    pos = 0
    for e in range(E):
        slots = np.nonzero(ids == e)[0]          # ascending flat slot order
        cnt = slots.shape[0]
        if cnt == 0:
            continue
        padded = -(-cnt // block_m) * block_m
        sorted_ids[pos:pos + cnt] = slots
        expert_ids[pos // block_m:(pos + padded) // block_m] = e
        pos += padded
    return sorted_ids, expert_ids, np.int32(pos)


def slot_experts(sorted_ids, expert_ids, num_post_pad, block_m, n_slots):
    """Expert of each flat slot as the aligned blocks assign it (-1 if none).

    This is the repro's reference loop: walk the blocks, skip blocks whose
    expert id is negative, and give each real entry of the block that expert.
    """
    row_expert = np.full(n_slots, -1, dtype=np.int64)
    for b in range(int(num_post_pad) // block_m):
        e = int(expert_ids[b])
        if e < 0:
            continue
        blk = np.asarray(sorted_ids[b * block_m:(b + 1) * block_m], dtype=np.int64)
        row_expert[blk[blk < n_slots]] = e
    return row_expert


# ---------------------------------------------------------------------------
# activation
# ---------------------------------------------------------------------------


def swigluoai(gate: np.ndarray, up: np.ndarray, alpha: float, beta: float, limit: float):
    g = np.minimum(gate, limit)
    u = np.clip(up, -limit, limit)
    return g * (1.0 / (1.0 + np.exp(-alpha * g))) * (u + beta)


def relu2(h: np.ndarray):
    r = np.maximum(h, 0.0)
    return r * r


def activation(h: np.ndarray, act: str, alpha: float, beta: float, limit: float):
    """h[..., N1] -> a[..., I].  Gated: gate = even columns, up = odd columns."""
    if act == "swigluoai":
        return swigluoai(h[..., 0::2], h[..., 1::2], alpha, beta, limit)
    if act == "relu2":
        return relu2(h)
    if act == "none":
        return h
    raise ValueError(act)


# ---------------------------------------------------------------------------
# the two grouped GEMMs, with the same block semantics as the library calls
# ---------------------------------------------------------------------------


def _bias_f64(w, e):
    return 0.0 if w.bias is None else bf16_to_f64(w.bias[e])


def gemm1(x_bits, size_m, top_k, w13, act, alpha, beta, limit,
          sorted_ids, expert_ids, num_post_pad, block_m, topk_w_flat=None, act_fmt="bf16"):
    """Grouped GEMM1 over aligned blocks.

    Row f of the result (flat slot f = t*top_k + j) is
    act(W13_e x_t + b13_e) with e the expert of f's block and t = f // top_k;
    with topk_w_flat given (routing weight on the input), the input row is
    w_f x_t instead.  act_fmt "mxfp8": x_t is taken at its MXFP8 value.
    Returns (out float64 [size_m*top_k, N_out], covered bool [size_m*top_k]).
    """
    n_slots = size_m * top_k
    x = bf16_to_f64(x_bits)
    if act_fmt == "mxfp8":
        x = mxfp8_round_trip(x)
    re = slot_experts(sorted_ids, expert_ids, num_post_pad, block_m, n_slots)
    n_out = w13.N // 2 if act == "swigluoai" else w13.N
    out = np.zeros((n_slots, n_out), dtype=np.float64)
    tw = None if topk_w_flat is None else np.asarray(topk_w_flat, dtype=np.float64).reshape(-1)
    for e in np.unique(re[re >= 0]):
        rows = np.nonzero(re == e)[0]
        W = decode_expert(w13, int(e))                       # [N1, K]
        xr = x[rows // top_k]
        if tw is not None:
            xr = xr * tw[rows][:, None]
        h = xr @ W.T + _bias_f64(w13, int(e))
        out[rows] = activation(h, act, alpha, beta, limit)
    return out, re >= 0


def gemm2(a_bits_or_f64, size_m, w2, topk_w_flat, mul_topk_weights,
          sorted_ids, expert_ids, num_post_pad, block_m, act_fmt="bf16"):
    """Grouped GEMM2 in the top_k = 1 view: row f = (W2_e a_f + b2_e) [* w_f].

    a is bf16 bits (uint16) or float64 rows indexed by flat slot.  act_fmt
    "mxfp8": a_f is taken at the MXFP8 value of its bf16 rounding (the
    activation is held in bf16 between the GEMMs).
    Returns (y float64 [size_m, N], covered bool [size_m]).
    """
    a = a_bits_or_f64
    a = bf16_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)
    if act_fmt == "mxfp8":
        a = mxfp8_round_trip(bf16_round(a))
    re = slot_experts(sorted_ids, expert_ids, num_post_pad, block_m, size_m)
    y = np.zeros((size_m, w2.N), dtype=np.float64)
    tw = np.asarray(topk_w_flat, dtype=np.float64).reshape(-1)
    for e in np.unique(re[re >= 0]):
        rows = np.nonzero(re == e)[0]
        W = decode_expert(w2, int(e))                        # [H, I]
        r = a[rows] @ W.T + _bias_f64(w2, int(e))
        if mul_topk_weights:
            r = r * tw[rows][:, None]
        y[rows] = r
    return y, re >= 0


def moe_sum(y, topk_ids, E):
    """out_t = sum over j of y[t*k + j], j ascending, skipping ids outside [0, E)."""
    ids = np.asarray(topk_ids)
    T, k = ids.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        valid = (ids[:, j] >= 0) & (ids[:, j] < E)
        out[valid] += y[np.arange(T)[valid] * k + j]
    return out


def forward(layer, block_m: int = 16, topk=None):
    """The whole layer for synthetic.Layer-like input -> dict of float64 results.

    topk, if given, is (ids, weights) to use instead of routing (lets a test
    feed the GPU's own routing when only the GEMM chain is under test).
    """
    L = layer
    T = L.x.shape[0]
    ids, w = route(L) if topk is None else topk
    on_input = getattr(L, "weight_on_input", False)
    act_fmt = getattr(L, "act_fmt", "bf16")
    sorted_ids, expert_ids, npp = align(ids, L.E, block_m)
    act, _ = gemm1(L.x, T, L.top_k, L.w13, L.act, L.alpha, L.beta, L.limit,
                   sorted_ids, expert_ids, npp, block_m,
                   topk_w_flat=w.reshape(-1) if on_input else None, act_fmt=act_fmt)
    y, _ = gemm2(act, T * L.top_k, L.w2, w.reshape(-1), L.mul_topk_weights and not on_input,
                 sorted_ids, expert_ids, npp, block_m, act_fmt=act_fmt)
    out = moe_sum(y, ids, L.E)
    return dict(topk_ids=ids, topk_w=w, sorted_ids=sorted_ids, expert_ids=expert_ids,
                num_post_pad=npp, act=act, y=y, out=out)


def forward_tokens(layer, tokens, topk=None):
    """The layer's output for a subset of tokens (same definition as forward()).

    Used to check full-size runs on sampled rows: only the experts those
    tokens route to are decoded, one at a time, so memory stays at one
    expert's float64 weights.  The (token, choice) rows routed to an expert
    are stacked and multiplied by its weights together (each row's result is
    its own dot products, as one at a time); the rows are then summed over the
    choices j in ascending order.  Returns float64 [len(tokens), H].
    """
    L = layer
    ids, w = route(L) if topk is None else topk
    tokens = list(tokens)
    x = bf16_to_f64(L.x)
    mx = getattr(L, "act_fmt", "bf16") == "mxfp8"
    on_input = getattr(L, "weight_on_input", False)
    y = np.zeros((len(tokens), L.top_k, L.H), dtype=np.float64)
    by_expert = {}
    for i, t in enumerate(tokens):
        for j in range(L.top_k):
            e = int(ids[t, j])
            if 0 <= e < L.E:
                by_expert.setdefault(e, []).append((i, t, j))
    for e, items in sorted(by_expert.items()):
        W13 = decode_expert(L.w13, e)
        W2 = decode_expert(L.w2, e)
        ii = np.array([it[0] for it in items])
        tt = np.array([it[1] for it in items])
        jj = np.array([it[2] for it in items])
        wr = np.asarray(w, dtype=np.float64)[tt, jj]
        xin = x[tt] * wr[:, None] if on_input else x[tt]
        if mx:
            xin = mxfp8_round_trip(xin)
        h = xin @ W13.T + _bias_f64(L.w13, e)
        a = activation(h, L.act, L.alpha, L.beta, L.limit)
        if mx:
            a = mxfp8_round_trip(bf16_round(a))
        yv = a @ W2.T + _bias_f64(L.w2, e)
        if L.mul_topk_weights and not on_input:
            yv = yv * wr[:, None]
        y[ii, jj] = yv
        del W13, W2
    out = np.zeros((len(tokens), L.H), dtype=np.float64)
    for j in range(L.top_k):
        out += y[:, j]
    return out


# ---------------------------------------------------------------------------
# comparison metric
# ---------------------------------------------------------------------------


def row_rel_err(o: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row ||o - ref||_2 / (||ref||_2 + 1e-9), the repro's error metric."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(o - ref, axis=-1) / (np.linalg.norm(ref, axis=-1) + 1e-9)

#!/usr/bin/env python3
"""Throughput of the fused W4A16 MoE layer on one MI355X.

Headline workload: the gpt-oss-20b-shaped MoE layer -- E=32 experts, top-4,
hidden = intermediate = 2880, NVFP4 (e2m1 + e4m3 scale per 16 + fp32 global
scale) weights, per-expert biases, swigluoai, routing weight applied in
GEMM2's epilogue -- on synthetic inputs (seeded; see synthetic/).  One step is
one moe_forward call (route -> align -> GEMM1 -> GEMM2 -> sum) over a batch
of T tokens with everything already resident in HBM.  The headline value is
at T = 4096; the same JSON line carries the other token counts of the sweep
and the other four workloads ("configs": the INT4-GPTQ g64 layer at T = 2048,
the gpt-oss-120b-shaped MXFP4 layer with skewed routing at T in {1, 16, 128,
1024, 8192}, the Nemotron-3-Nano-shaped ReLU^2 layer at T = 2048), each row
with its roofline bound and fraction.

Weight copies are rotated between calls so that no call finds its weights in
the 256 MB last-level cache left behind by the previous one (enough copies
that the touched experts of the copies together exceed it).  The weights are
loaded as a user of the library loads them: NVFP4 and MXFP4 families are
re-laid by K chunk once at load time (moe_*_scales_by_chunk and
moe_*_codes_by_chunk) and the checkpoint layout is then dropped, so one copy
of the codes stays on the device and every kernel reads that layout
(--no-codes-by-chunk keeps the checkpoint codes beside the scales by chunk,
--checkpoint-scales the checkpoint layout alone); GPTQ has one layout.

The dominant kernel (GEMM1 at the headline size) is timed on its own with one
HIP event pair around each launch, on the stream it is launched on; the mean
launch duration gives roofline.achieved (the same quantity a kernel trace
reports as the kernel's average duration).

Prints ONE JSON line.  --gpus N > 1 is refused: the library runs the layer on one GPU.

--act-order adds a leg on the INT4-GPTQ g64 layer of the same shape: the layer
with plain (group-ordered) weights against the same layer quantised in
activation order (both families sorted at load time, inputs gathered per slot
at run time), and the gather kernel alone; reported under "act_order".

--mxfp8 adds a leg on the gpt-oss-120b-shaped MXFP4 layer (E=128, top-4,
2880/2880): bf16 activations against MXFP8 activations (moe_forward_mxfp8),
and GEMM1 alone on the MX-scaled matrix cores against its fp8 peak; reported
under "mxfp8".
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
LLC_BYTES = 256 << 20        # MI355X last-level (Infinity) cache


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes_per_expert(L) -> int:
    """Bytes one touched expert must stream: 4-bit codes, scales, zeros, global scale, biases."""
    tot = 0
    for w in (L.w13, L.w2):
        tot += w.qweight[0].nbytes + w.scales[0].nbytes
        if w.zeros is not None:
            tot += w.zeros[0].nbytes
        if w.global_scale is not None:
            tot += 4
        if w.bias is not None:
            tot += w.bias[0].nbytes
    return tot


def algorithmic(L, T, ids):
    """(bytes, flops, touched experts) the layer must move / compute for T tokens
    with routing ids: the touched experts' weights, x, out and the logits."""
    touched = len(np.unique(ids[(ids >= 0) & (ids < L.E)]))
    nbytes = touched * alg_bytes_per_expert(L) + T * L.H * 2 * 2 + T * L.E * 4
    flops = 2 * T * L.top_k * L.H * (L.N1 + L.I)
    return nbytes, flops, touched


def gemm1_alg(L, T, ids):
    """GEMM1 alone: touched experts' w13 codes, scales, bias, global scale; x in, act out."""
    touched = len(np.unique(ids))
    w = L.w13
    b = touched * (w.qweight[0].nbytes + w.scales[0].nbytes + 4 +
                   (w.bias[0].nbytes if w.bias is not None else 0))
    b += T * L.H * 2 + T * L.top_k * L.I * 2
    f = 2 * T * L.top_k * L.H * L.N1
    return b, f


def roofline_row(L, T, ids, ms):
    nb, fl, touched = algorithmic(L, T, ids)
    t_hbm = nb / (HBM_PEAK_GBS * 1e9)
    t_mfma = fl / (BF16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return dict(T=T, ms=ms, tokens_per_s=T / (ms * 1e-3), touched_experts=touched,
                alg_bytes=nb, alg_flops=fl, GBps=nb / (ms * 1e-3) / 1e9,
                TFLOPs=fl / (ms * 1e-3) / 1e12, bound=bound,
                roofline_frac=max(t_hbm, t_mfma) / (ms * 1e-3))


def profiled_traffic():
    """GEMM1 HBM bytes per launch from the committed counter summary, or None.

    The summary records the GEMM source it was taken on; if the source has
    changed since, the figure no longer describes this kernel and None is
    returned.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_nvfp4_e32_traffic.md")
    src = os.path.join(ROOT, "bit_weight_expert_amd", "csrc", "gemm_impl.h")
    try:
        fields = dict(ln.split(":", 1) for ln in open(path) if ln.startswith(("traffic_", "kernel_")))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if not sha.startswith(fields["kernel_source_sha256_prefix"].strip()):
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def act_order_leg(args, time_calls, time_launches):
    """GPTQ g64 layer (E=32, top-4, 2880/2880): plain vs act-order weights."""
    import torch
    import synthetic as S
    import bit_weight_expert_amd as M

    c = dict(S.CONFIGS[3])
    c.pop("name")
    c.pop("T")
    ts = [int(t) for t in args.act_order_tokens.split(",") if t]
    t0 = time.time()
    Lp = S.make_layer(T=max(ts), seed=S.config_seed(3) + 1, **c)
    La = S.make_layer(T=max(ts), seed=S.config_seed(3) + 1, act_order=True, **c)
    log(f"act-order leg: generated the plain and act-order GPTQ layers in {time.time() - t0:.1f}s")
    dev = torch.device("cuda")

    def up(w):
        return M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales, w.zeros,
                                          w.global_scale, w.bias)

    def prep(w):
        d = up(w)
        qs, kp, st = M.moe_gptq_act_order_sort(d.qweight, torch.from_numpy(w.g_idx).to(dev),
                                               w.group)
        torch.cuda.synchronize()
        assert not st.any().item()
        d.qweight, d.k_perm = qs, kp
        return d

    fams = {"plain": (up(Lp.w13), up(Lp.w2)), "act_order": (prep(La.w13), prep(La.w2))}
    x = torch.from_numpy(Lp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(Lp.logits).to(dev)
    ws = torch.empty((M.moe_forward_workspace_bytes(max(ts), Lp.E, Lp.top_k, Lp.H, Lp.I),),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((max(ts), Lp.H), dtype=torch.bfloat16, device=dev)
    rows = []
    for T in ts:
        r = {"T": T}
        for name, (w13, w2) in fams.items():
            def f(i, w13=w13, w2=w2):
                M.moe_forward(x[:T], logits[:T], Lp.top_k, Lp.I, w13, w2, act=Lp.act,
                              route=Lp.route, renormalize=Lp.renormalize, alpha=Lp.alpha,
                              beta=Lp.beta, limit=Lp.limit, mul_topk_weights=Lp.mul_topk_weights,
                              workspace=ws, out=out[:T])
            r[f"{name}_us"] = time_calls(f, max(args.steps, 20), args.warmup) * 1e3
        # the gather of GEMM1's input alone: x rows -> one permuted row per slot
        ids = M.moe_route(logits[:T], Lp.top_k, Lp.route, None, Lp.renormalize)[0].reshape(-1)
        kp = fams["act_order"][0].k_perm
        xp = torch.empty((T * Lp.top_k, Lp.H), dtype=torch.bfloat16, device=dev)
        # (one event pair around each launch: back to back, the binding's host
        # time per call would exceed the few microseconds of the kernel)
        g_ms = time_launches(lambda i: M.moe_permute_slots(x[:T], Lp.top_k, kp, ids, out=xp),
                             max(args.steps, 20), args.warmup)[0]
        touched = len(set(ids.cpu().numpy().tolist()))
        nb = T * Lp.H * 2 + T * Lp.top_k * Lp.H * 2 + touched * Lp.H * 4
        r.update(gather_us=g_ms * 1e3, gather_alg_bytes=nb,
                 gather_GBps=nb / (g_ms * 1e-3) / 1e9,
                 gather_hbm_frac=nb / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 overhead_frac=r["act_order_us"] / r["plain_us"] - 1.0)
        log(f"act-order T={T}: plain {r['plain_us']:.1f} us, act-order {r['act_order_us']:.1f} us "
            f"(+{r['overhead_frac'] * 100:.1f}%), gather alone {r['gather_us']:.1f} us "
            f"{r['gather_GBps']:.0f} GB/s")
        rows.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
    return {"workload": "gpt-oss-20b-shaped MoE layer, INT4-GPTQ g64 (E=32, top_k=4, 2880/2880), "
                        "plain vs activation-order weights", "rows": rows}


FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s (e4m3 x e2m1 runs at the fp8 rate)


def mxfp8_leg(args, time_calls):
    """gpt-oss-120b-shaped MXFP4 layer: bf16 vs MXFP8 activations, and GEMM1 alone."""
    import torch
    import synthetic as S
    import bit_weight_expert_amd as M

    ts = [int(t) for t in args.mxfp8_tokens.split(",") if t]
    t0 = time.time()
    L = S.make_config(4)
    log(f"mxfp8 leg: generated the {S.CONFIGS[4]['name']} inputs in {time.time() - t0:.1f}s")
    dev = torch.device("cuda")
    copies = []
    for _ in range(max(1, min(args.copies, 3))):   # 3 x 2.4 GB: each call misses the 256 MB cache
        # chunked-only families, as the bf16 legs hold them (the MX kernels read
        # the codes and scales by 128-deep K chunk)
        copies.append(tuple(M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight,
                                                       w.scales, None, None, w.bias).chunked_only()
                            for w in (L.w13, L.w2)))
    x = torch.from_numpy(L.x.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(L.logits).to(dev)
    tmax = max(ts)
    ws = torch.empty((max(M.moe_forward_mxfp8_workspace_bytes(tmax, L.E, L.top_k, L.H, L.I),
                          M.moe_forward_workspace_bytes(tmax, L.E, L.top_k, L.H, L.I)),),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((tmax, L.H), dtype=torch.bfloat16, device=dev)
    rows = []
    for T in ts:
        r = {"T": T, "block_m": M.moe_forward_block_m(T, L.top_k, L.E)}
        for name, fn in (("bf16", M.moe_forward), ("mxfp8", M.moe_forward_mxfp8)):
            def f(i, fn=fn):
                w13, w2 = copies[i % len(copies)]
                fn(x[:T], logits[:T], L.top_k, L.I, w13, w2, act=L.act, route=L.route,
                   renormalize=L.renormalize, alpha=L.alpha, beta=L.beta, limit=L.limit,
                   mul_topk_weights=L.mul_topk_weights, workspace=ws, out=out[:T])
            r[f"{name}_us"] = time_calls(f, max(args.steps, 20), args.warmup) * 1e3
        r["speedup"] = r["bf16_us"] / r["mxfp8_us"]
        if r["block_m"] >= 64:
            # GEMM1 alone on the MX-scaled matrix cores
            bm = r["block_m"]
            ids, tw, si, ei, npp = M.moe_route_align(logits[:T], L.top_k, bm, L.route, None,
                                                     L.renormalize)
            xc, xs, _ = M.moe_mxfp8_quantize(x[:T])
            act = torch.empty((T * L.top_k, L.I), dtype=torch.bfloat16, device=dev)
            g_ms = time_calls(lambda i: M.moe_mx_gemm1(xc, xs, L.top_k, L.H, copies[i % len(copies)][0],
                                                       L.act, L.alpha, L.beta, L.limit, si, ei, npp,
                                                       bm, out=act), max(args.steps, 20), args.warmup)
            fl = 2.0 * T * L.top_k * L.H * L.w13.N
            r.update(gemm1_us=g_ms * 1e3, gemm1_TFLOPs=fl / (g_ms * 1e-3) / 1e12,
                     gemm1_fp8_frac=fl / (g_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS)
        log(f"mxfp8 T={T}: bf16 {r['bf16_us']:.1f} us, mxfp8 {r['mxfp8_us']:.1f} us "
            f"(x{r['speedup']:.2f})" + (f", MX GEMM1 {r['gemm1_us']:.1f} us = {r['gemm1_TFLOPs']:.0f} "
                                        f"TFLOP/s ({r['gemm1_fp8_frac'] * 100:.1f}% of fp8)"
                                        if "gemm1_us" in r else ""))
        rows.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
    return {"workload": "gpt-oss-120b-shaped MoE layer, MXFP4 weights (E=128, top_k=4, 2880/2880, "
                        "skewed routing), bf16 vs MXFP8 activations", "rows": rows}


def upload_copies(L, n, chunked=True, codes=True):
    """n device copies of the layer's two weight families (the same bytes);
    NVFP4 and MXFP4 families also get the load-time scales by K chunk and,
    with `codes`, the codes by K chunk."""
    import bit_weight_expert_amd as M
    copies = []
    for _ in range(n):
        pair = []
        for w in (L.w13, L.w2):
            d = M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales, w.zeros,
                                           w.global_scale, w.bias)
            kc_ok = w.fmt == "mxfp4" or (w.fmt == "nvfp4" and w.K % 64 == 0)
            if chunked and kc_ok and codes:
                d = d.chunked_only()            # the checkpoint copy is freed here
            elif chunked and kc_ok:
                d.scales_kc = (M.moe_nvfp4_scales_by_chunk(d) if w.fmt == "nvfp4"
                               else M.moe_mxfp4_scales_by_chunk(d))
            pair.append(d)
        copies.append(tuple(pair))
    return copies


def copies_for(L, ids_small) -> int:
    """Copies whose touched experts together exceed the last-level cache at the
    smallest batch of a sweep (so every call streams its weights from HBM)."""
    touched = max(1, len(np.unique(ids_small)))
    per_copy = touched * alg_bytes_per_expert(L)
    return int(min(8, max(2, -(-2 * LLC_BYTES // per_copy))))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--sweep", default="1,8,64,512,4096")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--cpu-sample", type=int, default=4096, help="tokens the oracle is timed on")
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph replay timings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other four workloads (GPTQ, gpt-oss-120b MXFP4, Nemotron, tiny)")
    ap.add_argument("--configs", default="3,4,5", help="the other workloads to time")
    ap.add_argument("--kernels", action="store_true",
                    help="also time GEMM1 and GEMM2 alone at every T of the headline sweep")
    ap.add_argument("--checkpoint-scales", action="store_true",
                    help="run on the checkpoint layout only (no scales or codes by K chunk)")
    ap.add_argument("--no-codes-by-chunk", action="store_true",
                    help="scales by K chunk only: the codes stay in the checkpoint layout")
    ap.add_argument("--act-order", action="store_true",
                    help="also time the GPTQ layer with act-order weights (and its gather)")
    ap.add_argument("--act-order-tokens", default="1,64,2048")
    ap.add_argument("--mxfp8", action="store_true",
                    help="also time the MXFP4 layer with MXFP8 activations")
    ap.add_argument("--mxfp8-tokens", default="1,128,1024,8192")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer "
              "is not sharded across GPUs by this library.", file=sys.stderr)
        return 2

    import torch
    import synthetic as S
    import bit_weight_expert_amd as M

    M.lib()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda")

    def time_calls(fn, steps, warmup):
        """ms per call of `steps` back-to-back calls, bracketed by synchronisation."""
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    def time_launches(fn, steps, warmup):
        """Mean duration (ms) of single launches, one event pair around each on the
        current stream (the stream the library launches on)."""
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i, (a, b) in enumerate(evs):
            a.record()
            fn(i)
            b.record()
        torch.cuda.synchronize()
        d = [a.elapsed_time(b) for a, b in evs]
        return sum(d) / len(d), statistics.median(d)

    def layer_leg(L, ts, copies, steps, graph=False, mxfp8=False):
        """Per-T rows of moe_forward over the layer's first T tokens."""
        x = torch.from_numpy(L.x.view(np.int16)).to(dev).view(torch.bfloat16)
        logits = torch.from_numpy(L.logits).to(dev)
        eb = None if L.expert_bias is None else torch.from_numpy(L.expert_bias).to(dev)
        ids_all = M.moe_route(logits, L.top_k, L.route, eb, L.renormalize)[0].cpu().numpy()
        tmax = max(ts)
        ws = torch.empty((M.moe_forward_workspace_bytes(tmax, L.E, L.top_k, L.H, L.I),),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((tmax, L.H), dtype=torch.bfloat16, device=dev)
        rows = []
        for T in ts:
            def fwd(i, T=T):
                w13, w2 = copies[i % len(copies)]
                M.moe_forward(x[:T], logits[:T], L.top_k, L.I, w13, w2, act=L.act, route=L.route,
                              expert_bias=eb, renormalize=L.renormalize, alpha=L.alpha,
                              beta=L.beta, limit=L.limit, mul_topk_weights=L.mul_topk_weights,
                              workspace=ws, out=out[:T])
            ms = time_calls(fwd, steps if T == tmax else max(steps, 50), args.warmup)
            r = roofline_row(L, T, ids_all[:T], ms)
            r["block_m"] = M.moe_forward_block_m(T, L.top_k, L.E)
            if graph:
                graphs = []
                for c in range(len(copies)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        fwd(c)
                    graphs.append(g)
                g_ms = time_calls(lambda i: graphs[i % len(graphs)].replay(), max(steps, 50),
                                  args.warmup)
                del graphs
                r["graph_ms"] = g_ms
                r["graph_roofline_frac"] = r["roofline_frac"] * ms / g_ms
            rows.append(r)
            log(f"  T={T}: {ms * 1e3:.1f} us/step, {r['tokens_per_s']:.0f} tok/s, "
                f"{r['GBps']:.0f} GB/s, {r['TFLOPs']:.1f} TFLOP/s, {r['bound']} roofline "
                f"{r['roofline_frac'] * 100:.1f}% (block_m {r['block_m']}, "
                f"{r['touched_experts']} experts)")
        return rows, (x, logits, eb, ids_all)

    # ---------------------------------------------------------------- headline
    sweep = sorted(set(int(t) for t in args.sweep.split(",") if t) | {args.tokens})
    t0 = time.time()
    L = S.make_config(2)
    assert L.T >= max(sweep)
    log(f"generated the {S.CONFIGS[2]['name']} inputs in {time.time() - t0:.1f}s")
    copies = upload_copies(L, args.copies, chunked=not args.checkpoint_scales,
                           codes=not args.no_codes_by_chunk)
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"{S.CONFIGS[2]['name']}:")
    rows, (x, logits, _, ids_all) = layer_leg(L, sweep, copies, args.steps, graph=not args.no_graph)
    results = {r["T"]: r for r in rows}

    def gemm_alone(T, which):
        """(mean, median) launch ms of GEMM1 or GEMM2 alone at T, rotating copies, on
        the aligned blocks of moe_forward's tile size."""
        bm = M.moe_forward_block_m(T, L.top_k, L.E)
        ids_t, w_t = M.moe_route(logits[:T], L.top_k, L.route, None, L.renormalize)
        si, ei, npp = M.moe_align(ids_t, L.E, bm)
        act_buf = torch.zeros((T * L.top_k, L.I), dtype=torch.bfloat16, device=dev)
        y_buf = torch.empty((T * L.top_k, L.H), dtype=torch.bfloat16, device=dev)
        tw = w_t.reshape(-1).contiguous()
        if which == 1:
            f = lambda i: M.moe_w4a16_gemm1(x[:T], L.top_k, copies[i % len(copies)][0], L.act,
                                            L.alpha, L.beta, L.limit, si, ei, npp, bm, out=act_buf)
        else:
            f = lambda i: M.moe_w4a16_gemm2(act_buf, copies[i % len(copies)][1], tw, True, si, ei,
                                            npp, bm, out=y_buf)
        return time_launches(f, max(args.steps, 20), args.warmup)

    # dominant kernel at the headline T: GEMM1, each launch timed on its stream
    T = args.tokens
    g1_mean, g1_med = gemm_alone(T, 1)
    gb, gf = gemm1_alg(L, T, ids_all[:T])
    g_bound = "hbm" if gb / (HBM_PEAK_GBS * 1e9) >= gf / (BF16_PEAK_TFLOPS * 1e12) else "mfma"
    if g_bound == "mfma":
        achieved, peak, unit = gf / (g1_mean * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = gb / (g1_mean * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    log(f"gemm1 alone at T={T}: mean launch {g1_mean * 1e3:.1f} us (median {g1_med * 1e3:.1f}), "
        f"{achieved:.1f} {unit} ({achieved / peak * 100:.1f}%)")
    kernels = None
    if args.kernels:
        kernels = []
        for t in sweep:
            m1, _ = gemm_alone(t, 1)
            m2, _ = gemm_alone(t, 2)
            b1, _ = gemm1_alg(L, t, ids_all[:t])
            touched = len(np.unique(ids_all[:t]))
            w2 = L.w2
            b2 = touched * (w2.qweight[0].nbytes + w2.scales[0].nbytes + 4 +
                            (w2.bias[0].nbytes if w2.bias is not None else 0)) + \
                t * L.top_k * (L.I + L.H) * 2
            kernels.append(dict(T=t, gemm1_us=m1 * 1e3, gemm1_alg_bytes=b1,
                                gemm1_GBps=b1 / (m1 * 1e-3) / 1e9, gemm2_us=m2 * 1e3,
                                gemm2_alg_bytes=b2, gemm2_GBps=b2 / (m2 * 1e-3) / 1e9))
            log(f"  kernels T={t}: gemm1 {m1 * 1e3:.1f} us ({b1 / (m1 * 1e-3) / 1e9:.0f} GB/s), "
                f"gemm2 {m2 * 1e3:.1f} us ({b2 / (m2 * 1e-3) / 1e9:.0f} GB/s)")
    head = results[args.tokens]
    del copies
    torch.cuda.empty_cache()

    # ---------------------------------------------------------- other configs
    configs = {}
    if not args.no_configs:
        for cfg in [int(c) for c in args.configs.split(",") if c]:
            c = S.CONFIGS[cfg]
            t0 = time.time()
            Lc = S.make_config(cfg)
            log(f"{c['name']} (generated in {time.time() - t0:.1f}s):")
            ts = list(c["T"])
            # copies: enough that the smallest batch's touched experts exceed the cache
            lg = torch.from_numpy(Lc.logits[:min(ts)]).to(dev)
            eb = None if Lc.expert_bias is None else torch.from_numpy(Lc.expert_bias).to(dev)
            ids_small = M.moe_route(lg, Lc.top_k, Lc.route, eb, Lc.renormalize)[0].cpu().numpy()
            cps = upload_copies(Lc, copies_for(Lc, ids_small), chunked=not args.checkpoint_scales,
                                codes=not args.no_codes_by_chunk)
            crow, _ = layer_leg(Lc, ts, cps, args.steps)
            configs[f"config{cfg}"] = {"workload": c["name"], "weight_copies_rotated": len(cps),
                                       "rows": [{k: (round(v, 6) if isinstance(v, float) else v)
                                                 for k, v in r.items()} for r in crow]}
            del cps, Lc
            torch.cuda.empty_cache()

    # ------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe as O
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            blas_threads = 1
        n = min(args.cpu_sample, args.tokens)
        Ls = L.take(n)
        times = []
        for _ in range(max(1, args.cpu_runs)):
            t0 = time.time()
            O.forward(Ls)
            times.append(time.time() - t0)
        dt = statistics.median(times)
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
               "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
               "runs_s": [round(t, 3) for t in times],
               "sample": f"first {n} tokens of the T={args.tokens} batch of the headline workload, "
                         f"whole layer (route, align, float64 dequant of every touched expert, "
                         f"both GEMMs, sum); median of {len(times)} runs; BLAS threads = cores"}
        log(f"oracle: {n} tokens, median {dt:.1f}s of {len(times)} runs, {blas_threads} BLAS threads")

    act_order = act_order_leg(args, time_calls, time_launches) if args.act_order else None
    mxfp8 = mxfp8_leg(args, time_calls) if args.mxfp8 else None

    line = {
        "metric": "fused W4A16 MoE layer tokens/s + % HBM/MFMA roofline, E32 top4 h2880",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gpt-oss-20b-shaped MoE layer: E=32, top_k=4, hidden=2880, "
                               "intermediate=2880, NVFP4 g16 weights + bias, swigluoai, "
                               f"T={args.tokens} tokens",
                   "tokens": args.tokens, "block_m": head["block_m"],
                   "weight_copies_rotated": args.copies,
                   "scales_by_chunk": not args.checkpoint_scales,
                   "codes_by_chunk": not (args.checkpoint_scales or args.no_codes_by_chunk),
                   "checkpoint_codes_resident": args.checkpoint_scales or args.no_codes_by_chunk},
        "roofline": {"kernel": "grouped GEMM1 (w13 + bias + swigluoai), gemm_prefill_kernel",
                     "bound": g_bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": profiled_traffic(),
                     "kernel_us": g1_mean * 1e3, "kernel_us_median": g1_med * 1e3,
                     "alg_bytes": gb, "alg_flops": gf},
        "layer_roofline": {"bound": head["bound"], "frac": head["roofline_frac"],
                           "GBps": head["GBps"], "TFLOPs": head["TFLOPs"]},
        "cpu_baseline": cpu,
        "sweep": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in results[t].items()}
                  for t in sweep],
        "configs": configs or None,
        "kernels": kernels,
        "act_order": act_order,
        "mxfp8": mxfp8,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Throughput of the fused W4A16 MoE layer on one MI355X.

Workload: the gpt-oss-20b-shaped MoE layer -- E=32 experts, top-4, hidden =
intermediate = 2880, NVFP4 (e2m1 + e4m3 scale per 16 + fp32 global scale)
weights, per-expert biases, swigluoai, routing weight applied in GEMM2's
epilogue -- on synthetic inputs (seeded; see synthetic/).  One step is one
moe_forward call (route -> align -> GEMM1 -> GEMM2 -> sum) over a batch of T
tokens with everything already resident in HBM.  The headline line is at
T = 4096; the same JSON line carries the other token counts of the sweep.

Weight copies are rotated between calls so that no call finds its weights in
the 256 MB last-level cache left behind by the previous one.  The weights are
loaded as a user of the library loads them: the checkpoint bytes plus the
NVFP4 scales and codes re-laid by K chunk (moe_nvfp4_scales_by_chunk and
moe_nvfp4_codes_by_chunk, done once at load time; the token counts up to 64
read the checkpoint codes).  --checkpoint-codes runs without the codes copy,
--checkpoint-scales without either.

Prints ONE JSON line.  --gpus N > 1 is refused: this build runs on one GPU.

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
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes_per_expert(L) -> int:
    """Bytes one touched expert must stream: 4-bit codes, scales, global scale, biases."""
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
    """(bytes, flops) the layer must move / compute for T tokens with routing ids."""
    touched = len(np.unique(ids[(ids >= 0) & (ids < L.E)]))
    nbytes = touched * alg_bytes_per_expert(L) + T * L.H * 2 * 2 + T * L.E * 4
    n1 = L.N1
    flops = 2 * T * L.top_k * L.H * (n1 + L.I)
    return nbytes, flops, touched


def gemm1_alg(L, T, ids):
    touched = len(np.unique(ids))
    w = L.w13
    b = touched * (w.qweight[0].nbytes + w.scales[0].nbytes + 4 + (w.bias[0].nbytes if w.bias is not None else 0))
    b += T * L.H * 2 + T * L.top_k * L.I * 2
    f = 2 * T * L.top_k * L.H * L.N1
    return b, f


def profiled_traffic():
    """GEMM1 HBM bytes per launch from the committed counter summary, or None.

    The summary records the GEMM source it was taken on; if the source has
    changed since, the figure no longer describes this kernel and None is
    returned.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm1_nvfp4_e32_t4096_traffic.md")
    src = os.path.join(ROOT, "bit_weight_expert_amd", "csrc", "gemm.hip")
    try:
        fields = dict(ln.split(":", 1) for ln in open(path) if ln.startswith(("traffic_", "kernel_")))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if not sha.startswith(fields["kernel_source_sha256_prefix"].strip()):
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def act_order_leg(args, time_calls):
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
        g_ms = time_calls(lambda i: M.moe_permute_slots(x[:T], Lp.top_k, kp, ids, out=xp),
                          max(args.steps, 20), args.warmup)
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
        pair = tuple(M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales,
                                                None, None, w.bias) for w in (L.w13, L.w2))
        for w in pair:   # the MX kernels' copy of the codes by 128-deep K chunk (load time)
            w.qweight_kc = M.moe_mxfp4_codes_by_chunk(w)
        copies.append(pair)
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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--sweep", default="1,8,64,512,4096")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--cpu-sample", type=int, default=4096, help="tokens the oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph replay timings")
    ap.add_argument("--checkpoint-scales", action="store_true",
                    help="run on the checkpoint layout only (no scales or codes by K chunk)")
    ap.add_argument("--checkpoint-codes", action="store_true",
                    help="scales by K chunk, codes in the checkpoint layout only")
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
              "is not sharded across GPUs in this build.", file=sys.stderr)
        return 2

    import torch
    import synthetic as S
    import bit_weight_expert_amd as M

    M.lib()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1

    sweep = sorted(set(int(t) for t in args.sweep.split(",") if t) | {args.tokens})
    t_max = max(sweep)
    t0 = time.time()
    L = S.make_config(2)
    assert L.T >= t_max
    log(f"generated the {S.CONFIGS[2]['name']} inputs in {time.time() - t0:.1f}s")

    dev = torch.device("cuda")
    x = torch.from_numpy(L.x.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(L.logits).to(dev)
    copies = []
    for r in range(args.copies):
        w13 = M.QuantWeights.from_arrays(L.w13.fmt, L.w13.group, L.w13.N, L.w13.K, L.w13.qweight,
                                         L.w13.scales, None, L.w13.global_scale, L.w13.bias)
        w2 = M.QuantWeights.from_arrays(L.w2.fmt, L.w2.group, L.w2.N, L.w2.K, L.w2.qweight,
                                        L.w2.scales, None, L.w2.global_scale, L.w2.bias)
        if not args.checkpoint_scales:
            # the load-time layout of the NVFP4 scales by K chunk (a copy of the
            # same bytes), which the 64/128-row GEMM kernel streams with the codes
            w13.scales_kc = M.moe_nvfp4_scales_by_chunk(w13)
            w2.scales_kc = M.moe_nvfp4_scales_by_chunk(w2)
            if not args.checkpoint_codes:
                # and the codes: a second copy, read by the same kernel
                w13.qweight_kc = M.moe_nvfp4_codes_by_chunk(w13)
                w2.qweight_kc = M.moe_nvfp4_codes_by_chunk(w2)
        copies.append((w13, w2))
    ws = torch.empty((M.moe_forward_workspace_bytes(t_max, L.E, L.top_k, L.H, L.I),),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((t_max, L.H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def fwd(T, i):
        w13, w2 = copies[i % len(copies)]
        M.moe_forward(x[:T], logits[:T], L.top_k, L.I, w13, w2, act=L.act, route=L.route,
                      renormalize=L.renormalize, alpha=L.alpha, beta=L.beta, limit=L.limit,
                      mul_topk_weights=L.mul_topk_weights, workspace=ws, out=out[:T])

    def time_calls(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps  # ms per call

    # routing ids of the batch (for the algorithmic byte counts: touched experts)
    ids_all = M.moe_route(logits, L.top_k, L.route, None, L.renormalize)[0].cpu().numpy()

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def graph_ms(T, steps):
        """Per-call time of moe_forward replayed from hipGraphs (one graph per weight copy)."""
        graphs = []
        for r in range(len(copies)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fwd(T, r)
            graphs.append(g)
        ms = time_calls(lambda i: graphs[i % len(graphs)].replay(), steps, args.warmup)
        del graphs
        return ms

    results = {}
    for T in sweep:
        steps = args.steps if T == args.tokens else max(args.steps, 50)
        ms = time_calls(lambda i: fwd(T, i), steps, args.warmup)
        g_ms = None if args.no_graph else graph_ms(T, steps)
        nb, fl, touched = algorithmic(L, T, ids_all[:T])
        t_hbm = nb / (HBM_PEAK_GBS * 1e9)
        t_mfma = fl / (BF16_PEAK_TFLOPS * 1e12)
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        results[T] = dict(T=T, ms=ms, tokens_per_s=T / (ms * 1e-3), touched_experts=touched,
                          graph_ms=g_ms,
                          graph_roofline_frac=None if g_ms is None else max(t_hbm, t_mfma) / (g_ms * 1e-3),
                          alg_bytes=nb, alg_flops=fl, GBps=nb / (ms * 1e-3) / 1e9,
                          TFLOPs=fl / (ms * 1e-3) / 1e12, bound=bound,
                          roofline_frac=max(t_hbm, t_mfma) / (ms * 1e-3))
        log(f"T={T}: {ms * 1e3:.1f} us/step (graph {('%.1f' % (g_ms * 1e3)) if g_ms else '-'}), "
            f"{results[T]['tokens_per_s']:.0f} tok/s, "
            f"{results[T]['GBps']:.0f} GB/s, {results[T]['TFLOPs']:.1f} TFLOP/s, "
            f"{bound} roofline {results[T]['roofline_frac'] * 100:.1f}%")

    # dominant kernel at the headline T: GEMM1, timed alone on the same stream
    T = args.tokens
    bm = M.moe_forward_block_m(T, L.top_k, L.E)
    ids_t, w_t = M.moe_route(logits[:T], L.top_k, L.route, None, L.renormalize)
    si, ei, npp = M.moe_align(ids_t, L.E, bm)
    act_buf = torch.empty((T * L.top_k, L.I), dtype=torch.bfloat16, device=dev)

    def g1(i):
        w13 = copies[i % len(copies)][0]
        M.moe_w4a16_gemm1(x[:T], L.top_k, w13, L.act, L.alpha, L.beta, L.limit, si, ei, npp, bm,
                          out=act_buf)

    g1_ms = time_calls(g1, args.steps, args.warmup)
    gb, gf = gemm1_alg(L, T, ids_all[:T])
    g_bound = "hbm" if gb / (HBM_PEAK_GBS * 1e9) >= gf / (BF16_PEAK_TFLOPS * 1e12) else "mfma"
    if g_bound == "mfma":
        achieved, peak, unit = gf / (g1_ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = gb / (g1_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    log(f"gemm1 alone at T={T}: {g1_ms * 1e3:.1f} us, {achieved:.1f} {unit} ({achieved / peak * 100:.1f}%)")

    # headline: the timed K steps at T = args.tokens, bracketed by synchronisation
    head = results[args.tokens]

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe as O
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            blas_threads = 1
        n = min(args.cpu_sample, T)
        t0 = time.time()
        O.forward(L.take(n))
        dt = time.time() - t0
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
               "sample": f"first {n} tokens of the T={T} batch, whole layer (route, align, float64 "
                         f"dequant of every touched expert, both GEMMs, sum); {dt:.1f}s wall"}
        log(f"oracle: {n} tokens in {dt:.1f}s")

    act_order = act_order_leg(args, time_calls) if args.act_order else None
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
                   "tokens": args.tokens, "block_m": bm, "weight_copies_rotated": args.copies,
                   "nvfp4_scales_by_chunk": not args.checkpoint_scales,
                   "nvfp4_codes_by_chunk": not (args.checkpoint_scales or args.checkpoint_codes)},
        "roofline": {"kernel": "grouped_gemm (GEMM1, w13 + swigluoai)", "bound": g_bound,
                     "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                     "traffic": profiled_traffic(), "kernel_us": g1_ms * 1e3},
        "layer_roofline": {"bound": head["bound"], "frac": head["roofline_frac"],
                           "GBps": head["GBps"], "TFLOPs": head["TFLOPs"]},
        "cpu_baseline": cpu,
        "act_order": act_order,
        "mxfp8": mxfp8,
        "sweep": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in results[t].items()}
                  for t in sweep],
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

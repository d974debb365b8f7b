"""Benchmark of the MoE FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skewed|hash|tiny]

One step = one call of moe_layer (route, quantize, routed experts, shared
expert, combine) over one batch of seeded synthetic input already resident in
HBM.  Prints ONE JSON line: whole-layer tokens/s of the decode batch (64
tokens), the roofline of its routed expert FFN (grouped GEMM1 + fused
SwiGLU/requant + GEMM2, timed with HIP events on the stream it runs on), the
prefill half of the metric (the same layer on 4096 tokens: tokens/s, routed
FFN TFLOP/s against the scaled-MFMA peak and its weight stream against HBM),
and the CPU oracle timed on a bounded token sample of the decode workload on
this host's cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_FP8_PEAK_TFLOPS = 5000.0    # dense FP8 (an FP4 x FP8 scaled MFMA issues at most at this rate)
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16
EXPERT_BYTES = None              # set from the workload
WEIGHT_COPIES = 2                # weight sets the timed calls rotate through


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="report graph replays of the layer (moe_graph_launch) as the step; "
                         "both are timed and reported either way")
    ap.add_argument("--experts", choices=("mxfp4", "fp8", "nvfp4", "w4afp8"), default="mxfp4",
                    help="routed expert weights: the MXFP4 checkpoint format, its per-128 "
                         "cast to FP8 (made on the GPU before timing), NVFP4 (the same "
                         "nibbles with synthetic per-16 E4M3 scales) or W4AFP8 (the nibbles "
                         "as INT4 with synthetic float32 scales per 128)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 4096-token prefill measurement that the decode line carries")
    ap.add_argument("--prefill-steps", type=int, default=30)
    return ap.parse_args()


def algorithmic(wl, n_touched, fmt="mxfp4"):
    """Bytes and flops the layer must move / compute (no padding, no
    intermediates): weights of the touched experts (FP4 nibbles + E8M0
    scales per 32 of w1, w3, w2; FP8 experts: E4M3 bytes + E8M0 per 128;
    NVFP4: nibbles + E4M3 per 16; W4AFP8: INT4 nibbles + float32 per 128),
    the bf16 shared expert and gate, x in, y out.  The routed expert FFN's
    share is the touched experts' weights: its FP8 activations, h and the
    per-pair outputs are intermediates of the layer, overhead rather than
    work."""
    T, H, I, E, k = wl.tokens, wl.hidden, wl.inter, wl.n_experts, wl.top_k
    per_expert = {"mxfp4": 3 * (I * H // 2 + I * H // 32), "fp8": 3 * (I * H + I * H // 128),
                  "nvfp4": 3 * (I * H // 2 + I * H // 16),
                  "w4afp8": 3 * (I * H // 2 + 4 * (I * H // 128))}[fmt]
    ffn_bytes = n_touched * per_expert
    shared = 3 * I * H * 2 if wl.shared else 0
    gate = E * H * 2 if wl.mode != "hash" else 0
    layer_bytes = n_touched * per_expert + shared + gate + 2 * T * H * 2
    flops_routed = 6 * T * k * H * I
    flops_shared = 6 * T * H * I if wl.shared else 0
    flops_router = 2 * T * H * E if wl.mode != "hash" else 0
    return dict(per_expert=per_expert, ffn_bytes=ffn_bytes, layer_bytes=layer_bytes,
                flops_routed=flops_routed, flops_shared=flops_shared, flops_router=flops_router)


def traffic_record(kernel_src_hash, workload):
    """HBM traffic of the routed expert FFN measured with rocprofv3 --pmc
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy kernel), if the record
    was taken on this workload and on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"expert_ffn_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("expert_gemm_src_sha256") != kernel_src_hash:
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(wl, inp, budget_s=20.0, weight_format="mxfp4"):
    """The oracle as it stands on a bounded token sample: as many tokens of
    the workload as fit in about budget_s seconds (at least one)."""
    import numpy as np
    from oracle import ffn
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    done, t_used, n = 0, 0.0, 1
    rng = np.random.default_rng(7)
    while t_used < budget_s and done < wl.tokens:
        n = min(n, wl.tokens - done)
        S = np.sort(rng.choice(wl.tokens, n, replace=False))
        sub = dict(inp)
        sub["x"] = inp["x"][S]
        sub["token_ids"] = inp["token_ids"][S]
        t0 = time.perf_counter()
        ffn.layer(sub, wl.top_k, wl.route_scale, wl.swiglu_limit, wl.mode, wl.seed,
                  weight_format=weight_format)
        dt = time.perf_counter() - t0
        done += n
        t_used += dt
        if dt < budget_s / 4:
            n *= 2
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": done / t_used, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{done} tokens of the {wl.name} workload (T={wl.tokens}), whole layer incl. "
                      f"routing and dequantization, {t_used:.1f} s"}


def measure(args, wl, steps, with_graph=True, with_cpu=False):
    """Times the layer (eager calls, and replays of the same call captured
    into a HIP graph) and the routed expert FFN alone on workload `wl`.
    Returns a dict of figures; the caller frees the inputs with it."""
    import ctypes

    import numpy as np
    import torch

    import block_scaled_fp4_sqrtsoftplus_amd as moe
    import synth

    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = synth.make_inputs(wl)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf(a):
        return d(a.view(np.int16)).view(torch.bfloat16)

    x = bf(inp["x"])
    w = {n: d(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    wg = bf(inp["w_gate"]) if wl.mode != "hash" else None
    bias = d(inp["bias"]) if inp.get("bias") is not None else None
    ids = d(inp["token_ids"])
    shared = ({"w1": bf(inp["shared_w1"]), "w3": bf(inp["shared_w3"]), "w2": bf(inp["shared_w2"])}
              if wl.shared else None)
    cfg = moe.Config(tokens=wl.tokens, hidden=wl.hidden, inter=wl.inter, n_experts=wl.n_experts,
                     top_k=wl.top_k, route_scale=wl.route_scale, swiglu_limit=wl.swiglu_limit,
                     route_mode=moe.ROUTE_HASH if wl.mode == "hash" else moe.ROUTE_SQRTSOFTPLUS,
                     hash_seed=wl.seed)
    if args.experts == "fp8":
        w = moe.expert_cast_fp8(cfg, w)
        cfg.expert_format = moe.EXPERTS_FP8
        torch.cuda.synchronize()
    if args.experts == "nvfp4":
        inp.update(synth.nvfp4_scales(wl))
        for n in ("w1_scale", "w3_scale", "w2_scale"):
            w[n] = d(inp[n])
        cfg.expert_format = moe.EXPERTS_NVFP4
    if args.experts == "w4afp8":
        inp.update(synth.w4afp8_scales(wl))
        for n in ("w1_scale", "w3_scale", "w2_scale"):
            w[n] = d(inp[n])
        cfg.expert_format = moe.EXPERTS_W4AFP8
    # Two copies of every weight (experts, gate, shared expert), used in
    # turn: no weight byte one timed call reads is still in the caches for the
    # next, as in a model whose consecutive layers have different weights
    # (with one copy, back-to-back calls read ~3% of the decode weights from
    # the last-level cache of the call before).
    clone = lambda t: None if t is None else t.clone()
    ws_copies = [w, {n: t.clone() for n, t in w.items()}]
    wg_copies = [wg, clone(wg)]
    sh_copies = [shared, None if shared is None else {n: t.clone() for n, t in shared.items()}]
    layers = [moe.Layer(cfg, ws_copies[i], w_gate=wg_copies[i], bias=bias, shared=sh_copies[i])
              for i in range(WEIGHT_COPIES)]
    y = torch.empty((wl.tokens, wl.hidden), dtype=torch.bfloat16, device=dev)
    routing = moe._routing_tensors(wl.tokens, wl.top_k, wl.n_experts, dev)
    print(f"[bench] {wl.name}: inputs ready in {time.time() - t0:.1f}s: {wl}", file=sys.stderr,
          flush=True)

    def timed(step_fn, n):
        for _ in range(args.warmup):
            step_fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start = time.perf_counter()
        ev0.record()
        for _ in range(n):
            step_fn()
        ev1.record()
        torch.cuda.synchronize()
        return (time.perf_counter() - t_start) * 1e3 / n, ev0.elapsed_time(ev1) / n

    def rotating(fns):
        state = {"i": 0}

        def call():
            fns[state["i"] % len(fns)]()
            state["i"] += 1
        return call

    # whole layer: eager calls (the step), then replays of the same call
    # captured into a HIP graph (one graph per weight copy)
    eager_ms, eager_gpu_ms = timed(
        rotating([lambda L=L: L(x, ids, y=y, routing=routing) for L in layers]), steps)
    graph_ms = graph_gpu_ms = None
    if with_graph:
        graphs = [moe.LayerGraph(L, x, token_ids=ids, y=y, routing=routing) for L in layers]
        graph_ms, graph_gpu_ms = timed(rotating([g.launch for g in graphs]), steps)
        for g in graphs:
            g.close()
    load = np.diff(routing["expert_offsets"].cpu().numpy())
    n_touched = int(np.sum(load > 0))

    # routed expert FFN (grouped GEMM1 + fused SwiGLU/requant + GEMM2) on the
    # same routing, timed with events on the stream it is launched on (the
    # current stream: torch's events record there)
    xq, xs = moe.quant_act(x)
    ffn_out = torch.empty((wl.tokens * wl.top_k, wl.hidden), dtype=torch.float32, device=dev)
    ws_n = moe.workspace_size(cfg, moe.OP_EXPERT_FFN)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    cc, rc = cfg.c(), moe._routing_c(routing)
    wcs = [moe._weights_c(wi) for wi in ws_copies]

    def ffn_call(wc):
        st = moe.lib.moe_expert_ffn(ctypes.byref(cc), moe._ptr(xq), moe._ptr(xs), ctypes.byref(rc),
                                    ctypes.byref(wc), moe._ptr(ffn_out), None, None,
                                    moe._ptr(ws), ws_n, moe._stream())
        if st != 0:
            raise moe.MoeError(st)

    _, ffn_ms = timed(rotating([lambda wc=wc: ffn_call(wc) for wc in wcs]), steps)

    alg = algorithmic(wl, n_touched, args.experts)
    # the NVFP4 path dequantizes to fp16 and runs on the fp16 MFMA (the bf16 / fp16 peak)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if args.experts == "nvfp4" else MFMA_FP8_PEAK_TFLOPS
    ffn_gbs = alg["ffn_bytes"] / (ffn_ms * 1e-3) / 1e9
    ffn_tflops = alg["flops_routed"] / (ffn_ms * 1e-3) / 1e12
    layer_t_roof = max(alg["layer_bytes"] / (HBM_PEAK_GBS * 1e9),
                       alg["flops_routed"] / (mfma_peak * 1e12)
                       + alg["flops_shared"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                       + alg["flops_router"] / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    cpu = None
    if with_cpu:
        cpu = cpu_baseline(wl, inp, weight_format=args.experts)   # inp holds the NVFP4 / W4AFP8 scales then
    src_name = {"nvfp4": "expert_gemm_nv.hip", "w4afp8": "expert_gemm_w4.hip"}.get(args.experts, "expert_gemm.hip")
    src = open(os.path.join(ROOT, "block_scaled_fp4_sqrtsoftplus_amd", "csrc", src_name), "rb").read()
    traffic = traffic_record(hashlib.sha256(src).hexdigest(),
                             wl.name + ("" if args.experts == "mxfp4" else "_" + args.experts))
    small = wl.tokens * wl.top_k <= 32 * wl.n_experts
    fam = {"fp8": "expert_gemm_stream8" if small else "expert_gemm_tile",
           "nvfp4": "expert_gemm_nv", "w4afp8": "expert_gemm_w4",
           "mxfp4": "expert_gemm_stream" if small else "expert_gemm_tile"}[args.experts]
    if args.experts in ("nvfp4", "w4afp8"):
        kname = f"{fam}<1> + {fam}<2>"
    elif args.experts == "fp8" and not small:
        kname = f"{fam}<1,{wl.hidden // 128},true> + {fam}<2,{wl.inter // 128},true>"
    else:
        kname = f"{fam}<1,{wl.hidden // 128}> + {fam}<2,{wl.inter // 128}>"
    return {
        "wl": wl, "eager_ms": eager_ms, "eager_gpu_ms": eager_gpu_ms, "graph_ms": graph_ms,
        "graph_gpu_ms": graph_gpu_ms, "n_touched": n_touched,
        "max_over_mean_load": round(float(load.max() / max(load.mean(), 1e-9)), 2),
        "alg": alg, "ffn_ms": ffn_ms, "ffn_gbs": ffn_gbs, "ffn_tflops": ffn_tflops,
        "mfma_peak": mfma_peak, "layer_t_roof": layer_t_roof, "cpu": cpu, "traffic": traffic,
        "kernel": f"routed expert FFN: {kname} (+ tile prefix)",
    }


def workload_summary(m, launch="eager"):
    """Both roofline fractions of a measured workload: the layer against
    max(bytes / HBM, sum of flops / MFMA peaks), and the routed expert FFN
    against HBM (its weight stream) and against the scaled-MFMA peak."""
    wl = m["wl"]
    ms = m["graph_ms"] if launch == "graph" else m["eager_ms"]
    return {
        "workload": f"T={wl.tokens} H={wl.hidden} I={wl.inter} E={wl.n_experts} top-{wl.top_k}",
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1),
        "layer_roofline_frac": round(m["layer_t_roof"] / (ms * 1e-3), 4),
        "routed_ffn_ms": round(m["ffn_ms"], 4),
        "routed_ffn_tflops": round(m["ffn_tflops"], 1),
        "routed_ffn_mfma_frac": round(m["ffn_tflops"] / m["mfma_peak"], 4),
        "routed_ffn_weight_gbs": round(m["ffn_gbs"], 1),
        "routed_ffn_hbm_frac": round(m["ffn_gbs"] / HBM_PEAK_GBS, 4),
        "experts_touched": m["n_touched"],
        "max_over_mean_load": m["max_over_mean_load"],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU expert-parallel path is a design, not code)"}))
        sys.exit(2)

    import torch

    import synth

    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    steps = args.steps or {"tiny": 200, "decode": 100, "prefill": 30, "skewed": 10, "hash": 10}[wl.name]
    m = measure(args, wl, steps, with_graph=True, with_cpu=not args.no_cpu_baseline)
    launch = "graph" if args.graph else "eager"
    ms_step = m["graph_ms"] if args.graph else m["eager_ms"]
    gpu_ms_step = m["graph_gpu_ms"] if args.graph else m["eager_gpu_ms"]
    alg = m["alg"]

    hbm_bound = alg["ffn_bytes"] / (HBM_PEAK_GBS * 1e9) >= alg["flops_routed"] / (m["mfma_peak"] * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(m["ffn_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(m["ffn_gbs"] / HBM_PEAK_GBS, 4), "traffic": m["traffic"]}
    else:
        roof = {"bound": "mfma", "achieved": round(m["ffn_tflops"], 1), "peak": m["mfma_peak"],
                "unit": "TFLOP/s", "frac": round(m["ffn_tflops"] / m["mfma_peak"], 4),
                "traffic": m["traffic"]}
    roof["kernel"] = m["kernel"]
    roof["ms_per_call"] = round(m["ffn_ms"], 4)
    roof["alg_bytes_per_call"] = alg["ffn_bytes"]
    roof["alg_flops_per_call"] = alg["flops_routed"]
    layer = workload_summary(m, launch)
    layer.update({"launch": launch, "gpu_ms_per_step": round(gpu_ms_step, 4),
                  "eager_ms_per_step": round(m["eager_ms"], 4),
                  "graph_ms_per_step": round(m["graph_ms"], 4), "alg_bytes": alg["layer_bytes"],
                  "hbm_gbs": round(alg["layer_bytes"] / (ms_step * 1e-3) / 1e9, 1)})
    cpu = m["cpu"]
    del m
    torch.cuda.empty_cache()

    # the prefill half of the metric: the same layer on a 4096-token batch
    prefill = None
    if wl.name == "decode" and not args.no_prefill:
        mp = measure(args, synth.WORKLOADS["prefill"], args.prefill_steps, with_graph=False)
        prefill = workload_summary(mp)
        prefill["kernel"] = mp["kernel"]
        prefill["traffic"] = mp["traffic"]
        del mp
        torch.cuda.empty_cache()

    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        dev = torch.device("cuda:0")
        src_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst_buf = torch.empty_like(src_buf)
        for _ in range(3):
            dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf

    fp8 = args.experts == "fp8"
    value = wl.tokens / (ms_step * 1e-3)
    out = {
        "metric": "MoE layer tokens/s + % roofline (HBM GB/s decode, scaled-MFMA TFLOPS prefill)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8e4m3 x fp8e4m3 -> f32", "mxfp4": "fp4e2m1 x fp8e4m3 -> f32",
                  "nvfp4": "fp16(fp4e2m1 x e4m3 scale) x fp16(fp8e4m3) -> f32",
                  "w4afp8": "fp8e4m3(int4 + 8) x fp8e4m3 -> f32, f32 scale per 128"}[args.experts]
                 + " (experts); bf16 -> f32 (router, shared)",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": f"{wl.name}: T={wl.tokens} H={wl.hidden} I={wl.inter} E={wl.n_experts} "
                               f"top-{wl.top_k} {'hash' if wl.mode == 'hash' else 'sqrtsoftplus'} routing"
                               f"{' + bf16 shared expert' if wl.shared else ''}"
                               f"{', FP8 experts (per-128 cast of the MXFP4 weights)' if fp8 else ''}"
                               f"{', NVFP4 experts (per-16 E4M3 scales)' if args.experts == 'nvfp4' else ''}"
                               f"{', W4AFP8 experts (INT4, f32 scale per 128)' if args.experts == 'w4afp8' else ''}",
                   "tokens": wl.tokens, "experts_touched": layer["experts_touched"],
                   "max_over_mean_load": layer["max_over_mean_load"]},
        "layer": layer,
        "roofline": roof,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

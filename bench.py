"""Throughput of the Llama-70B-shape decoder-layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one forward of the whole layer (input_layernorm, qkv_proj, RoPE +
KV write, paged attention, o_proj + residual, post_attention_layernorm,
gate_up_proj + SiluAndMul, down_proj) over one batch of seeded synthetic
inputs that are resident in HBM before timing starts.  Default workload: 32
sequences decoding one token each after a 2048-token cached context (70B
layer shapes, bf16).  The extra lines measure the 70B prefill, the
Qwen3-MoE layer (the MLP replaced by the routed experts) and one GPU's TP = 8
share of the 70B layer (no all-reduce: one GPU).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
METRIC = "70B-shape layer tokens/s (prefill, decode) + % MFMA/HBM peak, 1 MI355X"

# HBM bytes per launch of a dominant kernel from rocprofv3 counters: FETCH_SIZE x 2.0 + WRITE_SIZE
# x 1.0 (factors from a plain 1 GiB copy; profiles/pmc_copy_calibration.md).  Reported only while
# the kernel's source file is the one the counters were taken on.
COUNTER_TRAFFIC = {
    ("qwen3moe_prefill_4x2048", "moe_gate_up_silu"): {
        "bytes": 1979509634,
        "source": "llama_decoder_layer_amd/csrc/moe.hip",
        "sha1": "755722e27b7a0844d60c7110d6ebca39ad3481fe",
        "summary": "profiles/moe_gate_up_silu_qwen3moe_prefill_4x2048_counters.md",
    },
    ("llama70b_tp8shard_prefill_4x2048", "gate_up_silu"): {
        "bytes": 1535327477,
        "source": "llama_decoder_layer_amd/csrc/gemm.hip",
        "sha1": "b59e6a8385c5f8d8efa36a66f0e1b400cd7d33af",
        "summary": "profiles/gate_up_silu_tp8shard_prefill_4x2048_counters.md",
    },
    ("llama70b_tp8shard_decode_b32_ctx2048", "gate_up"): {
        "bytes": 129033522,
        "source": "llama_decoder_layer_amd/csrc/gemm_skinny.hip",
        "sha1": "ee8feba85821bd1f610cc90ce33abda82a193c67",
        "summary": "profiles/gate_up_tp8shard_decode_b32_ctx2048_counters.md",
    },
    ("llama70b_prefill_4x2048", "gate_up_silu"): {
        "bytes": 11743957635,
        "source": "llama_decoder_layer_amd/csrc/gemm.hip",
        "sha1": "b59e6a8385c5f8d8efa36a66f0e1b400cd7d33af",
        "summary": "profiles/gate_up_silu_prefill_4x2048_counters.md",
    },
    ("qwen3moe_decode_b32_ctx2048", "moe_gate_up_silu"): {
        "bytes": 703212909,
        "source": "llama_decoder_layer_amd/csrc/moe.hip",
        "sha1": "755722e27b7a0844d60c7110d6ebca39ad3481fe",
        "summary": "profiles/moe_gate_up_silu_qwen3moe_decode_b32_ctx2048.md",
    },
    ("llama70b_decode_b32_ctx2048", "gate_up_silu"): {
        "bytes": 945630302,
        "source": "llama_decoder_layer_amd/csrc/gemm_skinny.hip",
        "sha1": "ee8feba85821bd1f610cc90ce33abda82a193c67",
        "summary": "profiles/gate_up_silu_decode_b32_ctx2048.md",
    },
}


def counter_traffic(workload, kernel):
    import hashlib
    rec = COUNTER_TRAFFIC.get((workload, kernel))
    if rec is None:
        return None
    try:
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            if hashlib.sha1(f.read()).hexdigest() != rec["sha1"]:
                return None
    except OSError:
        return None
    return rec["bytes"]


def layer_flops(model, num_tokens, attn_pairs):
    H, I, Q = model.hidden_size, model.intermediate_size, model.q_size
    attn = 2 * num_tokens * H * (model.qkv_size + Q) + 4 * model.num_attention_heads * model.head_dim * attn_pairs
    if model.num_experts:  # router + each token's k experts (gate_up and down)
        P, Ie = num_tokens * model.num_experts_per_tok, model.moe_intermediate_size
        return attn + 2 * num_tokens * H * model.num_experts + 2 * P * H * 2 * Ie + 2 * P * Ie * H
    return attn + 2 * num_tokens * H * 2 * I + 2 * num_tokens * I * H


def kernel_bytes(model, name, T, kv_tokens, active_experts=0):
    """Algorithmic HBM bytes of one launch of kernel `name` (bf16): weights
    read once, activations in and out once, KV read once; an expert kernel
    reads the weights of the experts that have tokens (`active_experts`)."""
    H, I, Q, QKV = model.hidden_size, model.intermediate_size, model.q_size, model.qkv_size
    e = 2
    P, Ie = T * model.num_experts_per_tok, model.moe_intermediate_size
    return {
        "gate_up": 2 * I * H * e + T * H * e,  # split-K partials, SiluAndMul in the reduce
        "moe_gate_up_silu": active_experts * 2 * Ie * H * e + T * H * e + P * Ie * e,
        "moe_down": active_experts * H * Ie * e + P * Ie * e + P * H * e,
        "gate_up_silu": 2 * I * H * e + T * H * e + T * I * e,
        "down_proj": H * I * e + T * I * e + T * H * e,
        "qkv_proj": QKV * H * e + T * H * e + T * QKV * e,
        "o_proj_residual": H * Q * e + T * Q * e + 2 * T * H * e,
        "attention": kv_tokens * 2 * model.kv_size * e + T * Q * e,
    }.get(name)


def measure(wl, steps, warmup):
    """Times `steps` forwards (after `warmup`) of workload `wl`, then the same
    number again with the library's per-kernel HIP events on."""
    import torch

    import llama_decoder_layer_amd as lda
    import synth

    model = wl.model
    dev = "cuda"
    batch, hidden, residual, per_layer = synth.workload_tensors(wl, dev)
    pos, bt, sl = batch.positions.to(dev), batch.block_table.to(dev), batch.seq_lens.to(dev)
    qsl = None if batch.query_start_loc is None else batch.query_start_loc.to(dev)
    layers = [lda.Layer(model.config_dict(), p["weights"]) for p in per_layer]
    T, B = batch.num_tokens, batch.num_seqs
    ws = layers[0].alloc_workspace(T, B, batch.max_seq_len)
    bufs = [(torch.empty_like(hidden), torch.empty_like(hidden)) for _ in layers]
    torch.cuda.synchronize()

    def step():
        h, r = hidden, residual
        for L, p, (ho, ro) in zip(layers, per_layer, bufs):
            L.forward(h, r, pos, p["k_pool"], p["v_pool"], bt, sl, batch.max_seq_len, hidden_out=ho,
                      residual_out=ro, workspace=ws, query_start_loc=qsl)
            h, r = ho, ro

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps

    # per-kernel durations: HIP events the library records on its stream
    for L in layers:
        L.set_timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = {}
    for L in layers:
        for name, (tot, cnt) in L.timing_read().items():
            a, c = kt.get(name, (0.0, 0))
            kt[name] = (a + tot, c + cnt)
        L.set_timing(False)
    kernel_avg_ms = {k: v[0] / v[1] for k, v in kt.items()}
    active = 0
    if model.num_experts:  # experts the batch routed tokens to (the same every step)
        ids = layers[0].workspace_tensor(ws, "topk_ids", T, B, batch.max_seq_len)
        active = int(torch.unique(ids).numel())

    kv_tokens = int(batch.seq_lens.sum())
    # causal (query, key) pairs: a sequence with c cached and n new rows
    attn_pairs = sum(n * c + n * (n + 1) // 2 for c, n in
                     ((batch.ctx_lens[b], batch.new_rows(b)) for b in range(B)))
    dom = "moe_gate_up_silu" if model.num_experts else ("gate_up_silu" if "gate_up_silu" in kernel_avg_ms
                                                          else "gate_up")
    dur = kernel_avg_ms[dom] / 1e3
    if T == B:  # decode: one row per sequence, the step streams weights and KV
        alg = kernel_bytes(model, dom, T, kv_tokens, active)
        roof = {"bound": "hbm", "kernel": dom, "achieved": alg / dur / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": alg / dur / 1e9 / PEAK_HBM_GBS,
                "traffic": counter_traffic(wl.name, dom),
                "algorithmic_bytes_per_launch": alg, "avg_launch_us": dur * 1e6}
    else:
        H, I = model.hidden_size, model.intermediate_size
        alg = 2 * T * H * 2 * I
        if model.num_experts:
            alg = 2 * T * model.num_experts_per_tok * H * 2 * model.moe_intermediate_size
        roof = {"bound": "mfma", "kernel": dom, "achieved": alg / dur / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": alg / dur / 1e12 / PEAK_BF16_TFLOPS,
                "traffic": counter_traffic(wl.name, dom),
                "algorithmic_flops_per_launch": alg, "avg_launch_us": dur * 1e6}
        if roof["traffic"] is not None and not model.num_experts:  # HBM bytes a launch must move at least
            roof["algorithmic_bytes_per_launch"] = kernel_bytes(model, dom, T, kv_tokens)
    wbytes = sum(v.numel() * v.element_size() for k, v in per_layer[0]["weights"].items()
                 if not k.startswith("experts_"))
    if model.num_experts:  # only the routed-to experts' weights are read
        wbytes += active * 3 * model.moe_intermediate_size * model.hidden_size * 2
    step_bytes = len(layers) * (wbytes + kv_tokens * 2 * model.kv_size * 2 + 4 * T * model.hidden_size * 2)
    step_flops = len(layers) * layer_flops(model, T, attn_pairs)
    res = {
        "workload": wl.name, "value": round(T / (ms / 1e3), 2), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "roofline": roof,
        "step_fraction": {"hbm": step_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                          "mfma": step_flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS},
        "kernel_avg_us": {k: round(v * 1e3, 2) for k, v in sorted(kernel_avg_ms.items())},
        "wall_s_timed_region": round(wall, 3),
        **({"experts_with_tokens": active} if model.num_experts else {}),
        "config": ({"workload": wl.name, "num_seqs": B, "q_len": wl.q_len,
                    "ctx_len": wl.ctx if not isinstance(wl.ctx, tuple) else list(wl.ctx),
                    "layers": len(layers), "parallelism": "single GPU"} if not wl.mixed else
                   {"workload": wl.name, "num_seqs": B, "num_tokens": T,
                    "mix": "%d decode rows at context %d + one %d-row prefill chunk on context %d" % (
                        sum(1 for q, _ in wl.mix if q == 1), wl.mix[0][1], wl.mix[-1][0], wl.mix[-1][1]),
                    "layers": len(layers), "parallelism": "single GPU"}),
    }
    ctx = (batch, hidden, residual, per_layer)
    return res, ctx


STACK_SOURCE_LAYERS = 8


def measure_stack(wl, steps, warmup, graph=True):
    """A whole layer stack plus the final norm (llama_stack_forward), replayed
    from one captured HIP graph.  Weights are drawn for STACK_SOURCE_LAYERS
    layers and reused cyclically as the sources of the stack's copies: every
    layer still owns and streams its own weights (80 x 1.71 GB for the 70B
    body), while the host-side draw and the peak memory stay small."""
    import torch

    import llama_decoder_layer_amd as lda
    import synth

    model, dev = wl.model, "cuda"
    batch = synth.build_batch(wl)
    hidden, _ = synth.draw_activations(model, batch.num_tokens, wl.index, dev, residual=False)
    n_src = min(wl.layers, STACK_SOURCE_LAYERS)
    src = [synth.draw_weights(model, wl.index, l, dev) for l in range(n_src)]
    final = synth.draw_final_norm(model, wl.index, dev)
    stack = lda.Stack(model.config_dict(), [src[l % n_src] for l in range(wl.layers)], final)
    weight_bytes = sum(v.numel() * v.element_size() for v in src[0].values())
    del src
    torch.cuda.empty_cache()
    pools = [synth.build_kv_pool(wl, batch, l, dev) for l in range(wl.layers)]
    pos, bt, sl = batch.positions.to(dev), batch.block_table.to(dev), batch.seq_lens.to(dev)
    T, B = batch.num_tokens, batch.num_seqs
    ws = stack.alloc_workspace(T, B, batch.max_seq_len)
    out = torch.empty_like(hidden)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    if graph:
        g = stack.capture(hidden, pos, pools, bt, sl, batch.max_seq_len, out, ws, side)
        step = lambda: g.launch(side)
    else:
        step = lambda: stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=out, workspace=ws,
                                     stream=side)
    for _ in range(warmup):
        step()
    side.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(side)
    for _ in range(steps):
        step()
    t1.record(side)
    side.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps
    kv_tokens = int(batch.seq_lens.sum())
    step_bytes = wl.layers * (weight_bytes + kv_tokens * 2 * model.kv_size * 2 + 4 * T * model.hidden_size * 2)
    achieved = step_bytes / (ms / 1e3) / 1e9
    res = {
        "workload": wl.name, "value": round(T / (ms / 1e3), 2), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "roofline": {"bound": "hbm", "kernel": "whole step (%d layers + final norm)" % wl.layers,
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": None, "algorithmic_bytes_per_step": step_bytes},
        "wall_s_timed_region": round(wall, 3),
        "config": {"workload": wl.name, "num_seqs": B, "q_len": wl.q_len, "ctx_len": wl.ctx, "layers": wl.layers,
                   "final_norm": True, "hip_graph": bool(graph),
                   "weights": "drawn for %d layers, reused cyclically as the sources of %d separate layer copies"
                              % (n_src, wl.layers), "parallelism": "single GPU"},
    }
    if graph:
        g.close()
    stack.close()
    return res, None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b_decode_b32_ctx2048")
    ap.add_argument("--extra", default="llama70b_prefill_4x2048,qwen3moe_decode_b32_ctx2048,qwen3moe_prefill_4x2048,"
                                       "llama70b_tp8shard_decode_b32_ctx2048,llama70b_tp8shard_prefill_4x2048",
                    help="comma-separated workloads measured after the main one ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=None,
                    help="tokens of the step the oracle runs (default: all of a decode step, 256 of a prefill)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes, 3 times (a reference for "
                         "the HBM byte counters of a profiler), and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy, "launches": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences shard across GPUs with no exchange inside the layer)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    run = measure_stack if wl.layers > 4 else measure
    main_res, ctx = run(wl, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu_baseline and ctx is not None:
        batch, hidden, residual, per_layer = ctx
        rows = args.cpu_sample_rows or (batch.num_tokens if batch.num_tokens == batch.num_seqs else 256)
        cpu = cpu_baseline(wl, batch, hidden, residual, per_layer, rows)
    del ctx
    torch.cuda.empty_cache()
    extra = []
    if args.extra and args.extra != "none":
        for name in args.extra.split(","):
            xw = synth.WORKLOADS[name]
            r, c = (measure_stack if xw.layers > 4 else measure)(xw, max(3, args.steps // 4), min(args.warmup, 2))
            del c
            torch.cuda.empty_cache()
            extra.append(r)

    out = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.model.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations and KV context, N(0,0.02) weights)",
        "config": main_res["config"],
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "step_fraction": main_res.get("step_fraction"),
        "kernel_avg_us": main_res.get("kernel_avg_us"),
        **({"experts_with_tokens": main_res["experts_with_tokens"]} if "experts_with_tokens" in main_res else {}),
        "wall_s_timed_region": main_res["wall_s_timed_region"],
        "extra": extra,
    }
    print(json.dumps(out))


def cpu_baseline(wl, batch, hidden, residual, per_layer, rows, min_seconds=10.0):
    """The oracle (float64 numpy, as it stands) on a bounded sample of the
    same step -- the first `rows` tokens of the batch through every layer --
    repeated until about `min_seconds` of CPU work have run."""
    import numpy as np
    import torch

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    model = wl.model
    rows = min(rows, batch.num_tokens)
    rows_list = list(range(rows))
    seq_of = batch.seq_of_row()
    seq_ids = sorted({seq_of[r] for r in rows_list})
    cfg = model.config_dict()
    pos = batch.positions.numpy().astype(np.int64)
    h0 = f64(hidden)
    r0 = None if residual is None else f64(residual)
    ctx = []
    for p in per_layer:
        ctx.append([(b, f64(synth.gather_context(p["k_pool"], batch, b, batch.ctx_lens[b])),
                     f64(synth.gather_context(p["v_pool"], batch, b, batch.ctx_lens[b], "v"))) for b in seq_ids])
    weights = [p["weights"] for p in per_layer]
    iters, t0 = 0, time.perf_counter()
    while True:
        h, r = h0, r0
        for w_t, c in zip(weights, ctx):
            w = {k: f64(v) for k, v in w_t.items()}
            seqs = [oracle.Seq(list(batch.rows(b)), kc, vc) for b, kc, vc in c]
            o = oracle.decoder_layer(cfg, w, h, r, pos, seqs, want=rows_list)
            h = h.copy()
            r = np.zeros_like(h) if r is None else r.copy()
            h[rows_list] = o["hidden_out"]
            r[rows_list] = o["residual_out"]
        iters += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(rows * iters / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d tokens of the step through %d layer(s), %d repetition(s); float64 numpy "
                      "oracle including its weight widening" % (rows, batch.num_tokens, len(per_layer), iters),
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()

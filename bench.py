"""Throughput of the Llama-70B-shape decoder-layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--extra A,B,..]
                    [--no-cpu-baseline] [--cpu-seconds S]

A step is one forward of the whole layer (input_layernorm, qkv_proj, RoPE +
KV write, paged attention, o_proj + residual, post_attention_layernorm,
gate_up_proj + SiluAndMul, down_proj) -- through every layer of a stacked
workload -- over one batch of seeded synthetic inputs that are resident in HBM
before timing starts.  The main line is the 70B decode (32 sequences, one new
token each after a 2048-token context); the extra lines are the 70B prefills
(4 x 2048 and 1 x 32768), the 70B ragged decode through 4 layers, the
Qwen3-MoE layer, one GPU's TP = 8 share of the 70B layer, the mixed step
(32 decode rows + a 512-row prefill chunk) and the 80-layer body replayed
from one HIP graph.  Prints one JSON line.

Per workload:
  * value / ms_per_step: K steps back to back between two events, with a
    device synchronisation on both sides;
  * per_call_flushed: each of N further steps between its own events, with
    1 GiB written to a scratch buffer before each (outside the events) so the
    256 MB last-level cache holds nothing of the step's inputs; median, min;
  * kernel_avg_us: the library's own per-kernel events over K more steps;
    the roofline names the kernel with the largest time per step and divides
    its algorithmic work per launch by its average launch time;
  * cpu_baseline: the oracle (float64 numpy, as it stands) on a bounded
    sample of the same step, its weights widened before the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
METRIC = "70B-shape layer tokens/s (prefill, decode) + % MFMA/HBM peak, 1 MI355X"
FLUSH_BYTES = 1 << 30
DEFAULT_EXTRA = ("llama70b_prefill_4x2048,llama70b_prefill_1x32768,llama70b_ragged_decode_b64_4layer,"
                 "qwen3moe_decode_b32_ctx2048,qwen3moe_prefill_4x2048,llama70b_tp8shard_decode_b32_ctx2048,"
                 "llama70b_tp8shard_prefill_4x2048,llama70b_mixed_chunk512_decode32,llama70b_stack80_decode_b32_ctx2048")
# timed calls with a cache flush between them, per workload (the rest: 10)
FLUSHED_CALLS = {"llama70b_decode_b32_ctx2048": 20, "llama70b_ragged_decode_b64_4layer": 20,
                 "llama70b_prefill_4x2048": 10, "llama70b_prefill_1x32768": 5}

# HBM bytes per launch of a kernel from rocprofv3 counters: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
# (factors from a plain 1 GiB copy; profiles/pmc_copy_calibration.md).  Reported only while every
# source the kernel's code and launch plan come from is the one the counters were taken on.
PLAN_SOURCES = ("llama_decoder_layer_amd/csrc/common.h", "llama_decoder_layer_amd/csrc/kernels.h",
                "llama_decoder_layer_amd/csrc/api.cpp")
COUNTER_TRAFFIC = {
    ('llama70b_decode_b32_ctx2048', 'gate_up_silu'): {
        "bytes": 945640960, "sha1": 'cb80f7e7d58f8324e231e15be63b6e7fc1a2e247',
        "sources": ('llama_decoder_layer_amd/csrc/gemm_skinny.hip',),
        "summary": 'profiles/gate_up_silu_decode_b32_ctx2048_counters.md'},
    ('llama70b_prefill_4x2048', 'gate_up_silu'): {
        "bytes": 11769860136, "sha1": '18d4c16099ea8a4dfe1a3dd026d7dcc9eb895271',
        "sources": ('llama_decoder_layer_amd/csrc/gemm.hip',),
        "summary": 'profiles/gate_up_silu_prefill_4x2048_counters.md'},
    ('llama70b_prefill_1x32768', 'gate_up_silu'): {
        "bytes": 47224896288, "sha1": '18d4c16099ea8a4dfe1a3dd026d7dcc9eb895271',
        "sources": ('llama_decoder_layer_amd/csrc/gemm.hip',),
        "summary": 'profiles/gate_up_silu_prefill_1x32768_counters.md'},
    ('llama70b_ragged_decode_b64_4layer', 'attention'): {
        "bytes": 4469649868, "sha1": '9a5eb220a8bdd6807ae69859328fb0f75ae3ff8a',
        "sources": ('llama_decoder_layer_amd/csrc/attention_decode.hip', 'llama_decoder_layer_amd/csrc/attention.hip'),
        "summary": 'profiles/attention_ragged_decode_b64_4layer_counters.md'},
    ('qwen3moe_decode_b32_ctx2048', 'moe_gate_up_silu'): {
        "bytes": 699528320, "sha1": '1952190a6e5aa9cd4bde4c91f4976f45cea67fcd',
        "sources": ('llama_decoder_layer_amd/csrc/moe.hip',),
        "summary": 'profiles/moe_gate_up_silu_qwen3moe_decode_b32_ctx2048_counters.md'},
    ('qwen3moe_prefill_4x2048', 'moe_gate_up_silu'): {
        "bytes": 1889146576, "sha1": '1952190a6e5aa9cd4bde4c91f4976f45cea67fcd',
        "sources": ('llama_decoder_layer_amd/csrc/moe.hip',),
        "summary": 'profiles/moe_gate_up_silu_qwen3moe_prefill_4x2048_counters.md'},
    ('llama70b_tp8shard_decode_b32_ctx2048', 'gate_up'): {
        "bytes": 129028592, "sha1": 'cb80f7e7d58f8324e231e15be63b6e7fc1a2e247',
        "sources": ('llama_decoder_layer_amd/csrc/gemm_skinny.hip',),
        "summary": 'profiles/gate_up_tp8shard_decode_b32_ctx2048_counters.md'},
    ('llama70b_tp8shard_prefill_4x2048', 'gate_up_silu'): {
        "bytes": 1535366256, "sha1": '18d4c16099ea8a4dfe1a3dd026d7dcc9eb895271',
        "sources": ('llama_decoder_layer_amd/csrc/gemm.hip',),
        "summary": 'profiles/gate_up_silu_tp8shard_prefill_4x2048_counters.md'},
    ('llama70b_mixed_chunk512_decode32', 'gate_up_silu'): {
        "bytes": 1251943808, "sha1": '18d4c16099ea8a4dfe1a3dd026d7dcc9eb895271',
        "sources": ('llama_decoder_layer_amd/csrc/gemm.hip',),
        "summary": 'profiles/gate_up_silu_mixed_chunk512_decode32_counters.md'},
}


def sources_sha1(paths):
    import hashlib
    h = hashlib.sha1()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(workload, kernel):
    rec = COUNTER_TRAFFIC.get((workload, kernel))
    if rec is None:
        return None
    try:
        if sources_sha1(tuple(rec["sources"]) + PLAN_SOURCES) != rec["sha1"]:
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
    read once, activations in and out once, K/V read once; an expert kernel
    reads the weights of the experts that have tokens."""
    H, I, Q, QKV = model.hidden_size, model.intermediate_size, model.q_size, model.qkv_size
    e = 2
    P, Ie = T * model.num_experts_per_tok, model.moe_intermediate_size
    return {
        "gate_up": 2 * I * H * e + T * H * e,  # split-K partials, SiluAndMul in the reduce
        "gate_up_silu": 2 * I * H * e + T * H * e + T * I * e,
        "down_proj": H * I * e + T * I * e + T * H * e,
        "qkv_proj": QKV * H * e + T * H * e + T * QKV * e,
        "o_proj": H * Q * e + T * Q * e + T * H * e,
        "o_proj_residual": H * Q * e + T * Q * e + 2 * T * H * e,
        "attention": kv_tokens * 2 * model.kv_size * e + 2 * T * Q * e,
        "moe_gate_up_silu": active_experts * 2 * Ie * H * e + T * H * e + P * Ie * e,
        "moe_down": active_experts * H * Ie * e + P * Ie * e + P * H * e,
    }.get(name)


def kernel_flops(model, name, T, attn_pairs):
    """Algorithmic FLOPs of one launch of kernel `name`."""
    H, I, Q, QKV = model.hidden_size, model.intermediate_size, model.q_size, model.qkv_size
    P, Ie = T * model.num_experts_per_tok, model.moe_intermediate_size
    return {
        "gate_up_silu": 2 * T * H * 2 * I,
        "down_proj": 2 * T * I * H,
        "qkv_proj": 2 * T * H * QKV,
        "o_proj_residual": 2 * T * Q * H,
        "attention": 4 * model.num_attention_heads * model.head_dim * attn_pairs,
        "moe_gate_up_silu": 2 * P * H * 2 * Ie,
        "moe_down": 2 * P * Ie * H,
    }.get(name)


def _flush(buf):
    buf.add_(1)  # reads and writes all of it: 2 GiB of traffic evicts the 256 MB cache


def measure(wl, steps, warmup, flushed_calls, flush_buf):
    """Times `steps` forwards (after `warmup`) of workload `wl` back to back,
    then `flushed_calls` forwards one at a time after a cache flush, then
    `steps` more with the library's per-kernel HIP events on."""
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

    # one call at a time, each after a cache flush outside its events
    per_call = []
    for _ in range(flushed_calls):
        _flush(flush_buf)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        per_call.append(a.elapsed_time(b))

    # per-kernel durations: HIP events the library records on its stream
    for L in layers:
        L.set_timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = {}
    for L in layers:
        for name, (tot, cnt) in L.timing_read().items():
            a_, c_ = kt.get(name, (0.0, 0))
            kt[name] = (a_ + tot, c_ + cnt)
        L.set_timing(False)
    kernel_avg_ms = {k: v[0] / v[1] for k, v in kt.items()}
    kernel_step_ms = {k: v[0] / steps for k, v in kt.items()}
    active = 0
    if model.num_experts:  # experts the batch routed tokens to (the same every step)
        ids = layers[0].workspace_tensor(ws, "topk_ids", T, B, batch.max_seq_len)
        active = int(torch.unique(ids).numel())

    kv_tokens = int(batch.seq_lens.sum())
    # causal (query, key) pairs: a sequence with c cached and n new rows
    attn_pairs = sum(n * c + n * (n + 1) // 2 for c, n in
                     ((batch.ctx_lens[b], batch.new_rows(b)) for b in range(B)))
    decode = T == B
    work = ((lambda k: kernel_bytes(model, k, T, kv_tokens, active)) if decode
            else (lambda k: kernel_flops(model, k, T, attn_pairs)))
    # the kernel with the largest time per step (among those with a work figure)
    cands = [k for k in kernel_step_ms if work(k) is not None]
    dom = max(cands, key=lambda k: kernel_step_ms[k])
    dur = kernel_avg_ms[dom] / 1e3
    alg = work(dom)
    if decode:
        roof = {"bound": "hbm", "kernel": dom, "achieved": alg / dur / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": alg / dur / 1e9 / PEAK_HBM_GBS, "traffic": counter_traffic(wl.name, dom),
                "algorithmic_bytes_per_launch": alg, "avg_launch_us": dur * 1e6,
                "share_of_step": kernel_step_ms[dom] / ms}
    else:
        roof = {"bound": "mfma", "kernel": dom, "achieved": alg / dur / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": alg / dur / 1e12 / PEAK_BF16_TFLOPS,
                "traffic": counter_traffic(wl.name, dom), "algorithmic_flops_per_launch": alg,
                "avg_launch_us": dur * 1e6, "share_of_step": kernel_step_ms[dom] / ms}
        if roof["traffic"] is not None and kernel_bytes(model, dom, T, kv_tokens) is not None:
            roof["algorithmic_bytes_per_launch"] = kernel_bytes(model, dom, T, kv_tokens)
        if dom == "gate_up_silu":  # a dense bf16 product the vendor GEMM can be timed on
            roof["product_mnk"] = [T, 2 * model.intermediate_size, model.hidden_size]
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
        "per_call_flushed": {"calls": len(per_call), "flush_bytes_written": FLUSH_BYTES,
                             "median_ms": round(statistics.median(per_call), 4) if per_call else None,
                             "min_ms": round(min(per_call), 4) if per_call else None,
                             "tokens_per_s_at_median": round(T / (statistics.median(per_call) / 1e3), 2)
                             if per_call else None},
        "kernel_avg_us": {k: round(v * 1e3, 2) for k, v in sorted(kernel_avg_ms.items())},
        "kernel_us_per_step": {k: round(v * 1e3, 2) for k, v in sorted(kernel_step_ms.items())},
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
    for L in layers:
        L.close()
    del ws, bufs
    ctx = (batch, hidden, residual, per_layer)
    return res, ctx


STACK_SOURCE_LAYERS = 8


def measure_stack(wl, steps, warmup, flushed_calls, flush_buf, graph=True):
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
    w0 = src[0]  # kept for the oracle baseline's sampled layer
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
    per_call = []
    for _ in range(flushed_calls):
        with torch.cuda.stream(side):
            _flush(flush_buf)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(side)
        step()
        b.record(side)
        side.synchronize()
        per_call.append(a.elapsed_time(b))
    kv_tokens = int(batch.seq_lens.sum())
    step_bytes = wl.layers * (weight_bytes + kv_tokens * 2 * model.kv_size * 2 + 4 * T * model.hidden_size * 2)
    achieved = step_bytes / (ms / 1e3) / 1e9
    res = {
        "workload": wl.name, "value": round(T / (ms / 1e3), 2), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "roofline": {"bound": "hbm", "kernel": "whole step (%d layers + final norm)" % wl.layers,
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": None, "algorithmic_bytes_per_step": step_bytes},
        "per_call_flushed": {"calls": len(per_call), "flush_bytes_written": FLUSH_BYTES,
                             "median_ms": round(statistics.median(per_call), 4) if per_call else None,
                             "min_ms": round(min(per_call), 4) if per_call else None},
        "wall_s_timed_region": round(wall, 3),
        "config": {"workload": wl.name, "num_seqs": B, "q_len": wl.q_len, "ctx_len": wl.ctx, "layers": wl.layers,
                   "final_norm": True, "hip_graph": bool(graph),
                   "weights": "drawn for %d layers, reused cyclically as the sources of %d separate layer copies"
                              % (n_src, wl.layers), "parallelism": "single GPU"},
    }
    if graph:
        g.close()
    stack.close()
    # the oracle baseline samples layer 0 and scales its time by the layer count
    per_layer = [{"weights": w0, "k_pool": pools[0][0], "v_pool": pools[0][1]}] + [None] * (wl.layers - 1)
    return res, (batch, hidden, None, per_layer)


def hbm_read_ceiling(steps=10):
    """The read-only streaming kernel over the bytes and in the launch shape
    of the decode step's largest kernel (the 70B gate_up weight, one
    workgroup of 7 waves per CU), and over 4 GiB in 256 workgroups of 256
    threads; each with plain loads and with the nontemporal hint the decode
    path's weight and KV streams use.  Then 4 GiB gathered as 4 KiB blocks in
    random and in sequential order (nontemporal)."""
    import torch

    import llama_decoder_layer_amd as lda
    import synth

    m = synth.LLAMA70B
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    for name, nbytes, wgs, threads in (("gate_up_shape", 2 * m.intermediate_size * m.hidden_size * 2, cus, 448),
                                       ("4GiB_256x256", 4 << 30, 256, 256)):
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        sink = torch.empty(wgs * threads, dtype=torch.int32, device="cuda")
        for nt in (False, True):
            for _ in range(3):
                lda.stream_read(src, wgs, threads, sink, nontemporal=nt)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(steps):
                lda.stream_read(src, wgs, threads, sink, nontemporal=nt)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / steps * 1e3
            out[name + ("_nontemporal" if nt else "")] = {
                "bytes": nbytes, "workgroups": wgs, "threads": threads, "avg_us": round(us, 2),
                "GB_per_s": round(nbytes / (us / 1e6) / 1e9, 1),
                "frac_of_peak": round(nbytes / (us / 1e6) / 1e9 / PEAK_HBM_GBS, 4)}
        del src, sink
    # 4 GiB read as 4 KiB blocks (one KV head's K or V block of the cache) in a
    # seeded random order and in order, nontemporal: the decode attention's
    # access pattern over a paged cache
    nbytes, bb, wgs = 4 << 30, 4096, 2048
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.empty(wgs * bb // 16, dtype=torch.int32, device="cuda")
    g = torch.Generator().manual_seed(11)
    for name, ids in (("4GiB_4KiB_blocks_random", torch.randperm(nbytes // bb, generator=g)),
                      ("4GiB_4KiB_blocks_in_order", torch.arange(nbytes // bb))):
        ids = ids.to(torch.int32).to("cuda")
        lda.block_read(src, ids, bb, wgs, sink, nontemporal=True)  # checks the ids once
        for _ in range(2):
            lda.block_read(src, ids, bb, wgs, sink, nontemporal=True, check_ids=False)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            lda.block_read(src, ids, bb, wgs, sink, nontemporal=True, check_ids=False)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        out[name + "_nontemporal"] = {
            "bytes": nbytes, "workgroups": wgs, "threads": bb // 16, "avg_us": round(us, 2),
            "GB_per_s": round(nbytes / (us / 1e6) / 1e9, 1),
            "frac_of_peak": round(nbytes / (us / 1e6) / 1e9 / PEAK_HBM_GBS, 4)}
        del ids
    del src, sink
    return out


def cold_read_by_size(reps=7):
    """The nontemporal read-only kernel (one 7-wave workgroup per CU) over
    each of the 70B decode step's streams -- the four projection weights and
    the 32 x 2048 batch's K/V -- each read right after a 1 GiB cache flush:
    the time a kernel that only reads those bytes needs, ramp and tail
    included, against which each decode kernel's time is set.  Median of
    `reps` flushed reads per size."""
    import torch

    import llama_decoder_layer_amd as lda
    import synth

    m = synth.LLAMA70B
    H, I, D = m.hidden_size, m.intermediate_size, m.head_dim
    kv_heads, q_heads = m.num_key_value_heads, m.num_attention_heads
    sizes = (("qkv_proj", (q_heads + 2 * kv_heads) * D * H * 2), ("o_proj", H * q_heads * D * 2),
             ("down_proj", H * I * 2), ("gate_up", 2 * I * H * 2), ("kv_32x2048", 32 * 2048 * 2 * kv_heads * D * 2))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    flush_buf = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 448, dtype=torch.int32, device="cuda")
    out = {}
    for name, nbytes in sizes:
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        lda.stream_read(src, cus, 448, sink, nontemporal=True)
        us = []
        for _ in range(reps):
            _flush(flush_buf)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            lda.stream_read(src, cus, 448, sink, nontemporal=True)
            b.record()
            torch.cuda.synchronize()
            us.append(a.elapsed_time(b) * 1e3)
        med = statistics.median(us)
        out[name] = {"bytes": nbytes, "median_us": round(med, 2), "min_us": round(min(us), 2),
                     "GB_per_s": round(nbytes / (med / 1e6) / 1e9, 1)}
        del src
    return out


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    threads = affinity
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [affinity])
    except Exception:
        pass
    return model, affinity, threads


def cpu_baseline(wl, batch, hidden, residual, per_layer, min_seconds):
    """The oracle (float64 numpy, as it stands) on a bounded sample of the
    same step, its inputs and weights widened before the timed region.
    Decode: every row of the step through every layer; with several layers
    (the ragged 4-layer batch, the 80-layer stack) the first 4 sequences
    through layer 0, the time scaled by the layer count (the stack's final
    norm left out).  Prefill and mixed steps: the first 256 token rows.
    Repeated until about `min_seconds` of CPU work have run."""
    import numpy as np

    import oracle
    import synth

    f64 = lambda t: t.detach().to("cpu", torch_f64()).numpy()
    model = wl.model
    T = batch.num_tokens
    decode = T == batch.num_seqs
    rows = (4 if len(per_layer) > 1 else T) if decode else min(256, T)
    use_layers = per_layer[:1] if (decode and len(per_layer) > 1) else per_layer
    scale = len(per_layer) / len(use_layers)
    rows_list = list(range(rows))
    seq_of = batch.seq_of_row()
    seq_ids = sorted({seq_of[r] for r in rows_list})
    cfg = model.config_dict()
    pos = batch.positions.numpy().astype(np.int64)
    h0 = f64(hidden)
    r0 = None if residual is None else f64(residual)
    prepared = []
    for p in use_layers:
        w = {k: f64(v) for k, v in p["weights"].items()}
        seqs = [oracle.Seq(list(batch.rows(b)), f64(synth.gather_context(p["k_pool"], batch, b, batch.ctx_lens[b])),
                           f64(synth.gather_context(p["v_pool"], batch, b, batch.ctx_lens[b], "v"))) for b in seq_ids]
        prepared.append((w, seqs))
    iters, t0 = 0, time.perf_counter()
    while True:
        h, r = h0, r0
        for w, seqs in prepared:
            o = oracle.decoder_layer(cfg, w, h, r, pos, seqs, want=rows_list)
            h = h.copy()
            r = np.zeros_like(h) if r is None else r.copy()
            h[rows_list] = o["hidden_out"]
            r[rows_list] = o["residual_out"]
        iters += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = (time.perf_counter() - t0) * scale
    cpu_model, affinity, threads = cpu_info()
    return {"value": round(rows * iters / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d token rows of the step through %d of %d layer(s)%s, %d repetition(s); float64 numpy "
                      "oracle, weights and inputs widened before timing" % (
                          rows, T, len(use_layers), len(per_layer),
                          " (time scaled by %d layers)" % len(per_layer) if scale != 1 else "", iters),
            "seconds": round(time.perf_counter() - t0, 2), "cpu_model": cpu_model, "affinity_cores": affinity,
            "blas_threads": threads}


def torch_f64():
    import torch
    return torch.float64


def run_workload(name, steps, warmup, flushed_calls, flush_buf, cpu_seconds):
    import torch

    import synth

    wl = synth.WORKLOADS[name]
    run = measure_stack if wl.layers > 4 else measure
    res, ctx = run(wl, steps, warmup, flushed_calls, flush_buf)
    if ctx is not None and cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(wl, *ctx, min_seconds=cpu_seconds)
    del ctx
    torch.cuda.empty_cache()
    return res


def vendor_gemm_tflops(M, N, K, reps=5):
    """hipBLASLt (torch.matmul) on one bf16 product out[M, N] = x[M, K] w[N, K]^T:
    TFLOP/s over `reps` event-timed calls after 2 untimed ones."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(7)
    x = (torch.randn(M, K, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    for _ in range(2):
        torch.matmul(x, w.t())
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.matmul(x, w.t())
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    del x, w
    return 2.0 * M * N * K / us / 1e6


def device_record():
    """What the box reports: name, architecture and CU count from the device
    properties, the maximum shader clock from rocminfo (null if unavailable)."""
    import subprocess

    import torch

    p = torch.cuda.get_device_properties(0)
    rec = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
           "memory_bytes": p.total_memory, "max_clock_mhz": None}
    try:
        rec["max_clock_mhz"] = gpu_max_clock_mhz(
            subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout)
    except (OSError, subprocess.SubprocessError):
        pass
    return rec


def gpu_max_clock_mhz(rocminfo_text):
    """The first GPU agent's "Max Clock Freq. (MHz)" in rocminfo's output
    (agents whose Name is a gfx target), or None."""
    gpu = False
    for line in rocminfo_text.splitlines():
        t = line.strip()
        if t.startswith("Name:"):
            gpu = t.split(":", 1)[1].strip().startswith("gfx")
        elif gpu and t.startswith("Max Clock Freq. (MHz):"):
            try:
                return int(t.split(":", 1)[1].strip())
            except ValueError:
                return None
    return None


def attach_measured_ceilings(lines, ceiling):
    """Each line's dominant kernel against a ceiling measured on the same box
    and in the same process, beside the datasheet fraction: HBM-bound lines
    against the nontemporal read-only kernel (streaming in the decode gate_up
    launch shape; gathering 4 KiB blocks in random order where attention
    dominates), GEMM-bound lines against the vendor GEMM (hipBLASLt) on the
    same bf16 product.  Lines whose dominant kernel has no such counterpart
    (the grouped expert GEMMs) get none."""
    vendor = {}
    for r in lines:
        rf = r["roofline"]
        if rf.get("bound") == "hbm":
            key = "4GiB_4KiB_blocks_random_nontemporal" if rf.get("kernel") == "attention" else \
                "gate_up_shape_nontemporal"
            c = ceiling[key]["GB_per_s"]
            rf["measured_ceiling"] = {"source": "read-only kernel: " + key, "value": c, "unit": "GB/s",
                                      "frac": rf["achieved"] / c}
        elif rf.get("bound") == "mfma" and rf.get("product_mnk"):
            mnk = tuple(rf["product_mnk"])
            if mnk not in vendor:
                vendor[mnk] = vendor_gemm_tflops(*mnk)
            c = vendor[mnk]
            rf["measured_ceiling"] = {"source": "hipBLASLt on the same product (M, N, K) = %d, %d, %d" % mnk,
                                      "value": round(c, 1), "unit": "TFLOP/s", "frac": rf["achieved"] / c}


def library_gemm_reference(reps=5):
    """The vendor GEMM (hipBLASLt, through torch.matmul) beside this
    library's tiled kernel (llama_op_linear, plain store) on the 70B prefill
    projections at 8192 tokens: what MFMA rate the same bf16 products reach
    in the library's hand-tuned assembly, a reference for the tiled kernel.
    The layer itself never calls the library."""
    import torch

    import llama_decoder_layer_amd as lda

    shapes = (("qkv_proj", 8192, 10240, 8192), ("o_proj", 8192, 8192, 8192), ("gate_up_proj", 8192, 57344, 8192),
              ("down_proj", 8192, 8192, 28672))
    g = torch.Generator(device="cuda").manual_seed(5)
    out = {}
    for name, M, N, K in shapes:
        x = (torch.randn(M, K, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        ours = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        runs = {"this_library": lambda: lda.linear(x, w, out=ours),
                "hipblaslt": lambda: torch.matmul(x, w.t())}
        rec = {"M": M, "N": N, "K": K}
        for label, fn in runs.items():
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            rec[label] = {"avg_us": round(us, 1), "TFLOP_per_s": round(2.0 * M * N * K / us / 1e6, 1),
                          "frac_of_peak": round(2.0 * M * N * K / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
        ref = torch.matmul(x, w.t()).float()
        rec["max_abs_diff"] = float((ours.float() - ref).abs().max())
        out[name] = rec
        del x, w, ours, ref
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b_decode_b32_ctx2048")
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma-separated workloads measured after the main one ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work per oracle baseline")
    ap.add_argument("--flushed-calls", type=int, default=None, help="override the per-workload flushed call counts")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes, 3 times (a reference for "
                         "the HBM byte counters of a profiler), and exit")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor GEMM (hipBLASLt) beside this library's tiled kernel on the 70B "
                         "prefill projection shapes, and exit")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only run the read-only streaming kernel (the HBM read ceiling, and cold reads of "
                         "each decode stream's size) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences shard across GPUs with no exchange inside the layer)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy, "launches": 3}))
        return
    if args.library_gemm:
        print(json.dumps({"library_gemm_reference": library_gemm_reference()}))
        return
    if args.ceiling_only:
        print(json.dumps({"hbm_read_ceiling": hbm_read_ceiling(), "cold_read_by_size": cold_read_by_size()}))
        return

    flush_buf = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    calls = lambda n: args.flushed_calls if args.flushed_calls is not None else FLUSHED_CALLS.get(n, 10)
    main_res = run_workload(args.workload, args.steps, args.warmup, calls(args.workload), flush_buf, cpu_s)
    extra = []
    if args.extra and args.extra != "none":
        for name in args.extra.split(","):
            extra.append(run_workload(name, max(3, args.steps // 4), min(args.warmup, 2), calls(name), flush_buf,
                                      cpu_s / 2))
    ceiling = hbm_read_ceiling()
    cold = cold_read_by_size()
    attach_measured_ceilings([main_res] + extra, ceiling)
    wl = synth.WORKLOADS[args.workload]
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
        "cpu_baseline": main_res.get("cpu_baseline"),
        "step_fraction": main_res.get("step_fraction"),
        "per_call_flushed": main_res.get("per_call_flushed"),
        "kernel_avg_us": main_res.get("kernel_avg_us"),
        "kernel_us_per_step": main_res.get("kernel_us_per_step"),
        **({"experts_with_tokens": main_res["experts_with_tokens"]} if "experts_with_tokens" in main_res else {}),
        "wall_s_timed_region": main_res["wall_s_timed_region"],
        "hbm_read_ceiling": ceiling,
        "cold_read_by_size": cold,
        "device": device_record(),
        "extra": extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

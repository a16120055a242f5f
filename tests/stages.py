"""Stage-by-stage parity: every tensor the layer stores between two kernels
is checked against the oracle's step computed from the GPU's own input to
that step.

A bf16 layer stores r, h, q/k/v, the rotated q and k, attn, r2, h2 and act.
Comparing only the layer's outputs against the bf16-storage oracle mixes two
things: the arithmetic error of each kernel, and the bf16 rounding flips that
any two bf16 pipelines make at different elements (an fp32 sum and an fp64
sum of the same 8192 products round to different bf16 values in about 0.3% of
elements), which the attention, the residual stream, the norm and the MLP then
carry forward and amplify.  Here each stage takes exactly the bf16 values the
GPU stored before it, so what remains is that kernel's own arithmetic:
    max_i (|gpu_i - ref_i| - ulp_bf16/2) <= 1e-2 * RMS(ref)   and   cos >= 0.9999
with ref the oracle's float64 value of the stage before its bf16 rounding
(ulp at the larger magnitude of the two), and the literal criterion for fp32
layers.  Stages, as the pages order the layer (oracle/layer.py):
  h            RMSNorm of r = bf16(hidden + residual)       (input_layernorm)
  k, v         the k and v projections of the GPU's h        (qkv_proj)
  q_rot        RoPE of bf16(q projection of the GPU's h)     (qkv_proj, rotary_emb;
               with a q/k norm, of bf16(RMSNorm(bf16(q)))); q is stored before
               the rotation too, so one more ulp of the pair's input is allowed
  k_cache      (q/k norm layers) RoPE of bf16(RMSNorm(bf16(k))), against the
               new K slots; without the norm those are checked bit for bit
  attn         softmax attention of the GPU's q_rot over the GPU's cache
  residual_out o_proj of the GPU's attn plus r                (o_proj)
  h2           RMSNorm of the GPU's residual_out              (post_attention_layernorm)
  act          SiluAndMul of the gate_up projection of the GPU's h2
  hidden_out   down_proj of the GPU's act
In a mixture-of-experts layer act and hidden_out give way to, per (token,
expert) pair of the GPU's routing (whose logits, choices and weights are
checked against the oracle's on their own):
  moe_act      SiluAndMul of the expert's gate_up projection of the GPU's h2
  moe_part     the GPU's routing weight times the expert's down projection of
               the GPU's moe_act
  hidden_out   the sum of the GPU's moe_part rows over the token's experts
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from tests.parity import compare, np64


def check_stages(model, wn: dict, batch, hidden, residual, kp, vp, ws: dict, ho, ro, rows=None) -> dict:
    """wn: float64 weights; hidden/residual: the layer's GPU inputs; kp/vp:
    the GPU's KV pools after the call; ws: GPU workspace tensors by name
    (workspace()); ho/ro: the GPU's outputs; rows: token rows to check
    (default all).  Returns the statistics per stage."""
    cfg = model.config_dict()
    dt = model.dtype
    H, nq, nkv, d = model.hidden_size, model.num_attention_heads, model.num_key_value_heads, model.head_dim
    eps = model.rms_norm_eps
    rows = list(range(batch.num_tokens)) if rows is None else list(rows)
    dev = hidden.device
    idx = torch.tensor(rows, device=dev, dtype=torch.long)
    g = {n: np64(ws[n][idx]) for n in ("h", "qkv", "attn", "h2", "act") if n in ws}
    rnd = oracle.bf16_round if dt == "bf16" else (lambda x: x)
    stats = {}

    def stage(name, got, ref):
        stats[name] = compare("stage " + name, got, ref, None, dt)

    x = np64(hidden[idx])
    r = rnd(x if residual is None else x + np64(residual[idx]))
    stage("h", g["h"], oracle.rms_norm(r, wn["input_layernorm"], eps))

    qkv = oracle.linear(g["h"], wn["qkv_proj"])
    stage("k", g["qkv"][:, nq * d:(nq + nkv) * d], qkv[:, nq * d:(nq + nkv) * d])
    stage("v", g["qkv"][:, (nq + nkv) * d:], qkv[:, (nq + nkv) * d:])
    freqs = oracle.rope_frequencies(d, cfg["rope_theta"], cfg.get("rope_scaling"))
    pos = batch.positions.numpy().astype(np.int64)[rows]
    q = rnd(qkv[:, :nq * d]).reshape(-1, nq, d)
    if model.qk_norm:
        q = rnd(oracle.rms_norm(q, wn["q_norm"], eps))
    # two storage points in one stage: q itself is stored (and overwritten by
    # its rotation), so a q element the GPU rounded the other way moves both
    # members of its rotated pair by up to one ulp of the pair's larger input
    q_rot = oracle.apply_rope(q, pos, freqs).reshape(len(rows), -1)
    half = d // 2
    big = np.maximum(np.abs(q[..., :half]), np.abs(q[..., half:]))
    slack = np.concatenate([big, big], axis=-1).reshape(len(rows), -1)
    stats["q_rot"] = compare("stage q_rot", g["qkv"][:, :nq * d], q_rot, None, dt,
                             extra_ulp_of=slack if dt == "bf16" else None)

    seq_of = batch.seq_of_row()
    if model.qk_norm:
        # the new K slots of these rows: RoPE of the normed, rounded k
        k = rnd(qkv[:, nq * d:(nq + nkv) * d]).reshape(-1, nkv, d)
        k = rnd(oracle.rms_norm(k, wn["k_norm"], eps))
        b_ = torch.tensor([seq_of[t] for t in rows], dtype=torch.long)
        p_ = torch.from_numpy(pos)
        blk = batch.block_table[b_, p_ // 16].long().to(dev)
        slot = (p_ % 16).to(dev)
        stage("k_cache", np64(kp[blk, :, slot, :]), oracle.apply_rope(k, pos, freqs))

    # attention of the GPU's rotated q over the GPU's cache (positions 0..p)
    qg = g["qkv"][:, :nq * d].reshape(-1, nq, d)
    ref = np.empty((len(rows), nq * d))
    by_seq = {}
    for i, t in enumerate(rows):
        by_seq.setdefault(seq_of[t], []).append(i)
    for b, items in by_seq.items():
        L = max(int(pos[i]) for i in items) + 1
        K = np64(synth.gather_context(kp, batch, b, L))
        V = np64(synth.gather_context(vp, batch, b, L, "v"))
        for i in items:
            p = int(pos[i])
            ref[i] = oracle.attend(qg[i], K[:p + 1], V[:p + 1]).reshape(-1)
    stage("attn", g["attn"], ref)

    r2 = np64(ro[idx])
    stage("residual_out", r2, oracle.linear(g["attn"], wn["o_proj"]) + r)
    stage("h2", g["h2"], oracle.rms_norm(r2, wn["post_attention_layernorm"], eps))

    out = np64(ho[idx])
    if cfg.get("num_experts", 0) > 0:
        # the GPU's routing (checked against the oracle's separately) decides
        # which expert each pair runs; each stage then takes the GPU's input
        k, I = cfg["num_experts_per_tok"], cfg["moe_intermediate_size"]
        T = batch.num_tokens
        ids = ws["topk_ids"].reshape(T, k)[idx].cpu().numpy().astype(np.int64)
        wts = np64(ws["topk_weights"].reshape(T, k)[idx])
        sorted_ = ws["moe_sorted"].reshape(-1).cpu().numpy().astype(np.int64)
        row_of_pair = np.empty_like(sorted_)
        row_of_pair[sorted_] = np.arange(sorted_.size)
        mact = ws["moe_act"].reshape(T * k, I)
        mpart = ws["moe_part"].reshape(T * k, H)
        pairs = (np.asarray(rows, np.int64)[:, None] * k + np.arange(k)[None, :]).reshape(-1)
        act = np64(mact[torch.from_numpy(row_of_pair[pairs]).to(dev)]).reshape(len(rows), k, I)
        part = np64(mpart[torch.from_numpy(pairs).to(dev)]).reshape(len(rows), k, H)
        act_ref = np.empty_like(act)
        part_ref = np.empty_like(part)
        for e in np.unique(ids):
            sel = np.nonzero(ids == e)
            act_ref[sel] = oracle.silu_and_mul(oracle.linear(g["h2"][sel[0]], wn["experts_gate_up"][e]))
            part_ref[sel] = wts[sel][:, None] * oracle.linear(act[sel], wn["experts_down"][e])
        stage("moe_act", act, act_ref)
        stage("moe_part", part, part_ref)
        stage("hidden_out", out, part.sum(axis=1))
    else:
        stage("act", g["act"], oracle.silu_and_mul(oracle.linear(g["h2"], wn["gate_up_proj"])))
        stage("hidden_out", out, oracle.linear(g["act"], wn["down_proj"]))
    return stats


def summary(stats: dict) -> str:
    """One line: each stage's largest excess over half an ulp, in RMS units."""
    parts = []
    for k, v in stats.items():
        if isinstance(v, dict):
            parts.append("%s %.4f" % (k, v.get("max_excess_rel", v.get("max_rel", 0.0))))
    return "stages (max excess / RMS): " + ", ".join(parts)


def workspace(layer, ws, T, B, max_seq_len) -> dict:
    """The workspace tensors a layer forward left: h, qkv, attn, h2 and act
    of a dense layer; the routing and the per-pair expert tensors in place of
    act in a mixture-of-experts layer."""
    moe = layer.cfg.get("num_experts", 0) > 0
    names = ("h", "qkv", "attn", "h2") + (("topk_ids", "topk_weights", "moe_sorted", "moe_act", "moe_part")
                                          if moe else ("act",))
    return {n: layer.workspace_tensor(ws, n, T, B, max_seq_len) for n in names}


def nan_report(ws: dict, outputs: dict) -> str:
    """Where non-finite values sit: for each workspace tensor (in the order
    the layer writes them) and output, the rows holding any.  Called only when
    an output is non-finite, so it adds no synchronisation to a good run."""
    parts = []
    for n in ("h", "qkv", "attn", "h2", "act"):
        if n in ws:
            bad = (~torch.isfinite(ws[n].float())).any(dim=1).nonzero().flatten().tolist()
            parts.append("%s rows %s" % (n, bad[:12] if bad else "none"))
    for n, t in outputs.items():
        bad = (~torch.isfinite(t.float())).any(dim=1).nonzero().flatten().tolist()
        parts.append("%s rows %s" % (n, bad[:12] if bad else "none"))
    return "non-finite values: " + "; ".join(parts)


"""Helpers shared by the GPU parity tests: run the oracle on the exact tensors
the library consumed, and compare under the stated tolerance.

Tolerance, per output tensor (bf16 layers).  `exact` is the float64 oracle
with nothing rounded; `R` is the same oracle storing every tensor in bf16 at
the points where a bf16 model stores it (the pages fix the model dtype as
bfloat16), its output rounded to bf16 as the GPU's is.  R's distance from
`exact` is what bf16 storage by itself costs; the GPU, which stores at the
same points but makes its own rounding decisions, may differ from `exact` by
that much plus the stated arithmetic budget:
  * cosine(gpu, exact) >= 0.9999;
  * max|gpu - exact| <= max|R - exact| + 1e-2 * RMS(exact);
  * RMS(gpu - exact) <= 2 * RMS(R - exact) + 1e-3 * RMS(exact)  (a guard
    against small systematic errors that the max would hide).
In a chain of layers the budget is per layer: the output of the l-th layer
(l = 0, 1, ...) carries the arithmetic of l+1 layers and is allowed
(l+1) * 1e-2 * RMS (and (l+1) * 1e-3 in the RMS guard) on top of R's distance.
With no R (a single kernel whose only storage point is its own output) the
max criterion is max(|gpu - exact| - ulp_bf16/2) <= 1e-2 * RMS(exact).
A literal max|gpu - exact| <= 1e-2 * RMS cannot hold for bf16 outputs of this
size: the output rounding alone reaches ~1.5e-2 RMS, and independent 1-ulp
rounding decisions at the internal storage points propagate to ~1e-2 RMS.
The literal figure and the distance to R are reported alongside.
fp32 layers: max|gpu - exact| <= 1e-2 * RMS(exact) and cosine >= 0.9999,
unchanged, plus a tighter 1e-4 check.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synth

COS_MIN = 0.9999
MAX_REL = 1e-2


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.ravel()
    b = b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def compare(name: str, gpu: np.ndarray, ref_exact: np.ndarray, ref_r: np.ndarray = None,
            dtype: str = "bf16", depth: int = 1) -> dict:
    """Asserts the tolerance; returns the statistics."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref_exact.shape, (name, gpu.shape, ref_exact.shape)
    assert np.all(np.isfinite(gpu)), "%s: non-finite values" % name
    cos = cosine(gpu, ref_exact)
    rms = math.sqrt(float(np.mean(ref_exact * ref_exact)))
    err = np.abs(gpu - ref_exact)
    stat = {"n": int(gpu.size), "cos": cos, "max_rel": float(err.max()) / rms,
            "rms_err_rel": math.sqrt(float(np.mean(err * err))) / rms}
    assert cos >= COS_MIN, (name, stat)
    if dtype != "bf16":
        assert stat["max_rel"] <= MAX_REL, (name, stat)
        assert stat["max_rel"] <= 1e-4, (name, stat)
        return stat
    if ref_r is None:
        excess = err - 0.5 * ulp_bf16(np.maximum(np.abs(ref_exact), np.abs(gpu)))
        stat["max_excess_rel"] = float(excess.max()) / rms
        assert stat["max_excess_rel"] <= MAX_REL, (name, stat)
        return stat
    rerr = np.abs(oracle.bf16_round(ref_r) - ref_exact)
    stat["bf16_oracle_max_rel"] = float(rerr.max()) / rms
    stat["bf16_oracle_rms_err_rel"] = math.sqrt(float(np.mean(rerr * rerr))) / rms
    d = np.abs(gpu - ref_r)
    stat["max_rel_vs_bf16_oracle"] = float(d.max()) / rms
    assert stat["max_rel"] <= stat["bf16_oracle_max_rel"] + depth * MAX_REL, (name, stat)
    assert stat["rms_err_rel"] <= 2 * stat["bf16_oracle_rms_err_rel"] + depth * 1e-3, (name, stat)
    return stat


def oracle_weights(weights: dict) -> dict:
    return {k: np64(v) for k, v in weights.items()}


def oracle_seqs(model: synth.ModelShape, batch: synth.Batch, k_pool, v_pool, seq_ids=None):
    """oracle.Seq per sequence: rows of its new tokens and its cached context
    read back (logical order) from the pools as they were before the call."""
    seqs = []
    ids = range(batch.num_seqs) if seq_ids is None else seq_ids
    for b in ids:
        c = batch.ctx_lens[b]
        kc = np64(synth.gather_context(k_pool, batch, b, c))
        vc = np64(synth.gather_context(v_pool, batch, b, c, "v"))
        seqs.append(oracle.Seq(list(batch.rows(b)), kc, vc))
    return seqs


def run_oracle(model, weights_np, hidden, residual, batch, seqs, want=None, both=True):
    """(exact, rounded) oracle results; `rounded` None for fp32 layers."""
    cfg = model.config_dict()
    h = np64(hidden)
    r = None if residual is None else np64(residual)
    pos = batch.positions.numpy().astype(np.int64)
    exact = oracle.decoder_layer(cfg, weights_np, h, r, pos, seqs, rnd=None, want=want)
    rounded = None
    if model.dtype == "bf16" and both:
        rounded = oracle.decoder_layer(cfg, weights_np, h, r, pos, seqs, rnd=oracle.bf16_round, want=want)
    return exact, rounded


def device_batch(batch: synth.Batch, device):
    return (batch.positions.to(device), batch.block_table.to(device), batch.seq_lens.to(device))


def device_qsl(batch: synth.Batch, device):
    """query_start_loc on the device, or None for a uniform batch."""
    q = batch.query_start_loc
    return None if q is None else q.to(device)


def moe_fix_routing(cfg: dict, w_np: dict, trace: dict, result: dict, gpu_ids: np.ndarray, rnd=None,
                    delta: float = 2e-2) -> int:
    """Where several expert sets are correct, compare what is unique and check
    that the rest is valid.  For every output row whose GPU expert set differs
    from the oracle's: the oracle's own choice must be within ``delta`` * RMS
    (router logits) of a tie, every GPU expert must be within that distance of
    the k-th best logit, and the row's expected output is then the oracle's
    mixture over the GPU's experts (weights from the oracle's logits).
    ``gpu_ids`` [rows, k] in the result's row order.  Updates
    result["hidden_out"] in place; returns the number of such rows."""
    rnd = rnd or (lambda x: x)
    logits = trace["router_logits"]
    ids = trace["topk_ids"]
    k = cfg["num_experts_per_tok"]
    tol = delta * math.sqrt(float(np.mean(logits * logits)))
    margins = oracle.topk_margin(logits, k)
    fixed = 0
    for i in range(ids.shape[0]):
        g = [int(e) for e in gpu_ids[i]]
        assert len(set(g)) == k, ("repeated expert", i, g)
        if set(g) == set(int(e) for e in ids[i]):
            continue
        assert margins[i] <= tol, ("expert sets differ on a clear choice", i, margins[i], tol)
        kth = np.sort(logits[i])[::-1][k - 1]
        assert all(logits[i, e] >= kth - tol for e in g), ("GPU expert far from the top k", i, g)
        p = oracle.softmax(logits[i:i + 1])[0][g]
        if cfg.get("norm_topk_prob", True):
            p = p / p.sum()
        result["hidden_out"][i] = oracle.mix_experts(trace["h2"][i:i + 1], np.array([g]), p[None, :],
                                                     w_np["experts_gate_up"], w_np["experts_down"], rnd)[0]
        fixed += 1
    return fixed


def moe_check_weights(cfg: dict, trace: dict, gpu_ids: np.ndarray, gpu_w: np.ndarray, gpu_logits: np.ndarray,
                      atol: float = 2e-3) -> None:
    """GPU router logits against the oracle's (1e-2 * RMS) and the GPU's
    routing weights against the oracle's probabilities of the GPU's experts."""
    logits = trace["router_logits"]
    rms = math.sqrt(float(np.mean(logits * logits)))
    err = float(np.abs(gpu_logits - logits).max())
    assert err <= 1e-2 * rms, ("router logits", err, rms)
    p = oracle.softmax(logits)
    sel = np.take_along_axis(p, gpu_ids.astype(np.int64), axis=1)
    if cfg.get("norm_topk_prob", True):
        sel = sel / sel.sum(axis=1, keepdims=True)
    assert float(np.abs(gpu_w - sel).max()) <= atol, ("routing weights", float(np.abs(gpu_w - sel).max()))
    # best first
    g = np.take_along_axis(gpu_logits, gpu_ids.astype(np.int64), axis=1)
    assert np.all(np.diff(g, axis=1) <= 0), "experts not listed best first"

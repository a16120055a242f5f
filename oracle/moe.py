"""CPU oracle of the Qwen3-MoE layer's own steps, in float64 numpy.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU baseline leg of ``bench.py`` use it;
it imports nothing from the library.

What the pages fix:

* the model: ``Qwen3MoeForCausalLM`` with its ``config.json`` (page "LLama",
  hotelren.com/news/2693952, section "Qwen3MoeForCausalLM"): hidden 2048, 32
  query and 4 KV heads of 128, 128 experts, 8 chosen per token, expert width
  ``moe_intermediate_size`` 768, ``norm_topk_prob`` true, rope_theta 1e7
  without scaling, rms_norm_eps 1e-6;
* the sparse block (same page, box "Qwen3MoeSparseMoeBlock"): a replicated
  linear gate gives each token one logit per expert, the token keeps its 8
  best experts, each expert is a two-layer FFN (2048 -> 768 -> 2048) and the
  outputs are summed weighted by the gate probabilities; there is no shared
  expert;
* the fused form (page "模型库与算子层 — 代码走读", vllm-learning.pages.dev,
  section "Fused MoE"): merged expert weights ``w13`` [E, 2I, H] (gate rows
  then up rows, as the dense gate_up_proj) and ``w2`` [E, H, I], the router a
  linear layer [E, H], top-k of the router output.

Readings where the pages are silent or disagree (each is listed with its
reason in the design notes):

* gate probabilities are the softmax of the router logits over all experts;
  ``norm_topk_prob`` true divides the kept k probabilities by their sum (so
  they are the softmax over the k kept logits).  The page's worked example
  (weights .1 .2 .2 .1 .05 .05 .1 .1, sum 0.9) is the un-normalised case;
* an expert's FFN is the dense layer's MLP with the expert's weights:
  silu(x Wg^T) * (x Wu^T), then the down projection;
* equal logits: the lower expert index ranks first;
* Qwen3 attention normalises each query and key head with an RMSNorm over
  head_dim (weights [head_dim], the model's eps) before RoPE (``qk_norm``).
  The pages name vLLM's qwen3_moe.py as the model file but do not print its
  attention; this step is that architecture's, switched by a config flag.

Precision: float64; ``rnd`` rounds at the points where a bf16 model stores a
tensor: the expert activations (``act``) and each expert's weighted output
before the sum over the k experts (``moe_part``).
"""
from __future__ import annotations

import numpy as np

from .layer import linear, rms_norm, silu_and_mul


def _identity(x):
    return x


def softmax(z: np.ndarray) -> np.ndarray:
    """Row-wise softmax, shifted by the row maximum."""
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def router_logits(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """[T, E] = x Wr^T with the router stored [E, H]."""
    return linear(x, router_w)


def select_experts(logits: np.ndarray, top_k: int, norm_topk_prob: bool = True):
    """(ids [T, k], weights [T, k]) of each token: the k largest gate
    probabilities, best first (equal ones: lower expert index first), and
    their probabilities, divided by their sum when ``norm_topk_prob``."""
    p = softmax(logits)
    T, E = p.shape
    ids = np.empty((T, top_k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-p[t, e], e))
        ids[t] = order[:top_k]
    w = np.take_along_axis(p, ids, axis=1)
    if norm_topk_prob:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


def expert_ffn(x: np.ndarray, w13_e: np.ndarray, w2_e: np.ndarray, rnd=_identity) -> np.ndarray:
    """One expert on rows x: down(silu(gate) * up) with w13_e [2I, H] = [gate |
    up] and w2_e [H, I]."""
    act = rnd(silu_and_mul(linear(x, w13_e)))
    return linear(act, w2_e)


def mix_experts(x: np.ndarray, ids: np.ndarray, weights: np.ndarray, w13: np.ndarray, w2: np.ndarray,
                rnd=_identity) -> np.ndarray:
    """Sum over each token's chosen experts of weight * expert(x); each
    weighted expert output is stored (``rnd``) before the sum, which runs in
    the order of ``ids``.  Tokens sharing an expert go through it together."""
    T, k = ids.shape
    parts = np.zeros((T, k, x.shape[1]))
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        y = expert_ffn(x[rows], w13[e], w2[e], rnd)
        parts[rows, slots] = rnd(weights[rows, slots][:, None] * y)
    out = parts[:, 0].copy()
    for j in range(1, k):
        out += parts[:, j]
    return out


def sparse_moe_block(x: np.ndarray, router_w: np.ndarray, w13: np.ndarray, w2: np.ndarray, top_k: int,
                     norm_topk_prob: bool = True, rnd=None) -> dict:
    """The whole block on rows x [T, H].  Returns ``out`` [T, H] (unrounded),
    ``logits``, ``ids`` and ``weights``."""
    rnd = rnd or _identity
    logits = router_logits(x, router_w)
    ids, w = select_experts(logits, top_k, norm_topk_prob)
    return {"out": mix_experts(x, ids, w, w13, w2, rnd), "logits": logits, "ids": ids, "weights": w}


def head_rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x [T, heads, d]: each head vector divided by the root of its mean
    square plus eps, times w [d]."""
    return rms_norm(x, w, eps)


def topk_margin(logits: np.ndarray, top_k: int) -> np.ndarray:
    """Per token, the k-th largest logit minus the (k+1)-th: how far the
    choice of experts is from a tie (inf when every expert is kept)."""
    s = -np.sort(-logits, axis=1)
    if top_k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, top_k - 1] - s[:, top_k]

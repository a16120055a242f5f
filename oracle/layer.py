"""CPU oracle of one Llama decoder-layer forward, in float64 numpy.

TEST INFRASTRUCTURE.  This is the plain, slow reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it; the library never does, and this
module imports nothing from the library.

It follows the layer exactly as the pages describe it, one step per function:

* fused residual add + RMSNorm -- page "LLama" (hotelren.com/news/2693952),
  section "3 input_layernorm (RMSNorm)": with no incoming residual the hidden
  state itself becomes the residual; otherwise the pair is added and the sum
  becomes the residual, and the normalised sum is the hidden state.
* merged qkv projection and its split into q, k, v in that order, RoPE on q
  and k only, attention, o_proj -- same page, section "4 LlamaAttention"
  (forward code); "vLLM Llama 代码解析" (yeyulingfeng.com/a/605382), section
  "4.LlamaAttention".
* KV written to the cache before attention reads it -- "模型库与算子层 — 代码走读"
  (vllm-learning.pages.dev/topics/model-layers/code-walkthrough), section
  "Attention 层".
* post_attention_layernorm, merged gate_up projection, SiluAndMul
  (silu of the first half times the second half), down_proj -- "LLama"
  page, sections "post_attention_layernorm" and "LlamaMLP" (FFN formula and
  the SiluAndMul docstring); yeyulingfeng page, section "5.LlamaMLP".
* the (hidden, residual) pair handed from layer to layer -- yeyulingfeng page,
  section "2.1 LlamaModel.forward()".
* linear layers compute y = x W^T with W stored [out, in] -- vllm-learning
  page, section "Linear 层" (F.linear).

Readings where the pages are silent (each is listed with its reason in the
design notes): RMSNorm is x / sqrt(mean(x^2) + eps) * w; RoPE rotates the
pairs (i, i + d/2) by angle position * w_i with w_i = theta^(-2i/d), rescaled
by the published llama3 rule for the ``rope_scaling`` parameters of the
config; the attention scale is 1/sqrt(head_dim); a query at position p sees
keys 0..p including itself; query head h reads KV head h // (heads/kv_heads);
K/V of a sequence are kept here in logical (position) order, never paged.

Precision: everything is float64.  ``rnd`` optionally rounds to bfloat16
(round to nearest even) at the points where a bf16 model stores a tensor
(``STORAGE_POINTS``): the pages fix the model dtype as bfloat16 (config
``torch_dtype``), so that is the precision at which the model's tensors
exist between operations.  With ``rnd=None`` nothing is rounded.  The two
returned outputs are always left unrounded.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

STORAGE_POINTS = ("r", "h", "qkv", "q_norm", "k_norm", "q_rot", "k_rot", "attn", "r2", "h2", "act",
                  "moe_part")


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even.  x = m * 2^e with 0.5 <= |m| < 1 keeps round(m * 2^8)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0), e - 8)


def _identity(x):
    return x


# ---------------------------------------------------------------- RMSNorm --

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Each row divided by the root of its mean square plus eps, times w."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def fused_add_rms_norm(x, residual, w, eps, rnd=_identity):
    """Returns (normed, new_residual).  residual None: the input itself is the
    residual; otherwise input + residual is."""
    r = x.copy() if residual is None else x + residual
    r = rnd(r)
    return rnd(rms_norm(r, w, eps)), r


# ------------------------------------------------------------------- RoPE --

def rope_frequencies(head_dim: int, theta: float, scaling: Optional[dict]) -> np.ndarray:
    """Angular frequency of each rotated pair i = 0 .. head_dim/2 - 1.

    Base: w_i = theta^(-2i/head_dim).  With ``rope_type == "llama3"`` each
    frequency is rescaled by its wavelength L = 2*pi/w against
    orig/high and orig/low (orig = original_max_position_embeddings):
    short wavelengths (L < orig/high) keep w, long ones (L > orig/low) take
    w/factor, and in between w is blended as (1 - s) * w/factor + s * w with
    s = (orig/L - low) / (high - low).
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    w = theta ** (-2.0 * i / head_dim)
    if not scaling or scaling.get("rope_type", "default") == "default":
        return w
    if scaling["rope_type"] != "llama3":
        raise ValueError("unsupported rope_type %r" % scaling["rope_type"])
    factor = float(scaling["factor"])
    low = float(scaling["low_freq_factor"])
    high = float(scaling["high_freq_factor"])
    orig = float(scaling["original_max_position_embeddings"])
    out = np.empty_like(w)
    for j in range(w.size):
        wavelen = 2.0 * math.pi / w[j]
        if wavelen < orig / high:
            out[j] = w[j]
        elif wavelen > orig / low:
            out[j] = w[j] / factor
        else:
            s = (orig / wavelen - low) / (high - low)
            out[j] = (1.0 - s) * w[j] / factor + s * w[j]
    return out


def apply_rope(x: np.ndarray, positions: np.ndarray, freqs: np.ndarray) -> np.ndarray:
    """x [T, heads, d]; pair (i, i + d/2) of a token at position p turns by
    the angle p * freqs[i]:  (a, b) -> (a cos - b sin, b cos + a sin)."""
    half = x.shape[-1] // 2
    ang = positions.astype(np.float64)[:, None] * freqs[None, :]      # [T, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# -------------------------------------------------------------- attention --

def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """One query token.  q [heads, d]; keys, values [L, kv_heads, d] are the
    keys this query may see.  Query head h uses KV head h // (heads/kv_heads);
    weights are softmax(q.k / sqrt(d)) over the L keys."""
    nq, d = q.shape
    nkv = keys.shape[1]
    group = nq // nkv
    out = np.empty((nq, d))
    for g in range(nkv):
        qg = q[g * group:(g + 1) * group]                  # [group, d]
        s = qg @ keys[:, g, :].T / math.sqrt(d)            # [group, L]
        s = s - s.max(axis=1, keepdims=True)
        a = np.exp(s)
        a = a / a.sum(axis=1, keepdims=True)
        out[g * group:(g + 1) * group] = a @ values[:, g, :]
    return out


# -------------------------------------------------------------------- MLP --

def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_and_mul(x: np.ndarray) -> np.ndarray:
    """silu(x[..., :d]) * x[..., d:] with d = last dim // 2 (gate first)."""
    d = x.shape[-1] // 2
    return silu(x[..., :d]) * x[..., d:]


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T, W stored [out, in]."""
    return x @ w.T


# ------------------------------------------------------------------ layer --

class Seq:
    """One sequence of the batch: its token rows in ``hidden`` and its cached
    context (K already rotated) in logical order [ctx_len, kv_heads, d]."""

    def __init__(self, rows: Sequence[int], k_ctx: np.ndarray, v_ctx: np.ndarray):
        self.rows = list(rows)
        self.k_ctx = k_ctx
        self.v_ctx = v_ctx


def decoder_layer(cfg: dict, w: dict, hidden: np.ndarray, residual: Optional[np.ndarray],
                  positions: np.ndarray, seqs: Sequence[Seq], rnd=None,
                  want: Optional[Sequence[int]] = None, trace: Optional[dict] = None) -> dict:
    """One layer forward.

    cfg: config.json-style dict; w: float64 weights (input_layernorm,
    qkv_proj, o_proj, post_attention_layernorm, gate_up_proj, down_proj; a
    mixture-of-experts layer -- ``cfg["num_experts"]`` > 0 -- has router
    [E, H], experts_gate_up [E, 2I, H] and experts_down [E, H, I] in place of
    the last two, and ``cfg["qk_norm"]`` adds q_norm, k_norm [head_dim]);
    hidden/residual [T, H] (residual may be None); positions [T]; seqs the
    batch's sequences; rnd None or ``bf16_round``.

    ``trace``, if a dict, receives the intermediate tensors (for locating a
    disagreement): h [needed rows], q (rotated) [wanted rows], k (rotated)
    and v [needed rows], attn, h2, act [wanted rows], plus the row lists.

    ``want`` restricts the outputs to these token rows (default: all).  K/V
    are still computed for every row of a wanted row's sequence up to that
    row's position, since attention needs them.

    Returns dict with ``rows`` (output row order), ``hidden_out`` and
    ``residual_out`` [len(rows), H] (unrounded), and per sequence the new
    K (rotated) and V it appends: ``k_new[i]``, ``v_new[i]`` [n, kv, d] for
    the first n new tokens of ``seqs[i]`` that were computed.
    """
    rnd = rnd or _identity
    H = cfg["hidden_size"]
    nq, nkv, d = cfg["num_attention_heads"], cfg["num_key_value_heads"], cfg["head_dim"]
    eps = cfg["rms_norm_eps"]
    freqs = rope_frequencies(d, cfg["rope_theta"], cfg.get("rope_scaling"))
    T = hidden.shape[0]
    want = list(range(T)) if want is None else list(want)
    wanted = set(want)

    # rows that must go through norm + K/V projection: every new token of a
    # sequence up to the largest wanted position in it
    seq_of_row, need_rows, kv_count = {}, [], []
    for si, sq in enumerate(seqs):
        for j, row in enumerate(sq.rows):
            seq_of_row[row] = (si, j)
        idx = [j for j, row in enumerate(sq.rows) if row in wanted]
        n = (max(idx) + 1) if idx else 0
        kv_count.append(n)
        need_rows.extend(sq.rows[:n])
    need_pos = {row: k for k, row in enumerate(need_rows)}
    need = np.array(need_rows, dtype=np.int64)

    # input_layernorm with the fused residual add
    res_in = None if residual is None else residual[need]
    h, r = fused_add_rms_norm(hidden[need], res_in, w["input_layernorm"], eps, rnd)

    # merged qkv projection, split q | k | v; q only for wanted rows
    wq = w["qkv_proj"][: nq * d]
    wkv = w["qkv_proj"][nq * d:]
    kv = rnd(linear(h, wkv))
    k = kv[:, : nkv * d].reshape(-1, nkv, d)
    v = kv[:, nkv * d:].reshape(-1, nkv, d)
    want_idx = np.array([need_pos[row] for row in want], dtype=np.int64)
    q = rnd(linear(h[want_idx], wq)).reshape(-1, nq, d)

    # Qwen3: per-head RMSNorm of q and k before RoPE (oracle/moe.py)
    if cfg.get("qk_norm"):
        k = rnd(rms_norm(k, w["k_norm"], eps))
        q = rnd(rms_norm(q, w["q_norm"], eps))

    # RoPE on q and k only
    pos_need = positions[need]
    k = rnd(apply_rope(k, pos_need, freqs))
    q = rnd(apply_rope(q, positions[want], freqs))

    # KV append (logical order), then attention over positions 0..p
    k_new, v_new, k_all, v_all = [], [], [], []
    for si, sq in enumerate(seqs):
        n = kv_count[si]
        sel = np.array([need_pos[row] for row in sq.rows[:n]], dtype=np.int64)
        kn = k[sel] if n else np.zeros((0, nkv, d))
        vn = v[sel] if n else np.zeros((0, nkv, d))
        if n:
            p0 = int(positions[sq.rows[0]])
            if p0 != sq.k_ctx.shape[0] or any(int(positions[row]) != p0 + j
                                               for j, row in enumerate(sq.rows)):
                raise ValueError("positions must continue the cached context")
        k_new.append(kn)
        v_new.append(vn)
        k_all.append(np.concatenate([sq.k_ctx, kn], axis=0))
        v_all.append(np.concatenate([sq.v_ctx, vn], axis=0))

    attn = np.empty((len(want), nq * d))
    for i, row in enumerate(want):
        si, _ = seq_of_row[row]
        p = int(positions[row])
        attn[i] = attend(q[i], k_all[si][: p + 1], v_all[si][: p + 1]).reshape(-1)
    attn = rnd(attn)

    # o_proj, post_attention_layernorm with the fused residual add
    y = linear(attn, w["o_proj"])
    r_w = r[want_idx]
    r2 = y + r_w
    h2, r2s = fused_add_rms_norm(y, r_w, w["post_attention_layernorm"], eps, rnd)

    if cfg.get("num_experts", 0) > 0:
        # sparse MoE block in place of the MLP (oracle/moe.py)
        from .moe import sparse_moe_block
        moe = sparse_moe_block(h2, w["router"], w["experts_gate_up"], w["experts_down"],
                               cfg["num_experts_per_tok"], cfg.get("norm_topk_prob", True), rnd)
        out = moe["out"]
        act = None
    else:
        # gate_up projection, SiluAndMul, down projection
        act = rnd(silu_and_mul(linear(h2, w["gate_up_proj"])))
        out = linear(act, w["down_proj"])
        moe = None
    if trace is not None:
        trace.update({"need_rows": need_rows, "want_rows": want, "h": h, "q": q, "k": k, "v": v,
                      "attn": attn, "h2": h2, "act": act})
        if moe is not None:
            trace.update({"router_logits": moe["logits"], "topk_ids": moe["ids"], "topk_weights": moe["weights"]})
    return {"rows": want, "hidden_out": out, "residual_out": r2,
            "k_new": k_new, "v_new": v_new}


def decoder_stack(cfg: dict, layers: Sequence[dict], hidden, residual, positions,
                  seqs_per_layer: Sequence[Sequence[Seq]], rnd=None,
                  want: Optional[Sequence[int]] = None) -> list:
    """Consecutive layers, each with its own weights and KV cache, handing the
    (hidden, residual) pair on.  Between layers the pair is stored in the
    model dtype (``rnd``), as a bf16 model stores it.  Returns each layer's
    result dict (rows relative to the original batch)."""
    rnd_ = rnd or _identity
    if want is not None and any(len(s.rows) > 1 for s in seqs_per_layer[0]):
        raise ValueError("a row subset through a stack needs one token per sequence")
    outs = []
    h, r = hidden, residual
    rows = list(range(hidden.shape[0])) if want is None else list(want)
    for li, w in enumerate(layers):
        o = decoder_layer(cfg, w, h, r, positions, seqs_per_layer[li], rnd=rnd, want=rows)
        outs.append(o)
        hn = np.zeros_like(hidden)
        rn = np.zeros_like(hidden)
        hn[rows] = rnd_(o["hidden_out"])
        rn[rows] = rnd_(o["residual_out"])
        h, r = hn, rn
    return outs


def model_forward(cfg: dict, layers: Sequence[dict], final_norm_w: np.ndarray, hidden, positions,
                  seqs_per_layer: Sequence[Sequence[Seq]], rnd=None):
    """The model body without embedding and lm_head.  The layers run in order,
    the first with no residual, each handing (hidden, residual) to the next;
    the final RMSNorm then normalises hidden + residual -- page "LLama"
    (hotelren.com/news/2693952), section "最终 RMSNorm"; page
    yeyulingfeng.com/a/605382.html, section "2.1 LlamaModel.forward()" (its
    third step, the final norm of the pair).  Returns (output, per-layer
    result dicts)."""
    rnd_ = rnd or _identity
    outs = decoder_stack(cfg, layers, hidden, None, positions, seqs_per_layer, rnd=rnd)
    h = rnd_(outs[-1]["hidden_out"])
    r = rnd_(outs[-1]["residual_out"])
    out, _ = fused_add_rms_norm(h, r, final_norm_w, cfg["rms_norm_eps"], rnd=rnd_)
    return out, outs

"""Pins for the mixture-of-experts steps of the CPU oracle (oracle/moe.py) and
the Qwen3 attention extra (per-head q/k RMSNorm): the page's worked router
example, brute force written as plain loops on tiny inputs, special cases that
reduce to the dense MLP, and invariants.  Each targets a plausible slip: a
softmax over the kept logits only, a missing renormalisation, a router row
paired with the wrong expert, transposed expert weights, a sum that drops an
expert, a norm over the wrong axis."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _moe_weights(rng, E, H, I, scale=0.3):
    return (scale * rng.standard_normal((E, H)), scale * rng.standard_normal((E, 2 * I, H)),
            scale * rng.standard_normal((E, H, I)))


# ------------------------------------------------------- the pages' values --

def test_golden_qwen3_config_and_shapes():
    with open(os.path.join(GOLDEN, "qwen3moe_config.json")) as f:
        g = json.load(f)
    c = g["config"]
    m = synth.QWEN3MOE
    for key in ("hidden_size", "num_attention_heads", "num_key_value_heads", "head_dim",
                "intermediate_size", "rms_norm_eps", "rope_theta", "max_position_embeddings",
                "num_experts", "num_experts_per_tok", "moe_intermediate_size", "norm_topk_prob"):
        assert getattr(m, key) == c[key], key
    assert m.rope_scaling is None and c["rope_scaling"] is None
    assert c["hidden_act"] == "silu" and not c["attention_bias"]
    assert c["decoder_sparse_step"] == 1 and c["mlp_only_layers"] == []  # every layer sparse
    assert m.q_size == g["derived"]["q_size"] and m.kv_size == g["derived"]["kv_size"]
    w = synth.draw_weights(synth.ModelShape(64, 4, 2, 16, 128, 1e-6, 1e7, None, 64, "fp32",
                                            num_experts=8, num_experts_per_tok=2, moe_intermediate_size=24),
                           0, 0, "cpu")
    assert tuple(w["experts_gate_up"].shape) == (8, 48, 64)   # [E, 2I, H] as the fused layer's w13
    assert tuple(w["experts_down"].shape) == (8, 64, 24)      # [E, H, I] as its w2
    assert tuple(w["router"].shape) == (8, 64)


def test_router_worked_example():
    """Logits whose softmax puts the example's probabilities on its eight
    experts (and 0.1 spread over the other 120): the kept experts are exactly
    those eight, best first; without renormalisation their weights are the
    example's, with it (norm_topk_prob) the example's divided by 0.9."""
    with open(os.path.join(GOLDEN, "router_example.json")) as f:
        g = json.load(f)
    E, k = g["num_experts"], g["top_k"]
    experts, weights = g["experts"], g["weights"]
    p = np.full(E, (1.0 - sum(weights)) / (E - k))
    p[experts] = weights
    logits = np.log(p)[None, :] + 3.7          # any shift: softmax is shift-invariant
    ids, w = oracle.select_experts(logits, k, norm_topk_prob=False)
    assert sorted(ids[0].tolist()) == sorted(experts)
    # best first, equal probabilities in expert order
    assert ids[0].tolist() == [7, 9, 0, 34, 110, 127, 77, 89]
    want = dict(zip(experts, weights))
    np.testing.assert_allclose(w[0], [want[e] for e in ids[0]], rtol=1e-12)
    assert abs(w[0].sum() - 0.9) < 1e-12
    _, wn = oracle.select_experts(logits, k, norm_topk_prob=True)
    np.testing.assert_allclose(wn[0], [want[e] / 0.9 for e in ids[0]], rtol=1e-12)


# ------------------------------------------------------------- brute force --

def _silu(z):
    return z / (1.0 + math.exp(-z))


def _moe_loops(x, router_w, w13, w2, k, norm):
    """The block for one token at a time in plain Python loops."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    out = np.zeros((T, H))
    for t in range(T):
        logit = [sum(x[t, h] * router_w[e, h] for h in range(H)) for e in range(E)]
        m = max(logit)
        ex = [math.exp(v - m) for v in logit]
        tot = sum(ex)
        prob = [v / tot for v in ex]
        order = sorted(range(E), key=lambda e: (-prob[e], e))[:k]
        wsum = sum(prob[e] for e in order) if norm else 1.0
        for e in order:
            gate = [sum(x[t, h] * w13[e, i, h] for h in range(H)) for i in range(I)]
            up = [sum(x[t, h] * w13[e, I + i, h] for h in range(H)) for i in range(I)]
            act = [_silu(gate[i]) * up[i] for i in range(I)]
            for o in range(H):
                out[t, o] += prob[e] / wsum * sum(act[i] * w2[e, o, i] for i in range(I))
    return out


@pytest.mark.parametrize("k,norm", [(2, True), (3, False), (1, True), (5, True)])
def test_sparse_moe_block_brute_force(k, norm):
    rng = np.random.default_rng(11 + k)
    E, H, I, T = 5, 6, 4, 7           # H != I so a transposed expert weight cannot pass
    router_w, w13, w2 = _moe_weights(rng, E, H, I)
    x = rng.standard_normal((T, H))
    got = oracle.sparse_moe_block(x, router_w, w13, w2, k, norm)
    np.testing.assert_allclose(got["out"], _moe_loops(x, router_w, w13, w2, k, norm), rtol=1e-11, atol=1e-12)
    assert got["ids"].shape == (T, k) and got["weights"].shape == (T, k)
    if norm:
        np.testing.assert_allclose(got["weights"].sum(axis=1), 1.0, rtol=1e-12)


# ----------------------------------------------------------- special cases --

def _dense_mlp(x, gate_up, down):
    I = gate_up.shape[0] // 2
    g = x @ gate_up[:I].T
    u = x @ gate_up[I:].T
    return (g / (1.0 + np.exp(-g)) * u) @ down.T


def test_identical_experts_reduce_to_the_dense_mlp():
    """With every expert the same FFN the renormalised weights sum to one, so
    the block is that FFN whatever the router chooses."""
    rng = np.random.default_rng(3)
    E, H, I, T = 6, 8, 5, 9
    router_w, w13, w2 = _moe_weights(rng, E, H, I)
    w13[:] = w13[0]
    w2[:] = w2[0]
    x = rng.standard_normal((T, H))
    got = oracle.sparse_moe_block(x, router_w, w13, w2, 3, True)["out"]
    np.testing.assert_allclose(got, _dense_mlp(x, w13[0], w2[0]), rtol=1e-11, atol=1e-12)


def test_dominant_expert_top1_is_that_expert():
    """top_k = 1 keeps one expert with weight exactly 1 after renormalising:
    the output is that expert's FFN, and the router picks the expert whose
    router row aligns with the token."""
    rng = np.random.default_rng(4)
    E, H, I = 6, 8, 5
    _, w13, w2 = _moe_weights(rng, E, H, I)
    router_w = np.zeros((E, H))
    router_w[np.arange(E), np.arange(E)] = 10.0        # expert e listens to feature e
    x = np.zeros((E, H))
    x[np.arange(E), (np.arange(E) * 5) % E] = 1.0       # token t speaks feature 5t mod E
    got = oracle.sparse_moe_block(x, router_w, w13, w2, 1, True)
    np.testing.assert_array_equal(got["ids"][:, 0], (np.arange(E) * 5) % E)
    np.testing.assert_allclose(got["weights"], 1.0)
    for t in range(E):
        e = got["ids"][t, 0]
        np.testing.assert_allclose(got["out"][t], _dense_mlp(x[t:t + 1], w13[e], w2[e])[0], rtol=1e-12)


def test_all_experts_kept_is_the_softmax_mixture():
    rng = np.random.default_rng(5)
    E, H, I, T = 4, 6, 3, 5
    router_w, w13, w2 = _moe_weights(rng, E, H, I)
    x = rng.standard_normal((T, H))
    got = oracle.sparse_moe_block(x, router_w, w13, w2, E, False)["out"]
    z = x @ router_w.T
    p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    want = sum(p[:, e:e + 1] * _dense_mlp(x, w13[e], w2[e]) for e in range(E))
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_expert_permutation_invariance():
    """Relabelling the experts (router rows and expert weights together)
    changes the chosen ids by the relabelling and nothing else."""
    rng = np.random.default_rng(6)
    E, H, I, T = 7, 8, 4, 10
    router_w, w13, w2 = _moe_weights(rng, E, H, I)
    x = rng.standard_normal((T, H))
    perm = rng.permutation(E)                # new expert j is old expert perm[j]
    a = oracle.sparse_moe_block(x, router_w, w13, w2, 3, True)
    b = oracle.sparse_moe_block(x, router_w[perm], w13[perm], w2[perm], 3, True)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-13)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(np.sort(inv[a["ids"]], axis=1), np.sort(b["ids"], axis=1))


def test_topk_margin_and_tie_order():
    logits = np.array([[0.5, 2.0, 2.0, -1.0, 1.0]])
    np.testing.assert_allclose(oracle.topk_margin(logits, 2), [1.0])
    np.testing.assert_allclose(oracle.topk_margin(logits, 1), [0.0])     # a tie at the boundary
    ids, _ = oracle.select_experts(logits, 3)
    assert ids[0].tolist() == [1, 2, 4]
    assert np.isinf(oracle.topk_margin(logits, 5)[0])


# ------------------------------------------------------ the Qwen3 layer --

def _qcfg(E=4, k=2, qk_norm=True, Ie=24):
    return {"hidden_size": 32, "num_attention_heads": 4, "num_key_value_heads": 2, "head_dim": 8,
            "intermediate_size": 40, "rms_norm_eps": 1e-6, "rope_theta": 1e7, "rope_scaling": None,
            "num_experts": E, "num_experts_per_tok": k, "moe_intermediate_size": Ie,
            "norm_topk_prob": True, "qk_norm": qk_norm}


def _qweights(cfg, rng):
    H, nq, nkv, d = (cfg["hidden_size"], cfg["num_attention_heads"], cfg["num_key_value_heads"],
                     cfg["head_dim"])
    E, Ie = cfg["num_experts"], cfg["moe_intermediate_size"]
    router_w, w13, w2 = _moe_weights(rng, E, H, Ie, 0.2)
    return {"input_layernorm": 1 + 0.3 * rng.standard_normal(H),
            "qkv_proj": 0.2 * rng.standard_normal(((nq + 2 * nkv) * d, H)),
            "o_proj": 0.2 * rng.standard_normal((H, nq * d)),
            "post_attention_layernorm": 1 + 0.3 * rng.standard_normal(H),
            "router": router_w, "experts_gate_up": w13, "experts_down": w2,
            "q_norm": 1 + 0.3 * rng.standard_normal(d), "k_norm": 1 + 0.3 * rng.standard_normal(d)}


def test_single_expert_layer_is_the_dense_layer():
    """One expert, top-1, no q/k norm: the MoE layer is the dense layer with
    that expert as its MLP."""
    rng = np.random.default_rng(8)
    cfg = _qcfg(E=1, k=1, qk_norm=False)
    w = _qweights(cfg, rng)
    T = 6
    x = rng.standard_normal((T, 32))
    r = rng.standard_normal((T, 32))
    seqs = [oracle.Seq(range(T), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)))]
    got = oracle.decoder_layer(cfg, w, x, r, np.arange(T), seqs)
    dense_cfg = dict(cfg, num_experts=0)
    dw = {n: w[n] for n in ("input_layernorm", "qkv_proj", "o_proj", "post_attention_layernorm")}
    dw["gate_up_proj"] = w["experts_gate_up"][0]
    dw["down_proj"] = w["experts_down"][0]
    dense_cfg["intermediate_size"] = cfg["moe_intermediate_size"]
    want = oracle.decoder_layer(dense_cfg, dw, x, r, np.arange(T), seqs)
    np.testing.assert_allclose(got["hidden_out"], want["hidden_out"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["residual_out"], want["residual_out"], rtol=1e-12, atol=1e-13)


def test_qk_norm_normalises_each_head_before_rope():
    """With unit q/k norm weights every rotated query and key head has norm
    sqrt(head_dim) (RoPE keeps norms; the norm is per head, not per row)."""
    rng = np.random.default_rng(9)
    cfg = _qcfg()
    w = _qweights(cfg, rng)
    w["q_norm"] = np.ones(8)
    w["k_norm"] = np.ones(8)
    cfg["rms_norm_eps"] = 1e-12
    T = 5
    tr = {}
    x = 3.0 * rng.standard_normal((T, 32))
    seqs = [oracle.Seq(range(T), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)))]
    oracle.decoder_layer(cfg, w, x, None, np.arange(T), seqs, trace=tr)
    np.testing.assert_allclose(np.linalg.norm(tr["q"], axis=-1), math.sqrt(8), rtol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(tr["k"], axis=-1), math.sqrt(8), rtol=1e-9)
    # and the weights scale each head component-wise: a weight of 2 on one
    # component doubles that component of the normalised (pre-RoPE) head at
    # position 0, where RoPE is the identity
    w["k_norm"] = np.ones(8)
    w["k_norm"][3] = 2.0
    tr2 = {}
    oracle.decoder_layer(cfg, w, x, None, np.arange(T), seqs, trace=tr2)
    np.testing.assert_allclose(tr2["k"][0, :, 3], 2.0 * tr["k"][0, :, 3], rtol=1e-12)
    np.testing.assert_allclose(np.delete(tr2["k"][0], 3, axis=-1), np.delete(tr["k"][0], 3, axis=-1),
                               rtol=1e-12)


def test_head_rms_norm_closed_form():
    x = np.full((2, 3, 4), -0.5)
    w = np.array([1.0, 2.0, 3.0, 4.0])
    eps = 1e-3
    got = oracle.head_rms_norm(x, w, eps)
    np.testing.assert_allclose(got, np.broadcast_to(-0.5 / math.sqrt(0.25 + eps) * w, x.shape), rtol=1e-13)


def test_moe_layer_traces_routing():
    rng = np.random.default_rng(10)
    cfg = _qcfg(E=6, k=2)
    w = _qweights(cfg, rng)
    T = 7
    tr = {}
    x = rng.standard_normal((T, 32))
    seqs = [oracle.Seq(range(T), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)))]
    out = oracle.decoder_layer(cfg, w, x, None, np.arange(T), seqs, trace=tr)
    np.testing.assert_allclose(tr["router_logits"], tr["h2"] @ w["router"].T, rtol=1e-12)
    mix = oracle.mix_experts(tr["h2"], tr["topk_ids"], tr["topk_weights"], w["experts_gate_up"],
                             w["experts_down"])
    np.testing.assert_allclose(out["hidden_out"], mix, rtol=1e-12)

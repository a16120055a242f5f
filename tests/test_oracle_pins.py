"""Pins for the CPU oracle: each test ties one oracle step to something other
than the oracle itself -- a closed form, an invariant, a library routine of
torch (an independent implementation), brute force on a tiny input, or the
values the pages print.  A plausible slip (dropped term, wrong sign or index,
transposed operand, swapped halves) fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _cfg(H=64, nq=4, nkv=2, d=16, I=96, theta=1e4, scaling=None, eps=1e-5):
    return {"hidden_size": H, "num_attention_heads": nq, "num_key_value_heads": nkv,
            "head_dim": d, "intermediate_size": I, "rms_norm_eps": eps,
            "rope_theta": theta, "rope_scaling": scaling}


def _weights(cfg, rng, norm_std=0.5):
    H, nq, nkv, d, I = (cfg["hidden_size"], cfg["num_attention_heads"],
                        cfg["num_key_value_heads"], cfg["head_dim"], cfg["intermediate_size"])
    return {
        "input_layernorm": 1.0 + norm_std * rng.standard_normal(H),
        "qkv_proj": 0.2 * rng.standard_normal(((nq + 2 * nkv) * d, H)),
        "o_proj": 0.2 * rng.standard_normal((H, nq * d)),
        "post_attention_layernorm": 1.0 + norm_std * rng.standard_normal(H),
        "gate_up_proj": 0.2 * rng.standard_normal((2 * I, H)),
        "down_proj": 0.2 * rng.standard_normal((H, I)),
    }


# ------------------------------------------------------------------ bf16 --

def test_bf16_round_ties_to_even():
    u = 2.0 ** -7                       # bf16 spacing in [1, 2)
    assert oracle.bf16_round(1.0 + u / 2) == 1.0            # tie -> even (1.0)
    assert oracle.bf16_round(1.0 + 3 * u / 2) == 1.0 + 2 * u  # tie -> even
    assert oracle.bf16_round(1.0 + 0.51 * u) == 1.0 + u
    assert oracle.bf16_round(-3.0) == -3.0
    assert oracle.bf16_round(0.0) == 0.0


def test_bf16_round_matches_torch_conversion():
    x = RNG.standard_normal(100000).astype(np.float32) * np.float32(37.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x.astype(np.float64)), ref)


# --------------------------------------------------------------- RMSNorm --

def test_rms_norm_constant_row_closed_form():
    H, c, eps = 64, 0.37, 1e-5
    w = RNG.standard_normal(H)
    out = oracle.rms_norm(np.full((1, H), c), w, eps)
    np.testing.assert_allclose(out[0], c / math.sqrt(c * c + eps) * w, rtol=1e-14)


def test_rms_norm_unit_weight_mean_square():
    x = RNG.standard_normal((5, 128)) * 0.01        # small rows so eps matters
    out = oracle.rms_norm(x, np.ones(128), 1e-5)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(out * out, axis=1), ms / (ms + 1e-5), rtol=1e-12)


def test_rms_norm_scale_invariance_and_torch():
    x = RNG.standard_normal((7, 96))
    w = RNG.standard_normal(96)
    a = oracle.rms_norm(x, w, 1e-5)
    b = oracle.rms_norm(1000.0 * x, w, 1e-5)
    np.testing.assert_allclose(a, b, rtol=1e-5)
    ref = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-14)


def test_fused_add_rms_norm_paths():
    x = RNG.standard_normal((3, 32))
    res = RNG.standard_normal((3, 32))
    w = RNG.standard_normal(32)
    h, r = oracle.fused_add_rms_norm(x, None, w, 1e-5)
    np.testing.assert_array_equal(r, x)                          # None: residual = input
    np.testing.assert_array_equal(h, oracle.rms_norm(x, w, 1e-5))
    h, r = oracle.fused_add_rms_norm(x, res, w, 1e-5)
    np.testing.assert_array_equal(r, x + res)
    np.testing.assert_array_equal(h, oracle.rms_norm(x + res, w, 1e-5))
    # bf16 storage: the residual is rounded, and the norm uses the rounded sum
    h, r = oracle.fused_add_rms_norm(x, res, w, 1e-5, oracle.bf16_round)
    np.testing.assert_array_equal(r, oracle.bf16_round(x + res))
    np.testing.assert_array_equal(h, oracle.bf16_round(oracle.rms_norm(r, w, 1e-5)))


# ------------------------------------------------------------------ RoPE --

def _rope_complex(x, pos, freqs):
    """Independent formulation: pair (a, b) as the complex number a + ib,
    multiplied by e^{i p w}."""
    t = torch.from_numpy(x)
    half = x.shape[-1] // 2
    z = torch.complex(t[..., :half], t[..., half:])
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * torch.from_numpy(freqs)[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    out = z * rot
    return torch.cat([out.real, out.imag], dim=-1).numpy()


def test_rope_base_frequencies_textbook():
    f = oracle.rope_frequencies(64, 10000.0, None)
    ref = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    np.testing.assert_allclose(f, ref, rtol=1e-15)
    assert f[0] == 1.0


def test_rope_matches_complex_multiplication():
    x = RNG.standard_normal((9, 3, 16))
    pos = np.array([0, 1, 2, 5, 17, 100, 4095, 8191, 131071])
    f = oracle.rope_frequencies(16, 10000.0, None)
    np.testing.assert_allclose(oracle.apply_rope(x, pos, f), _rope_complex(x, pos, f),
                               rtol=1e-12, atol=1e-12)


def test_rope_identity_at_zero_and_norm_preserving():
    x = RNG.standard_normal((4, 2, 32))
    f = oracle.rope_frequencies(32, 5e5, synth.LLAMA3_SCALING)
    np.testing.assert_array_equal(oracle.apply_rope(x, np.zeros(4, dtype=np.int64), f), x)
    y = oracle.apply_rope(x, np.array([3, 999, 40000, 131071]), f)
    n0 = x[..., :16] ** 2 + x[..., 16:] ** 2
    n1 = y[..., :16] ** 2 + y[..., 16:] ** 2
    np.testing.assert_allclose(n0, n1, rtol=1e-12)


def test_rope_relative_position_and_composition():
    d = 32
    f = oracle.rope_frequencies(d, 5e5, synth.LLAMA3_SCALING)
    q = RNG.standard_normal((1, 1, d))
    k = RNG.standard_normal((1, 1, d))
    rq = lambda p: oracle.apply_rope(q, np.array([p]), f)[0, 0]
    rk = lambda p: oracle.apply_rope(k, np.array([p]), f)[0, 0]
    for m, n, delta in [(7, 3, 11), (9000, 100, 20000), (0, 5, 3)]:
        assert abs(rq(m) @ rk(n) - rq(m + delta) @ rk(n + delta)) < 1e-9
    # R(a) R(b) = R(a + b)
    a, b = 123, 4567
    two = oracle.apply_rope(oracle.apply_rope(q, np.array([a]), f), np.array([b]), f)
    np.testing.assert_allclose(two, oracle.apply_rope(q, np.array([a + b]), f), rtol=1e-9, atol=1e-9)


def test_llama3_bands_and_edges():
    d, theta = 128, 5e5
    base = oracle.rope_frequencies(d, theta, None)
    f = oracle.rope_frequencies(d, theta, synth.LLAMA3_SCALING)
    same = np.isclose(f, base, rtol=1e-15, atol=0)
    div8 = np.isclose(f, base / 8, rtol=1e-15, atol=0)
    # wavelength bands: below 8192/4 = 2048 unchanged, above 8192/1 divided by 8
    lam = 2 * math.pi / base
    assert np.array_equal(same, lam < 2048)
    assert np.array_equal(div8, lam > 8192)
    assert same.sum() == 29 and div8.sum() == 29
    mid = ~(same | div8)
    assert mid.sum() == 6
    assert np.all(f[mid] < base[mid]) and np.all(f[mid] > base[mid] / 8)
    assert f[0] == 1.0
    assert f[63] == theta ** (-126 / 128) / 8
    assert np.all(np.diff(f) < 0)


@pytest.mark.parametrize("edge", [2048.0, 8192.0])
def test_llama3_continuous_at_band_edges(edge):
    # a 4-wide head has w_1 = theta^(-1/2); pick theta so w_1's wavelength
    # sits just below / just above the edge
    vals = []
    for side in (1 - 1e-9, 1 + 1e-9):
        theta = (edge * side / (2 * math.pi)) ** 2
        vals.append(oracle.rope_frequencies(4, theta, synth.LLAMA3_SCALING)[1])
    assert abs(vals[0] - vals[1]) / vals[0] < 1e-7


def test_llama3_factor_one_is_plain_rope():
    sc = dict(synth.LLAMA3_SCALING, factor=1.0)
    np.testing.assert_allclose(oracle.rope_frequencies(128, 5e5, sc),
                               oracle.rope_frequencies(128, 5e5, None), rtol=1e-15)


def test_llama3_interior_pairs_match_fixture():
    """The six pairs between the wavelength edges: their scaled frequencies,
    read back as blend weights s = (w'/w - 1/8) / (1 - 1/8), equal the
    hand-evaluated weights of tests/golden/llama3_interior.json (4 decimals).
    A blend harmonic in the factor, or one linear in the wavelength instead of
    in its inverse, moves every s by more than 0.1."""
    with open(os.path.join(GOLDEN, "llama3_interior.json")) as f:
        g = json.load(f)
    d, theta = g["head_dim"], g["theta"]
    base = oracle.rope_frequencies(d, theta, None)
    f = oracle.rope_frequencies(d, theta, synth.LLAMA3_SCALING)
    factor = synth.LLAMA3_SCALING["factor"]
    ratio = f / base
    interior = [i for i in range(d // 2) if not (np.isclose(ratio[i], 1.0, rtol=1e-15, atol=0)
                                                 or np.isclose(ratio[i], 1 / factor, rtol=1e-15, atol=0))]
    assert interior == g["pairs"]
    s = (ratio[interior] - 1 / factor) / (1 - 1 / factor)
    np.testing.assert_allclose(s, g["s"], rtol=0, atol=5.1e-5)
    np.testing.assert_allclose(2 * math.pi / base[interior], g["wavelength"], rtol=0, atol=0.051)
    assert int(np.sum(np.isclose(ratio, 1.0, rtol=1e-15, atol=0))) == g["unchanged_pairs"]
    assert int(np.sum(np.isclose(ratio, 1 / factor, rtol=1e-15, atol=0))) == g["divided_pairs"]


# ------------------------------------------------------------- attention --

def _sdpa_causal(q, k, v, q_pos):
    """torch's scaled_dot_product_attention with an explicit causal mask by
    position.  q [T, nq, d]; k, v [L, nkv, d] (key j at position j)."""
    L = k.shape[0]
    mask = torch.from_numpy(np.arange(L)[None, :] <= q_pos[:, None])
    o = F.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(0, 1)[None], torch.from_numpy(k).transpose(0, 1)[None],
        torch.from_numpy(v).transpose(0, 1)[None], attn_mask=mask, enable_gqa=True)
    return o[0].transpose(0, 1).numpy()


def test_attend_matches_sdpa_brute_force():
    L, nq, nkv, d = 13, 6, 2, 8
    q = RNG.standard_normal((L, nq, d))
    k = RNG.standard_normal((L, nkv, d))
    v = RNG.standard_normal((L, nkv, d))
    ref = _sdpa_causal(q, k, v, np.arange(L))
    for p in range(L):
        np.testing.assert_allclose(oracle.attend(q[p], k[: p + 1], v[: p + 1]), ref[p],
                                   rtol=1e-12, atol=1e-13)


def test_attend_special_cases():
    nq, nkv, d = 4, 2, 8
    k = RNG.standard_normal((10, nkv, d))
    v = RNG.standard_normal((10, nkv, d))
    # a single key: output is that value exactly
    out = oracle.attend(RNG.standard_normal((nq, d)), k[:1], v[:1])
    np.testing.assert_array_equal(out, np.repeat(v[0], nq // nkv, axis=0))
    # q = 0: uniform weights, output is the mean of the values
    out = oracle.attend(np.zeros((nq, d)), k, v)
    np.testing.assert_allclose(out, np.repeat(v.mean(axis=0), 2, axis=0), rtol=1e-13)
    # the output lies inside the values' range (convex combination)
    out = oracle.attend(5 * RNG.standard_normal((nq, d)), k, v)
    for h in range(nq):
        g = h // 2
        assert np.all(out[h] <= v[:, g].max(axis=0) + 1e-12)
        assert np.all(out[h] >= v[:, g].min(axis=0) - 1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    nq, nkv, d, L = 8, 2, 16, 20
    q = RNG.standard_normal((nq, d))
    k = RNG.standard_normal((L, nkv, d))
    v = RNG.standard_normal((L, nkv, d))
    gqa = oracle.attend(q, k, v)
    mha = oracle.attend(q, np.repeat(k, nq // nkv, axis=1), np.repeat(v, nq // nkv, axis=1))
    np.testing.assert_allclose(gqa, mha, rtol=1e-13, atol=1e-15)
    # q head 5 reads kv head 1 (contiguous groups of 4)
    alone = oracle.attend(q[5:6], k[:, 1:2], v[:, 1:2])
    np.testing.assert_allclose(alone[0], gqa[5], rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------- MLP --

def test_silu_and_mul():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([40.0])), [40.0], rtol=1e-15)
    z = RNG.standard_normal(1000) * 6
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-15)
    # gate is the first half: gate large, up = 1 gives ~gate; swapped halves would
    # give silu(1) * gate
    x = np.concatenate([np.full(4, 30.0), np.ones(4)])[None]
    np.testing.assert_allclose(oracle.silu_and_mul(x)[0], np.full(4, 30.0), rtol=1e-12)
    u = RNG.standard_normal((3, 10))
    np.testing.assert_allclose(oracle.silu_and_mul(np.concatenate([u, np.ones((3, 10))], 1)),
                               oracle.silu(u), rtol=0)


def test_linear_convention():
    x = RNG.standard_normal((5, 8))
    w = np.zeros((3, 8))
    w[0, 2] = w[1, 7] = w[2, 0] = 1.0        # output j picks input col
    np.testing.assert_array_equal(oracle.linear(x, w), x[:, [2, 7, 0]])


# ------------------------------------------------------------ whole layer --

def _layer_unfused_torch(cfg, w, stream, positions, k_ctx, v_ctx, freqs):
    """The layer written the other way the pages write it (the vllm-learning
    page's LlamaDecoderLayer / Attention): separate q, k, v projections, the
    residual added inside the layer, one residual-stream tensor in and out --
    built from torch library routines only."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    H, nq, nkv, d = (cfg["hidden_size"], cfg["num_attention_heads"],
                     cfg["num_key_value_heads"], cfg["head_dim"])
    eps = cfg["rms_norm_eps"]
    wqkv = t(w["qkv_proj"])
    wq, wk, wv = wqkv[: nq * d], wqkv[nq * d: (nq + nkv) * d], wqkv[(nq + nkv) * d:]
    I = cfg["intermediate_size"]
    wg, wu = t(w["gate_up_proj"])[:I], t(w["gate_up_proj"])[I:]
    hidden = t(stream)
    residual = hidden
    x = F.rms_norm(hidden, (H,), weight=t(w["input_layernorm"]), eps=eps)
    q = F.linear(x, wq).reshape(-1, nq, d).numpy()
    k = F.linear(x, wk).reshape(-1, nkv, d).numpy()
    v = F.linear(x, wv).reshape(-1, nkv, d).numpy()
    q = _rope_complex(q, positions, freqs)
    k = _rope_complex(k, positions, freqs)
    K = np.concatenate([k_ctx, k])
    V = np.concatenate([v_ctx, v])
    a = _sdpa_causal(q, K, V, positions).reshape(-1, nq * d)
    hidden = residual + F.linear(t(a), t(w["o_proj"]))
    residual = hidden
    x = F.rms_norm(hidden, (H,), weight=t(w["post_attention_layernorm"]), eps=eps)
    hidden = residual + F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), t(w["down_proj"]))
    return hidden.numpy()


# the last case: a query width (4 x 16) other than the hidden size (80)
@pytest.mark.parametrize("scaling,ctx,H", [(None, 0, 64), (None, 5, 64), (synth.LLAMA3_SCALING, 9, 64), (None, 7, 80)])
def test_layer_matches_unfused_library_formulation(scaling, ctx, H):
    cfg = _cfg(H=H, theta=5e5 if scaling else 1e4, scaling=scaling)
    rng = np.random.default_rng(7)
    w = _weights(cfg, rng)
    T = 11
    nkv, d = cfg["num_key_value_heads"], cfg["head_dim"]
    k_ctx = rng.standard_normal((ctx, nkv, d))
    v_ctx = rng.standard_normal((ctx, nkv, d))
    hidden = rng.standard_normal((T, cfg["hidden_size"]))
    residual = rng.standard_normal((T, cfg["hidden_size"]))
    pos = np.arange(ctx, ctx + T)
    out = oracle.decoder_layer(cfg, w, hidden, residual, pos, [oracle.Seq(range(T), k_ctx, v_ctx)])
    freqs = (np.array([cfg["rope_theta"] ** (-2.0 * i / d) for i in range(d // 2)])
             if scaling is None else oracle.rope_frequencies(d, cfg["rope_theta"], scaling))
    ref = _layer_unfused_torch(cfg, w, hidden + residual, pos, k_ctx, v_ctx, freqs)
    np.testing.assert_allclose(out["hidden_out"] + out["residual_out"], ref, rtol=1e-10, atol=1e-10)
    # the first-layer path (no incoming residual) on the same stream value
    out0 = oracle.decoder_layer(cfg, w, hidden + residual, None, pos,
                                [oracle.Seq(range(T), k_ctx, v_ctx)])
    np.testing.assert_allclose(out0["hidden_out"] + out0["residual_out"], ref, rtol=1e-10, atol=1e-10)


def test_model_forward_matches_unfused_stack_and_final_norm():
    """The model body: three layers handing the pair on, then the final norm
    of hidden + residual, equals the unfused formulation chained on one
    residual stream followed by torch's RMSNorm."""
    cfg = _cfg()
    rng = np.random.default_rng(9)
    ws = [_weights(cfg, rng) for _ in range(3)]
    final_w = 1.0 + 0.5 * rng.standard_normal(cfg["hidden_size"])
    T, ctx = 6, 4
    nkv, d = cfg["num_key_value_heads"], cfg["head_dim"]
    ctxs = [(rng.standard_normal((ctx, nkv, d)), rng.standard_normal((ctx, nkv, d))) for _ in ws]
    hidden = rng.standard_normal((T, cfg["hidden_size"]))
    pos = np.arange(ctx, ctx + T)
    seqs = [[oracle.Seq(range(T), kc, vc)] for kc, vc in ctxs]
    out, per_layer = oracle.model_forward(cfg, ws, final_w, hidden, pos, seqs)
    freqs = np.array([cfg["rope_theta"] ** (-2.0 * i / d) for i in range(d // 2)])
    stream = hidden
    for w, (kc, vc) in zip(ws, ctxs):
        stream = _layer_unfused_torch(cfg, w, stream, pos, kc, vc, freqs)
    ref = F.rms_norm(torch.from_numpy(stream), (cfg["hidden_size"],), weight=torch.from_numpy(final_w),
                     eps=cfg["rms_norm_eps"]).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10)
    assert len(per_layer) == 3
    # the norm sees the sum: with a unit weight every row has mean square ms / (ms + eps)
    out1, _ = oracle.model_forward(cfg, ws, np.ones(cfg["hidden_size"]), hidden, pos, seqs)
    ms = np.mean(stream ** 2, axis=1)
    np.testing.assert_allclose(np.mean(out1 ** 2, axis=1), ms / (ms + cfg["rms_norm_eps"]), rtol=1e-12)


def test_layer_kv_append_values():
    """The appended K is the rotated k projection, V the raw v projection."""
    cfg = _cfg()
    rng = np.random.default_rng(3)
    w = _weights(cfg, rng)
    T, H, nq, nkv, d = 6, 64, 4, 2, 16
    hidden = rng.standard_normal((T, H))
    pos = np.arange(2, 2 + T)
    seq = oracle.Seq(range(T), rng.standard_normal((2, nkv, d)), rng.standard_normal((2, nkv, d)))
    out = oracle.decoder_layer(cfg, w, hidden, None, pos, [seq])
    h = oracle.rms_norm(hidden, w["input_layernorm"], 1e-5)
    qkv = h @ w["qkv_proj"].T
    k = qkv[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d)
    v = qkv[:, (nq + nkv) * d:].reshape(T, nkv, d)
    np.testing.assert_allclose(out["v_new"][0], v, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out["k_new"][0], _rope_complex(k, pos, oracle.rope_frequencies(d, 1e4, None)),
                               rtol=1e-12, atol=1e-13)


def test_causality_and_row_subset_and_batch_independence():
    cfg = _cfg()
    rng = np.random.default_rng(11)
    w = _weights(cfg, rng)
    H, nkv, d = 64, 2, 16
    hidden = rng.standard_normal((16, H))
    residual = rng.standard_normal((16, H))
    # two sequences of 8 tokens, contexts 3 and 0
    kc = rng.standard_normal((3, nkv, d))
    vc = rng.standard_normal((3, nkv, d))
    empty = np.zeros((0, nkv, d))
    pos = np.concatenate([np.arange(3, 11), np.arange(0, 8)])
    seqs = [oracle.Seq(range(0, 8), kc, vc), oracle.Seq(range(8, 16), empty, empty)]
    full = oracle.decoder_layer(cfg, w, hidden, residual, pos, seqs)
    # perturbing later tokens leaves earlier rows bitwise unchanged
    h2 = hidden.copy()
    h2[5:8] += 1.0
    pert = oracle.decoder_layer(cfg, w, h2, residual, pos, seqs)
    np.testing.assert_array_equal(pert["hidden_out"][:5], full["hidden_out"][:5])
    assert not np.allclose(pert["hidden_out"][5:8], full["hidden_out"][5:8])
    np.testing.assert_array_equal(pert["hidden_out"][8:], full["hidden_out"][8:])
    # a row subset reproduces those rows
    sub = oracle.decoder_layer(cfg, w, hidden, residual, pos, seqs, want=[2, 9, 15])
    np.testing.assert_allclose(sub["hidden_out"], full["hidden_out"][[2, 9, 15]], rtol=1e-12, atol=1e-13)
    # a sequence alone gives the same rows as inside the batch
    alone = oracle.decoder_layer(cfg, w, hidden[8:], residual[8:], pos[8:],
                                 [oracle.Seq(range(8), empty, empty)])
    np.testing.assert_allclose(alone["hidden_out"], full["hidden_out"][8:], rtol=1e-12, atol=1e-13)


def test_prefill_then_decode_equals_prefill():
    cfg = _cfg(theta=5e5, scaling=synth.LLAMA3_SCALING)
    rng = np.random.default_rng(5)
    w = _weights(cfg, rng)
    S, H, nkv, d = 10, 64, 2, 16
    hidden = rng.standard_normal((S, H))
    residual = rng.standard_normal((S, H))
    empty = np.zeros((0, nkv, d))
    full = oracle.decoder_layer(cfg, w, hidden, residual, np.arange(S), [oracle.Seq(range(S), empty, empty)])
    pre = oracle.decoder_layer(cfg, w, hidden[:-1], residual[:-1], np.arange(S - 1),
                               [oracle.Seq(range(S - 1), empty, empty)])
    dec = oracle.decoder_layer(cfg, w, hidden[-1:], residual[-1:], np.array([S - 1]),
                               [oracle.Seq([0], pre["k_new"][0], pre["v_new"][0])])
    np.testing.assert_allclose(dec["hidden_out"][0], full["hidden_out"][-1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["residual_out"][0], full["residual_out"][-1], rtol=1e-12, atol=1e-13)


def test_bf16_storage_mode_close_to_exact():
    cfg = _cfg()
    rng = np.random.default_rng(9)
    w = _weights(cfg, rng)
    hidden = rng.standard_normal((12, 64))
    seq = [oracle.Seq(range(12), np.zeros((0, 2, 16)), np.zeros((0, 2, 16)))]
    a = oracle.decoder_layer(cfg, w, hidden, None, np.arange(12), seq)
    b = oracle.decoder_layer(cfg, w, hidden, None, np.arange(12), seq, rnd=oracle.bf16_round)
    x, y = a["hidden_out"].ravel(), b["hidden_out"].ravel()
    assert not np.array_equal(x, y)
    assert x @ y / np.linalg.norm(x) / np.linalg.norm(y) > 0.9999
    # the None path takes the input itself as the residual: same as adding zeros
    hb = oracle.bf16_round(hidden)
    c = oracle.decoder_layer(cfg, w, hb, None, np.arange(12), seq, rnd=oracle.bf16_round)
    z = oracle.decoder_layer(cfg, w, hb, np.zeros_like(hb), np.arange(12), seq, rnd=oracle.bf16_round)
    np.testing.assert_array_equal(c["residual_out"], z["residual_out"])
    np.testing.assert_array_equal(c["hidden_out"], z["hidden_out"])


def _layer_bf16_storage_torch(cfg, w, hidden, residual, positions, k_ctx, v_ctx, freqs):
    """The layer as a bf16 model stores it, written with torch routines in
    float64 and torch's own bfloat16 conversion at each storage point: the
    residual r, the normed h, the q/k/v projections, rotated q and k, the
    attention output, the post-attention residual r2, its normed h2 and the
    SiluAndMul output.  Returns (hidden_out, residual_out) before their own
    final rounding."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    bf = lambda x: x.to(torch.bfloat16).to(torch.float64)
    H, nq, nkv, d, I = (cfg["hidden_size"], cfg["num_attention_heads"], cfg["num_key_value_heads"],
                        cfg["head_dim"], cfg["intermediate_size"])
    eps = cfg["rms_norm_eps"]
    wqkv = t(w["qkv_proj"])
    wq, wk, wv = wqkv[: nq * d], wqkv[nq * d: (nq + nkv) * d], wqkv[(nq + nkv) * d:]
    r = bf(t(hidden) + t(residual))
    h = bf(F.rms_norm(r, (H,), weight=t(w["input_layernorm"]), eps=eps))
    q = bf(F.linear(h, wq)).reshape(-1, nq, d).numpy()
    k = bf(F.linear(h, wk)).reshape(-1, nkv, d).numpy()
    v = bf(F.linear(h, wv)).reshape(-1, nkv, d).numpy()
    q = bf(t(_rope_complex(q, positions, freqs))).numpy()
    k = bf(t(_rope_complex(k, positions, freqs))).numpy()
    a = _sdpa_causal(q, np.concatenate([k_ctx, k]), np.concatenate([v_ctx, v]), positions)
    a = bf(t(a.reshape(-1, nq * d)))
    r2 = F.linear(a, t(w["o_proj"])) + r
    h2 = bf(F.rms_norm(bf(r2), (H,), weight=t(w["post_attention_layernorm"]), eps=eps))
    gu = F.linear(h2, t(w["gate_up_proj"]))
    act = bf(F.silu(gu[:, :I]) * gu[:, I:])
    return F.linear(act, t(w["down_proj"])).numpy(), r2.numpy()


@pytest.mark.parametrize("scaling,ctx", [(None, 0), (synth.LLAMA3_SCALING, 7)])
def test_bf16_storage_points_match_torch_bf16_pipeline(scaling, ctx):
    """The oracle's bf16-storage mode rounds exactly where a bf16 model stores
    a tensor.  Against a torch pipeline with torch's bf16 conversion at the
    same points, the returned residual agrees to float64 rounding and the
    returned hidden state to far below one bf16 ulp.  A storage point dropped
    or added (say r2 left unrounded before its norm) moves h2 by up to half
    an ulp and flips a large share of its roundings, which this fails."""
    cfg = _cfg(H=128, d=32, I=192, theta=5e5 if scaling else 1e4, scaling=scaling)
    rng = np.random.default_rng(17)
    w = {k: oracle.bf16_round(v) for k, v in _weights(cfg, rng).items()}
    T = 9
    nkv, d = cfg["num_key_value_heads"], cfg["head_dim"]
    k_ctx = oracle.bf16_round(rng.standard_normal((ctx, nkv, d)))
    v_ctx = oracle.bf16_round(rng.standard_normal((ctx, nkv, d)))
    hidden = oracle.bf16_round(rng.standard_normal((T, cfg["hidden_size"])))
    residual = oracle.bf16_round(rng.standard_normal((T, cfg["hidden_size"])))
    pos = np.arange(ctx, ctx + T)
    out = oracle.decoder_layer(cfg, w, hidden, residual, pos, [oracle.Seq(range(T), k_ctx, v_ctx)],
                               rnd=oracle.bf16_round)
    freqs = oracle.rope_frequencies(d, cfg["rope_theta"], scaling)
    ref_h, ref_r = _layer_bf16_storage_torch(cfg, w, hidden, residual, pos, k_ctx, v_ctx, freqs)
    np.testing.assert_allclose(out["residual_out"], ref_r, rtol=1e-12, atol=1e-12)
    rms = float(np.sqrt(np.mean(ref_h ** 2)))
    assert float(np.abs(out["hidden_out"] - ref_h).max()) <= 1e-9 * rms
    # the unrounded oracle is a different function: its distance is bf16-sized
    exact = oracle.decoder_layer(cfg, w, hidden, residual, pos, [oracle.Seq(range(T), k_ctx, v_ctx)])
    assert float(np.abs(exact["hidden_out"] - ref_h).max()) > 1e-4 * rms


def test_stack_hands_pair_on():
    cfg = _cfg()
    rng = np.random.default_rng(21)
    ws = [_weights(cfg, rng) for _ in range(3)]
    hidden = rng.standard_normal((4, 64))
    residual = rng.standard_normal((4, 64))
    pos = np.array([3, 5, 2, 7])
    seqs = [[oracle.Seq([b], rng.standard_normal((int(pos[b]), 2, 16)),
                        rng.standard_normal((int(pos[b]), 2, 16))) for b in range(4)] for _ in range(3)]
    outs = oracle.decoder_stack(cfg, ws, hidden, residual, pos, seqs, want=[1, 3])
    h, r = hidden, residual
    for l in range(3):
        o = oracle.decoder_layer(cfg, ws[l], h, r, pos, seqs[l])
        h, r = o["hidden_out"], o["residual_out"]
    np.testing.assert_allclose(outs[-1]["hidden_out"], h[[1, 3]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(outs[-1]["residual_out"], r[[1, 3]], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- the pages' values --

def test_golden_config_and_shapes():
    with open(os.path.join(GOLDEN, "llama70b_config.json")) as f:
        g = json.load(f)
    c = g["config"]
    m = synth.LLAMA70B
    for key in ("hidden_size", "num_attention_heads", "num_key_value_heads", "head_dim",
                "intermediate_size", "rms_norm_eps", "rope_theta", "max_position_embeddings"):
        assert getattr(m, key) == c[key], key
    assert m.rope_scaling == c["rope_scaling"]
    assert c["hidden_act"] == "silu" and not c["attention_bias"] and not c["mlp_bias"]
    assert m.q_size == g["derived"]["q_size"] and m.kv_size == g["derived"]["kv_size"]
    # the oracle's split and output widths at this config (shapes only: a
    # zero-size batch is enough)
    cfg = m.config_dict()
    assert cfg["num_attention_heads"] * cfg["head_dim"] == 8192
    assert synth.LLAMA70B.hidden_size == g["derived"]["mlp_output_last_dim"]

"""Bit-exact checks of the values a forward writes into the paged KV cache.

The cache holds, for each new token (position p of sequence b, slot
block_table[b][p // 16] * 16 + p % 16):
  * V: a bit copy of the token's v projection, the v part of the workspace
    tensor "qkv";
  * K: the rotated k projection.  The library's RoPE kernel turns the pair
    (x0, x1) = (k_i, k_{i + d/2}) by the table entry (c, s) of position p as
        y0 = fmaf(x0, c, -(x1 * s)),   y1 = fmaf(x1, c, x0 * s)
    in float32 and rounds each once to the layer dtype (header
    llama_layer.h, llama_layer_rope_table).  The k part of "qkv" keeps the
    projection before the rotation.
The emulation below computes exactly that on the host: float32 products
rounded to nearest even, a fused multiply-add rounded once, then the bf16
rounding (round to nearest even) torch's conversion applies.
"""
from __future__ import annotations

import numpy as np
import torch


def fmaf(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """float32 fused multiply-add a*b + c, rounded once to nearest even.

    a*b of two float32 values is exact in float64 (48 significant bits).  The
    float64 sum s of that product and c may be inexact; TwoSum gives the
    exact remainder e, and only where s sits exactly halfway between two
    float32 values does e decide the direction (a plain float64 -> float32
    cast would round that tie to even)."""
    a64 = np.asarray(a, np.float32).astype(np.float64)
    b64 = np.asarray(b, np.float32).astype(np.float64)
    c64 = np.asarray(c, np.float32).astype(np.float64)
    p = a64 * b64
    s = p + c64
    bp = s - p
    e = (p - (s - bp)) + (c64 - bp)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    toward = np.where(s > r64, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    other = np.nextafter(r, toward)
    tie = (s != r64) & (s == (r64 + other.astype(np.float64)) * 0.5)
    up = np.maximum(r, other)
    down = np.minimum(r, other)
    out = r.copy()
    out = np.where(tie & (e > 0), up, out)
    out = np.where(tie & (e < 0), down, out)
    return out.astype(np.float32)


def mul_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """float32 product rounded to nearest even (exact in float64, then one
    rounding)."""
    return (np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64)).astype(
        np.float32)


def rope_fp32(x0: np.ndarray, x1: np.ndarray, c: np.ndarray, s: np.ndarray):
    """The kernel's rotation of pairs (x0, x1) by (c, s), float32 results."""
    y0 = fmaf(x0, c, -mul_f32(x1, s))
    y1 = fmaf(x1, c, mul_f32(x0, s))
    return y0, y1


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> the layer dtype's bit patterns (int16 bf16 by RNE, or
    int32 float32)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


def check_kv_bits(model, batch, kp: torch.Tensor, vp: torch.Tensor, qkv: torch.Tensor, table: np.ndarray,
                  rows=None, check_k: bool = True) -> int:
    """Asserts the new tokens' V slots equal the v part of the workspace qkv
    bit for bit and (check_k) their K slots equal the emulated rotation of its
    k part with the library's table.  rows: token rows to check (default
    all).  Returns the number of K/V slots checked."""
    nq, nkv, d = model.num_attention_heads, model.num_key_value_heads, model.head_dim
    half = d // 2
    ib = torch.int16 if model.dtype == "bf16" else torch.int32
    seq_of = batch.seq_of_row()
    rows = list(range(batch.num_tokens)) if rows is None else list(rows)
    pos = batch.positions.numpy()
    t_rows = torch.tensor(rows, dtype=torch.long)
    p = torch.from_numpy(pos[rows].astype(np.int64))
    b = torch.tensor([seq_of[r] for r in rows], dtype=torch.long)
    blk = batch.block_table[b, p // 16].long()
    slot = p % 16
    dev = kp.device
    blk_d, slot_d, rows_d = blk.to(dev), slot.to(dev), t_rows.to(dev)
    # cache contents of the checked slots: [n, nkv, d]
    k_got = kp[blk_d, :, slot_d, :].contiguous().view(ib).cpu().numpy()
    v_got = vp[blk_d, :, :, slot_d].contiguous().view(ib).cpu().numpy()
    q_rows = qkv[rows_d].contiguous()
    v_src = q_rows[:, (nq + nkv) * d:].contiguous().view(ib).cpu().numpy().reshape(len(rows), nkv, d)
    assert np.array_equal(v_got, v_src), "V slots differ from the projection's v bits"
    if check_k:
        k_src = q_rows[:, nq * d:(nq + nkv) * d].float().cpu().numpy().reshape(len(rows), nkv, d)
        cs = table[pos[rows]]                       # [n, half, 2]
        c = cs[:, None, :, 0]
        s = cs[:, None, :, 1]
        y0, y1 = rope_fp32(k_src[..., :half], k_src[..., half:], c, s)
        want = to_bits(np.concatenate([y0, y1], axis=-1), model.dtype)
        bad = np.argwhere(k_got != want)
        assert bad.size == 0, ("K slots differ from the emulated rotation", bad[:5].tolist(), bad.shape[0])
    return len(rows) * nkv

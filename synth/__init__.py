"""Seeded synthetic inputs for the Llama decoder-layer forward.

This module holds model shapes, workload shapes and random draws only.  No step
of the layer's arithmetic lives here: it draws weights, activations, KV-cache
contexts, context lengths and block tables, and lays a logical KV context out
in the paged pool format that the library's header documents.  The CPU oracle
(through the tests) and the HIP path consume exactly the same tensors.

Shapes come from the DeepSeek-R1-Distill-Llama-70B ``config.json`` printed on
the page "LLama" (hotelren.com/news/2693952, model-parameters block): hidden
8192, 64 query heads, 8 KV heads, head_dim 128, intermediate 28672,
rms_norm_eps 1e-5, rope_theta 5e5 with llama3 scaling (factor 8, low 1, high 4,
original 8192), max_position_embeddings 131072, bf16.

Value distributions: linear weights N(0, 0.02^2) (``initializer_range``),
RMSNorm weights 1 + N(0, 0.02^2), hidden states, residual stream and cached
K/V contexts N(0, 1).  Seeds follow ``1000*(workload_index+1) + 97*layer +
tensor_id`` with one generator per tensor.  Float draws happen on the device
the tensor will live on (a GPU and a CPU therefore see different values,
which never matters: every comparison runs both sides on the same tensors); integer draws (context lengths, block permutations) always happen
on the CPU so they are the same everywhere.
"""
from __future__ import annotations

import dataclasses
import itertools
import math
from typing import Optional

import torch

# tensor ids used in seeds
T_W_IN, T_W_QKV, T_W_O, T_W_POST, T_W_GU, T_W_DOWN = 0, 1, 2, 3, 4, 5
T_HIDDEN, T_RESIDUAL, T_KCTX, T_VCTX, T_CTXLEN, T_BLOCKPERM = 6, 7, 8, 9, 10, 11
T_W_FINAL = 12  # the model body's final norm (drawn with layer 0's seed base)
T_W_ROUTER, T_W_EXP13, T_W_EXP2, T_W_QNORM, T_W_KNORM = 13, 14, 15, 16, 17

KV_BLOCK = 16


@dataclasses.dataclass(frozen=True)
class ModelShape:
    hidden_size: int
    num_attention_heads: int
    num_key_value_heads: int
    head_dim: int
    intermediate_size: int
    rms_norm_eps: float
    rope_theta: float
    rope_scaling: Optional[dict]
    max_position_embeddings: int
    dtype: str  # "bf16" or "fp32"
    # a mixture-of-experts layer (num_experts > 0) replaces the MLP by
    # num_experts FFNs of width moe_intermediate_size, num_experts_per_tok
    # chosen per token; qk_norm adds a per-head RMSNorm of q and k
    num_experts: int = 0
    num_experts_per_tok: int = 0
    moe_intermediate_size: int = 0
    norm_topk_prob: bool = True
    qk_norm: bool = False

    @property
    def q_size(self) -> int:
        return self.num_attention_heads * self.head_dim

    @property
    def kv_size(self) -> int:
        return self.num_key_value_heads * self.head_dim

    @property
    def qkv_size(self) -> int:
        return self.q_size + 2 * self.kv_size

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def config_dict(self) -> dict:
        """The model's fields under their ``config.json`` names."""
        d = {
            "hidden_size": self.hidden_size,
            "num_attention_heads": self.num_attention_heads,
            "num_key_value_heads": self.num_key_value_heads,
            "head_dim": self.head_dim,
            "intermediate_size": self.intermediate_size,
            "rms_norm_eps": self.rms_norm_eps,
            "rope_theta": self.rope_theta,
            "rope_scaling": dict(self.rope_scaling) if self.rope_scaling else None,
            "max_position_embeddings": self.max_position_embeddings,
            "hidden_act": "silu",
            "attention_bias": False,
            "mlp_bias": False,
            "torch_dtype": "bfloat16" if self.dtype == "bf16" else "float32",
        }
        if self.num_experts:
            d.update({"num_experts": self.num_experts, "num_experts_per_tok": self.num_experts_per_tok,
                      "moe_intermediate_size": self.moe_intermediate_size,
                      "norm_topk_prob": self.norm_topk_prob})
        if self.qk_norm:
            d["qk_norm"] = True
        return d


LLAMA3_SCALING = {
    "rope_type": "llama3",
    "factor": 8.0,
    "low_freq_factor": 1.0,
    "high_freq_factor": 4.0,
    "original_max_position_embeddings": 8192,
}

LLAMA70B = ModelShape(8192, 64, 8, 128, 28672, 1e-5, 500000.0, LLAMA3_SCALING, 131072, "bf16")
TINY = ModelShape(256, 4, 2, 64, 688, 1e-5, 10000.0, None, 4096, "fp32")
# one GPU's share of the 70B layer under the pages' tensor parallelism at
# TP = 8: the column-parallel qkv and gate_up keep 8 query heads, 1 KV head
# and 28672 / 8 intermediate features per GPU; the row-parallel o_proj and
# down_proj read those shards (K = 1024 and 3584) and produce partial sums
# that an all-reduce would complete
LLAMA70B_TP8 = ModelShape(8192, 8, 1, 128, 3584, 1e-5, 500000.0, LLAMA3_SCALING, 131072, "bf16")
# Qwen3-30B-A3B (config.json on the page "LLama", section
# "Qwen3MoeForCausalLM"): every layer is sparse (decoder_sparse_step 1, no
# mlp_only_layers), so intermediate_size (the dense width) is never used.
QWEN3MOE = ModelShape(2048, 32, 4, 128, 6144, 1e-6, 1e7, None, 262144, "bf16",
                      num_experts=128, num_experts_per_tok=8, moe_intermediate_size=768,
                      norm_topk_prob=True, qk_norm=True)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One batch shape: ``num_seqs`` sequences, each appending ``q_len`` new
    tokens after a cached context.  ``ctx`` is either a fixed context length
    or a (lo, hi) inclusive range drawn per sequence.  A mixed batch instead
    lists ``mix``: one (new tokens, cached context) pair per sequence, in row
    order (q_len is then 0)."""
    index: int
    name: str
    model: ModelShape
    num_seqs: int
    q_len: int
    ctx: object = 0
    layers: int = 1
    residual_none: bool = False
    spare_blocks: int = 4
    mix: Optional[tuple] = None

    @property
    def num_tokens(self) -> int:
        if self.mix is not None:
            return sum(q for q, _ in self.mix)
        return self.num_seqs * self.q_len

    @property
    def mixed(self) -> bool:
        return self.mix is not None


WORKLOADS = {
    w.name: w
    for w in [
        Workload(0, "tiny_prefill_32", TINY, 1, 32, 0, 1, True),
        Workload(1, "llama70b_decode_b32_ctx2048", LLAMA70B, 32, 1, 2048),
        Workload(2, "llama70b_prefill_4x2048", LLAMA70B, 4, 2048, 0),
        Workload(3, "llama70b_prefill_1x32768", LLAMA70B, 1, 32768, 0),
        Workload(4, "llama70b_ragged_decode_b64_4layer", LLAMA70B, 64, 1, (128, 32768), 4),
        # a chunked-prefill step: 32 decode sequences at context 2048 plus one
        # 512-token prefill chunk on a 4096-token context, in one call
        Workload(5, "llama70b_mixed_chunk512_decode32", LLAMA70B, 33, 0,
                 mix=tuple([(1, 2048)] * 32 + [(512, 4096)])),
        # the 70B model body: 80 layers and the final norm, 32 decode rows
        Workload(6, "llama70b_stack80_decode_b32_ctx2048", LLAMA70B, 32, 1, 2048, 80),
        # the Qwen3-MoE layer on the same two batch shapes as the 70B layer
        Workload(7, "qwen3moe_decode_b32_ctx2048", QWEN3MOE, 32, 1, 2048),
        Workload(8, "qwen3moe_prefill_4x2048", QWEN3MOE, 4, 2048, 0),
        # one GPU's TP = 8 share of the 70B layer on the 70B batch shapes
        Workload(9, "llama70b_tp8shard_decode_b32_ctx2048", LLAMA70B_TP8, 32, 1, 2048),
        Workload(10, "llama70b_tp8shard_prefill_4x2048", LLAMA70B_TP8, 4, 2048, 0),
    ]
}
WORKLOAD_LIST = sorted(WORKLOADS.values(), key=lambda w: w.index)


def seed_of(workload_index: int, layer: int, tensor_id: int) -> int:
    return 1000 * (workload_index + 1) + 97 * layer + tensor_id


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


def draw_normal(shape, seed: int, device, dtype: torch.dtype, mean: float = 0.0,
                std: float = 1.0, chunk: int = 1 << 26) -> torch.Tensor:
    """N(mean, std^2) drawn in fp32 and rounded (round-to-nearest-even) to
    ``dtype``; drawn in chunks so no full fp32 copy of a large tensor exists."""
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if mean != 0.0:
            x.add_(mean)
        flat[s:e] = x.to(dtype)
    return out


def draw_weights(model: ModelShape, workload_index: int, layer: int, device,
                 linear_std: float = 0.02, norm_mean: float = 1.0,
                 norm_std: float = 0.02) -> dict:
    """Packed weights of one layer, each row-major [out, in]: qkv rows
    [q heads | k heads | v heads], gate_up rows [gate | up].  A
    mixture-of-experts model has router [E, H], experts_gate_up [E, 2I, H]
    (each expert [gate | up]) and experts_down [E, H, I] instead of the MLP;
    qk_norm adds q_norm and k_norm [head_dim] (drawn like the norm weights)."""
    dt = model.torch_dtype
    H, I = model.hidden_size, model.intermediate_size
    s = lambda tid: seed_of(workload_index, layer, tid)
    w = {
        "input_layernorm": draw_normal((H,), s(T_W_IN), device, dt, norm_mean, norm_std),
        "qkv_proj": draw_normal((model.qkv_size, H), s(T_W_QKV), device, dt, 0.0, linear_std),
        "o_proj": draw_normal((H, model.q_size), s(T_W_O), device, dt, 0.0, linear_std),
        "post_attention_layernorm": draw_normal((H,), s(T_W_POST), device, dt, norm_mean, norm_std),
    }
    if model.num_experts:
        E, Ie = model.num_experts, model.moe_intermediate_size
        w["router"] = draw_normal((E, H), s(T_W_ROUTER), device, dt, 0.0, linear_std)
        w["experts_gate_up"] = draw_normal((E, 2 * Ie, H), s(T_W_EXP13), device, dt, 0.0, linear_std)
        w["experts_down"] = draw_normal((E, H, Ie), s(T_W_EXP2), device, dt, 0.0, linear_std)
    else:
        w["gate_up_proj"] = draw_normal((2 * I, H), s(T_W_GU), device, dt, 0.0, linear_std)
        w["down_proj"] = draw_normal((H, I), s(T_W_DOWN), device, dt, 0.0, linear_std)
    if model.qk_norm:
        d = model.head_dim
        w["q_norm"] = draw_normal((d,), s(T_W_QNORM), device, dt, norm_mean, norm_std)
        w["k_norm"] = draw_normal((d,), s(T_W_KNORM), device, dt, norm_mean, norm_std)
    return w


def draw_final_norm(model: ModelShape, workload_index: int, device, norm_mean: float = 1.0,
                    norm_std: float = 0.02) -> torch.Tensor:
    """The final RMSNorm weight of a layer stack, 1 + N(0, 0.02^2) like the
    layers' norm weights."""
    return draw_normal((model.hidden_size,), seed_of(workload_index, 0, T_W_FINAL), device, model.torch_dtype,
                       norm_mean, norm_std)


def draw_activations(model: ModelShape, num_tokens: int, workload_index: int, device,
                     residual: bool = True, layer: int = 0):
    """hidden and residual-stream inputs [T, H], both N(0, 1)."""
    dt = model.torch_dtype
    h = draw_normal((num_tokens, model.hidden_size), seed_of(workload_index, layer, T_HIDDEN), device, dt)
    r = None
    if residual:
        r = draw_normal((num_tokens, model.hidden_size), seed_of(workload_index, layer, T_RESIDUAL), device, dt)
    return h, r


@dataclasses.dataclass
class Batch:
    """Per-call metadata of one forward (host-side copies; ``to(device)``
    gives the device tensors).  Sequence b owns rows ``rows(b)``; a mixed
    batch (``q_lens`` set, ``q_len`` 0) also carries ``query_start_loc``."""
    num_seqs: int
    q_len: int
    ctx_lens: list
    seq_lens: torch.Tensor      # int32 [B], KV length after the call
    positions: torch.Tensor     # int32 [T]
    block_table: torch.Tensor   # int32 [B, max_blocks_per_seq], -1 past the end
    num_blocks: int
    spare_blocks: list          # block ids referenced by no sequence
    q_lens: Optional[list] = None

    @property
    def mixed(self) -> bool:
        return self.q_lens is not None

    @property
    def num_tokens(self) -> int:
        return sum(self.q_lens) if self.mixed else self.num_seqs * self.q_len

    def new_rows(self, b: int) -> int:
        return self.q_lens[b] if self.mixed else self.q_len

    def row_start(self, b: int) -> int:
        return sum(self.q_lens[:b]) if self.mixed else b * self.q_len

    def rows(self, b: int) -> range:
        s = self.row_start(b)
        return range(s, s + self.new_rows(b))

    @property
    def query_start_loc(self) -> Optional[torch.Tensor]:
        """int32 [B+1] row offsets of a mixed batch (None for a uniform one)."""
        if not self.mixed:
            return None
        return torch.tensor([0] + list(itertools.accumulate(self.q_lens)), dtype=torch.int32)

    def seq_of_row(self) -> list:
        return [b for b in range(self.num_seqs) for _ in self.rows(b)]

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max().item())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def slot(self, b: int, pos: int) -> int:
        return int(self.block_table[b, pos // KV_BLOCK]) * KV_BLOCK + pos % KV_BLOCK


def draw_ctx_lens(workload: Workload) -> list:
    if isinstance(workload.ctx, tuple):
        lo, hi = workload.ctx
        g = _gen(seed_of(workload.index, 0, T_CTXLEN), "cpu")
        return [int(v) for v in torch.randint(lo, hi + 1, (workload.num_seqs,), generator=g)]
    return [int(workload.ctx)] * workload.num_seqs


def build_batch(workload: Workload, ctx_lens: Optional[list] = None) -> Batch:
    """Context lengths, positions and a block table whose blocks are placed by
    a seeded random permutation of the pool (plus a few spare blocks that no
    sequence references)."""
    if workload.mixed:
        return build_mixed_batch(workload.index, [q for q, _ in workload.mix],
                                 list(ctx_lens) if ctx_lens is not None else [c for _, c in workload.mix],
                                 workload.spare_blocks)
    B, q = workload.num_seqs, workload.q_len
    if ctx_lens is None:
        ctx_lens = draw_ctx_lens(workload)
    seq_lens = [c + q for c in ctx_lens]
    nblk = [(s + KV_BLOCK - 1) // KV_BLOCK for s in seq_lens]
    total = sum(nblk) + workload.spare_blocks
    g = _gen(seed_of(workload.index, 0, T_BLOCKPERM), "cpu")
    perm = torch.randperm(total, generator=g).to(torch.int32)
    maxb = max(nblk)
    table = torch.full((B, maxb), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
    spare = [int(x) for x in perm[off:]]
    positions = torch.cat([torch.arange(c, c + q, dtype=torch.int32) for c in ctx_lens])
    return Batch(B, q, list(ctx_lens), torch.tensor(seq_lens, dtype=torch.int32), positions,
                 table, total, spare)


def build_mixed_batch(workload_index: int, q_lens: list, ctx_lens: list, spare_blocks: int = 4) -> Batch:
    """A mixed batch: sequence b has ctx_lens[b] cached positions and
    q_lens[b] >= 1 new rows (one row: a decode step; more: a prefill chunk on
    its context); rows are grouped by sequence in order.  Blocks are placed
    by a seeded random permutation, as in build_batch."""
    B = len(q_lens)
    if B != len(ctx_lens) or min(q_lens) < 1:
        raise ValueError("one (q_len >= 1, ctx) pair per sequence")
    seq_lens = [c + q for c, q in zip(ctx_lens, q_lens)]
    nblk = [(s + KV_BLOCK - 1) // KV_BLOCK for s in seq_lens]
    total = sum(nblk) + spare_blocks
    g = _gen(seed_of(workload_index, 0, T_BLOCKPERM), "cpu")
    perm = torch.randperm(total, generator=g).to(torch.int32)
    table = torch.full((B, max(nblk)), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
    spare = [int(x) for x in perm[off:]]
    positions = torch.cat([torch.arange(c, c + q, dtype=torch.int32) for c, q in zip(ctx_lens, q_lens)])
    return Batch(B, 0, list(ctx_lens), torch.tensor(seq_lens, dtype=torch.int32), positions, table, total, spare,
                 list(q_lens))


def sentinel_fill(t: torch.Tensor) -> torch.Tensor:
    """All-ones bit pattern: a NaN in both bf16 and fp32."""
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(-1)
    else:
        t.view(torch.int32).fill_(-1)
    return t


def pool_shape(model: ModelShape, num_blocks: int, plane: str = "k"):
    """K plane [num_blocks][kv_heads][16][head_dim]; V plane
    [num_blocks][kv_heads][head_dim][16] (the library header's layout)."""
    if plane == "k":
        return (num_blocks, model.num_key_value_heads, KV_BLOCK, model.head_dim)
    return (num_blocks, model.num_key_value_heads, model.head_dim, KV_BLOCK)


def _slot_major(pool: torch.Tensor, plane: str) -> torch.Tensor:
    """View of a plane as [blocks, kv_heads, 16, d] (a view, not a copy)."""
    return pool if plane == "k" else pool.transpose(2, 3)


def scatter_context(pool: torch.Tensor, batch: Batch, b: int, ctx: torch.Tensor, plane: str = "k") -> None:
    """Lay a logical context ``ctx`` [L, kv_heads, d] of sequence ``b`` into
    the paged pool at positions 0..L-1."""
    view = _slot_major(pool, plane)
    L = ctx.shape[0]
    full, rem = L // KV_BLOCK, L % KV_BLOCK
    if full:
        ids = batch.block_table[b, :full].long().to(pool.device)
        view[ids] = ctx[: full * KV_BLOCK].reshape(full, KV_BLOCK, ctx.shape[1], ctx.shape[2]).transpose(1, 2)
    if rem:
        blk = int(batch.block_table[b, full])
        view[blk, :, :rem, :] = ctx[full * KV_BLOCK:].transpose(0, 1)


def gather_context(pool: torch.Tensor, batch: Batch, b: int, length: int, plane: str = "k") -> torch.Tensor:
    """Read positions 0..length-1 of sequence ``b`` out of the paged pool as a
    logical [length, kv_heads, d] tensor."""
    view = _slot_major(pool, plane)
    nb = (length + KV_BLOCK - 1) // KV_BLOCK
    if nb == 0:
        return pool.new_empty((0, view.shape[1], view.shape[3]))
    ids = batch.block_table[b, :nb].long().to(pool.device)
    blocks = view.index_select(0, ids)                     # [nb, kv, 16, d]
    flat = blocks.permute(0, 2, 1, 3).reshape(nb * KV_BLOCK, view.shape[1], view.shape[3])
    return flat[:length]


def build_kv_pool(workload: Workload, batch: Batch, layer: int, device):
    """K and V pools for one layer: every slot sentinel-filled (NaN bits),
    then each sequence's cached context (positions 0..ctx-1) drawn N(0,1).
    Cached K counts as already rotated."""
    model = workload.model
    kp = sentinel_fill(torch.empty(pool_shape(model, batch.num_blocks, "k"), dtype=model.torch_dtype, device=device))
    vp = sentinel_fill(torch.empty(pool_shape(model, batch.num_blocks, "v"), dtype=model.torch_dtype, device=device))
    gk = _gen(seed_of(workload.index, layer, T_KCTX), device)
    gv = _gen(seed_of(workload.index, layer, T_VCTX), device)
    nkv, d = model.num_key_value_heads, model.head_dim
    for b, c in enumerate(batch.ctx_lens):
        if c == 0:
            continue
        for gen, pool, plane in ((gk, kp, "k"), (gv, vp, "v")):
            x = torch.randn((c, nkv, d), generator=gen, device=device, dtype=torch.float32)
            scatter_context(pool, batch, b, x.to(model.torch_dtype), plane)
    return kp, vp


def workload_tensors(workload: Workload, device, layers: Optional[int] = None):
    """Everything one forward (or a stack of ``layers`` forwards) consumes."""
    layers = workload.layers if layers is None else layers
    batch = build_batch(workload)
    h, r = draw_activations(workload.model, batch.num_tokens, workload.index, device,
                            residual=not workload.residual_none)
    per_layer = []
    for l in range(layers):
        w = draw_weights(workload.model, workload.index, l, device)
        kp, vp = build_kv_pool(workload, batch, l, device)
        per_layer.append({"weights": w, "k_pool": kp, "v_pool": vp})
    return batch, h, r, per_layer


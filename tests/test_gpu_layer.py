"""GPU parity of the whole layer forward (llama_layer_forward) against the
oracle, at sizes the oracle finishes in seconds: several GEMM tiles with
ragged tails, key partitions, block boundaries, prefill with and without a
cached context, decode at several batch sizes, the fp32 tiny workload, and
the first-layer (no residual) path.  Also: the KV cache is written exactly at
the new tokens' slots and nowhere else, and repeated calls are bitwise
identical."""
import ctypes

import numpy as np
import pytest
import torch

import llama_decoder_layer_amd as lda
import synth
import oracle
from tests import stages
from tests.kvbits import check_kv_bits
from tests.parity import (COS_MIN, compare, cosine, device_batch, device_qsl, np64, oracle_seqs, oracle_weights,
                          run_oracle)

pytestmark = pytest.mark.gpu
DEV = "cuda"

# a small bf16 model of the 70B layer's structure: GQA 4:1, head_dim 128,
# llama3 RoPE with the 70B parameters
MID = synth.ModelShape(1024, 8, 2, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")
# the 70B layer's group size (8 query heads per KV head) at a small width
MID8 = synth.ModelShape(1024, 8, 1, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")
# head_dim 64 variant
MID64 = synth.ModelShape(512, 16, 4, 64, 1408, 1e-5, 10000.0, None, 8192, "bf16")


def _run(workload, ctx_lens=None, layers=1, check_kv=True, repeat=False, qsl=None, kv_hook=None):
    """qsl: "auto" = query_start_loc of a mixed batch (None otherwise); a
    tensor to pass one explicitly (e.g. for a uniform batch).  kv_hook(batch,
    k_pool, v_pool) may reshape the drawn cached context in place.

    Every layer is checked against the oracle fed the GPU's own inputs to that
    layer (teacher forcing); a chain of layers is also compared end to end
    (cosine) with the oracle chained on itself."""
    model = workload.model
    batch = synth.build_batch(workload, ctx_lens)
    print("case", workload.name, "ctx", batch.ctx_lens[:8], "T", batch.num_tokens, flush=True)
    hidden, residual = synth.draw_activations(model, batch.num_tokens, workload.index, DEV,
                                              residual=not workload.residual_none)
    pos, bt, sl = device_batch(batch, DEV)
    if qsl is None:
        qsl = device_qsl(batch, DEV)
    meta0 = [t.clone() for t in (pos, bt, sl) + ((qsl,) if qsl is not None else ())]
    h, r = hidden, residual
    results = []
    T, B = batch.num_tokens, batch.num_seqs
    for l in range(layers):
        w = synth.draw_weights(model, workload.index, l, DEV)
        kp, vp = synth.build_kv_pool(workload, batch, l, DEV)
        if kv_hook is not None:
            kv_hook(batch, kp, vp)
        kp0, vp0 = kp.clone(), vp.clone()
        layer = lda.Layer(model.config_dict(), w)
        ws = layer.alloc_workspace(T, B, batch.max_seq_len)
        ho, ro = layer.forward(h, r, pos, kp, vp, bt, sl, batch.max_seq_len, workspace=ws, query_start_loc=qsl)
        torch.cuda.synchronize()
        qkv = layer.workspace_tensor(ws, "qkv", T, B, batch.max_seq_len).clone()
        table = layer.rope_table()
        wst = stages.workspace(layer, ws, T, B, batch.max_seq_len)
        if repeat:
            kp1, vp1 = kp.clone(), vp.clone()
            ho2, ro2 = layer.forward(h, r, pos, kp, vp, bt, sl, batch.max_seq_len, workspace=ws,
                                     query_start_loc=qsl)
            torch.cuda.synchronize()
            assert torch.equal(ho.view(torch.int16), ho2.view(torch.int16))
            assert torch.equal(ro.view(torch.int16), ro2.view(torch.int16))
            assert torch.equal(kp.view(torch.int16), kp1.view(torch.int16))
            assert torch.equal(vp.view(torch.int16), vp1.view(torch.int16))
        _check_metadata_unchanged(meta0, pos, bt, sl, qsl)
        if not (torch.isfinite(ho.float()).all() and torch.isfinite(ro.float()).all()):
            raise AssertionError("layer %d: %s" % (l, stages.nan_report(wst, {"hidden_out": ho, "residual_out": ro})))
        results.append((w, kp0, vp0, kp, vp, h, r, ho, ro, qkv, table, wst))
        h, r = ho, ro
        layer.close()

    dtype = model.dtype
    cfg = model.config_dict()
    posn = batch.positions.numpy().astype(np.int64)
    chained = None
    for l, (w, kp0, vp0, kp, vp, hin, rin, ho, ro, qkv, table, wst) in enumerate(results):
        seqs = oracle_seqs(model, batch, kp0, vp0)
        wn = oracle_weights(w)
        # teacher forcing: the oracle takes the GPU's own (bf16) inputs to this layer
        exact, rounded = run_oracle(model, wn, hin, rin, batch, seqs)
        s1 = compare("hidden_out[%d]" % l, np64(ho), exact["hidden_out"],
                     None if rounded is None else rounded["hidden_out"], dtype)
        s2 = compare("residual_out[%d]" % l, np64(ro), exact["residual_out"],
                     None if rounded is None else rounded["residual_out"], dtype)
        print("layer", l, "hidden_out", s1, "residual_out", s2, flush=True)
        print("layer", l, stages.summary(stages.check_stages(model, wn, batch, hin, rin, kp, vp, wst, ho, ro)),
              flush=True)
        if check_kv:
            _check_kv(model, batch, kp0, vp0, kp, vp, exact, rounded, qkv=qkv, table=table)
        if layers > 1:
            # the oracle chained on its own exact outputs, for an end-to-end cosine
            ch = chained if chained is not None else (np64(hidden), None if residual is None else np64(residual))
            ce = oracle.decoder_layer(cfg, wn, ch[0], ch[1], posn, seqs)
            chained = (ce["hidden_out"], ce["residual_out"])
    if layers > 1:
        for name, got, ref in (("hidden_out", results[-1][7], chained[0]), ("residual_out", results[-1][8], chained[1])):
            cos = cosine(np64(got), ref)
            print("chained %d layers %s cos %.7f" % (layers, name, cos), flush=True)
            assert cos >= COS_MIN, (name, cos)
    return [(ho, ro, kp, vp) for (_, _, _, kp, vp, _, _, ho, ro, _, _, _) in results]


def _check_metadata_unchanged(meta0, pos, bt, sl, qsl):
    """The forward reads positions, block_table, seq_lens and query_start_loc
    and never writes them."""
    now = (pos, bt, sl) + ((qsl,) if qsl is not None else ())
    for a, b in zip(meta0, now):
        assert torch.equal(a, b), "forward changed its metadata input"


def _new_slot_mask(batch):
    """[num_blocks, 16] bool: the slots of the batch's new tokens."""
    mask = torch.zeros(batch.num_blocks, 16, dtype=torch.bool)
    for b in range(batch.num_seqs):
        p = torch.arange(batch.ctx_lens[b], batch.ctx_lens[b] + batch.new_rows(b))
        mask[batch.block_table[b, p // 16].long(), p % 16] = True
    return mask


def _check_placement(model, batch, kp0, vp0, kp, vp):
    """Bit-exact: every byte outside the new tokens' slots is unchanged."""
    ibits = torch.int16 if model.dtype == "bf16" else torch.int32
    mask = _new_slot_mask(batch).to(kp.device)
    mk = mask[:, None, :, None].expand_as(kp)
    mv = mask[:, None, None, :].expand_as(vp)
    for name, new, old, m in (("K", kp, kp0, mk), ("V", vp, vp0, mv)):
        bad = (new.view(ibits) != old.view(ibits)) & ~m
        if bad.any():
            idx = bad.nonzero()[:8].tolist()  # (block, kv head, slot or component, component or slot)
            blk, hd = idx[0][0], idx[0][1]
            slot = idx[0][2] if name == "K" else idx[0][3]
            owner = (batch.block_table == blk).nonzero().tolist()  # (sequence, block index in its table)
            where = [(s, j * 16 + slot, batch.ctx_lens[s]) for s, j in owner]  # (sequence, position, context)
            row_old = old[blk, hd, slot, :4] if name == "K" else old[blk, hd, :4, slot]
            row_new = new[blk, hd, slot, :4] if name == "K" else new[blk, hd, :4, slot]
            raise AssertionError(
                "%s plane changed outside the new slots at %d entries, first %s; that block belongs to "
                "(sequence, position, context) %s; old %s new %s; changed (block, head) pairs %s" % (
                    name, int(bad.sum()), idx, where, row_old.tolist(), row_new.tolist(),
                    sorted(set((b, h) for b, h, _, _ in bad.nonzero().tolist()))[:12]))
    # and every new slot was written (no sentinel left)
    assert not torch.isnan(kp[mk].float()).any() and not torch.isnan(vp[mv].float()).any()


def _check_kv(model, batch, kp0, vp0, kp, vp, exact, rounded, qkv=None, table=None):
    """Placement bit-exact over the whole pool; with the workspace's qkv and
    the layer's RoPE table, the new slots' values bit-exact too (V a copy of
    the projection's v, K the kernel's documented float32 rotation of its k;
    K only without the q/k norm, whose reciprocal square root has no exact
    host emulation); and against the oracle under the tolerance."""
    _check_placement(model, batch, kp0, vp0, kp, vp)
    if qkv is not None:
        n = check_kv_bits(model, batch, kp, vp, qkv, table, check_k=not model.qk_norm)
        print("KV slots bit-exact:", n, "(K and V)" if not model.qk_norm else "(V)", flush=True)
    ks, vs, kref, vref, kr, vr = [], [], [], [], [], []
    for b in range(batch.num_seqs):
        c, n = batch.ctx_lens[b], int(batch.seq_lens[b])
        ks.append(np64(synth.gather_context(kp, batch, b, n, "k")[c:]))
        vs.append(np64(synth.gather_context(vp, batch, b, n, "v")[c:]))
        kref.append(exact["k_new"][b])
        vref.append(exact["v_new"][b])
        if rounded is not None:
            kr.append(rounded["k_new"][b])
            vr.append(rounded["v_new"][b])
    compare("k_cache", np.concatenate(ks), np.concatenate(kref), np.concatenate(kr) if kr else None, model.dtype)
    compare("v_cache", np.concatenate(vs), np.concatenate(vref), np.concatenate(vr) if vr else None, model.dtype)


def test_tiny_fp32_prefill():
    _run(synth.WORKLOADS["tiny_prefill_32"])


def test_mid_prefill_ragged_tiles():
    _run(synth.Workload(20, "mid_prefill_3x100", MID, 3, 100, 0), repeat=True)


def test_mid_prefill_on_cached_context():
    _run(synth.Workload(21, "mid_prefill_2x70_ctx", MID, 2, 70, 0), ctx_lens=[37, 200])


def test_mid_decode_block_and_partition_edges():
    _run(synth.Workload(22, "mid_decode_b6", MID, 6, 1, 0), ctx_lens=[0, 1, 15, 16, 1000, 3000], repeat=True)


def test_mid_decode_b40():
    _run(synth.Workload(23, "mid_decode_b40", MID, 40, 1, (1, 2000)))


def test_mid_decode_b65_tiled_path():
    _run(synth.Workload(24, "mid_decode_b65", MID, 65, 1, (100, 700)))


def test_mid_first_layer_no_residual():
    _run(synth.Workload(25, "mid_decode_b8_nores", MID, 8, 1, (10, 300), residual_none=True))


def test_mid_two_layer_stack():
    _run(synth.Workload(26, "mid_decode_b12_2layer", MID, 12, 1, (50, 900), layers=2), layers=2)


def test_mid8_prefill_ragged_query_tiles():
    _run(synth.Workload(27, "mid8_prefill_2x100", MID8, 2, 100, 0), repeat=True)


def test_mid8_prefill_on_cached_context():
    _run(synth.Workload(28, "mid8_prefill_3x37_ctx", MID8, 3, 37, 0), ctx_lens=[5, 300, 64])


def test_mid8_decode():
    _run(synth.Workload(29, "mid8_decode_b9", MID8, 9, 1, (1, 1500)))


def test_mid64_prefill_and_decode():
    _run(synth.Workload(30, "mid64_prefill_2x80", MID64, 2, 80, 0), ctx_lens=[0, 19])
    _run(synth.Workload(31, "mid64_decode_b5", MID64, 5, 1, (3, 700)))


# ---- mixed batches: per-sequence query counts through query_start_loc ----

def test_mid_mixed_prefill_chunks_and_decode():
    # decode rows, prefill chunks on cached contexts and a fresh prefill in one
    # call; 123 rows: the tiled projections and the query-tile table
    mix = ((1, 300), (37, 50), (64, 0), (1, 2000), (20, 777))
    _run(synth.Workload(32, "mid_mixed_5seq", MID, len(mix), 0, mix=mix), repeat=True)


def test_mid8_mixed_few_rows():
    # 24 rows: the weight-streaming projections with a mixed attention batch
    mix = ((1, 100), (1, 1500), (17, 40), (5, 0))
    _run(synth.Workload(33, "mid8_mixed_4seq", MID8, len(mix), 0, mix=mix))
    # short contexts: no key partitions, decode rows written directly
    mix = ((1, 30), (20, 10), (1, 5))
    _run(synth.Workload(47, "mid8_mixed_short", MID8, len(mix), 0, mix=mix))


def test_mid64_mixed():
    mix = ((33, 10), (1, 500), (2, 700))
    _run(synth.Workload(34, "mid64_mixed_3seq", MID64, len(mix), 0, mix=mix))


def test_mid8_mixed_long_context_key_partitions():
    # few query tiles on long contexts: the prefill kernel splits each tile's
    # keys into partitions (cut at or before the tile's first query position,
    # so a tile starting mid-way through a 64-key tile spans two), the single-
    # row sequences run on the decode kernel with the same partitions (one
    # partition: written directly; a row at position 0: one key), and the
    # combine merges only the rows that were split
    mix = ((1, 100), (64, 3000), (1, 1500), (40, 1000), (1, 2999), (1, 0), (3, 511))
    _run(synth.Workload(41, "mid8_mixed_long_ctx", MID8, len(mix), 0, mix=mix), repeat=True)


def test_mid64_mixed_key_partitions():
    mix = ((1, 1800), (48, 1500), (1, 900), (2, 1023))
    _run(synth.Workload(42, "mid64_mixed_long_ctx", MID64, len(mix), 0, mix=mix))


# 16 query heads per KV head: one wave serves two heads over 16-row tiles
MID16 = synth.ModelShape(1024, 16, 1, 64, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")


def test_mid16_mixed_and_prefill_key_partitions():
    mix = ((1, 700), (40, 1100), (3, 50), (1, 1))
    _run(synth.Workload(43, "mid16_mixed", MID16, len(mix), 0, mix=mix))
    _run(synth.Workload(44, "mid16_prefill_1x48_ctx1500", MID16, 1, 48, 1500))


# the two remaining (head_dim, heads per KV head) forms of the prefill kernel:
# 128 x 16 (two heads per wave, 16-query tiles) and 64 x 8 (one head per wave)
MID128G16 = synth.ModelShape(2048, 16, 1, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")
MID64G8 = synth.ModelShape(512, 8, 1, 64, 1408, 1e-5, 10000.0, None, 8192, "bf16")


@pytest.mark.parametrize("model, tag, base", [(MID128G16, "mid128g16", 214), (MID64G8, "mid64g8", 218)])
def test_remaining_prefill_forms_and_their_decode(model, tag, base):
    # prefill chunks on cached contexts, a ragged last query tile
    _run(synth.Workload(base, tag + "_prefill_3x37_ctx", model, 3, 37, 0), ctx_lens=[5, 300, 64])
    # a uniform chunk on a long context: key partitions and the combine
    _run(synth.Workload(base + 1, tag + "_prefill_1x64_ctx2000", model, 1, 64, 2000))
    # a mixed batch: decode rows beside prefill chunks, with key partitions
    mix = ((1, 700), (40, 1100), (3, 50), (1, 1))
    _run(synth.Workload(base + 2, tag + "_mixed", model, len(mix), 0, mix=mix))
    # uniform decode: the attention kernel sums the qkv partials itself
    _run(synth.Workload(base + 3, tag + "_decode_b7", model, 7, 1, (1, 1800)))


# hidden sizes that give the decode qkv projection 2 and 4 split-K planes (the
# 70B-like shapes above all give 8), which the decode attention kernel sums
# in its prologue; the query width (8 x 64) differs from the hidden size
SPLIT2 = synth.ModelShape(640, 8, 2, 64, 1536, 1e-5, 10000.0, None, 8192, "bf16")
SPLIT4 = synth.ModelShape(768, 8, 2, 64, 1536, 1e-5, 10000.0, None, 8192, "bf16")


@pytest.mark.parametrize("model, tag, base", [(SPLIT2, "h640", 222), (SPLIT4, "h768", 226)])
def test_decode_qkv_partial_plane_counts(model, tag, base):
    _run(synth.Workload(base, tag + "_decode_b7", model, 7, 1, (1, 1800)))
    _run(synth.Workload(base + 1, tag + "_decode_b24", model, 24, 1, (100, 900)))
    _run(synth.Workload(base + 2, tag + "_prefill_2x70_ctx", model, 2, 70, 0), ctx_lens=[0, 333])
    mix = ((1, 500), (30, 200), (1, 17))
    _run(synth.Workload(base + 3, tag + "_mixed", model, len(mix), 0, mix=mix))


# the weight-streaming kernel's tall-weight forms (gate_up of at least 49152
# rows, K % 256 == 0): 7 waves of 32 rows when the rows tile exactly onto 256
# CUs (57344 rows, the 70B gate_up's count), else 4 waves (49152 rows); each
# at 1, 2, 4 and 8 token tiles (12, 32, 64, 100 rows)
TALL7 = synth.ModelShape(512, 8, 2, 64, 28672, 1e-5, 10000.0, None, 8192, "bf16")
TALL4 = synth.ModelShape(512, 8, 2, 64, 24576, 1e-5, 10000.0, None, 8192, "bf16")


@pytest.mark.parametrize("model, tag, base", [(TALL7, "tall7", 230), (TALL4, "tall4", 234)])
def test_tall_gate_up_forms(model, tag, base):
    for i, rows in enumerate((12, 32, 64, 100)):
        _run(synth.Workload(base + i, "%s_decode_b%d" % (tag, rows), model, rows, 1, (1, 600)))


# a 5120-row qkv (32 query heads, 4 KV heads of 128, as the Qwen3-MoE layer's
# attention) is the weight the 5-wave single-tile forms of the weight-streaming
# kernel suit: 4 split-K planes at 33..128 rows, which the decode attention then
# sums in its prologue at head_dim 128
QDENSE = synth.ModelShape(2048, 32, 4, 128, 2816, 1e-6, 1e7, None, 32768, "bf16")


def test_five_wave_qkv_forms():
    _run(synth.Workload(240, "qdense_decode_b48", QDENSE, 48, 1, (1, 900)))
    _run(synth.Workload(241, "qdense_decode_b100", QDENSE, 100, 1, (1, 400)))


def test_mid8_uniform_prefill_split_keys():
    # a uniform (no query_start_loc) chunk on a long context splits too
    _run(synth.Workload(45, "mid8_prefill_1x64_ctx2000", MID8, 1, 64, 2000), repeat=True)


def _ramp_keys(scale_per_key):
    """kv_hook: cached key at position p multiplied by 1 + p * scale_per_key,
    so scores grow along the context and each new tile's max keeps rising."""
    def hook(batch, kp, vp):
        for b, c in enumerate(batch.ctx_lens):
            if c == 0:
                continue
            x = synth.gather_context(kp, batch, b, c).float()
            ramp = 1.0 + scale_per_key * torch.arange(c, device=x.device, dtype=torch.float32)
            synth.scatter_context(kp, batch, b, (x * ramp[:, None, None]).to(kp.dtype))
    return hook


def test_mid8_prefill_rising_scores_move_reference_max():
    # The online softmax keeps its reference max until a tile's max exceeds
    # it by 8 (log2 units).  With keys growing 1 + p/250 along the context
    # the reference moves on about a sixth of the later (wave, tile) steps
    # of the first case (127 of 736, counted on the CPU from the same inputs)
    # and is kept with P above 1 on the rest; with 1 + p/40 it moves on most
    # of them.  Cases: a chunk on a long context (split keys merged by the
    # combine), two chunks on a short one, a mixed batch with decode rows, and
    # a decode batch.
    _run(synth.Workload(70, "mid8_prefill_1x64_ctx1500_ramp", MID8, 1, 64, 1500), kv_hook=_ramp_keys(1 / 250))
    _run(synth.Workload(71, "mid8_prefill_2x150_ctx300_ramp", MID8, 2, 150, 300), kv_hook=_ramp_keys(1 / 40))
    mix = ((1, 1200), (48, 900), (1, 64))
    _run(synth.Workload(72, "mid8_mixed_ramp", MID8, len(mix), 0, mix=mix), kv_hook=_ramp_keys(1 / 250))
    # decode kernel: 6 sequences on one KV head split their keys into many
    # short partitions, each with its own reference max for the combine
    _run(synth.Workload(74, "mid8_decode_b6_ramp", MID8, 6, 1, 0), ctx_lens=[17, 300, 1000, 1999, 2500, 64],
         kv_hook=_ramp_keys(1 / 250))


def test_tiny_fp32_mixed():
    # fp32 and a 2:1 group: the generic attention kernel reads the row map
    mix = ((1, 20), (9, 3), (4, 0))
    _run(synth.Workload(35, "tiny_mixed_3seq", synth.TINY, len(mix), 0, mix=mix))


def test_explicit_query_start_loc_matches_uniform():
    # a uniform batch given its query_start_loc takes the tile-table path (and
    # a decode batch the decode path): results are bit-identical to NULL
    for wl, ctx in [(synth.Workload(36, "mid8_prefill_2x100_q", MID8, 2, 100, 0), [0, 33]),
                    (synth.Workload(37, "mid_decode_b7_q", MID, 7, 1, 0), [3, 15, 16, 17, 400, 1000, 2500]),
                    # split key ranges: the same partitions either way
                    (synth.Workload(46, "mid8_prefill_2x64_q", MID8, 2, 64, 0), [1500, 2000])]:
        batch = synth.build_batch(wl, ctx)
        qsl = torch.arange(0, batch.num_tokens + 1, wl.q_len, dtype=torch.int32, device=DEV)
        a = _run(wl, ctx_lens=ctx, check_kv=False)
        b = _run(wl, ctx_lens=ctx, check_kv=False, qsl=qsl)
        for x, y in zip(a[0], b[0]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_query_start_loc_host_checks():
    model = MID
    wl = synth.Workload(38, "mid_mixed_checks", model, 3, 0, mix=((1, 10), (2, 5), (1, 7)))
    batch = synth.build_batch(wl)
    hidden, residual = synth.draw_activations(model, batch.num_tokens, wl.index, DEV)
    pos, bt, sl = device_batch(batch, DEV)
    w = synth.draw_weights(model, wl.index, 0, DEV)
    kp, vp = synth.build_kv_pool(wl, batch, 0, DEV)
    layer = lda.Layer(model.config_dict(), w)
    try:
        with pytest.raises(ValueError):  # wrong length, caught by the binding
            layer.forward(hidden, residual, pos, kp, vp, bt, sl, batch.max_seq_len,
                          query_start_loc=torch.zeros(3, dtype=torch.int32, device=DEV))
        with pytest.raises(lda.LlamaError, match="every sequence needs a query row"):
            # two rows for three sequences
            layer.forward(hidden[:2], residual[:2], pos[:2], kp, vp, bt, sl, batch.max_seq_len,
                          query_start_loc=torch.tensor([0, 1, 1, 2], dtype=torch.int32, device=DEV))
    finally:
        layer.close()


def test_forward_host_checks_write_nothing():
    # Host-side rejections of llama_layer_forward: each returns an error
    # before any launch, so the outputs and the KV cache keep their contents.
    model = MID
    wl = synth.Workload(73, "mid_decode_checks", model, 3, 1, (20, 90))
    batch = synth.build_batch(wl)
    hidden, residual = synth.draw_activations(model, batch.num_tokens, wl.index, DEV)
    pos, bt, sl = device_batch(batch, DEV)
    w = synth.draw_weights(model, wl.index, 0, DEV)
    kp, vp = synth.build_kv_pool(wl, batch, 0, DEV)
    kp0, vp0 = kp.clone(), vp.clone()
    T, H = hidden.shape
    ho = torch.full_like(hidden, 7.0)
    ro = torch.full_like(hidden, -7.0)
    L = lda.lib()
    layer = lda.Layer(model.config_dict(), w)
    ws = layer.alloc_workspace(T, batch.num_seqs, batch.max_seq_len)

    def call(h=hidden, T_=T, B=batch.num_seqs, msl=batch.max_seq_len, hout=ho, rout=ro):
        kv = lda.KvCache(kp.data_ptr(), vp.data_ptr(), kp.shape[0])
        return L.llama_layer_forward(layer._h, h.data_ptr(), residual.data_ptr(), pos.data_ptr(), T_,
                                     ctypes.byref(kv), bt.data_ptr(), bt.shape[1], sl.data_ptr(), None, B, msl,
                                     hout.data_ptr(), rout.data_ptr(), ws.data_ptr(), None)

    try:
        flat = torch.empty(T * H + 1, dtype=hidden.dtype, device=DEV)
        misaligned = flat[1:].view(T, H)
        misaligned.copy_(hidden)
        cases = [
            (dict(T_=0), "must be positive"),                                    # empty batch
            (dict(B=0), "must be positive"),                                     # no sequences
            (dict(T_=2), "multiple of num_seqs"),                                # ragged uniform batch
            (dict(msl=bt.shape[1] * 16 + 1), "cannot hold"),                     # table too short
            (dict(rout=ho), "aliases"),                                          # outputs alias
            (dict(h=misaligned), "16-byte aligned"),                             # misaligned activations
        ]
        for kw, msg in cases:
            st = call(**kw)
            assert st == lda.Status.INVALID_ARGUMENT, (kw, st)
            assert msg in L.llama_layer_last_error().decode(), (kw, L.llama_layer_last_error())
        torch.cuda.synchronize()
        assert bool((ho == 7.0).all()) and bool((ro == -7.0).all())
        assert torch.equal(kp.view(torch.int16), kp0.view(torch.int16))
        assert torch.equal(vp.view(torch.int16), vp0.view(torch.int16))
        # and the same call with valid arguments runs
        assert call() == lda.Status.OK
        torch.cuda.synchronize()
        assert not bool((ho == 7.0).all())
    finally:
        layer.close()


def test_mid_decode_b128_and_b129():
    # 128 rows: the largest weight-streaming batch (8 token tiles); 129: tiled
    _run(synth.Workload(39, "mid_decode_b128", MID, 128, 1, (1, 600)))
    _run(synth.Workload(40, "mid_decode_b129", MID, 129, 1, (1, 600)))


def test_debug_mode_metadata_checks(monkeypatch):
    # LLAMA_DEBUG=1: one kernel checks block ids, positions, KV lengths and
    # row ranges before anything runs, and a broken condition is rejected
    # with nothing written.  Every broken input below stays inside allocated
    # memory (block ids point into spare pool blocks the call is not told
    # of), so the layer could not fault even if the check missed one.
    model = MID8
    wl = synth.Workload(48, "mid8_debug_b4", model, 4, 1, (20, 100))
    batch = synth.build_batch(wl)
    print("case", wl.name, "ctx", batch.ctx_lens, flush=True)
    hidden, residual = synth.draw_activations(model, batch.num_tokens, wl.index, DEV)
    pos, bt, sl = device_batch(batch, DEV)
    w = synth.draw_weights(model, wl.index, 0, DEV)
    kp, vp = synth.build_kv_pool(wl, batch, 0, DEV)
    n = kp.shape[0]
    kbig = torch.cat([kp, kp[:4]])  # 4 spare blocks past the declared pool
    vbig = torch.cat([vp, vp[:4]])
    layer = lda.Layer(model.config_dict(), w)
    try:
        ho_ref, ro_ref = layer.forward(hidden, residual, pos, kbig[:n].clone(), vbig[:n].clone(), bt, sl,
                                       batch.max_seq_len)
        monkeypatch.setenv("LLAMA_DEBUG", "1")
        ho, ro = layer.forward(hidden, residual, pos, kbig[:n].clone(), vbig[:n].clone(), bt, sl, batch.max_seq_len)
        torch.cuda.synchronize()
        assert torch.equal(ho.view(torch.int16), ho_ref.view(torch.int16))
        assert torch.equal(ro.view(torch.int16), ro_ref.view(torch.int16))

        def rejected(match, pos_=pos, bt_=bt, sl_=sl, qsl=None, rows=None, msl=batch.max_seq_len):
            h_, r_ = (hidden, residual) if rows is None else rows
            k0, v0 = kbig.clone(), vbig.clone()
            hout = torch.full_like(h_, 7.0)
            rout = torch.full_like(r_, 7.0)
            with pytest.raises(lda.LlamaError, match=match) as ei:
                layer.forward(h_, r_, pos_, kbig[:n], vbig[:n], bt_, sl_, msl, hidden_out=hout,
                              residual_out=rout, query_start_loc=qsl)
            assert ei.value.status == lda.Status.INVALID_ARGUMENT
            torch.cuda.synchronize()
            assert bool((hout == 7.0).all()) and bool((rout == 7.0).all())
            assert torch.equal(kbig.view(torch.int16), k0.view(torch.int16))
            assert torch.equal(vbig.view(torch.int16), v0.view(torch.int16))

        bad = bt.clone()
        bad[1, 0] = n + 1  # allocated, but past kv_cache.num_blocks
        rejected("block_table", bt_=bad)
        bad = bt.clone()
        bad[0, 5] = n + 3  # sequence 0's last block (KV length 89), where its new token goes
        rejected("block_table", bt_=bad)
        p2 = pos.clone()
        p2[1] -= 1  # no longer seq_lens - 1
        rejected("position", pos_=p2)
        s2 = sl.clone()
        s2[0] = batch.max_seq_len + 1
        rejected("seq_lens", sl_=s2)

        # a mixed batch: row ranges out of order
        mix = ((1, 30), (5, 10), (1, 7))
        wm = synth.Workload(49, "mid8_debug_mixed", model, len(mix), 0, mix=mix)
        bm = synth.build_batch(wm)
        hm, rm = synth.draw_activations(model, bm.num_tokens, wm.index, DEV)
        pm, btm, slm = device_batch(bm, DEV)
        qsl = device_qsl(bm, DEV)
        assert bm.num_blocks <= n
        layer.forward(hm, rm, pm, kbig[:n].clone(), vbig[:n].clone(), btm, slm, bm.max_seq_len,
                      query_start_loc=qsl)
        q2 = torch.tensor([0, 6, 1, 7], dtype=torch.int32, device=DEV)  # rows of 1 and 5 swapped
        assert qsl.tolist() == [0, 1, 6, 7]
        rejected("query_start_loc", pos_=pm, bt_=btm, sl_=slm, qsl=q2, rows=(hm, rm), msl=bm.max_seq_len)
    finally:
        layer.close()


# hidden 8192 with a narrow attention (32 query heads on 8 KV heads, K = 4096
# for o_proj) and MLP (K = 1024 for down_proj): at decode both projections
# have 8192 output rows, one 32-row workgroup per CU, and a short K, so they
# split K inside the workgroup and write their final rows (o_proj with the
# residual add) instead of partial planes
WIDE = synth.ModelShape(8192, 32, 8, 128, 1024, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")


def test_wide_decode_in_workgroup_split_k():
    for idx, b in ((54, 8), (55, 32), (56, 64)):  # 1, 2 and 4 token tiles
        _run(synth.Workload(idx, "wide_decode_b%d" % b, WIDE, b, 1, (10, 300)))


def test_mid_positions_at_the_configured_maximum():
    # the last position max_position_embeddings - 1 = 131071: the far end of
    # the llama3 RoPE table, decode over 64 key partitions of 2048 (merged by
    # the combine), and a 64-row chunk on a 131008-token context whose query
    # tiles split their keys into 8 partitions
    _run(synth.Workload(66, "mid_decode_maxpos", MID, 2, 1, 0), ctx_lens=[131071, 70000])
    _run(synth.Workload(67, "mid_chunk_maxpos", MID, 1, 64, 0), ctx_lens=[131008])


def test_decode_new_token_opens_a_block_head_dim_64():
    # every new token at slot 0 of a fresh block (contexts multiples of 16)
    _run(synth.Workload(238, "mid64_decode_b6_block_starts", MID64, 6, 1, 0), ctx_lens=[16, 32, 416, 64, 0, 160])
    _run(synth.Workload(239, "h640_decode_b12_block_starts", SPLIT2, 12, 1, 0),
         ctx_lens=[92, 493, 425, 25, 546, 529, 141, 232, 145, 367, 504, 416])

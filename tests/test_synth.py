"""The seeded input generator: reproducible draws, block tables that place
every sequence's blocks without overlap, and the paged-pool layout helpers
(scatter then gather gives the context back; the V plane keeps the 16 slots
of one component contiguous)."""
import torch

import synth

SMALL = synth.ModelShape(256, 4, 2, 64, 512, 1e-5, 1e4, None, 4096, "bf16")


def test_draws_are_seeded():
    a = synth.draw_weights(SMALL, 3, 1, "cpu")
    b = synth.draw_weights(SMALL, 3, 1, "cpu")
    c = synth.draw_weights(SMALL, 3, 2, "cpu")
    for k in a:
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
    assert abs(a["qkv_proj"].float().std().item() - 0.02) < 0.002
    assert abs(a["input_layernorm"].float().mean().item() - 1.0) < 0.01


def test_block_table_is_a_placement():
    wl = synth.WORKLOADS["llama70b_ragged_decode_b64_4layer"]
    lens = synth.draw_ctx_lens(wl)
    assert len(lens) == 64 and min(lens) >= 128 and max(lens) <= 32768
    assert lens == synth.draw_ctx_lens(wl)
    b = synth.build_batch(wl)
    used = []
    for i in range(b.num_seqs):
        nb = (int(b.seq_lens[i]) + 15) // 16
        row = b.block_table[i]
        assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
        used += row[:nb].tolist()
    assert len(set(used)) == len(used)
    assert sorted(used + b.spare_blocks) == list(range(b.num_blocks))
    assert b.positions.tolist() == [c for c in lens]


def test_pool_round_trip_and_layout():
    wl = synth.Workload(40, "t", SMALL, 3, 1, 0)
    b = synth.build_batch(wl, [0, 17, 50])
    kp, vp = synth.build_kv_pool(wl, b, 0, "cpu")
    for s in range(3):
        for plane, pool in (("k", kp), ("v", vp)):
            c = synth.gather_context(pool, b, s, b.ctx_lens[s], plane)
            assert c.shape == (b.ctx_lens[s], 2, 64) and torch.isfinite(c.float()).all()
    # slots past each context stay sentinel (NaN)
    blk = int(b.block_table[1, 1])
    assert torch.isnan(kp[blk, :, 1:, :].float()).all() and torch.isnan(vp[blk, :, :, 1:].float()).all()
    x = torch.randn(50, 2, 64).to(torch.bfloat16)
    synth.scatter_context(vp, b, 2, x, "v")
    synth.scatter_context(kp, b, 2, x, "k")
    assert torch.equal(synth.gather_context(vp, b, 2, 50, "v"), x)
    assert torch.equal(synth.gather_context(kp, b, 2, 50, "k"), x)
    blk = int(b.block_table[2, 0])
    assert torch.equal(vp[blk, 1, 5, 3], x[3, 1, 5])   # V: [block][head][component][slot]
    assert torch.equal(kp[blk, 1, 3, 5], x[3, 1, 5])   # K: [block][head][slot][component]


def test_mixed_batch_rows_positions_and_offsets():
    mix = ((1, 300), (37, 50), (64, 0), (1, 16))
    wl = synth.Workload(90, "mixed_check", synth.TINY, len(mix), 0, mix=mix)
    batch = synth.build_batch(wl)
    assert batch.mixed and batch.num_tokens == 103 == wl.num_tokens
    assert batch.query_start_loc.tolist() == [0, 1, 38, 102, 103]
    assert [list(batch.rows(b)) for b in (0, 3)] == [[0], [102]]
    assert batch.seq_of_row() == [0] + [1] * 37 + [2] * 64 + [3]
    # each sequence's rows continue its cached context
    for b, (q, c) in enumerate(mix):
        assert batch.positions[batch.rows(b).start: batch.rows(b).stop].tolist() == list(range(c, c + q))
        assert int(batch.seq_lens[b]) == c + q
        nblk = (c + q + 15) // 16
        assert (batch.block_table[b, :nblk] >= 0).all() and (batch.block_table[b, nblk:] == -1).all()
    # every referenced block is distinct and inside the pool
    used = batch.block_table[batch.block_table >= 0]
    assert used.unique().numel() == used.numel() and int(used.max()) < batch.num_blocks

"""GPU parity of the single-step entry points (the kernels the forward
launches) against the oracle's steps, on seeded inputs."""
import numpy as np
import pytest
import torch

import llama_decoder_layer_amd as lda
import oracle
from tests.parity import compare, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _randn(shape, seed, dtype=torch.bfloat16, std=1.0, mean=0.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * std + mean).to(dtype).to(DEV)


# 300 and 544 tokens take 192-row token tiles (less padding than 256)
@pytest.mark.parametrize("M", [1, 7, 16, 32, 33, 64, 65, 128, 300, 544, 1024])
@pytest.mark.parametrize("N,K", [(256, 512), (1536, 1024)])
def test_linear_store(M, N, K):
    print("linear_store", M, N, K, flush=True)
    x = _randn((M, K), 1 + M)
    w = _randn((N, K), 2 + N, std=0.02)
    y = lda.linear(x, w)
    torch.cuda.synchronize()
    ref = oracle.linear(np64(x), np64(w))
    compare("linear", np64(y), ref, dtype="bf16")


@pytest.mark.timeout(300)
def test_linear_store_chunked_tile_order():
    # more than 32 token tiles (34, the last one partial) over 64 weight tiles
    # of 256 rows: the tiled kernel's XCD-grouped order, walking the weight
    # tiles in two chunks of 32
    M, N, K = 8500, 16384, 128
    print("linear_store chunked order", M, N, K, flush=True)
    x = _randn((M, K), 31)
    w = _randn((N, K), 32, std=0.05)
    y = lda.linear(x, w)
    torch.cuda.synchronize()
    ref = oracle.linear(np64(x), np64(w))
    compare("linear chunked order", np64(y), ref, dtype="bf16")


@pytest.mark.parametrize("M", [5, 32, 64, 100, 200, 544])
def test_linear_add(M):
    print("linear_add", M, flush=True)
    N, K = 1024, 768
    x = _randn((M, K), 11)
    w = _randn((N, K), 12, std=0.02)
    r = _randn((M, N), 13)
    out = r.clone()
    lda.linear(x, w, lda.Epilogue.ADD, out=out)
    torch.cuda.synchronize()
    exact = oracle.linear(np64(x), np64(w)) + np64(r)
    compare("linear_add", np64(out), exact, dtype="bf16")


@pytest.mark.parametrize("M", [3, 32, 64, 100, 129, 300])
def test_linear_silu_mul(M):
    print("linear_silu", M, flush=True)
    I, K = 384, 512
    x = _randn((M, K), 21)
    w = _randn((2 * I, K), 22, std=0.05)
    # asymmetric halves so swapped gate/up would show
    w[I:] *= 3.0
    wr = lda.reorder_gate_up(w)
    out = lda.linear(x, wr, lda.Epilogue.SILU_MUL)
    torch.cuda.synchronize()
    exact = oracle.silu_and_mul(oracle.linear(np64(x), np64(w)))
    compare("silu_mul", np64(out), exact, dtype="bf16")


def test_reorder_gate_up_is_a_permutation():
    I, K = 64, 64
    w = torch.arange(2 * I, dtype=torch.float32)[:, None].repeat(1, K).to(torch.bfloat16).to(DEV)
    r = lda.reorder_gate_up(w)
    rows = r[:, 0].float().cpu().numpy().astype(int)
    expect = []
    for grp in range(2 * I // 32):
        expect += list(range(16 * grp, 16 * grp + 16)) + list(range(I + 16 * grp, I + 16 * grp + 16))
    assert rows.tolist() == expect


@pytest.mark.parametrize("dtype", [torch.float32])
@pytest.mark.parametrize("M,N,K", [(1, 16, 8), (33, 70, 45), (32, 688, 256)])
def test_linear_fp32(dtype, M, N, K):
    x = _randn((M, K), 31, dtype)
    w = _randn((N, K), 32, dtype, std=0.1)
    y = lda.linear(x, w)
    torch.cuda.synchronize()
    compare("linear_f32", np64(y), oracle.linear(np64(x), np64(w)), dtype="fp32")
    w2 = _randn((2 * N, K), 33, dtype, std=0.1)
    y2 = lda.linear(x, w2, lda.Epilogue.SILU_MUL)
    torch.cuda.synchronize()
    compare("silu_f32", np64(y2), oracle.silu_and_mul(oracle.linear(np64(x), np64(w2))), dtype="fp32")


@pytest.mark.parametrize("rows,H", [(1, 128), (7, 1024), (33, 8192), (5, 16384), (257, 8192)])
def test_add_rmsnorm_bf16(rows, H):
    print("rmsnorm", rows, H, flush=True)
    x = _randn((rows, H), 41)
    r = _randn((rows, H), 42)
    w = _randn((H,), 43, std=0.5, mean=1.0)
    h, ro = lda.add_rmsnorm(x, r, w, 1e-5)
    torch.cuda.synchronize()
    # the residual is the bf16-rounded sum: bit-exact against the oracle's
    # storage rounding
    hr, rr = oracle.fused_add_rms_norm(np64(x), np64(r), np64(w), 1e-5, oracle.bf16_round)
    np.testing.assert_array_equal(np64(ro), rr)
    he, _ = oracle.fused_add_rms_norm(np64(x), np64(r), np64(w), 1e-5)
    compare("rmsnorm", np64(h), he, oracle.rms_norm(rr, np64(w), 1e-5), dtype="bf16")
    # None path: residual_out is a bit copy of x
    h0, r0 = lda.add_rmsnorm(x, None, w, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(r0.view(torch.int16), x.view(torch.int16))
    compare("rmsnorm0", np64(h0), oracle.rms_norm(np64(x), np64(w), 1e-5), dtype="bf16")


def test_add_rmsnorm_fp32():
    x = _randn((9, 256), 51, torch.float32)
    r = _randn((9, 256), 52, torch.float32)
    w = _randn((256,), 53, torch.float32, std=0.5, mean=1.0)
    h, ro = lda.add_rmsnorm(x, r, w, 1e-5)
    torch.cuda.synchronize()
    he, re_ = oracle.fused_add_rms_norm(np64(x), np64(r), np64(w), 1e-5)
    compare("rmsnorm_f32", np64(h), he, dtype="fp32")
    compare("residual_f32", np64(ro), re_, dtype="fp32")


def test_diag_block_read_reads_the_listed_blocks():
    # each thread folds word t of every block its workgroup reads: compare
    # with the same fold on the host (uneven split: 37 blocks, 4 workgroups)
    rng = np.random.default_rng(3)
    nb, bb, wgs = 64, 4096, 4
    words = rng.integers(0, 2 ** 32, size=(nb, bb // 16, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).reshape(-1)).to(DEV)
    ids = rng.permutation(nb)[:37].astype(np.int32)
    sink = torch.empty(wgs * bb // 16, dtype=torch.int32, device=DEV)
    for nt in (False, True):
        lda.block_read(src, torch.from_numpy(ids).to(DEV), bb, wgs, sink, nontemporal=nt)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32).reshape(wgs, bb // 16)
        per = (len(ids) + wgs - 1) // wgs
        fold = np.bitwise_xor.reduce(words, axis=2)  # [nb, words]
        for w in range(wgs):
            sel = ids[w * per:(w + 1) * per]
            want = np.bitwise_xor.reduce(fold[sel], axis=0) if len(sel) else np.zeros(bb // 16, np.uint32)
            assert np.array_equal(got[w], want), (nt, w)

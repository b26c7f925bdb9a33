"""The seeded generator: determinism, the shapes it promises, and the pool
structure (every owned slot referenced once, everything else NaN)."""

import numpy as np
import pytest
import torch

from workloads import WORKLOADS, build_batch, make_workload, repermute_pool, workload_lengths


def lengths(name):
    seed = WORKLOADS[name][0]
    return workload_lengths(name, np.random.SeedSequence(seed).spawn(4))


def test_same_seed_same_bytes():
    a = make_workload("tiny_mixed_3seq")
    b = make_workload("tiny_mixed_3seq")
    for n in ("q", "k_cache", "v_cache", "block_table", "cu_seqlens_q", "seqused_k"):
        x, y = getattr(a, n), getattr(b, n)
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), n


def test_tiny_workload_shape():
    b = make_workload("tiny_mixed_3seq")
    assert b.cu_seqlens_q.tolist() == [0, 1, 6, 22]
    assert b.seqused_k.tolist() == [7, 20, 40]
    assert tuple(b.q.shape) == (22, 4, 64) and tuple(b.k_cache.shape) == (16, 16, 2, 64)
    assert b.block_table.shape == (3, 3) and b.max_seqlen_q == 16 and b.max_seqlen_k == 40
    assert b.softmax_scale == 0.125 and b.causal


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_lengths(name):
    q, k, pool = lengths(name)
    assert q.shape == k.shape and (q >= 0).all() and (k >= 1).all()
    if name == "decode_256seq_ctx1k":
        assert len(q) == 256 and (q == 1).all() and k.min() >= 1000 and k.max() <= 1100
    if name == "mixed_prefill512x8_decode248":
        assert len(q) == 256 and (q == 512).sum() == 8 and (q == 1).sum() == 248
        assert (k[q == 512] >= 512).all() and (k[q == 512] <= 2048).all()
        assert k[q == 1].min() >= 4 and k[q == 1].max() <= 8192
        assert not (q[:8] == 512).all()            # shuffled order
    if name.startswith("prefill512x8_only"):
        assert len(q) == 8 and (q == 512).all()
    if name == "decode248_only":
        assert len(q) == 248 and (q == 1).all()
    if name == "decode_gqa8_64seq_ctx2k_4k":
        assert len(q) == 64 and k.min() >= 2048 and k.max() <= 4096
    if name.startswith("long_"):
        assert len(q) == 16 and k.min() >= 32768 and k.max() <= 131072
        assert (q == (16 if "q16" in name else 1)).all()


def test_mixed_subsets_share_draws():
    q, k, _ = lengths("mixed_prefill512x8_decode248")
    qp, kp, _ = lengths("prefill512x8_only")
    qd, kd, _ = lengths("decode248_only")
    assert (kp == k[q == 512]).all() and (kd == k[q == 1]).all()
    for d in (96, 256):
        qx, kx, _ = lengths(f"prefill512x8_only_d{d}")
        assert (qx == qp).all() and (kx == kp).all()


def test_pool_structure():
    b = build_batch("t", [1, 3, 0, 7], [5, 16, 9, 33], 4, 2, 8, True, seed=3,
                    block_size=4, pool_blocks=40)
    table = b.block_table.numpy()
    owned = np.zeros((40, 4), dtype=int)
    for s, L in enumerate([5, 16, 9, 33]):
        for j in range(L):
            owned[table[s, j // 4], j % 4] += 1
        assert (table[s, -(-L // 4):] == b.trap_block).all()
    assert owned.max() == 1
    k = b.k_cache.float().numpy()
    assert np.isnan(k[owned == 0]).all() and np.isfinite(k[owned == 1]).all()
    assert np.isnan(k[b.trap_block]).all()


def test_repermute_keeps_logical_content():
    b = build_batch("t", [2, 1], [13, 6], 4, 2, 8, True, seed=5, block_size=4)
    c = repermute_pool(b, seed=9)
    for s, L in enumerate([13, 6]):
        for j in range(L):
            x = b.k_cache[b.block_table[s, j // 4], j % 4]
            y = c.k_cache[c.block_table[s, j // 4], j % 4]
            assert torch.equal(x, y)
    assert not torch.equal(b.block_table, c.block_table)

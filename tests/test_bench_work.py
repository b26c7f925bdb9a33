"""The benchmark's algorithmic work (the numerators of every roofline figure)
against values derived by hand from the definitions: KV bytes = every valid
context token's K and V read once, Q + out = read and written once, flops =
4 d Hq per admissible (query, key) pair, with the end-aligned causal mask."""

import bench
from workloads import build_batch, make_workload


def test_tiny_batch_work():
    # 3 sequences (q, L) = (1, 7), (5, 20), (16, 40); 4 q-heads, 2 kv-heads, d 64.
    # Admissible pairs per head: 7 + (16 + ... + 20) + (25 + ... + 40) = 7 + 90 + 520
    b = make_workload("tiny_mixed_3seq")
    total, kv, flops = bench.algorithmic_work(b)
    assert kv == 67 * 2 * 64 * 2 * 2 == 34304
    assert total - kv == 2 * 22 * 4 * 64 * 2 == 22528
    assert flops == 4 * 64 * 4 * 617 == 631808


def test_noncausal_and_fp8_work():
    # without the mask every row sees its whole context: 1*7 + 5*20 + 16*40 pairs
    b = build_batch("nc", [1, 5, 16], [7, 20, 40], 4, 2, 64, False, seed=3)
    assert bench.algorithmic_work(b)[2] == 4 * 64 * 4 * 747
    # fp8 caches: one byte per cached element
    b8 = build_batch("f8", [1, 5, 16], [7, 20, 40], 4, 2, 64, True, seed=3,
                     kv_dtype="fp8_e4m3fn", k_scale=0.5, v_scale=0.5)
    assert bench.algorithmic_work(b8)[1] == 67 * 2 * 64 * 2


def test_rows_without_keys_add_no_work():
    # 5 causal queries over 3 keys: rows see 0, 0, 1, 2, 3 keys
    b = build_batch("e", [5], [3], 2, 1, 8, True, seed=4)
    assert bench.algorithmic_work(b)[2] == 4 * 8 * 2 * 6

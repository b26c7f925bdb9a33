"""GPU parity with cache blocks of 32 and 64 keys (read as 16-key sub-blocks):
every kernel path against the fp64 oracle, and bit-exact invariance under
block permutation and NaN poison of unused slots."""

import numpy as np
import pytest
import torch

import paged_kv_cache_unified_amd as pa
from gpu_util import bits, full_parity, require_gpu, run_pa, say
from workloads import build_batch, repermute_pool

pytestmark = pytest.mark.gpu

DEV = "cuda"

# name: (q_lens, k_lens, hq, hkv, d, causal, options, kv format)
CASES = {
    # persistent decode, one part per row
    "decode": ([1] * 12, [1, 17, 31, 32, 33, 64, 65, 100, 500, 700, 1000, 0], 32, 8, 128, True,
               {}, "bf16"),
    # persistent decode, even split (a long row), two-token rows
    "decode_even": ([1, 2, 1, 2, 1, 1], [9000, 3000, 5, 64, 1200, 0], 16, 2, 64, True, {}, "bf16"),
    # persistent decode, fixed forced parts
    "decode_splits": ([1, 1, 1, 1], [700, 2100, 64, 31], 32, 8, 128, True,
                      dict(force_num_splits=3), "bf16"),
    # the one-work-group-per-item narrow path
    "narrow_grid": ([1, 2, 1, 4, 1], [700, 33, 1, 2000, 64], 32, 8, 128, True,
                    dict(force_tile=3), "bf16"),
    # wide tiles (prefill chunks) next to decode rows, causal and not
    "mixed": ([300, 1, 40, 1, 129], [900, 77, 40, 1500, 200], 32, 4, 128, True, {}, "bf16"),
    "mixed_noncausal": ([64, 1, 17], [300, 100, 1000], 8, 8, 64, False, {}, "bf16"),
    "wide_splits": ([200, 33], [2500, 90], 32, 8, 128, True, dict(force_num_splits=3), "bf16"),
    # every sequence one wide tile: streaming K/V loads
    "one_tile_wide": ([5, 32, 17, 1, 32], [40, 3000, 17, 900, 32], 32, 8, 128, True, {}, "bf16"),
    # fp8 caches
    "decode_fp8": ([1] * 6, [40, 300, 1000, 65, 4000, 1], 32, 8, 128, True, {}, "fp8_e4m3fn"),
    "mixed_fp8": ([100, 1, 1], [700, 64, 2000], 32, 8, 128, True, {}, "fp8_e4m3fn"),
}


@pytest.mark.parametrize("block", [32, 64])
@pytest.mark.parametrize("case", sorted(CASES))
def test_block_size_parity(case, block):
    require_gpu()
    q_lens, k_lens, hq, hkv, d, causal, opt, kv = CASES[case]
    b = build_batch(f"bs{block}_{case}", q_lens, k_lens, hq, hkv, d, causal,
                    seed=300 + block + len(case), device=DEV, block_size=block, kv_dtype=kv,
                    **(dict(k_scale=1 / 32, v_scale=1 / 16) if kv != "bf16" else {}))
    opts = pa.options(**opt) if opt else None
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    say(f"block={block} {case} plan persistent={plan['persistent']} balanced={plan['balanced']} "
        f"splits={plan['num_splits']}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"block={block} {case}")


@pytest.mark.parametrize("block", [32, 64])
def test_block_size_permutation_and_poison_bit_exact(block):
    require_gpu()
    q_lens, k_lens = [1, 5, 16, 3, 100, 1], [7, 20, 40, 300, 250, 3000]
    b = build_batch("bsperm", q_lens, k_lens, 32, 8, 128, True, seed=90 + block, device=DEV,
                    block_size=block)
    b2 = repermute_pool(b, seed=91 + block)
    clean = build_batch("bsperm", q_lens, k_lens, 32, 8, 128, True, seed=90 + block, device=DEV,
                        block_size=block, poison=False)
    clean.k_cache = torch.where(torch.isnan(b.k_cache), torch.zeros_like(b.k_cache), b.k_cache)
    clean.v_cache = torch.where(torch.isnan(b.v_cache), torch.zeros_like(b.v_cache), b.v_cache)
    say(f"block={block} permutation and poison")
    o1, o2, o3 = run_pa(b), run_pa(b2), run_pa(clean)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(bits(o1), bits(o2))
    assert torch.equal(bits(o1), bits(o3))
    full_parity(b, o1, f"block={block} perm")

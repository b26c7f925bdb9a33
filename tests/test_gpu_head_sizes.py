"""GPU parity at head sizes 96 and 256: the decode, narrow and wide paths
(d = 96 wide tiles in the d = 128 LDS layout with zero padding; d = 256 with
the output accumulators in AGPRs), with forced splits, fp8 and fp16 caches,
and the merges."""

import pytest
import torch

import paged_kv_cache_unified_amd as pa
from gpu_util import bits, full_parity, require_gpu, run_pa, say
from workloads import build_batch, repermute_pool

pytestmark = pytest.mark.gpu

DEV = "cuda"

# name: (q_lens, k_lens, hq, hkv, causal, options, kv format)
CASES = {
    "decode": ([1] * 9, [1, 17, 64, 65, 300, 700, 1500, 2, 0], 32, 8, True, {}, "bf16"),
    "decode_even": ([1, 2, 1, 1], [9000, 3000, 64, 0], 16, 2, True, {}, "bf16"),
    "decode_splits": ([1, 1, 2], [700, 2100, 31], 32, 4, True, dict(force_num_splits=3), "bf16"),
    "narrow_grid": ([1, 2, 1, 4, 1], [700, 33, 1, 2000, 64], 32, 8, True, dict(force_tile=3), "bf16"),
    "prefill_mixed": ([100, 1, 40, 1, 17], [900, 77, 40, 1500, 200], 32, 4, True, {}, "bf16"),
    "prefill_noncausal": ([33, 1, 17], [300, 100, 1000], 8, 8, False, {}, "bf16"),
    "prefill_splits": ([64, 9], [2500, 90], 16, 4, True, dict(force_num_splits=3), "bf16"),
    "fp8_decode": ([1] * 5, [40, 300, 1000, 65, 4000], 32, 8, True, {}, "fp8_e4m3fn"),
    "f16_mixed": ([50, 1, 1], [700, 64, 2000], 32, 8, True, {}, "f16"),
    "fp8_prefill": ([70, 1, 33], [600, 50, 2000], 32, 8, True, {}, "fp8_e4m3fn"),
    "wide_forced": ([1, 3, 1, 16], [500, 40, 1200, 16], 32, 8, True, dict(force_tile=2), "bf16"),
}


@pytest.mark.parametrize("d", [96, 256])
@pytest.mark.parametrize("case", sorted(CASES))
def test_head_size_parity(case, d):
    require_gpu()
    q_lens, k_lens, hq, hkv, causal, opt, kv = CASES[case]
    extra = dict(k_scale=1 / 32, v_scale=1 / 16) if kv == "fp8_e4m3fn" else {}
    b = build_batch(f"d{d}_{case}", q_lens, k_lens, hq, hkv, d, causal, seed=700 + d + len(case),
                    device=DEV, kv_dtype=kv, **extra)
    opts = pa.options(**opt) if opt else None
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    say(f"d={d} {case} plan persistent={plan['persistent']} tile_rows={plan['tile_rows']} "
        f"splits={plan['num_splits']}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"d={d} {case}")


@pytest.mark.parametrize("d", [96, 256])
def test_head_size_permutation_bit_exact(d):
    require_gpu()
    b = build_batch(f"d{d}perm", [1, 5, 16, 3, 40], [7, 20, 40, 300, 250], 16, 4, d, True,
                    seed=720 + d, device=DEV)
    b2 = repermute_pool(b, seed=721 + d)
    say(f"d={d} permutation")
    o1, o2 = run_pa(b), run_pa(b2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(bits(o1), bits(o2))

"""GPU parity with IEEE fp16 q / out / caches (the fp16 MFMAs on every kernel
path), fp16 q next to an fp8 cache, bit-exact invariance under block
permutation, and the cache write of fp16 tokens (copy, and E4M3 codes)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_unified_amd as pa
from gpu_util import bits, full_parity, require_gpu, run_pa, say
from workloads import build_batch, repermute_pool

pytestmark = pytest.mark.gpu

DEV = "cuda"

# name: (q_lens, k_lens, hq, hkv, d, causal, options, kv format)
CASES = {
    "decode": ([1] * 10, [1, 17, 64, 65, 300, 700, 1000, 1500, 2, 0], 32, 8, 128, True, {}, "f16"),
    "decode_even_d64": ([1, 2, 1, 1], [9000, 3000, 64, 0], 16, 2, 64, True, {}, "f16"),
    "decode_splits": ([1, 1, 2], [700, 2100, 31], 32, 4, 128, True, dict(force_num_splits=3), "f16"),
    "narrow_grid": ([1, 2, 1, 4, 1], [700, 33, 1, 2000, 64], 32, 8, 128, True,
                    dict(force_tile=3), "f16"),
    "mixed": ([300, 1, 40, 1, 129], [900, 77, 40, 1500, 200], 32, 4, 128, True, {}, "f16"),
    "mixed_noncausal_d64": ([64, 1, 17], [300, 100, 1000], 8, 8, 64, False, {}, "f16"),
    "wide_splits": ([200, 33], [2500, 90], 32, 8, 128, True, dict(force_num_splits=3), "f16"),
    "one_tile_wide": ([5, 32, 17, 1, 32], [40, 3000, 17, 900, 32], 32, 8, 128, False, {}, "f16"),
    "fp8_cache_decode": ([1] * 6, [40, 300, 1000, 65, 4000, 1], 32, 8, 128, True, {}, "fp8_e4m3fn"),
    "fp8_cache_mixed": ([100, 1, 1], [700, 64, 2000], 32, 8, 128, True, {}, "fp8_e4m3fn"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp16_parity(case):
    require_gpu()
    q_lens, k_lens, hq, hkv, d, causal, opt, kv = CASES[case]
    extra = dict(k_scale=1 / 32, v_scale=1 / 16) if kv == "fp8_e4m3fn" else {}
    b = build_batch(f"f16_{case}", q_lens, k_lens, hq, hkv, d, causal, seed=600 + len(case),
                    device=DEV, kv_dtype=kv, q_dtype="f16", **extra)
    assert b.q.dtype == torch.float16
    opts = pa.options(**opt) if opt else None
    say(f"fp16 {case}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    full_parity(b, out, f"fp16 {case}")


def test_fp16_permutation_bit_exact():
    require_gpu()
    q_lens, k_lens = [1, 5, 16, 3, 100, 1], [7, 20, 40, 300, 250, 3000]
    b = build_batch("f16perm", q_lens, k_lens, 32, 8, 128, True, seed=610, device=DEV,
                    kv_dtype="f16")
    b2 = repermute_pool(b, seed=611)
    say("fp16 permutation")
    o1, o2 = run_pa(b), run_pa(b2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(bits(o1), bits(o2))


@pytest.mark.parametrize("fmt", ["f16", "fp8_e4m3fn"])
def test_fp16_cache_write_bit_exact(fmt):
    require_gpu()
    g = torch.Generator(device="cpu").manual_seed(613)
    NB, B, hkv, d, N = 20, 32, 4, 128, 200
    key = (torch.randn(N, hkv, d, generator=g) * 3).to(torch.float16)
    value = (torch.randn(N, hkv, d, generator=g) * 3).to(torch.float16)
    slots = torch.randperm(NB * B, generator=g)[:N].to(torch.int32)
    slots[::5] = -1
    ks, vs = 0.0625, 0.25
    if fmt == "f16":
        kc = torch.randn(NB, B, hkv, d, generator=g).to(torch.float16)
        vc = torch.randn(NB, B, hkv, d, generator=g).to(torch.float16)
        host = lambda t: t.float().numpy()
    else:
        kc = torch.randint(0, 256, (NB, B, hkv, d), generator=g, dtype=torch.uint8).view(torch.float8_e4m3fn)
        vc = torch.randint(0, 256, (NB, B, hkv, d), generator=g, dtype=torch.uint8).view(torch.float8_e4m3fn)
        host = lambda t: t.view(torch.uint8).numpy()
    ek, ev = oracle.cache_write(key.float().numpy(), value.float().numpy(), host(kc), host(vc),
                                slots.numpy(), kv_format=fmt, k_scale=ks, v_scale=vs)
    dk, dv = kc.to(DEV), vc.to(DEV)
    say(f"fp16 cache write -> {fmt}")
    pa.cache_write(key.to(DEV), value.to(DEV), dk, dv, slots.to(DEV), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    if fmt == "f16":
        gk, gv = dk.cpu().view(torch.int16).numpy(), dv.cpu().view(torch.int16).numpy()
        ek = torch.from_numpy(ek).to(torch.float16).view(torch.int16).numpy()
        ev = torch.from_numpy(ev).to(torch.float16).view(torch.int16).numpy()
    else:
        gk, gv = host(dk.cpu()), host(dv.cpu())
    assert (gk == ek).all() and (gv == ev).all()

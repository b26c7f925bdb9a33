"""GPU: pa_cache_write against the oracle's write, bit for bit (bf16 copies
and fp8 E4M3 codes, including rounding ties, saturation, subnormals, NaN and
signed zero), with skipped (negative) slots and untouched slots kept."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_unified_amd as pa
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def special_values(n, scale):
    """bf16 values whose quotient by `scale` hits E4M3 ties, the saturation
    edge, subnormals and specials (scale is a power of two, so x / scale is
    exact)."""
    grid = oracle.decode_e4m3fn(np.arange(127))
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([mids, -mids, grid, [448.0, 460.0, 464.0, 470.0, 1e4, -1e4,
                                                0.0, -0.0, np.nan, -np.nan]])
    x = torch.tensor(vals * scale, dtype=torch.float32).to(torch.bfloat16)
    reps = -(-n // x.numel())
    return x.repeat(reps)[:n]


@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("shape", [(8, 128, 16), (2, 64, 16), (8, 128, 32), (2, 64, 64)],
                         ids=["hkv8d128", "hkv2d64", "hkv8d128b32", "hkv2d64b64"])
def test_cache_write_bit_exact(fmt, shape):
    require_gpu()
    hkv, d, bs = shape
    g = torch.Generator(device="cpu").manual_seed(hkv * 1000 + d + bs)
    NB, N = 640 // bs, 300
    key = torch.randn(N, hkv, d, generator=g).to(torch.bfloat16)
    value = torch.randn(N, hkv, d, generator=g).to(torch.bfloat16)
    ks, vs = 0.125, 0.5
    if fmt == "fp8_e4m3fn":
        key.view(-1)[: 4000] = special_values(4000, ks)
        value.view(-1)[: 4000] = special_values(4000, vs)
    perm = torch.randperm(NB * bs, generator=g)[:N].to(torch.int32)
    perm[::7] = -1                                            # skipped tokens
    if fmt == "bf16":
        kc = torch.randn(NB, bs, hkv, d, generator=g).to(torch.bfloat16)
        vc = torch.randn(NB, bs, hkv, d, generator=g).to(torch.bfloat16)
        host = lambda t: t.float().numpy()
    else:
        kc = torch.randint(0, 256, (NB, bs, hkv, d), generator=g, dtype=torch.uint8).view(torch.float8_e4m3fn)
        vc = torch.randint(0, 256, (NB, bs, hkv, d), generator=g, dtype=torch.uint8).view(torch.float8_e4m3fn)
        host = lambda t: t.view(torch.uint8).numpy()
    ek, ev = oracle.cache_write(key.float().numpy(), value.float().numpy(), host(kc), host(vc),
                                perm.numpy(), kv_format=fmt, k_scale=ks, v_scale=vs)
    dk, dv = kc.to(DEV), vc.to(DEV)
    say(f"cache write {fmt} hkv={hkv} d={d} block={bs}")
    pa.cache_write(key.to(DEV), value.to(DEV), dk, dv, perm.to(DEV), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    gk, gv = host(dk.cpu()), host(dv.cpu())
    if fmt == "bf16":
        # bit patterns (NaN-safe)
        gk, gv = dk.cpu().view(torch.int16).numpy(), dv.cpu().view(torch.int16).numpy()
        ek = torch.from_numpy(ek).to(torch.bfloat16).view(torch.int16).numpy()
        ev = torch.from_numpy(ev).to(torch.bfloat16).view(torch.int16).numpy()
    bad_k = np.argwhere(gk != ek)
    bad_v = np.argwhere(gv != ev)
    assert bad_k.size == 0, f"{len(bad_k)} key elements differ, first {bad_k[0].tolist()}"
    assert bad_v.size == 0, f"{len(bad_v)} value elements differ, first {bad_v[0].tolist()}"


@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3fn"])
def test_cache_write_skips_slots_outside_the_cache(fmt):
    """Slots at or past NB * B are skipped like negative ones: the cache gets
    exactly the in-range tokens and the memory right after it (a guard region
    of the same allocation, where such a slot would land) is untouched."""
    require_gpu()
    hkv, d, bs, NB, guard, N = 4, 128, 16, 24, 8, 96
    g = torch.Generator(device="cpu").manual_seed(4242)
    key = torch.randn(N, hkv, d, generator=g).to(torch.bfloat16)
    value = torch.randn(N, hkv, d, generator=g).to(torch.bfloat16)
    slots = torch.randperm(NB * bs, generator=g)[:N].to(torch.int32)
    # every 5th token aims just past the cache, into the guard blocks
    slots[::5] = NB * bs + torch.randint(0, guard * bs, (len(slots[::5]),), generator=g,
                                         dtype=torch.int32)
    in_range = torch.where(slots < NB * bs, slots, torch.full_like(slots, -1))
    if fmt == "bf16":
        big_k = torch.randn(NB + guard, bs, hkv, d, generator=g).to(torch.bfloat16)
        big_v = torch.randn(NB + guard, bs, hkv, d, generator=g).to(torch.bfloat16)
        host = lambda t: t.float().numpy()
    else:
        big_k = torch.randint(0, 256, (NB + guard, bs, hkv, d), generator=g,
                              dtype=torch.uint8).view(torch.float8_e4m3fn)
        big_v = torch.randint(0, 256, (NB + guard, bs, hkv, d), generator=g,
                              dtype=torch.uint8).view(torch.float8_e4m3fn)
        host = lambda t: t.view(torch.uint8).numpy()
    ek, ev = oracle.cache_write(key.float().numpy(), value.float().numpy(), host(big_k[:NB]),
                                host(big_v[:NB]), in_range.numpy(), kv_format=fmt,
                                k_scale=0.25, v_scale=0.5)
    dk, dv = big_k.to(DEV), big_v.to(DEV)
    say(f"cache write {fmt}: slots outside the cache")
    pa.cache_write(key.to(DEV), value.to(DEV), dk[:NB], dv[:NB], slots.to(DEV), k_scale=0.25,
                   v_scale=0.5)
    torch.cuda.synchronize()
    raw = lambda t: t.view(torch.uint8) if fmt != "bf16" else t.view(torch.int16)
    assert torch.equal(raw(dk[NB:].cpu()), raw(big_k[NB:])), "guard region after k_cache written"
    assert torch.equal(raw(dv[NB:].cpu()), raw(big_v[NB:])), "guard region after v_cache written"
    gk, gv = host(dk[:NB].cpu()), host(dv[:NB].cpu())
    np.testing.assert_array_equal(gk.view(np.uint8) if fmt != "bf16" else gk, ek)
    np.testing.assert_array_equal(gv.view(np.uint8) if fmt != "bf16" else gv, ev)

"""Seeded random batches crossing every option of the call, against the oracle.

The other GPU tests sweep one dimension at a time.  Here each case draws all
of them at once: sequence count, query lengths (0, 1, short, several tiles,
ragged tails, more queries than keys), contexts, head counts, head size
(64/96/128/256), block size (16/32/64), element type (bf16/fp16), cache
format (16-bit or fp8 E4M3 with scales), causal mode, and the launch options
(forced key splits, forced tile kinds where the batch allows them).  Sizes
keep the fp64 oracle at about a second per case.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_unified_amd as pa
from gpu_util import full_parity, require_gpu, run_pa, say
from workloads import build_batch

pytestmark = pytest.mark.gpu

DEV = "cuda"
HEADS = [(4, 2), (8, 8), (16, 1), (32, 8), (32, 4), (8, 1)]
QLENS = [0, 1, 1, 2, 5, 16, 17, 33, 64, 130]


def _draw(seed):
    rng = np.random.default_rng(seed)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 96, 128, 256]))
    B = int(rng.choice([16, 32, 64]))
    causal = bool(rng.random() < 0.7)
    decode = rng.random() < 0.35
    S = int(rng.integers(1, 24))
    if decode:
        q = rng.choice([0, 1, 1, 1, 2], size=S) if hq // hkv <= 8 else np.ones(S, int)
    else:
        q = rng.choice(QLENS, size=S)
    k = rng.integers(0, 1200, size=S)
    k = np.where(rng.random(S) < 0.2, np.maximum(k // 8, 0), k)      # some very short contexts
    k = np.where(q > k, np.where(rng.random(S) < 0.3, k, q), k)      # a few with q > context
    # keep the oracle quick: query rows x keys x heads x d
    while int((q * np.maximum(k, 1)).sum()) * hq * d > 6e8:
        k = k // 2
    elem = "f16" if rng.random() < 0.3 else "bf16"
    fp8 = rng.random() < 0.3
    kw = dict(block_size=B)
    if fp8:
        kw.update(kv_dtype="fp8_e4m3fn", k_scale=float(rng.choice([1 / 64, 0.5, 1.0])),
                  v_scale=float(rng.choice([1 / 64, 0.25, 1.0])), q_dtype=elem)
    else:
        kw.update(kv_dtype=elem)
    G = hq // hkv
    narrow_fits = int(q.max()) * G <= 16
    choices = [{}, {}, {"force_num_splits": int(rng.choice([2, 3, 7]))}, {"force_tile": 2}]
    if narrow_fits:
        choices += [{"force_tile": 1}, {"force_tile": 3}]
    if d in (64, 128) and not fp8:
        choices += [{"force_tile": 4}]
    opt = choices[int(rng.integers(len(choices)))]
    return dict(q=q, k=k, hq=hq, hkv=hkv, d=d, causal=causal, kw=kw, opt=opt, fp8=fp8)


@pytest.mark.parametrize("seed", range(32))
def test_random_mixed_options(seed):
    require_gpu()
    c = _draw(5000 + seed)
    b = build_batch(f"mix{seed}", c["q"], c["k"], c["hq"], c["hkv"], c["d"], c["causal"],
                    seed=7000 + seed, device=DEV, **c["kw"])
    opts = pa.options(**c["opt"]) if c["opt"] or c["fp8"] else None
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    say(f"mix{seed}: S={len(b.q_lens)} T={b.q.shape[0]} hq={c['hq']} hkv={c['hkv']} d={c['d']} "
        f"B={c['kw']['block_size']} {c['kw']['kv_dtype']} q={b.q.dtype} causal={c['causal']} "
        f"opt={c['opt']} plan: persistent={plan['persistent']} balanced={plan['balanced']} "
        f"tile_rows={plan['tile_rows']} splits={plan['num_splits']}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"mix{seed}")

"""CPU models of the kernels' work division (tests/kernel_models.py), run over
seeded random batches with the plans the library's host planner picks: every
(sequence, kv-head) gets each key sub-block exactly once and each part index
exactly once, no kernel reads a block-table column past ceil(L / B), every
ring load (refills of the next item included) targets an owned sub-block,
every split partial lands inside the workspace the host sized, and even-split
stream positions stay in int32 — also when seqused_k exceeds max_seqlen_k.
No GPU: planning reads descriptors only."""

import ctypes

import numpy as np
import pytest

import paged_kv_cache_unified_amd as pa
from kernel_models import Batch, cdiv, check_trace, decode_kernel, fwd_kernel


def _desc(addr, dtype, shape):
    shape = list(shape)
    strides = [int(np.prod(shape[i + 1:])) for i in range(len(shape))]
    t = pa.PaTensor()
    t.data = addr
    t.dtype = dtype
    t.ndim = len(shape)
    for i, (n, st) in enumerate(zip(shape, strides)):
        t.shape[i] = n
        t.stride[i] = st
    return t


def plan_of(b: Batch, num_blocks: int, opts=None, num_cus=256):
    """pa_plan_describe on descriptors of fake (never dereferenced) pointers."""
    mb = max(1, cdiv(max([b.max_k] + [0]), b.block_size))
    ds = [_desc(1 << 40, pa.PA_BF16, (b.T, b.num_q_heads, b.head_dim)),
          _desc(2 << 40, pa.PA_BF16, (num_blocks, b.block_size, b.num_kv_heads, b.head_dim)),
          _desc(3 << 40, pa.PA_BF16, (num_blocks, b.block_size, b.num_kv_heads, b.head_dim)),
          _desc(4 << 40, pa.PA_BF16, (b.T, b.num_q_heads, b.head_dim)),
          _desc(5 << 40, pa.PA_INT32, (b.S + 1,)),
          _desc(6 << 40, pa.PA_INT32, (b.S,)),
          _desc(7 << 40, pa.PA_INT32, (b.S, mb))]
    info = pa.PaPlanInfo()
    rc = pa.lib.pa_plan_describe(*[ctypes.byref(d) for d in ds], int(max(b.q_lens + [0])),
                                 int(b.max_k), ctypes.byref(opts) if opts is not None else None,
                                 num_cus, ctypes.byref(info))
    assert rc == 0, pa.lib.pa_last_error().decode()
    return info.as_dict()


def random_batch(rng, decode: bool, B: int):
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    d = int(rng.choice([64, 96, 128, 256]))
    S = int(rng.choice([1, 3, 17, 64, 255, 600] if decode else [1, 3, 17, 64]))
    kind = rng.integers(4) if S <= 64 else int(rng.choice([0, 1, 3]))
    if kind == 0:
        k = rng.integers(1000, 1101, S)
    elif kind == 1:
        k = np.clip(np.round(np.exp(rng.normal(np.log(400), 1.0, S))), 4, 8192)
    elif kind == 2:
        k = rng.integers(0, 40000, S)
    else:
        k = rng.integers(0, 300, S)
    k = k.astype(int)
    if decode:
        qmax = max(1, 16 // g)
        q = rng.integers(0, qmax + 1, S) if rng.random() < 0.3 else np.ones(S, int)
    else:
        q = rng.choice([0, 1, 1, 5, 16, 33, 200, 512], S)
        k = np.minimum(k, 6000)
    q = q.astype(int)
    max_k = int(k.max()) if S else 0
    if rng.random() < 0.25 and max_k > 64:           # seqused_k above max_seqlen_k
        max_k = int(max_k * rng.uniform(0.3, 0.9))
    b = Batch(list(q), list(k), hkv * g, hkv, d, B, max_k, causal=bool(rng.random() < 0.8))
    nblocks = max(1, int(np.sum([cdiv(min(x, max_k), 16) for x in k])) + 1)
    return b, nblocks


@pytest.mark.parametrize("B", [16, 32, 64])
def test_decode_kernel_work_model(B):
    rng = np.random.default_rng(7000 + B)
    kinds = {"even": 0, "fixed": 0}
    for trial in range(36):
        b, nb = random_batch(rng, decode=True, B=B)
        opts = None
        if trial % 5 == 4:
            opts = pa.options(force_num_splits=int(rng.choice([2, 3, 7, 1000])))
        elif trial % 7 == 3:
            opts = pa.options(decode_grid=int(rng.choice([8, 16, 384])))
        plan = plan_of(b, nb, opts)
        if not plan["persistent"]:
            continue
        kinds["even" if plan["balanced"] else "fixed"] += 1
        tr = decode_kernel(b, plan)
        check_trace(b, plan, tr)
    assert kinds["even"] >= 5 and kinds["fixed"] >= 5, kinds


@pytest.mark.parametrize("B", [16, 32, 64])
def test_grid_kernel_work_model(B):
    rng = np.random.default_rng(8000 + B)
    lpt = unit_xcd = 0
    for trial in range(24):
        b, nb = random_batch(rng, decode=trial % 4 == 0, B=B)
        opts = None
        if trial % 3 == 1:
            opts = pa.options(force_num_splits=int(rng.choice([2, 3, 7, 1000])))
        if trial % 4 == 0:
            if max(b.q_lens) * b.G > 16:
                continue
            opts = pa.options(force_tile=3)
        plan = plan_of(b, nb, opts)
        if plan["persistent"]:                # a batch of short queries: the decode kernel
            check_trace(b, plan, decode_kernel(b, plan))
            continue
        lpt += plan["longest_first"]
        unit_xcd += plan["unit_xcd"]
        tr = fwd_kernel(b, plan)
        check_trace(b, plan, tr)
    assert lpt >= 5 and unit_xcd >= 1, (lpt, unit_xcd)


def test_even_split_with_overstated_context_stays_in_the_workspace():
    """seqused_k far above max_seqlen_k on the even split: the device reads
    the clamped length, so part counts stay within the plan's bound."""
    b = Batch([1] * 12, [50000, 40, 3000, 70000, 2047, 90000, 80, 6000, 300, 16, 1200, 4000],
              32, 8, 128, 16, max_k=4096)
    plan = plan_of(b, 2000)
    assert plan["persistent"] and plan["balanced"]
    check_trace(b, plan, decode_kernel(b, plan))


def test_models_catch_a_planted_bound_error():
    """The checks are not vacuous: a workspace bound one part below the most
    parts any row has is reported as an overflow, and a block-table narrower
    than the contexts as a read past the table."""
    b = Batch([1] * 8, [3000, 5000, 100, 9000, 20, 7000, 64, 4000], 32, 8, 128, 16, max_k=9000)
    plan = plan_of(b, 3000)
    assert plan["balanced"]
    tr = decode_kernel(b, plan)
    check_trace(b, plan, tr)
    most = max(it.parts for it in tr.items)
    assert most > 1
    with pytest.raises(AssertionError):
        check_trace(b, dict(plan, num_splits=most - 1), tr)
    with pytest.raises(AssertionError):
        check_trace(b, dict(plan, partial_rows=max(tr.ws_rows)), tr)
    shorter = Batch(b.q_lens, [min(x, 4000) for x in b.k_lens], 32, 8, 128, 16, max_k=9000)
    with pytest.raises(AssertionError):
        check_trace(shorter, plan, tr)

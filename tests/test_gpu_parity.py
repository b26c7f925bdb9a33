"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Shapes sweep head counts, head_dim, causal mode, query lengths (0, 1, short,
several tiles, ragged tails) and contexts in one process, so a kernel
specialisation keyed on the wrong constants shows up.
"""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_unified_amd as pa
from gpu_util import bits, check_close, full_parity, require_gpu, run_pa, say
from workloads import build_batch, make_workload, repermute_pool

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_tiny_workload():
    require_gpu()
    b = make_workload("tiny_mixed_3seq", device=DEV)
    say("tiny_mixed_3seq")
    out = run_pa(b)
    torch.cuda.synchronize()
    err, frob = full_parity(b, out, "tiny_mixed_3seq")
    say(f"  max err {err:.2e} frob {frob:.2e}")


SWEEP_HEADS = [(4, 2), (32, 8), (32, 4), (8, 8), (16, 1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", SWEEP_HEADS, ids=lambda h: f"hq{h[0]}_hkv{h[1]}")
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_random_sweep(d, heads, causal):
    require_gpu()
    hq, hkv = heads
    rng = np.random.default_rng(1000 + 7 * d + hq + 3 * hkv + int(causal))
    q_lens = np.array([0, 1, 2, 5, 16, 17, 33, 1, 64, 65, 3, 1])
    # contexts from q_len up to ~600, a few with q_len > ctx for the causal case
    k_lens = np.array([max(int(x), int(ql)) for x, ql in
                       zip(rng.integers(1, 600, size=len(q_lens)), q_lens)])
    k_lens[1] = 1
    if causal:
        k_lens[3] = 3          # 5 queries over 3 keys: first two rows have no key
    b = build_batch("sweep", q_lens, k_lens, hq, hkv, d, causal, seed=int(rng.integers(1 << 30)),
                    device=DEV)
    say(f"sweep d={d} hq={hq} hkv={hkv} causal={causal}")
    out = run_pa(b)
    torch.cuda.synchronize()
    full_parity(b, out, f"sweep d{d} {heads} causal={causal}")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
def test_forced_splits(splits):
    require_gpu()
    b = build_batch("split", [1, 1, 4, 17, 1, 40], [700, 129, 300, 1000, 64, 40], 32, 8, 128,
                    True, seed=77, device=DEV)
    say(f"forced splits {splits}")
    out = run_pa(b, opts=pa.options(force_num_splits=splits))
    torch.cuda.synchronize()
    full_parity(b, out, f"splits={splits}")


@pytest.mark.parametrize("tile", [1, 2])
def test_forced_tiles_on_decode(tile):
    require_gpu()
    b = build_batch("tiles", [1, 2, 1, 3], [300, 17, 1, 64], 16, 4, 128, True, seed=78,
                    device=DEV)
    say(f"forced tile {tile}")
    out = run_pa(b, opts=pa.options(force_tile=tile))
    torch.cuda.synchronize()
    full_parity(b, out, f"tile={tile}")


def test_block_permutation_bit_exact():
    require_gpu()
    b = build_batch("perm", [1, 5, 16, 3, 100], [7, 20, 40, 300, 250], 32, 8, 128, True,
                    seed=79, device=DEV)
    b2 = repermute_pool(b, seed=80)
    say("block permutation")
    o1 = run_pa(b)
    o2 = run_pa(b2)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o2))
    full_parity(b, o1, "perm")


def test_nan_poison_bit_exact():
    require_gpu()
    b = build_batch("poison", [1, 5, 16, 3, 1], [7, 20, 40, 300, 33], 8, 2, 64, True,
                    seed=81, device=DEV)
    clean = build_batch("poison", [1, 5, 16, 3, 1], [7, 20, 40, 300, 33], 8, 2, 64, True,
                        seed=81, device=DEV, poison=False)
    # same values where owned; zero everywhere else
    nan_mask = torch.isnan(b.k_cache)
    clean.k_cache = torch.where(nan_mask, torch.zeros_like(b.k_cache), b.k_cache)
    clean.v_cache = torch.where(torch.isnan(b.v_cache), torch.zeros_like(b.v_cache), b.v_cache)
    say("nan poison")
    o1 = run_pa(b)
    o2 = run_pa(clean)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(bits(o1), bits(o2))


def test_single_key_is_exact():
    require_gpu()
    for causal in (True, False):
        b = build_batch("one", [1, 1, 7], [1, 1, 7], 8, 2, 128, causal, seed=82, device=DEV)
        say(f"single key causal={causal}")
        out = run_pa(b)
        torch.cuda.synchronize()
        for s in range(2):
            v0 = b.v_cache[b.block_table[s, 0], 0]                 # [Hkv, d]
            assert torch.equal(bits(out[s]), bits(v0.repeat_interleave(4, dim=0)))
        if causal:   # row 0 of a fresh causal prefill sees key 0 only
            v0 = b.v_cache[b.block_table[2, 0], 0]
            assert torch.equal(bits(out[2]), bits(v0.repeat_interleave(4, dim=0)))


def test_deterministic_runs():
    require_gpu()
    b = build_batch("det", [1, 33, 1, 200], [2000, 500, 900, 1000], 32, 8, 128, True,
                    seed=83, device=DEV)
    say("determinism")
    outs = [run_pa(b) for _ in range(3)]
    outs.append(run_pa(b, opts=pa.options(force_num_splits=5)))
    outs.append(run_pa(b, opts=pa.options(force_num_splits=5)))
    torch.cuda.synchronize()
    assert torch.equal(bits(outs[0]), bits(outs[1])) and torch.equal(bits(outs[0]), bits(outs[2]))
    assert torch.equal(bits(outs[3]), bits(outs[4]))


def test_empty_rows_are_zero():
    require_gpu()
    b = build_batch("empty", [2, 0, 3, 1, 4], [0, 5, 2, 4, 0], 8, 2, 64, True, seed=84,
                    device=DEV)
    say("empty rows")
    out = run_pa(b)
    torch.cuda.synchronize()
    assert torch.all(out[0:2] == 0) and torch.all(out[2] == 0)
    assert torch.all(out[6:10] == 0)
    full_parity(b, out, "empty rows")


def test_shared_prefix_blocks():
    """Block ids repeated across sequences (a shared, cached prefix)."""
    require_gpu()
    b = build_batch("share", [1, 3, 1], [100, 120, 64], 32, 8, 128, True, seed=85, device=DEV)
    t = b.block_table.clone()
    t[1, :4] = t[0, :4]     # sequence 1 reuses sequence 0's first 64 keys
    t[2, :4] = t[0, :4]
    b.block_table = t
    say("shared prefix")
    out = run_pa(b)
    torch.cuda.synchronize()
    full_parity(b, out, "shared prefix")


def test_strided_views_and_side_stream():
    """q/out as head-slices of wider buffers; launch on a non-default stream."""
    require_gpu()
    b = build_batch("strided", [1, 17, 4], [50, 80, 300], 8, 2, 128, True, seed=86, device=DEV)
    wide = torch.zeros(b.total_q, 12, 128, dtype=torch.bfloat16, device=DEV)
    wide[:, 2:10] = b.q
    b.q = wide[:, 2:10]
    out_wide = torch.full((b.total_q, 10, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = out_wide[:, 1:9]
    s = torch.cuda.Stream()
    say("strided + side stream")
    run_pa(b, out=out, stream=s)
    s.synchronize()
    full_parity(b, out, "strided")
    assert torch.isnan(out_wide[:, 0].float()).all() and torch.isnan(out_wide[:, 9].float()).all()


def test_check_contents_rejects_bad_metadata():
    require_gpu()
    b = build_batch("bad", [1, 2], [20, 40], 8, 2, 64, True, seed=87, device=DEV)
    t = b.block_table.clone()
    t[1, 1] = b.num_blocks + 5
    b.block_table = t
    out = torch.zeros_like(b.q)
    with pytest.raises(pa.PaError, match="PA_ERR_CONTENT"):
        pa.unified_attention(*b.args(out), opts=pa.options(check_contents=True))


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 1000])
@pytest.mark.parametrize("shape", [(32, 8, 128), (16, 2, 64)], ids=["g4d128", "g8d64"])
def test_persistent_decode_ragged(splits, shape):
    """Narrow batches on the persistent decode kernel: ragged contexts (0 to
    5000 keys), several query tokens per sequence, per-sequence split counts."""
    require_gpu()
    hq, hkv, d = shape
    G = hq // hkv
    qmax = 16 // G
    q_lens = [1, 1, 2, qmax, qmax - 1 if qmax > 1 else 1, 1, 1, qmax, 0, 1, 2 if qmax >= 2 else 1, 1]
    k_lens = [1, 17, 300, 1000, 2500, 64, 65, 4, 10, 0, 5000, 129]
    b = build_batch("pers", q_lens, k_lens, hq, hkv, d, True, seed=90 + splits, device=DEV)
    opts = None if splits == 0 else pa.options(force_num_splits=splits)
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    assert plan["persistent"] == 1
    say(f"persistent decode splits={splits} shape={shape} plan={plan['num_splits']}x{plan['split_keys']}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"persistent splits={splits}")


def even_split_lengths(grid):
    """Ragged decode batch for the even split: long and empty rows, a sequence
    without queries, two query tokens (rows with no key under the causal mask)."""
    rng = np.random.default_rng(97 + grid)
    S = 24
    q_lens = rng.integers(1, 3, size=S)
    k_lens = rng.integers(0, 6000, size=S)
    q_lens[3] = 0
    k_lens[5] = 0
    k_lens[7] = 1
    k_lens[0] = 9000
    return q_lens, k_lens


@pytest.mark.gpu
@pytest.mark.parametrize("grid", [8, 64])
def test_even_split_few_waves(grid):
    """Even split on a small decode grid: several chunks per wave, rows cut
    across chunks and waves, rows with no key, a sequence with no query."""
    require_gpu()
    q_lens, k_lens = even_split_lengths(grid)
    b = build_batch("even", q_lens, k_lens, 32, 8, 128, True, seed=97 + grid, device=DEV)
    opts = pa.options(decode_grid=grid)
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    assert plan["persistent"] == 1 and plan["balanced"] == 1
    say(f"even split grid={grid} plan={plan['num_splits']}x{plan['split_keys']}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"even split grid={grid}")


def test_narrow_grid_path():
    """The one-work-group-per-item narrow path (force_tile=3)."""
    require_gpu()
    b = build_batch("grid", [1, 2, 1, 4, 1], [700, 33, 1, 2000, 64], 32, 8, 128, True, seed=95,
                    device=DEV)
    for splits in (0, 3):
        o = pa.options(force_tile=3, force_num_splits=splits)
        plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=o)
        assert plan["persistent"] == 0
        say(f"narrow grid splits={splits}")
        out = run_pa(b, opts=o)
        torch.cuda.synchronize()
        full_parity(b, out, f"narrow grid splits={splits}")


def test_many_sequences_fall_back_to_grid():
    """More sequences than the persistent kernel enumerates (2048)."""
    require_gpu()
    rng = np.random.default_rng(96)
    S = 2100
    b = build_batch("many", np.ones(S, int), rng.integers(1, 40, size=S), 8, 2, 64, True,
                    seed=96, device=DEV)
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9])
    assert plan["persistent"] == 0
    say("2100 sequences")
    out = run_pa(b)
    torch.cuda.synchronize()
    full_parity(b, out, "many sequences")


@pytest.mark.parametrize("S,kind,splits", [(700, "ragged", 0), (1500, "uniform", 0),
                                           (1500, "uniform", 3), (2048, "ragged", 0)],
                         ids=["s700_even", "s1500_fixed", "s1500_fixed_split3", "s2048_fixed"])
def test_persistent_decode_many_sequences(S, kind, splits):
    """The persistent decode kernel up to its 2048 sequences: each thread of a
    work-group owns up to 8 sequences of the per-sequence tables (lengths,
    prefix sums of units and partial slots) that every item lookup searches;
    empty sequences (q = 0) among them."""
    require_gpu()
    rng = np.random.default_rng(S + splits)
    if kind == "ragged":
        k = np.clip(np.round(np.exp(rng.normal(np.log(120.0), 1.0, size=S))), 1, 3000).astype(int)
    else:
        k = rng.integers(150, 200, size=S)
    q = np.ones(S, int)
    q[rng.random(S) < 0.02] = 0
    b = build_batch("many_decode", q, k, 8, 2, 64, True, seed=S + splits, device=DEV)
    opts = pa.options(force_num_splits=splits) if splits else None
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    assert plan["persistent"] == 1 and plan["balanced"] == (1 if kind == "ragged" and S < 2048 else 0)
    say(f"persistent decode S={S} {kind} splits={plan['num_splits']} balanced={plan['balanced']}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"persistent decode S={S} {kind}")


@pytest.mark.parametrize("splits", [0, 3])
def test_longest_first_ragged_units(splits):
    """Wide plans rank (sequence, tile, split) units longest-first on the device:
    ragged prefills, chunks, decode rows, empty sequences and key splits must
    each be computed exactly once (out starts as NaN)."""
    require_gpu()
    rng = np.random.default_rng(97 + splits)
    q_lens = [300, 1, 0, 77, 5, 512, 33, 1, 128, 2]
    k_lens = [max(q, int(x)) for q, x in zip(q_lens, rng.integers(0, 2500, size=len(q_lens)))]
    k_lens[2] = 0
    b = build_batch("lpt", q_lens, k_lens, 32, 8, 128, True, seed=int(rng.integers(1 << 30)),
                    device=DEV)
    opts = None if splits == 0 else pa.options(force_num_splits=splits)
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    assert plan["longest_first"] == 1
    say(f"longest-first splits={splits} plan={plan['num_splits']}x{plan['split_keys']}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"longest-first splits={splits}")


@pytest.mark.parametrize("causal,splits", [(True, 0), (False, 0), (True, 3)],
                         ids=["causal", "noncausal", "causal_splits3"])
def test_one_tile_wide_plans(causal, splits):
    """Every sequence one wide tile (at most 32 tokens at G = 4): the kernel
    variant whose K/V loads stream, since no other tile reads them.  Against
    the oracle (out starts as NaN), and bit-exact under block permutation and
    NaN poison of unowned slots."""
    require_gpu()
    q_lens = [5, 32, 17, 1, 32, 0, 9]
    k_lens = [40, 3000, 17, 900, 32, 10, 1300]
    if not causal:
        k_lens[2] = 300
    b = build_batch("one_tile", q_lens, k_lens, 32, 8, 128, causal, seed=131 + splits, device=DEV)
    opts = None if splits == 0 else pa.options(force_num_splits=splits)
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    assert plan["slots_direct"] == 1 and plan["tile_rows"] == 128 and plan["persistent"] == 0
    assert plan["longest_first"] == 1 and plan["unit_xcd"] == 1
    say(f"one-tile wide causal={causal} splits={plan['num_splits']}")
    b2 = repermute_pool(b, seed=132 + splits)
    clean = build_batch("one_tile", q_lens, k_lens, 32, 8, 128, causal, seed=131 + splits,
                        device=DEV, poison=False)
    clean.k_cache = torch.where(torch.isnan(b.k_cache), torch.zeros_like(b.k_cache), b.k_cache)
    clean.v_cache = torch.where(torch.isnan(b.v_cache), torch.zeros_like(b.v_cache), b.v_cache)
    o1, o2, o3 = run_pa(b, opts=opts), run_pa(b2, opts=opts), run_pa(clean, opts=opts)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(bits(o1), bits(o2))
    assert torch.equal(bits(o1), bits(o3))
    full_parity(b, o1, f"one-tile wide causal={causal} splits={splits}")


def test_many_sequences_with_wide_tiles_keep_index_order():
    """More than 2048 sequences with a wide tile: index-ordered grid."""
    require_gpu()
    rng = np.random.default_rng(98)
    S = 2100
    q_lens = np.ones(S, int)
    q_lens[[0, 700, 2099]] = [40, 17, 64]
    k_lens = np.maximum(q_lens, rng.integers(1, 60, size=S))
    b = build_batch("many_wide", q_lens, k_lens, 8, 2, 64, True, seed=98, device=DEV)
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9])
    assert plan["longest_first"] == 0 and plan["persistent"] == 0
    say("2100 sequences with wide tiles")
    out = run_pa(b)
    torch.cuda.synchronize()
    full_parity(b, out, "many sequences, wide")


# ---------------------------------------------------------------------------
# fp8 E4M3 caches: converted to bf16 after the load, scales folded into the
# score scale (k_scale) and the output (v_scale)
# ---------------------------------------------------------------------------

FP8_CASES = {
    # name: (q_lens, k_lens, Hq, Hkv, d, causal, force_tile, force_splits)
    "decode_persistent_g4d128": ([1, 1, 2, 4, 1, 0, 1], [1, 300, 1000, 2500, 17, 5, 4100],
                                 32, 8, 128, True, 0, 0),
    "decode_persistent_g8d64_split3": ([1, 2, 1, 1], [700, 129, 2000, 33], 16, 2, 64, True, 0, 3),
    "narrow_grid": ([1, 2, 1, 4], [700, 33, 2000, 64], 32, 8, 128, True, 3, 0),
    "wide_prefill_causal": ([300, 1, 77, 5, 128], [900, 60, 77, 400, 1500], 32, 8, 128, True, 0, 0),
    "wide_noncausal_split2": ([16, 40, 3], [3000, 700, 90], 32, 4, 128, False, 0, 2),
    "wide_d64_g2": ([64, 17, 1], [200, 1000, 5], 8, 4, 64, True, 0, 0),
}


@pytest.mark.parametrize("case", sorted(FP8_CASES))
def test_fp8_cache_parity(case):
    require_gpu()
    q_lens, k_lens, hq, hkv, d, causal, tile, splits = FP8_CASES[case]
    b = build_batch("fp8", q_lens, k_lens, hq, hkv, d, causal, seed=200 + len(case), device=DEV,
                    kv_dtype="fp8_e4m3fn", k_scale=0.25, v_scale=0.0625)
    opts = pa.options(force_tile=tile, force_num_splits=splits) if (tile or splits) else None
    say(f"fp8 {case}")
    out = run_pa(b, opts=opts)
    torch.cuda.synchronize()
    full_parity(b, out, f"fp8 {case}")


def test_fp8_permutation_poison_and_scale_bit_exact():
    """Block placement and the NaN codes of unowned slots do not change a bit
    of the output; v_scale = 2 doubles every output exactly."""
    require_gpu()
    args = ([1, 5, 16, 3, 40], [7, 20, 40, 300, 250], 32, 8, 128, True)
    b = build_batch("p8", *args, seed=301, device=DEV, kv_dtype="fp8_e4m3fn", k_scale=0.5,
                    v_scale=0.125)
    clean = build_batch("p8", *args, seed=301, device=DEV, kv_dtype="fp8_e4m3fn", k_scale=0.5,
                        v_scale=0.125, poison=False)
    nan_k = b.k_cache.view(torch.uint8) == 0x7F
    nan_v = b.v_cache.view(torch.uint8) == 0x7F
    clean.k_cache.view(torch.uint8)[nan_k] = 0
    clean.v_cache.view(torch.uint8)[nan_v] = 0
    say("fp8 permutation / poison / v_scale")
    o1 = run_pa(b)
    o2 = run_pa(repermute_pool(b, seed=302))
    o3 = run_pa(clean)
    # same codes, twice the value scale (a batch regenerated with another scale
    # would round to different codes: E4M3's subnormal grid does not scale)
    o4 = run_pa(dataclasses.replace(b, v_scale=0.25))
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(bits(o1), bits(o2))
    assert torch.equal(bits(o1), bits(o3))
    assert torch.equal(o4.float(), 2.0 * o1.float())
    full_parity(b, o1, "fp8 p/p/s")


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_wide_tile_sequence_without_keys(causal):
    """A sequence with queries and no context (L = 0) on a wide tile (40 tokens
    x G = 4 = 160 packed rows): every row is exactly 0; its neighbour is
    checked against the oracle."""
    require_gpu()
    b = build_batch("nokeys", [40, 33, 1], [0, 33, 70], 16, 4, 128, causal, seed=91, device=DEV)
    plan = pa.plan_describe(*b.args(b.new_out())[:9])
    assert plan["tile_rows"] > 16 and plan["persistent"] == 0
    say(f"wide tile without keys causal={causal}")
    out = run_pa(b)
    torch.cuda.synchronize()
    assert torch.equal(bits(out[:40]), torch.zeros_like(bits(out[:40])))
    full_parity(b, out, f"no keys causal={causal}")


@pytest.mark.parametrize("tile", [0, 2, 3], ids=["plan", "wide", "grid_narrow"])
def test_context_longer_than_max_seqlen_k_is_clamped(tile):
    """seqused_k above max_seqlen_k (a broken precondition) is read as
    max_seqlen_k: the result equals the call with the lengths clamped, bit for
    bit, and no split partial lands outside the workspace the plan sized."""
    require_gpu()
    q_lens = [1, 1, 1, 1] if tile in (0, 3) else [1, 20, 3, 40]
    b = build_batch("clamp", q_lens, [900, 2500, 3000, 60], 32, 8, 128, True, seed=92,
                    device=DEV)
    max_k = 2048
    clamped = b.seqused_k.clamp(max=max_k)
    outs = []
    for sk in (b.seqused_k, clamped):
        out = torch.full_like(b.q, float("nan"))
        args = list(b.args(out))
        args[5] = sk
        args[8] = max_k
        opts = pa.options(force_tile=tile)
        n = pa.workspace_bytes(*args[:9], opts)
        ws = torch.full((max(n, 1) + 4096,), 0x7F, dtype=torch.uint8, device=DEV)
        pa.unified_attention(*args, opts=opts, workspace=ws[:max(n, 1)])
        torch.cuda.synchronize()
        assert torch.all(ws[max(n, 1):] == 0x7F), "a partial landed past the workspace"
        outs.append(out)
    say(f"clamp tile={tile}")
    assert torch.equal(bits(outs[0]), bits(outs[1]))
    b.seqused_k = clamped
    b.k_lens = np.minimum(b.k_lens, max_k)
    full_parity(b, outs[1], f"clamped tile={tile}")


def test_library_workspace_grows_under_two_threads():
    """Two host threads on one stream call the plain entry point (library
    workspace) with batches whose split workspaces keep growing; every output
    equals the single-thread result of the same batch bit for bit."""
    import threading
    require_gpu()
    batches = [build_batch(f"grow{i}", [1] * (4 + 4 * i), [3000 + 700 * i] * (4 + 4 * i), 32, 8,
                           128, True, seed=93 + i, device=DEV) for i in range(6)]
    expect = []
    for b in batches:
        o = torch.full_like(b.q, float("nan"))
        n = pa.workspace_bytes(*b.args(o)[:9], pa.options())
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        pa.unified_attention(*b.args(o), opts=pa.options(), workspace=ws)
        torch.cuda.synchronize()
        expect.append(o)
    outs = [[None] * len(batches) for _ in range(2)]
    errors = []

    def worker(w):
        try:
            for rep in range(3):
                for i in (range(len(batches)) if w == 0 else reversed(range(len(batches)))):
                    o = torch.full_like(batches[i].q, float("nan"))
                    pa.unified_attention(*batches[i].args(o))
                    outs[w][i] = o
        except Exception as e:   # reported in the main thread
            errors.append(e)

    say("two threads growing the library workspace")
    ts = [threading.Thread(target=worker, args=(w,)) for w in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for w in range(2):
        for i, e in enumerate(expect):
            assert torch.equal(bits(outs[w][i]), bits(e)), (w, i)


EIGHT_HEADS = [(32, 8), (4, 2), (16, 1), (32, 4), (8, 8)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", EIGHT_HEADS, ids=lambda h: f"hq{h[0]}_hkv{h[1]}")
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_eight_wave_tiles(d, heads, causal):
    """force_tile = 4: 256-row tiles on the eight-wave kernel (two wave groups
    in opposite phases), ragged query lengths that end tiles anywhere, rows
    without keys, a decode row (narrow path with eight waves)."""
    require_gpu()
    hq, hkv = heads
    rng = np.random.default_rng(2000 + 7 * d + hq + 3 * hkv + int(causal))
    q_lens = np.array([300, 1, 65, 129, 0, 17, 256, 5, 40])
    k_lens = np.array([max(int(x), int(ql)) for x, ql in
                       zip(rng.integers(1, 1500, size=len(q_lens)), q_lens)])
    k_lens[1] = 700
    if causal:
        k_lens[7] = 3          # 5 queries over 3 keys: first two rows have no key
    b = build_batch("eight", q_lens, k_lens, hq, hkv, d, causal, seed=int(rng.integers(1 << 30)),
                    device=DEV)
    plan = pa.plan_describe(*b.args(b.new_out())[:9], opts=pa.options(force_tile=4))
    assert plan["tile_rows"] == 256 // (hq // hkv) * (hq // hkv)
    say(f"eight-wave d={d} hq={hq} hkv={hkv} causal={causal}")
    out = run_pa(b, opts=pa.options(force_tile=4))
    torch.cuda.synchronize()
    full_parity(b, out, f"eight d{d} {heads} causal={causal}")


@pytest.mark.parametrize("splits", [2, 7])
def test_eight_wave_tiles_with_splits_and_permutation(splits):
    require_gpu()
    b = build_batch("eight_split", [300, 1, 64, 200], [3000, 900, 2100, 200], 32, 8, 128, True,
                    seed=94 + splits, device=DEV)
    b2 = repermute_pool(b, seed=95)
    opts = pa.options(force_tile=4, force_num_splits=splits)
    say(f"eight-wave splits={splits}")
    o1 = run_pa(b, opts=opts)
    o2 = run_pa(b2, opts=opts)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o2))
    full_parity(b, o1, f"eight splits={splits}")

"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself (a library attention routine, a 50-digit brute force, closed
forms, hand-derived fixtures and invariants of the mathematics).

Every pin takes the oracle module as an argument so that the mutation tests can
run the same pins against deliberately broken copies of the oracle and show
that each plausible mistake is caught by at least one pin.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from workloads import build_batch, make_workload, repermute_pool

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# helpers (test-side; none of them computes attention)
# ---------------------------------------------------------------------------

def host_batch(b):
    return b.host()


def call(orc, h, **over):
    a = dict(h)
    a.update(over)
    return orc.paged_attention(a["q"], a["k_cache"], a["v_cache"], a["cu_seqlens_q"],
                               a["seqused_k"], a["block_table"], a["softmax_scale"],
                               a["causal"], **({"key_window": a["key_window"]}
                                               if "key_window" in a else {}))


def scatter_dense(dense, block_table, pool, block_size):
    """Write each sequence's logical ``[L, Hkv, d]`` rows into the pool, block
    by block (the inverse of reading through the block table)."""
    for s, rows in enumerate(dense):
        L = rows.shape[0]
        for b in range(-(-L // block_size)):
            lo = b * block_size
            n = min(block_size, L - lo)
            pool[block_table[s][b], :n] = rows[lo:lo + n]


def small_batch(q_lens, k_lens, hq, hkv, d, causal, seed, block_size=4, pool_extra=3):
    nblk = sum(-(-int(L) // block_size) for L in k_lens)
    b = build_batch("pin", q_lens, k_lens, hq, hkv, d, causal, seed, device="cpu",
                    block_size=block_size, pool_blocks=nblk + 1 + pool_extra)
    return b


def sdpa_reference(q_seq, k_dense, v_dense, scale, causal):
    """torch SDPA in float64 on one sequence: q [q_s, Hq, d], k/v [L, Hkv, d]."""
    qs, L = q_seq.shape[0], k_dense.shape[0]
    qt = torch.as_tensor(q_seq, dtype=torch.float64).permute(1, 0, 2)[None]
    kt = torch.as_tensor(k_dense, dtype=torch.float64).permute(1, 0, 2)[None]
    vt = torch.as_tensor(v_dense, dtype=torch.float64).permute(1, 0, 2)[None]
    mask = None
    if causal:
        # keep the lower triangle shifted right by L - q_s (end-aligned causal)
        mask = torch.ones(qs, L, dtype=torch.bool).tril(diagonal=L - qs)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                       enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_golden_closed_forms(orc):
    """Hand-derived cases in tests/golden/closed_form.json."""
    with open(os.path.join(GOLDEN, "closed_form.json")) as f:
        cases = json.load(f)["cases"]
    sym = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0),
           "2ln3": 2.0 * math.log(3.0)}

    def num(x):
        if isinstance(x, list):
            return [num(y) for y in x]
        return sym[x] if isinstance(x, str) else float(x)

    for c in cases:
        q = np.array(num(c["q"]))
        k = np.array(num(c["k"]))
        v = np.array(num(c["v"]))
        B = c["block_size"]
        L = k.shape[0]
        nblk = -(-L // B)
        pool_k = np.full((nblk, B) + k.shape[1:], np.nan)
        pool_v = np.full((nblk, B) + v.shape[1:], np.nan)
        table = np.arange(nblk)[None]
        scatter_dense([k], table, pool_k, B)
        scatter_dense([v], table, pool_v, B)
        out, lse = orc.paged_attention(q, pool_k, pool_v, [0, q.shape[0]], [L], table,
                                       c["softmax_scale"], c["causal"])
        np.testing.assert_allclose(out, np.array(num(c["expected_out"])), rtol=1e-14,
                                   atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(num(c["expected_lse"])), rtol=1e-14,
                                   atol=1e-14, err_msg=c["name"])


def pin_single_key_exact(orc):
    """One admissible key: weight exactly 1, output exactly that key's value."""
    for causal in (True, False):
        b = small_batch([1, 3], [1, 3], 4, 2, 8, causal, seed=11)
        h = host_batch(b)
        out, _ = call(orc, h)
        v0 = h["v_cache"][h["block_table"][0, 0], 0]            # [Hkv, d]
        G = 2
        assert np.array_equal(out[0], np.repeat(v0, G, axis=0).astype(np.float64))
        if causal:   # first row of a fresh causal prefill (q_s == L_s) sees key 0 only
            v1 = h["v_cache"][h["block_table"][1, 0], 0]
            assert np.array_equal(out[1], np.repeat(v1, G, axis=0).astype(np.float64))


def pin_uniform_scores_prefix_mean(orc):
    """q = 0 makes every admissible score equal: the output is the plain mean of
    V over the admissible keys.  For a causal chunk of q_s queries over L keys,
    query i averages keys 0 .. L - q_s + i; this fixes the causal alignment."""
    q_lens, k_lens = [1, 4, 6, 5], [9, 13, 6, 30]
    for causal in (True, False):
        b = small_batch(q_lens, k_lens, 4, 2, 8, causal, seed=12)
        h = host_batch(b)
        h["q"] = np.zeros_like(h["q"])
        out, _ = call(orc, h)
        cu = np.concatenate([[0], np.cumsum(q_lens)])
        for s, (qs, L) in enumerate(zip(q_lens, k_lens)):
            rows = [h["v_cache"][h["block_table"][s, j // 4], j % 4].astype(np.float64)
                    for j in range(L)]           # [L][Hkv, d], written out key by key
            for i in range(qs):
                n_keys = (L - qs + i + 1) if causal else L
                mean = sum(rows[:n_keys]) / n_keys
                np.testing.assert_allclose(out[cu[s] + i], np.repeat(mean, 2, axis=0),
                                           rtol=1e-13, atol=1e-14)


def pin_sdpa_dense(orc):
    """Paged oracle == torch SDPA (float64) on the dense logical K/V, with an
    end-aligned causal mask built from ``tril``."""
    rng = np.random.default_rng(21)
    for (hq, hkv, causal) in [(8, 2, True), (8, 2, False), (3, 3, True), (6, 1, True)]:
        q_lens = [1, 3, 7, 1, 12, 4]
        k_lens = [9, 30, 7, 50, 17, 4]
        d, B = 16, 4
        b = small_batch(q_lens, k_lens, hq, hkv, d, causal, seed=22)
        h = host_batch(b)
        dense_k = [rng.standard_normal((L, hkv, d)) for L in k_lens]
        dense_v = [rng.standard_normal((L, hkv, d)) for L in k_lens]
        pool_k = h["k_cache"].astype(np.float64)
        pool_v = h["v_cache"].astype(np.float64)
        scatter_dense(dense_k, h["block_table"], pool_k, B)
        scatter_dense(dense_v, h["block_table"], pool_v, B)
        scale = float(np.float32(0.37))
        out, _ = call(orc, h, k_cache=pool_k, v_cache=pool_v, softmax_scale=scale)
        cu = np.concatenate([[0], np.cumsum(q_lens)])
        for s in range(len(q_lens)):
            ref = sdpa_reference(h["q"][cu[s]:cu[s + 1]], dense_k[s], dense_v[s], scale,
                                 causal)
            np.testing.assert_allclose(out[cu[s]:cu[s + 1]], ref, rtol=1e-12, atol=1e-12)


def pin_causal_reductions(orc):
    """q_s = 1: causal equals non-causal.  q_s = L_s: equals SDPA's own
    (top-left) causal mask, which coincides with end alignment when square."""
    b = small_batch([1, 1, 1], [5, 17, 2], 4, 4, 8, True, seed=31)
    h = host_batch(b)
    o1, l1 = call(orc, h)
    o2, l2 = call(orc, h, causal=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    b = small_batch([6, 11], [6, 11], 4, 2, 8, True, seed=32)
    h = host_batch(b)
    out, _ = call(orc, h)
    cu = [0, 6, 17]
    for s, L in enumerate([6, 11]):
        k = np.stack([h["k_cache"][h["block_table"][s, j // 4], j % 4] for j in range(L)])
        v = np.stack([h["v_cache"][h["block_table"][s, j // 4], j % 4] for j in range(L)])
        qt = torch.as_tensor(h["q"][cu[s]:cu[s + 1]], dtype=torch.float64).permute(1, 0, 2)
        kt = torch.as_tensor(k, dtype=torch.float64).permute(1, 0, 2)
        vt = torch.as_tensor(v, dtype=torch.float64).permute(1, 0, 2)
        ref = F.scaled_dot_product_attention(qt[None], kt[None], vt[None], is_causal=True,
                                             scale=float(np.float32(h["softmax_scale"])),
                                             enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[cu[s]:cu[s + 1]], ref, rtol=1e-12, atol=1e-12)


def pin_gqa_replication(orc):
    """Replicating each kv-head G times (so Hkv' = Hq) leaves the result unchanged."""
    b = small_batch([2, 5, 1], [9, 14, 21], 8, 2, 8, True, seed=41)
    h = host_batch(b)
    out, lse = call(orc, h)
    G = 4
    rep_k = np.repeat(h["k_cache"], G, axis=2)
    rep_v = np.repeat(h["v_cache"], G, axis=2)
    out2, lse2 = call(orc, h, k_cache=rep_k, v_cache=rep_v)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-14)


def pin_permutation_and_poison(orc):
    """Output is bitwise independent of the physical placement of blocks and of
    whatever the unowned slots hold."""
    b = small_batch([1, 5, 16, 3], [7, 20, 40, 3], 4, 2, 16, True, seed=51)
    h = host_batch(b)
    out, lse = call(orc, h)
    b2 = repermute_pool(b, seed=52)
    out2, lse2 = call(orc, host_batch(b2))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    zk = np.nan_to_num(h["k_cache"], nan=0.0)
    zv = np.nan_to_num(h["v_cache"], nan=0.0)
    out3, lse3 = call(orc, h, k_cache=zk, v_cache=zv)
    assert np.array_equal(out, out3) and np.array_equal(lse, lse3)
    assert np.isfinite(out).all()


def pin_invariants(orc):
    """Convexity, linearity in V, shift invariance in K, row independence."""
    q_lens, k_lens = [3, 1, 8], [10, 25, 8]
    b = small_batch(q_lens, k_lens, 4, 2, 8, True, seed=61)
    h = host_batch(b)
    out, _ = call(orc, h)
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    table = h["block_table"]
    # convexity: each output lies within [min, max] of V over its admissible keys
    for s, (qs, L) in enumerate(zip(q_lens, k_lens)):
        v = np.stack([h["v_cache"][table[s, j // 4], j % 4] for j in range(L)])
        for i in range(qs):
            vis = v[:L - qs + i + 1]                                  # [n, Hkv, d]
            lo = np.repeat(vis.min(axis=0), 2, axis=0)
            hi = np.repeat(vis.max(axis=0), 2, axis=0)
            assert np.all(out[cu[s] + i] >= lo - 1e-12) and np.all(out[cu[s] + i] <= hi + 1e-12)
    # linearity in V
    rng = np.random.default_rng(62)
    v2 = rng.standard_normal(h["v_cache"].shape)
    o_a, _ = call(orc, h, v_cache=np.nan_to_num(h["v_cache"]))
    o_b, _ = call(orc, h, v_cache=v2)
    o_c, _ = call(orc, h, v_cache=2.5 * np.nan_to_num(h["v_cache"]) - 0.75 * v2)
    np.testing.assert_allclose(o_c, 2.5 * o_a - 0.75 * o_b, rtol=1e-12, atol=1e-12)
    # shift invariance: adding one vector to every key row leaves softmax unchanged
    u = rng.standard_normal(h["k_cache"].shape[-1])
    o_s, _ = call(orc, h, k_cache=h["k_cache"].astype(np.float64) + u)
    np.testing.assert_allclose(o_s, out, rtol=1e-11, atol=1e-12)
    # row independence: reversing the sequence order only permutes output rows
    order = [2, 1, 0]
    q_parts = [h["q"][cu[s]:cu[s + 1]] for s in order]
    out_r, _ = call(orc, h, q=np.concatenate(q_parts), block_table=table[order],
                    seqused_k=np.array(k_lens)[order],
                    cu_seqlens_q=np.concatenate([[0], np.cumsum(np.array(q_lens)[order])]))
    expect = np.concatenate([out[cu[s]:cu[s + 1]] for s in order])
    np.testing.assert_allclose(out_r, expect, rtol=1e-14, atol=1e-15)


def pin_lse_merge(orc):
    """Split every row's keys into windows, compute each window's (out, lse),
    merge: equals the unsplit result.  One part merges to itself; parts with no
    key drop out."""
    q_lens, k_lens = [1, 4, 2], [37, 12, 50]
    b = small_batch(q_lens, k_lens, 4, 2, 8, True, seed=71)
    h = host_batch(b)
    out, lse = call(orc, h)
    for bounds in ([0, 16, 32, 64], [0, 5, 6, 29, 64], [0, 64, 128, 256]):
        parts = [call(orc, h, key_window=(lo, hi)) for lo, hi in zip(bounds[:-1], bounds[1:])]
        m_out, m_lse = orc.merge_lse([p[0] for p in parts], [p[1] for p in parts])
        np.testing.assert_allclose(m_out, out, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(m_lse, lse, rtol=1e-13, atol=1e-14)
    one_out, one_lse = orc.merge_lse([out], [lse])
    assert np.array_equal(one_out, out) and np.array_equal(one_lse, lse)
    empty = np.full_like(lse, -np.inf)
    e_out, e_lse = orc.merge_lse([out, np.full_like(out, 123.0)], [lse, empty])
    np.testing.assert_allclose(e_out, out, rtol=1e-15, atol=0)
    np.testing.assert_allclose(e_lse, lse, rtol=1e-15, atol=0)
    # lse of a whole row equals log-sum-exp of its scaled scores, brute force
    s, i = 0, 0
    L = k_lens[s]
    k = np.stack([h["k_cache"][h["block_table"][s, j // 4], j % 4] for j in range(L)])
    sc = float(np.float32(h["softmax_scale"]))
    scores = [sc * float(np.dot(h["q"][i, 0].astype(np.float64), k[j, 0].astype(np.float64)))
              for j in range(L)]
    import mpmath
    with mpmath.workdps(40):
        ref = float(mpmath.log(sum(mpmath.exp(mpmath.mpf(x)) for x in scores)))
    assert abs(lse[0, 0] - ref) <= 1e-12 * max(1.0, abs(ref))


def pin_empty_rows(orc):
    """Rows with no admissible key (L = 0, or causal with q_s > L_s) give 0 and
    lse = -inf; q_s = 0 sequences contribute no rows."""
    b = small_batch([2, 0, 3, 1], [0, 5, 2, 4], 2, 1, 8, True, seed=81)
    h = host_batch(b)
    out, lse = call(orc, h)
    assert np.all(out[0:2] == 0) and np.all(np.isneginf(lse[0:2]))
    # sequence 2: q_s = 3, L = 2 -> query 0 at position -1 sees nothing
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(lse[3:]))


def pin_rows_api(orc):
    """The selected-rows entry point equals the whole-batch result on those rows."""
    b = small_batch([1, 5, 16, 3], [7, 20, 40, 3], 8, 2, 16, True, seed=91)
    h = host_batch(b)
    out, lse = call(orc, h)
    tokens = np.array([0, 1, 3, 5, 6, 12, 21, 24, 24])
    heads = np.array([0, 7, 3, 4, 1, 6, 2, 5, 0])
    o, l = orc.paged_attention_rows(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                    h["seqused_k"], h["block_table"], h["softmax_scale"],
                                    h["causal"], tokens, heads)
    np.testing.assert_allclose(o, out[tokens, heads], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l, lse[tokens, heads], rtol=1e-14, atol=1e-15)


def _mp_compare(orc, h, dps=30, rtol=1e-12):
    from oracle.brute import brute_force_attention, to_float_array
    out, lse = call(orc, h)
    bo, bl = brute_force_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                   h["seqused_k"], h["block_table"], h["softmax_scale"],
                                   h["causal"], dps=dps)
    np.testing.assert_allclose(out, to_float_array(bo), rtol=rtol, atol=1e-13)
    np.testing.assert_allclose(lse, to_float_array(bl), rtol=rtol, atol=1e-13)


def pin_brute_tiny_workload(orc):
    """The 3-sequence tiny workload (query lens 1/5/16, context 7/20/40, 4 q-heads,
    2 kv-heads, head_dim 64, 16-block pool) against the 50-digit brute force."""
    b = make_workload("tiny_mixed_3seq")
    _mp_compare(orc, host_batch(b), dps=50)


def pin_brute_grid(orc, full=True):
    """Exhaustive tiny grid against the brute force: q_s 1..4, L q_s..9,
    block size 1/2/4, (Hq, Hkv) in (1,1), (2,1), (4,2), d 1/2/4, both masks."""
    pairs = [(qs, L) for qs in range(1, 5) for L in range(qs, 10)]
    q_lens = [p[0] for p in pairs]
    k_lens = [p[1] for p in pairs]
    combos = list(itertools.product((1, 2, 4), ((1, 1), (2, 1), (4, 2)), (1, 2, 4),
                                    (True, False)))
    if not full:
        combos = combos[::9]
    for n, (B, (hq, hkv), d, causal) in enumerate(combos):
        b = small_batch(q_lens, k_lens, hq, hkv, d, causal, seed=100 + n, block_size=B)
        _mp_compare(orc, host_batch(b), dps=25)


# cheap pins first: the mutation tests stop at the first failure
def pin_fp8_decoder(orc):
    """E4M3 ("fn") decoding: every one of the 256 codes against torch's own
    float8_e4m3fn conversion (a library routine), plus values derived by hand
    from the format's definition (bias 7, subnormals below 2^-6, no infinity,
    S.1111.111 NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.decode_e4m3fn(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    assert np.array_equal(mine[~np.isnan(lib)], lib[~np.isnan(lib)])
    hand = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5}
    for c, v in hand.items():
        assert orc.decode_e4m3fn(np.array([c]))[0] == v, (hex(c), v)
    assert np.isnan(orc.decode_e4m3fn(np.array([0x7F, 0xFF]))).all()
    assert math.copysign(1.0, orc.decode_e4m3fn(np.array([0x80]))[0]) == -1.0


def pin_fp8_cache_path(orc):
    """The fp8 path equals the bf16 path run on caches decoded by torch and
    scaled (an independent decoder), and the scales act exactly as the
    definition says: v_scale multiplies every output, k_scale multiplies the
    scores (the same as multiplying softmax_scale)."""
    b = build_batch("pin8", [1, 3, 5], [9, 20, 30], 8, 2, 16, True, 31, device="cpu",
                    block_size=4, kv_dtype="fp8_e4m3fn", k_scale=0.25, v_scale=0.5)
    h = b.host()
    out8, lse8 = orc.paged_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                     h["seqused_k"], h["block_table"], h["softmax_scale"],
                                     h["causal"], kv_format="fp8_e4m3fn",
                                     k_scale=b.k_scale, v_scale=b.v_scale)
    kd = b.k_cache.to(torch.float64).numpy() * b.k_scale    # NaN codes stay NaN
    vd = b.v_cache.to(torch.float64).numpy() * b.v_scale
    ref, lref = orc.paged_attention(h["q"], kd, vd, h["cu_seqlens_q"], h["seqused_k"],
                                    h["block_table"], h["softmax_scale"], h["causal"])
    assert np.isfinite(out8).all()
    np.testing.assert_allclose(out8, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse8, lref, rtol=1e-12, atol=1e-12)
    kw = dict(kv_format="fp8_e4m3fn", k_scale=b.k_scale)
    o1, _ = orc.paged_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                h["seqused_k"], h["block_table"], h["softmax_scale"],
                                h["causal"], v_scale=1.0, **kw)
    o2, _ = orc.paged_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                h["seqused_k"], h["block_table"], h["softmax_scale"],
                                h["causal"], v_scale=2.0, **kw)
    assert np.array_equal(o2, 2.0 * o1)                     # powers of two scale exactly
    o3, _ = orc.paged_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                h["seqused_k"], h["block_table"], h["softmax_scale"] * 0.25,
                                h["causal"], kv_format="fp8_e4m3fn", k_scale=1.0, v_scale=1.0)
    np.testing.assert_allclose(o3, o1, rtol=1e-12, atol=1e-14)


def pin_fp8_encoder(orc):
    """E4M3 ("fn") encoding: in range, torch's float32 -> float8_e4m3fn
    conversion (round to nearest even) on random and boundary values; beyond
    it, saturation by the reading the cache write takes; ties and specials by
    hand from the format's definition."""
    rng = np.random.default_rng(7)
    grid = orc.decode_e4m3fn(np.arange(127))
    mids = (grid[:-1] + grid[1:]) / 2                     # exact ties, all of them
    x = np.concatenate([rng.normal(0, 40, 20000), rng.normal(0, 0.005, 5000),
                        rng.uniform(-463.99, 463.99, 5000), mids, -mids, grid, -grid,
                        np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    x = x[np.abs(x) < 464]
    mine = orc.encode_e4m3fn(x)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, lib)
    hand = {1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A, 1.5 * 2.0 ** -9: 0x02, 0.5 * 2.0 ** -9: 0x00,
            448.0: 0x7E, 463.99: 0x7E, 464.0: 0x7E, 1e6: 0x7E, -1e6: 0xFE, -0.0: 0x80,
            2.0 ** -6: 0x08, 15.5 * 2.0 ** -10: 0x08}
    for v, c in hand.items():
        assert int(orc.encode_e4m3fn(np.float32(v))) == c, (v, hex(c))
    assert int(orc.encode_e4m3fn(np.float32(np.nan))) & 0x7F == 0x7F
    # decode(encode(x)) is x for every grid value
    assert np.array_equal(orc.decode_e4m3fn(orc.encode_e4m3fn(grid.astype(np.float32))), grid)


def pin_cache_write(orc):
    """Writing tokens then reading them through the block table returns them
    (bf16) or their round-trip values (fp8); untouched and skipped slots keep
    their contents."""
    rng = np.random.default_rng(11)
    NB, B, Hkv, d = 5, 4, 2, 8
    key = rng.normal(size=(6, Hkv, d)).astype(np.float32)
    val = rng.normal(size=(6, Hkv, d)).astype(np.float32)
    slots = np.array([3, 7, -1, 12, 0, 19])
    kc = rng.normal(size=(NB, B, Hkv, d)).astype(np.float32)
    vc = rng.normal(size=(NB, B, Hkv, d)).astype(np.float32)
    k2, v2 = orc.cache_write(key, val, kc, vc, slots)
    for i, s_ in enumerate(slots):
        if s_ >= 0:
            assert np.array_equal(k2[s_ // B, s_ % B], key[i])
            assert np.array_equal(v2[s_ // B, s_ % B], val[i])
    touched = np.zeros((NB, B), bool)
    for s_ in slots[slots >= 0]:
        touched[s_ // B, s_ % B] = True
    assert np.array_equal(k2[~touched], kc[~touched]) and np.array_equal(v2[~touched], vc[~touched])
    kc8 = rng.integers(0, 0x7F, size=(NB, B, Hkv, d)).astype(np.uint8)
    k8, v8 = orc.cache_write(key, val, kc8, kc8.copy(), slots, kv_format="fp8_e4m3fn",
                             k_scale=0.125, v_scale=0.25)
    for i, s_ in enumerate(slots):
        if s_ >= 0:
            back = orc.decode_e4m3fn(k8[s_ // B, s_ % B]) * 0.125
            grid_step = np.maximum(np.abs(key[i]) * 2.0 ** -3, 2.0 ** -9 * 0.125)
            assert (np.abs(back - key[i]) <= grid_step / 2 * (1 + 1e-12)).all()
    assert np.array_equal(k8[~touched], kc8[~touched])


ALL_PINS = [
    pin_golden_closed_forms,
    pin_single_key_exact,
    pin_uniform_scores_prefix_mean,
    pin_causal_reductions,
    pin_empty_rows,
    pin_permutation_and_poison,
    pin_sdpa_dense,
    pin_gqa_replication,
    pin_invariants,
    pin_lse_merge,
    pin_rows_api,
    pin_brute_tiny_workload,
    pin_brute_grid,
    pin_fp8_decoder,
    pin_fp8_cache_path,
    pin_fp8_encoder,
    pin_cache_write,
]

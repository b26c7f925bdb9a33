"""GPU: the exported log-sum-exp against the oracle's, and cascade
composition: attention over a shared prefix (non-causal) merged with
attention over each sequence's own suffix (causal) equals one pass over the
whole context (the merge identity the oracle is pinned by)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_unified_amd as pa
from gpu_util import check_close, require_gpu, say, with_scales
from workloads import build_batch

pytestmark = pytest.mark.gpu

DEV = "cuda"
LSE_ATOL = 2e-3        # fp32 lse from fp32 sums: |error| ~ 1e-5 expected


def run_lse(b, opts=None):
    out = torch.full_like(b.q, float("nan"))
    lse = torch.full((b.total_q, b.num_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    pa.unified_attention_lse(*b.args(out)[:4], lse, *b.args(out)[4:], opts=with_scales(b, opts))
    return out, lse


def check_lse(g, r, what):
    g = g.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(r)), f"{what}: -inf rows differ"
    fin = np.isfinite(r)
    assert np.isfinite(g[fin]).all(), f"{what}: non-finite lse"
    err = np.abs(g[fin] - r[fin]).max() if fin.any() else 0.0
    assert err <= LSE_ATOL, f"{what}: lse error {err:.2e}"
    return err


CASES = {
    "decode_persistent": ([1, 1, 1, 2, 0, 1], [300, 1, 2000, 64, 5, 0], 32, 8, 128, True, None, "bf16"),
    "decode_split": ([1, 1, 1], [3000, 700, 5], 16, 2, 64, True, dict(force_num_splits=4), "bf16"),
    "grid_narrow": ([1, 2, 1], [700, 33, 9], 32, 8, 128, True, dict(force_tile=3), "bf16"),
    "wide_causal": ([200, 1, 33, 5], [700, 40, 33, 2], 32, 8, 128, True, None, "bf16"),
    "wide_noncausal_split": ([16, 40], [3000, 90], 32, 4, 128, False, dict(force_num_splits=3), "bf16"),
    "fp8_wide_and_decode": ([1, 100, 1], [500, 400, 3000], 32, 8, 128, True, None, "fp8_e4m3fn"),
    "f16_decode_persistent": ([1, 1, 1, 2, 0, 1], [300, 1, 9000, 64, 5, 0], 32, 8, 128, True, None, "f16"),
    "f16_wide_split": ([200, 1, 33], [2500, 40, 90], 32, 4, 128, True, dict(force_num_splits=3), "f16"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_lse_export(case):
    require_gpu()
    q, k, hq, hkv, d, causal, o, fmt = CASES[case]
    b = build_batch("lse", q, k, hq, hkv, d, causal, seed=400 + len(case), device=DEV,
                    kv_dtype=fmt, k_scale=0.25, v_scale=0.5)
    say(f"lse {case}")
    out, lse = run_lse(b, pa.options(**o) if o else None)
    torch.cuda.synchronize()
    h = b.host()
    ref, lref = oracle.paged_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                       h["seqused_k"], h["block_table"], h["softmax_scale"],
                                       h["causal"], **b.kv_kwargs())
    check_close(out.float().cpu().numpy(), ref, f"lse {case} out")
    check_lse(lse, lref, f"lse {case}")


@pytest.mark.parametrize("elem", ["bf16", "f16"])
def test_cascade_shared_prefix(elem):
    """Sequences share a 64-key prefix (the same four physical blocks)."""
    require_gpu()
    P = 64
    q_lens = [1, 7, 1, 33, 2]
    suf = [50, 7, 300, 40, 2]
    L = [P + s for s in suf]
    hq, hkv, d = 32, 8, 128
    b = build_batch("casc", q_lens, L, hq, hkv, d, True, seed=501, device=DEV, kv_dtype=elem)
    table = b.block_table.clone()
    table[:, : P // 16] = table[0, : P // 16]                 # one shared prefix
    b.block_table = table
    say(f"cascade {elem}: one pass")
    one, lse_one = run_lse(b)
    # prefix pass: every query sees the whole prefix (non-causal over P keys)
    bp = build_batch("casc", q_lens, L, hq, hkv, d, True, seed=501, device=DEV, kv_dtype=elem)
    bp.k_cache, bp.v_cache, bp.q = b.k_cache, b.v_cache, b.q
    bp.block_table = table[:, : P // 16].contiguous()
    bp.seqused_k = torch.full_like(b.seqused_k, P)
    bp.k_lens = np.full_like(b.k_lens, P)
    bp.max_seqlen_k = P
    bp.causal = False
    say("cascade: prefix pass")
    o_pre, l_pre = run_lse(bp)
    # suffix pass: causal over each sequence's own blocks
    bs = build_batch("casc", q_lens, L, hq, hkv, d, True, seed=501, device=DEV, kv_dtype=elem)
    bs.k_cache, bs.v_cache, bs.q = b.k_cache, b.v_cache, b.q
    bs.block_table = table[:, P // 16:].contiguous()
    bs.seqused_k = b.seqused_k - P
    bs.k_lens = b.k_lens - P
    bs.max_seqlen_k = int(bs.k_lens.max())
    say("cascade: suffix pass")
    o_suf, l_suf = run_lse(bs)
    merged = torch.full_like(one, float("nan"))
    l_m = torch.full_like(lse_one, float("nan"))
    pa.merge_attention(o_pre, l_pre, o_suf, l_suf, merged, l_m)
    torch.cuda.synchronize()
    h = b.host()
    ref, lref = oracle.paged_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                       h["seqused_k"], h["block_table"], h["softmax_scale"],
                                       h["causal"], **b.kv_kwargs())
    check_close(merged.float().cpu().numpy(), ref, "cascade merged vs oracle")
    check_close(one.float().cpu().numpy(), ref, "one pass vs oracle")
    check_lse(l_m, lref, "cascade lse")
    # merged and one-pass results agree to bf16 rounding
    diff = (merged.float() - one.float()).abs().max().item()
    assert diff <= 2e-2, diff

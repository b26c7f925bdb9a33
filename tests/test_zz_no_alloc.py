"""GPU: pa_unified_attention_noalloc (split workspace in the library's static
device scratch, no allocation) against pa_unified_attention_ex with a caller
workspace and the same options, bit for bit, on two calls in a row, the second
with a smaller batch (the scratch keeps the first call's contents), and both
against the fp64 oracle.  A batch whose plan needs more than the scratch
holds is refused before anything is launched."""

import pytest
import torch

import paged_kv_cache_unified_amd as pa
from gpu_util import bits, full_parity, require_gpu, say
from workloads import build_batch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def ex_call(b, opts):
    out = torch.full_like(b.q, float("nan"))
    n = pa.workspace_bytes(*b.args(out)[:9], opts)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    pa.unified_attention(*b.args(out), opts=opts, workspace=ws)
    return out, n


def noalloc_call(b, opts):
    out = torch.full_like(b.q, float("nan"))
    pa.unified_attention_noalloc(*b.args(out), opts=opts)
    return out


# (name, q_lens, k_lens, Hq, Hkv, d, causal, options): each needs a split workspace
CASES = [
    # wide tiles with longest-first order and key splits, then a smaller one
    ("grid", [1, 40, 200, 1, 3, 17], [3000, 900, 1500, 60, 2500, 17], 32, 8, 128, True,
     dict(force_num_splits=3)),
    ("grid_small", [1, 20, 5], [700, 300, 90], 32, 8, 128, False, dict(force_num_splits=2)),
    # persistent decode, even split of a ragged batch, then a smaller one
    ("even", [1] * 12, [9000, 40, 3000, 1, 2047, 5000, 80, 6000, 300, 16, 1200, 4000], 32, 8,
     128, True, {}),
    ("even_small", [1] * 5, [2100, 30, 1500, 7, 1100], 32, 8, 128, True, {}),
]


@pytest.mark.parametrize("pair", [(0, 1), (2, 3), (0, 3)], ids=["grid", "even", "mixed_kinds"])
def test_noalloc_matches_ex_twice(pair):
    require_gpu()
    for i in pair:
        name, ql, kl, hq, hkv, d, causal, o = CASES[i]
        b = build_batch(name, ql, kl, hq, hkv, d, causal, seed=300 + i, device=DEV)
        opts = pa.options(**o)
        ref, n = ex_call(b, opts)
        assert 0 < n <= pa.NOALLOC_SCRATCH_BYTES, (name, n)
        say(f"noalloc {name}: workspace {n} bytes")
        got = noalloc_call(b, opts)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"{name}: differs from pa_unified_attention_ex"
        full_parity(b, got, f"noalloc {name}")


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    require_gpu()
    b = build_batch("big", [1] * 8, [60000] * 8, 32, 8, 128, True, seed=310, device=DEV)
    opts = pa.options(force_num_splits=1000)
    out = torch.full_like(b.q, float("nan"))
    assert pa.workspace_bytes(*b.args(out)[:9], opts) > pa.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pa.PaError) as e:
        pa.unified_attention_noalloc(*b.args(out), opts=opts)
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a refused call wrote its output"

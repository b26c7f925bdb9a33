"""Calls captured in a HIP graph (torch.cuda.graph) and replayed.

Serving loops capture the attention call once and replay it every step.  A
captured call must hold no allocation, memset or host synchronisation, and
every replay must recompute everything from the inputs: the longest-first
order, the split partials and the part counts live in a workspace that the
test fills with garbage before each replay.  Each graph is replayed several
times, with other library calls and synchronisations in between, and every
replay must equal the eager call bit for bit (outputs are deterministic: the
unit order decides only which work-group computes a unit).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_unified_amd as pa
from gpu_util import bits, full_parity, require_gpu, run_pa, say, with_scales
from workloads import build_batch

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPLAYS = 4


def _case(kind):
    rng = np.random.default_rng({"decode_fixed": 11, "decode_even": 12, "mixed": 13,
                                 "prefill_splits": 14, "decode_fp8": 15}[kind])
    if kind in ("decode_fixed", "decode_fp8"):
        q = np.ones(300, int)
        k = rng.integers(1000, 1101, size=300)
    elif kind == "decode_even":
        q = np.ones(40, int)
        k = np.clip(np.round(np.exp(rng.normal(np.log(400.0), 1.0, size=40))), 4, 6000).astype(int)
    else:
        q = np.array([512, 1, 1, 200, 1, 33, 0, 1])
        k = np.maximum(q, rng.integers(0, 2500, size=len(q)))
    fp8 = dict(kv_dtype="fp8_e4m3fn", k_scale=1 / 64, v_scale=1 / 64) if kind == "decode_fp8" else {}
    b = build_batch(f"graph_{kind}", q, k, 32, 8, 128, True, seed=int(rng.integers(1 << 30)),
                    device=DEV, **fp8)
    opts = pa.options(force_num_splits=3) if kind == "prefill_splits" else pa.options()
    return b, with_scales(b, opts)


def _other_batch():
    """A different batch run eagerly between replays (other grid, other workspace)."""
    return build_batch("graph_other", [1, 7, 64], [300, 90, 700], 8, 2, 64, True, seed=5,
                       device=DEV)


@pytest.mark.parametrize("kind", ["decode_fixed", "decode_even", "mixed", "prefill_splits",
                                  "decode_fp8"])
def test_graph_replays_match_eager(kind):
    require_gpu()
    b, opts = _case(kind)
    plan = pa.plan_describe(*b.args(torch.empty_like(b.q))[:9], opts=opts)
    say(f"graph {kind}: persistent={plan['persistent']} balanced={plan['balanced']} "
        f"splits={plan['num_splits']} longest_first={plan['longest_first']}")
    n = pa.workspace_size(*b.args(torch.empty_like(b.q))[:9], opts)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)

    eager = torch.full_like(b.q, float("nan"))
    pa.unified_attention(*b.args(eager), opts=opts, workspace=ws)
    torch.cuda.synchronize()
    full_parity(b, eager, f"graph {kind} eager")

    out = torch.full_like(b.q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up off the default stream
        pa.unified_attention(*b.args(out), opts=opts, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.unified_attention(*b.args(out), opts=opts, workspace=ws)
    torch.cuda.synchronize()

    other = _other_batch()
    other_ref = run_pa(other)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        ws.fill_(0xFF)                            # stale partials, counts and unit order
        o2 = run_pa(other)                        # eager library work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(eager)), f"{kind}: replay {i} differs from eager"
        assert torch.equal(bits(o2), bits(other_ref)), f"{kind}: eager call {i} between replays"
    say(f"  {REPLAYS} replays bit-exact")


def test_graph_replays_noalloc():
    """The entry point without allocation (static device scratch), captured:
    replays equal its eager call, and the _ex path's result."""
    require_gpu()
    b, opts = _case("mixed")
    assert pa.workspace_size(*b.args(torch.empty_like(b.q))[:9], opts) <= pa.NOALLOC_SCRATCH_BYTES
    ref = run_pa(b, opts=pa.options())
    eager = torch.full_like(b.q, float("nan"))
    pa.unified_attention_noalloc(*b.args(eager), opts=opts)
    torch.cuda.synchronize()
    assert torch.equal(bits(eager), bits(ref))
    out = torch.full_like(b.q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pa.unified_attention_noalloc(*b.args(out), opts=opts)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.unified_attention_noalloc(*b.args(out), opts=opts)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        run_pa(_other_batch())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(eager)), f"noalloc replay {i} differs from eager"
    say(f"noalloc: {REPLAYS} replays bit-exact")

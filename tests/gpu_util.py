"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle.

Tolerance (bf16 inputs and output, fp32 accumulation): elementwise
``|gpu - ref| <= 2e-2 + 2e-2 * |ref|`` with the GPU value upcast from bf16, plus
a relative Frobenius error guard of 1e-2 per compared block of rows (expected
~2e-3: bf16 rounding of P and of the output).  The guard is what catches a
dropped key block at long contexts, where outputs are small and the
elementwise bar alone is loose.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_unified_amd as pa

ATOL = 2e-2
RTOL = 2e-2
FROB = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X; none found")
    return torch.device("cuda:0")


def with_scales(b, opts):
    """opts carrying the batch's fp8 scales (None stays None for bf16 caches)."""
    if b.kv_format != "fp8_e4m3fn":
        return opts
    o = opts if opts is not None else pa.options()
    o.k_scale, o.v_scale = b.k_scale, b.v_scale
    return o


def run_pa(b, opts=None, out=None, stream=None):
    """The GPU path through the C ABI (plain entry point, or _ex with opts)."""
    opts = with_scales(b, opts)
    if out is None:
        out = torch.full_like(b.q, float("nan"))
    ws = None
    if opts is not None:
        n = pa.workspace_size(*b.args(out)[:9], opts)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=b.q.device)
    if stream is not None:
        with torch.cuda.stream(stream):
            pa.unified_attention(*b.args(out), opts=opts, workspace=ws)
    else:
        pa.unified_attention(*b.args(out), opts=opts, workspace=ws)
    return out


def check_close(gpu, ref, what=""):
    """c11 bar; returns (max abs err, rel frobenius)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bad = err > ATOL + RTOL * np.abs(r)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, e.g. at "
                             f"{idx.tolist()}: gpu {g[tuple(idx[0])]} ref {r[tuple(idx[0])]}")
    den = np.linalg.norm(r)
    frob = float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g))
    assert frob <= FROB, f"{what}: relative Frobenius error {frob:.3e} > {FROB}"
    return float(err.max()) if err.size else 0.0, frob


def full_parity(b, out, what=""):
    """Whole-batch comparison with the oracle (small batches)."""
    h = b.host()
    ref, _ = oracle.paged_attention(h["q"], h["k_cache"], h["v_cache"], h["cu_seqlens_q"],
                                    h["seqused_k"], h["block_table"], h["softmax_scale"],
                                    h["causal"], **b.kv_kwargs())
    return check_close(out.float().cpu().numpy(), ref, what)


def sampled_parity(b, out, seq_ids, what=""):
    """Oracle on the listed sequences only (large batches)."""
    sub, rows = b.host_subset(seq_ids)
    ref, _ = oracle.paged_attention(sub["q"], sub["k_cache"], sub["v_cache"],
                                    sub["cu_seqlens_q"], sub["seqused_k"], sub["block_table"],
                                    sub["softmax_scale"], sub["causal"], **b.kv_kwargs())
    g = out.index_select(0, torch.as_tensor(rows, device=out.device)).float().cpu().numpy()
    return check_close(g, ref, what)


def bits(t):
    return t.view(torch.int16)

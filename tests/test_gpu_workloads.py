"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (default plan, library workspace).

* Sampled parity: the oracle computes whole sequences picked from the batch
  (longest and shortest context first, then the first and last sequence, then
  prefill chunks and decodes); the GPU output rows of those sequences must
  meet the tolerance bar.  The long-context batches compare four sequences,
  the longest (about 250 merged key parts) and the shortest among them.
* Block-histogram closed form: with q = 0 every admissible key gets weight
  exactly 1, so each output row is the plain mean of V over its admissible
  keys.  Filling V so that key j holds a one-hot vector at position
  (j // 16) % head_dim (its LOGICAL block index) makes that mean an exact
  histogram of logical block indices: count_d / n_keys.  fp32 sums of 0/1
  values are exact, so the GPU result must equal that ratio rounded to bf16,
  within one bf16 ulp.  A dropped, duplicated or misaddressed cache block
  changes a count and fails this at any context length.
"""

import numpy as np
import pytest
import torch

from gpu_util import require_gpu, run_pa, sampled_parity, say
from workloads import make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda"

WORKLOAD_NAMES = [
    "decode_256seq_ctx1k",
    "mixed_prefill512x8_decode248",
    "prefill512x8_only",
    "prefill512x8_only_d96",
    "prefill512x8_only_d256",
    "decode248_only",
    "decode_gqa8_64seq_ctx2k_4k",
    "long_decode_16seq_ctx32k_128k",
    "long_q16_noncausal_16seq_ctx32k_128k",
]
# cache formats other than bf16: sampled parity only (the histogram test writes
# float one-hot values into a bf16 cache)
PARITY_ONLY = ["decode_256seq_ctx1k_fp8"]


def pick_sequences(b, limit):
    q, k = b.q_lens, b.k_lens
    picks = [int(np.argmax(k)), int(np.argmin(k)), 0, len(q) - 1]
    if (q > 1).any() and (q == 1).any():
        picks += list(np.nonzero(q > 1)[0][:2]) + list(np.nonzero(q == 1)[0][:2])
    seen = []
    for s in picks:
        if int(s) not in seen:
            seen.append(int(s))
    return seen[:limit]


@pytest.mark.parametrize("name", WORKLOAD_NAMES + PARITY_ONLY)
def test_workload_sampled_parity(name):
    require_gpu()
    say(f"workload {name}: generate")
    b = make_workload(name, device=DEV)
    say(f"workload {name}: run")
    out = run_pa(b)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite output"
    limit = 4 if name.startswith("long_") else 6
    seqs = pick_sequences(b, limit)
    say(f"workload {name}: oracle on sequences {seqs}")
    err, frob = sampled_parity(b, out, seqs, name)
    say(f"  max err {err:.2e} rel frob {frob:.2e}")
    del b, out
    torch.cuda.empty_cache()


def histogram_v(b):
    """V cache with one-hot logical-block codes; unowned slots stay NaN."""
    D = b.head_dim
    v = torch.zeros_like(b.v_cache)
    table = b.block_table.long()
    for s in range(b.num_seqs):
        L = int(b.k_lens[s])
        nblk = -(-L // 16)
        if nblk == 0:
            continue
        phys = table[s, :nblk]
        code = torch.arange(nblk, device=v.device) % D
        v[phys, :, :, :] = 0
        v[phys[:, None], :, :, code[:, None]] = 1.0
    nan_mask = torch.isnan(b.v_cache)
    v[nan_mask] = float("nan")
    return v


def expected_histogram(b):
    D = b.head_dim
    cu = b.cu_seqlens_q.cpu().numpy()
    T = b.total_q
    exp = np.zeros((T, D), dtype=np.float64)
    for s in range(b.num_seqs):
        L, ql = int(b.k_lens[s]), int(b.q_lens[s])
        codes = (np.arange(L) // 16) % D
        csum = np.zeros((L + 1, D))
        if L:
            onehot = np.zeros((L, D))
            onehot[np.arange(L), codes] = 1.0
            csum[1:] = np.cumsum(onehot, axis=0)
        for i in range(ql):
            n = (L - ql + i + 1) if b.causal else L
            n = max(0, min(n, L))
            if n:
                exp[cu[s] + i] = csum[n] / n
    return exp


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_workload_block_histogram(name):
    require_gpu()
    say(f"histogram {name}: generate")
    b = make_workload(name, device=DEV)
    b.q = torch.zeros_like(b.q)
    b.v_cache = histogram_v(b)
    say(f"histogram {name}: run")
    out = run_pa(b)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()                                # [T, Hq, D]
    e = expected_histogram(b)[:, None, :]
    ulp = 2.0 ** -8
    bad = np.abs(g - e) > ulp * np.abs(e) + 1e-7
    assert not bad.any(), (f"{int(bad.sum())} entries off, first at {np.argwhere(bad)[0].tolist()}: "
                           f"gpu {g[tuple(np.argwhere(bad)[0])]} expected {e[np.argwhere(bad)[0][0], 0, np.argwhere(bad)[0][2]]}")
    assert np.array_equal(g == 0, np.broadcast_to(e == 0, g.shape))
    say(f"  exact histogram over {b.total_q} tokens")
    del b, out
    torch.cuda.empty_cache()

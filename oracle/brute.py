"""Scalar brute force of paged attention in 50-digit arithmetic (mpmath).

TEST INFRASTRUCTURE ONLY (see the header of ``oracle/attention.py``): only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use it.

It is a second, independent statement of the same definition, written as
plain loops over (token, head, key, element) with no vectorisation, no masking
arrays and no shared helpers, so that it can pin the vectorised oracle on tiny
inputs.  Semantics are those listed in ``oracle/attention.py``.
"""

from __future__ import annotations

import mpmath
import numpy as np


def brute_force_attention(q, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table,
                          softmax_scale, causal, dps: int = 50):
    """Return (out [T][Hq][d], lse [T][Hq]) as nested lists of ``mpmath.mpf``."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens_q]
    ctx = [int(x) for x in seqused_k]
    table = [[int(x) for x in row] for row in np.asarray(block_table)]
    T, Hq, d = q.shape
    block_size, Hkv = kc.shape[1], kc.shape[2]
    group = Hq // Hkv
    with mpmath.workdps(dps):
        scale = mpmath.mpf(float(np.float32(softmax_scale)))
        out = [[[mpmath.mpf(0)] * d for _ in range(Hq)] for _ in range(T)]
        lse = [[mpmath.mpf("-inf")] * Hq for _ in range(T)]
        for t in range(T):
            s = 0
            while not (cu[s] <= t < cu[s + 1]):
                s += 1
            q_len = cu[s + 1] - cu[s]
            i = t - cu[s]
            L = ctx[s]
            last_key = L - q_len + i if causal else L - 1
            for h in range(Hq):
                kv = h // group
                scores = []
                for j in range(min(L, last_key + 1)):
                    phys = table[s][j // block_size]
                    slot = j % block_size
                    acc = mpmath.mpf(0)
                    for c in range(d):
                        acc += mpmath.mpf(q[t, h, c]) * mpmath.mpf(kc[phys, slot, kv, c])
                    scores.append((j, phys, slot, scale * acc))
                if not scores:
                    continue
                top = max(sc for _, _, _, sc in scores)
                total = mpmath.mpf(0)
                num = [mpmath.mpf(0)] * d
                for j, phys, slot, sc in scores:
                    w = mpmath.exp(sc - top)
                    total += w
                    for c in range(d):
                        num[c] += w * mpmath.mpf(vc[phys, slot, kv, c])
                out[t][h] = [x / total for x in num]
                lse[t][h] = top + mpmath.log(total)
    return out, lse


def to_float_array(nested):
    """Nested lists of mpf -> float64 numpy array."""
    return np.array(nested, dtype=object).astype(np.float64)

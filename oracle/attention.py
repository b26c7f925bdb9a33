"""fp64 CPU oracle for unified paged attention.

TEST INFRASTRUCTURE ONLY.  The only code allowed to import, call or run this
module is ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py``.  The GPU library never links or calls it, and it shares no
code with the GPU library.

What it computes is the plain definition of the operation:

* A varlen batch, as in the ``flash_attn_varlen_func`` statement of the problem
  (page "[Kernel] Unified Triton kernel that doesn't distinguish between
  prefill + decode", PR description): the queries of all sequences are
  concatenated and ``cu_seqlens_q`` holds the offsets; each sequence may be a
  decode step (one query), a chunk of a chunked prefill or a whole prefill, all
  in one call (page "[Kernel] [V1] Improved performance for V1 Triton (ROCm)
  backend", section "How is this performance improvement achieved?").
* GQA: q-head ``h`` reads kv-head ``h // G`` with ``G = Hq // Hkv`` (the
  flash-attn convention that the unified kernel mimics, same PR description).
* The KV cache is ``[num_blocks, block_size, num_kv_heads, head_dim]`` (the
  FlashAttention key-cache layout, same PR description; the value cache is taken
  to have the same layout) and is reached through a per-sequence block table:
  context token ``j`` of sequence ``s`` is slot ``j % block_size`` of physical
  block ``block_table[s, j // block_size]``.
* Masking is causal or off (the non-causal mode is the one requested in the
  review of the unified-kernel page for cascade attention and MLA).  The causal
  mask is aligned to the end of each sequence's context: query ``i`` of a
  sequence with ``q_s`` queries and ``L_s`` context tokens sits at position
  ``L_s - q_s + i`` and sees keys ``0 .. L_s - q_s + i``.  This is the only
  reading under which a decode token sees its whole context and a prefill chunk
  sees its cached prefix, which is what serving chunked prefill and decode in
  one causal kernel requires.
* Per row: ``softmax(scale * q . k_j)`` over the admissible keys, then the
  weighted sum of the ``v_j``.  A row with no admissible key returns 0 and
  ``lse = -inf`` (the pages are silent; this is the defined reading).

All arithmetic is float64.  ``softmax_scale`` is first rounded to float32 so
the oracle uses exactly the value a float32 kernel argument carries.

16-bit caches (``kv_format`` "bf16" or "f16") are given as their values, which
float64 holds exactly.  fp8 caches (``kv_format="fp8_e4m3fn"``): the cache
holds one-byte codes of the
OCP 8-bit floating point format E4M3 in its "fn" variant (finite only; the
KV-cache format discussed in the review of page "[Kernel] [V1] Improved
performance for V1 Triton (ROCm) backend").  A code stands for
``decode(code) * scale`` with one scale per cache tensor (``k_scale``,
``v_scale``, rounded to float32 like ``softmax_scale``); ``decode_e4m3fn``
writes the format's definition out.
"""

from __future__ import annotations

import numpy as np

__all__ = ["paged_attention", "paged_attention_rows", "gather_context",
           "attend_rows", "merge_lse", "decode_e4m3fn", "encode_e4m3fn", "cache_write"]

KV_FORMATS = ("bf16", "f16", "fp8_e4m3fn")


def decode_e4m3fn(codes):
    """float64 values of OCP 8-bit E4M3 ("fn") codes.

    Bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the
    mantissa field m.  e > 0: (1 + m/8) * 2^(e-7); e = 0: (m/8) * 2^-6
    (subnormals and zero); e = 15 with m = 7 is NaN, and there is no infinity,
    so the largest finite magnitude is (1 + 6/8) * 2^8 = 448.
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def encode_e4m3fn(x):
    """E4M3 ("fn") codes of float32 values: the nearest value of the format's
    grid, ties to the even code (even mantissa field), magnitudes at or past
    464 (halfway between 448 and the next step, which the format lacks)
    saturated to 448, NaN kept as NaN (0x7F with the sign bit).

    Written as a search over the 127 finite non-negative values, so it shares
    nothing with a bit-level rounding.
    """
    x = np.asarray(x, dtype=np.float32)
    grid = decode_e4m3fn(np.arange(127))                 # codes 0x00..0x7E, increasing
    a = np.abs(x.astype(np.float64))
    sign = np.where(np.signbit(x), 0x80, 0)
    idx = np.searchsorted(grid, a, side="left")          # first grid value >= a
    idx = np.clip(idx, 1, 126)
    lo, hi = grid[idx - 1], grid[idx]
    below = a - lo
    above = hi - a
    pick_hi = (above < below) | ((above == below) & (idx % 2 == 0))
    code = np.where(pick_hi, idx, idx - 1)
    code = np.where(a <= grid[0], 0, code)               # exact zero
    code = np.where(a >= 464.0, 0x7E, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return (sign | code).astype(np.uint8)


def cache_write(key, value, k_cache, v_cache, slot_mapping, kv_format="bf16", k_scale=1.0,
                v_scale=1.0):
    """New caches with token i's ``[Hkv, d]`` key / value written to slot
    ``slot_mapping[i]`` (block ``slot // B``, position ``slot % B``); negative
    slots are skipped.  bf16 / f16: values copied (float arrays); fp8: codes of
    ``float32(x) / float32(scale)``.  Inputs are not modified.
    """
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    B = kc.shape[1]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, pos = slot // B, slot % B
        if kv_format in ("bf16", "f16"):
            kc[blk, pos] = key[i]
            vc[blk, pos] = value[i]
        elif kv_format == "fp8_e4m3fn":
            kq = np.asarray(key[i], dtype=np.float32) / np.float32(k_scale)
            vq = np.asarray(value[i], dtype=np.float32) / np.float32(v_scale)
            kc[blk, pos] = encode_e4m3fn(kq)
            vc[blk, pos] = encode_e4m3fn(vq)
        else:
            raise ValueError(f"kv_format must be one of {KV_FORMATS}")
    return kc, vc


def _context(cache, table_row, context_len, kv_format, scale):
    """Gathered ``[L, Hkv, d]`` float64 values of one sequence's cache."""
    if kv_format in ("bf16", "f16"):
        return gather_context(cache, table_row, context_len)
    if kv_format == "fp8_e4m3fn":
        codes = gather_context(cache, table_row, context_len).astype(np.int64)
        return decode_e4m3fn(codes) * float(np.float32(scale))
    raise ValueError(f"kv_format must be one of {KV_FORMATS}")


def gather_context(cache, block_table_row, context_len):
    """Logical ``[L, Hkv, d]`` float64 view of one sequence's cache contents.

    Only the first ``ceil(L / block_size)`` entries of the block-table row and
    only slots below ``L`` are touched.
    """
    L = int(context_len)
    B = cache.shape[1]
    j = np.arange(L)
    phys = np.asarray(block_table_row)[j // B]
    return np.asarray(cache[phys, j % B], dtype=np.float64)


def attend_rows(Qrows, positions, K, V, q_len, context_len, scale, causal,
                key_window=None):
    """Attention of query rows of one (sequence, kv-head) against its context.

    Qrows: ``[n, d]`` queries.  positions: ``[n]`` index ``i`` of each row's
    token within its sequence (``0 <= i < q_len``).  K, V: ``[L, d]``.
    key_window: optional ``(lo, hi)``; keys outside it are not admissible (used
    to form the partial results that the log-sum-exp merge combines).
    Returns ``(out [n, d], lse [n])`` in float64; lse in natural-log units of
    the scaled scores.
    """
    Qrows = np.asarray(Qrows, dtype=np.float64)
    n, d = Qrows.shape
    L = int(context_len)
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if n == 0 or L == 0:
        return out, lse
    i = np.asarray(positions, dtype=np.int64)[:, None]
    j = np.arange(L, dtype=np.int64)[None, :]
    admissible = np.ones((n, L), dtype=bool)
    if causal:
        admissible &= j <= (L - int(q_len) + i)
    if key_window is not None:
        lo, hi = key_window
        admissible &= (j >= lo) & (j < hi)
    scores = scale * (Qrows @ np.asarray(K, dtype=np.float64).T)   # [n, L]
    scores = np.where(admissible, scores, -np.inf)
    has_key = admissible.any(axis=1)
    m = np.where(has_key, scores.max(axis=1, initial=-np.inf), 0.0)
    p = np.where(admissible, np.exp(scores - m[:, None]), 0.0)
    denom = p.sum(axis=1)
    safe = np.where(has_key, denom, 1.0)
    out = (p @ np.asarray(V, dtype=np.float64)) / safe[:, None]
    out[~has_key] = 0.0
    lse = np.where(has_key, m + np.log(safe), -np.inf)
    return out, lse


def _checked_meta(q, k_cache, cu_seqlens_q, seqused_k, block_table):
    T, Hq, d = q.shape
    NB, B, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("head_dim of q and cache differ")
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seqused_k, dtype=np.int64)
    table = np.asarray(block_table, dtype=np.int64)
    S = L.shape[0]
    if cu.shape[0] != S + 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens_q must be non-decreasing prefix sums from 0 to total_q")
    for s in range(S):
        need = -(-int(L[s]) // B)
        if need > table.shape[1]:
            raise ValueError(f"sequence {s}: block table too short for its context")
        if need and (table[s, :need].min() < 0 or table[s, :need].max() >= NB):
            raise ValueError(f"sequence {s}: block id out of range")
    return T, Hq, d, Hkv, Hq // Hkv, cu, L, table


def paged_attention(q, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table,
                    softmax_scale, causal, key_window=None, kv_format="bf16", k_scale=1.0,
                    v_scale=1.0):
    """Whole-batch oracle.  Returns ``(out [T, Hq, d], lse [T, Hq])`` float64."""
    T, Hq, d, Hkv, G, cu, L, table = _checked_meta(q, k_cache, cu_seqlens_q,
                                                   seqused_k, block_table)
    scale = float(np.float32(softmax_scale))
    out = np.zeros((T, Hq, d), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    for s in range(L.shape[0]):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        q_len = t1 - t0
        if q_len == 0:
            continue
        K = _context(k_cache, table[s], L[s], kv_format, k_scale)
        V = _context(v_cache, table[s], L[s], kv_format, v_scale)
        positions = np.repeat(np.arange(q_len), G)          # row = (token, head in group)
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            Qrows = np.asarray(q[t0:t1, heads, :], dtype=np.float64).reshape(q_len * G, d)
            o, l = attend_rows(Qrows, positions, K[:, g, :], V[:, g, :], q_len, L[s],
                               scale, causal, key_window)
            out[t0:t1, heads, :] = o.reshape(q_len, G, d)
            lse[t0:t1, heads] = l.reshape(q_len, G)
    return out, lse


def paged_attention_rows(q, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table,
                         softmax_scale, causal, tokens, heads, kv_format="bf16", k_scale=1.0,
                         v_scale=1.0):
    """Oracle for selected (token, q-head) rows only; returns ``(out [n, d], lse [n])``."""
    T, Hq, d, Hkv, G, cu, L, table = _checked_meta(q, k_cache, cu_seqlens_q,
                                                   seqused_k, block_table)
    scale = float(np.float32(softmax_scale))
    tokens = np.asarray(tokens, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    seq_of = np.searchsorted(cu, tokens, side="right") - 1
    out = np.zeros((tokens.shape[0], d), dtype=np.float64)
    lse = np.full(tokens.shape[0], -np.inf, dtype=np.float64)
    for s in np.unique(seq_of):
        K = _context(k_cache, table[s], L[s], kv_format, k_scale)
        V = _context(v_cache, table[s], L[s], kv_format, v_scale)
        q_len = int(cu[s + 1] - cu[s])
        for g in np.unique(heads[seq_of == s] // G):
            sel = np.nonzero((seq_of == s) & (heads // G == g))[0]
            Qrows = np.asarray(q[tokens[sel], heads[sel], :], dtype=np.float64)
            o, l = attend_rows(Qrows, tokens[sel] - cu[s], K[:, g, :], V[:, g, :], q_len,
                               L[s], scale, causal)
            out[sel] = o
            lse[sel] = l
    return out, lse


def merge_lse(outs, lses):
    """Combine partial results over disjoint key sets.

    outs: ``[P, ..., d]`` each normalised over its own keys; lses: ``[P, ...]``
    natural-log sums of exponentiated scaled scores (``-inf`` for a part with no
    key).  With ``L* = max_p lse_p`` and ``w_p = exp(lse_p - L*)`` the merged
    row is ``sum_p w_p out_p / sum_p w_p`` and its lse ``L* + ln sum_p w_p``.
    A row whose parts are all empty gives 0 and ``-inf``.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    top = lses.max(axis=0)
    any_key = np.isfinite(top)
    top_safe = np.where(any_key, top, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - top_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    wsum_safe = np.where(any_key, wsum, 1.0)
    merged = (w[..., None] * outs).sum(axis=0) / wsum_safe[..., None]
    merged = np.where(any_key[..., None], merged, 0.0)
    lse = np.where(any_key, top_safe + np.log(wsum_safe), -np.inf)
    return merged, lse

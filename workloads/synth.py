"""Seeded synthetic batches for varlen paged attention.

Layouts follow the varlen, paged statement of the problem:

* ``q`` / ``out``: bf16 ``[total_q, num_q_heads, head_dim]``, the queries of all
  sequences concatenated; ``cu_seqlens_q`` (int32 ``[S+1]``) holds the offsets.
* ``k_cache`` / ``v_cache``: bf16 ``[num_blocks, block_size, num_kv_heads,
  head_dim]`` (the key-cache layout the FlashAttention backend uses, page
  "[Kernel] Unified Triton kernel that doesn't distinguish between prefill +
  decode", PR description).
* ``block_table``: int32 ``[S, max_blocks_per_seq]``; logical block ``j`` of
  sequence ``s`` lives in physical block ``block_table[s, j]``.
* ``seqused_k``: int32 ``[S]``, the context length of each sequence including
  its new tokens.

Nothing here computes attention.  Values are N(0, 1) rounded to bf16 (round to
nearest even, by torch).  Physical block ids are a seeded permutation of the
pool.  Every slot no sequence owns (the tail of a last block, unreferenced
blocks and the "trap" block that block-table padding points at) is NaN, so a
kernel that reads outside a sequence's context shows it in its output.

Seeds: ``numpy.random.SeedSequence(seed)`` spawns four children, used in this
order: lengths, sequence order, block permutation, values.

fp8 caches (``kv_dtype="fp8_e4m3fn"``): N(0, 1) draws clipped to [-6, 6],
divided by the tensor's scale and rounded to the OCP E4M3 ("fn") format by
torch; the codes are inputs like any other values, and the NaN poison is the
code 0x7F.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

BLOCK_SIZE = 16


@dataclass
class Batch:
    """One synthetic batch: device tensors plus host copies of the metadata."""

    name: str
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    cu_seqlens_q: torch.Tensor
    seqused_k: torch.Tensor
    block_table: torch.Tensor
    q_lens: np.ndarray
    k_lens: np.ndarray
    max_seqlen_q: int
    max_seqlen_k: int
    softmax_scale: float
    causal: bool
    trap_block: int
    seed: int
    kv_format: str = "bf16"          # "f16", or "fp8_e4m3fn" (one-byte codes)
    k_scale: float = 1.0             # fp8: a key code stands for decode(code) * k_scale
    v_scale: float = 1.0
    extra: Dict[str, object] = field(default_factory=dict)

    # ---- shape helpers -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def block_size(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    def new_out(self) -> torch.Tensor:
        return torch.empty_like(self.q)

    def args(self, out: torch.Tensor):
        """Positional arguments in the order of ``unified_attention``."""
        return (self.q, self.k_cache, self.v_cache, out, self.cu_seqlens_q,
                self.seqused_k, self.block_table, self.max_seqlen_q,
                self.max_seqlen_k, self.softmax_scale, self.causal)

    # ---- host copies for the oracle -------------------------------------
    def _cache_host(self, t: torch.Tensor) -> np.ndarray:
        # 16-bit: values as float32 (exact); fp8: the raw one-byte codes
        if self.kv_format != "fp8_e4m3fn":
            return t.float().cpu().numpy()
        return t.view(torch.uint8).cpu().numpy()

    def kv_kwargs(self) -> Dict[str, object]:
        """Cache format arguments of the oracle."""
        return dict(kv_format=self.kv_format, k_scale=self.k_scale, v_scale=self.v_scale)

    def host(self) -> Dict[str, object]:
        """Whole batch as numpy arrays (values as float32, exact for bf16;
        fp8 caches as their uint8 codes)."""
        return dict(
            q=self.q.float().cpu().numpy(),
            k_cache=self._cache_host(self.k_cache),
            v_cache=self._cache_host(self.v_cache),
            cu_seqlens_q=self.cu_seqlens_q.cpu().numpy().astype(np.int64),
            seqused_k=self.seqused_k.cpu().numpy().astype(np.int64),
            block_table=self.block_table.cpu().numpy().astype(np.int64),
            softmax_scale=self.softmax_scale,
            causal=self.causal,
            **self.kv_kwargs(),
        )

    def host_subset(self, seq_ids: Sequence[int]) -> Tuple[Dict[str, object], np.ndarray]:
        """Host copy of only the listed sequences, their blocks copied into a
        compact pool (ids renumbered).  Returns the arrays and, for each token
        of the subset, its row in the full batch's ``q``/``out``."""
        seq_ids = [int(s) for s in seq_ids]
        cu = self.cu_seqlens_q.cpu().numpy().astype(np.int64)
        table = self.block_table.cpu().numpy().astype(np.int64)
        rows, blocks, new_tables = [], [], []
        base = 0
        for s in seq_ids:
            lo, hi = int(cu[s]), int(cu[s + 1])
            rows.append(np.arange(lo, hi, dtype=np.int64))
            nblk = -(-int(self.k_lens[s]) // self.block_size)
            blocks.append(table[s, :nblk])
            new_tables.append(np.arange(base, base + nblk, dtype=np.int64))
            base += nblk
        rows_all = np.concatenate(rows) if rows else np.zeros(0, np.int64)
        phys_all = np.concatenate(blocks) if blocks else np.zeros(0, np.int64)
        idx = torch.as_tensor(phys_all, device=self.k_cache.device, dtype=torch.long)
        ridx = torch.as_tensor(rows_all, device=self.q.device, dtype=torch.long)
        mb = max([len(t) for t in new_tables] + [1])
        tab = np.zeros((len(seq_ids), mb), dtype=np.int64)
        for i, t in enumerate(new_tables):
            tab[i, :len(t)] = t
        q_lens = self.q_lens[seq_ids].astype(np.int64)
        sub = dict(
            q=self.q.index_select(0, ridx).float().cpu().numpy(),
            k_cache=self._cache_host(_rows(self.k_cache, idx)),
            v_cache=self._cache_host(_rows(self.v_cache, idx)),
            cu_seqlens_q=np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64),
            seqused_k=self.k_lens[seq_ids].astype(np.int64),
            block_table=tab,
            softmax_scale=self.softmax_scale,
            causal=self.causal,
            **self.kv_kwargs(),
        )
        return sub, rows_all

    def to(self, device) -> "Batch":
        b = Batch(**{**self.__dict__})
        for name in ("q", "k_cache", "v_cache", "cu_seqlens_q", "seqused_k", "block_table"):
            setattr(b, name, getattr(self, name).to(device))
        return b


def _rows(t: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """t[idx] along dim 0 (through a uint8 view for fp8 tensors)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).index_select(0, idx).view(torch.float8_e4m3fn)
    return t.index_select(0, idx)


def _fill_normal_fp8(shape, gen: torch.Generator, device, scale: float,
                     chunk: int = 1 << 26) -> torch.Tensor:
    """N(0,1) float32 draws clipped to [-6, 6], divided by scale and rounded
    to E4M3 ("fn") codes by torch.  torch turns magnitudes past the format's
    range into NaN, so scale must be at least 6 / 448."""
    if scale < 6.0 / 448.0:
        raise ValueError("fp8 scale below 6/448 would overflow E4M3")
    out = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        x = torch.randn(hi - lo, generator=gen, device=device,
                        dtype=torch.float32).clamp_(-6.0, 6.0) / scale
        flat[lo:hi] = x.to(torch.float8_e4m3fn)
    return out


_TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def _fill_normal_bf16(shape, gen: torch.Generator, device, chunk: int = 1 << 26,
                      dtype: str = "bf16") -> torch.Tensor:
    """N(0,1) float32 draws rounded (to nearest even) to bf16 or fp16,
    produced in chunks to bound memory."""
    tdt = _TORCH16[dtype]
    out = torch.empty(shape, dtype=tdt, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        flat[lo:hi] = torch.randn(hi - lo, generator=gen, device=device,
                                  dtype=torch.float32).to(tdt)
    return out


def build_batch(name: str, q_lens, k_lens, num_q_heads: int, num_kv_heads: int,
                head_dim: int, causal: bool, seed: int, device="cpu",
                block_size: int = BLOCK_SIZE, pool_blocks: Optional[int] = None,
                poison: bool = True, softmax_scale: Optional[float] = None,
                children=None, kv_dtype: str = "bf16", k_scale: float = 1.0,
                v_scale: float = 1.0, q_dtype: Optional[str] = None) -> Batch:
    """Build a batch from explicit per-sequence query and context lengths.

    ``pool_blocks`` fixes the pool size; by default the pool holds exactly the
    blocks the sequences need plus one trap block.  ``kv_dtype`` is "bf16",
    "f16" or "fp8_e4m3fn" (then ``k_scale`` / ``v_scale`` are the per-tensor
    scales).  ``q_dtype`` ("bf16" or "f16") defaults to the cache's 16-bit
    type, or bf16 next to an fp8 cache; q and a 16-bit cache share one type.
    """
    if kv_dtype not in ("bf16", "f16", "fp8_e4m3fn"):
        raise ValueError("kv_dtype must be bf16, f16 or fp8_e4m3fn")
    if q_dtype is None:
        q_dtype = kv_dtype if kv_dtype != "fp8_e4m3fn" else "bf16"
    if q_dtype not in _TORCH16 or (kv_dtype != "fp8_e4m3fn" and q_dtype != kv_dtype):
        raise ValueError("q_dtype must be bf16 or f16, the same as a 16-bit cache")
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    assert q_lens.shape == k_lens.shape and q_lens.ndim == 1
    if children is None:
        children = np.random.SeedSequence(seed).spawn(4)
    S = int(q_lens.shape[0])
    B = int(block_size)
    nblk = -(-k_lens // B)
    used = int(nblk.sum())
    pool = int(pool_blocks) if pool_blocks is not None else used + 1
    if pool < used + 1:
        raise ValueError(f"pool of {pool} blocks cannot hold {used} blocks plus a trap block")
    perm = np.random.default_rng(children[2]).permutation(pool)
    trap = int(perm[used])
    max_k = int(k_lens.max()) if S else 0
    max_q = int(q_lens.max()) if S else 0
    mb = max(1, -(-max_k // B))
    table = np.full((S, mb), trap, dtype=np.int64)
    off = 0
    owned = np.zeros((pool, B), dtype=bool)
    for s in range(S):
        n = int(nblk[s])
        phys = perm[off:off + n]
        table[s, :n] = phys
        off += n
        if n:
            owned[phys[:-1], :] = True
            tail = int(k_lens[s]) - (n - 1) * B
            owned[phys[-1], :tail] = True
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    T = int(cu[-1])

    vseed = int(np.random.default_rng(children[3]).integers(0, 2**62))
    gen = torch.Generator(device=device)
    gen.manual_seed(vseed)
    q = _fill_normal_bf16((T, num_q_heads, head_dim), gen, device, dtype=q_dtype)
    if kv_dtype != "fp8_e4m3fn":
        k_cache = _fill_normal_bf16((pool, B, num_kv_heads, head_dim), gen, device, dtype=kv_dtype)
        v_cache = _fill_normal_bf16((pool, B, num_kv_heads, head_dim), gen, device, dtype=kv_dtype)
    else:
        k_scale = float(np.float32(k_scale))
        v_scale = float(np.float32(v_scale))
        k_cache = _fill_normal_fp8((pool, B, num_kv_heads, head_dim), gen, device, k_scale)
        v_cache = _fill_normal_fp8((pool, B, num_kv_heads, head_dim), gen, device, v_scale)
    if poison:
        not_owned = torch.as_tensor(~owned, device=device)
        if kv_dtype != "fp8_e4m3fn":
            k_cache[not_owned] = float("nan")
            v_cache[not_owned] = float("nan")
        else:
            k_cache.view(torch.uint8)[not_owned] = 0x7F     # E4M3 ("fn") NaN
            v_cache.view(torch.uint8)[not_owned] = 0x7F

    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    i32 = dict(dtype=torch.int32, device=device)
    return Batch(
        name=name, q=q, k_cache=k_cache, v_cache=v_cache,
        cu_seqlens_q=torch.as_tensor(cu, **i32),
        seqused_k=torch.as_tensor(k_lens, **i32),
        block_table=torch.as_tensor(table, **i32),
        q_lens=q_lens, k_lens=k_lens, max_seqlen_q=max_q, max_seqlen_k=max_k,
        softmax_scale=float(softmax_scale), causal=bool(causal), trap_block=trap,
        seed=int(seed), kv_format=kv_dtype,
        k_scale=float(k_scale) if kv_dtype == "fp8_e4m3fn" else 1.0,
        v_scale=float(v_scale) if kv_dtype == "fp8_e4m3fn" else 1.0)


def repermute_pool(batch: Batch, seed: int) -> Batch:
    """Same logical K/V under a different physical placement: physical id p
    becomes sigma[p] for a seeded permutation sigma of the pool."""
    sigma = np.random.default_rng(seed).permutation(batch.num_blocks)
    sig = torch.as_tensor(sigma, dtype=torch.long, device=batch.k_cache.device)
    k_new = torch.empty_like(batch.k_cache)
    v_new = torch.empty_like(batch.v_cache)
    if batch.k_cache.dtype == torch.float8_e4m3fn:
        k_new.view(torch.uint8)[sig] = batch.k_cache.view(torch.uint8)
        v_new.view(torch.uint8)[sig] = batch.v_cache.view(torch.uint8)
    else:
        k_new[sig] = batch.k_cache
        v_new[sig] = batch.v_cache
    table = batch.block_table.cpu().numpy().astype(np.int64)
    new_table = sigma[table].astype(np.int32)
    b = Batch(**{**batch.__dict__})
    b.k_cache, b.v_cache = k_new, v_new
    b.block_table = torch.as_tensor(new_table, device=batch.block_table.device)
    b.trap_block = int(sigma[batch.trap_block])
    return b


# ---------------------------------------------------------------------------
# The named workloads.  Shapes follow the serving scenarios the pages measure
# (Llama-3.1-8B with 32 q-heads / 8 kv-heads / head_dim 128; one GPU's share of
# Llama-3.1-70B at TP=2 with 32 q-heads / 4 kv-heads), as synthetic stand-ins:
# no dataset or weights are used.
# ---------------------------------------------------------------------------

WORKLOADS = {
    # name: (seed, Hq, Hkv, d, causal)
    "tiny_mixed_3seq": (1, 4, 2, 64, True),
    "decode_256seq_ctx1k": (2, 32, 8, 128, True),
    "mixed_prefill512x8_decode248": (3, 32, 8, 128, True),
    "prefill512x8_only": (3, 32, 8, 128, True),
    # the same prefill chunks at head sizes 96 and 256 (these sizes run
    # prefill on narrow tiles)
    "prefill512x8_only_d96": (3, 32, 8, 96, True),
    "prefill512x8_only_d256": (3, 32, 8, 256, True),
    "decode248_only": (3, 32, 8, 128, True),
    "decode_gqa8_64seq_ctx2k_4k": (4, 32, 4, 128, True),
    "long_decode_16seq_ctx32k_128k": (5, 32, 8, 128, True),
    "long_q16_noncausal_16seq_ctx32k_128k": (5, 32, 8, 128, False),
    # the headline decode batch with an fp8 E4M3 cache (scales 1/64)
    "decode_256seq_ctx1k_fp8": (2, 32, 8, 128, True),
}

# cache format and scales of the workloads that do not use bf16 caches
WORKLOAD_KV = {
    "decode_256seq_ctx1k_fp8": ("fp8_e4m3fn", 1.0 / 64, 1.0 / 64),
}


def workload_lengths(name: str, children) -> Tuple[np.ndarray, np.ndarray, Optional[int]]:
    """Per-sequence (query lengths, context lengths, fixed pool size or None)."""
    rng_len = np.random.default_rng(children[0])
    rng_ord = np.random.default_rng(children[1])
    if name == "tiny_mixed_3seq":
        return np.array([1, 5, 16]), np.array([7, 20, 40]), 16
    if name in ("decode_256seq_ctx1k", "decode_256seq_ctx1k_fp8"):
        L = rng_len.integers(1000, 1100, size=256, endpoint=True)
        return np.ones(256, np.int64), L, None
    if name in ("mixed_prefill512x8_decode248", "prefill512x8_only", "decode248_only",
                "prefill512x8_only_d96", "prefill512x8_only_d256"):
        prefix = rng_len.integers(0, 1536, size=8, endpoint=True)
        Lp = prefix + 512
        Ld = np.clip(np.round(np.exp(rng_len.normal(math.log(400.0), 1.0, size=248))), 4, 8192)
        Ld = Ld.astype(np.int64)
        qs = np.concatenate([np.full(8, 512), np.ones(248, np.int64)])
        ks = np.concatenate([Lp, Ld])
        order = rng_ord.permutation(256)
        qs, ks = qs[order], ks[order]
        if name.startswith("prefill512x8_only"):
            keep = qs > 1
            return qs[keep], ks[keep], None
        if name == "decode248_only":
            keep = qs == 1
            return qs[keep], ks[keep], None
        return qs, ks, None
    if name == "decode_gqa8_64seq_ctx2k_4k":
        L = rng_len.integers(2048, 4096, size=64, endpoint=True)
        return np.ones(64, np.int64), L, None
    if name in ("long_decode_16seq_ctx32k_128k", "long_q16_noncausal_16seq_ctx32k_128k"):
        L = rng_len.integers(32768, 131072, size=16, endpoint=True)
        q = 1 if name.startswith("long_decode") else 16
        return np.full(16, q, np.int64), L, None
    raise KeyError(name)


def make_workload(name: str, device="cpu", poison: bool = True) -> Batch:
    seed, hq, hkv, d, causal = WORKLOADS[name]
    children = np.random.SeedSequence(seed).spawn(4)
    q_lens, k_lens, pool = workload_lengths(name, children)
    kv, ks, vs = WORKLOAD_KV.get(name, ("bf16", 1.0, 1.0))
    return build_batch(name, q_lens, k_lens, hq, hkv, d, causal, seed, device=device,
                       pool_blocks=pool, poison=poison, children=children, kv_dtype=kv,
                       k_scale=ks, v_scale=vs)

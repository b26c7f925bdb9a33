"""CPU models of how the HIP kernels divide a batch into work (test
infrastructure; no GPU).

Each model replays, in plain Python, the integer bookkeeping one kernel does
on the device — which wave or work-group takes which (sequence, key range,
kv-head), which block-table entries it reads, which cache blocks its loads
touch (ring refills included) and which workspace rows it writes — from the
same plan the host library picks (``pa_plan_describe``).  The tests check the
replay for exact coverage and for every bound the kernels rely on.  The models
mirror ``pa_kernels.hip`` step by step; a change to the kernels' enumeration
must be made here too.

Constants are those of ``pa_internal.h``.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

SUB = 16                 # keys of a sub-block (kBlockSize)
STAGE = 64               # keys of a wide-path stage (kStageKeys)
MAX_ITEM_BLOCKS = 256    # persistent decode: block ids per item (kMaxSplitKeys / 16)
MAX_SPLIT_KEYS = 4096
NARROW_ROWS = 16
WIDE_OFFS_ENTRIES = MAX_SPLIT_KEYS // SUB + 4
INT32_MAX = 2 ** 31 - 1


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Batch:
    q_lens: List[int]
    k_lens: List[int]          # seqused_k as passed (may exceed max_k: clamped on the device)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int            # 16, 32 or 64
    max_k: int
    causal: bool = True

    @property
    def S(self):
        return len(self.q_lens)

    @property
    def G(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def T(self):
        return int(sum(self.q_lens))

    @property
    def cu(self):
        return [0] + list(np.cumsum(self.q_lens).astype(int))

    def L(self, s):
        """context_len(): seqused_k clamped to [0, max_seqlen_k]"""
        return min(max(int(self.k_lens[s]), 0), self.max_k)

    def bt_index(self, j):
        """block-table column read for 16-key sub-block j (sub_block_id)"""
        return j >> {16: 0, 32: 1, 64: 2}[self.block_size]


@dataclass
class Item:
    """One unit of streamed work as a kernel sees it."""
    s: int
    kvh: int
    sigma: int
    parts: int
    blk0: int              # first 16-key sub-block
    nb: int                # sub-blocks streamed
    kbeg: int
    kend: int
    rows: int              # packed rows of the tile (tokens x G)
    tok0: int              # first token (absolute) of the tile
    n_tok: int
    who: Tuple[int, ...] = ()


@dataclass
class Trace:
    items: List[Item] = field(default_factory=list)
    bt_reads: List[Tuple[int, int]] = field(default_factory=list)      # (s, column)
    live_loads: List[Tuple[int, int, int]] = field(default_factory=list)  # (s, sub-block, kvh)
    ws_rows: List[int] = field(default_factory=list)                   # workspace row indices
    max_stream_pos: int = 0


# ---------------------------------------------------------------------------
# pa_decode_kernel: persistent decode (fixed parts or even split)
# ---------------------------------------------------------------------------
def decode_kernel(b: Batch, plan: Dict, ring: int = 2) -> Trace:
    S, Hkv, G = b.S, b.num_kv_heads, b.G
    nwg = int(plan["num_workgroups"])
    assert nwg % 8 == 0
    balanced = bool(plan["balanced"])
    target = int(plan["split_keys"])
    n_split = int(plan["num_splits"])
    q0t = b.cu
    lent = [b.L(s) for s in range(S)]

    def seq_units(s):
        ql = q0t[s + 1] - q0t[s]
        if balanced:
            return max(cdiv(lent[s], SUB), 1) if ql > 0 else 0
        if ql <= 0:
            return 0
        return min(max(cdiv(lent[s], target), 1), n_split)

    pref = [0]
    for s in range(S):
        pref.append(pref[-1] + seq_units(s))
    n_units = pref[S] * (1 if balanced else Hkv)
    workers = nwg * 4
    chunk, n_pairs = 1, 0
    slots = [0] * (S + 1)
    if balanced:
        all_ = n_units * Hkv
        cap = workers * MAX_ITEM_BLOCKS
        kpw = max(1, cdiv(all_, cap))
        chunk = max(cdiv(all_, workers * kpw), target // SUB)
        n_pairs = cdiv(n_units, chunk) * Hkv
        # compact partial slots: one per chunk a sequence touches
        for s in range(S):
            x0, x1 = pref[s], pref[s + 1]
            slots[s + 1] = slots[s] + ((x1 - 1) // chunk - x0 // chunk + 1 if x1 > x0 else 0)
    tq = int(plan["tile_tokens"])
    n_items = 0 if balanced else n_units
    per_xcd = (n_items + 7) >> 3
    wpx = (nwg >> 3) * 4

    def largest_le(x):
        lo, hi = 0, S - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if pref[mid] <= x:
                lo = mid
            else:
                hi = mid - 1
        return lo

    tr = Trace()

    for blk in range(nwg):
        xcd = blk & 7
        range_end = min(n_items, (xcd + 1) * per_xcd)
        for wave in range(4):
            item0 = xcd * per_xcd + (blk >> 3) * 4 + wave
            gw = xcd * wpx + (blk >> 3) * 4 + wave

            def item_at(m):
                it = item0 + m * wpx
                return it if it < range_end else n_items

            def describe(q, pos):
                if not balanced:
                    item = item_at(pos)
                    d = dict(valid=item < n_items, s=0, kvh=0, sigma=0, units=0, q0=0, q_len=0,
                             L=0, kbeg=0, kend=0, blk0=0, nb=0, c=0, next=pos + 1)
                    if not d["valid"]:
                        return d
                    unit = item // Hkv
                    s = largest_le(unit)
                    L = lent[s]
                    d.update(s=s, kvh=item - unit * Hkv, sigma=unit - pref[s],
                             units=pref[s + 1] - pref[s], q0=q0t[s], q_len=q0t[s + 1] - q0t[s],
                             L=L)
                    d["kbeg"] = d["sigma"] * target
                    d["kend"] = max(0, min(L, d["kbeg"] + target))
                    d["blk0"] = d["kbeg"] // SUB
                    d["nb"] = cdiv(d["kend"], SUB) - d["blk0"] if d["kend"] > d["kbeg"] else 0
                    return d
                d = dict(valid=q < n_pairs, s=0, kvh=0, sigma=0, units=0, q0=0, q_len=0, L=0,
                         kbeg=0, kend=0, blk0=0, nb=0, c=0, next=0)
                if not d["valid"]:
                    return d
                c = q // Hkv
                xe = min((c + 1) * chunk, n_units)
                s = largest_le(pos)
                L = lent[s]
                nbe = max(cdiv(L, SUB), 1)
                x0 = pref[s]
                b0 = pos - x0
                b1 = min(nbe, b0 + (xe - pos))
                d.update(slot=slots[s] + c - x0 // chunk)
                d.update(s=s, kvh=q - c * Hkv, sigma=c - x0 // chunk,
                         units=(x0 + nbe - 1) // chunk - x0 // chunk + 1, q0=q0t[s],
                         q_len=q0t[s + 1] - q0t[s], L=L, kbeg=b0 * SUB,
                         kend=max(0, min(L, b1 * SUB)), blk0=b0, c=q, next=pos + (b1 - b0))
                d["nb"] = cdiv(d["kend"], SUB) - b0 if d["kend"] > d["kbeg"] else 0
                tr.max_stream_pos = max(tr.max_stream_pos, pos, d["next"], xe,
                                        (q // Hkv + 1) * chunk)
                return d

            def after(d):
                if not d["valid"]:
                    return d
                if not balanced:
                    return describe(0, d["next"])
                q, pos = d["c"], d["next"]
                if pos >= min((q // Hkv + 1) * chunk, n_units):
                    q += workers
                    if q >= n_pairs:
                        return describe(q, 0)
                    pos = (q // Hkv) * chunk
                return describe(q, pos)

            if (gw >= n_pairs) if balanced else (item_at(0) >= n_items):
                continue
            cur = describe(gw, (gw // Hkv) * chunk) if balanced else describe(0, 0)
            nxt = after(cur)
            for d in (cur, nxt):          # block ids of the first two items (load_ids)
                if d["valid"]:
                    for i in range(d["nb"]):
                        tr.bt_reads.append((d["s"], b.bt_index(d["blk0"] + i)))
            nx2 = after(nxt)
            if nx2["valid"]:
                for i in range(nx2["nb"]):
                    tr.bt_reads.append((nx2["s"], b.bt_index(nx2["blk0"] + i)))
            # the ring's first loads
            for j in range(ring):
                if cur["nb"] > j:
                    tr.live_loads.append((cur["s"], cur["blk0"] + j, cur["kvh"]))
            while True:
                assert cur["valid"]
                nbp = max(ring, cdiv(cur["nb"], ring) * ring)
                for i in range(0, nbp, ring):
                    for j in range(ring):
                        t = i + j + ring
                        in_cur = t < cur["nb"]
                        in_nxt = (not in_cur) and t >= nbp and t - nbp < nxt["nb"]
                        if in_cur:
                            tr.live_loads.append((cur["s"], cur["blk0"] + t, cur["kvh"]))
                        elif in_nxt:
                            tr.live_loads.append((nxt["s"], nxt["blk0"] + t - nbp, nxt["kvh"]))
                rows = cur["q_len"] * G
                tr.items.append(Item(cur["s"], cur["kvh"], cur["sigma"], cur["units"], cur["blk0"],
                                     cur["nb"], cur["kbeg"], cur["kend"], rows, cur["q0"],
                                     cur["q_len"], (blk, wave)))
                if cur["units"] > 1:
                    for r in range(min(rows, NARROW_ROWS)):
                        if r // G >= tq:
                            continue
                        tok = cur["q0"] + r // G
                        hn = cur["kvh"] * G + r % G
                        if balanced:
                            tr.ws_rows.append((cur["slot"] * tq + r // G) * b.num_q_heads + hn)
                        else:
                            tr.ws_rows.append((cur["sigma"] * b.T + tok) * b.num_q_heads + hn)
                if not nxt["valid"]:
                    break
                cur, nxt = nxt, nx2
                nx2 = after(nxt)
                if nx2["valid"]:
                    for i in range(nx2["nb"]):
                        tr.bt_reads.append((nx2["s"], b.bt_index(nx2["blk0"] + i)))
    return tr


# ---------------------------------------------------------------------------
# pa_fwd_kernel: the grid kernel (index order, or longest-first order)
# ---------------------------------------------------------------------------
def unit_stages(b: Batch, plan: Dict, q_len: int, L: int, tile: int, sigma: int) -> int:
    Tq, sk = int(plan["tile_tokens"]), int(plan["split_keys"])
    tok0 = tile * Tq
    n_tok = min(Tq, q_len - tok0)
    k_need = min(L, L - q_len + tok0 + n_tok) if b.causal else L
    kbeg = sigma * sk
    kend = min(k_need, kbeg + sk)
    return cdiv(kend - kbeg, STAGE) if kend > kbeg else 0


def rank_order(b: Batch, plan: Dict, lpt_units: int) -> List[Tuple[int, int, int]]:
    """pa_rank_kernel: the (s, tile, sigma) of every rank (-1 past the last)."""
    Tq, sk, n_split = int(plan["tile_tokens"]), int(plan["split_keys"]), int(plan["num_splits"])
    units = []
    for s in range(b.S):
        q, L = b.q_lens[s], b.L(s)
        parts = min(max(cdiv(L, sk), 1), n_split)
        nt = cdiv(q, Tq)
        for j in range(nt * parts):
            tile, sg = j % nt, j // nt
            units.append((unit_stages(b, plan, q, L, tile, sg), s, tile, sg))
    assert len(units) <= lpt_units, "more units than order entries"
    assert all(0 <= u[0] <= 64 for u in units), "stage count outside the histogram"
    # ranks by decreasing stage count; ties in any order
    units.sort(key=lambda u: -u[0])
    order = [(s, t, g) for _, s, t, g in units]
    return order + [(-1, 0, 0)] * (lpt_units - len(order))


def fwd_kernel(b: Batch, plan: Dict) -> Trace:
    S, Hkv, G = b.S, b.num_kv_heads, b.G
    Tq, sk, n_split = int(plan["tile_tokens"]), int(plan["split_keys"]), int(plan["num_splits"])
    nwg = int(plan["num_workgroups"])
    lpt = bool(plan["longest_first"])
    num_slots = int(plan["num_slots"])
    cu = b.cu
    tr = Trace()
    lpt_units = num_slots * n_split
    order = rank_order(b, plan, lpt_units) if lpt else None
    num_items = num_slots * Hkv * n_split
    items_per_xcd = nwg // 8
    kv_major = Tq * G > NARROW_ROWS          # wide plans number items kv-head major
    for blk in range(nwg):
        if lpt:
            if plan.get("unit_xcd"):
                # a unit's kv-heads on consecutive blocks of one XCD
                j = blk >> 3
                r, kvh = (j // Hkv) * 8 + (blk & 7), j % Hkv
            else:
                r, kvh = blk // Hkv, blk % Hkv
            if r >= lpt_units:
                continue
            s, tile, sigma = order[r]
            if s < 0:
                continue
        else:
            item = (blk & 7) * items_per_xcd + (blk >> 3)
            if item >= num_items:
                continue
            sigma = item % n_split
            rest = item // n_split
            if kv_major:
                slot, kvh = rest % num_slots, rest // num_slots
            else:
                kvh, slot = rest % Hkv, rest // Hkv
            if plan["slots_direct"]:
                s, tile = slot, 0
            else:
                lo, hi = 0, S - 1
                while lo < hi:
                    mid = (lo + hi + 1) >> 1
                    if cu[mid] // Tq + mid <= slot:
                        lo = mid
                    else:
                        hi = mid - 1
                s, tile = lo, slot - (cu[lo] // Tq + lo)
        # fill_item
        q0, q_len = cu[s], cu[s + 1] - cu[s]
        tok0 = tile * Tq
        if tok0 >= q_len:
            continue
        n_tok = min(Tq, q_len - tok0)
        rows = n_tok * G
        L = b.L(s)
        parts = min(max(cdiv(L, sk), 1), n_split)
        if sigma >= parts:
            continue
        diag = L - q_len
        k_need = min(L, diag + tok0 + n_tok) if b.causal else L
        kbeg = sigma * sk
        kend = min(k_need, kbeg + sk)
        blk0 = kbeg // SUB
        nblk = cdiv(kend, SUB) - blk0 if kend > kbeg else 0
        it = Item(s, kvh, sigma, parts, blk0, nblk, kbeg, kend, rows, q0 + tok0, n_tok, (blk,))
        tr.items.append(it)
        for i in range(nblk):
            tr.bt_reads.append((s, b.bt_index(blk0 + i)))
            tr.live_loads.append((s, blk0 + i, kvh))
        if rows > NARROW_ROWS:
            n_stage = cdiv(kend - kbeg, STAGE) if kend > kbeg else 0
            assert 4 * n_stage + 4 <= WIDE_OFFS_ENTRIES, "wide path: offset table overflow"
        else:
            nb_wave = cdiv(nblk, 4)
            assert nb_wave <= 64, "narrow path: a wave's block ids exceed one VGPR"
        if parts > 1:
            for r in range(rows):
                tok = q0 + tok0 + r // G
                hn = kvh * G + r % G
                tr.ws_rows.append((sigma * b.T + tok) * b.num_q_heads + hn)
    return tr


# ---------------------------------------------------------------------------
# checks shared by both kernels
# ---------------------------------------------------------------------------
def check_trace(b: Batch, plan: Dict, tr: Trace) -> None:
    """Exact coverage and every bound; raises AssertionError on a violation."""
    G, Hq, T = b.G, b.num_q_heads, b.T
    n_split = int(plan["num_splits"])
    persistent = bool(plan["persistent"])
    # every (sequence, kv-head) with queries: parts 0..units-1 exactly once, and
    # every 16-key sub-block of its admissible keys exactly once per query tile
    by_row: Dict[Tuple[int, int, int], List[Item]] = {}
    for it in tr.items:
        by_row.setdefault((it.s, it.kvh, it.tok0 - b.cu[it.s] if not persistent else 0), []).append(it)
    Tq = int(plan["tile_tokens"])
    for s in range(b.S):
        ql, L = b.q_lens[s], b.L(s)
        if ql == 0:
            continue
        tiles = [0] if persistent else list(range(0, ql, Tq))
        for kvh in range(b.num_kv_heads):
            for t0 in tiles:
                its = by_row.get((s, kvh, t0), [])
                assert its, f"sequence {s} kv-head {kvh} tile {t0}: no item"
                parts = {it.parts for it in its}
                assert len(parts) == 1, f"sequence {s}: items disagree on the part count"
                n = parts.pop()
                assert 1 <= n <= n_split, f"sequence {s}: {n} parts, bound {n_split}"
                assert sorted(it.sigma for it in its) == list(range(n)), \
                    f"sequence {s} kv-head {kvh}: parts {sorted(it.sigma for it in its)}"
                n_tok = min(Tq, ql - t0) if not persistent else ql
                need = (min(L, L - ql + t0 + n_tok) if b.causal else L) if not persistent else L
                got = sorted(j for it in its for j in range(it.blk0, it.blk0 + it.nb))
                assert got == list(range(cdiv(need, SUB))), \
                    f"sequence {s} kv-head {kvh} tile {t0}: sub-blocks not covered exactly once"
                for it in its:
                    assert it.kend <= L and it.kbeg <= max(it.kend, it.kbeg)
                    if persistent:
                        assert it.nb <= MAX_ITEM_BLOCKS, "item longer than its block-id table"
    # block-table reads only within ceil(L / B) columns
    for s, col in tr.bt_reads:
        assert 0 <= col < cdiv(b.L(s), b.block_size), f"sequence {s}: reads block-table column {col}"
    for s, j, kvh in tr.live_loads:
        assert 0 <= j < cdiv(b.L(s), SUB) and 0 <= kvh < b.num_kv_heads, \
            f"live load of sequence {s} sub-block {j} kv-head {kvh}"
    # workspace rows inside the partials the host sized, each written once
    bound = int(plan["partial_rows"])
    for r in tr.ws_rows:
        assert 0 <= r < bound, f"workspace row {r} past {bound}"
    assert len(set(tr.ws_rows)) == len(tr.ws_rows), "two parts write one partial row"
    assert tr.max_stream_pos <= INT32_MAX

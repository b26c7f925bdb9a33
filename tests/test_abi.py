"""C-ABI tests that need no GPU: the library loads, exports every function
include/pa.h declares, and rejects every invalid descriptor with the right
status before touching the device.  Descriptors here point at host memory,
which validation never dereferences."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import paged_kv_cache_unified_amd as pa
from workloads import build_batch, make_workload

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert "pa_unified_attention" in names and "pa_unified_attention_ex" in names
    for n in names:
        assert hasattr(pa.lib, n), f"libpa.so does not export {n}"
    assert set(names) == set(pa._SIGNATURES), "binding and header disagree"


def test_version_and_status_strings():
    import __graft_entry__
    assert pa.version() == __graft_entry__.header_version() == 6
    for code in range(-9, 1):
        assert pa.lib.pa_status_string(code).decode()
    assert pa.lib.pa_status_string(-100).decode() == "unknown status"


def cpu_args(**over):
    b = build_batch("abi", [1, 3, 2], [5, 17, 40], 8, 2, 128, True, seed=1)
    a = dict(q=b.q, k_cache=b.k_cache, v_cache=b.v_cache, out=torch.empty_like(b.q),
             cu_seqlens_q=b.cu_seqlens_q, seqused_k=b.seqused_k, block_table=b.block_table,
             max_seqlen_q=b.max_seqlen_q, max_seqlen_k=b.max_seqlen_k,
             softmax_scale=b.softmax_scale, causal=True)
    a.update(over)
    return a


def call(a, opts=None):
    ds = [pa.describe(a[n]) for n in ("q", "k_cache", "v_cache", "out", "cu_seqlens_q",
                                       "seqused_k", "block_table")]
    refs = [ctypes.byref(d) for d in ds]
    if opts is None:
        return pa.lib.pa_unified_attention(*refs, a["max_seqlen_q"], a["max_seqlen_k"],
                                           a["softmax_scale"], int(a["causal"]), None)
    return pa.lib.pa_unified_attention_ex(*refs, a["max_seqlen_q"], a["max_seqlen_k"],
                                          a["softmax_scale"], int(a["causal"]),
                                          ctypes.byref(opts), None, 0, None)


def status_of(**over):
    rc = call(cpu_args(**over))
    return pa.STATUS[rc], pa.lib.pa_last_error().decode()


def test_null_descriptor():
    a = cpu_args()
    ds = [pa.describe(a[n]) for n in ("q", "k_cache", "v_cache", "out", "cu_seqlens_q",
                                       "seqused_k", "block_table")]
    refs = [ctypes.byref(d) for d in ds]
    refs[2] = None
    rc = pa.lib.pa_unified_attention(*refs, 3, 40, 0.1, 1, None)
    assert pa.STATUS[rc] == "PA_ERR_NULL"


@pytest.mark.parametrize("over,expect", [
    (dict(q=torch.zeros(6, 8, 128, dtype=torch.float16)), "PA_ERR_DTYPE"),
    (dict(cu_seqlens_q=torch.tensor([0, 1, 4, 6], dtype=torch.int64)), "PA_ERR_DTYPE"),
    (dict(out=torch.zeros(6, 8, 128, dtype=torch.float32)), "PA_ERR_DTYPE"),
    (dict(q=torch.zeros(6, 8, 128, 1, dtype=torch.bfloat16)), "PA_ERR_SHAPE"),
    (dict(out=torch.zeros(7, 8, 128, dtype=torch.bfloat16)), "PA_ERR_SHAPE"),
    (dict(cu_seqlens_q=torch.tensor([0, 1, 6], dtype=torch.int32)), "PA_ERR_SHAPE"),
    (dict(block_table=torch.zeros(2, 3, dtype=torch.int32)), "PA_ERR_SHAPE"),
    (dict(max_seqlen_k=10_000), "PA_ERR_SHAPE"),
    (dict(max_seqlen_q=-1), "PA_ERR_SHAPE"),
])
def test_shape_and_dtype_errors(over, expect):
    st, msg = status_of(**over)
    assert st == expect, msg
    assert msg


def test_head_ratio_and_unsupported():
    b = cpu_args()
    # Hq not a multiple of Hkv (= 2)
    q = torch.zeros(6, 5, 128, dtype=torch.bfloat16)
    assert status_of(q=q, out=torch.zeros_like(q))[0] == "PA_ERR_SHAPE"
    # G = 3 is a valid ratio but not built
    k = torch.zeros(b["k_cache"].shape[0], 16, 2, 128, dtype=torch.bfloat16)
    q = torch.zeros(6, 6, 128, dtype=torch.bfloat16)
    assert status_of(q=q, out=torch.zeros_like(q), k_cache=k, v_cache=k.clone())[0] == "PA_ERR_UNSUPPORTED"
    # head sizes 64, 96, 128, 256 are built (no eight-wave tiles at 96 and
    # 256), others are not
    q = torch.zeros(6, 8, 32, dtype=torch.bfloat16)
    k = torch.zeros(b["k_cache"].shape[0], 16, 2, 32, dtype=torch.bfloat16)
    assert status_of(q=q, out=torch.zeros_like(q), k_cache=k, v_cache=k.clone())[0] == "PA_ERR_UNSUPPORTED"
    for d in (96, 256):
        bb = build_batch("abi", [1, 40, 2], [5, 70, 40], 8, 2, d, True, seed=1)
        args = bb.args(torch.empty_like(bb.q))[:9]
        assert pa.plan_describe(*args)["persistent"] == 0
        assert pa.plan_describe(*args)["tile_rows"] == 128
        assert pa.plan_describe(*args, opts=pa.options(force_tile=2))["tile_rows"] == 128
        with pytest.raises(pa.PaError, match="PA_ERR_UNSUPPORTED"):
            pa.plan_describe(*args, opts=pa.options(force_tile=4))
    # block sizes 16, 32 and 64 are built (the host plan accepts them), others are not
    for B in (32, 64):
        bb = build_batch("abi", [1, 3, 2], [5, 17, 40], 8, 2, 128, True, seed=1, block_size=B)
        assert pa.plan_describe(*bb.args(torch.empty_like(bb.q))[:9])["persistent"] == 1
    for B in (8, 48, 128):
        k = torch.zeros(4, B, 2, 128, dtype=torch.bfloat16)
        assert status_of(k_cache=k, v_cache=k.clone())[0] == "PA_ERR_UNSUPPORTED", B


def test_element_types():
    """q, out and 16-bit caches are all bf16 or all fp16 (fp8 caches go with either)."""
    a = cpu_args()
    h = {n: a[n].half() for n in ("q", "k_cache", "v_cache")}
    # fp16 q with bf16 caches, or fp16 everything but out
    assert status_of(q=h["q"], out=torch.empty_like(h["q"]))[0] == "PA_ERR_DTYPE"
    assert status_of(q=h["q"], k_cache=h["k_cache"], v_cache=h["v_cache"])[0] == "PA_ERR_DTYPE"
    # all fp16 passes validation (the host plan accepts it)
    bb = build_batch("abi", [1, 3, 2], [5, 17, 40], 8, 2, 128, True, seed=1, kv_dtype="f16")
    assert bb.q.dtype == torch.float16
    assert pa.plan_describe(*bb.args(torch.empty_like(bb.q))[:9])["persistent"] == 1
    # fp16 q next to an fp8 cache
    b8 = build_batch("abi", [1, 3, 2], [5, 17, 40], 8, 2, 128, True, seed=1,
                     kv_dtype="fp8_e4m3fn", k_scale=0.5, v_scale=0.5, q_dtype="f16")
    assert pa.plan_describe(*b8.args(torch.empty_like(b8.q))[:9])["persistent"] == 1


def test_strides_alignment_alias():
    a = cpu_args()
    # q with a non-unit innermost stride
    big = torch.zeros(6, 8, 256, dtype=torch.bfloat16)
    assert status_of(q=big[:, :, ::2])[0] == "PA_ERR_UNSUPPORTED"
    # q token stride not a multiple of 8 elements
    odd = torch.zeros(6 * 8 * 128 + 4, dtype=torch.bfloat16)[4:].view(6, 8, 128)
    st, _ = status_of(q=odd)
    assert st == "PA_ERR_ALIGN"
    # out aliasing q
    assert status_of(q=a["q"], out=a["q"])[0] == "PA_ERR_ALIAS"
    kv = a["k_cache"].reshape(-1)[: 6 * 8 * 128].view(6, 8, 128)
    assert status_of(k_cache=a["k_cache"], v_cache=a["v_cache"], out=kv)[0] == "PA_ERR_ALIAS"
    # v with different strides than k
    k = a["k_cache"]
    vv = torch.zeros(k.shape[0] * 2, *k.shape[1:], dtype=torch.bfloat16)[::2]
    assert status_of(v_cache=vv)[0] == "PA_ERR_SHAPE"
    # non-contiguous cache interior
    kk = torch.zeros(k.shape[0], 16, 4, 128, dtype=torch.bfloat16)[:, :, ::2]
    assert status_of(k_cache=kk, v_cache=kk.clone())[0] in ("PA_ERR_UNSUPPORTED", "PA_ERR_SHAPE")


def test_empty_batch_is_ok_without_device():
    q = torch.zeros(0, 8, 128, dtype=torch.bfloat16)
    a = cpu_args(q=q, out=torch.zeros_like(q), cu_seqlens_q=torch.zeros(1, dtype=torch.int32),
                 seqused_k=torch.zeros(0, dtype=torch.int32),
                 block_table=torch.zeros(0, 3, dtype=torch.int32), max_seqlen_q=0, max_seqlen_k=0)
    assert call(a) == 0
    # queries present but no sequences: inconsistent
    a2 = cpu_args(cu_seqlens_q=torch.zeros(1, dtype=torch.int32),
                  seqused_k=torch.zeros(0, dtype=torch.int32),
                  block_table=torch.zeros(0, 3, dtype=torch.int32))
    assert pa.STATUS[call(a2)] == "PA_ERR_SHAPE"


def test_bad_options_and_workspace():
    a = cpu_args()
    assert pa.STATUS[call(a, pa.options(force_tile=7))] == "PA_ERR_UNSUPPORTED"
    # a narrow tile holds at most 16 packed rows: 5 tokens * G 4 do not fit
    assert pa.STATUS[call(dict(a, max_seqlen_q=5), pa.options(force_tile=1))] == "PA_ERR_UNSUPPORTED"
    # a forced split needs a workspace; none given (contexts > 64 keys so 2 splits remain)
    b = build_batch("ws", [1, 3, 2], [5, 170, 300], 8, 2, 128, True, seed=1)
    a2 = dict(a, q=b.q, out=torch.empty_like(b.q), k_cache=b.k_cache, v_cache=b.v_cache,
              cu_seqlens_q=b.cu_seqlens_q, seqused_k=b.seqused_k, block_table=b.block_table,
              max_seqlen_k=300)
    assert pa.STATUS[call(a2, pa.options(force_num_splits=2))] == "PA_ERR_WORKSPACE"


def plan_of(b, **opt):
    out = torch.empty_like(b.q)
    return pa.plan_describe(b.q, b.k_cache, b.v_cache, out, b.cu_seqlens_q, b.seqused_k,
                            b.block_table, b.max_seqlen_q, b.max_seqlen_k,
                            opts=pa.options(**opt) if opt else None, num_cus=256)


def test_plan_even_split_work_groups():
    # an even decode split over 16-bit caches launches one work-group per CU
    # (each wave streams a longer chunk); fp8 caches keep every resident
    # work-group (two per CU here), and a requested grid is kept
    b = build_batch("l", np.ones(16, int), np.full(16, 2048), 32, 8, 128, True, 5)
    p = plan_of(b)
    assert p["persistent"] == 1 and p["balanced"] == 1 and p["num_workgroups"] == 256
    b16 = build_batch("l", np.ones(16, int), np.full(16, 2048), 32, 8, 128, True, 5,
                      kv_dtype="f16", q_dtype="f16")
    assert plan_of(b16)["num_workgroups"] == 256
    b8 = build_batch("l", np.ones(16, int), np.full(16, 2048), 32, 8, 128, True, 5,
                     kv_dtype="fp8_e4m3fn", k_scale=1.0 / 64, v_scale=1.0 / 64)
    p8 = plan_of(b8)
    assert p8["balanced"] == 1 and p8["num_workgroups"] == 512
    assert plan_of(b, decode_grid=384)["num_workgroups"] == 384
    # fixed parts (a batch that fills every wave) keep the resident grid
    bd = build_batch("d", np.ones(256, int), np.full(256, 1050), 32, 8, 128, True, 2)
    pd = plan_of(bd)
    assert pd["balanced"] == 0 and pd["num_workgroups"] == 512


def test_plan_heuristic_on_workload_shapes():
    # decode: persistent kernel, one narrow tile per sequence, no split (2048
    # (sequence, kv-head) items are 4x the 512 resident work-groups)
    b = build_batch("d", np.ones(256, int), np.full(256, 1050), 32, 8, 128, True, 2)
    p = plan_of(b)
    assert p["persistent"] == 1 and p["tile_tokens"] == 1 and p["num_splits"] == 1
    assert p["num_workgroups"] == 256 * 2 and p["workspace_bytes"] == 0
    # few long sequences: even split on the device, chunks of >= 16 blocks;
    # num_splits bounds the parts of any row (128 blocks: 128 / 16 + 1)
    b = build_batch("l", np.ones(16, int), np.full(16, 2048), 32, 8, 128, True, 5)
    p = plan_of(b)
    assert p["persistent"] == 1 and p["balanced"] == 1
    assert p["split_keys"] == 256 and p["num_splits"] == 9
    assert p["workspace_bytes"] >= 9 * 16 * 32 * 129 * 4 + 16 * 8 * 4
    # very long rows: the smallest chunk grows so a row has at most ~256 parts
    bl = build_batch("l", np.ones(2, int), np.array([131072, 40]), 32, 8, 128, True, 5)
    pl = plan_of(bl)
    assert pl["balanced"] == 1 and pl["split_keys"] == 32 * 16 and pl["num_splits"] == 8192 // 32 + 1
    # a forced split count gives fixed-size parts
    p = plan_of(b, force_num_splits=3)
    assert p["balanced"] == 0 and p["num_splits"] == 3 and p["split_keys"] == 704
    assert p["workspace_bytes"] >= p["num_splits"] * 16 * 32 * 129 * 4 + 16 * 4
    # prefill chunks: 128-row tiles (32 tokens at G = 4), slots bounded by T/Tq + S;
    # 28 slots x 8 kv-heads fill less than 4 work-groups per CU, so keys split
    # into >= 512-key ranges (700 keys: 2 of 384)
    b = build_batch("p", [512, 1, 300], [700, 90, 300], 32, 8, 128, True, 3)
    p = plan_of(b)
    assert p["tile_tokens"] == 32 and p["slots_direct"] == 0 and p["persistent"] == 0
    assert p["num_slots"] == 813 // 32 + 3
    assert p["num_splits"] == 2 and p["split_keys"] == 384
    assert p["longest_first"] == 1
    # a full prefill batch does not split: 8 x 512 queries over 2048 keys
    bf = build_batch("f", np.full(8, 512), np.full(8, 2048), 32, 8, 128, True, 4)
    pf = plan_of(bf)
    # no split: the workspace holds only the longest-first unit order (16 B a unit)
    assert pf["num_splits"] == 1 and pf["workspace_bytes"] == -(-pf["num_slots"] * 16 // 256) * 256
    assert pf["num_slots"] * 8 >= 4 * 256 and pf["longest_first"] == 1
    # decode plans and batches of more than 2048 sequences keep the index order
    assert plan_of(build_batch("d", np.ones(8, int), np.full(8, 100), 32, 8, 128, True, 2))[
        "longest_first"] == 0
    qs = np.ones(2049, int)
    qs[0] = 64
    assert plan_of(build_batch("m", qs, np.full(2049, 64), 8, 2, 64, True, 6))["longest_first"] == 0
    # a forced split count is honoured up to one 64-key stage per split
    p = plan_of(b, force_num_splits=3)
    assert p["num_splits"] == 3 and p["split_keys"] == 256
    p = plan_of(b, force_num_splits=1000)
    assert p["split_keys"] == 64 and p["num_splits"] == 700 // 64 + 1


def test_workspace_size_matches_plan():
    b = build_batch("ws", [1, 5, 16], [70, 200, 400], 4, 2, 64, True, seed=1)
    out = torch.empty_like(b.q)
    o = pa.options(force_num_splits=2)
    n = pa.workspace_size(b.q, b.k_cache, b.v_cache, out, b.cu_seqlens_q, b.seqused_k,
                          b.block_table, b.max_seqlen_q, b.max_seqlen_k, o)
    p = pa.plan_describe(b.q, b.k_cache, b.v_cache, out, b.cu_seqlens_q, b.seqused_k,
                         b.block_table, b.max_seqlen_q, b.max_seqlen_k, o)
    assert n == p["workspace_bytes"] > 0
    # without a split only the longest-first unit order (16 B a unit) remains
    p0 = pa.plan_describe(b.q, b.k_cache, b.v_cache, out, b.cu_seqlens_q, b.seqused_k,
                          b.block_table, b.max_seqlen_q, b.max_seqlen_k)
    n0 = pa.workspace_size(b.q, b.k_cache, b.v_cache, out, b.cu_seqlens_q, b.seqused_k,
                           b.block_table, b.max_seqlen_q, b.max_seqlen_k)
    assert p0["num_splits"] == 1 and p0["longest_first"] == 1
    assert n0 == p0["workspace_bytes"] == -(-p0["num_slots"] * 16 // 256) * 256


def test_fp8_cache_descriptors():
    """fp8 E4M3 caches: both caches must share the format, the plan matches the
    bf16 one, and byte-based alignment rules apply."""
    b = build_batch("abi8", [1, 3, 2], [5, 17, 40], 8, 2, 128, True, seed=1,
                    kv_dtype="fp8_e4m3fn", k_scale=0.5, v_scale=0.25)
    base = cpu_args()
    a = dict(base, k_cache=b.k_cache, v_cache=b.v_cache)
    # a mixed pair is a dtype error
    for k, v in ((b.k_cache, base["v_cache"]), (base["k_cache"], b.v_cache)):
        rc = call(dict(base, k_cache=k, v_cache=v))
        assert pa.STATUS[rc] == "PA_ERR_DTYPE", pa.lib.pa_last_error().decode()
    # valid fp8 descriptors plan like bf16 ones
    d8 = pa.plan_describe(*[a[n] for n in ("q", "k_cache", "v_cache", "out", "cu_seqlens_q",
                                            "seqused_k", "block_table")],
                          a["max_seqlen_q"], a["max_seqlen_k"], num_cus=256)
    d16 = pa.plan_describe(*[base[n] for n in ("q", "k_cache", "v_cache", "out", "cu_seqlens_q",
                                               "seqused_k", "block_table")],
                           base["max_seqlen_q"], base["max_seqlen_k"], num_cus=256)
    assert d8 == d16
    # the block stride must be a multiple of 16 bytes (8 fp8 elements is not)
    wide = torch.zeros((b.k_cache.shape[0], 16 * 2 * 128 + 8), dtype=torch.uint8)
    kv = wide[:, :16 * 2 * 128].view(torch.float8_e4m3fn).view(-1, 16, 2, 128)
    assert kv.stride(0) == 16 * 2 * 128 + 8
    rc = call(dict(base, k_cache=kv, v_cache=kv))
    assert pa.STATUS[rc] == "PA_ERR_ALIGN", pa.lib.pa_last_error().decode()
    # the scales travel in pa_options
    o = pa.options(k_scale=0.5, v_scale=0.25)
    assert abs(o.k_scale - 0.5) < 1e-7 and abs(o.v_scale - 0.25) < 1e-7


def test_cache_write_validation():
    """pa_cache_write rejects bad descriptors on the host."""
    NB, Hkv, d = 6, 2, 64
    key = torch.zeros(5, Hkv, d, dtype=torch.bfloat16)
    kc = torch.zeros(NB, 16, Hkv, d, dtype=torch.bfloat16)
    slots = torch.tensor([0, 3, -1, 17, 40], dtype=torch.int32)

    def rc(**over):
        a = dict(key=key, value=key.clone(), k_cache=kc, v_cache=kc.clone(), slots=slots)
        a.update(over)
        ds = [pa.describe(a[n]) for n in ("key", "value", "k_cache", "v_cache", "slots")]
        r = pa.lib.pa_cache_write(*[ctypes.byref(x) for x in ds], 0.0, 0.0, None)
        return pa.STATUS.get(r, r)

    assert rc(slots=slots.to(torch.int64)) == "PA_ERR_DTYPE"
    assert rc(key=key.float()) == "PA_ERR_DTYPE"
    assert rc(v_cache=kc.to(torch.float8_e4m3fn)) == "PA_ERR_DTYPE"      # formats differ
    assert rc(slots=slots[:4]) == "PA_ERR_SHAPE"
    assert rc(key=torch.zeros(5, Hkv + 1, d, dtype=torch.bfloat16),
              value=torch.zeros(5, Hkv + 1, d, dtype=torch.bfloat16)) == "PA_ERR_SHAPE"
    assert rc(k_cache=kc, v_cache=kc) == "PA_ERR_ALIAS"
    assert rc(key=key[:0], value=key[:0], slots=slots[:0]) == "PA_OK"      # nothing to write
    assert "pa_cache_write" in declared_functions()


def test_lse_and_merge_validation():
    a = cpu_args()
    T, Hq = a["q"].shape[0], a["q"].shape[1]
    lse = torch.zeros(T, Hq, dtype=torch.float32)
    ds = [pa.describe(a[n]) for n in ("q", "k_cache", "v_cache", "out")]
    meta = [pa.describe(a[n]) for n in ("cu_seqlens_q", "seqused_k", "block_table")]

    def rc_lse(l):
        dl = pa.describe(l) if l is not None else None
        r = pa.lib.pa_unified_attention_lse(*[ctypes.byref(d) for d in ds],
                                            ctypes.byref(dl) if dl is not None else None,
                                            *[ctypes.byref(d) for d in meta], a["max_seqlen_q"],
                                            a["max_seqlen_k"], a["softmax_scale"], 1, None, None,
                                            0, None)
        return pa.STATUS.get(r, r)

    assert rc_lse(None) == "PA_ERR_NULL"
    assert rc_lse(lse.double()) == "PA_ERR_DTYPE"
    assert rc_lse(torch.zeros(T, Hq + 1, dtype=torch.float32)) == "PA_ERR_SHAPE"
    out = a["out"]

    def rc_merge(**over):
        m = dict(oa=out.clone(), la=lse.clone(), ob=out.clone(), lb=lse.clone(), o=out, lo=None)
        m.update(over)
        dd = [pa.describe(m[n]) for n in ("oa", "la", "ob", "lb", "o")]
        dlo = pa.describe(m["lo"]) if m["lo"] is not None else None
        r = pa.lib.pa_merge_attention(*[ctypes.byref(d) for d in dd],
                                      ctypes.byref(dlo) if dlo is not None else None, None)
        return pa.STATUS.get(r, r)

    assert rc_merge(la=lse.double()) == "PA_ERR_DTYPE"
    assert rc_merge(ob=torch.zeros(T, Hq, 64, dtype=torch.bfloat16)) == "PA_ERR_SHAPE"
    assert rc_merge(oa=out) == "PA_ERR_ALIAS"
    assert rc_merge(o=torch.zeros(T, Hq, 32, dtype=torch.bfloat16),
                    oa=torch.zeros(T, Hq, 32, dtype=torch.bfloat16),
                    ob=torch.zeros(T, Hq, 32, dtype=torch.bfloat16)) == "PA_ERR_UNSUPPORTED"


def test_noalloc_refuses_before_touching_the_device():
    """pa_unified_attention_noalloc: an empty batch is OK, a plan that needs
    more workspace than the static scratch and check_contents are refused on
    the host (no device needed for either)."""
    b = build_batch("big", [1] * 8, [60000] * 8, 32, 8, 128, True, seed=310, device="cpu")
    out = b.new_out()
    opts = pa.options(force_num_splits=1000)
    assert pa.workspace_bytes(*b.args(out)[:9], opts) > pa.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pa.PaError) as e:
        pa.unified_attention_noalloc(*b.args(out), opts=opts)
    assert e.value.status == -7 and "static scratch" in str(e.value)
    small = build_batch("small", [1, 1], [100, 200], 32, 8, 128, True, seed=311, device="cpu")
    with pytest.raises(pa.PaError) as e:
        pa.unified_attention_noalloc(*small.args(small.new_out()),
                                     opts=pa.options(check_contents=True))
    assert e.value.status == -4
    empty = build_batch("empty", [], [], 32, 8, 128, True, seed=312, device="cpu")
    pa.unified_attention_noalloc(*empty.args(empty.new_out()))


def test_empty_batch_still_checks_the_options():
    """An empty batch (no sequence, or no query token) launches nothing, but
    its options are checked as for any other batch: an unsupported force_tile
    fails the call and gives no workspace size."""
    for S in (0, 2):
        b = build_batch("abi", [0] * S, [5] * S, 8, 2, 128, True, seed=2)
        a = dict(q=b.q, k_cache=b.k_cache, v_cache=b.v_cache, out=torch.empty_like(b.q),
                 cu_seqlens_q=b.cu_seqlens_q, seqused_k=b.seqused_k, block_table=b.block_table,
                 max_seqlen_q=1, max_seqlen_k=16, softmax_scale=0.1, causal=True)
        assert b.q.shape[0] == 0
        assert pa.STATUS[call(a, pa.options(force_tile=7))] == "PA_ERR_UNSUPPORTED"
        assert pa.STATUS[call(a, pa.options())] == "PA_OK"
        args = b.args(torch.empty_like(b.q))[:9]
        with pytest.raises(pa.PaError, match="force_tile must be"):
            pa.workspace_bytes(*args, pa.options(force_tile=7))
        assert pa.workspace_bytes(*args, pa.options()) == 0

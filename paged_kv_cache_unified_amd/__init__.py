"""Unified paged attention for AMD MI355X (gfx950): thin Python binding of libpa.

Every step of the computation runs in the HIP kernels of ``libpa.so``; this
module only turns torch tensors into the C ABI's descriptors (``include/pa.h``)
and passes the current HIP stream.  There is no fallback: if the library is not
built, importing this package raises.

    unified_attention(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k,
                      block_table, max_seqlen_q, max_seqlen_k, softmax_scale,
                      causal)
"""

from __future__ import annotations

import ctypes
import os
import struct
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_BF16, PA_INT32, PA_FP32, PA_FP8_E4M3, PA_F16 = 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 64 << 20    # PA_NOALLOC_SCRATCH_BYTES of include/pa.h
_DTYPES = {torch.bfloat16: PA_BF16, torch.int32: PA_INT32, torch.float32: PA_FP32,
           torch.float8_e4m3fn: PA_FP8_E4M3, torch.float16: PA_F16}


class PaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class PaOptions(ctypes.Structure):
    _fields_ = [("force_num_splits", ctypes.c_int32), ("force_tile", ctypes.c_int32),
                ("check_contents", ctypes.c_int32), ("decode_grid", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class PaPlanInfo(ctypes.Structure):
    _fields_ = [("tile_tokens", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("slots_direct", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("split_keys", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("persistent", ctypes.c_int32), ("balanced", ctypes.c_int32),
                ("longest_first", ctypes.c_int32), ("unit_xcd", ctypes.c_int32),
                ("partial_rows", ctypes.c_int64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_DTYPE", -3: "PA_ERR_SHAPE",
          -4: "PA_ERR_UNSUPPORTED", -5: "PA_ERR_ALIGN", -6: "PA_ERR_ALIAS",
          -7: "PA_ERR_WORKSPACE", -8: "PA_ERR_CONTENT", -9: "PA_ERR_HIP"}

# C-ABI symbols and their prototypes, in the order of include/pa.h
_T = ctypes.POINTER(PaTensor)
_SIGNATURES = {
    "pa_unified_attention": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, _T, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                            ctypes.c_void_p]),
    "pa_unified_attention_ex": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, _T, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                               ctypes.POINTER(PaOptions), ctypes.c_void_p,
                                               ctypes.c_size_t, ctypes.c_void_p]),
    "pa_unified_attention_noalloc": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, _T, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_float,
                                                    ctypes.c_int32, ctypes.POINTER(PaOptions),
                                                    ctypes.c_void_p]),
    "pa_unified_attention_lse": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, _T, _T, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                                ctypes.POINTER(PaOptions), ctypes.c_void_p,
                                                ctypes.c_size_t, ctypes.c_void_p]),
    "pa_merge_attention": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, ctypes.c_void_p]),
    "pa_workspace_bytes": (ctypes.c_size_t, [_T, _T, _T, _T, _T, _T, _T, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.POINTER(PaOptions)]),
    "pa_workspace_size": (ctypes.c_size_t, [_T, _T, _T, _T, _T, _T, _T, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.POINTER(PaOptions)]),
    "pa_plan_describe": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, _T, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.POINTER(PaOptions),
                                        ctypes.c_int32, ctypes.POINTER(PaPlanInfo)]),
    "pa_cache_write": (ctypes.c_int, [_T, _T, _T, _T, _T, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_void_p]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_int, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_cache_unified_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


# pa_tensor's bytes: data pointer, dtype code, ndim, shape[4], stride[4]
_PA_TENSOR = struct.Struct("=Qii4q4q")
_PAD = [(0,) * (4 - n) for n in range(5)]


def describe(t: Optional[torch.Tensor]) -> PaTensor:
    """Descriptor of a tensor (data pointer, dtype code, shape, strides)."""
    if t is None:
        return PaTensor()
    nd = t.dim()
    if nd > 4:
        raise ValueError("at most 4 dimensions")
    pad = _PAD[nd]
    return PaTensor.from_buffer_copy(_PA_TENSOR.pack(t.data_ptr(), _DTYPES.get(t.dtype, 0), nd,
                                                     *t.shape, *pad, *t.stride(), *pad))


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device) -> int:
    """The current HIP stream of the tensor's device (0 for host tensors)."""
    if device.type != "cuda":
        return 0
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _check(rc: int):
    if rc != 0:
        raise PaError(rc, lib.pa_last_error().decode())


def _descs(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table):
    ds = [describe(t) for t in (q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table)]
    return ds, [ctypes.byref(x) for x in ds]


def options(force_num_splits: int = 0, force_tile: int = 0, check_contents: bool = False,
            decode_grid: int = 0, k_scale: float = 0.0, v_scale: float = 0.0) -> PaOptions:
    """pa_options; k_scale / v_scale are the fp8 caches' dequantisation scales
    (0 reads as 1)."""
    return PaOptions(int(force_num_splits), int(force_tile), int(bool(check_contents)),
                     int(decode_grid), float(k_scale), float(v_scale))


def unified_attention(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                      max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float, causal: bool,
                      *, opts: Optional[PaOptions] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention of the whole varlen batch into ``out`` ([T, Hq, d], q's dtype).

    q and out are bf16 or fp16; caches are of q's dtype or
    ``torch.float8_e4m3fn`` (E4M3 codes; their scales go in ``opts``).

    With ``opts`` or ``workspace`` given, calls ``pa_unified_attention_ex``
    (``workspace`` then must be a device tensor of at least ``workspace_size``
    bytes); otherwise ``pa_unified_attention`` with the library workspace.
    """
    ds, refs = _descs(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table)
    stream = ctypes.c_void_p(_stream_handle(q.device))
    if opts is None and workspace is None:
        rc = lib.pa_unified_attention(*refs, int(max_seqlen_q), int(max_seqlen_k),
                                      float(softmax_scale), int(bool(causal)), stream)
    else:
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        rc = lib.pa_unified_attention_ex(*refs, int(max_seqlen_q), int(max_seqlen_k),
                                         float(softmax_scale), int(bool(causal)),
                                         ctypes.byref(opts) if opts is not None else None,
                                         ws_ptr, ws_bytes, stream)
    _check(rc)
    return out


def unified_attention_noalloc(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                              max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                              causal: bool, *, opts: Optional[PaOptions] = None) -> torch.Tensor:
    """As ``unified_attention`` through ``pa_unified_attention_noalloc``: the
    split workspace is the library's static device scratch (no allocation);
    calls that overlap on one GPU race."""
    ds, refs = _descs(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table)
    stream = ctypes.c_void_p(_stream_handle(q.device))
    _check(lib.pa_unified_attention_noalloc(*refs, int(max_seqlen_q), int(max_seqlen_k),
                                            float(softmax_scale), int(bool(causal)),
                                            ctypes.byref(opts) if opts is not None else None,
                                            stream))
    return out


def unified_attention_lse(q, k_cache, v_cache, out, lse, cu_seqlens_q, seqused_k, block_table,
                          max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                          causal: bool, *, opts: Optional[PaOptions] = None,
                          workspace: Optional[torch.Tensor] = None):
    """As ``unified_attention``, also writing each row's natural-log
    log-sum-exp into ``lse`` (fp32 [T, Hq])."""
    ds = [describe(t) for t in (q, k_cache, v_cache, out, lse, cu_seqlens_q, seqused_k,
                                block_table)]
    stream = ctypes.c_void_p(_stream_handle(q.device))
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_unified_attention_lse(*[ctypes.byref(d) for d in ds], int(max_seqlen_q),
                                        int(max_seqlen_k), float(softmax_scale), int(bool(causal)),
                                        ctypes.byref(opts) if opts is not None else None,
                                        ws_ptr, ws_bytes, stream))
    return out, lse


def merge_attention(out_a, lse_a, out_b, lse_b, out, lse_out=None):
    """Combine two results of the same rows over disjoint key sets."""
    ds = [describe(t) for t in (out_a, lse_a, out_b, lse_b, out)]
    dl = describe(lse_out) if lse_out is not None else None
    stream = ctypes.c_void_p(_stream_handle(out.device))
    _check(lib.pa_merge_attention(*[ctypes.byref(d) for d in ds],
                                  ctypes.byref(dl) if dl is not None else None, stream))
    return out, lse_out


def workspace_bytes(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                    max_seqlen_q: int, max_seqlen_k: int, opts: Optional[PaOptions] = None) -> int:
    """Bytes of caller workspace ``pa_unified_attention_ex`` needs (0: none)."""
    ds, refs = _descs(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table)
    n = lib.pa_workspace_bytes(*refs, int(max_seqlen_q), int(max_seqlen_k),
                               ctypes.byref(opts) if opts is not None else None)
    if n == ctypes.c_size_t(-1).value:
        raise PaError(-3, lib.pa_last_error().decode())
    return int(n)


workspace_size = workspace_bytes


def plan_describe(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                  max_seqlen_q: int, max_seqlen_k: int, opts: Optional[PaOptions] = None,
                  num_cus: int = 0) -> dict:
    ds, refs = _descs(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table)
    info = PaPlanInfo()
    _check(lib.pa_plan_describe(*refs, int(max_seqlen_q), int(max_seqlen_k),
                                ctypes.byref(opts) if opts is not None else None, int(num_cus),
                                ctypes.byref(info)))
    return info.as_dict()


def cache_write(key, value, k_cache, v_cache, slot_mapping, k_scale: float = 0.0,
                v_scale: float = 0.0):
    """Write new tokens (bf16 or fp16 [N, Hkv, d]) into the paged caches at
    ``slot_mapping`` (int32 [N], block * block_size + position; negative
    skips).  Caches of the tokens' dtype receive the values; fp8 caches receive
    E4M3 codes of x / scale."""
    ds = [describe(t) for t in (key, value, k_cache, v_cache, slot_mapping)]
    stream = ctypes.c_void_p(_stream_handle(key.device))
    _check(lib.pa_cache_write(*[ctypes.byref(d) for d in ds], float(k_scale), float(v_scale),
                              stream))
    return k_cache, v_cache


def version() -> int:
    return int(lib.pa_version())

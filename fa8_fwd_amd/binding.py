"""ctypes binding of libfa8.so: argument marshalling from torch tensors to the C ABI of
include/fa8.h. Every step of the computation runs in the library's HIP kernels; torch only
provides device memory and the current stream. Raises if the library is missing."""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa8.so")

FA8_OK, FA8_ERR_INVALID, FA8_ERR_UNSUPPORTED, FA8_ERR_HIP = 0, 1, 2, 3
FA8_OUT_BF16, FA8_OUT_FP16 = 0, 1
SPLIT_GRANULE = 64
DECODE_BLOCK_ROWS = 32
MAX_SPLITS = 256
DECODE_AUTO, DECODE_PER_HEAD, DECODE_HEAD_GROUP = -1, 0, 1


class FA8Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fa8 status {status}: {msg}")
        self.status = status


class Descale(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class DecodePlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("block_keys", ctypes.c_int32), ("key_groups", ctypes.c_int32),
                ("heads_per_workgroup", ctypes.c_int32), ("workgroups", ctypes.c_int64)]


class FwdParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_batch_stride", ctypes.c_int64), ("q_row_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("k_batch_stride", ctypes.c_int64), ("k_row_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
        ("v_batch_stride", ctypes.c_int64), ("v_row_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p), ("seqused_k", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64), ("page_size", ctypes.c_int32),
        ("q_descale", Descale), ("k_descale", Descale), ("v_descale", Descale),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32), ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
        ("out", ctypes.c_void_p),
        ("o_batch_stride", ctypes.c_int64), ("o_row_stride", ctypes.c_int64), ("o_head_stride", ctypes.c_int64),
        ("out_dtype", ctypes.c_int32),
        ("lse", ctypes.c_void_p),
        ("lse_batch_stride", ctypes.c_int64), ("lse_head_stride", ctypes.c_int64), ("lse_row_stride", ctypes.c_int64),
        ("sink", ctypes.c_void_p),
    ]


_lib = None


class MXScales(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_batch_stride", ctypes.c_int64), ("q_row_stride", ctypes.c_int64),
                ("q_head_stride", ctypes.c_int64),
                ("k", ctypes.c_void_p), ("k_batch_stride", ctypes.c_int64), ("k_row_stride", ctypes.c_int64),
                ("k_head_stride", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_batch_stride", ctypes.c_int64), ("v_block_stride", ctypes.c_int64),
                ("v_head_stride", ctypes.c_int64)]


def lib_path() -> str:
    return _LIB_PATH


class QuantParams(ctypes.Structure):
    """fa8_quant_params of include/fa8.h."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("in_dtype", ctypes.c_int32),
        ("q_batch_stride", ctypes.c_int64), ("q_row_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("q_out", ctypes.c_void_p),
        ("o_batch_stride", ctypes.c_int64), ("o_row_stride", ctypes.c_int64), ("o_head_stride", ctypes.c_int64),
        ("q_descale", ctypes.c_void_p),
    ]


def load():
    """Load libfa8.so (built in-tree by fa8_fwd_amd.build); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FA8Error(-1, f"{_LIB_PATH} is missing: build it with `python -m fa8_fwd_amd.build` "
                           f"(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(FwdParams)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.fa8_fwd_prefill.argtypes = [P, vp]
    lib.fa8_fwd_prefill_mx.argtypes = [P, ctypes.POINTER(MXScales), vp]
    lib.fa8_fwd_decode_splitkv.argtypes = [P, i32, vp, vp, vp]
    lib.fa8_fwd_decode_splitkv_ex.argtypes = [P, i32, i32, vp, vp, vp]
    lib.fa8_fwd_decode_splitkv_ex.restype = ctypes.c_int
    lib.fa8_fwd_decode_noalloc.argtypes = [P, i32, vp]
    lib.fa8_fwd_decode_noalloc.restype = ctypes.c_int
    lib.fa8_decode_schedule_bytes.argtypes = [i32]
    lib.fa8_decode_schedule_bytes.restype = ctypes.c_size_t
    lib.fa8_decode_scheduled_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.fa8_decode_scheduled_workspace_bytes.restype = ctypes.c_size_t
    lib.fa8_decode_num_workers.argtypes = [P, i32]
    lib.fa8_decode_num_workers.restype = i32
    lib.fa8_decode_schedule.argtypes = [P, i32, vp, vp]
    lib.fa8_decode_schedule.restype = ctypes.c_int
    lib.fa8_fwd_decode_scheduled.argtypes = [P, i32, vp, i32, vp, vp, vp]
    lib.fa8_fwd_decode_scheduled.restype = ctypes.c_int
    lib.fa8_combine_scheduled.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, i32, vp, i64, i64, i64, i32, vp, i64,
                                          i64, i64, vp, vp]
    lib.fa8_combine_scheduled.restype = ctypes.c_int
    lib.fa8_combine.argtypes = [vp, vp, i32, i32, i32, vp, i32, i32, vp, i64, i64, i64, i32, vp, i64, i64, i64, vp, vp]
    lib.fa8_check_params.argtypes = [P, i32]
    QP = ctypes.POINTER(QuantParams)
    lib.fa8_quantize_q_workspace_bytes.argtypes = [QP]
    lib.fa8_quantize_q_workspace_bytes.restype = ctypes.c_int64
    lib.fa8_quantize_q.argtypes = [QP, vp, vp]
    lib.fa8_quantize_q.restype = ctypes.c_int
    for f in ("fa8_fwd_prefill", "fa8_fwd_prefill_mx", "fa8_fwd_decode_splitkv", "fa8_combine", "fa8_check_params"):
        getattr(lib, f).restype = ctypes.c_int
    lib.fa8_decode_num_splits.argtypes = [i32, i32, i32, i32]
    lib.fa8_decode_num_splits.restype = i32
    lib.fa8_decode_plan.argtypes = [P, i32, ctypes.POINTER(DecodePlan)]
    lib.fa8_decode_plan.restype = ctypes.c_int
    lib.fa8_decode_plan_ex.argtypes = [P, i32, i32, ctypes.POINTER(DecodePlan)]
    lib.fa8_decode_plan_ex.restype = ctypes.c_int
    lib.fa8_decode_num_splits_for.argtypes = [P, i32]
    lib.fa8_decode_num_splits_for.restype = i32
    lib.fa8_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.fa8_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa8_last_error.restype = ctypes.c_char_p
    lib.fa8_last_error.argtypes = []
    lib.fa8_version.restype = ctypes.c_char_p
    lib.fa8_version.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != FA8_OK:
        raise FA8Error(status, load().fa8_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _fp8_bytes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn or t.dtype == torch.uint8:
        return t
    raise FA8Error(FA8_ERR_INVALID, f"{name} must be float8_e4m3fn (or its uint8 bytes), got {t.dtype}")


def _sink_ptr(sink: Optional[torch.Tensor], heads_q: int) -> Optional[int]:
    if sink is None:
        return None
    if sink.dtype != torch.float32 or sink.numel() != heads_q or (sink.dim() > 0 and sink.stride(-1) != 1):
        raise FA8Error(FA8_ERR_INVALID, "sink must be a contiguous float32 tensor of heads_q logits")
    return sink.data_ptr()


def _descale(x: Optional[torch.Tensor], batch: int, heads_kv: int) -> Descale:
    if x is None:
        return Descale(None, 0, 0)
    if x.dtype != torch.float32:
        raise FA8Error(FA8_ERR_INVALID, "descales must be float32")
    if x.dim() == 0 or (x.dim() == 1 and x.numel() == 1):
        return Descale(x.data_ptr(), 0, 0)
    if x.dim() != 2:
        raise FA8Error(FA8_ERR_INVALID, "a descale is 0-d or (batch, kv_heads)")
    sb = x.stride(0) if x.shape[0] != 1 else 0
    sh = x.stride(1) if x.shape[1] != 1 else 0
    if x.shape[0] not in (1, batch) or x.shape[1] not in (1, heads_kv):
        raise FA8Error(FA8_ERR_INVALID, f"descale shape {tuple(x.shape)} does not broadcast to ({batch}, {heads_kv})")
    return Descale(x.data_ptr(), sb, sh)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_OUT = {torch.bfloat16: FA8_OUT_BF16, torch.float16: FA8_OUT_FP16}


def _params(q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_k, block_table, max_seqlen_q, max_seqlen_k,
            q_descale, k_descale, v_descale, softmax_scale, causal, window_left, window_right):
    q = _fp8_bytes(q, "q")
    k = _fp8_bytes(k, "k")
    v = _fp8_bytes(v, "v")
    p = FwdParams()
    varlen_q = cu_seqlens_q is not None
    if varlen_q:
        if q.dim() != 3:
            raise FA8Error(FA8_ERR_INVALID, "varlen q must be [total_q, heads_q, d]")
        batch = cu_seqlens_q.numel() - 1
        p.q_batch_stride, p.q_row_stride, p.q_head_stride = 0, q.stride(0), q.stride(1)
        hq, d = q.shape[1], q.shape[2]
        if max_seqlen_q is None:
            raise FA8Error(FA8_ERR_INVALID, "varlen q needs max_seqlen_q")
    else:
        if q.dim() != 4:
            raise FA8Error(FA8_ERR_INVALID, "q must be [batch, seqlen_q, heads_q, d]")
        batch, sq, hq, d = q.shape
        p.q_batch_stride, p.q_row_stride, p.q_head_stride = q.stride(0), q.stride(1), q.stride(2)
        max_seqlen_q = sq if max_seqlen_q is None else max_seqlen_q
    if q.stride(-1) != 1 or k.stride(-1) != 1 or v.stride(-1) != 1:
        raise FA8Error(FA8_ERR_INVALID, "the last dimension of q, k and v must be contiguous")
    if block_table is not None:
        if k.dim() != 4:
            raise FA8Error(FA8_ERR_INVALID, "paged k/v must be [num_pages, page_size, heads_kv, d]")
        p.page_size = k.shape[1]
        p.block_table = block_table.data_ptr()
        p.block_table_stride = block_table.stride(0)
        if block_table.stride(1) != 1:
            raise FA8Error(FA8_ERR_INVALID, "block_table rows must be contiguous")
        if max_seqlen_k is None:
            max_seqlen_k = block_table.shape[1] * p.page_size
        hkv = k.shape[2]
        p.k_batch_stride, p.k_row_stride, p.k_head_stride = k.stride(0), k.stride(1), k.stride(2)
        p.v_batch_stride, p.v_row_stride, p.v_head_stride = v.stride(0), v.stride(1), v.stride(2)
    elif cu_seqlens_k is not None:
        if k.dim() != 3:
            raise FA8Error(FA8_ERR_INVALID, "varlen k/v must be [total_k, heads_kv, d]")
        hkv = k.shape[1]
        if max_seqlen_k is None:
            raise FA8Error(FA8_ERR_INVALID, "varlen k/v needs max_seqlen_k")
        p.k_batch_stride, p.k_row_stride, p.k_head_stride = 0, k.stride(0), k.stride(1)
        p.v_batch_stride, p.v_row_stride, p.v_head_stride = 0, v.stride(0), v.stride(1)
    else:
        if k.dim() != 4:
            raise FA8Error(FA8_ERR_INVALID, "k/v must be [batch, seqlen_k, heads_kv, d]")
        hkv = k.shape[2]
        max_seqlen_k = k.shape[1] if max_seqlen_k is None else max_seqlen_k
        p.k_batch_stride, p.k_row_stride, p.k_head_stride = k.stride(0), k.stride(1), k.stride(2)
        p.v_batch_stride, p.v_row_stride, p.v_head_stride = v.stride(0), v.stride(1), v.stride(2)
    p.batch, p.heads_q, p.heads_kv, p.d, p.dv = batch, hq, hkv, d, v.shape[-1]
    p.max_seqlen_q, p.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    p.q, p.k, p.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k), ("seqused_k", seqused_k),
                    ("block_table", block_table)):
        if t is not None and t.dtype != torch.int32:
            raise FA8Error(FA8_ERR_INVALID, f"{name} must be int32")
    p.cu_seqlens_q, p.cu_seqlens_k, p.seqused_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_k)
    p.q_descale = _descale(q_descale, batch, hkv)
    p.k_descale = _descale(k_descale, batch, hkv)
    p.v_descale = _descale(v_descale, batch, hkv)
    p.softmax_scale = float(softmax_scale) if softmax_scale else 0.0
    p.causal = 1 if causal else 0
    p.window_left, p.window_right = int(window_left), int(window_right)
    return p


def _set_out(p: FwdParams, out: torch.Tensor, lse: Optional[torch.Tensor], varlen_q: bool):
    if out.dtype not in _OUT:
        raise FA8Error(FA8_ERR_INVALID, "out must be bfloat16 or float16")
    if out.stride(-1) != 1:
        raise FA8Error(FA8_ERR_INVALID, "out's last dimension must be contiguous")
    p.out, p.out_dtype = out.data_ptr(), _OUT[out.dtype]
    if varlen_q:
        p.o_batch_stride, p.o_row_stride, p.o_head_stride = 0, out.stride(0), out.stride(1)
    else:
        p.o_batch_stride, p.o_row_stride, p.o_head_stride = out.stride(0), out.stride(1), out.stride(2)
    if lse is not None:
        if lse.dtype != torch.float32:
            raise FA8Error(FA8_ERR_INVALID, "lse must be float32")
        p.lse = lse.data_ptr()
        if varlen_q:   # [heads_q, total_q]
            p.lse_batch_stride, p.lse_head_stride, p.lse_row_stride = 0, lse.stride(0), lse.stride(1)
        else:          # [batch, heads_q, seqlen_q]
            p.lse_batch_stride, p.lse_head_stride, p.lse_row_stride = lse.stride(0), lse.stride(1), lse.stride(2)


def _alloc_out(q: torch.Tensor, dv: int, out_dtype, varlen_q: bool, return_lse: bool, batch, hq, max_sq):
    shape = tuple(q.shape[:-1]) + (dv,)
    out = torch.empty(shape, dtype=out_dtype, device=q.device)
    lse = None
    if return_lse:
        if varlen_q:
            lse = torch.empty((hq, q.shape[0]), dtype=torch.float32, device=q.device)
        else:
            lse = torch.empty((batch, hq, max_sq), dtype=torch.float32, device=q.device)
    return out, lse


def prefill(q, k, v, *, cu_seqlens_q=None, cu_seqlens_k=None, seqused_k=None, block_table=None,
            max_seqlen_q=None, max_seqlen_k=None, q_descale=None, k_descale=None, v_descale=None,
            softmax_scale: float = 0.0, causal: bool = False, window_left: int = -1, window_right: int = -1,
            out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16, return_lse: bool = False,
            lse: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None, stream=None):
    """Full FP8 attention forward (fa8_fwd_prefill). Returns out, or (out, lse). sink: optional
    [heads_q] fp32 learnable sink logits."""
    lib = load()
    p = _params(q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_k, block_table, max_seqlen_q, max_seqlen_k,
                q_descale, k_descale, v_descale, softmax_scale, causal, window_left, window_right)
    varlen_q = cu_seqlens_q is not None
    if out is None:
        out, lse2 = _alloc_out(q, p.dv, out_dtype, varlen_q, return_lse and lse is None, p.batch, p.heads_q,
                               p.max_seqlen_q)
        lse = lse if lse is not None else lse2
    elif return_lse and lse is None:
        _, lse = _alloc_out(q, p.dv, out.dtype, varlen_q, True, p.batch, p.heads_q, p.max_seqlen_q)
    _set_out(p, out, lse, varlen_q)
    p.sink = _sink_ptr(sink, p.heads_q)
    _check(lib.fa8_fwd_prefill(ctypes.byref(p), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def _scale_bytes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must hold E8M0 scale bytes (torch.uint8), got {t.dtype}")
    if t.dim() != 4 or t.stride(-1) != 1:
        raise ValueError(f"{name} must be 4-D with a contiguous last dimension")
    return t


def prefill_mx(q, k, v, q_scale, k_scale, v_scale, *, softmax_scale: float = 0.0, causal: bool = False,
               window_left: int = -1, window_right: int = -1, out: Optional[torch.Tensor] = None,
               out_dtype=torch.bfloat16, return_lse: bool = False, lse: Optional[torch.Tensor] = None,
               sink: Optional[torch.Tensor] = None, stream=None):
    """MXFP8 attention forward (fa8_fwd_prefill_mx). q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d] E4M3;
    q_scale [B, Sq, Hq, d/32], k_scale [B, Sk, Hkv, d/32], v_scale [B, ceil(Sk/32), Hkv, dv] E8M0
    bytes (uint8). Returns out, or (out, lse)."""
    lib = load()
    p = _params(q, k, v, None, None, None, None, None, None, None, None, None, softmax_scale, causal,
                window_left, window_right)
    if out is None:
        out, lse2 = _alloc_out(q, p.dv, out_dtype, False, return_lse and lse is None, p.batch, p.heads_q,
                               p.max_seqlen_q)
        lse = lse if lse is not None else lse2
    elif return_lse and lse is None:
        _, lse = _alloc_out(q, p.dv, out.dtype, False, True, p.batch, p.heads_q, p.max_seqlen_q)
    _set_out(p, out, lse, False)
    p.sink = _sink_ptr(sink, p.heads_q)
    qs, ks, vs = _scale_bytes(q_scale, "q_scale"), _scale_bytes(k_scale, "k_scale"), _scale_bytes(v_scale, "v_scale")
    m = MXScales(qs.data_ptr(), qs.stride(0), qs.stride(1), qs.stride(2),
                 ks.data_ptr(), ks.stride(0), ks.stride(1), ks.stride(2),
                 vs.data_ptr(), vs.stride(0), vs.stride(1), vs.stride(2))
    _check(lib.fa8_fwd_prefill_mx(ctypes.byref(p), ctypes.byref(m), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_num_splits(batch: int, heads_kv: int, max_seqlen_k: int, cu_count: int = 0) -> int:
    return int(load().fa8_decode_num_splits(batch, heads_kv, max_seqlen_k, cu_count))


def decode_num_splits_for(q, k, v, *, cu_count: int = 0, **kw) -> int:
    """Split count the library picks for this decode problem (fa8_decode_num_splits_for)."""
    p = _params(q, k, v, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"), kw.get("seqused_k"), kw.get("block_table"),
                kw.get("max_seqlen_q"), kw.get("max_seqlen_k"), None, None, None, 0.0, False, -1, -1)
    return int(load().fa8_decode_num_splits_for(ctypes.byref(p), cu_count))


def decode_plan(q, k, v, *, num_splits: int, kernel: int = DECODE_AUTO, **kw) -> dict:
    """How fa8_fwd_decode_splitkv_ex computes this problem (fa8_decode_plan_ex): kernel,
    block_keys, key_groups, heads_per_workgroup, workgroups."""
    p = _params(q, k, v, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"), kw.get("seqused_k"), kw.get("block_table"),
                kw.get("max_seqlen_q"), kw.get("max_seqlen_k"), None, None, None, 0.0, False, -1, -1)
    info = DecodePlan()
    _check(load().fa8_decode_plan_ex(ctypes.byref(p), num_splits, kernel, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in DecodePlan._fields_}


def decode_workspace_bytes(num_splits: int, batch: int, max_seqlen_q: int, heads_q: int, dv: int) -> int:
    return int(load().fa8_decode_workspace_bytes(num_splits, batch, max_seqlen_q, heads_q, dv))


def decode_splitkv(q, k, v, *, num_splits: int, o_partial=None, lse_partial=None, cu_seqlens_q=None,
                   cu_seqlens_k=None, seqused_k=None, block_table=None, max_seqlen_q=None, max_seqlen_k=None,
                   q_descale=None, k_descale=None, v_descale=None, softmax_scale: float = 0.0, causal: bool = False,
                   window_left: int = -1, window_right: int = -1, kernel: int = DECODE_AUTO, stream=None):
    """Split-KV partial pass (fa8_fwd_decode_splitkv_ex; kernel: DECODE_AUTO, DECODE_PER_HEAD or
    DECODE_HEAD_GROUP). Returns (o_partial, lse_partial) with shapes [S, B, max_seqlen_q, Hq, dv]
    and [S, B, max_seqlen_q, Hq] (fp32)."""
    lib = load()
    p = _params(q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_k, block_table, max_seqlen_q, max_seqlen_k,
                q_descale, k_descale, v_descale, softmax_scale, causal, window_left, window_right)
    S, B, SQ, HQ, DV = num_splits, p.batch, p.max_seqlen_q, p.heads_q, p.dv
    if o_partial is None:
        o_partial = torch.empty((S, B, SQ, HQ, DV), dtype=torch.float32, device=q.device)
    if lse_partial is None:
        lse_partial = torch.empty((S, B, SQ, HQ), dtype=torch.float32, device=q.device)
    if o_partial.numel() < S * B * SQ * HQ * DV or lse_partial.numel() < S * B * SQ * HQ:
        raise FA8Error(FA8_ERR_INVALID, "partial buffers too small")
    if not (o_partial.is_contiguous() and lse_partial.is_contiguous()):
        raise FA8Error(FA8_ERR_INVALID, "partial buffers must be contiguous")
    _check(lib.fa8_fwd_decode_splitkv_ex(ctypes.byref(p), S, kernel, o_partial.data_ptr(), lse_partial.data_ptr(),
                                         _stream(stream)))
    return o_partial, lse_partial


def combine(o_partial, lse_partial, *, batch: int, max_seqlen_q: int, heads_q: int, dv: int, out: torch.Tensor,
            cu_seqlens_q=None, lse: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None, stream=None):
    """LSE combine of split partials into out (fa8_combine); sink: optional [heads_q] fp32 logits."""
    lib = load()
    S = o_partial.shape[0]
    varlen = cu_seqlens_q is not None
    if out.dtype not in _OUT:
        raise FA8Error(FA8_ERR_INVALID, "out must be bfloat16 or float16")
    if varlen:
        ob, orow, oh = 0, out.stride(0), out.stride(1)
    else:
        ob, orow, oh = out.stride(0), out.stride(1), out.stride(2)
    lb = lh = lr = 0
    if lse is not None:
        if varlen:
            lb, lh, lr = 0, lse.stride(0), lse.stride(1)
        else:
            lb, lh, lr = lse.stride(0), lse.stride(1), lse.stride(2)
    _check(lib.fa8_combine(o_partial.data_ptr(), lse_partial.data_ptr(), S, batch, max_seqlen_q, _ptr(cu_seqlens_q),
                           heads_q, dv, out.data_ptr(), ob, orow, oh, _OUT[out.dtype], _ptr(lse), lb, lh, lr,
                           _sink_ptr(sink, heads_q), _stream(stream)))
    return out


def decode(q, k, v, *, num_splits: Optional[int] = None, out=None, out_dtype=torch.bfloat16, return_lse=False,
           workspace: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None, kernel: int = DECODE_AUTO,
           stream=None, **kw):
    """Split-KV decode followed by the combine. num_splits=None uses fa8_decode_num_splits_for; the
    sink (optional [heads_q] fp32 logits) enters in the combine."""
    cu_q = kw.get("cu_seqlens_q")
    p = _params(q, k, v, cu_q, kw.get("cu_seqlens_k"), kw.get("seqused_k"), kw.get("block_table"),
                kw.get("max_seqlen_q"), kw.get("max_seqlen_k"), None, None, None, 0.0, False, -1, -1)
    if num_splits is None:
        num_splits = int(load().fa8_decode_num_splits_for(ctypes.byref(p), 0))
    S, B, SQ, HQ, DV = num_splits, p.batch, p.max_seqlen_q, p.heads_q, p.dv
    op = lp = None
    if workspace is not None:
        n_o, n_l = S * B * SQ * HQ * DV, S * B * SQ * HQ
        off_l = ((n_o * 4 + 255) // 256) * 256 // 4
        flat = workspace.view(torch.float32).reshape(-1)
        op = flat[:n_o].view(S, B, SQ, HQ, DV)
        lp = flat[off_l:off_l + n_l].view(S, B, SQ, HQ)
    op, lp = decode_splitkv(q, k, v, num_splits=num_splits, o_partial=op, lse_partial=lp, kernel=kernel, stream=stream,
                            **kw)
    varlen = cu_q is not None
    if out is None:
        out, lse = _alloc_out(q, DV, out_dtype, varlen, return_lse, B, HQ, SQ)
    else:
        lse = _alloc_out(q, DV, out.dtype, varlen, True, B, HQ, SQ)[1] if return_lse else None
    combine(op, lp, batch=B, max_seqlen_q=SQ, heads_q=HQ, dv=DV, out=out, cu_seqlens_q=cu_q, lse=lse, sink=sink,
            stream=stream)
    return (out, lse) if return_lse else out


MAX_WORKERS = 65535


def _decode_params(q, k, v, kw):
    return _params(q, k, v, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"), kw.get("seqused_k"), kw.get("block_table"),
                   kw.get("max_seqlen_q"), kw.get("max_seqlen_k"), kw.get("q_descale"), kw.get("k_descale"),
                   kw.get("v_descale"), kw.get("softmax_scale", 0.0), kw.get("causal", False),
                   kw.get("window_left", -1), kw.get("window_right", -1))


def decode_num_workers(q, k, v, *, cu_count: int = 0, **kw) -> int:
    """Workers of the balanced decode the library picks for this problem (fa8_decode_num_workers)."""
    return int(load().fa8_decode_num_workers(ctypes.byref(_decode_params(q, k, v, kw)), cu_count))


def decode_schedule(q, k, v, *, num_workers: int, schedule: Optional[torch.Tensor] = None, stream=None, **kw):
    """Writes the balanced decode schedule (fa8_decode_schedule) into `schedule` (int32, allocated
    when None) and returns it."""
    lib = load()
    p = _decode_params(q, k, v, kw)
    if schedule is None:
        schedule = torch.empty(int(lib.fa8_decode_schedule_bytes(p.batch)) // 4, dtype=torch.int32, device=q.device)
    if schedule.dtype != torch.int32 or not schedule.is_contiguous():
        raise FA8Error(FA8_ERR_INVALID, "schedule must be a contiguous int32 tensor")
    if schedule.numel() * 4 < int(lib.fa8_decode_schedule_bytes(p.batch)):
        raise FA8Error(FA8_ERR_INVALID, "schedule buffer too small")
    _check(lib.fa8_decode_schedule(ctypes.byref(p), num_workers, schedule.data_ptr(), _stream(stream)))
    return schedule


def decode_scheduled(q, k, v, *, num_workers: int, schedule: torch.Tensor, o_partial=None, lse_partial=None,
                     kernel: int = DECODE_AUTO, stream=None, **kw):
    """Partials of the balanced decode (fa8_fwd_decode_scheduled), which also writes the schedule
    into `schedule`: o_partial [W + B, Sq, Hq, dv] and lse_partial [W + B, Sq, Hq] fp32."""
    lib = load()
    p = _decode_params(q, k, v, kw)
    slots = num_workers + p.batch
    if o_partial is None:
        o_partial = torch.empty((slots, p.max_seqlen_q, p.heads_q, p.dv), dtype=torch.float32, device=q.device)
    if lse_partial is None:
        lse_partial = torch.empty((slots, p.max_seqlen_q, p.heads_q), dtype=torch.float32, device=q.device)
    if o_partial.numel() < slots * p.max_seqlen_q * p.heads_q * p.dv or lse_partial.numel() < slots * p.max_seqlen_q * p.heads_q:
        raise FA8Error(FA8_ERR_INVALID, "partial buffers too small")
    _check(lib.fa8_fwd_decode_scheduled(ctypes.byref(p), num_workers, schedule.data_ptr(), kernel, o_partial.data_ptr(),
                                        lse_partial.data_ptr(), _stream(stream)))
    return o_partial, lse_partial


def combine_scheduled(o_partial, lse_partial, schedule, *, num_workers: int, batch: int, max_seqlen_q: int,
                      heads_q: int, dv: int, out: torch.Tensor, cu_seqlens_q=None, lse: Optional[torch.Tensor] = None,
                      sink: Optional[torch.Tensor] = None, stream=None):
    """Merge of the balanced decode's partials (fa8_combine_scheduled)."""
    lib = load()
    varlen = cu_seqlens_q is not None
    if out.dtype not in _OUT:
        raise FA8Error(FA8_ERR_INVALID, "out must be bfloat16 or float16")
    ob, orow, oh = (0, out.stride(0), out.stride(1)) if varlen else (out.stride(0), out.stride(1), out.stride(2))
    lb = lh = lr = 0
    if lse is not None:
        lb, lh, lr = (0, lse.stride(0), lse.stride(1)) if varlen else (lse.stride(0), lse.stride(1), lse.stride(2))
    _check(lib.fa8_combine_scheduled(o_partial.data_ptr(), lse_partial.data_ptr(), schedule.data_ptr(), num_workers,
                                     batch, max_seqlen_q, _ptr(cu_seqlens_q), heads_q, dv, out.data_ptr(), ob, orow,
                                     oh, _OUT[out.dtype], _ptr(lse), lb, lh, lr, _sink_ptr(sink, heads_q),
                                     _stream(stream)))
    return out


def decode_balanced(q, k, v, *, num_workers: Optional[int] = None, out=None, out_dtype=torch.bfloat16,
                    return_lse=False, sink: Optional[torch.Tensor] = None, kernel: int = DECODE_AUTO, stream=None, **kw):
    """Balanced split-KV decode: partials (with their schedule), then the combine. num_workers=None
    uses fa8_decode_num_workers."""
    p = _decode_params(q, k, v, kw)
    if num_workers is None:
        num_workers = int(load().fa8_decode_num_workers(ctypes.byref(p), 0))
    sched = torch.empty(int(load().fa8_decode_schedule_bytes(p.batch)) // 4, dtype=torch.int32, device=q.device)
    op, lp = decode_scheduled(q, k, v, num_workers=num_workers, schedule=sched, kernel=kernel, stream=stream, **kw)
    cu_q = kw.get("cu_seqlens_q")
    varlen = cu_q is not None
    if out is None:
        out, lse = _alloc_out(q, p.dv, out_dtype, varlen, return_lse, p.batch, p.heads_q, p.max_seqlen_q)
    else:
        lse = _alloc_out(q, p.dv, out.dtype, varlen, True, p.batch, p.heads_q, p.max_seqlen_q)[1] if return_lse else None
    combine_scheduled(op, lp, sched, num_workers=num_workers, batch=p.batch, max_seqlen_q=p.max_seqlen_q,
                      heads_q=p.heads_q, dv=p.dv, out=out, cu_seqlens_q=cu_q, lse=lse, sink=sink, stream=stream)
    return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_noalloc(q, k, v, *, out: torch.Tensor, lse: Optional[torch.Tensor] = None, num_splits: int = 0,
                   sink: Optional[torch.Tensor] = None, stream=None, **kw):
    """Split-KV decode and combine in one call with the partials in the library's own scratch
    (fa8_fwd_decode_noalloc): out (and lse) must be given, nothing is allocated."""
    lib = load()
    cu_q = kw.get("cu_seqlens_q")
    p = _params(q, k, v, cu_q, kw.get("cu_seqlens_k"), kw.get("seqused_k"), kw.get("block_table"),
                kw.get("max_seqlen_q"), kw.get("max_seqlen_k"), kw.get("q_descale"), kw.get("k_descale"),
                kw.get("v_descale"), kw.get("softmax_scale", 0.0), kw.get("causal", False), kw.get("window_left", -1),
                kw.get("window_right", -1))
    _set_out(p, out, lse, cu_q is not None)
    p.sink = _sink_ptr(sink, p.heads_q)
    _check(lib.fa8_fwd_decode_noalloc(ctypes.byref(p), num_splits, _stream(stream)))
    return out


def check_params(q, k, v, num_splits: int = 0, **kw) -> int:
    """Host-side validation only (fa8_check_params); tensors may live on the CPU."""
    lib = load()
    cu_q = kw.pop("cu_seqlens_q", None)
    p = _params(q, k, v, cu_q, kw.pop("cu_seqlens_k", None), kw.pop("seqused_k", None), kw.pop("block_table", None),
                kw.pop("max_seqlen_q", None), kw.pop("max_seqlen_k", None), kw.pop("q_descale", None),
                kw.pop("k_descale", None), kw.pop("v_descale", None), kw.pop("softmax_scale", 0.0),
                kw.pop("causal", False), kw.pop("window_left", -1), kw.pop("window_right", -1))
    out = kw.pop("out", None)
    if out is not None:
        _set_out(p, out, kw.pop("lse", None), cu_q is not None)
    return int(lib.fa8_check_params(ctypes.byref(p), num_splits))


def last_error() -> str:
    return load().fa8_last_error().decode()


def version() -> str:
    return load().fa8_version().decode()


def quantize_q(q: torch.Tensor, heads_kv: int, *, cu_seqlens_q=None, max_seqlen_q: Optional[int] = None,
               out: Optional[torch.Tensor] = None, descale: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None):
    """Per-(batch, kv head) E4M3 quantization of a bf16/fp16 Q (fa8_quantize_q). Returns
    (q_fp8 as uint8 with q's shape, descale [batch, heads_kv] fp32)."""
    lib = load()
    if q.dtype not in _OUT:
        raise FA8Error(FA8_ERR_INVALID, "q must be bfloat16 or float16")
    p = QuantParams()
    varlen = cu_seqlens_q is not None
    if varlen:
        if q.dim() != 3:
            raise FA8Error(FA8_ERR_INVALID, "varlen q must be [total_q, heads_q, d]")
        batch = cu_seqlens_q.numel() - 1
        if max_seqlen_q is None:
            raise FA8Error(FA8_ERR_INVALID, "varlen q needs max_seqlen_q")
        p.q_batch_stride, p.q_row_stride, p.q_head_stride = 0, q.stride(0), q.stride(1)
        hq, d = q.shape[1], q.shape[2]
    else:
        if q.dim() != 4:
            raise FA8Error(FA8_ERR_INVALID, "q must be [batch, seqlen_q, heads_q, d]")
        batch, sq, hq, d = q.shape
        max_seqlen_q = sq if max_seqlen_q is None else max_seqlen_q
        p.q_batch_stride, p.q_row_stride, p.q_head_stride = q.stride(0), q.stride(1), q.stride(2)
    if q.stride(-1) != 1:
        raise FA8Error(FA8_ERR_INVALID, "q's last dimension must be contiguous")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    if descale is None:
        descale = torch.empty((batch, heads_kv), dtype=torch.float32, device=q.device)
    if varlen:
        p.o_batch_stride, p.o_row_stride, p.o_head_stride = 0, out.stride(0), out.stride(1)
    else:
        p.o_batch_stride, p.o_row_stride, p.o_head_stride = out.stride(0), out.stride(1), out.stride(2)
    p.batch, p.heads_q, p.heads_kv, p.d, p.max_seqlen_q = batch, hq, heads_kv, d, int(max_seqlen_q)
    p.q, p.in_dtype, p.cu_seqlens_q = q.data_ptr(), _OUT[q.dtype], _ptr(cu_seqlens_q)
    p.q_out, p.q_descale = out.data_ptr(), descale.data_ptr()
    nbytes = int(lib.fa8_quantize_q_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise FA8Error(FA8_ERR_INVALID, "workspace too small")
    _check(lib.fa8_quantize_q(ctypes.byref(p), workspace.data_ptr(), _stream(stream)))
    return out, descale

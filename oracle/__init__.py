"""CPU oracle for the FP8 attention forward. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. It never imports the HIP package and shares no code with it.

* ``attention``: exact fp64 attention on E4M3-dequantized inputs (plain C, OpenMP), for all
  rows or a requested subset, optionally restricted to a key range per row. This is the
  definition the method approximates ("Native FP8 (E4M3 Q/K/V) forward for Hopper",
  Summary/Design: E4M3 Q/K/V, q/k descales folded into the softmax scale, v descale into the
  final normalization, each 0-d or per (batch, kv_head); LSE with the 2^8 bias removed, i.e.
  the plain natural-log LSE).
* ``combine``: the log-sum-exp merge of split partial results (the split-KV combine that the
  same page times inside each decode step), written out in fp64.
* ``e4m3_table``: the oracle's own E4M3FN decode table (OCP definition).
* MXFP8 inputs: when the input carries E8M0 block scales (``q_mx``, ``k_mx``, ``v_mx``),
  ``attention`` dequantizes each 32-element block along the contraction dimension with its
  scale before the same fp64 definition (FlashAttention-4 MXFP8 page, sections 1 and 2.1; E8M0
  from the OCP Microscaling Formats specification).

The emulator of the method's own steps (tiles, lazy rescale, biased FP8 P) is in
``oracle.emulator``; it is a diagnostic, not the parity reference.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa8_oracle.c")
_LIB = os.path.join(_HERE, "libfa8_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O3 -fopenmp, no fast-math, generic x86-64)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_ss", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_base", ctypes.c_void_p),
        ("seqlen_q", ctypes.c_void_p),
        ("k_ss", ctypes.c_int64), ("k_sh", ctypes.c_int64), ("v_ss", ctypes.c_int64), ("v_sh", ctypes.c_int64),
        ("k_base", ctypes.c_void_p), ("v_base", ctypes.c_void_p), ("seqlen_k", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int64), ("page_size", ctypes.c_int32),
        ("k_ps", ctypes.c_int64), ("v_ps", ctypes.c_int64),
        ("q_descale", ctypes.c_void_p), ("k_descale", ctypes.c_void_p), ("v_descale", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_double),
        ("causal", ctypes.c_int32), ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
        ("sink", ctypes.c_void_p),
        ("q_mx", ctypes.c_void_p), ("qmx_ss", ctypes.c_int64), ("qmx_sh", ctypes.c_int64), ("qmx_base", ctypes.c_void_p),
        ("k_mx", ctypes.c_void_p), ("kmx_ss", ctypes.c_int64), ("kmx_sh", ctypes.c_int64), ("kmx_base", ctypes.c_void_p),
        ("v_mx", ctypes.c_void_p), ("vmx_sb", ctypes.c_int64), ("vmx_sh", ctypes.c_int64), ("vmx_base", ctypes.c_void_p),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.fa8_oracle_attention.restype = ctypes.c_int
        lib.fa8_oracle_attention.argtypes = [ctypes.POINTER(_Params), ctypes.c_int64] + [ctypes.c_void_p] * 7 + [ctypes.c_int32]
        lib.fa8_oracle_e4m3_table.restype = None
        lib.fa8_oracle_e4m3_table.argtypes = [ctypes.c_void_p]
        _lib = lib
    return _lib


def e4m3_table() -> np.ndarray:
    out = np.zeros(256, np.float64)
    _load().fa8_oracle_e4m3_table(out.ctypes.data)
    return out


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _descale64(x, batch: int, heads_kv: int) -> Optional[np.ndarray]:
    if x is None:
        return None
    a = np.asarray(x, np.float64)
    if a.ndim == 0:
        return np.full(batch * heads_kv, float(a), np.float64)
    return np.ascontiguousarray(np.broadcast_to(a, (batch, heads_kv))).reshape(-1).astype(np.float64)


def seqlens(inp):
    """(Sq_b, Sk_b) per batch from the input description."""
    if inp.cu_seqlens_q is not None:
        sq = np.diff(np.asarray(inp.cu_seqlens_q, np.int64))
    else:
        sq = np.full(inp.batch, inp.max_seqlen_q, np.int64)
    if inp.seqused_k is not None:
        sk = np.asarray(inp.seqused_k, np.int64)
    elif inp.cu_seqlens_k is not None:
        sk = np.diff(np.asarray(inp.cu_seqlens_k, np.int64))
    else:
        sk = np.full(inp.batch, inp.max_seqlen_k, np.int64)
    return sq, sk


def all_rows(inp):
    """(b, h, i) for every output row, in output-layout order (batch, query, head)."""
    sq, _ = seqlens(inp)
    rb, rh, ri = [], [], []
    for b in range(inp.batch):
        n = int(sq[b])
        i = np.repeat(np.arange(n, dtype=np.int32), inp.heads_q)
        h = np.tile(np.arange(inp.heads_q, dtype=np.int32), n)
        rb.append(np.full(n * inp.heads_q, b, np.int32))
        rh.append(h)
        ri.append(i)
    if not rb:
        z = np.zeros(0, np.int32)
        return z, z, z
    return np.concatenate(rb), np.concatenate(rh), np.concatenate(ri)


def attention(inp, rows=None, key_range=None, threads: Optional[int] = None, softmax_scale: Optional[float] = None,
              sink=None):
    """Exact fp64 attention for the requested rows.

    inp: an object with the fields of ``fa8_fwd_amd.inputs.AttnInputs`` (duck-typed).
    rows: (rb, rh, ri) int arrays, default every row (see ``all_rows``).
    key_range: optional (klo, khi) int64 arrays, one per row, intersected with the mask.
    Returns (O [n, dv] float64, LSE [n] float64).
    """
    lib = _load()
    B, Hq, Hkv, d, dv = inp.batch, inp.heads_q, inp.heads_kv, inp.d, inp.dv
    if rows is None:
        rows = all_rows(inp)
    rb, rh, ri = (np.ascontiguousarray(np.asarray(x, np.int32)) for x in rows)
    n = len(rb)
    sq, sk = seqlens(inp)
    q = np.ascontiguousarray(inp.q)
    k = np.ascontiguousarray(inp.k)
    v = np.ascontiguousarray(inp.v)
    p = _Params()
    p.batch, p.heads_q, p.heads_kv, p.d, p.dv = B, Hq, Hkv, d, dv
    p.q, p.k, p.v = q.ctypes.data, k.ctypes.data, v.ctypes.data
    if inp.cu_seqlens_q is not None:           # [total_q, Hq, d]
        q_base = np.asarray(inp.cu_seqlens_q[:-1], np.int64) * (Hq * d)
    else:                                       # [B, Sq, Hq, d]
        q_base = np.arange(B, dtype=np.int64) * (inp.max_seqlen_q * Hq * d)
    p.q_ss, p.q_sh = Hq * d, d
    q_base = np.ascontiguousarray(q_base)
    p.q_base = q_base.ctypes.data
    sq32 = np.ascontiguousarray(sq.astype(np.int32))
    sk32 = np.ascontiguousarray(sk.astype(np.int32))
    p.seqlen_q, p.seqlen_k = sq32.ctypes.data, sk32.ctypes.data
    p.k_ss, p.k_sh, p.v_ss, p.v_sh = Hkv * d, d, Hkv * dv, dv
    keep = [q_base, sq32, sk32]
    if inp.block_table is not None:
        bt = np.ascontiguousarray(np.asarray(inp.block_table, np.int32))
        keep.append(bt)
        p.block_table, p.bt_stride, p.page_size = bt.ctypes.data, bt.shape[1], inp.page_size
        p.k_ps, p.v_ps = inp.page_size * Hkv * d, inp.page_size * Hkv * dv
        p.k_base = p.v_base = None
    else:
        if inp.cu_seqlens_k is not None:
            kb = np.asarray(inp.cu_seqlens_k[:-1], np.int64)
        else:
            kb = np.arange(B, dtype=np.int64) * inp.max_seqlen_k
        k_base = np.ascontiguousarray(kb * (Hkv * d))
        v_base = np.ascontiguousarray(kb * (Hkv * dv))
        keep += [k_base, v_base]
        p.k_base, p.v_base = k_base.ctypes.data, v_base.ctypes.data
        p.block_table, p.bt_stride, p.page_size, p.k_ps, p.v_ps = None, 0, 0, 0, 0
    dqs = [_descale64(x, B, Hkv) for x in (inp.q_descale, inp.k_descale, inp.v_descale)]
    keep += dqs
    p.q_descale, p.k_descale, p.v_descale = (_ptr(x) for x in dqs)
    sc = softmax_scale if softmax_scale is not None else inp.softmax_scale
    p.softmax_scale = sc if sc and sc > 0 else 1.0 / math.sqrt(d)
    p.causal = 1 if inp.causal else 0
    p.window_left, p.window_right = int(inp.window_left), int(inp.window_right)
    # learnable sink: one logit per query head joining the softmax denominator (``sink``
    # overrides the input's own ``sink`` field, if any)
    z = sink if sink is not None else getattr(inp, "sink", None)
    if z is not None:
        z = np.ascontiguousarray(np.asarray(z, np.float64).reshape(-1))
        if z.size != Hq:
            raise ValueError("sink must hold one logit per query head")
        keep.append(z)
    p.sink = _ptr(z)
    # MXFP8 block scales (E8M0 bytes), when the input carries them: Q [.., Hq, d/32] per query
    # row, K [.., Hkv, d/32] per key row, V [B, ceil(Sk/32), Hkv, dv] per 32-key block (dense
    # K/V only)
    q_mx, k_mx, v_mx = (getattr(inp, f, None) for f in ("q_mx", "k_mx", "v_mx"))
    if q_mx is not None or k_mx is not None or v_mx is not None:
        if inp.block_table is not None:
            raise ValueError("MX scales need non-paged K/V")
        nq, nk = d // 32, d // 32
        if q_mx is not None:
            q_mx = np.ascontiguousarray(np.asarray(q_mx, np.uint8))
            if inp.cu_seqlens_q is not None:
                qb = np.asarray(inp.cu_seqlens_q[:-1], np.int64) * (Hq * nq)
            else:
                qb = np.arange(B, dtype=np.int64) * (inp.max_seqlen_q * Hq * nq)
            qb = np.ascontiguousarray(qb)
            keep += [q_mx, qb]
            p.q_mx, p.qmx_ss, p.qmx_sh, p.qmx_base = q_mx.ctypes.data, Hq * nq, nq, qb.ctypes.data
        if k_mx is not None:
            k_mx = np.ascontiguousarray(np.asarray(k_mx, np.uint8))
            if inp.cu_seqlens_k is not None:
                kb2 = np.asarray(inp.cu_seqlens_k[:-1], np.int64) * (Hkv * nk)
            else:
                kb2 = np.arange(B, dtype=np.int64) * (inp.max_seqlen_k * Hkv * nk)
            kb2 = np.ascontiguousarray(kb2)
            keep += [k_mx, kb2]
            p.k_mx, p.kmx_ss, p.kmx_sh, p.kmx_base = k_mx.ctypes.data, Hkv * nk, nk, kb2.ctypes.data
        if v_mx is not None:
            if inp.cu_seqlens_k is not None or inp.seqused_k is not None:
                raise ValueError("V block scales need the dense K/V layout")
            v_mx = np.ascontiguousarray(np.asarray(v_mx, np.uint8))
            nblk = (inp.max_seqlen_k + 31) // 32
            vb = np.ascontiguousarray(np.arange(B, dtype=np.int64) * (nblk * Hkv * dv))
            keep += [v_mx, vb]
            p.v_mx, p.vmx_sb, p.vmx_sh, p.vmx_base = v_mx.ctypes.data, Hkv * dv, dv, vb.ctypes.data
    klo = khi = None
    if key_range is not None:
        klo = np.ascontiguousarray(np.asarray(key_range[0], np.int64))
        khi = np.ascontiguousarray(np.asarray(key_range[1], np.int64))
    out = np.zeros((n, dv), np.float64)
    lse = np.zeros(n, np.float64)
    nt = threads if threads is not None else (os.cpu_count() or 1)
    rc = lib.fa8_oracle_attention(ctypes.byref(p), n, rb.ctypes.data, rh.ctypes.data, ri.ctypes.data,
                                  _ptr(klo), _ptr(khi), out.ctypes.data, lse.ctypes.data, int(nt))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse


def attention_full(inp, threads: Optional[int] = None):
    """Every row, reshaped: O like Q's layout with dv ([B,Sq,Hq,dv] or [total_q,Hq,dv]) and
    LSE [B, Hq, Sq] (dense) or [Hq, total_q] (varlen)."""
    o, l = attention(inp, threads=threads)
    Hq, dv = inp.heads_q, inp.dv
    if inp.cu_seqlens_q is not None:
        total = int(inp.cu_seqlens_q[-1])
        return o.reshape(total, Hq, dv), l.reshape(total, Hq).T.copy()
    B, S = inp.batch, inp.max_seqlen_q
    return o.reshape(B, S, Hq, dv), l.reshape(B, S, Hq).transpose(0, 2, 1).copy()


def combine(o_parts: np.ndarray, lse_parts: np.ndarray, sink=None):
    """Merge S split results: LSE = log sum_s exp(LSE_s); O = sum_s exp(LSE_s - LSE) O_s.

    o_parts: [S, ..., dv]; lse_parts: [S, ...] (natural log, -inf for an empty split).
    Rows where every split is empty give O = 0 and LSE = -inf. fp64 throughout.
    sink: optional sink logit per row (broadcast to lse_parts.shape[1:]): it joins the
    denominator as one more term with no value, i.e. a split with LSE = sink and O = 0.
    """
    o = np.asarray(o_parts, np.float64)
    l = np.asarray(lse_parts, np.float64)
    if sink is not None:
        z = np.broadcast_to(np.asarray(sink, np.float64), l.shape[1:])
        o = np.concatenate([o, np.zeros((1,) + o.shape[1:])], axis=0)
        l = np.concatenate([l, z[None]], axis=0)
    mx = np.max(l, axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(l - safe[None])                  # exp(-inf) = 0 for empty splits
    tot = np.sum(w, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
        wn = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)
    out = np.sum(wn[..., None] * o, axis=0)
    return out, lse

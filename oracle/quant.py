"""Per-(batch, kv head) FP8 quantization of Q, the step before the attention path. TEST
INFRASTRUCTURE ONLY (only tests/ may use it).

The block quantization formula of the FlashAttention-3 page ("Low-Precision FP8 Attention with
Block Scaling"): scale = max|X_block| / 448, X_fp8 = clip(round(X / scale), -448, 448). The block
here is every query row of one sequence and the q heads that share one kv head: the granularity
of the path's q descale (a 0-d or (batch, kv_heads) descale, the Hopper FP8 page, Design).
Reading of the arithmetic (both sides decide each code in fp32, in this order):
  amax = max |x| over the block (exact: the inputs are bf16/fp16 values),
  s    = fp32(amax / 448),   s = 1 for a block of zeros,
  y    = fp32(x / s)          (IEEE division, round to nearest even),
  code = E4M3FN(clip(y, -448, 448)), round to nearest even.
The attention path then uses s as q_descale[b, kvh].
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .emulator import e4m3_encode_rne

E4M3_MAX = np.float32(448.0)


def quantize_q(q: np.ndarray, heads_kv: int, cu_seqlens_q: Optional[np.ndarray] = None):
    """q: float32 values of a bf16/fp16 Q, [B, Sq, Hq, d] or varlen [total_q, Hq, d] with
    cu_seqlens_q ([B + 1]). Returns (codes uint8 of q's shape, descale float32 [B, heads_kv]).
    Rows past a sequence's end (varlen) belong to no block and are left as code 0."""
    q = np.asarray(q, np.float32)
    hq = q.shape[-2]
    g = hq // heads_kv
    codes = np.zeros(q.shape, np.uint8)
    if cu_seqlens_q is not None:
        cu = np.asarray(cu_seqlens_q, np.int64)
        blocks = [(b, slice(int(cu[b]), int(cu[b + 1]))) for b in range(len(cu) - 1)]
        get = lambda b, rows, hs: q[rows, hs]
        put = lambda b, rows, hs, v: codes.__setitem__((rows, hs), v)
        batch = len(cu) - 1
    else:
        batch = q.shape[0]
        blocks = [(b, slice(0, q.shape[1])) for b in range(batch)]
        get = lambda b, rows, hs: q[b, rows, hs]
        put = lambda b, rows, hs, v: codes.__setitem__((b, rows, hs), v)
    descale = np.ones((batch, heads_kv), np.float32)
    for b, rows in blocks:
        for kvh in range(heads_kv):
            hs = slice(kvh * g, (kvh + 1) * g)
            x = get(b, rows, hs)
            amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
            s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
            y = np.clip((x / s).astype(np.float32), -E4M3_MAX, E4M3_MAX)
            put(b, rows, hs, e4m3_encode_rne(y))
            descale[b, kvh] = s
    return codes, descale

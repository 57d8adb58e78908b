"""Step-by-step CPU emulator of the MXFP8 attention forward. TEST INFRASTRUCTURE ONLY (diagnostic).

Not the parity reference (``oracle.attention`` on the block-dequantized inputs is). It follows
the MXFP8 forward of the FlashAttention-4 MXFP8 page (sections 2.1 and 2.1.3) in numpy, fp32
where the method works in fp32:

1. Q, K, V dequantized exactly: E4M3 element times its E8M0 block scale 2^(e - 127) (one scale
   per 32 elements along each product's contraction dimension: d for Q and K, keys for V);
2. per KV tile of ``tile_n`` keys: scores (fp32 of the exact dots), masked -> -inf; tile row
   max in log2 units mt = max(s) * c, c = fp32(scale * log2 e); lazy rescale with ``tau`` as in
   the E4M3 method (the stored max m moves only when m = -inf or mt - m > tau);
3. P converted to MXFP8 per query row and block of 32 keys: from the block's largest score x_b
   (the page reuses the softmax's own maxima for the block amax 2^(x_b - m)), the shared
   exponent X = ceil(x_b - m - log2 448) -- the smallest power of two that keeps every element
   of the block at or below 448 (``rule="ceil"``) -- or OCP's floor(log2 amax) - 8, which lets
   the block's largest elements exceed 448 and clips them (``rule="floor"``); X clamped to
   [-127, 127]; P8 = E4M3_RNE(2^(x - m - X)) (saturating);
4. l = alpha*l + sum(P8 * 2^X) (the stored P with its scales);
5. two-level PV: O_tile = (P8 * 2^X) @ V for the tile alone, then O = alpha*O + O_tile;
6. end: O = O / l, LSE = ln2 * (m + log2 l) (no P offset in the MX path).

Returns O and LSE in the output layout of ``oracle.attention_full`` for dense inputs.
"""
from __future__ import annotations

import math

import numpy as np

from . import e4m3_table
from .emulator import e4m3_encode_rne

LOG2E = 1.4426950408889634
LOG2_448 = math.log2(448.0)


def e8m0(e: np.ndarray) -> np.ndarray:
    e = np.asarray(e, np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).astype(np.int64)))


def dequantize(inp):
    """fp64 Q [B,Sq,Hq,d], K [B,Sk,Hkv,d], V [B,Sk,Hkv,dv] of a dense MXFP8 input."""
    t = e4m3_table()
    B, Sq, Sk, Hq, Hkv, d, dv = (inp.batch, inp.max_seqlen_q, inp.max_seqlen_k, inp.heads_q, inp.heads_kv,
                                 inp.d, inp.dv)
    q = (t[inp.q].reshape(B, Sq, Hq, d // 32, 32) * e8m0(inp.q_mx)[..., None]).reshape(B, Sq, Hq, d)
    k = (t[inp.k].reshape(B, Sk, Hkv, d // 32, 32) * e8m0(inp.k_mx)[..., None]).reshape(B, Sk, Hkv, d)
    vs = np.repeat(e8m0(inp.v_mx), 32, axis=1)[:, :Sk]        # [B, Sk, Hkv, dv]
    v = t[inp.v] * vs
    return q, k, v


def _run_rows(q, k, v, b, h, kvh, i, Sq, Sk, c, tau, rule, lo_all, hi_all, dec, dv, counter):
    """The method on query rows i (indices into the sequence) of (batch b, query head h)."""
    lo, hi = lo_all[i], hi_all[i]
    nr = len(i)
    m = np.full(nr, -np.inf, np.float32)
    l = np.zeros(nr, np.float32)
    o = np.zeros((nr, dv), np.float32)
    qr = q[b, i, h]
    for t0 in range(0, Sk, counter["tile_n"]):
        js = np.arange(t0, min(t0 + counter["tile_n"], Sk))
        sc = (qr @ k[b, js, kvh].T).astype(np.float32)
        vis = (js[None, :] >= lo[:, None]) & (js[None, :] < hi[:, None])
        sc = np.where(vis, sc, np.float32(-np.inf))
        mt = (sc.max(axis=1) * c).astype(np.float32)
        with np.errstate(invalid="ignore"):
            move = (mt - m) > np.float32(tau)
        with np.errstate(over="ignore", invalid="ignore"):
            alpha = np.where(move, np.exp2((m - np.where(move, mt, 0)).astype(np.float32)), np.float32(1.0))
        alpha = np.where(move & np.isneginf(m), np.float32(0.0), alpha).astype(np.float32)
        m = np.where(move, mt, m).astype(np.float32)
        x = (sc.astype(np.float64) * np.float64(c)).astype(np.float32)      # log2 units
        p8s = np.zeros_like(x, dtype=np.float64)                           # stored P times scale
        live = ~np.isneginf(m)
        msafe = np.where(live, m, np.float32(0.0))
        for j0 in range(0, len(js), 32):
            blk = slice(j0, j0 + 32)
            with np.errstate(invalid="ignore"):
                y = (x[:, blk].max(axis=1) - msafe).astype(np.float32)
            if rule == "ceil":
                X = np.ceil(y.astype(np.float64) - LOG2_448)
            else:
                X = np.floor(y.astype(np.float64)) - 8.0
            X = np.where(np.isfinite(X) & live, np.clip(X, -127, 127), -127.0)
            arg = (x[:, blk].astype(np.float64) - msafe[:, None] - X[:, None]).astype(np.float32)
            p = np.where(live[:, None], np.exp2(arg), np.float32(0.0)).astype(np.float32)
            counter["clipped"] += int((p > 448.0).sum())
            p8s[:, blk] = dec[e4m3_encode_rne(p, saturate=True)] * np.exp2(X)[:, None]
        p8s = np.where(vis, p8s, 0.0)
        l = (alpha * l + p8s.sum(axis=1).astype(np.float32)).astype(np.float32)
        o_tile = (p8s @ v[b, js, kvh]).astype(np.float32)
        o = (alpha[:, None] * o + o_tile).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        on = np.where(l[:, None] > 0, o.astype(np.float64) / l[:, None], 0.0)
        ln = np.where(l > 0, math.log(2.0) * (m.astype(np.float64) + np.log2(np.where(l > 0, l, 1.0))), -np.inf)
    return on, ln


def _setup(inp):
    q, k, v = dequantize(inp)
    Sq, Sk = inp.max_seqlen_q, inp.max_seqlen_k
    scale = inp.softmax_scale if inp.softmax_scale and inp.softmax_scale > 0 else 1.0 / math.sqrt(inp.d)
    c = np.float32(scale * LOG2E)
    i = np.arange(Sq)
    ip = i + Sk - Sq
    hi = np.full(Sq, Sk)
    wr = 0 if inp.causal else inp.window_right
    if wr >= 0:
        hi = np.minimum(hi, ip + wr + 1)
    lo = np.zeros(Sq, np.int64)
    if inp.window_left >= 0:
        lo = np.maximum(lo, ip - inp.window_left)
    return q, k, v, c, lo, hi


def emulate_mx(inp, tile_n: int = 128, tau: float = 0.75, rule: str = "ceil", stats=None):
    """Every row: O [B, Sq, Hq, dv] and LSE [B, Hq, Sq] (float64)."""
    assert rule in ("ceil", "floor")
    q, k, v, c, lo, hi = _setup(inp)
    dec = e4m3_table()
    B, Sq, Sk, Hq, Hkv, dv = inp.batch, inp.max_seqlen_q, inp.max_seqlen_k, inp.heads_q, inp.heads_kv, inp.dv
    g = Hq // Hkv
    out = np.zeros((B, Sq, Hq, dv))
    lse = np.full((B, Hq, Sq), -np.inf)
    counter = {"clipped": 0, "tile_n": tile_n}
    rows = np.arange(Sq)
    for b in range(B):
        for h in range(Hq):
            out[b, :, h], lse[b, h] = _run_rows(q, k, v, b, h, h // g, rows, Sq, Sk, c, tau, rule, lo, hi, dec, dv,
                                               counter)
    if stats is not None:
        stats["clipped"] = counter["clipped"]
    return out, lse


def emulate_mx_rows(inp, rows_of: dict, heads=None, tile_n: int = 128, tau: float = 0.75, rule: str = "ceil"):
    """The rows rows_of[b] (indices into sequence b) of the query heads `heads` (default all):
    {(b, h): (O [n, dv], LSE [n])}. Rows are independent in the method, so these equal the rows
    of a full run."""
    q, k, v, c, lo, hi = _setup(inp)
    dec = e4m3_table()
    g = inp.heads_q // inp.heads_kv
    counter = {"clipped": 0, "tile_n": tile_n}
    res = {}
    for b in sorted(rows_of):
        i = np.asarray(rows_of[b], np.int64)
        for h in (heads if heads is not None else range(inp.heads_q)):
            res[(b, h)] = _run_rows(q, k, v, b, h, h // g, i, inp.max_seqlen_q, inp.max_seqlen_k, c, tau, rule, lo,
                                    hi, dec, inp.dv, counter)
    return res

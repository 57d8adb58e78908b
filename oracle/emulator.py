"""Step-by-step CPU emulator of the FP8 attention method. TEST INFRASTRUCTURE ONLY (diagnostic).

Not the parity reference (that is ``oracle.attention``). This follows the method's own steps in
the order the pages give them, in numpy fp32 where the method works in fp32:

1. per KV tile of ``tile_n`` keys: scores s (fp32) of the exact E4M3 dot products, masked -> -inf;
2. tile row max in scaled log2 units mt = max(s) * c, c = fp32(scale * dq * dk * log2 e)
   (q/k descales folded into the softmax scale: "Native FP8 (E4M3 Q/K/V) forward for Hopper",
   Design, Descales);
3. lazy rescale: the stored max m moves to mt only when m is -inf or mt - m > tau, and then the
   running O and l are multiplied by alpha = 2^(m - mt) (the bound tau <= log2(448) - 8 keeps the
   biased P below the E4M3 ceiling: sheared-forward fp8 page, "Correctness fix over #1:
   rescale_threshold");
4. p = 2^(s*c - m + bias), bias = 8 (the 2^8 pre-scale of P, Design "P in FP8" and the sheared
   page's Summary), cast to E4M3 with round-to-nearest-even (saturating at 448, counted as a clip);
5. l = alpha*l + sum(p)  (unrounded p by default);
6. two-level PV: O_tile = P8 @ V for this tile alone, then O = alpha*O + O_tile (Design,
   "Two-level PV accumulation");
7. end of a KV range: O = O * dv / l, LSE = ln2 * (m + log2 l - bias) (bias removed from the LSE);
8. learnable sink (optional, one logit z per query head, natural-log units): the page on the
   sheared fp8 port (Summary) carries the 2^8 offset through the row sum and the sink term, so at
   the end of the range z2 = z * log2 e enters the row sum with the same bias, after raising the
   stored max to z2 when z2 is larger (a reading: the pages do not say how a sink above the row
   max is handled; raising the max keeps every term below 2^bias):
   m' = max(m, z2), l = 2^(m - m') l + 2^(z2 - m' + bias), O = 2^(m - m') O.
   With ``sink_stage="combine"`` the sink is left out of each range and joins the combine as one
   more term instead (the split-KV path: the partials hold no sink).

Several splits over contiguous KV ranges are merged with ``oracle.combine``.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import combine, e4m3_table, seqlens

LOG2E = 1.4426950408889634
E4M3_MAX = 448.0


def e4m3_encode_rne(x: np.ndarray, saturate: bool = True) -> np.ndarray:
    """float32 -> E4M3FN codes, round to nearest even (OCP definition: bias 7, 3 mantissa bits,
    subnormal spacing 2^-9, max 448). Beyond 448: saturate to 448 (saturate=True) or NaN
    (code 0x7F) when the value rounds past 448, i.e. |x| >= 464."""
    x = np.asarray(x, np.float32).astype(np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    code = np.zeros(a.shape, np.uint8)
    nan = np.isnan(a)
    # quantum of the binade containing a: 2^(e-3) for normals (e >= -6), 2^-9 for subnormals
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    q = np.exp2(e - 3.0)
    n = a / q                                    # exact (power-of-two division)
    r = np.floor(n)
    frac = n - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1)), r + 1, r)
    v = r * q                                    # rounded magnitude, exact
    # re-derive exponent/mantissa of the rounded value
    big = v > E4M3_MAX
    v = np.where(big, E4M3_MAX, v)
    with np.errstate(divide="ignore"):
        ev = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    sub = v < 2.0 ** -6
    mant_sub = np.round(v / 2.0 ** -9).astype(np.int64)
    mant_norm = np.round((v / np.exp2(ev) - 1.0) * 8.0).astype(np.int64)
    efield = (ev + 7).astype(np.int64)
    c = np.where(sub, mant_sub, (efield << 3) | mant_norm)
    c = np.where(v == 0, 0, c)
    code = c.astype(np.uint8)
    if not saturate:
        code = np.where(big, np.uint8(0x7F), code)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """The value e4m3_encode_rne(x, saturate=True) encodes, computed directly for x >= 0 (the
    emulator's P): with x = f 2^e, f in [0.5, 1), the E4M3 quantum is 2^(max(e, -5) - 4) (three
    mantissa bits; subnormal spacing 2^-9 below 2^-6), the value is rounded to it with ties to
    even, and 448 caps it. Returned as float64."""
    x = np.asarray(x, np.float32).astype(np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -5) - 4)
    return np.minimum(np.round(x / q) * q, E4M3_MAX)


def emulate(inp, tile_n: int = 64, tau: float = 0.75, bias: float = 8.0, num_splits: int = 1, sink_stage: str = "finalize",
            l_from_rounded: bool = False, heads: Optional[list] = None, batches: Optional[list] = None,
            stats: Optional[dict] = None, interleave: int = 1, granule: Optional[int] = None,
            rows_of: Optional[dict] = None, split_granules: Optional[dict] = None):
    """Run the method on every query row of the selected (batch, head) pairs.

    Splits cut the keys into contiguous runs of granules of `granule` keys (default tile_n;
    split s takes granules [s*G/S, (s+1)*G/S) of the G granules covering [0, Sk)). Inside a
    split, tile t (tile_n keys, counted from key 0) goes to running state t mod `interleave`;
    each state runs the online softmax on its own, and the states of a split are merged with
    the log-sum-exp combine, like the splits themselves (the split-KV construction: parts of the
    KV range rescaled independently and merged by their LSEs, "Native FP8 (E4M3 Q/K/V) forward
    for Hopper", Design, Decode launches).

    split_granules, if given, maps a batch index to its splits as a list of granule ranges
    [(g0, g1), ...] (granules of `granule` keys counted from key 0), in place of the equal
    shares of num_splits; the splits are merged by the combine as usual.

    rows_of, if given, maps a batch index to the query rows (indices into that sequence) to run;
    every row's online softmax is independent of the others, so a subset gives exactly the rows
    a full run gives.

    Returns a dict {(b, h): (O [n, dv] float64, LSE [n] float64)}, n = Sq_b (or the subset).
    stats, if given, receives 'clipped' (number of P values that exceeded 448) and 'pmax'.
    """
    g_keys = granule if granule is not None else tile_n
    assert g_keys % tile_n == 0 and interleave >= 1
    dec = e4m3_table()
    B, Hq, Hkv, d, dv = inp.batch, inp.heads_q, inp.heads_kv, inp.d, inp.dv
    g = Hq // Hkv
    sq_all, sk_all = seqlens(inp)
    scale = inp.softmax_scale if inp.softmax_scale and inp.softmax_scale > 0 else 1.0 / math.sqrt(d)
    zs = getattr(inp, "sink", None)
    zs = None if zs is None else np.asarray(zs, np.float64).reshape(-1)

    def desc(x, b, kvh):
        if x is None:
            return 1.0
        a = np.asarray(x, np.float64)
        if a.ndim == 0:
            return float(a)
        return float(a[b if a.shape[0] > 1 else 0, kvh if a.shape[1] > 1 else 0])

    out = {}
    clipped = 0
    pmax = 0.0
    for b in (batches if batches is not None else (sorted(rows_of) if rows_of is not None else range(B))):
        sq, sk = int(sq_all[b]), int(sk_all[b])
        # gather this batch's Q rows and K/V rows (by token index)
        if inp.cu_seqlens_q is not None:
            q0 = int(inp.cu_seqlens_q[b])
            qb = inp.q[q0:q0 + sq]
        else:
            qb = inp.q[b, :sq]
        j = np.arange(sk)
        if inp.block_table is not None:
            pg = inp.block_table[b, j // inp.page_size]
            kb = inp.k[pg, j % inp.page_size]
            vb = inp.v[pg, j % inp.page_size]
        elif inp.cu_seqlens_k is not None:
            k0 = int(inp.cu_seqlens_k[b])
            kb, vb = inp.k[k0:k0 + sk], inp.v[k0:k0 + sk]
        else:
            kb, vb = inp.k[b, :sk], inp.v[b, :sk]
        i = np.arange(sq)
        if rows_of is not None:
            i = np.asarray(rows_of[b], np.int64)
            qb = qb[i]
        nr = len(i)
        ip = i + sk - sq
        hi = np.full(nr, sk)
        wr = 0 if inp.causal else inp.window_right
        if wr >= 0:
            hi = np.minimum(hi, ip + wr + 1)
        lo = np.zeros(nr, np.int64)
        if inp.window_left >= 0:
            lo = np.maximum(lo, ip - inp.window_left)
        # the query heads of one kv head share its K/V and its descales: their rows are stacked
        # and run together (every row's online softmax is independent of the others)
        sel_heads = list(heads if heads is not None else range(Hq))
        for kvh in sorted(set(h // g for h in sel_heads)):
            hs = [h for h in sel_heads if h // g == kvh]
            nh = len(hs)
            c = np.float32(scale * desc(inp.q_descale, b, kvh) * desc(inp.k_descale, b, kvh) * LOG2E)
            dvs = desc(inp.v_descale, b, kvh)
            qf = dec[np.concatenate([qb[:, h, :] for h in hs])]     # [nh * nr, d] exact
            kf = dec[kb[:, kvh, :]]                      # [sk, d]
            vf = dec[vb[:, kvh, :]]                      # [sk, dv]
            lo_r, hi_r = np.tile(lo, nh), np.tile(hi, nh)
            zrow = None if zs is None else np.repeat(np.asarray([zs[h] for h in hs], np.float64), nr)
            n_all = nh * nr
            ntiles = (sk + tile_n - 1) // tile_n
            per = g_keys // tile_n
            ngran = (sk + g_keys - 1) // g_keys
            parts_o, parts_l = [], []
            if split_granules is not None:
                # a sequence with no granules has one empty split (O = 0, LSE = -inf)
                ranges = [(g0 * per, min(g1 * per, ntiles)) for g0, g1 in split_granules[b]] or [(0, 0)]
            else:
                ranges = [(((s * ngran) // num_splits) * per, min((((s + 1) * ngran) // num_splits) * per, ntiles))
                          for s in range(num_splits)]
            for (t0, t1), k in [(r, k) for r in ranges for k in range(interleave)]:
                m = np.full(n_all, -np.inf, np.float32)
                l = np.zeros(n_all, np.float32)
                o = np.zeros((n_all, dv), np.float32)
                for t in range(t0, t1):
                    if t % interleave != k:
                        continue
                    js = np.arange(t * tile_n, min((t + 1) * tile_n, sk))
                    sc = (qf @ kf[js].T).astype(np.float32)          # exact dots, rounded to fp32
                    vis = (js[None, :] >= lo_r[:, None]) & (js[None, :] < hi_r[:, None])
                    sc = np.where(vis, sc, np.float32(-np.inf))
                    mt = (sc.max(axis=1) * c).astype(np.float32)
                    with np.errstate(invalid="ignore"):
                        move = (mt - m) > np.float32(tau)
                    alpha = np.where(move, np.exp2((m - np.where(move, mt, 0)).astype(np.float32)), np.float32(1.0))
                    alpha = np.where(move & np.isneginf(m), np.float32(0.0), alpha).astype(np.float32)
                    m = np.where(move, mt, m).astype(np.float32)
                    mb = np.where(np.isneginf(m), np.float32(0.0), np.float32(bias) - m).astype(np.float32)
                    x = (sc.astype(np.float64) * np.float64(c) + mb[:, None].astype(np.float64)).astype(np.float32)
                    p = np.exp2(x).astype(np.float32)                 # masked: 2^-inf = 0
                    p = np.where(vis & ~np.isneginf(m)[:, None], p, np.float32(0.0))
                    if p.size:
                        pmax = max(pmax, float(p.max()))
                        clipped += int((p > E4M3_MAX).sum())
                    p8 = e4m3_round(p)
                    psum = p8.sum(axis=1) if l_from_rounded else p.astype(np.float64).sum(axis=1)
                    l = (alpha * l + psum.astype(np.float32)).astype(np.float32)
                    o_tile = (p8 @ vf[js]).astype(np.float32)
                    o = (alpha[:, None] * o + o_tile).astype(np.float32)
                if zrow is not None and sink_stage == "finalize":
                    z2 = (zrow * LOG2E).astype(np.float32)
                    mf = np.maximum(m, z2).astype(np.float32)
                    with np.errstate(invalid="ignore"):
                        a = np.where(np.isneginf(m), np.float32(0.0), np.exp2((m - mf).astype(np.float32))).astype(np.float32)
                    l = (a * l + np.exp2((z2 - mf + np.float32(bias)).astype(np.float32))).astype(np.float32)
                    o = (a[:, None] * o).astype(np.float32)
                    m = mf
                with np.errstate(divide="ignore", invalid="ignore"):
                    on = np.where(l[:, None] > 0, o.astype(np.float64) * dvs / l[:, None], 0.0)
                    ls = np.where(l > 0, math.log(2.0) * (m.astype(np.float64) + np.log2(np.where(l > 0, l, 1.0)) - bias), -np.inf)
                parts_o.append(on)
                parts_l.append(ls)
            if interleave > 1:
                # merge the running states of each split first (a split's partial), then splits
                merged = [combine(np.stack(parts_o[i:i + interleave]), np.stack(parts_l[i:i + interleave]))
                          for i in range(0, len(parts_o), interleave)]
                parts_o = [x[0] for x in merged]
                parts_l = [x[1] for x in merged]
            zc = zrow if (zrow is not None and sink_stage == "combine") else None
            if len(ranges) == 1 and zc is None:
                ro, rl = parts_o[0], parts_l[0]
            else:
                ro, rl = combine(np.stack(parts_o), np.stack(parts_l), sink=zc)
            for j, h in enumerate(hs):
                out[(b, h)] = (ro[j * nr:(j + 1) * nr], rl[j * nr:(j + 1) * nr])
    if stats is not None:
        stats["clipped"] = clipped
        stats["pmax"] = pmax
    return out

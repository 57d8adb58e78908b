"""Shared test helpers: move seeded inputs to the GPU, call the C ABI through the binding,
compare with the CPU oracle. Test infrastructure only."""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

import oracle
from fa8_fwd_amd import binding

ATOL = 2e-2
RTOL = 2e-2
LSE_ATOL = 1e-2
GRANULE = binding.SPLIT_GRANULE
BLOCK_ROWS = binding.DECODE_BLOCK_ROWS


def dev():
    return torch.device("cuda:0")


def to_dev(x, dtype=None):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def tensors(inp):
    """Device tensors and keyword arguments for the binding from an AttnInputs."""
    kw = dict(
        cu_seqlens_q=to_dev(inp.cu_seqlens_q), cu_seqlens_k=to_dev(inp.cu_seqlens_k),
        seqused_k=to_dev(inp.seqused_k), block_table=to_dev(inp.block_table),
        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k,
        q_descale=to_dev(inp.q_descale), k_descale=to_dev(inp.k_descale), v_descale=to_dev(inp.v_descale),
        softmax_scale=inp.softmax_scale, causal=inp.causal, window_left=inp.window_left,
        window_right=inp.window_right)
    return to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), kw


def out_dtype(inp):
    return torch.float16 if inp.out_dtype == "fp16" else torch.bfloat16


def sink_tensor(inp):
    z = getattr(inp, "sink", None)
    return None if z is None else to_dev(np.asarray(z, np.float32))


def run_prefill(inp, return_lse=True):
    q, k, v, kw = tensors(inp)
    out, lse = binding.prefill(q, k, v, out_dtype=out_dtype(inp), return_lse=True, sink=sink_tensor(inp), **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def decode_schedule(inp, num_splits):
    """(block_keys, key_groups) of the decode kernel the library picks (fa8_decode_plan)."""
    q, k, v, kw = tensors(inp)
    plan = binding.decode_plan(q, k, v, num_splits=num_splits, **kw)
    return plan["block_keys"], plan["key_groups"]


def run_decode(inp, num_splits=None):
    q, k, v, kw = tensors(inp)
    out, lse = binding.decode(q, k, v, num_splits=num_splits, out_dtype=out_dtype(inp), return_lse=True,
                              sink=sink_tensor(inp), **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def compare(got: np.ndarray, ref: np.ndarray, what: str = "", atol=ATOL, rtol=RTOL):
    """allclose at the benchmark spec's tolerance; returns (max abs err, rel-RMS err)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    rms = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 0.0
    rel_rms = math.sqrt(float(np.mean((got - ref) ** 2))) / rms if rms > 0 else 0.0
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} elements outside {atol}+{rtol}*|ref| "
                             f"(max abs err {err.max():.4g}); first at {idx.tolist()}: got "
                             f"{[float(got[tuple(i)]) for i in idx]} ref {[float(ref[tuple(i)]) for i in idx]}")
    return float(err.max()) if err.size else 0.0, rel_rms


def compare_lse(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_r = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_r), f"{what}: -inf pattern of LSE differs"
    if (~inf_r).any():
        e = np.abs(got[~inf_r] - ref[~inf_r]).max()
        assert e <= LSE_ATOL, f"{what}: LSE max abs err {e}"


def rows_layout(inp, o_rows):
    """Reshape oracle rows (all_rows order) to the output layout."""
    if inp.cu_seqlens_q is not None:
        return o_rows.reshape(int(inp.cu_seqlens_q[-1]), inp.heads_q, -1)
    return o_rows.reshape(inp.batch, inp.max_seqlen_q, inp.heads_q, -1)


def split_key_ranges(inp, num_splits: int):
    """Per-row key ranges of each split of the split-KV decode, from the partition documented in
    include/fa8.h: packed rows r = i*g + (h mod g) in blocks of BLOCK_ROWS rows; each block's
    visible key union is rounded out to GRANULE-key granules and cut into num_splits runs.
    Returns (rows (rb, rh, ri), [ (klo, khi) per split ])."""
    rb, rh, ri = oracle.all_rows(inp)
    sq_all, sk_all = oracle.seqlens(inp)
    g = inp.heads_q // inp.heads_kv
    wl = inp.window_left
    wr = 0 if inp.causal else inp.window_right

    def lo_of(i, sq, sk):
        return max(0, i + sk - sq - wl) if wl >= 0 else 0

    def hi_of(i, sq, sk):
        return min(sk, i + sk - sq + wr + 1) if wr >= 0 else sk

    ranges = [(np.zeros(len(rb), np.int64), np.zeros(len(rb), np.int64)) for _ in range(num_splits)]
    for n in range(len(rb)):
        b, h, i = int(rb[n]), int(rh[n]), int(ri[n])
        sq, sk = int(sq_all[b]), int(sk_all[b])
        r = i * g + (h % g)
        blk = r // BLOCK_ROWS
        r0, r1 = blk * BLOCK_ROWS, min(blk * BLOCK_ROWS + BLOCK_ROWS, sq * g) - 1
        i0, i1 = r0 // g, r1 // g
        lo, hi = lo_of(i0, sq, sk), hi_of(i1, sq, sk)
        if hi <= lo:
            lo = hi = 0
        g0, g1 = lo // GRANULE, -(-hi // GRANULE)
        cnt = g1 - g0
        for s in range(num_splits):
            s0 = g0 + (s * cnt) // num_splits
            s1 = g0 + ((s + 1) * cnt) // num_splits
            ranges[s][0][n] = max(lo, s0 * GRANULE)
            ranges[s][1][n] = min(hi, s1 * GRANULE)
    return (rb, rh, ri), ranges


def prefill_tile(d: int, dv: int) -> int:
    """KV tile of the prefill kernel: 128 keys when d + dv <= 256, else 64 (the lazy-rescale
    decisions, and so the exact rounding, depend on the tile the kernel uses)."""
    return 128 if d + dv <= 256 else 64


def emulate_full(inp, num_splits: int = 1, with_lse: bool = False, tile_n: int = GRANULE, **kw):
    # kw: passed to the emulator (interleave, granule, l_from_rounded, ...)
    """The oracle package's step-by-step method emulator, reshaped to the output layout (and the
    LSE to [B, Hq, Sq] / [Hq, total_q] when with_lse)."""
    from oracle import emulator
    kw.setdefault("l_from_rounded", True)      # the kernel sums the rounded P
    res = emulator.emulate(inp, tile_n=tile_n, num_splits=num_splits, **kw)
    if inp.cu_seqlens_q is not None:
        tot = int(inp.cu_seqlens_q[-1])
        out = np.zeros((tot, inp.heads_q, inp.dv))
        lse = np.full((inp.heads_q, tot), -np.inf)
        for (b, h), (o, l) in res.items():
            a, z = inp.cu_seqlens_q[b], inp.cu_seqlens_q[b + 1]
            out[a:z, h] = o
            lse[h, a:z] = l
    else:
        out = np.zeros((inp.batch, inp.max_seqlen_q, inp.heads_q, inp.dv))
        lse = np.full((inp.batch, inp.heads_q, inp.max_seqlen_q), -np.inf)
        for (b, h), (o, l) in res.items():
            out[b, :, h] = o
            lse[b, h] = l
    # the method's last step: round to the output dtype (RNE), as the kernel's store does
    out = torch.from_numpy(out).to(out_dtype(inp)).double().numpy()
    return (out, lse) if with_lse else out


def method_bound(inp, ref: np.ndarray) -> np.ndarray:
    """Per-element error bound of the method from its arithmetic. Each P element is rounded to
    E4M3: p~ = p (1 + e), |e| <= 2^-4 in the normal range; subnormals (P < 2^-6, while the row's
    largest P is >= 2^8) carry an absolute error <= 2^-10, i.e. < 2^-18 of the row sum each.
    With the row sum taken over the rounded P, O = sum w_j (1 + e_j) v_j / sum w_j (1 + e_j), so
    |O - O_ref| <= 2^-4/(1 - 2^-4) * (sum_j w_j |v_j| + |O_ref|) + Sk 2^-17 max|v|, plus the
    output rounding (bf16: 2^-8 relative, fp16: 2^-11) and ~1e-4 for fp32 accumulation.
    sum_j w_j |v_j| (with the v descale) comes from the oracle run on |V| (sign bits cleared)."""
    import copy
    absinp = copy.copy(inp)
    absinp.v = inp.v & np.uint8(0x7F)
    a, _ = oracle.attention_full(absinp)
    _, sk = oracle.seqlens(inp)
    table = oracle.e4m3_table()
    vmax = float(np.nanmax(np.abs(table[inp.v])))
    if getattr(inp, "v_mx", None) is not None:       # MXFP8 V: the largest block scale
        vmax *= 2.0 ** (int(np.max(inp.v_mx)) - 127)
    dvmax = float(np.max(inp.v_descale)) if inp.v_descale is not None else 1.0
    out_rel = 2.0 ** -11 if inp.out_dtype == "fp16" else 2.0 ** -8
    e = 2.0 ** -4 / (1 - 2.0 ** -4)
    return e * (a + np.abs(ref)) + float(sk.max()) * 2.0 ** -17 * vmax * dvmax + out_rel * np.abs(ref) + 1e-4


def compare_bound(got, ref, bound, what=""):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the method's rounding bound; first at "
                             f"{idx.tolist()} err {[float(err[tuple(i)]) for i in idx]} "
                             f"bound {[float(bound[tuple(i)]) for i in idx]}")


def compare_to_emulator(got, emu, ref, what=""):
    """The kernel follows the method step by step, so it must sit much closer to the emulator
    than either sits to the exact reference (rare one-ulp E4M3 flips of P are the only source of
    difference). Requires RMS(kernel - emu) <= 0.35 * RMS(emu - ref) + 1e-4."""
    got = np.asarray(got, np.float64)
    d_ke = math.sqrt(float(np.mean((got - emu) ** 2)))
    d_er = math.sqrt(float(np.mean((emu - ref) ** 2)))
    assert d_ke <= 0.35 * d_er + 1e-4, f"{what}: kernel-emulator RMS {d_ke:.3g} vs emulator-oracle RMS {d_er:.3g}"
    return d_ke, d_er


# Largest LSE error of the method: l is a sum of E4M3-rounded P, |sum p~ / sum p - 1| <= 2^-4.
LSE_METHOD = -math.log(1 - 2.0 ** -4) + 1e-4


def check_against_oracle(inp, got, glse, what, strict=True, emu=True, num_splits=1, tile_n=GRANULE,
                         interleave=1, granule=None, sink_stage="finalize"):
    """Parity of one kernel result with the oracle.

    strict: every element within 2e-2 + 2e-2 |ref| (the stated tolerance), except elements where
      the method itself (the emulator) misses it by the same amount: those must stay inside the
      method's rounding bound with |kernel - emulator| <= |emulator - ref| / 4 + 2^-8 |ref| + 2e-3.
      Needs emu; their count is reported.
    not strict: every element inside the method's rounding bound (few-key rows, sharp softmax).
    LSE: within the method's bound -ln(1 - 2^-4); rows beyond 1e-2 are counted and reported.
    emu: also the global kernel-emulator RMS check of compare_to_emulator; the emulator runs the
      kernel's schedule (tile_n keys per step, `interleave` running states per split, splits cut
      on `granule`-key granules).
    Returns a one-line summary."""
    ref, rlse = oracle.attention_full(inp)
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = method_bound(inp, ref)
    emu_o = emu_l = None
    if emu:
        emu_o, emu_l = emulate_full(inp, num_splits=num_splits, with_lse=True, tile_n=tile_n, interleave=interleave,
                                    granule=granule, sink_stage=sink_stage)
    n_method = 0
    if strict:
        bad = err > ATOL + RTOL * np.abs(ref)
        if bad.any():
            if emu_o is None:
                compare(got, ref, what)        # raises with details
            same = np.abs(got - emu_o) <= 0.25 * np.abs(emu_o - ref) + 2.0 ** -8 * np.abs(ref) + 2e-3
            ok = same & (err <= bound)
            if not ok[bad].all():
                idx = np.argwhere(bad & ~ok)[:5]
                raise AssertionError(
                    f"{what}: {int((bad & ~ok).sum())} elements outside 2e-2 abs/rel not explained by the method: "
                    f"at {idx.tolist()} got {[float(got[tuple(i)]) for i in idx]} ref {[float(ref[tuple(i)]) for i in idx]} "
                    f"emulator {[float(emu_o[tuple(i)]) for i in idx]}")
            n_method = int(bad.sum())
    else:
        compare_bound(got, ref, bound, what)
    # LSE
    glse = np.asarray(glse, np.float64)
    inf_r = np.isneginf(rlse)
    assert np.array_equal(np.isneginf(glse), inf_r), f"{what}: -inf pattern of LSE differs"
    le = np.abs(np.where(inf_r, 0.0, glse - rlse))
    # the LSE of a row with few keys carries the relative rounding of its sum of E4M3 P values
    assert le.max(initial=0.0) <= LSE_METHOD, f"{what}: LSE max abs err {le.max():.3g} beyond the method bound"
    n_lse = int((le > LSE_ATOL).sum())
    rms = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 0.0
    rel = math.sqrt(float(np.mean((got - ref) ** 2))) / rms if rms > 0 else 0.0
    msg = (f"{what}: max abs err {err.max():.3e} rel-RMS {rel * 100:.3f}% beyond-2e-2-as-method "
           f"{n_method}/{err.size} lse-max {le.max(initial=0.0):.2e} lse>1e-2 {n_lse}/{le.size}")
    if emu:
        d_ke, d_er = compare_to_emulator(got, emu_o, ref, what)
        msg += f"; RMS kernel-emulator {d_ke:.2e} vs emulator-exact {d_er:.2e}"
    return msg

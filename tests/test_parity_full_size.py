"""GPU parity at the workloads' full sizes, launched as the benchmark launches them (the
library's own split heuristic), against the fp64 CPU oracle on rows it computes one by one:
every row where that is cheap (decode), else a seeded sample that includes the first and last
rows, row-block and tile boundaries and the ragged tails. Tolerance: |gpu - ref| <= 2e-2 +
2e-2 |ref| on the bf16/fp16 output, LSE within 1e-2 (a few elements of sharp-softmax rows may
instead sit inside the method's own rounding bound)."""
import copy

import numpy as np
import pytest

import oracle
from fa8_fwd_amd import inputs as gen

from helpers import ATOL, LSE_ATOL, LSE_METHOD, RTOL, run_decode, run_prefill
from test_mx_gpu import run_mx

pytestmark = pytest.mark.gpu


def _sample_rows(inp, per_seq: int, seed: int):
    """(rb, rh, ri): for each sequence, the boundary rows {0, 1, 31, 32, 127, 128, last-1, last}
    plus `per_seq` seeded random rows, each with every query head."""
    rng = np.random.default_rng(seed)
    sq, _ = oracle.seqlens(inp)
    rb, rh, ri = [], [], []
    for b in range(inp.batch):
        n = int(sq[b])
        if n == 0:
            continue
        pick = {0, 1, 31, 32, 127, 128, n - 2, n - 1}
        pick.update(rng.integers(0, n, per_seq).tolist())
        rows = np.array(sorted(i for i in pick if 0 <= i < n), np.int32)
        for i in rows:
            rb.append(np.full(inp.heads_q, b, np.int32))
            rh.append(np.arange(inp.heads_q, dtype=np.int32))
            ri.append(np.full(inp.heads_q, i, np.int32))
    return np.concatenate(rb), np.concatenate(rh), np.concatenate(ri)


def _gather(inp, got, glse, rows):
    """Kernel output and LSE at the oracle's rows (output layout [B,Sq,Hq,dv] / [total_q,Hq,dv],
    LSE [B,Hq,Sq] / [Hq,total_q])."""
    rb, rh, ri = (np.asarray(x, np.int64) for x in rows)
    if inp.cu_seqlens_q is not None:
        t = np.asarray(inp.cu_seqlens_q, np.int64)[rb] + ri
        return got[t, rh], glse[rh, t]
    return got[rb, ri, rh], glse[rb, rh, ri]


def _visible_keys(inp, rows):
    """Keys visible to each row: bottom-right causal alignment and window bounds."""
    rb, _, ri = (np.asarray(x, np.int64) for x in rows)
    sq, sk = (np.asarray(x, np.int64) for x in oracle.seqlens(inp))
    ip = ri + sk[rb] - sq[rb]
    wr = 0 if inp.causal else inp.window_right
    hi = np.minimum(sk[rb], ip + wr + 1) if wr >= 0 else sk[rb]
    lo = np.maximum(0, ip - inp.window_left) if inp.window_left >= 0 else np.zeros_like(ip)
    return np.clip(hi - lo, 0, None)


def _method_bound_rows(inp, rows, ref):
    """The method's own rounding bound at these rows (the bound of the small-size parity tests:
    E4M3 rounding of P, 2^-4 relative, over sum_j w_j |v_j| + |O|, plus subnormal P, output
    rounding and fp32 accumulation)."""
    absinp = copy.copy(inp)
    absinp.v = inp.v & np.uint8(0x7F)
    a, _ = oracle.attention(absinp, rows=rows)
    _, sk = oracle.seqlens(inp)
    vmax = float(np.nanmax(np.abs(oracle.e4m3_table()[inp.v])))
    if getattr(inp, "v_mx", None) is not None:       # MXFP8 V: the largest block scale
        vmax *= 2.0 ** (int(np.max(inp.v_mx)) - 127)
    dvmax = float(np.max(inp.v_descale)) if inp.v_descale is not None else 1.0
    out_rel = 2.0 ** -11 if inp.out_dtype == "fp16" else 2.0 ** -8
    e = 2.0 ** -4 / (1 - 2.0 ** -4)
    return e * (a + np.abs(ref)) + float(sk.max()) * 2.0 ** -17 * vmax * dvmax + out_rel * np.abs(ref) + 1e-4


def _check_rows(inp, got, glse, rows, what):
    """Every element within 2e-2 + 2e-2 |ref|, except at most one in a thousand that the method
    itself can miss by that much (a sharp softmax: per-(b, kv head) descales up to 2 on q and k),
    and those inside the method's rounding bound. LSE within the method's bound -ln(1 - 2^-4) (a
    sum of E4M3-rounded P) on every row and within 1e-2 on rows that see at least 256 keys (the
    rounding of a few-key row's sum does not average out)."""
    ref, rlse = oracle.attention(inp, rows=rows)
    o, l = _gather(inp, got, glse, rows)
    o = np.asarray(o, np.float64)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    n_bad = int(bad.sum())
    if n_bad:
        bound = _method_bound_rows(inp, rows, ref)
        beyond = bad & (err > bound)
        assert not beyond.any(), (f"{what}: {int(beyond.sum())} elements beyond the method's rounding bound, first at "
                                  f"{np.argwhere(beyond)[:3].tolist()}")
        assert n_bad <= 1e-3 * err.size, f"{what}: {n_bad}/{err.size} elements outside 2e-2 abs/rel"
    l = np.asarray(l, np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse)), f"{what}: -inf pattern of LSE differs"
    le = np.abs(np.where(np.isneginf(rlse), 0.0, l - rlse))
    assert le.max(initial=0.0) <= LSE_METHOD, f"{what}: LSE max abs err {le.max():.3g} beyond the method bound"
    n_lse = int((le > LSE_ATOL).sum())
    many = _visible_keys(inp, rows) >= 256
    assert not (le[many] > LSE_ATOL).any(), f"{what}: LSE beyond 1e-2 on a row with >= 256 visible keys"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rel = float(np.sqrt(np.mean((o - ref) ** 2))) / rms
    print(f"{what}: {len(rows[0])} rows, max abs err {err.max():.3e}, rel-RMS {rel * 100:.3f}%, "
          f"beyond 2e-2 (inside the method bound) {n_bad}/{err.size}, LSE max err {le.max(initial=0.0):.2e} "
          f"(beyond 1e-2: {n_lse}/{le.size})", flush=True)
    return ref, o


def test_paged_gqa_decode_full_size_every_row():
    # 64 sequences, 32/8 heads, d=128, 16-token pages, lengths uniform in [1k, 8k]
    inp = gen.paged_gqa_decode(1)
    got, glse = run_decode(inp)
    _check_rows(inp, got, glse, oracle.all_rows(inp), "paged GQA decode b64 (every row)")


def test_causal_prefill_full_size_sampled_rows():
    # B=2, 8192 x 8192, 32/8 heads, d=128, scalar descales: 40 rows per sequence, all heads
    inp = gen.causal_prefill(2)
    got, glse = run_prefill(inp)
    assert np.all(np.isfinite(got))
    _check_rows(inp, got, glse, _sample_rows(inp, 32, seed=7), "causal prefill b2 s8192 (sampled rows)")


def test_long_kv_decode_full_size_every_row():
    # B=4, 8/1 heads, 131072 keys in 64-token pages, V ~ N(0.5, 1): parity plus no shrinkage of
    # the output mean with the key count
    inp = gen.long_kv_decode(3)
    got, glse = run_decode(inp)
    ref, o = _check_rows(inp, got, glse, oracle.all_rows(inp), "long-KV decode b4 k131072 (every row)")
    ratio = float(o.mean() / ref.mean())
    print(f"long-KV output mean ratio gpu/oracle {ratio:.5f}", flush=True)
    assert 0.99 <= ratio <= 1.01


@pytest.mark.parametrize("d,dv", [(256, 256), (192, 128)])
def test_mixed_varlen_full_size_sampled_rows(d, dv):
    # 8 sequences, Sq in [256, 4096], Sk in [Sq, 4096], 16/8 heads, causal 1024-key window, fp16
    inp = gen.mixed_varlen(4, d=d, dv=dv)
    got, glse = run_prefill(inp)
    assert np.all(np.isfinite(got))
    _check_rows(inp, got, glse, _sample_rows(inp, 24, seed=11), f"mixed varlen d{d} dv{dv} (sampled rows)")


def test_mxfp8_causal_prefill_full_size_sampled_rows():
    # the MXFP8 workload the benchmark times: B=2, 8192 x 8192, 32/8 heads, d=128, N(0,1) data
    # encoded as MXFP8 (E8M0 scales per 32 elements of d for Q/K, per 32 keys for V)
    inp = gen.make_mx(2, 2, 8192, 8192, 32, 8, 128, 128, causal=True)
    got, glse = run_mx(inp)
    assert np.all(np.isfinite(got))
    _check_rows(inp, got, glse, _sample_rows(inp, 32, seed=9), "mxfp8 causal prefill b2 s8192 (sampled rows)")

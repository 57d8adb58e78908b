"""GPU parity: the HIP kernels through the C ABI against the fp64 CPU oracle, element by element,
under the one rule of helpers.check_rows: |gpu - ref| <= 2e-2 + 2e-2 |ref| on the bf16/fp16
output except at most one element in a thousand, each of those inside the method's error bound
and missed by the method itself (its emulator at the default schedule); LSE within 1e-2 on rows
that see at least 256 keys."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

from helpers import (GRANULE, LSE_ATOL, LSE_MANY_KEYS, check_against_oracle, compare, compare_lse, decode_schedule,
                     decode_splits, milder_descales, prefill_tile, run_decode, run_prefill, split_key_ranges, tensors)

pytestmark = pytest.mark.gpu


# per-(b, kv head) descales that sharpen the softmax (q and k) and scale the output (v), within
# the range where each row's softmax stays in the regime of the stated tolerance
SHARP = (("uniform", 0.5, 1.2), ("uniform", 0.5, 1.2), ("uniform", 0.5, 1.5))


def _prefill_sched(inp):
    return dict(tile_n=prefill_tile(inp.d, inp.dv))


def _check(inp, got, glse, what):
    print(check_against_oracle(inp, got, glse, what, entry="prefill", sched=_prefill_sched(inp)), flush=True)


def _prefill_check(inp, what):
    got, glse = run_prefill(inp)
    _check(inp, got, glse, what)
    return got


def test_tiny_config():
    _prefill_check(gen.tiny(0), "tiny b1 h1 q128 k256 d64")


@pytest.mark.parametrize("d,dv", [(64, 64), (96, 96), (128, 128), (192, 192), (256, 256), (192, 128)])
@pytest.mark.parametrize("mode", ["full", "causal", "window"])
def test_prefill_head_dims_and_masks(d, dv, mode):
    causal = mode != "full"
    wl = 37 if mode == "window" else -1
    inp = gen.make_dense(100 + d + dv, 2, 203, 331, 4, 2, d, dv, causal=causal, window_left=wl,
                         descales=(0.5, 0.5, 1.5))
    _prefill_check(inp, f"prefill d{d} dv{dv} {mode} q203 k331")


@pytest.mark.parametrize("d,dv", [(128, 128), (256, 256), (192, 128)])
def test_prefill_per_head_descales_sharp_softmax(d, dv):
    # per-(b, kv_head) descales up to 1.2 on q and k sharpen the softmax (scores up to 1.44x the
    # plain scale), and up to 1.5 on v
    inp = gen.make_dense(100 + d + dv, 2, 203, 331, 4, 2, d, dv, descales=SHARP)
    _prefill_check(inp, f"prefill sharp descales d{d}")


def test_prefill_causal_gqa_ragged():
    # several row blocks, ragged tail, Sq < Sk (bottom-right), GQA 8:1, scalar descales
    inp = gen.make_dense(5, 2, 300, 517, 16, 2, 128, 128, causal=True, descales=(0.5, 0.5, 1.5))
    _prefill_check(inp, "prefill causal q300 k517 gqa8")


def test_prefill_sq_longer_than_sk_has_empty_rows():
    inp = gen.make_dense(6, 1, 150, 70, 2, 1, 128, 128, causal=True)
    got = _prefill_check(inp, "empty rows")   # rows 80.. see 1..70 keys
    _, glse = run_prefill(inp)
    assert np.all(got[0, :80] == 0) and np.all(np.isneginf(glse[0, :, :80]))


@pytest.mark.parametrize("wl,wr", [(100, 30), (-1, 50), (0, 0)])
def test_prefill_two_sided_window(wl, wr):
    # non-causal local windows: row i sees keys i' - wl .. i' + wr, i' = i + Sk - Sq (bottom-right
    # alignment); (0, 0) leaves each row its own key alone
    inp = gen.make_dense(30 + max(wl, 0) + wr, 2, 203, 331, 4, 2, 128, 128, window_left=wl, window_right=wr)
    _prefill_check(inp, f"prefill window ({wl}, {wr}) q203 k331")


def test_prefill_varlen_window_fp16():
    inp = gen.mixed_varlen(4, d=256, dv=256, nseq=4, lo=64, hi=700, window=128)
    _prefill_check(inp, "varlen d256 window128 fp16")
    inp = gen.mixed_varlen(4, d=192, dv=128, nseq=4, lo=64, hi=700, window=128)
    _prefill_check(inp, "varlen d192/128 window128 fp16")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_varlen_many_sequences_every_row(causal):
    # 11 sequences x 3 kv heads = 33 (batch, kv head) groups, dealt to the 8 XCDs round-robin
    # (slots with no group exist), and up to 11 row blocks per sequence (the deal rotates every
    # 8; ranks count from each sequence's own last row block when causal, its first otherwise,
    # and the groups' order rotates within each rank): every row of every head is checked, so a
    # lost or doubled work item shows
    rng = np.random.default_rng(12)
    sq = rng.integers(1, 1300, 11)
    sq[3] = 1400
    sk = sq + 256 + rng.integers(0, 200, 11)    # every row sees at least 257 keys
    inp = gen.make_varlen(12, sq, sk, 6, 3, 64, 64, causal=causal)
    _prefill_check(inp, f"varlen 11 seqs, 3 kv heads, {'causal' if causal else 'no mask'}")


def test_prefill_varlen_empty_rows():
    inp = gen.mixed_varlen(9, d=128, dv=128, nseq=5, lo=30, hi=300, window=64, allow_empty_rows=True)
    _prefill_check(inp, "varlen with Sq > Sk rows")


def test_prefill_paged_equals_contiguous_bitwise():
    inp = gen.make_paged(7, [300, 17, 640, 129], 8, 2, 128, 128, page_size=16, sq=40, varlen_q=False, causal=True)
    got, glse = run_prefill(inp)
    _check(inp, got, glse, "paged prefill")   # a 17-key sequence
    # same tokens, contiguous varlen K/V
    sk = inp.seqused_k.astype(np.int64)
    ks, vs = [], []
    for b in range(inp.batch):
        j = np.arange(sk[b])
        pg = inp.block_table[b, j // 16]
        ks.append(inp.k[pg, j % 16])
        vs.append(inp.v[pg, j % 16])
    cont = gen.make_dense(7, 4, 40, 1, 8, 2, 128, 128, causal=True)
    cont.q = inp.q
    cont.k, cont.v = np.concatenate(ks), np.concatenate(vs)
    cont.cu_seqlens_k = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    cont.max_seqlen_k = int(sk.max())
    got2, glse2 = run_prefill(cont)
    assert np.array_equal(got, got2) and np.array_equal(glse, glse2)


@pytest.mark.parametrize("d,dv", [(64, 64), (128, 128), (256, 256), (192, 128)])
def test_prefill_output_layouts_bitwise(d, dv):
    # the output written through 16-byte row stores (16-byte aligned output, strides multiples of
    # 8 elements) equals the output written into a padded view (head stride dv + 4 elements,
    # 8-byte aligned) bit for bit, and the oracle check holds for the padded one too
    inp = gen.make_dense(60 + d, 2, 203, 331, 4, 2, d, dv, causal=True)
    q, k, v, kw = tensors(inp)
    a = torch.empty((2, 203, 4, dv), dtype=torch.bfloat16, device=q.device)
    big = torch.zeros((2, 203, 4, dv + 4), dtype=torch.bfloat16, device=q.device)
    b = big[..., 4:]
    la = binding.prefill(q, k, v, out=a, return_lse=True, **kw)[1]
    lb = binding.prefill(q, k, v, out=b, return_lse=True, **kw)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert torch.all(big[..., :4] == 0)     # nothing written outside the view
    _check(inp, b.float().cpu().numpy(), lb.cpu().numpy(), f"prefill d{d} dv{dv} padded output")


def test_prefill_deterministic():
    inp = gen.make_dense(8, 1, 256, 256, 4, 4, 128, 128, causal=True)
    a, la = run_prefill(inp)
    b, lb = run_prefill(inp)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("mode", ["omitted", "scalar", "per_bh", "broadcast_b"])
def test_descale_modes(mode):
    inp = gen.make_dense(9, 3, 70, 150, 4, 2, 128, 128, causal=True)
    rng = np.random.default_rng(0)
    if mode == "scalar":
        inp.q_descale, inp.k_descale, inp.v_descale = (np.array(x, np.float32) for x in (0.7, 1.3, 1.5))
    elif mode == "per_bh":
        inp.q_descale, inp.k_descale, inp.v_descale = (rng.uniform(0.5, hi, (3, 2)).astype(np.float32)
                                                       for hi in (1.2, 1.2, 1.5))
    elif mode == "broadcast_b":
        # (1, Hkv) descales broadcast over the batch without a copy
        dq = rng.uniform(0.5, 2, (1, 2)).astype(np.float32)
        inp.q_descale = dq
    got, glse = run_prefill(inp)
    _check(inp, got, glse, f"descales {mode}")


def _decode_check(inp, num_splits, what, kernel=binding.DECODE_AUTO):
    got, glse = run_decode(inp, num_splits, kernel)
    ns = decode_splits(inp, num_splits)
    bk, kg = decode_schedule(inp, ns, kernel)
    print(check_against_oracle(inp, got, glse, what, entry="decode", num_splits=ns,
                               sched=dict(tile_n=bk, interleave=kg, granule=GRANULE)), flush=True)
    return got


@pytest.mark.parametrize("kernel", [binding.DECODE_HEAD_GROUP, binding.DECODE_PER_HEAD])
@pytest.mark.parametrize("num_splits", [1, 3, None])
def test_decode_paged_gqa(num_splits, kernel):
    # the paged GQA decode workload at batch 8: lengths 1k-4k, per-(b, kv_head) descales (q, k
    # milder: helpers.milder_descales); both decode kernels (whole-row and per-head)
    inp = milder_descales(gen.paged_gqa_decode(1, batch=8, lo=1024, hi=4096), 81)
    _decode_check(inp, num_splits, f"paged decode b8 splits={num_splits} kernel={kernel}", kernel)


@pytest.mark.parametrize("layout", ["dense", "varlen"])
def test_decode_contiguous_kv(layout):
    # split-KV decode on contiguous K/V (fixed-length BSHD and packed varlen)
    if layout == "dense":
        inp = gen.make_dense(40, 3, 1, 777, 8, 2, 128, 128, descales=SHARP)
    else:
        inp = gen.make_varlen(41, [1, 1, 1, 1], [300, 64, 1, 2000], 8, 2, 128, 128)
    _decode_check(inp, 3, f"decode contiguous {layout}")


def test_decode_short_sequences():
    # lengths 1 .. 400 with the workload's descales (uniform in [0.5, 2] per (b, kv head))
    inp = gen.paged_gqa_decode(2, batch=8, lo=1, hi=400)
    _decode_check(inp, 3, "paged decode short sequences")


@pytest.mark.parametrize("sq,page", [(4, 16), (4, 64), (2, 64)])
@pytest.mark.parametrize("causal,wl", [(True, -1), (True, 100), (False, -1)])
def test_decode_multi_token(sq, page, causal, wl):
    sk = [300, 1000, 64, 1]
    inp = gen.make_paged(10 + sq, sk, 8, 2, 128, 128, page_size=page, sq=sq, varlen_q=True, causal=causal,
                         window_left=wl, descales=SHARP)
    _decode_check(inp, 4, f"decode sq{sq} page{page} causal{causal} wl{wl}")


@pytest.mark.parametrize("page", [16, 64])
def test_decode_two_sided_window(page):
    # four query tokens per sequence, non-causal window reaching 100 keys back and 2 ahead
    inp = gen.make_paged(40 + page, [300, 1000, 64, 1], 8, 2, 128, 128, page_size=page, sq=4, varlen_q=True,
                         window_left=100, window_right=2, descales=SHARP)
    _decode_check(inp, 4, f"decode two-sided window page{page}")


@pytest.mark.parametrize("d,dv", [(64, 64), (96, 96), (192, 192), (256, 256), (192, 128)])
def test_decode_head_dims(d, dv):
    inp = gen.make_paged(20 + d, [500, 77, 1200], 16, 4, d, dv, page_size=16, sq=1, varlen_q=True)
    _decode_check(inp, 2, f"decode d{d} dv{dv}")


def test_decode_partials_match_oracle_ranges():
    # partial LSEs use the same rounded-P sums as the final LSE: few keys per split, method bound
    inp = gen.make_paged(30, [700, 1500, 90], 8, 2, 128, 128, page_size=16, sq=2, varlen_q=True, causal=True)
    S = 5
    q, k, v, kw = tensors(inp)
    op, lp = binding.decode_splitkv(q, k, v, num_splits=S, **kw)
    torch.cuda.synchronize()
    op, lp = op.cpu().numpy(), lp.cpu().numpy()
    rows, ranges = split_key_ranges(inp, S)
    rb, rh, ri = rows
    for s in range(S):
        ro, rl = oracle.attention(inp, rows=rows, key_range=ranges[s])
        go = op[s, rb, ri, rh]
        gl = lp[s, rb, ri, rh]
        compare(go, ro, f"partial split {s}")    # every element within 2e-2 abs/rel, no exception
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin)
        le = np.abs(gl[fin] - rl[fin])
        assert le.max() <= 0.0646, f"partial lse split {s}"
        many = (ranges[s][1] - ranges[s][0])[fin] >= LSE_MANY_KEYS
        assert (le[many] <= LSE_ATOL).all(), f"partial lse split {s} on a range of >= {LSE_MANY_KEYS} keys"


@pytest.mark.parametrize("d,page", [(128, 16), (128, 64), (128, 8), (128, 4), (64, 16), (256, 16), (96, 16)])
def test_decode_empty_and_poisoned_pages(d, page):
    # a zero-length sequence and NaN-filled unused pages / tail slots must not reach the output
    # (page sizes at, above and below the rows one 64-lane load covers: 64 / (d / 16))
    inp = gen.make_paged(31, [0, 33, 200, 16, 129], 8, 2, d, d, page_size=page, sq=1, varlen_q=True)
    used = set()
    for b, s in enumerate(inp.seqused_k):
        used.update(inp.block_table[b, : (int(s) + page - 1) // page].tolist())
    for pg in range(inp.k.shape[0]):
        if pg not in used:
            inp.k[pg] = 0x7F
            inp.v[pg] = 0x7F
    for b, s in enumerate(inp.seqused_k):
        s = int(s)
        if s % page:
            pg = inp.block_table[b, s // page]
            inp.k[pg, s % page:] = 0x7F
            inp.v[pg, s % page:] = 0x7F
    got = _decode_check(inp, 3, f"decode with poison d{d} page{page}")
    assert np.all(got[0] == 0)


def test_long_kv_no_shrinkage():
    # V ~ N(0.5, 1), one split and many: parity, and the output mean stays that of the oracle
    inp = gen.long_kv_decode(3, batch=2, seqlen=32768, page_size=64)
    ref, _ = oracle.attention_full(inp)
    for S in (1, 64):
        got = _decode_check(inp, S, f"long kv 32k splits={S}")
        ratio = got.mean() / ref.mean()
        print(f"long kv 32k splits={S}: mean ratio {ratio:.5f}", flush=True)
        assert 0.99 <= ratio <= 1.01


@pytest.mark.parametrize("S,DV", [(6, 128), (40, 128), (40, 96), (40, 192), (33, 256), (64, 64)])
def test_combine_entry_point_alone(S, DV):
    # random partials with some empty splits, combined on the GPU vs the oracle's combine (more
    # than 16 splits take the split-parallel combine)
    rng = np.random.default_rng(1)
    B, SQ, HQ = 3, 2, 4
    op = rng.standard_normal((S, B, SQ, HQ, DV)).astype(np.float32)
    lp = (rng.standard_normal((S, B, SQ, HQ)) * 3).astype(np.float32)
    lp[1] = -np.inf
    lp[:, 2, 1, 3] = -np.inf          # one row with every split empty
    ref_o, ref_l = oracle.combine(op, lp)
    ref_o[2, 1, 3] = 0
    dev = torch.device("cuda:0")
    out = torch.empty((B, SQ, HQ, DV), dtype=torch.float16, device=dev)
    lse = torch.empty((B, HQ, SQ), dtype=torch.float32, device=dev)
    binding.combine(torch.from_numpy(op).to(dev), torch.from_numpy(lp).to(dev), batch=B, max_seqlen_q=SQ,
                    heads_q=HQ, dv=DV, out=out, lse=lse)
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy(), ref_o, "combine")
    compare_lse(lse.cpu().numpy(), ref_l.transpose(0, 2, 1), "combine lse")


# ---- learnable sink (one logit per query head in the softmax denominator) ----

@pytest.mark.parametrize("mean", [0.0, 6.0])
def test_prefill_with_sink(mean):
    # causal GQA with a ragged tail; mean 6 makes the sink a large share of each denominator
    base = gen.make_dense(5, 2, 300, 517, 16, 2, 128, 128, causal=True, descales=(0.5, 0.5, 1.5))
    inp = gen.with_sink(base, 8, mean=mean, std=1.0)
    _prefill_check(inp, f"prefill with sink mean {mean}")


def test_prefill_sink_empty_rows():
    # Sq > Sk causal: rows without keys give O = 0 and LSE = the sink
    inp = gen.with_sink(gen.make_dense(6, 1, 150, 70, 2, 1, 128, 128, causal=True), 9)
    got, glse = run_prefill(inp)
    _check(inp, got, glse, "prefill sink empty rows")
    assert np.all(got[0, :80] == 0)
    np.testing.assert_allclose(glse[0, :, :80], np.broadcast_to(inp.sink[:, None], (2, 80)), rtol=0, atol=1e-6)


@pytest.mark.parametrize("num_splits", [1, 3, None])
def test_decode_paged_with_sink(num_splits):
    inp = gen.with_sink(milder_descales(gen.paged_gqa_decode(1, batch=8, lo=1024, hi=4096), 82), 10, mean=4.0,
                        std=2.0)
    _decode_check(inp, num_splits, f"paged decode with sink splits={num_splits}")


@pytest.mark.parametrize("S", [6, 40])
def test_combine_with_sink(S):
    rng = np.random.default_rng(2)
    B, SQ, HQ, DV = 3, 2, 4, 128
    op = rng.standard_normal((S, B, SQ, HQ, DV)).astype(np.float32)
    lp = (rng.standard_normal((S, B, SQ, HQ)) * 3).astype(np.float32)
    lp[:, 2, 1, 3] = -np.inf          # a row with every split empty: O = 0, LSE = the sink
    z = np.array([0.5, -1.0, 2.0, 8.0], np.float32)
    ref_o, ref_l = oracle.combine(op, lp, sink=z[None, None, :])
    dev = torch.device("cuda:0")
    out = torch.empty((B, SQ, HQ, DV), dtype=torch.float16, device=dev)
    lse = torch.empty((B, HQ, SQ), dtype=torch.float32, device=dev)
    binding.combine(torch.from_numpy(op).to(dev), torch.from_numpy(lp).to(dev), batch=B, max_seqlen_q=SQ,
                    heads_q=HQ, dv=DV, out=out, lse=lse, sink=torch.from_numpy(z).to(dev))
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy(), ref_o, "combine with sink")
    compare_lse(lse.cpu().numpy(), ref_l.transpose(0, 2, 1), "combine with sink lse")
    assert np.all(out.float().cpu().numpy()[2, 1, 3] == 0)

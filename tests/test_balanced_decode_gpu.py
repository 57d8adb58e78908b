"""The balanced split-KV decode (include/fa8.h: fa8_decode_schedule, fa8_fwd_decode_scheduled,
fa8_combine_scheduled): per-request split counts computed on the device into a caller-owned
schedule. The schedule is integer work and must equal, entry for entry, the definition in the
header computed on the CPU (helpers.balanced_schedule); the outputs follow the one parity rule
against the oracle with the emulator run on the same segments; each segment's partial matches the
oracle on its key range; a graph replaying the three calls picks up new lengths each replay."""
import numpy as np
import pytest
import torch

import oracle
from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

from helpers import (GRANULE, LSE_ATOL, LSE_MANY_KEYS, LSE_METHOD, balanced_schedule, check_against_oracle,
                     decode_schedule, method_bound_rows, milder_descales, run_decode_balanced, score_error, tensors)

pytestmark = pytest.mark.gpu

SHARP = (("uniform", 0.5, 1.2), ("uniform", 0.5, 1.2), ("uniform", 0.5, 1.5))


def _workers(inp, num_workers):
    if num_workers is not None:
        return num_workers
    q, k, v, kw = tensors(inp)
    return binding.decode_num_workers(q, k, v, **kw)


def _check_schedule(inp, num_workers, with_decode=True):
    # the schedule written by fa8_decode_schedule and the one the decode writes (derived by its
    # waves up to 64 sequences, by the schedule kernel beyond) both equal the definition
    q, k, v, kw = tensors(inp)
    scheds = [binding.decode_schedule(q, k, v, num_workers=num_workers, **kw)]
    if with_decode:
        s2 = torch.full_like(scheds[0], -7)
        binding.decode_scheduled(q, k, v, num_workers=num_workers, schedule=s2, **kw)
        scheds.append(s2)
    torch.cuda.synchronize()
    G, gst, pst, segs = balanced_schedule(inp, num_workers)
    B = inp.batch
    for sched in scheds:
        got = sched.cpu().numpy().astype(np.int64)
        assert got[0] == G and got[1] == num_workers
        assert np.array_equal(got[2:3 + B], gst) and np.array_equal(got[3 + B:4 + 2 * B], pst)
    assert pst[-1] <= num_workers + B - 1
    return segs


def _balanced_check(inp, num_workers, what, kernel=binding.DECODE_AUTO):
    W = _workers(inp, num_workers)
    segs = _check_schedule(inp, W)
    got, glse = run_decode_balanced(inp, W, kernel)
    bk, kg = decode_schedule(inp, 1, kernel)
    print(check_against_oracle(inp, got, glse, f"{what} W={W}", entry="decode", split_granules=segs,
                               sched=dict(tile_n=bk, interleave=kg, granule=GRANULE)), flush=True)
    return got


def test_schedule_matches_definition_many_sequences():
    # 3000 sequences (three chunks of the schedule kernel's 1024-thread scan), lengths 0 .. 300 with
    # runs of empty ones, two query tokens each, a causal 100-key window; several worker counts
    rng = np.random.default_rng(3)
    sk = rng.integers(0, 300, 3000)
    sk[100:140] = 0
    inp = gen.make_paged(70, sk, 4, 2, 64, 64, page_size=16, sq=2, varlen_q=True, causal=True, window_left=100)
    for W in (1, 7, 512, 4096, 60000):
        _check_schedule(inp, W, with_decode=W <= 512)
    # 64 sequences (the largest batch whose decode waves derive the schedule themselves) and 65
    for nb in (64, 65):
        small = gen.make_paged(76 + nb, rng.integers(0, 3000, nb), 8, 2, 128, 128, page_size=16, sq=1, varlen_q=True)
        _check_schedule(small, 97)


@pytest.mark.parametrize("kernel", [binding.DECODE_HEAD_GROUP, binding.DECODE_PER_HEAD])
@pytest.mark.parametrize("num_workers", [None, 37])
def test_balanced_paged_gqa(num_workers, kernel):
    # the paged GQA decode workload at batch 16 (lengths 1k-8k, per-(b, kv head) descales, q and k
    # milder: helpers.milder_descales)
    inp = milder_descales(gen.paged_gqa_decode(1, batch=16), 83)
    _balanced_check(inp, num_workers, f"balanced paged decode b16 kernel={kernel}", kernel)


def test_balanced_skewed_lengths():
    # lengths from 0 to 8000 in one batch: many workers inside the long sequences, several short
    # sequences inside one worker
    inp = gen.make_paged(71, [8000, 1, 0, 64, 65, 3000, 17, 129, 5000, 0, 2], 32, 8, 128, 128, page_size=16, sq=1,
                         varlen_q=True, descales=SHARP)
    _balanced_check(inp, 64, "balanced decode skewed lengths")
    _balanced_check(inp, 5, "balanced decode skewed lengths")


@pytest.mark.parametrize("causal,wl", [(True, -1), (True, 100), (False, -1)])
def test_balanced_multi_token(causal, wl):
    inp = gen.make_paged(72, [300, 1000, 64, 1], 8, 2, 128, 128, page_size=64, sq=4, varlen_q=True, causal=causal,
                         window_left=wl, descales=SHARP)
    _balanced_check(inp, 9, f"balanced decode sq4 causal{causal} wl{wl}")


@pytest.mark.parametrize("d,dv", [(64, 64), (96, 96), (256, 256), (192, 128)])
def test_balanced_head_dims_contiguous_and_paged(d, dv):
    inp = gen.make_paged(73 + d, [500, 77, 1200], 16, 4, d, dv, page_size=16, sq=1, varlen_q=True)
    _balanced_check(inp, 11, f"balanced decode d{d} dv{dv} paged")
    dense = gen.make_dense(74 + d, 3, 1, 777, 8, 2, d, dv, descales=SHARP)
    _balanced_check(dense, 6, f"balanced decode d{d} dv{dv} dense")


def test_balanced_with_sink_and_long_kv():
    base = milder_descales(gen.paged_gqa_decode(1, batch=8, lo=1024, hi=4096), 84)
    _balanced_check(gen.with_sink(base, 10, mean=4.0, std=2.0), None, "balanced decode with sink")
    _balanced_check(gen.long_kv_decode(3, batch=2, seqlen=32768), None, "balanced long-KV decode 32k")


def test_balanced_partials_match_oracle_ranges():
    # every segment's partial (O normalized over the segment's keys, LSE) against the oracle on
    # that key range
    inp = gen.make_paged(75, [700, 1500, 90, 0, 2048], 8, 2, 128, 128, page_size=16, sq=2, varlen_q=True, causal=True)
    W = 13
    segs = _check_schedule(inp, W)
    q, k, v, kw = tensors(inp)
    sched = torch.empty(binding.load().fa8_decode_schedule_bytes(inp.batch) // 4, dtype=torch.int32, device=q.device)
    op, lp = binding.decode_scheduled(q, k, v, num_workers=W, schedule=sched, **kw)
    torch.cuda.synchronize()
    op, lp = op.cpu().numpy(), lp.cpu().numpy()
    _, _, pst, _ = balanced_schedule(inp, W)
    sq_all, sk_all = oracle.seqlens(inp)
    n_checked = 0
    for b in range(inp.batch):
        for jj, (g0, g1) in enumerate(segs[b]):
            slot = int(pst[b]) + jj
            n = int(sq_all[b])
            rb = np.repeat(np.full(n, b, np.int32), inp.heads_q)
            ri = np.repeat(np.arange(n, dtype=np.int32), inp.heads_q)
            rh = np.tile(np.arange(inp.heads_q, dtype=np.int32), n)
            klo = np.full(len(rb), g0 * GRANULE, np.int64)
            khi = np.full(len(rb), g1 * GRANULE, np.int64)
            rows = (rb, rh, ri)
            ro, rl = oracle.attention(inp, rows=rows, key_range=(klo, khi))
            go, gl = op[slot, ri, rh].astype(np.float64), lp[slot, ri, rh]
            assert np.all(np.isfinite(go))
            # the one rule's count and bound, on the segment's keys
            err = np.abs(go - ro)
            n_bad = int((err > 2e-2 + 2e-2 * np.abs(ro)).sum())
            assert n_bad <= max(1, err.size // 1000), f"segment b{b} #{jj}: {n_bad} beyond 2e-2"
            delta = score_error(inp, rows, key_range=(klo, khi))
            assert (err <= method_bound_rows(inp, rows, ro, delta, key_range=(klo, khi))).all()
            fin = np.isfinite(rl)
            assert np.array_equal(np.isfinite(gl), fin)
            le = np.abs(gl[fin] - rl[fin])
            assert (le <= LSE_METHOD + delta[fin]).all()
            vis = np.minimum(khi, oracle.seqlens(inp)[1][rb]) - klo
            assert (le[vis[fin] >= LSE_MANY_KEYS] <= LSE_ATOL).all()
            n_checked += 1
    assert n_checked == int(pst[-1])


def test_balanced_graph_replay_sees_new_lengths():
    # schedule, partials and combine captured once; replays with the lengths changed in place
    # between them must match eager runs on the new lengths bit for bit (a fresh schedule each
    # replay)
    inp = gen.paged_gqa_decode(1, batch=8, lo=1024, hi=4096)
    q, k, v, kw = tensors(inp)
    W = binding.decode_num_workers(q, k, v, **kw)
    used = kw["seqused_k"]
    out = torch.empty((8, 32, 128), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((32, 8), dtype=torch.float32, device=q.device)
    sched = torch.empty(binding.load().fa8_decode_schedule_bytes(8) // 4, dtype=torch.int32, device=q.device)
    op = torch.empty((W + 8, 1, 32, 128), dtype=torch.float32, device=q.device)
    lp = torch.empty((W + 8, 1, 32), dtype=torch.float32, device=q.device)

    def step():
        binding.decode_scheduled(q, k, v, num_workers=W, schedule=sched, o_partial=op, lse_partial=lp, **kw)
        binding.combine_scheduled(op, lp, sched, num_workers=W, batch=8, max_seqlen_q=1, heads_q=32, dv=128, out=out,
                                  cu_seqlens_q=kw["cu_seqlens_q"], lse=lse)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    orig = used.clone()
    for r, scale in enumerate((1.0, 0.5, 0.25, 1.0)):
        used.copy_((orig.float() * scale).to(torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got_o, out) and torch.equal(got_l, lse), f"replay {r}"
    used.copy_(orig)
    torch.cuda.synchronize()

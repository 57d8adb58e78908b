"""The three entry points captured in one HIP graph (torch.cuda.CUDAGraph over the binding's
calls on the capturing stream) and replayed several times, with eager work and synchronizations
between the replays: every replay must reproduce the eager results bit for bit. Launch choices
come from host-known values only and the library allocates and synchronizes nothing, so the
captured launches are the eager ones."""
import numpy as np
import pytest
import torch

from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

from helpers import tensors

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    dec = gen.paged_gqa_decode(1, batch=8, lo=1024, hi=4096)
    pre = gen.make_dense(7, 2, 300, 517, 16, 2, 128, 128, causal=True, descales=(0.5, 0.5, 1.5))
    dq, dk, dv, dkw = tensors(dec)
    pq, pk, pv, pkw = tensors(pre)
    B, HQ, SQ, DV = dec.batch, dec.heads_q, dec.max_seqlen_q, dec.dv
    S = binding.decode_num_splits_for(dq, dk, dv, **dkw)
    op = torch.empty((S, B, SQ, HQ, DV), dtype=torch.float32, device=dev)
    lp = torch.empty((S, B, SQ, HQ), dtype=torch.float32, device=dev)
    d_out = torch.empty((dq.shape[0], HQ, DV), dtype=torch.bfloat16, device=dev)
    p_out = torch.empty(tuple(pq.shape[:-1]) + (pre.dv,), dtype=torch.bfloat16, device=dev)
    p_lse = torch.empty((pre.batch, pre.heads_q, pre.max_seqlen_q), dtype=torch.float32, device=dev)

    def work():
        binding.decode_splitkv(dq, dk, dv, num_splits=S, o_partial=op, lse_partial=lp, **dkw)
        binding.combine(op, lp, batch=B, max_seqlen_q=SQ, heads_q=HQ, dv=DV, out=d_out,
                        cu_seqlens_q=dkw["cu_seqlens_q"])
        binding.prefill(pq, pk, pv, out=p_out, lse=p_lse, **pkw)

    work()
    torch.cuda.synchronize()
    ref_d, ref_p, ref_l = d_out.clone(), p_out.clone(), p_lse.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream's side, as torch recommends
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for t in (d_out, p_out, p_lse):
            t.fill_(float("nan"))          # a plain kernel, not a memset node
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d_out.view(torch.int16), ref_d.view(torch.int16)), f"decode output differs on replay {rep}"
        assert torch.equal(p_out.view(torch.int16), ref_p.view(torch.int16)), f"prefill output differs on replay {rep}"
        assert torch.equal(p_lse.view(torch.int32), ref_l.view(torch.int32)), f"prefill LSE differs on replay {rep}"
        # eager work of the program between replays
        work()
        torch.cuda.synchronize()
        assert torch.equal(d_out.view(torch.int16), ref_d.view(torch.int16))
    print(f"graph replays bit-identical to eager (decode S={S}, prefill 300x517)", flush=True)

"""Page bases beyond 4 GiB. A paged input is placed at the end of a K/V page pool of more than
5 GiB (the block table shifted by the pad pages, which are never read), and every entry point
that walks a block table must give bit-identical results to the same input in a small pool: the
byte offset of a page is formed in 64 bits, and only the row offsets inside one page are 32-bit
(the limit the library checks). Covers the several-heads decode kernel, the one-kv-head kernel
with small pages (per-lane page lookup) and with 64-token pages (one page per load
instruction), and the paged prefill."""
import numpy as np
import pytest
import torch

from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

from helpers import out_dtype, tensors

pytestmark = pytest.mark.gpu

PAD_BYTES = 5 << 30


def _shift(k, v, bt):
    """The pools k, v ([pages, page_size, hkv, d]) copied to the end of pools with at least
    PAD_BYTES of pad pages in front, and the block table shifted to match."""
    pad = -(-PAD_BYTES // min(k[0].numel(), v[0].numel()))   # E4M3 bytes: one page's bytes
    big_k = torch.empty((pad + k.shape[0],) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    big_v = torch.empty((pad + v.shape[0],) + tuple(v.shape[1:]), dtype=v.dtype, device=v.device)
    big_k[pad:] = k
    big_v[pad:] = v
    assert pad * k[0].numel() >= (1 << 32) and pad * v[0].numel() >= (1 << 32)
    return big_k, big_v, bt + pad


def _decode_both(inp, kernel):
    kern = binding.DECODE_PER_HEAD if kernel == "lanes" else binding.DECODE_AUTO
    q, k, v, kw = tensors(inp)
    res = []
    for pools in ((k, v, kw["block_table"]), _shift(k, v, kw["block_table"])):
        kk, vv, bt = pools
        args = dict(kw, block_table=bt)
        out, lse = binding.decode(q, kk, vv, out_dtype=out_dtype(inp), return_lse=True, kernel=kern, **args)
        torch.cuda.synchronize()
        res.append((out.float().cpu(), lse.cpu()))
        del kk, vv
    torch.cuda.empty_cache()
    return res


@pytest.mark.parametrize("kernel", ["heads", "lanes"])
def test_paged_gqa_decode_pages_beyond_4gib(kernel):
    inp = gen.paged_gqa_decode(1, batch=8, lo=1024, hi=4096)
    print(f"decode ({kernel} kernel), pages beyond 4 GiB: B{inp.batch} page {inp.page_size}", flush=True)
    (o0, l0), (o1, l1) = _decode_both(inp, kernel)
    assert torch.isfinite(o0).all()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_long_pages_decode_pages_beyond_4gib():
    inp = gen.long_kv_decode(3, batch=2, seqlen=8192)
    print(f"decode (64-token pages), pages beyond 4 GiB: B{inp.batch} Sk {inp.max_seqlen_k}", flush=True)
    (o0, l0), (o1, l1) = _decode_both(inp, "default")
    assert torch.isfinite(o0).all()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_paged_prefill_pages_beyond_4gib():
    inp = gen.make_paged(7, [300, 17, 640, 129], 8, 2, 128, 128, page_size=16, sq=40, varlen_q=False, causal=True)
    print("paged prefill, pages beyond 4 GiB", flush=True)
    q, k, v, kw = tensors(inp)
    res = []
    for kk, vv, bt in ((k, v, kw["block_table"]), _shift(k, v, kw["block_table"])):
        out, lse = binding.prefill(q, kk, vv, out_dtype=out_dtype(inp), return_lse=True, **dict(kw, block_table=bt))
        torch.cuda.synchronize()
        res.append((out.float().cpu(), lse.cpu()))
        del kk, vv
    torch.cuda.empty_cache()
    (o0, l0), (o1, l1) = res
    assert torch.isfinite(o0).all()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)

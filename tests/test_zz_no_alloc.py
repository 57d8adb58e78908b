"""fa8_fwd_decode_noalloc (for callers that cannot allocate) against the caller-buffer path it
varies, fa8_fwd_decode_splitkv into caller partials followed by fa8_combine: bit-identical outputs
and LSEs on two calls in a row, the second with a smaller problem (the scratch keeps the first
call's contents), and sizes beyond the scratch rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

from helpers import tensors

pytestmark = pytest.mark.gpu


def _both(inp, num_splits):
    q, k, v, kw = tensors(inp)
    ref, ref_lse = binding.decode(q, k, v, num_splits=num_splits, return_lse=True, **kw)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    binding.decode_noalloc(q, k, v, out=out, lse=lse, num_splits=num_splits or 0, **kw)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse


def test_noalloc_decode_matches_caller_buffers_twice():
    big = gen.paged_gqa_decode(1, batch=16, lo=1024, hi=4096)            # 32/8 heads, d128, pages of 16
    small = gen.make_paged(61, [700, 33, 1], 8, 2, 128, 128, page_size=16, sq=1, varlen_q=True)
    for inp, ns in ((big, 8), (small, 3)):
        ref, ref_lse, out, lse = _both(inp, ns)
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), inp.name
    # the library's own split count (num_splits = 0), and a long single-kv-head problem (many splits)
    ref, ref_lse, out, lse = _both(gen.long_kv_decode(3, batch=2, seqlen=32768), None)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_noalloc_decode_rejects_partials_beyond_the_scratch():
    # 256 splits x 64 sequences x 32 heads x (128 + 1) x 4 bytes > 32 MiB: rejected, nothing launched
    inp = gen.make_paged(62, [100] * 64, 32, 8, 128, 128, page_size=16, sq=1, varlen_q=True)
    q, k, v, kw = tensors(inp)
    out = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=q.device)
    assert binding.decode_workspace_bytes(256, 64, 1, 32, 128) > binding.NOALLOC_SCRATCH_BYTES
    with pytest.raises(binding.FA8Error) as e:
        binding.decode_noalloc(q, k, v, out=out, num_splits=256, **kw)
    assert e.value.status == binding.FA8_ERR_INVALID and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 0)

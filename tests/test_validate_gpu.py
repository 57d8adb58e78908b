"""The optional device-data validator (FA8_VALIDATE=1, include/fa8.h): index arrays that break the
caller's contract are reported as FA8_ERR_INVALID before anything is launched, valid ones give
results bit-identical to a run without the validator, and the validator sees index data written
on the caller's stream just before the call. Every buffer is sized so that even a launch would
stay inside its allocations (the checks do not rely on the validator to be memory-safe)."""
import os

import numpy as np
import pytest
import torch

from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

from helpers import tensors

pytestmark = pytest.mark.gpu


@pytest.fixture
def validator():
    old = os.environ.get("FA8_VALIDATE")
    os.environ["FA8_VALIDATE"] = "1"
    yield
    if old is None:
        del os.environ["FA8_VALIDATE"]
    else:
        os.environ["FA8_VALIDATE"] = old


def _paged():
    # 4 sequences of up to 300 keys, 16-token pages; block table 64 entries wide (1024 keys), every
    # entry a real page, and the pool placed one page into a larger buffer so that page index -1
    # is still inside the allocation
    inp = gen.make_paged(50, [300, 17, 256, 129], 8, 2, 128, 128, page_size=16, sq=1, varlen_q=True,
                         max_seqlen_k=320)
    q, k, v, kw = tensors(inp)
    n = k.shape[0]
    kbig = torch.zeros((n + 1,) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    vbig = torch.zeros_like(kbig)
    kbig[1:], vbig[1:] = k, v
    wide = torch.full((4, 64), n - 1, dtype=torch.int32, device=k.device)
    wide[:, :kw["block_table"].shape[1]] = kw["block_table"]
    kw = dict(kw, block_table=wide)
    return q, kbig[1:], vbig[1:], kw


def _decode(q, k, v, kw, stream=None):
    out = binding.decode(q, k, v, num_splits=3, return_lse=True, stream=stream, **kw)
    torch.cuda.synchronize()
    return out


def test_validator_valid_inputs_bitwise(validator):
    q, k, v, kw = _paged()
    a, la = _decode(q, k, v, kw)
    os.environ["FA8_VALIDATE"] = "0"
    b, lb = _decode(q, k, v, kw)
    assert torch.equal(a, b) and torch.equal(la, lb)
    # prefill on varlen K/V
    inp = gen.make_varlen(51, [40, 1, 77], [100, 64, 300], 8, 2, 128, 128, causal=True)
    qq, kk, vv, kw2 = tensors(inp)
    os.environ["FA8_VALIDATE"] = "1"
    c = binding.prefill(qq, kk, vv, **kw2)
    os.environ["FA8_VALIDATE"] = "0"
    d = binding.prefill(qq, kk, vv, **kw2)
    torch.cuda.synchronize()
    assert torch.equal(c, d)


def test_validator_rejects_length_beyond_max(validator):
    q, k, v, kw = _paged()
    used = kw["seqused_k"].clone()
    used[2] = kw["max_seqlen_k"] + 1          # still covered by the 64-entry table
    with pytest.raises(binding.FA8Error) as e:
        _decode(q, k, v, dict(kw, seqused_k=used))
    assert e.value.status == binding.FA8_ERR_INVALID and "seqused_k" in str(e.value)


def test_validator_rejects_negative_page(validator):
    q, k, v, kw = _paged()
    table = kw["block_table"].clone()
    table[1, 0] = -1                           # inside sequence 1's 17 keys
    with pytest.raises(binding.FA8Error) as e:
        _decode(q, k, v, dict(kw, block_table=table))
    assert e.value.status == binding.FA8_ERR_INVALID and "page" in str(e.value)


def test_validator_rejects_non_monotone_cu_seqlens(validator):
    inp = gen.make_varlen(52, [40, 30, 77], [100, 64, 300], 8, 2, 128, 128, causal=True)
    q, k, v, kw = tensors(inp)
    bad_q = torch.tensor([0, 40, 35, 147], dtype=torch.int32, device=q.device)     # a negative length
    with pytest.raises(binding.FA8Error) as e:
        binding.prefill(q, k, v, **dict(kw, cu_seqlens_q=bad_q))
    assert e.value.status == binding.FA8_ERR_INVALID and "cu_seqlens_q" in str(e.value)
    bad_k = torch.tensor([0, 100, 90, 464], dtype=torch.int32, device=q.device)
    with pytest.raises(binding.FA8Error) as e:
        binding.prefill(q, k, v, **dict(kw, cu_seqlens_k=bad_k))
    assert e.value.status == binding.FA8_ERR_INVALID and "cu_seqlens_k" in str(e.value)
    torch.cuda.synchronize()


def test_validator_sees_writes_on_the_callers_stream(validator):
    # the bad length is written on a side stream behind a ~20 ms spin kernel, and the decode is
    # called on that stream: the validator must wait for it (it synchronizes the stream)
    q, k, v, kw = _paged()
    used = kw["seqused_k"].clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)
        used[0] = kw["max_seqlen_k"] + 5
        with pytest.raises(binding.FA8Error) as e:
            binding.decode(q, k, v, num_splits=3, stream=s, **dict(kw, seqused_k=used))
    torch.cuda.synchronize()
    assert e.value.status == binding.FA8_ERR_INVALID

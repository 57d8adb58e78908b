"""GPU parity of the Q quantizer (fa8_quantize_q) with the oracle's quantizer: every E4M3 code
and every descale bit for bit (integer and byte work), bf16 and fp16 inputs, dense and varlen
layouts, decode and prefill shapes, and a quantized Q run through the prefill path."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

from helpers import check_against_oracle, prefill_tile, tensors

pytestmark = pytest.mark.gpu


def _q(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape,hkv", [((2, 300, 16, 128), 2), ((64, 1, 32, 128), 8), ((3, 77, 8, 64), 8),
                                       ((1, 40, 6, 256), 3), ((2, 33, 4, 96), 1), ((1, 17, 4, 192), 2)])
def test_quantizer_bit_exact_dense(dtype, shape, hkv):
    q = _q(shape, 1, dtype, 2.0)
    q[0, 0, 0, 0] = -0.0
    dev = torch.device("cuda:0")
    got, s = binding.quantize_q(q.to(dev), hkv)
    torch.cuda.synchronize()
    ref, rs = quant.quantize_q(q.float().numpy(), hkv)
    assert np.array_equal(got.cpu().numpy(), ref), f"{int((got.cpu().numpy() != ref).sum())} codes differ"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_quantizer_bit_exact_varlen_with_zero_and_empty_blocks():
    q = _q((120, 8, 128), 2, torch.float16, 0.05)
    cu = torch.tensor([0, 50, 50, 97, 120], dtype=torch.int32)
    q[50:97, 4:] = 0.0                                   # batch 2, kv head 1: a block of zeros
    dev = torch.device("cuda:0")
    got, s = binding.quantize_q(q.to(dev), 2, cu_seqlens_q=cu.to(dev), max_seqlen_q=50)
    torch.cuda.synchronize()
    ref, rs = quant.quantize_q(q.float().numpy(), 2, cu_seqlens_q=cu.numpy())
    assert np.array_equal(got.cpu().numpy(), ref)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert s.cpu().numpy()[1].tolist() == [1.0, 1.0] and s.cpu().numpy()[2, 1] == 1.0


def test_quantizer_block_maximum_in_every_chunk_position():
    # 293 rows = ten 32-row chunks, the last one partial: the max pass takes chunks four at a time
    # (groups 0-3, 4-7 and the partial 8-9), so each batch puts its block's one large element in
    # a different chunk (first and last of a group, the partial group, the ragged last rows);
    # the other kv head's block keeps its maximum in the first row
    rows, positions = 293, [0, 127, 128, 200, 255, 256, 292]
    q = _q((len(positions), rows, 4, 64), 9, torch.bfloat16, 0.01)
    for b, r in enumerate(positions):
        q[b, r, b % 2, 7] = 3.0 + b          # kv head 0: q heads 0 and 1
        q[b, 0, 2, 0] = -2.0                 # kv head 1
    dev = torch.device("cuda:0")
    got, s = binding.quantize_q(q.to(dev), 2)
    torch.cuda.synchronize()
    ref, rs = quant.quantize_q(q.float().numpy(), 2)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.allclose(rs[:, 0], (3.0 + np.arange(len(positions))) / 448.0, rtol=1e-2)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_quantizer_bit_exact_across_the_scale_range():
    # bf16 blocks whose maxima put s = amax / 448 exactly at 2^-96 (the smallest s of the
    # kernel's short quotient path), one bf16 step below it, among the subnormals, and up to the
    # top of the bf16 range; elements of +-0 and subnormal values inside normal blocks
    thr = 1.75 * 2.0 ** -88                      # 448 * 2^-96, a bf16 value
    below = (1.75 - 2.0 ** -7) * 2.0 ** -88      # the bf16 value just below it
    amaxes = [thr, below, 2.0 ** -126, 2.0 ** -130, 1e-30, 1e-26, 1e-3, 1.0, 448.0, 3.0e5, 1e30, 3.0e38,
              thr * 2, below / 2, 5.0e-39, 65504.0]
    g = torch.Generator().manual_seed(7)
    q = torch.empty((2, 40, 8, 64))
    for blk, a in enumerate(amaxes):
        b, kvh = divmod(blk, 8)
        x = (torch.rand((40, 64), generator=g) * 2 - 1) * a
        x[0, 0] = a if blk % 2 == 0 else -a     # the block maximum, either sign
        x[1, 0:4] = torch.tensor([0.0, -0.0, 2.0 ** -133, -(2.0 ** -140)])
        q[b, :, kvh, :] = x
    q = q.to(torch.bfloat16)
    assert torch.isfinite(q.float()).all()
    dev = torch.device("cuda:0")
    got, s = binding.quantize_q(q.to(dev), 8)
    torch.cuda.synchronize()
    ref, rs = quant.quantize_q(q.float().numpy(), 8)
    # the test's scales: both quotient paths are exercised
    sref = rs.reshape(-1)
    assert (sref >= np.float32(2.0 ** -96)).any() and (sref < np.float32(2.0 ** -96)).any()
    assert np.float32(2.0 ** -96) in sref
    diff = got.cpu().numpy() != ref
    assert not diff.any(), f"{int(diff.sum())} codes differ, first at {np.argwhere(diff)[:3].tolist()}"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_quantized_q_through_prefill():
    # bf16 Q quantized on the GPU, then the FP8 prefill with the produced per-(b, kv head) descale,
    # against the oracle on the same codes and descales
    base = gen.make_dense(30, 2, 200, 333, 8, 2, 128, 128, causal=True, descales=(None, 0.5, 1.5))
    qb = _q((2, 200, 8, 128), 3, torch.bfloat16, 0.3)
    dev = torch.device("cuda:0")
    codes, s = binding.quantize_q(qb.to(dev), 2)
    torch.cuda.synchronize()
    inp = base
    inp.q = codes.cpu().numpy()
    inp.q_descale = s.cpu().numpy()
    q, k, v, kw = tensors(inp)
    out, lse = binding.prefill(q, k, v, return_lse=True, **kw)
    torch.cuda.synchronize()
    print(check_against_oracle(inp, out.float().cpu().numpy(), lse.cpu().numpy(), "quantized q prefill",
                               sched=dict(tile_n=prefill_tile(128, 128))), flush=True)

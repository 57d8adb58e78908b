"""Seeded synthetic inputs for the FP8 attention forward.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the CPU oracle (in tests) and the HIP path consume
exactly the same bytes from it.

Draw order for every generator (one ``torch.Generator`` on the CPU, seeded once):
lengths first (when they are random), then Q, K, V (``randn`` in float32, scaled
and shifted, then cast to ``torch.float8_e4m3fn``, i.e. round to nearest even),
then the block-table page permutation (when paged), then descales (when random).

Shapes follow the usual flash-attention conventions:
  * dense Q/O ``[B, Sq, H, d]``; varlen Q/O ``[total_q, H, d]`` with ``cu_seqlens_q``;
  * dense K/V ``[B, Sk, Hkv, d]``; varlen ``[total_k, Hkv, d]`` with ``cu_seqlens_k``;
  * paged K/V ``[num_pages, page_size, Hkv, d]`` with ``block_table [B, W]`` and
    ``seqused_k [B]``; the last page of the pool is a spare ("poison") page that
    unused table entries point at.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class AttnInputs:
    batch: int
    heads_q: int
    heads_kv: int
    d: int
    dv: int
    q: np.ndarray                      # uint8 E4M3FN bytes
    k: np.ndarray
    v: np.ndarray
    max_seqlen_q: int
    max_seqlen_k: int
    cu_seqlens_q: Optional[np.ndarray] = None   # int32 [B+1]
    cu_seqlens_k: Optional[np.ndarray] = None   # int32 [B+1]
    seqused_k: Optional[np.ndarray] = None      # int32 [B]
    block_table: Optional[np.ndarray] = None    # int32 [B, W]
    page_size: int = 0
    q_descale: Optional[np.ndarray] = None      # float32, shape () or [B, Hkv]
    k_descale: Optional[np.ndarray] = None
    v_descale: Optional[np.ndarray] = None
    softmax_scale: float = 0.0                  # <= 0 means 1/sqrt(d)
    causal: bool = False
    window_left: int = -1
    window_right: int = -1
    out_dtype: str = "bf16"                     # "bf16" | "fp16"
    name: str = ""
    sink: Optional[np.ndarray] = None           # float32 [Hq] learnable sink logits, or None
    # MXFP8 block scales (E8M0 bytes), dense layouts: Q [B, Sq, Hq, d/32] and K [B, Sk, Hkv,
    # d/32] per 32 elements of d; V [B, ceil(Sk/32), Hkv, dv] per 32 keys
    q_mx: Optional[np.ndarray] = None
    k_mx: Optional[np.ndarray] = None
    v_mx: Optional[np.ndarray] = None

    # --- per-batch lengths, resolved from whichever layout is in use ---
    def seqlens_q(self) -> np.ndarray:
        if self.cu_seqlens_q is not None:
            return np.diff(self.cu_seqlens_q).astype(np.int64)
        return np.full(self.batch, self.max_seqlen_q, np.int64)

    def seqlens_k(self) -> np.ndarray:
        if self.seqused_k is not None:
            return self.seqused_k.astype(np.int64)
        if self.cu_seqlens_k is not None:
            return np.diff(self.cu_seqlens_k).astype(np.int64)
        return np.full(self.batch, self.max_seqlen_k, np.int64)

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def varlen_q(self) -> bool:
        return self.cu_seqlens_q is not None


def e4m3_bytes(gen: torch.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """N(mean, std^2) float32 samples cast to E4M3FN (round to nearest even), as uint8."""
    x = torch.randn(tuple(int(s) for s in shape), generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _descale(gen: torch.Generator, mode, batch: int, heads_kv: int):
    """mode: None (omitted), a float (0-d), or ("uniform", lo, hi) per (b, kv_head)."""
    if mode is None:
        return None
    if isinstance(mode, (int, float)):
        return np.array(float(mode), dtype=np.float32)
    kind, lo, hi = mode
    assert kind == "uniform"
    u = torch.rand((batch, heads_kv), generator=gen, dtype=torch.float32)
    return (lo + (hi - lo) * u).numpy().astype(np.float32)


def make_dense(seed: int, batch: int, sq: int, sk: int, heads_q: int, heads_kv: int, d: int, dv: int,
               causal: bool = False, window_left: int = -1, window_right: int = -1,
               v_mean: float = 0.0, descales=(None, None, None), softmax_scale: float = 0.0,
               out_dtype: str = "bf16", name: str = "") -> AttnInputs:
    """Fixed-length BSHD Q/K/V."""
    g = torch.Generator().manual_seed(seed)
    q = e4m3_bytes(g, (batch, sq, heads_q, d))
    k = e4m3_bytes(g, (batch, sk, heads_kv, d))
    v = e4m3_bytes(g, (batch, sk, heads_kv, dv), mean=v_mean)
    dq, dk, dvs = (_descale(g, m, batch, heads_kv) for m in descales)
    return AttnInputs(batch, heads_q, heads_kv, d, dv, q, k, v, sq, sk,
                      q_descale=dq, k_descale=dk, v_descale=dvs, softmax_scale=softmax_scale,
                      causal=causal, window_left=window_left, window_right=window_right,
                      out_dtype=out_dtype, name=name)


def make_varlen(seed: int, seqlens_q, seqlens_k, heads_q: int, heads_kv: int, d: int, dv: int,
                causal: bool = False, window_left: int = -1, window_right: int = -1,
                v_mean: float = 0.0, descales=(None, None, None), softmax_scale: float = 0.0,
                out_dtype: str = "bf16", name: str = "") -> AttnInputs:
    """Packed varlen Q and K/V (cu_seqlens); lengths are given explicitly."""
    sq = np.asarray(seqlens_q, np.int64)
    sk = np.asarray(seqlens_k, np.int64)
    batch = len(sq)
    g = torch.Generator().manual_seed(seed)
    q = e4m3_bytes(g, (int(sq.sum()), heads_q, d))
    k = e4m3_bytes(g, (int(sk.sum()), heads_kv, d))
    v = e4m3_bytes(g, (int(sk.sum()), heads_kv, dv), mean=v_mean)
    dq, dk, dvs = (_descale(g, m, batch, heads_kv) for m in descales)
    cuq = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    cuk = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    return AttnInputs(batch, heads_q, heads_kv, d, dv, q, k, v, int(sq.max()), int(sk.max()),
                      cu_seqlens_q=cuq, cu_seqlens_k=cuk,
                      q_descale=dq, k_descale=dk, v_descale=dvs, softmax_scale=softmax_scale,
                      causal=causal, window_left=window_left, window_right=window_right,
                      out_dtype=out_dtype, name=name)


def make_paged(seed: int, seqlens_k, heads_q: int, heads_kv: int, d: int, dv: int, page_size: int,
               sq: int = 1, varlen_q: bool = True, causal: bool = False, window_left: int = -1,
               window_right: int = -1, v_mean: float = 0.0, descales=(None, None, None),
               softmax_scale: float = 0.0, out_dtype: str = "bf16", max_seqlen_k: Optional[int] = None,
               extra_pages: int = 1, name: str = "", gen: Optional[torch.Generator] = None) -> AttnInputs:
    """Paged K/V cache with a random page permutation and sq query tokens per sequence.

    Every sequence b owns ceil(s_b / page_size) pages taken, in order, from one random
    permutation of the pool; table entries past a sequence's own pages point at the
    pool's last page (a spare page no sequence owns).
    """
    sk = np.asarray(seqlens_k, np.int64)
    batch = len(sk)
    g = gen if gen is not None else torch.Generator().manual_seed(seed)
    npages_b = (sk + page_size - 1) // page_size
    used = int(npages_b.sum())
    num_pages = used + extra_pages
    mx = int(max_seqlen_k if max_seqlen_k is not None else sk.max())
    width = max(1, (mx + page_size - 1) // page_size)
    if varlen_q:
        q = e4m3_bytes(g, (batch * sq, heads_q, d))
    else:
        q = e4m3_bytes(g, (batch, sq, heads_q, d))
    k = e4m3_bytes(g, (num_pages, page_size, heads_kv, d))
    v = e4m3_bytes(g, (num_pages, page_size, heads_kv, dv), mean=v_mean)
    perm = torch.randperm(used, generator=g).numpy().astype(np.int32)
    table = np.full((batch, width), num_pages - 1, np.int32)
    off = 0
    for b in range(batch):
        n = int(npages_b[b])
        table[b, :n] = perm[off:off + n]
        off += n
    dq, dk, dvs = (_descale(g, m, batch, heads_kv) for m in descales)
    cuq = np.arange(0, batch * sq + 1, sq, dtype=np.int32) if varlen_q else None
    return AttnInputs(batch, heads_q, heads_kv, d, dv, q, k, v, sq, mx,
                      cu_seqlens_q=cuq, seqused_k=sk.astype(np.int32), block_table=table,
                      page_size=page_size, q_descale=dq, k_descale=dk, v_descale=dvs,
                      softmax_scale=softmax_scale, causal=causal, window_left=window_left,
                      window_right=window_right, out_dtype=out_dtype, name=name)


def with_sink(inp: AttnInputs, seed: int, mean: float = 0.0, std: float = 1.0) -> AttnInputs:
    """A copy of inp with a learnable sink: one fp32 logit per query head, N(mean, std^2), drawn
    from its own seeded generator (the other tensors are shared, not redrawn)."""
    g = torch.Generator().manual_seed(seed)
    z = torch.randn((inp.heads_q,), generator=g, dtype=torch.float32) * std + mean
    return dataclasses.replace(inp, sink=z.numpy().astype(np.float32), name=inp.name + "_sink")


def with_mx(inp: AttnInputs, seed: int, lo: int = 122, hi: int = 132) -> AttnInputs:
    """A copy of a dense input with MXFP8 block scales: E8M0 bytes uniform in [lo, hi] (scales
    2^(lo-127) .. 2^(hi-127)), drawn Q, K, V in that order from their own seeded generator; the
    E4M3 elements are the input's own. The per-tensor descales are dropped (the block scales
    take their place)."""
    if inp.cu_seqlens_q is not None or inp.cu_seqlens_k is not None or inp.block_table is not None:
        raise ValueError("MX scales are generated for dense layouts")
    g = torch.Generator().manual_seed(seed)
    B, Sq, Sk = inp.batch, inp.max_seqlen_q, inp.max_seqlen_k
    qs = torch.randint(lo, hi + 1, (B, Sq, inp.heads_q, inp.d // 32), generator=g, dtype=torch.int32)
    ks = torch.randint(lo, hi + 1, (B, Sk, inp.heads_kv, inp.d // 32), generator=g, dtype=torch.int32)
    vs = torch.randint(lo, hi + 1, (B, (Sk + 31) // 32, inp.heads_kv, inp.dv), generator=g, dtype=torch.int32)
    return dataclasses.replace(inp, q_mx=qs.numpy().astype(np.uint8), k_mx=ks.numpy().astype(np.uint8),
                               v_mx=vs.numpy().astype(np.uint8), q_descale=None, k_descale=None,
                               v_descale=None, name=inp.name + "_mx")


def _mx_blocks(x: torch.Tensor, axis: int):
    """MXFP8 encoding of float32 x in blocks of 32 consecutive elements along `axis` (the tail
    block zero-padded): E8M0 scale 2^X with X = ceil(log2(amax / 448)), the smallest power of two
    that keeps the block's largest magnitude at or below 448 (clamped to [-127, 127]; X = -127
    for an all-zero block), and E4M3 elements x / 2^X cast with round to nearest even (torch's
    cast). Returns (uint8 codes shaped like x, uint8 scale bytes with that axis divided by 32)."""
    x = x.movedim(axis, -1)
    n = x.shape[-1]
    nb = (n + 31) // 32
    pad = torch.zeros(x.shape[:-1] + (nb * 32,), dtype=torch.float32)
    pad[..., :n] = x
    blk = pad.reshape(x.shape[:-1] + (nb, 32))
    amax = blk.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.full_like(amax, -127.0))
    e = e.clamp(-127, 127)
    codes = (blk / torch.exp2(e)[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    codes = codes.reshape(pad.shape)[..., :n].movedim(-1, axis).contiguous()
    scales = (e + 127).to(torch.uint8).movedim(-1, axis).contiguous()
    return codes.numpy(), scales.numpy()


def _mx_blocks_random(x: torch.Tensor, axis: int, gen: torch.Generator, lo: int, hi: int):
    """MXFP8 encoding of float32 x in blocks of 32 along `axis` with a random shared exponent per
    block: X uniform in [lo, hi], raised where needed to ceil(log2(amax / 448)) so that no element
    exceeds 448; elements x / 2^X cast to E4M3 (round to nearest even). The dequantized values are
    x up to the E4M3 rounding, while the element magnitudes and scale bytes vary by up to
    2^(hi - lo) from block to block."""
    x = x.movedim(axis, -1)
    n = x.shape[-1]
    nb = (n + 31) // 32
    pad = torch.zeros(x.shape[:-1] + (nb * 32,), dtype=torch.float32)
    pad[..., :n] = x
    blk = pad.reshape(x.shape[:-1] + (nb, 32))
    amax = blk.abs().amax(dim=-1)
    need = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.full_like(amax, -127.0))
    e = torch.randint(lo, hi + 1, amax.shape, generator=gen).to(torch.float32)
    e = torch.maximum(e, need).clamp(-127, 127)
    codes = (blk / torch.exp2(e)[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    codes = codes.reshape(pad.shape)[..., :n].movedim(-1, axis).contiguous()
    scales = (e + 127).to(torch.uint8).movedim(-1, axis).contiguous()
    return codes.numpy(), scales.numpy()


def make_mx_random_exponents(seed: int, batch: int, sq: int, sk: int, heads_q: int, heads_kv: int, d: int,
                             dv: int, lo: int = -5, hi: int = 5, causal: bool = False, window_left: int = -1,
                             out_dtype: str = "bf16") -> AttnInputs:
    """Like make_mx, but every block takes a random shared exponent in [lo, hi] (at least the one
    its largest element needs): the attention values are N(0,1) data as in make_mx, while the
    E4M3 elements and E8M0 scale bytes spread over 2^(hi - lo) from block to block. Draw order:
    Q, K, V values, then the exponents of Q, K, V blocks."""
    g = torch.Generator().manual_seed(seed)
    qf = torch.randn((batch, sq, heads_q, d), generator=g, dtype=torch.float32)
    kf = torch.randn((batch, sk, heads_kv, d), generator=g, dtype=torch.float32)
    vf = torch.randn((batch, sk, heads_kv, dv), generator=g, dtype=torch.float32)
    q, qs = _mx_blocks_random(qf, -1, g, lo, hi)
    k, ks = _mx_blocks_random(kf, -1, g, lo, hi)
    v, vs = _mx_blocks_random(vf, 1, g, lo, hi)
    return AttnInputs(batch, heads_q, heads_kv, d, dv, q, k, v, sq, sk, causal=causal, window_left=window_left,
                      out_dtype=out_dtype, name=f"mx_random_exponents_{lo}_{hi}", q_mx=qs, k_mx=ks, v_mx=vs)


def make_mx(seed: int, batch: int, sq: int, sk: int, heads_q: int, heads_kv: int, d: int, dv: int,
            causal: bool = False, window_left: int = -1, window_right: int = -1, v_mean: float = 0.0,
            softmax_scale: float = 0.0, out_dtype: str = "bf16", name: str = "") -> AttnInputs:
    """Fixed-length BSHD Q/K/V drawn N(0,1) in float32 (V shifted by v_mean) and encoded as MXFP8:
    blocks of 32 along d for Q and K, along the keys for V (_mx_blocks)."""
    g = torch.Generator().manual_seed(seed)
    qf = torch.randn((batch, sq, heads_q, d), generator=g, dtype=torch.float32)
    kf = torch.randn((batch, sk, heads_kv, d), generator=g, dtype=torch.float32)
    vf = torch.randn((batch, sk, heads_kv, dv), generator=g, dtype=torch.float32) + v_mean
    q, qs = _mx_blocks(qf, -1)
    k, ks = _mx_blocks(kf, -1)
    v, vs = _mx_blocks(vf, 1)
    return AttnInputs(batch, heads_q, heads_kv, d, dv, q, k, v, sq, sk, softmax_scale=softmax_scale,
                      causal=causal, window_left=window_left, window_right=window_right, out_dtype=out_dtype,
                      name=name, q_mx=qs, k_mx=ks, v_mx=vs)


def random_lengths(gen: torch.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi] (inclusive)."""
    return torch.randint(lo, hi + 1, (n,), generator=gen).numpy().astype(np.int64)


# ---------------------------------------------------------------------------
# The five workloads of the method's headline measurements, optionally scaled down
# for parity tests. `scale` divides lengths; shapes/heads/dtypes are kept.
# ---------------------------------------------------------------------------

def tiny(seed: int = 0) -> AttnInputs:
    """B=1, H=1, Sq=128, Sk=256, d=dv=64, non-causal, descales 1.0, bf16 out."""
    return make_dense(seed, 1, 128, 256, 1, 1, 64, 64, descales=(1.0, 1.0, 1.0), name="tiny_b1_h1_q128_k256_d64")


def paged_gqa_decode(seed: int = 1, batch: int = 64, lo: int = 1024, hi: int = 8192, page_size: int = 16,
                     heads_q: int = 32, heads_kv: int = 8, d: int = 128, sq: int = 1,
                     max_seqlen_k: Optional[int] = None, causal: bool = False) -> AttnInputs:
    """Llama-3.1-8B-like decode: 32/8 heads, d=128, 1 query token, 16-token pages, lengths
    uniform in [1k, 8k], random block table, per-(b, kv_head) descales uniform in [0.5, 2]."""
    g = torch.Generator().manual_seed(seed)
    sk = random_lengths(g, batch, lo, hi)
    mx = max_seqlen_k if max_seqlen_k is not None else hi
    return make_paged(seed, sk, heads_q, heads_kv, d, d, page_size, sq=sq, varlen_q=True, causal=causal,
                      descales=(("uniform", 0.5, 2.0),) * 3, max_seqlen_k=mx, gen=g,
                      name=f"paged_gqa_decode_b{batch}_h{heads_q}x{heads_kv}_d{d}_p{page_size}_k{lo}-{hi}")


def causal_prefill(seed: int = 2, batch: int = 2, seqlen: int = 8192, heads_q: int = 32, heads_kv: int = 8,
                   d: int = 128, descales=(0.5, 0.5, 1.5)) -> AttnInputs:
    """Causal prefill B=2, Sq=Sk=8192, 32/8 heads, d=128, scalar descales, bf16 out."""
    return make_dense(seed, batch, seqlen, seqlen, heads_q, heads_kv, d, d, causal=True, descales=descales,
                      name=f"causal_prefill_b{batch}_s{seqlen}_h{heads_q}x{heads_kv}_d{d}")


def long_kv_decode(seed: int = 3, batch: int = 4, seqlen: int = 131072, page_size: int = 64, heads_q: int = 8,
                   heads_kv: int = 1, d: int = 128, v_mean: float = 0.5) -> AttnInputs:
    """Long-KV decode: 8/1 heads, d=128, one query token, 64-token pages, V ~ N(0.5, 1)."""
    sk = np.full(batch, seqlen, np.int64)
    return make_paged(seed, sk, heads_q, heads_kv, d, d, page_size, sq=1, varlen_q=True, v_mean=v_mean,
                      descales=(1.0, 1.0, 1.0),
                      name=f"long_kv_decode_b{batch}_h{heads_q}x{heads_kv}_d{d}_p{page_size}_k{seqlen}")


def mixed_varlen(seed: int = 4, d: int = 256, dv: int = 256, nseq: int = 8, lo: int = 256, hi: int = 4096,
                 heads_q: int = 16, heads_kv: int = 8, window: int = 1024, allow_empty_rows: bool = False) -> AttnInputs:
    """Varlen causal sliding-window prefill: 8 sequences, Sq in [256, 4096], Sk in [Sq, 4096]
    (Sk < Sq too when allow_empty_rows), 16/8 heads, window of `window` keys including the
    query's own position (window_left = window - 1), fp16 out."""
    g = torch.Generator().manual_seed(seed)
    sq = random_lengths(g, nseq, lo, hi)
    if allow_empty_rows:
        sk = random_lengths(g, nseq, lo, hi)
    else:
        sk = np.array([int(random_lengths(g, 1, int(s), hi)[0]) for s in sq], np.int64)
    inp = make_varlen(seed + 1000, sq, sk, heads_q, heads_kv, d, dv, causal=True, window_left=window - 1,
                      window_right=0, descales=(1.0, 1.0, 1.0), out_dtype="fp16",
                      name=f"mixed_varlen_n{nseq}_h{heads_q}x{heads_kv}_d{d}x{dv}_w{window}")
    return inp

"""Pins of the oracle's MXFP8 inputs (E4M3 elements with one E8M0 scale per 32 elements along
each product's contraction dimension: d for Q and K, the keys for V; FlashAttention-4 MXFP8
page, sections 1 and 2.1; E8M0 per the OCP Microscaling Formats specification): the unit scale
reduces to the pinned E4M3 oracle, power-of-two scalings act exactly as the format says, an
independent dequantization (E8M0 built from float32 bit fields, blocks by reshape) followed by
materialized fp64 attention agrees, and the NaN scale code propagates."""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from fa8_fwd_amd import inputs as gen


def mx_input(seed=3, B=2, Sq=40, Sk=70, Hq=4, Hkv=2, d=64, dv=64, causal=True, wl=-1):
    base = gen.make_dense(seed, B, Sq, Sk, Hq, Hkv, d, dv, causal=causal, window_left=wl)
    return base, gen.with_mx(base, seed + 100)


def unit(mx):
    return dataclasses.replace(mx, q_mx=np.full_like(mx.q_mx, 127), k_mx=np.full_like(mx.k_mx, 127),
                               v_mx=np.full_like(mx.v_mx, 127))


def e8m0_from_bits(e: np.ndarray) -> np.ndarray:
    """2^(e-127) as the float32 whose exponent field is e and whose mantissa is zero."""
    bits = (np.asarray(e, np.uint32) << np.uint32(23)).astype(np.uint32)
    return bits.view(np.float32).astype(np.float64)


def test_unit_scales_reduce_to_e4m3_oracle(oracle_lib):
    base, mx = mx_input()
    o0, l0 = oracle.attention(base)
    o1, l1 = oracle.attention(unit(mx))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("k", [-5, 1, 3])
def test_q_scale_is_softmax_scale_power_of_two(oracle_lib, k):
    # every Q block scaled by 2^k multiplies every score by 2^k: the same as softmax_scale * 2^k
    base, mx = mx_input(seed=4)
    u = unit(mx)
    sh = dataclasses.replace(u, q_mx=np.full_like(mx.q_mx, 127 + k))
    o1, l1 = oracle.attention(sh)
    o0, l0 = oracle.attention(base, softmax_scale=2.0 ** k / math.sqrt(base.d))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_v_scale_scales_output_exactly(oracle_lib):
    base, mx = mx_input(seed=5)
    o0, l0 = oracle.attention(base)
    o1, l1 = oracle.attention(dataclasses.replace(unit(mx), v_mx=np.full_like(mx.v_mx, 127 + 4)))
    assert np.array_equal(o1, o0 * 16.0) and np.array_equal(l0, l1)


def test_block_scale_moves_between_q_and_k(oracle_lib):
    # block c of every Q row times 2^3 and block c of every K row times 2^-3 leave every
    # product, hence the whole output, unchanged (power-of-two factors are exact in fp64)
    _, mx = mx_input(seed=6, d=128, dv=64)
    qs, ks = mx.q_mx.copy(), mx.k_mx.copy()
    qs[..., 2] += 3
    ks[..., 2] -= 3
    o0, l0 = oracle.attention(mx)
    o1, l1 = oracle.attention(dataclasses.replace(mx, q_mx=qs, k_mx=ks))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("Sq,Sk,d,dv,causal,wl", [(9, 45, 64, 64, False, -1), (33, 70, 128, 64, True, -1),
                                                   (20, 97, 64, 128, True, 40)])
def test_independent_dequantization_and_materialized_attention(oracle_lib, Sq, Sk, d, dv, causal, wl):
    base, mx = mx_input(seed=7, B=2, Sq=Sq, Sk=Sk, Hq=4, Hkv=2, d=d, dv=dv, causal=causal, wl=wl)
    t = oracle.e4m3_table()
    B, Hq, Hkv = mx.batch, mx.heads_q, mx.heads_kv
    q = t[mx.q].reshape(B, Sq, Hq, d // 32, 32) * e8m0_from_bits(mx.q_mx)[..., None]
    k = t[mx.k].reshape(B, Sk, Hkv, d // 32, 32) * e8m0_from_bits(mx.k_mx)[..., None]
    nblk = (Sk + 31) // 32
    vpad = np.zeros((B, nblk * 32, Hkv, dv))
    vpad[:, :Sk] = t[mx.v]
    v = (vpad.reshape(B, nblk, 32, Hkv, dv) * e8m0_from_bits(mx.v_mx)[:, :, None])[:, :, :, :, :]
    v = v.reshape(B, nblk * 32, Hkv, dv)[:, :Sk]
    q, k = q.reshape(B, Sq, Hq, d), k.reshape(B, Sk, Hkv, d)
    g = Hq // Hkv
    o_ref, l_ref = oracle.attention(mx)
    o_ref = o_ref.reshape(B, Sq, Hq, dv)
    l_ref = l_ref.reshape(B, Sq, Hq)
    i = np.arange(Sq)[:, None] + (Sk - Sq)
    j = np.arange(Sk)[None, :]
    vis = np.ones((Sq, Sk), bool)
    if causal:
        vis &= j <= i
    if wl >= 0:
        vis &= j >= i - wl
    for b in range(B):
        for h in range(Hq):
            s = (q[b, :, h] @ k[b, :, h // g].T) / math.sqrt(d)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            o = (w @ v[b, :, h // g]) / w.sum(axis=1, keepdims=True)
            np.testing.assert_allclose(o_ref[b, :, h], o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(l_ref[b, :, h], m[:, 0] + np.log(w.sum(axis=1)), rtol=1e-12, atol=1e-12)


def test_nan_scale_code_propagates(oracle_lib):
    _, mx = mx_input(seed=8, causal=False)
    vs = mx.v_mx.copy()
    vs[0, 1, 0, 5] = 255                   # keys 32..63 of batch 0, kv head 0, column 5
    o, _ = oracle.attention(dataclasses.replace(mx, v_mx=vs))
    o = o.reshape(mx.batch, mx.max_seqlen_q, mx.heads_q, mx.dv)
    g = mx.heads_q // mx.heads_kv
    assert np.isnan(o[0, :, :g, 5]).all()             # every row of that kv head's q heads
    assert np.isfinite(np.delete(o[0, :, :g], 5, axis=-1)).all()
    assert np.isfinite(o[1]).all() and np.isfinite(o[0, :, g:]).all()


# ----------------------------------------------------------------------------------------
# The MXFP8 method emulator (diagnostic) and the MX input encoding
# ----------------------------------------------------------------------------------------

def test_mx_encoding_keeps_block_max_in_range():
    # make_mx's blocks: largest magnitude of every block in [224, 448] after scaling and rounding, and
    # codes times scales reproduce the float32 draws to E4M3 precision
    from oracle import emulator_mx
    inp = gen.make_mx(30, 1, 70, 90, 2, 1, 64, 64)
    t = oracle.e4m3_table()
    qb = np.abs(t[inp.q]).reshape(1, 70, 2, 2, 32).max(axis=-1)
    assert (qb >= 224).all() and (qb <= 448).all()          # E4M3 rounding may land on 224
    vb = np.abs(t[np.concatenate([inp.v, np.zeros((1, 6, 1, 64), np.uint8)], axis=1)]).reshape(1, 3, 32, 1, 64).max(axis=2)
    assert (vb >= 224).all() and (vb <= 448).all()
    q, k, v = emulator_mx.dequantize(inp)
    assert 0.5 < np.std(q) < 1.5 and 0.5 < np.std(v) < 1.5


def test_emulator_mx_ceil_rule_never_clips_floor_rule_clips(oracle_lib):
    # the shared exponent ceil(log2(amax / 448)) keeps every P of a block at or below 448; OCP's
    # floor(log2 amax) - 8 lets the block's largest P reach [256, 512) and clips some at 448
    from oracle import emulator_mx
    inp = gen.make_mx(31, 1, 64, 256, 2, 1, 64, 64, causal=True)
    s1, s2 = {}, {}
    emulator_mx.emulate_mx(inp, rule="ceil", stats=s1)
    emulator_mx.emulate_mx(inp, rule="floor", stats=s2)
    assert s1["clipped"] == 0 and s2["clipped"] > 0


@pytest.mark.parametrize("causal", [False, True])
def test_emulator_mx_tracks_oracle(oracle_lib, causal):
    # on N(0,1) data encoded as MXFP8, the method's own error stays inside the stated tolerance,
    # and the clipping rule is worse than the ceil rule on the same input
    from oracle import emulator_mx
    inp = gen.make_mx(32, 2, 100, 300, 4, 2, 128, 128, causal=causal)
    ro, rl = oracle.attention_full(inp)
    eo, el = emulator_mx.emulate_mx(inp, rule="ceil")
    fo, _ = emulator_mx.emulate_mx(inp, rule="floor")
    assert np.all(np.abs(eo - ro) <= 2e-2 + 2e-2 * np.abs(ro))
    fin = np.isfinite(rl)
    assert np.max(np.abs(el[fin] - rl[fin])) <= -math.log(1 - 2.0 ** -4)
    assert np.sqrt(np.mean((fo - ro) ** 2)) > np.sqrt(np.mean((eo - ro) ** 2))

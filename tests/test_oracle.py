"""Pins of the CPU oracle (and of the method emulator) to things other than themselves:
library routines (torch's E4M3 cast, torch's scaled_dot_product_attention in float64),
arbitrary-precision brute force (mpmath), closed forms and invariants of attention, and the
values the pages print (E4M3 range, the lazy-rescale bound, the long-KV error scale)."""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import emulator, quant
from fa8_fwd_amd import inputs as gen

E4M3 = torch.float8_e4m3fn


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(E4M3).to(torch.float64).numpy()


# ----------------------------------------------------------------------------------------
# E4M3FN decode and encode
# ----------------------------------------------------------------------------------------

def test_e4m3_table_matches_torch_all_codes(oracle_lib):
    t = oracle.e4m3_table()
    ref = torch_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])


def test_e4m3_printed_facts(oracle_lib):
    # FA3 guide, "The Low-Precision Dilemma": range [-448, 448]; 3 mantissa bits
    t = oracle.e4m3_table()
    fin = t[np.isfinite(t)]
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert t[0x38] == 1.0 and t[0x39] == 1.125          # spacing 2^-3 at 1.0
    assert t[0x01] == 2.0 ** -9                          # smallest subnormal


def _midpoints():
    t = oracle.e4m3_table()
    pos = np.sort(t[(t >= 0) & np.isfinite(t)])
    mids = (pos[:-1] + pos[1:]) / 2
    xs = [pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
          np.nextafter(mids.astype(np.float32), np.float32(1e9))]
    x = np.concatenate([np.asarray(a, np.float32) for a in xs])
    return np.concatenate([x, -x])


def test_emulator_encoder_matches_torch_on_boundaries():
    x = _midpoints()
    ours = emulator.e4m3_encode_rne(x, saturate=False)
    ref = torch.from_numpy(x).to(E4M3).view(torch.uint8).numpy()
    # -0.0 encodes as 0x80 in both
    assert np.array_equal(ours, ref)


def test_emulator_direct_rounding_matches_encoder():
    # the emulator rounds P with e4m3_round; it must give exactly the value of the pinned encoder
    # (saturating) on every E4M3 boundary, its neighbours, subnormals, values past 448 and random
    # non-negative floats
    tab = oracle.e4m3_table()
    vals = np.unique(np.abs(tab[np.isfinite(tab)]))
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)), [464.0, 470.0, 1e6, 0.0],
                        np.random.default_rng(3).random(200000).astype(np.float32) * 500,
                        np.exp2(np.random.default_rng(4).uniform(-14, 9, 200000)).astype(np.float32)]).astype(np.float32)
    assert np.array_equal(emulator.e4m3_round(x), tab[emulator.e4m3_encode_rne(x, saturate=True)])


def test_emulator_encoder_matches_torch_random():
    g = torch.Generator().manual_seed(123)
    x = (torch.randn(1_000_000, generator=g) * torch.exp2(torch.randint(-12, 9, (1_000_000,), generator=g).float()))
    x = x.clamp(-448, 448).numpy().astype(np.float32)
    ours = emulator.e4m3_encode_rne(x, saturate=False)
    ref = torch.from_numpy(x).to(E4M3).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------------------
# Attention: library routine and brute force
# ----------------------------------------------------------------------------------------

def _dense_torch(inp):
    """Dequantized dense tensors via torch's own E4M3 decode, [B, H, S, d] float64."""
    q = torch_decode(inp.q).transpose(0, 2, 1, 3)
    k = torch_decode(inp.k).transpose(0, 2, 1, 3)
    v = torch_decode(inp.v).transpose(0, 2, 1, 3)
    return torch.from_numpy(q.copy()), torch.from_numpy(k.copy()), torch.from_numpy(v.copy())


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,d,dv", [(2, 17, 33, 4, 2, 64, 64), (1, 40, 40, 2, 2, 96, 96),
                                                (2, 9, 70, 6, 3, 192, 128), (1, 31, 31, 2, 1, 256, 256)])
def test_oracle_vs_torch_sdpa_noncausal(oracle_lib, B, Sq, Sk, Hq, Hkv, d, dv):
    inp = gen.make_dense(7, B, Sq, Sk, Hq, Hkv, d, dv, descales=(1.0, 1.0, 1.0))
    o, lse = oracle.attention_full(inp)
    q, k, v = _dense_torch(inp)
    g = Hq // Hkv
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1.0 / math.sqrt(d))
    ref = ref.transpose(1, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # LSE against torch.logsumexp of the scaled scores
    s = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_oracle_vs_torch_sdpa_causal_square(oracle_lib):
    # with Sq == Sk, bottom-right and top-left alignment coincide: torch's is_causal applies
    inp = gen.make_dense(8, 2, 50, 50, 4, 4, 128, 128, causal=True)
    o, _ = oracle.attention_full(inp)
    q, k, v = _dense_torch(inp)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=1 / math.sqrt(128))
    np.testing.assert_allclose(o, ref.transpose(1, 2).numpy(), rtol=1e-12, atol=1e-12)


def _mp_attention(qf, kf, vf, vis, scale, digits=50):
    """Materialized-score attention in mpmath at `digits` significant digits."""
    mpmath.mp.dps = digits
    Sq, Sk = vis.shape
    out = np.zeros((Sq, vf.shape[1]))
    lse = np.full(Sq, -np.inf)
    for i in range(Sq):
        js = [j for j in range(Sk) if vis[i, j]]
        if not js:
            continue
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b)) for a, b in zip(qf[i], kf[j])) for j in js]
        m = max(s)
        w = [mpmath.e ** (x - m) for x in s]
        l = mpmath.fsum(w)
        for c in range(vf.shape[1]):
            out[i, c] = float(mpmath.fsum(wi * mpmath.mpf(float(vf[j, c])) for wi, j in zip(w, js)) / l)
        lse[i] = float(m + mpmath.log(l))
    return out, lse


@pytest.mark.parametrize("causal,wl,wr,Sq,Sk", [(False, -1, -1, 5, 7), (True, -1, -1, 5, 7), (True, -1, -1, 7, 4),
                                                 (False, 2, 1, 6, 6), (True, 1, -1, 3, 8), (False, -1, 0, 4, 6)])
def test_oracle_vs_mpmath_bruteforce(oracle_lib, causal, wl, wr, Sq, Sk):
    inp = gen.make_dense(11, 1, Sq, Sk, 2, 1, 8, 8, causal=causal, window_left=wl, window_right=wr,
                         descales=(0.5, 2.0, 1.5))
    o, lse = oracle.attention_full(inp)
    qf, kf, vf = torch_decode(inp.q)[0], torch_decode(inp.k)[0, :, 0], torch_decode(inp.v)[0, :, 0]
    scale = (1 / math.sqrt(8)) * 0.5 * 2.0
    # visibility written from the bottom-right alignment reading: the newest query sees every key
    for h in range(2):
        vis = np.zeros((Sq, Sk), bool)
        for i in range(Sq):
            ip = i + Sk - Sq
            for j in range(Sk):
                ok = True
                if causal and j > ip:
                    ok = False
                if (not causal) and wr >= 0 and j > ip + wr:
                    ok = False
                if wl >= 0 and j < ip - wl:
                    ok = False
                vis[i, j] = ok
        ref, rl = _mp_attention(qf[:, h], kf, vf, vis, scale)
        ref = ref * 1.5
        np.testing.assert_allclose(o[0, :, h], ref, rtol=1e-13, atol=1e-14)
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lse[0, h]), fin)
        np.testing.assert_allclose(lse[0, h][fin], rl[fin], rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------------------

def test_single_key_closed_form(oracle_lib):
    inp = gen.make_dense(3, 2, 4, 1, 2, 2, 64, 64, descales=(1.0, 1.0, 2.0))
    o, lse = oracle.attention_full(inp)
    v = torch_decode(inp.v)
    for b in range(2):
        for h in range(2):
            for i in range(4):
                assert np.array_equal(o[b, i, h], 2.0 * v[b, 0, h])
    q, k = torch_decode(inp.q), torch_decode(inp.k)
    s = np.einsum("bihc,bjhc->bhij", q, k)[..., 0] / 8.0
    np.testing.assert_allclose(lse, s, rtol=1e-15, atol=0)


def test_causal_window_zero_selects_diagonal(oracle_lib):
    inp = gen.make_dense(4, 1, 6, 10, 1, 1, 64, 64, causal=True, window_left=0)
    o, _ = oracle.attention_full(inp)
    v = torch_decode(inp.v)
    for i in range(6):
        assert np.array_equal(o[0, i, 0], v[0, i + 4, 0])


def test_uniform_scores_give_mean(oracle_lib):
    inp = gen.make_dense(5, 1, 3, 37, 1, 1, 64, 64)
    inp.q[:] = 0  # all scores zero
    o, lse = oracle.attention_full(inp)
    v = torch_decode(inp.v)[0, :, 0]
    for i in range(3):
        np.testing.assert_allclose(o[0, i, 0], v.mean(axis=0), rtol=1e-14, atol=1e-15)
        assert abs(lse[0, 0, i] - math.log(37)) < 1e-15


def test_two_keys_closed_form(oracle_lib):
    inp = gen.make_dense(6, 1, 5, 2, 1, 1, 64, 64)
    o, _ = oracle.attention_full(inp)
    q, k, v = torch_decode(inp.q)[0, :, 0], torch_decode(inp.k)[0, :, 0], torch_decode(inp.v)[0, :, 0]
    for i in range(5):
        delta = (q[i] @ k[1] - q[i] @ k[0]) / 8.0
        ref = (v[0] + math.exp(delta) * v[1]) / (1 + math.exp(delta))
        np.testing.assert_allclose(o[0, i, 0], ref, rtol=1e-13, atol=1e-15)


def test_constant_v_exact(oracle_lib):
    inp = gen.make_dense(9, 2, 8, 300, 4, 2, 128, 128, causal=True, descales=(1.0, 1.0, 0.75))
    inp.v[:] = 0x3C  # 1.5
    o, _ = oracle.attention_full(inp)
    # exact up to the rounding of two 300-term fp64 sums (n * eps ~ 3e-14)
    np.testing.assert_allclose(o, 1.5 * 0.75, rtol=4e-14, atol=0)


def test_rows_are_stochastic(oracle_lib):
    # V rows = unit vectors e_j  ->  O[i, :Sk] is the probability row P[i, :]
    Sk = 48
    inp = gen.make_dense(10, 1, 20, Sk, 1, 1, 64, 64, causal=True)
    inp.v[:] = 0
    for j in range(Sk):
        inp.v[0, j, 0, j] = 0x38
    o, _ = oracle.attention_full(inp)
    P = o[0, :, 0, :Sk]
    assert (P >= 0).all()
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # causal bottom-right: row i has exactly i + Sk - Sq + 1 nonzero entries
    for i in range(20):
        assert np.count_nonzero(P[i]) == i + Sk - 20 + 1


def test_empty_rows(oracle_lib):
    # Sq > Sk causal: the first Sq - Sk rows see no key
    inp = gen.make_dense(12, 1, 10, 4, 2, 2, 64, 64, causal=True)
    o, lse = oracle.attention_full(inp)
    assert np.all(o[0, :6] == 0) and np.all(np.isneginf(lse[0, :, :6]))
    assert np.all(np.isfinite(lse[0, :, 6:]))


# ----------------------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------------------

def test_gqa_equals_repeated_mha(oracle_lib):
    inp = gen.make_dense(13, 2, 12, 40, 8, 2, 64, 64, causal=True, descales=(("uniform", 0.5, 2.0),) * 3)
    o, lse = oracle.attention_full(inp)
    rep = gen.make_dense(13, 2, 12, 40, 8, 2, 64, 64)
    rep.heads_kv = 8
    rep.k = np.repeat(inp.k, 4, axis=2)
    rep.v = np.repeat(inp.v, 4, axis=2)
    rep.q, rep.causal = inp.q, True
    rep.q_descale, rep.k_descale, rep.v_descale = (np.repeat(x, 4, axis=1) for x in (inp.q_descale, inp.k_descale, inp.v_descale))
    o2, lse2 = oracle.attention_full(rep)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_paged_equals_contiguous(oracle_lib):
    inp = gen.make_paged(14, [37, 5, 64, 100], 4, 2, 64, 64, page_size=16, sq=3, varlen_q=False, causal=True)
    o, lse = oracle.attention_full(inp)
    # gather the same tokens into a contiguous varlen layout
    sk = inp.seqused_k.astype(np.int64)
    ks, vs = [], []
    for b in range(inp.batch):
        j = np.arange(sk[b])
        pg = inp.block_table[b, j // 16]
        ks.append(inp.k[pg, j % 16])
        vs.append(inp.v[pg, j % 16])
    cont = gen.make_dense(14, 4, 3, 1, 4, 2, 64, 64, causal=True)
    cont.q = inp.q
    cont.k, cont.v = np.concatenate(ks), np.concatenate(vs)
    cont.cu_seqlens_k = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    cont.max_seqlen_k = int(sk.max())
    o2, lse2 = oracle.attention_full(cont)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_key_permutation_invariance(oracle_lib):
    inp = gen.make_dense(15, 1, 6, 90, 2, 2, 128, 128)
    o, _ = oracle.attention_full(inp)
    perm = np.random.default_rng(0).permutation(90)
    inp.k, inp.v = inp.k[:, perm], inp.v[:, perm]
    o2, _ = oracle.attention_full(inp)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)


def test_descale_roles(oracle_lib):
    inp = gen.make_dense(16, 1, 8, 64, 2, 1, 64, 64, descales=(1.0, 1.0, 1.0))
    o1, l1 = oracle.attention_full(inp)
    inp.v_descale = np.array(4.0, np.float32)
    o2, l2 = oracle.attention_full(inp)
    assert np.array_equal(o2, 4.0 * o1) and np.array_equal(l1, l2)
    # (scale, dq, dk) enter only through their product
    inp.v_descale = None
    inp.q_descale, inp.k_descale = np.array(2.0, np.float32), np.array(0.25, np.float32)
    o3, l3 = oracle.attention_full(inp, )
    inp.q_descale = inp.k_descale = None
    inp.softmax_scale = 0.5 / math.sqrt(64)
    o4, l4 = oracle.attention_full(inp)
    np.testing.assert_allclose(o3, o4, rtol=1e-15, atol=1e-16)


def test_split_combine_equals_unsplit(oracle_lib):
    inp = gen.make_paged(17, [300, 1000, 33], 8, 2, 128, 128, page_size=16, sq=2, varlen_q=True,
                         descales=(("uniform", 0.5, 2.0),) * 3)
    rows = oracle.all_rows(inp)
    o, lse = oracle.attention(inp, rows=rows)
    sk = inp.seqused_k.astype(np.int64)[rows[0]]
    S = 5
    parts_o, parts_l = [], []
    for s in range(S):
        lo, hi = (sk * s) // S, (sk * (s + 1)) // S
        po, pl = oracle.attention(inp, rows=rows, key_range=(lo, hi))
        parts_o.append(po)
        parts_l.append(pl)
    # one deliberately empty split
    eo, el = oracle.attention(inp, rows=rows, key_range=(np.zeros_like(sk), np.zeros_like(sk)))
    assert np.all(eo == 0) and np.all(np.isneginf(el))
    parts_o.append(eo)
    parts_l.append(el)
    co, cl = oracle.combine(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(co, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cl, lse, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("sk", [1024, 8192, 32768, 131072])
def test_no_shrinkage_with_kv_length(oracle_lib, sk):
    # V ~ N(0.5, 1), 8 query heads on one kv head, Sk from 1k to 128k keys (the Hopper FP8 page's
    # long-KV accuracy lengths). (1) The oracle agrees with an independent evaluation of the same
    # definition that sums in 80-bit extended precision (the normalizer by math.fsum, i.e. exactly
    # rounded) to 1e-12 relative. (2) Each row's output mean over its 128 columns stays within
    # 4 sigma of the dequantized V mean, sigma = std(V) / sqrt(128 n_eff) with n_eff =
    # (sum w)^2 / sum w^2 the row's effective key count: no shrinkage with the key count.
    inp = gen.make_paged(18, [sk], 8, 1, 128, 128, page_size=64, sq=1, v_mean=0.5)
    o, lse = oracle.attention(inp)
    tab = oracle.e4m3_table()
    pages = inp.block_table[0, : (sk + 63) // 64]
    k = tab[inp.k[pages]].reshape(-1, 128)[:sk]
    v = tab[inp.v[pages]].reshape(-1, 128)[:sk]
    q = tab[inp.q[0]]                                   # [8 heads, 128]
    s = (q @ k.T) / math.sqrt(128)                      # exact dots (integers x 2^-18), one rounding by the scale
    vmean, vstd = float(v.mean()), float(v.std())
    for h in range(8):
        w = np.exp(s[h] - s[h].max())
        l = math.fsum(w.tolist())
        ref = (w.astype(np.longdouble) @ v.astype(np.longdouble)) / np.longdouble(l)
        assert np.max(np.abs(o[h] - ref.astype(np.float64))) <= 1e-12 * max(1.0, float(np.abs(ref).max()))
        assert abs(lse[h] - (s[h].max() + math.log(l))) <= 1e-12 * abs(lse[h]) + 1e-12
        n_eff = l * l / float(np.sum(w * w))
        assert abs(float(o[h].mean()) - vmean) <= 4 * vstd / math.sqrt(128 * n_eff), (h, n_eff)


# ----------------------------------------------------------------------------------------
# The method emulator: the pages' lazy-rescale bound, the bias, and the printed error scale
# ----------------------------------------------------------------------------------------

def test_tau_bound_closed_form():
    # sheared-forward fp8 page, "Correctness fix": threshold <= log2(448) - 8 = 0.807; 0.75 used
    bound = math.log2(448.0) - 8.0
    assert abs(bound - 0.807) < 5e-4
    assert 0.75 <= bound
    assert 2.0 ** (8 + 0.75) < 448.0 <= 2.0 ** (8 + bound) + 1e-9


def _staircase(step_codes, tile_n=16):
    """One query (1.0 in dim 0) against tiles whose keys all score `step` more than the tile before:
    with softmax_scale = ln 2 the scaled log2 score equals the raw dot product."""
    ntiles = len(step_codes)
    inp = gen.make_dense(19, 1, 1, ntiles * tile_n, 1, 1, 16, 16, softmax_scale=math.log(2.0))
    inp.q[:] = 0
    inp.q[0, 0, 0, 0] = 0x38
    inp.k[:] = 0
    for t, c in enumerate(step_codes):
        inp.k[0, t * tile_n:(t + 1) * tile_n, 0, 0] = c
    return inp


def test_lazy_rescale_tau_075_never_clips_tau_4_clips(oracle_lib):
    t = oracle.e4m3_table()
    codes = [int(np.nonzero(t == float(x))[0][0]) for x in (0, 1, 2, 3, 4, 5)]   # scores 0,1,..,5
    inp = _staircase(codes)
    ref, _ = oracle.attention(inp)
    st = {}
    good = emulator.emulate(inp, tile_n=16, tau=0.75, stats=st)[(0, 0)][0]
    assert st["clipped"] == 0 and st["pmax"] <= 2.0 ** 8.75
    np.testing.assert_allclose(good[0], ref[0], rtol=2e-2, atol=2e-2)
    st4 = {}
    bad = emulator.emulate(inp, tile_n=16, tau=4.0, stats=st4)[(0, 0)][0]
    assert st4["clipped"] > 0                       # the failure mode the bound prevents
    # half-step staircase: slack accumulates to 0.5 < tau, then moves; still no clip at 0.75
    half = [int(np.nonzero(t == float(x))[0][0]) for x in (0, 0.5, 1, 1.5, 2, 2.5, 3)]
    st5 = {}
    emulator.emulate(_staircase(half), tile_n=16, tau=0.75, stats=st5)
    assert st5["clipped"] == 0 and st5["pmax"] > 2.0 ** 8.0


def test_bias_keeps_small_probabilities(oracle_lib):
    # one key at log2-score 0 and 1024 keys at -10: without the 2^8 bias their p = 2^-10 rounds to 0
    t = oracle.e4m3_table()
    inp = gen.make_dense(20, 1, 1, 1025, 1, 1, 16, 16, softmax_scale=math.log(2.0))
    inp.q[:] = 0
    inp.q[0, 0, 0, 0] = 0x38
    inp.k[:] = 0
    inp.k[0, 0, 0, 0] = int(np.nonzero(t == 10.0)[0][0])
    inp.v[:] = 0x38        # the 1024 small-probability keys carry V = 1, the top key V = 0:
    inp.v[0, 0] = 0        # exact output 0.5, half of it from the keys the bias must keep
    ref, _ = oracle.attention(inp)
    assert abs(ref[0, 0] - 0.5) < 1e-12
    with8 = emulator.emulate(inp, tile_n=64, bias=8.0)[(0, 0)][0]
    with0 = emulator.emulate(inp, tile_n=64, bias=0.0)[(0, 0)][0]
    e8 = np.abs(with8 - ref).max() / np.abs(ref).max()
    e0 = np.abs(with0 - ref).max() / np.abs(ref).max()
    assert e8 < 0.02 and e0 > 0.2


@pytest.mark.parametrize("sk", [1024, 8192])
def test_emulator_error_scale_matches_printed(oracle_lib, sk):
    # "Long-KV accuracy": error relative to the fp64 reference RMS, mean-0.5 V, one split,
    # 0.17% at 1k and 0.15% at 8k for the two-level FP8 kernels. Same order here.
    inp = gen.make_paged(21, [sk], 8, 1, 128, 128, page_size=64, sq=1, v_mean=0.5)
    ref, _ = oracle.attention(inp)
    emu = np.concatenate([emulator.emulate(inp, tile_n=64, heads=[h])[(0, h)][0] for h in range(8)])
    rel = np.sqrt(np.mean((emu - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert 0.0003 < rel < 0.006, rel


def test_emulator_interleaved_states(oracle_lib):
    # Running states that take alternate key blocks and are merged by their LSEs are still the
    # method (the split-KV construction applied inside a split). Pins: with interleave 1 and
    # granule = tile the result is bitwise the plain emulation; constant V gives exactly V from
    # every state and so from the merge; the error scale against the fp64 reference stays at the
    # FP8 level of the single-state run.
    inp = gen.make_paged(22, [1000, 333, 64], 8, 2, 128, 128, page_size=16, sq=1, v_mean=0.5)
    plain = emulator.emulate(inp, tile_n=64, num_splits=3)
    same = emulator.emulate(inp, tile_n=64, num_splits=3, granule=64, interleave=1)
    for key in plain:
        assert np.array_equal(plain[key][0], same[key][0]) and np.array_equal(plain[key][1], same[key][1])
    inter = emulator.emulate(inp, tile_n=16, num_splits=3, granule=64, interleave=2, l_from_rounded=True)
    ref, _ = oracle.attention(inp)
    rb, rh, ri = oracle.all_rows(inp)
    emu = np.stack([inter[(int(b), int(h))][0][int(i)] for b, h, i in zip(rb, rh, ri)])
    rel = np.sqrt(np.mean((emu - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert 0.0003 < rel < 0.006, rel
    const = gen.make_paged(23, [1000, 333, 64], 8, 2, 128, 128, page_size=16, sq=1)
    const.v[:] = 0x38                                   # E4M3 code of 1.0
    res = emulator.emulate(const, tile_n=16, num_splits=3, granule=64, interleave=2, l_from_rounded=True)
    for (o, _) in res.values():
        assert np.abs(o - 1.0).max() < 1e-5


# ----------------------------------------------------------------------------------------
# Learnable sink: one logit z_h per query head in the softmax denominator, with no value
# ("Native FP8 (E4M3 Q/K/V) forward for Hopper", Summary, lists it among the supported
# features; the sheared fp8 page, Summary, carries the 2^8 offset through the sink term)
# ----------------------------------------------------------------------------------------

def _mp_attention_sink(qf, kf, vf, vis, scale, z, digits=50):
    """Materialized-score attention with a sink logit z, in mpmath."""
    mpmath.mp.dps = digits
    Sq, Sk = vis.shape
    out = np.zeros((Sq, vf.shape[1]))
    lse = np.zeros(Sq)
    zm = mpmath.mpf(float(z))
    for i in range(Sq):
        js = [j for j in range(Sk) if vis[i, j]]
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b)) for a, b in zip(qf[i], kf[j])) for j in js]
        den = mpmath.fsum([mpmath.e ** x for x in s] + [mpmath.e ** zm])
        for c in range(vf.shape[1]):
            out[i, c] = float(mpmath.fsum(mpmath.e ** x * mpmath.mpf(float(vf[j, c])) for x, j in zip(s, js)) / den)
        lse[i] = float(mpmath.log(den))
    return out, lse


@pytest.mark.parametrize("causal,wl,Sq,Sk", [(False, -1, 5, 7), (True, -1, 7, 4), (True, 1, 3, 8)])
def test_sink_vs_mpmath_bruteforce(oracle_lib, causal, wl, Sq, Sk):
    z = np.array([0.7, -1.3])
    inp = gen.make_dense(11, 1, Sq, Sk, 2, 1, 8, 8, causal=causal, window_left=wl, descales=(0.5, 2.0, 1.5))
    o, lse = oracle.attention(inp, sink=z)
    o = o.reshape(Sq, 2, 8)
    lse = lse.reshape(Sq, 2)
    qf, kf, vf = torch_decode(inp.q)[0], torch_decode(inp.k)[0, :, 0], torch_decode(inp.v)[0, :, 0]
    scale = (1 / math.sqrt(8)) * 0.5 * 2.0
    for h in range(2):
        vis = np.zeros((Sq, Sk), bool)
        for i in range(Sq):
            ip = i + Sk - Sq
            for j in range(Sk):
                vis[i, j] = not ((causal and j > ip) or (wl >= 0 and j < ip - wl))
        ref, rl = _mp_attention_sink(qf[:, h], kf, vf, vis, scale, z[h])
        np.testing.assert_allclose(o[:, h], 1.5 * ref, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, h], rl, rtol=1e-13, atol=1e-13)


def test_sink_single_key_closed_form(oracle_lib):
    # one key: O = dv v / (1 + e^(z - s)), LSE = ln(e^s + e^z)
    inp = gen.make_dense(3, 2, 4, 1, 2, 2, 64, 64, descales=(1.0, 1.0, 2.0))
    z = np.array([0.25, -3.0])
    o, lse = oracle.attention(inp, sink=z)
    o = o.reshape(2, 4, 2, 64)
    lse = lse.reshape(2, 4, 2)
    q, k, v = torch_decode(inp.q), torch_decode(inp.k), torch_decode(inp.v)
    s = np.einsum("bihc,bjhc->bihj", q, k)[..., 0] / 8.0           # [b, i, h]
    want = 2.0 * v[:, 0][:, None, :, :] / (1.0 + np.exp(z[None, None, :] - s))[..., None]
    np.testing.assert_allclose(o, want, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, np.logaddexp(s, z[None, None, :]), rtol=1e-15, atol=1e-15)


def test_sink_minus_infinity_is_no_sink(oracle_lib):
    inp = gen.make_dense(9, 2, 33, 70, 4, 2, 64, 64, causal=True, descales=(0.5, 0.5, 1.5))
    o0, l0 = oracle.attention(inp)
    o1, l1 = oracle.attention(inp, sink=np.full(4, -np.inf))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_sink_empty_rows(oracle_lib):
    # Sq > Sk causal: rows without keys give O = 0 and LSE = the sink logit
    inp = gen.make_dense(12, 1, 10, 4, 2, 2, 64, 64, causal=True)
    z = np.array([1.5, -0.5])
    o, lse = oracle.attention(inp, sink=z)
    o = o.reshape(10, 2, 64)
    lse = lse.reshape(10, 2)
    assert np.all(o[:6] == 0)
    assert np.array_equal(lse[:6], np.broadcast_to(z, (6, 2)))


def test_sink_relation_to_plain_attention(oracle_lib):
    # the sink only rescales: O_z = O exp(LSE - LSE_z) and LSE_z = ln(e^LSE + e^z), row by row
    inp = gen.make_paged(17, [300, 1000, 33], 8, 2, 128, 128, page_size=16, sq=2, varlen_q=True,
                         descales=(("uniform", 0.5, 2.0),) * 3)
    z = np.linspace(-2.0, 3.0, 8)
    rows = oracle.all_rows(inp)
    o, lse = oracle.attention(inp, rows=rows)
    oz, lz = oracle.attention(inp, rows=rows, sink=z)
    zr = z[rows[1]]
    np.testing.assert_allclose(lz, np.logaddexp(lse, zr), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oz, o * np.exp(lse - lz)[:, None], rtol=1e-12, atol=1e-13)


def test_sink_split_combine_equals_unsplit(oracle_lib):
    # split partials carry no sink; the combine adds it once
    inp = gen.make_paged(17, [300, 1000, 33], 8, 2, 128, 128, page_size=16, sq=2, varlen_q=True,
                         descales=(("uniform", 0.5, 2.0),) * 3)
    z = np.linspace(-2.0, 3.0, 8)
    rows = oracle.all_rows(inp)
    oz, lz = oracle.attention(inp, rows=rows, sink=z)
    sk = inp.seqused_k.astype(np.int64)[rows[0]]
    parts = [oracle.attention(inp, rows=rows, key_range=((sk * s) // 4, (sk * (s + 1)) // 4)) for s in range(4)]
    co, cl = oracle.combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]), sink=z[rows[1]])
    np.testing.assert_allclose(co, oz, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cl, lz, rtol=1e-13, atol=1e-13)


def test_emulator_with_sink_tracks_oracle(oracle_lib):
    # the method with a sink (here a quarter to a half of each row's denominator), at the end of
    # the range or in the combine, stays at the FP8 error level of the method without one; a sink
    # term off by a factor would move O by tens of percent
    base = gen.make_dense(21, 1, 64, 1500, 4, 2, 128, 128, causal=True, descales=(0.5, 0.5, 1.0))
    inp = gen.with_sink(base, 5, mean=6.5, std=0.5)

    def rel_err(x, ns, stage):
        ref, _ = oracle.attention_full(x)
        res = emulator.emulate(x, tile_n=128, num_splits=ns, sink_stage=stage, l_from_rounded=True)
        got = np.zeros_like(ref)
        for (b, h), (o, l) in res.items():
            got[b, :, h] = o
        return float(np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2)))

    e0 = rel_err(base, 1, "finalize")
    for stage, ns in (("finalize", 1), ("combine", 3)):
        e = rel_err(inp, ns, stage)
        assert e <= 1.3 * e0 + 1e-3, (stage, e, e0)


# ----------------------------------------------------------------------------------------
# Q quantizer (per (batch, kv head) block: scale = amax / 448, codes = E4M3(x / scale))
# ----------------------------------------------------------------------------------------

def _bf16_values(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).float().numpy()


def test_quantizer_block_max_maps_to_448(oracle_lib):
    q = _bf16_values((2, 40, 8, 64), 1, 3.0)
    codes, s = quant.quantize_q(q, heads_kv=2)
    dec = oracle.e4m3_table()[codes]
    for b in range(2):
        for kvh in range(2):
            blk = q[b, :, kvh * 4:(kvh + 1) * 4]
            d = dec[b, :, kvh * 4:(kvh + 1) * 4]
            assert s[b, kvh] == np.float32(np.abs(blk).max() / np.float32(448))
            # the block maximum maps to +-448; so does nothing below 432 (half the 32-wide step
            # under 448 away)
            assert np.all(np.abs(d)[np.abs(blk) == np.abs(blk).max()] == 448.0)
            y = np.abs(blk) / s[b, kvh]
            assert np.all(y[np.abs(d) == 448.0] >= 432.0)


def test_quantizer_exact_on_representable_inputs(oracle_lib):
    # x = 2^k * (E4M3 values) with one value at 448: scale = 2^k exactly, codes are the inputs'
    table = oracle.e4m3_table()
    rng = np.random.default_rng(3)
    want = rng.integers(0, 256, size=(1, 17, 4, 32)).astype(np.uint8)
    want[np.isnan(table[want])] = 0x38
    want[0, 0, 0, 0] = 0x7E                       # 448: the block maximum
    x = (table[want] * 2.0 ** -5).astype(np.float32)
    codes, s = quant.quantize_q(x, heads_kv=1)
    assert s[0, 0] == np.float32(2.0 ** -5)
    # equal values may take either sign of zero; compare decoded values
    assert np.array_equal(table[codes], table[want])


def test_quantizer_power_of_two_scaling_invariance(oracle_lib):
    # scaling a block by 2^k scales its descale by 2^k and leaves its codes unchanged
    q = _bf16_values((3, 25, 8, 128), 4)
    c1, s1 = quant.quantize_q(q, heads_kv=4)
    q2 = q.copy()
    q2[1] *= 8.0
    c2, s2 = quant.quantize_q(q2, heads_kv=4)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2[1], s1[1] * 8) and np.array_equal(s2[[0, 2]], s1[[0, 2]])


def test_quantizer_error_within_half_step(oracle_lib):
    # |dec(code) - x / s| <= half the E4M3 spacing at that magnitude (2^(e-4), subnormal 2^-10),
    # and the codes are monotone in x
    q = _bf16_values((1, 64, 2, 128), 5, 0.1)
    codes, s = quant.quantize_q(q, heads_kv=1)
    y = (q / s[0, 0]).astype(np.float64)
    d = oracle.e4m3_table()[codes]
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    assert np.all(np.abs(d - y) <= 2.0 ** (e - 4) + 1e-12)
    order = np.argsort(y.reshape(-1), kind="stable")
    assert np.all(np.diff(d.reshape(-1)[order]) >= 0)


def test_quantizer_zero_block_and_varlen(oracle_lib):
    q = _bf16_values((30, 4, 64), 6)
    cu = np.array([0, 10, 10, 30], np.int32)          # one empty sequence
    q[:10, 2:] = 0.0                                  # batch 0, kv head 1: all zeros
    codes, s = quant.quantize_q(q, heads_kv=2, cu_seqlens_q=cu)
    assert s[0, 1] == 1.0 and np.all(codes[:10, 2:] == 0)
    assert np.all(s[1] == 1.0)                         # the empty sequence
    ref, rs = quant.quantize_q(q[10:30][None], heads_kv=2)
    assert np.array_equal(codes[10:30], ref[0]) and np.array_equal(s[2], rs[0])

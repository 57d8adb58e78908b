"""The precision of the FP8 matrix cores' dot products, which every score of the kernels carries
(include/fa8.h, score precision; helpers.MFMA_DOT_REL). A probe kernel (tests/probes/mfma_dot.hip)
computes S = K Q^T for d = 128 exactly as the attention kernels issue it (two 64-element k-steps
of the block-scaled 32x32x64 FP8 MFMA, chained through the accumulator), and each 32-element
block alone summed in fp32; both are compared with the exact fp64 dot products on the CPU.
Inputs: plain E4M3 N(0,1) data (unit scales), N(0,1) data encoded as MXFP8, and E4M3 elements with
independent random block scales 2^-5 .. 2^5."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from fa8_fwd_amd import inputs as gen

from helpers import MFMA_DOT_REL

pytestmark = pytest.mark.gpu

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libmfma_dot.so")


def _probe(K, ks, Q, qs):
    lib = ctypes.CDLL(_LIB)          # built by __graft_entry__.build(); a missing file fails the test
    nk, nq = -(-K.shape[0] // 32) * 32, -(-Q.shape[0] // 32) * 32

    def pad(x, n, fill):
        y = np.full((n,) + x.shape[1:], fill, x.dtype)
        y[:x.shape[0]] = x
        return np.ascontiguousarray(y)

    K, ks, Q, qs = pad(K, nk, 0), pad(ks, nk, 127), pad(Q, nq, 0), pad(qs, nq, 127)
    assert K.shape == (nk, 128) and ks.shape == (nk, 4) and Q.shape == (nq, 128) and qs.shape == (nq, 4)
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(x).to(dev) for x in (K, ks, Q, qs)]
    out = torch.empty((2, nk, nq), dtype=torch.float32, device=dev)
    rc = lib.mfma_dot_probe_run(*(ctypes.c_void_p(x.data_ptr()) for x in t), nk, nq, ctypes.c_void_p(out.data_ptr()))
    assert rc == 0, rc
    tab = oracle.e4m3_table()
    e8 = lambda e: np.ldexp(1.0, e.astype(np.int64) - 127)
    kd = tab[K].reshape(nk, 4, 32) * e8(ks)[:, :, None]
    qd = tab[Q].reshape(nq, 4, 32) * e8(qs)[:, :, None]
    exact = np.einsum("kbe,qbe->kq", kd, qd)
    absum = np.einsum("kbe,qbe->kq", np.abs(kd), np.abs(qd))
    return out.cpu().numpy().astype(np.float64), exact, absum


@pytest.mark.parametrize("case", ["unit scales", "mxfp8 encoded", "random block scales"])
def test_fp8_mfma_dot_error_relative_to_absolute_products(case):
    if case == "unit scales":
        inp = gen.make_dense(146, 1, 203, 331, 4, 2, 128, 128)
        K, Q = inp.k[0, :, 0], inp.q[0, :, 1]
        ks, qs = np.full((K.shape[0], 4), 127, np.uint8), np.full((Q.shape[0], 4), 127, np.uint8)
    elif case == "mxfp8 encoded":
        inp = gen.make_mx(2, 1, 256, 256, 4, 2, 128, 128)
        K, ks, Q, qs = inp.k[0, :, 0], inp.k_mx[0, :, 0], inp.q[0, :, 0], inp.q_mx[0, :, 0]
    else:
        inp = gen.with_mx(gen.make_dense(146, 2, 203, 331, 4, 2, 128, 128, causal=True), 147)
        K, ks, Q, qs = inp.k[1, :, 0], inp.k_mx[1, :, 0], inp.q[1, :, 1], inp.q_mx[1, :, 1]
    got, exact, absum = _probe(K, ks, Q, qs)
    ok = absum > 0
    for name, g in (("chained k-steps", got[0]), ("32-element blocks alone", got[1])):
        rel = np.abs(g - exact)[ok] / absum[ok]
        print(f"{case}, {name}: max |err| / sum|products| = {rel.max():.3g} (2^{np.log2(rel.max() + 1e-300):.1f}); "
              f"exact in {np.mean(g[ok] == exact[ok]):.1%} of the dot products", flush=True)
        assert rel.max() <= MFMA_DOT_REL


# ---------------------------------------------------------------------------------------------
# The accumulator input of the FP8 matrix cores (tests/probes/mfma_acc.hip), which the prefill
# kernels rely on when they accumulate PV onto O directly instead of folding a per-tile product
# into O in fp32: chaining products through the accumulator must be as accurate as the fp32
# fold, with no drift over long key ranges.
# ---------------------------------------------------------------------------------------------
_ACC_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libmfma_acc.so")


def _acc_probe(A, B, C0, mode):
    lib = ctypes.CDLL(_ACC_LIB)
    steps, nblk = A.shape[:2]
    assert A.shape == (steps, nblk, 64, 32) and B.shape == A.shape and C0.shape == (nblk, 64, 16)
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (A, B, C0.astype(np.float32))]
    D = torch.empty((nblk, 64, 16), dtype=torch.float32, device=dev)
    rc = lib.mfma_acc_probe_run(*(ctypes.c_void_p(x.data_ptr()) for x in t), steps, nblk, mode,
                                ctypes.c_void_p(D.data_ptr()))
    assert rc == 0, rc
    return D.cpu().numpy().astype(np.float64)


def _acc_exact(A, B, C0):
    """C0 + sum over steps of the 32x32 products, in the accumulator's order (lane L, register r:
    row 8(r/4) + 4(L/32) + r%4, column L%32), and the same sum of |products|. Row i of A is lanes
    i and i+32 (byte y of lane i+32h pairs with byte y of B's lane j+32h)."""
    tab = oracle.e4m3_table()
    steps, nblk = A.shape[:2]
    Af = tab[A].reshape(steps, nblk, 2, 32, 32)
    Bf = tab[B].reshape(steps, nblk, 2, 32, 32)
    M = np.einsum("sbhiy,sbhjy->bij", Af, Bf)
    Mabs = np.einsum("sbhiy,sbhjy->bij", np.abs(Af), np.abs(Bf))
    L = np.arange(64)[:, None]
    r = np.arange(16)[None, :]
    i = 8 * (r // 4) + 4 * (L // 32) + r % 4
    j = np.broadcast_to(L % 32, i.shape)
    return C0 + M[:, i, j], Mabs[:, i, j]


def _e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_mfma_accumulator_input_at_fp32_precision():
    rng = np.random.default_rng(41)
    # one product onto accumulators of 2^12: the error stays a few fp32 ulps of C plus the
    # dot product's own error (no alignment of the products to the accumulator's exponent)
    A, B = _e4m3(rng.standard_normal((1, 32, 64, 32))), _e4m3(rng.standard_normal((1, 32, 64, 32)))
    C0 = (rng.standard_normal((32, 64, 16)) * 4096.0).astype(np.float32).astype(np.float64)
    exact, absum = _acc_exact(A, B, C0)
    got = _acc_probe(A, B, C0, 0)
    ulp = np.spacing(np.abs(C0).astype(np.float32)).astype(np.float64)
    err = np.abs(got - exact)
    assert (err <= 4 * ulp + MFMA_DOT_REL * absum).all(), float((err / (4 * ulp + MFMA_DOT_REL * absum)).max())
    # 2048 chained products (131072 keys) of attention-like P = E4M3(2^(x - m + 8)) and V of
    # mean 0.5: chained through the accumulator vs each product added in fp32
    steps, nblk = 2048, 4
    x = rng.standard_normal((steps, nblk, 64, 32))
    P = _e4m3(np.exp2(np.minimum(x - x.max() + 8, 8.7)))
    V = _e4m3(rng.standard_normal((steps, nblk, 64, 32)) + 0.5)
    C0 = np.zeros((nblk, 64, 16))
    exact, absum = _acc_exact(V, P, C0)
    chained, folded = _acc_probe(V, P, C0, 0), _acc_probe(V, P, C0, 1)
    for name, g in (("chained", chained), ("fp32 fold", folded)):
        rel = (g - exact) / absum
        big = np.abs(exact) > 0.1 * absum
        ratio = float(np.mean(g[big] / exact[big]))
        print(f"131072 keys, {name}: max |err| / sum|pv| = {np.abs(rel).max():.3g}, mean {rel.mean():.3g}, "
              f"mean ratio to exact {ratio:.9f}", flush=True)
        assert np.abs(rel).max() <= 2.0 ** -16
        assert abs(ratio - 1.0) <= 1e-6


def test_fp8_mfma_accumulator_small_products_after_large_ones():
    # the adversarial case for one-level accumulation: 4096 keys with P = 256 first, then 126976
    # keys with P in 2^-9 .. 2^-4 (E4M3's smallest values) onto the large accumulator, V > 0 so
    # that any truncation of small products shows as a bias. The matrix cores do drop products
    # far below the accumulator's last bit (such a product is not rounded into it), but the
    # loss stays below 1e-5 of the sum, far under P's own E4M3 rounding (2^-4)
    rng = np.random.default_rng(43)
    steps, nblk = 2048, 4
    x = np.where(np.arange(steps)[:, None, None, None] < 64, 8.0, rng.uniform(-9, -4, (steps, nblk, 64, 32)))
    P = _e4m3(np.exp2(x))
    V = _e4m3(np.abs(rng.standard_normal((steps, nblk, 64, 32))) + 0.5)
    C0 = np.zeros((nblk, 64, 16))
    exact, absum = _acc_exact(V, P, C0)
    chained = _acc_probe(V, P, C0, 0)
    rel = (chained - exact) / absum
    ratio = float(np.mean(chained / exact))
    print(f"dominant then small products: max |err| / sum|pv| = {np.abs(rel).max():.3g}, mean ratio {ratio:.9f}",
          flush=True)
    assert np.abs(rel).max() <= 2.0 ** -16
    assert abs(ratio - 1.0) <= 1e-5

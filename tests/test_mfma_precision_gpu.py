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

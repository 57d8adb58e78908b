"""The C-ABI library loads, exports every entry point include/fa8.h declares, and its host-side
validation rejects bad arguments before any launch. No GPU is needed."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from fa8_fwd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa8_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_header_symbols():
    lib = binding.load()
    names = declared_functions()
    assert {"fa8_fwd_prefill", "fa8_fwd_decode_splitkv", "fa8_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fa8.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", binding.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa8_[a-z0-9_]+)", out))
    assert set(names) <= exported
    assert binding.version().startswith("fa8")


def test_header_compiles_as_c():
    src = '#include "fa8.h"\nint main(void){ fa8_fwd_params p; (void)p; return (int)FA8_OK; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-x", "c", "-",
                        "-fsyntax-only"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layout_matches_c():
    # offsetof of the last field and sizeof, computed by the C compiler from the header
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "fa8.h"\nint main(void){printf("%zu %zu %zu",'
           ' sizeof(fa8_fwd_params), offsetof(fa8_fwd_params, lse_row_stride), offsetof(fa8_fwd_params, softmax_scale));'
           'return 0;}\n')
    exe = "/tmp/fa8_layout_probe"
    r = subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-x", "c", "-", "-o", exe], input=src,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    size, off_last, off_scale = map(int, subprocess.run([exe], capture_output=True, text=True).stdout.split())
    assert ctypes.sizeof(binding.FwdParams) == size
    assert binding.FwdParams.lse_row_stride.offset == off_last
    assert binding.FwdParams.softmax_scale.offset == off_scale
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "fa8.h"\nint main(void){printf("%zu %zu",'
           ' sizeof(fa8_decode_plan_info), offsetof(fa8_decode_plan_info, workgroups));return 0;}\n')
    r = subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-x", "c", "-", "-o", exe], input=src,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    size, off_wg = map(int, subprocess.run([exe], capture_output=True, text=True).stdout.split())
    assert ctypes.sizeof(binding.DecodePlan) == size
    assert binding.DecodePlan.workgroups.offset == off_wg


def _cpu(shape, dtype=torch.uint8):
    return torch.zeros(shape, dtype=dtype)


def _base(d=128, dv=128, hq=8, hkv=2, sq=16, sk=64, b=2):
    q = _cpu((b, sq, hq, d))
    k = _cpu((b, sk, hkv, d))
    v = _cpu((b, sk, hkv, dv))
    out = _cpu((b, sq, hq, dv), torch.bfloat16)
    return q, k, v, out


def test_valid_params_ok():
    q, k, v, out = _base()
    assert binding.check_params(q, k, v, out=out) == binding.FA8_OK
    assert binding.check_params(q, k, v, num_splits=4) == binding.FA8_OK


@pytest.mark.parametrize("d,dv", [(32, 32), (128, 64), (160, 160), (512, 512), (64, 128)])
def test_unsupported_head_dims(d, dv):
    q, k, v, out = _base(d=d, dv=dv)
    assert binding.check_params(q, k, v, out=out) == binding.FA8_ERR_UNSUPPORTED
    assert "not supported" in binding.last_error()


def test_gqa_ratio_must_divide():
    q, k, v, out = _base(hq=6, hkv=4)
    assert binding.check_params(q, k, v, out=out) == binding.FA8_ERR_INVALID
    assert "multiple" in binding.last_error()


def test_bad_num_splits():
    q, k, v, out = _base()
    assert binding.check_params(q, k, v, num_splits=binding.MAX_SPLITS + 1) == binding.FA8_ERR_INVALID
    assert binding.check_params(q, k, v, num_splits=-1) == binding.FA8_ERR_INVALID


def test_misaligned_stride_rejected():
    q = _cpu((2, 16, 8, 144))[..., :128]      # head stride 144 is a multiple of 16: fine
    k = _cpu((2, 64, 2, 128))
    v = _cpu((2, 64, 2, 128))
    out = _cpu((2, 16, 8, 128), torch.bfloat16)
    assert binding.check_params(q, k, v, out=out) == binding.FA8_OK
    q2 = _cpu((2, 16, 8, 136))[..., :128]     # head stride 136 is not
    assert binding.check_params(q2, k, v, out=out) == binding.FA8_ERR_INVALID


def test_bad_window_and_dtype():
    q, k, v, out = _base()
    assert binding.check_params(q, k, v, out=out, window_left=-2) == binding.FA8_ERR_INVALID
    with pytest.raises(binding.FA8Error):
        binding.check_params(q.to(torch.float16), k, v, out=out)     # not E4M3 bytes
    with pytest.raises(binding.FA8Error):
        binding.check_params(q, k, v, out=out.to(torch.float32))


def test_paged_needs_power_of_two_pages_and_seqused():
    q = _cpu((4, 1, 8, 128))
    k = _cpu((10, 12, 2, 128))
    v = _cpu((10, 12, 2, 128))
    table = torch.zeros((4, 8), dtype=torch.int32)
    used = torch.full((4,), 40, dtype=torch.int32)
    out = _cpu((4, 1, 8, 128), torch.bfloat16)
    assert binding.check_params(q, k, v, out=out, block_table=table, seqused_k=used) == binding.FA8_ERR_INVALID
    assert "power of two" in binding.last_error()
    k = _cpu((10, 16, 2, 128))
    v = _cpu((10, 16, 2, 128))
    assert binding.check_params(q, k, v, out=out, block_table=table, seqused_k=used) == binding.FA8_OK
    assert binding.check_params(q, k, v, out=out, block_table=table) == binding.FA8_ERR_INVALID
    # a table narrower than max_seqlen_k / page_size
    assert binding.check_params(q, k, v, out=out, block_table=table, seqused_k=used,
                                max_seqlen_k=16 * 9) == binding.FA8_ERR_INVALID


def test_empty_problem_is_ok():
    q, k, v, out = _base(b=0)
    assert binding.check_params(q, k, v, out=out) == binding.FA8_OK
    q, k, v, out = _base(sq=0)
    assert binding.check_params(q, k, v, out=out) == binding.FA8_OK


def test_null_out_rejected_for_prefill():
    lib = binding.load()
    q, k, v, out = _base()
    p = binding._params(q, k, v, None, None, None, None, None, None, None, None, None, 0.0, False, -1, -1)
    assert lib.fa8_check_params(ctypes.byref(p), 0) == binding.FA8_ERR_INVALID


def test_workspace_bytes():
    n = binding.decode_workspace_bytes(4, 64, 1, 32, 128)
    o = 4 * 64 * 32 * 128 * 4
    l = 4 * 64 * 32 * 4
    assert n == (-(-o // 256)) * 256 + (-(-l // 256)) * 256
    assert binding.decode_workspace_bytes(-1, 1, 1, 1, 64) == 0


def test_num_splits_heuristic_bounds():
    for b, h, s in [(1, 1, 1), (64, 8, 8192), (4, 1, 131072), (1, 8, 100), (512, 8, 1024), (1, 1, 1 << 29)]:
        n = binding.decode_num_splits(b, h, s)
        assert 1 <= n <= binding.MAX_SPLITS
    # long single-sequence decode gets many splits; a full batch gets few
    assert binding.decode_num_splits(4, 1, 131072) >= 64
    assert binding.decode_num_splits(512, 8, 8192) <= 2


def _paged_decode_args(b=64, hq=32, hkv=8, d=128, page=16, max_sk=8192):
    # host-side values only (nothing is read on the device): a few pages suffice
    q = _cpu((b, hq, d))
    k = _cpu((4, page, hkv, d))
    v = _cpu((4, page, hkv, d))
    kw = dict(cu_seqlens_q=torch.arange(b + 1, dtype=torch.int32), seqused_k=torch.full((b,), 100, dtype=torch.int32),
              block_table=torch.zeros((b, max_sk // page), dtype=torch.int32), max_seqlen_q=1, max_seqlen_k=max_sk)
    return q, k, v, kw


def test_num_splits_for_picks_per_kernel():
    # paged GQA decode shape: the several-heads kernel has 64 x 2 one-wave units per split, so
    # 4 x 256 CUs / 128 = 8 splits; the per-head kernel has 64 x 8 units, 16 x 256 / 512 = 8
    q, k, v, kw = _paged_decode_args()
    assert binding.decode_num_splits_for(q, k, v, **kw) == 8
    # the standalone helper is the per-head kernel's heuristic with one row block per kv head
    assert binding.decode_num_splits(64, 8, 8192) == 8
    # long single-kv-head decode: capped at FA8_MAX_SPLITS, at least 4 granules per split
    q, k, v, kw = _paged_decode_args(b=4, hq=8, hkv=1, page=64, max_sk=131072)
    n = binding.decode_num_splits_for(q, k, v, **kw)
    assert 64 <= n <= binding.MAX_SPLITS
    assert binding.decode_num_splits(4, 1, 131072) == n      # 8/1 heads: one row block, per-head kernel
    # short sequences: at least four 64-key granules per split
    q, k, v, kw = _paged_decode_args(b=1, max_sk=512)
    assert binding.decode_num_splits_for(q, k, v, **kw) == 2
    assert binding.decode_num_splits(1, 8, 512) == 2


def test_decode_plan():
    q, k, v, kw = _paged_decode_args()
    plan = binding.decode_plan(q, k, v, num_splits=16, **kw)
    # paged GQA decode (4 rows per kv head): 4 kv heads per wave fill its 16 MFMA rows, 16-key
    # steps, 64 batches x 2 head groups x 16 splits
    assert plan == dict(kernel=1, block_keys=16, key_groups=1, heads_per_workgroup=4, workgroups=64 * 2 * 16)
    assert binding.decode_plan(q, k, v, num_splits=16, kernel=binding.DECODE_HEAD_GROUP, **kw) == plan
    plan = binding.decode_plan(q, k, v, num_splits=16, kernel=binding.DECODE_PER_HEAD, **kw)
    assert plan == dict(kernel=0, block_keys=64, key_groups=1, heads_per_workgroup=1, workgroups=64 * 8 * 16)
    with pytest.raises(binding.FA8Error):
        binding.decode_plan(q, k, v, num_splits=0, **kw)
    with pytest.raises(binding.FA8Error) as e:
        binding.decode_plan(q, k, v, num_splits=4, kernel=7, **kw)
    assert e.value.status == binding.FA8_ERR_INVALID
    # d = 96 has no several-heads kernel: asking for it is unsupported, the library's choice is not
    q96, k96, v96 = (torch.zeros(t.shape[:-1] + (96,), dtype=torch.uint8) for t in (q, k, v))
    with pytest.raises(binding.FA8Error) as e:
        binding.decode_plan(q96, k96, v96, num_splits=4, kernel=binding.DECODE_HEAD_GROUP, **kw)
    assert e.value.status == binding.FA8_ERR_UNSUPPORTED
    assert binding.decode_plan(q96, k96, v96, num_splits=4, **kw)["kernel"] == 0


def test_decode_ex_rejects_before_launch():
    # the explicit-kernel entry point validates the choice before touching any pointer
    lib = binding.load()
    q, k, v, kw = _paged_decode_args()
    p = binding._params(q, k, v, kw["cu_seqlens_q"], None, kw["seqused_k"], kw["block_table"], 1, 8192,
                        None, None, None, 0.0, False, -1, -1)
    assert lib.fa8_fwd_decode_splitkv_ex(ctypes.byref(p), 4, 5, None, None, None) == binding.FA8_ERR_INVALID
    q96, k96, v96 = (torch.zeros(t.shape[:-1] + (96,), dtype=torch.uint8) for t in (q, k, v))
    p = binding._params(q96, k96, v96, kw["cu_seqlens_q"], None, kw["seqused_k"], kw["block_table"], 1, 8192,
                        None, None, None, 0.0, False, -1, -1)
    assert lib.fa8_fwd_decode_splitkv_ex(ctypes.byref(p), 4, binding.DECODE_HEAD_GROUP, None, None,
                                         None) == binding.FA8_ERR_UNSUPPORTED


def test_prefill_grid_limit():
    # a launch holds at most 2^32 - 1 threads along x: 2^24 workgroups of 256 threads. Varlen
    # inputs deal 8 * ceil(B * Hkv / 8) groups x ceil(max_seqlen_q / 128) row blocks x g heads:
    # 64 sequences of up to 512K tokens with 64/8 heads need exactly 2^24 and are rejected before
    # any launch; half that length fits (host values only, nothing is read)
    lib = binding.load()
    b, hq, hkv, d = 64, 64, 8, 128

    def status(max_sq):
        q = torch.zeros((16, hq, d), dtype=torch.uint8)
        k = torch.zeros((16, hkv, d), dtype=torch.uint8)
        cu = torch.zeros(b + 1, dtype=torch.int32)
        p = binding._params(q, k, k, cu, cu, None, None, max_sq, max_sq, None, None, None, 0.0, True, -1, -1)
        binding._set_out(p, torch.zeros((16, hq, d), dtype=torch.bfloat16), None, True)
        return lib.fa8_fwd_prefill(ctypes.byref(p), None)

    # 8 * 64 * 4096 * 8 = 2^24 workgroups of 256 threads
    assert status(512 * 1024) == binding.FA8_ERR_INVALID
    assert "2^32 threads" in binding.last_error()
    # the same check without launching
    q = torch.zeros((16, hq, d), dtype=torch.uint8)
    k = torch.zeros((16, hkv, d), dtype=torch.uint8)
    cu = torch.zeros(b + 1, dtype=torch.int32)
    out = torch.zeros((16, hq, d), dtype=torch.bfloat16)
    assert binding.check_params(q, k, k, cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=512 * 1024,
                                max_seqlen_k=512 * 1024, causal=True, out=out) == binding.FA8_ERR_INVALID


def test_quantize_q_host_validation():
    # argument errors are reported before any launch (no GPU needed)
    import ctypes
    from fa8_fwd_amd import binding
    lib = binding.load()
    p = binding.QuantParams()
    p.batch, p.heads_q, p.heads_kv, p.d, p.max_seqlen_q = 2, 6, 4, 128, 16   # 6 % 4 != 0
    p.in_dtype = binding.FA8_OUT_BF16
    assert lib.fa8_quantize_q(ctypes.byref(p), None, None) == binding.FA8_ERR_INVALID
    p.heads_q, p.d = 8, 80
    assert lib.fa8_quantize_q(ctypes.byref(p), None, None) == binding.FA8_ERR_UNSUPPORTED
    p.d, p.in_dtype = 128, 7
    assert lib.fa8_quantize_q(ctypes.byref(p), None, None) == binding.FA8_ERR_INVALID
    p.in_dtype, p.batch = binding.FA8_OUT_FP16, 0          # empty problem: nothing to do
    assert lib.fa8_quantize_q(ctypes.byref(p), None, None) == binding.FA8_OK
    p.batch = 3
    assert lib.fa8_quantize_q_workspace_bytes(ctypes.byref(p)) == 3 * 4 * 1 * 4   # 16 rows: one 32-row chunk


def test_kernels_use_no_scratch():
    """The last build recorded each kernel's registers and scratch: no template instance spills
    in its loop or calls a helper with a stack frame, and the prefill and the decode kernels keep
    the waves per SIMD their launch bounds ask for."""
    from fa8_fwd_amd import build as B
    if not os.path.exists(B.RESOURCES):
        pytest.skip("library not built")
    usage = __import__("json").load(open(B.RESOURCES))
    assert usage, "no kernel resource remarks recorded"
    for name, u in usage.items():
        assert int(u["ScratchSize"]) <= B.MAX_SCRATCH_BYTES, (name, u)
        assert u.get("Dynamic Stack") != "True", name
        if "fa8_prefill_kernel" in name or "fa8_decode_heads_kernel" in name:
            assert int(u["Occupancy"]) >= 2, (name, u)
    assert any("fa8_prefill_kernel" in n for n in usage) and any("fa8_decode_kernel" in n for n in usage)


def test_prefill_mx_host_validation():
    """fa8_fwd_prefill_mx rejects what it does not take before any launch (host pointers are
    never dereferenced on these paths)."""
    lib = binding.load()
    q = torch.zeros((1, 64, 2, 128), dtype=torch.uint8)
    k = torch.zeros((1, 64, 1, 128), dtype=torch.uint8)
    v = torch.zeros((1, 64, 1, 128), dtype=torch.uint8)
    qs = torch.zeros((1, 64, 2, 4), dtype=torch.uint8)
    ks = torch.zeros((1, 64, 1, 4), dtype=torch.uint8)
    vs = torch.zeros((1, 2, 1, 128), dtype=torch.uint8)
    out = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16)

    def call(qq=q, kk=k, vv=v, qsc=qs, ksc=ks, vsc=vs, **kw):
        p = binding._params(qq, kk, vv, kw.get("cu_q"), None, None, None, kw.get("max_sq"), None,
                            kw.get("dq"), None, None, 0.0, True, -1, -1)
        binding._set_out(p, out if qq.shape[-1] == 128 else torch.zeros(tuple(qq.shape[:-1]) + (vv.shape[-1],),
                                                                         dtype=torch.bfloat16), None, False)
        m = binding.MXScales(qsc.data_ptr(), qsc.stride(0), qsc.stride(1), qsc.stride(2),
                             ksc.data_ptr(), ksc.stride(0), ksc.stride(1), ksc.stride(2),
                             vsc.data_ptr(), vsc.stride(0), vsc.stride(1), vsc.stride(2))
        return lib.fa8_fwd_prefill_mx(ctypes.byref(p), ctypes.byref(m), None)

    assert lib.fa8_fwd_prefill_mx(None, None, None) == binding.FA8_ERR_INVALID
    # descales are replaced by the block scales
    assert call(dq=torch.ones(())) == binding.FA8_ERR_INVALID
    assert "descale" in binding.last_error()
    # (96, 96) has no MX kernel
    q96, k96, v96 = (torch.zeros(t.shape[:-1] + (96,), dtype=torch.uint8) for t in (q, k, v))
    assert call(qq=q96, kk=k96, vv=v96, qsc=qs[..., :3].contiguous(), ksc=ks[..., :3].contiguous(),
                vsc=vs[..., :96].contiguous()) == binding.FA8_ERR_UNSUPPORTED
    # varlen Q is not taken
    qv = torch.zeros((64, 2, 128), dtype=torch.uint8)
    cu = torch.tensor([0, 64], dtype=torch.int32)
    assert call(qq=qv, cu_q=cu, max_sq=64) == binding.FA8_ERR_UNSUPPORTED
    # V scale rows must keep 16-byte alignment
    vs_bad = torch.zeros((1, 2, 1, 136), dtype=torch.uint8)[..., :128]
    assert call(vsc=vs_bad) == binding.FA8_ERR_INVALID
    assert "16" in binding.last_error()

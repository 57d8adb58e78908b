"""Writes tests/golden/manifest.json: the sha256 of every seeded input buffer of the five measured
workloads (tiny, paged GQA decode, causal prefill, long-KV decode, mixed varlen at both head-dim
pairs), and of the CPU oracle's output on the tiny workload. The GPU path and the oracle consume
these exact bytes; the manifest pins the generators (and the oracle's tiny result) against silent
change. Calls only fa8_fwd_amd.inputs (random draws, no method arithmetic) and oracle/.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

FIELDS = ("q", "k", "v", "cu_seqlens_q", "cu_seqlens_k", "seqused_k", "block_table", "q_descale", "k_descale",
          "v_descale")


def workloads():
    from fa8_fwd_amd import inputs as gen
    return {
        "tiny": lambda: gen.tiny(0),
        "paged_gqa_decode": lambda: gen.paged_gqa_decode(1),
        "causal_prefill": lambda: gen.causal_prefill(2),
        "long_kv_decode": lambda: gen.long_kv_decode(3),
        "mixed_varlen_d256": lambda: gen.mixed_varlen(4, d=256, dv=256),
        "mixed_varlen_d192_128": lambda: gen.mixed_varlen(4, d=192, dv=128),
    }


def digest(a) -> str:
    a = np.ascontiguousarray(a)
    h = hashlib.sha256()
    h.update(str(a.dtype).encode() + str(a.shape).encode())
    h.update(a.tobytes())
    return h.hexdigest()


def input_hashes(inp) -> dict:
    return {f: digest(getattr(inp, f)) for f in FIELDS if getattr(inp, f) is not None}


def oracle_hash(inp) -> str:
    import oracle
    o, l = oracle.attention_full(inp, threads=1)
    return digest(np.concatenate([o.reshape(-1), l.reshape(-1)]))


def build() -> dict:
    out = {"inputs": {}, "oracle": {}}
    for name, make in workloads().items():
        inp = make()
        out["inputs"][name] = input_hashes(inp)
        if name == "tiny":
            out["oracle"][name] = oracle_hash(inp)
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "manifest.json"), "w") as f:
        json.dump(build(), f, indent=1, sort_keys=True)
        f.write("\n")

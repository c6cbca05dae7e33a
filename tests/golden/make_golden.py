"""Writes tests/golden/tiny_r4_c2_d16_oracle.json: the CPU oracle's results on
the tiny workload (cu_seqlens [0, 37, 64], ratio 4, coff 2, head_dim 16,
seed 0), as a regression fixture.  It calls only the oracle and the seeded
input generator; it never touches the HIP library.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from gated_pooling_amd import inputs  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main():
    wl = inputs.WORKLOADS["tiny_r4_c2_d16"]
    N = oracle.total_comp(wl.cu_seqlens, wl.ratio)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    kvb, scb, apen, doutb = inputs.bits(kv), inputs.bits(sc), ape.numpy(), inputs.bits(dout)
    args = (kvb, scb, apen, wl.cu_seqlens, wl.total_tokens, wl.ratio, wl.coff, wl.head_dim)
    out = oracle.fwd_f32(*args)
    dkv, dsc, dape, _, _ = oracle.bwd_f32(*args, doutb)
    fix = {
        "about": "CPU oracle (fp32 evaluation order) on the tiny workload, seed 0; written by make_golden.py",
        "workload": wl.name, "cu_seqlens": list(wl.cu_seqlens), "total_tokens": wl.total_tokens,
        "ratio": wl.ratio, "coff": wl.coff, "head_dim": wl.head_dim, "total_comp": N,
        "inputs_sha256": {"kv": digest(kvb), "score": digest(scb), "ape": digest(apen), "dout": digest(doutb)},
        "out_bits": [[f"{v:04x}" for v in row] for row in out],
        "dkv_sha256": digest(dkv), "dscore_sha256": digest(dsc),
        "dape": [[float(f"{v:.12e}") for v in row] for row in dape],
    }
    with open(os.path.join(HERE, "tiny_r4_c2_d16_oracle.json"), "w") as f:
        json.dump(fix, f, indent=1)


if __name__ == "__main__":
    main()

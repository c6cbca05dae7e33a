"""Parity of one tuning configuration of libcsa against the oracle.

libcsa reads its tuning knobs (CSA_* environment variables: columns per lane,
grid caps, workgroup size, column slice, uniform-row path, prefetch depth)
once per process, so each configuration runs in a process of its own:

    CSA_BWD_PREFETCH=4 python -m tests.tuning_parity
    CSA_R128_BWD_WGS=5 python -m tests.tuning_parity r128    # ratio-128 packs only

Every case is checked bit for bit (out, dKV, dScore, zero ownership) and
dAPE to its tolerance, exactly as in the main parity tests.  Prints one line
per case and exits non-zero on the first mismatch.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import gated_pooling_amd as G
from gated_pooling_amd import inputs
from tests.test_parity_gpu import check_against_oracle, run_gpu


def cases():
    for name in ("1x8192_d512_r4_c2", "ragged_d128_r4_c2", "ragged_d128_r4_c1", "tiny_r4_c2_d16",
                 "1x8192_d128_r2_c2"):
        wl = inputs.WORKLOADS[name]
        yield name, wl, True
    rng = np.random.default_rng(77)
    lengths = rng.integers(0, 300, size=60).tolist()   # 60 segments: LDS table
    yield "random60_d256_r2_c2", inputs.custom("r60", lengths, int(sum(lengths)) + 5, 2, 2, 256, seed=3), True
    lengths = rng.integers(0, 200, size=9).tolist()    # padded rows (96 = 48 chunks of 2) and odd d
    yield "random9_d96_r4_c2", inputs.custom("r9", lengths, int(sum(lengths)) + 3, 4, 2, 96, seed=6), True
    yield "random9_d65_r2_c1", inputs.custom("r9b", lengths, int(sum(lengths)) + 3, 2, 1, 65, seed=7), False
    lengths = rng.integers(0, 12, size=2500).tolist()  # above the LDS table limit: workspace table
    yield "random2500_d128_r4_c2", inputs.custom("r2500", lengths, int(sum(lengths)) + 9, 4, 2, 128, seed=4), False


def cases_r128():
    """ratio-128 packs: several blocks per segment, tails, a segment shorter
    than 128, padding rows, both coffs, one and several column slices."""
    rng = np.random.default_rng(1280)
    for i, (c, d, nseg) in enumerate(((2, 128, 4), (1, 64, 5), (2, 192, 3), (1, 256, 2))):
        lengths = rng.integers(0, 900, size=nseg).tolist()
        lengths[1] = int(rng.integers(1, 128))
        T = int(sum(lengths)) + int(rng.integers(1, 200))
        yield f"r128_S{nseg}_c{c}_d{d}", inputs.custom("t128", lengths, T, 128, c, d, seed=60 + i), bool(i % 2)


def main(argv):
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    G.lib()
    for name, wl, host in (cases_r128() if "r128" in argv else cases()):
        cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
        N = G.csa_compressor_total_comp(cu, r)
        kv, sc, ape, dout = inputs.make_tensors(wl, N)
        got = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N, host=host)
        check_against_oracle(cu, T, r, c, d, kv, sc, ape, dout, got)
        print(f"ok {name}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

"""The fp32 eager PyTorch formulation that bench.py times as context agrees
with the oracle (CPU, small packs).  It is compared with the double-precision
oracle, since its own fp32 evaluation order differs from the pinned one."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from bench import EagerCompressor
from gated_pooling_amd import inputs


@pytest.mark.parametrize("name", ["tiny_r4_c2_d16"])
@pytest.mark.parametrize("coff", [1, 2])
@pytest.mark.parametrize("ratio", [2, 4])
def test_eager_matches_double_oracle(name, coff, ratio):
    base = inputs.WORKLOADS[name]
    lengths = np.diff(base.cu_seqlens).tolist() + [0, 3, 9]
    wl = inputs.custom("e", lengths, int(sum(lengths)) + 5, ratio, coff, 16, seed=2)
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    N = oracle.total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    ec = EagerCompressor(cu, T, r, c, d, torch.device("cpu"))
    assert ec.N == N
    out, dkv, dsc, dape = ec.step(kv, sc, ape, dout)
    kvd = oracle.f64_from_bits(inputs.bits(kv))
    scd = oracle.f64_from_bits(inputs.bits(sc))
    doutd = oracle.f64_from_bits(inputs.bits(dout))
    out_ref = oracle.fwd_f64(kvd, scd, ape.double().numpy(), cu, T, r, c, d)
    dkv_ref, dsc_ref, dape_ref = oracle.bwd_f64(kvd, scd, ape.double().numpy(), cu, T, r, c, d, doutd)
    np.testing.assert_allclose(out.numpy(), out_ref, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dkv.numpy(), dkv_ref, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dsc.numpy(), dsc_ref, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(dape.numpy(), dape_ref, rtol=1e-4, atol=1e-6)

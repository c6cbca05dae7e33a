"""The seeded workload generator follows its stated recipe."""
import numpy as np
import torch

from gated_pooling_amd import inputs
from tests import brute


def test_ragged_pack_recipe():
    for c in (1, 2):
        wl = inputs.WORKLOADS[f"ragged_d128_r4_c{c}"]
        cu = wl.cu_seqlens
        L = np.diff(cu)
        assert wl.total_tokens == 32768 and cu[0] == 0
        assert 28000 <= cu[-1] <= 32768 - 1  # padding rows exist
        assert L[0] == 1 and L[-1] == 0 and (L == 3).any()  # short and empty segments
        assert ((L % 4) != 0).sum() >= 3  # seqlen % ratio tails
        assert L.max() <= 4096


def test_generator_is_deterministic_and_shaped():
    wl = inputs.WORKLOADS["tiny_r4_c2_d16"]
    N = brute.count_outputs(wl.cu_seqlens, wl.ratio)
    a = inputs.make_tensors(wl, N)
    b = inputs.make_tensors(wl, N)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    kv, sc, ape, dout = a
    assert kv.shape == (64, 32) and kv.dtype == torch.bfloat16
    assert sc.shape == (64, 32) and ape.shape == (4, 32) and ape.dtype == torch.float32
    assert dout.shape == (15, 16)
    assert 0.005 < float(ape.std()) < 0.05


def test_headline_shapes():
    wl = inputs.WORKLOADS[inputs.HEADLINE]
    assert wl.cu_seqlens == (0, 8192, 16384, 24576)
    assert (wl.total_tokens, wl.ratio, wl.coff, wl.head_dim) == (24576, 4, 2, 512)

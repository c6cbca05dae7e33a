"""Golden fixtures: hand-worked examples (exact) and the oracle's own
regression fixture on the tiny workload."""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gated_pooling_amd import inputs

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
HAND = json.load(open(os.path.join(HERE, "hand_examples.json")))["examples"]


def _bf16_bits(values):
    return inputs.bits(torch.tensor(values, dtype=torch.float32).to(torch.bfloat16))


@pytest.mark.parametrize("ex", HAND, ids=[e["name"] for e in HAND])
def test_hand_example_exact(ex):
    """Both oracles reproduce the paper-derived values exactly (every weight
    is 1/K with K a power of two, so nothing rounds)."""
    cu, T, r, c, d = ex["cu_seqlens"], ex["total_tokens"], ex["ratio"], ex["coff"], ex["head_dim"]
    W = c * d
    kv = _bf16_bits(ex["kv"])
    sc = np.zeros((T, W), np.uint16)
    ape = np.zeros((r, W), np.float32)
    dout = _bf16_bits(ex["dout"])
    out = oracle.f64_from_bits(oracle.fwd_f32(kv, sc, ape, cu, T, r, c, d))
    assert np.array_equal(out, np.array(ex["out"], float))
    dkv, dsc, dape, _, _ = oracle.bwd_f32(kv, sc, ape, cu, T, r, c, d, dout)
    assert np.array_equal(oracle.f64_from_bits(dkv), np.array(ex["dkv"], float))
    assert np.array_equal(oracle.f64_from_bits(dsc), np.array(ex["dscore"], float))
    assert np.array_equal(dape, np.array(ex["dape"], float))
    # never-consumed slots are +0.0 exactly (bit pattern 0x0000)
    zero = np.array(ex["dkv"], float) == 0
    assert np.all(dkv[zero] == 0) and np.all(dsc[zero] == 0)
    kv64 = oracle.f64_from_bits(kv)
    o64 = oracle.fwd_f64(kv64, np.zeros((T, W)), np.zeros((r, W)), cu, T, r, c, d)
    assert np.array_equal(o64, np.array(ex["out"], float))
    dkv64, dsc64, dape64 = oracle.bwd_f64(kv64, np.zeros((T, W)), np.zeros((r, W)), cu, T, r, c, d,
                                         np.array(ex["dout"], float))
    assert np.array_equal(dkv64, np.array(ex["dkv"], float))
    assert np.array_equal(dsc64, np.array(ex["dscore"], float))
    assert np.array_equal(dape64, np.array(ex["dape"], float))


def test_tiny_regression_fixture():
    """The oracle and the seeded generator still produce the committed tiny
    fixture (guards against unintended changes to either)."""
    fix = json.load(open(os.path.join(HERE, "tiny_r4_c2_d16_oracle.json")))
    wl = inputs.WORKLOADS[fix["workload"]]
    N = oracle.total_comp(wl.cu_seqlens, wl.ratio)
    assert N == fix["total_comp"] == 15
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    kvb, scb, apen, doutb = inputs.bits(kv), inputs.bits(sc), ape.numpy(), inputs.bits(dout)
    dig = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()  # noqa: E731
    assert dig(kvb) == fix["inputs_sha256"]["kv"]
    assert dig(scb) == fix["inputs_sha256"]["score"]
    assert dig(apen) == fix["inputs_sha256"]["ape"]
    assert dig(doutb) == fix["inputs_sha256"]["dout"]
    args = (kvb, scb, apen, wl.cu_seqlens, wl.total_tokens, wl.ratio, wl.coff, wl.head_dim)
    out = oracle.fwd_f32(*args)
    assert [[f"{v:04x}" for v in row] for row in out] == fix["out_bits"]
    dkv, dsc, dape, _, _ = oracle.bwd_f32(*args, doutb)
    assert dig(dkv) == fix["dkv_sha256"] and dig(dsc) == fix["dscore_sha256"]
    np.testing.assert_allclose(dape, np.array(fix["dape"]), rtol=1e-11, atol=0)

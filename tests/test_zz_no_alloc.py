"""The allocation-free backward (csa_compressor_bwd_noalloc) against the
backward with a caller workspace (csa_compressor_bwd), through the C ABI.

Both run the same kernels, so dKV, dScore and dAPE must be bit-identical.
Each case makes two calls in a row on the library's scratch, the second on a
smaller problem, so the second call runs on what the first left behind.  The
size limit is checked on the host: a problem whose workspace exceeds the
scratch is refused before anything is enqueued.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import gated_pooling_amd as G
from gated_pooling_amd import inputs

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0
SCRATCH_BYTES = 40 * 2 ** 20


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    return torch.device("cuda:0")


def _both(dev, wl, host):
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    W, S = c * d, len(cu) - 1
    N = G.csa_compressor_total_comp(cu, r)
    assert G.csa_compressor_bwd_workspace_size(r, c, d, S, T, N) <= SCRATCH_BYTES
    kv, sc, ape, dout = (t.to(dev) for t in inputs.make_tensors(wl, N))
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    cu_h = G.host_cu(cu if host else None)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    res = []
    for noalloc in (False, True):
        dkv = torch.full((T, W), NAN_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
        dsc = torch.full((T, W), NAN_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
        dape = torch.full((r, W), float("nan"), device=dev)
        if noalloc:
            G.csa_compressor_bwd_noalloc(P(kv), P(sc), P(ape), P(cu_d), cu_h, S, T, N, r, c, d, P(dout), P(dkv),
                                         P(dsc), P(dape), 1, s)
        else:
            nb = G.csa_compressor_bwd_workspace_size(r, c, d, S, T, N)
            ws = G.workspace(nb, dev)
            G.csa_compressor_bwd(P(kv), P(sc), P(ape), P(cu_d), cu_h, S, T, N, r, c, d, P(dout), P(dkv), P(dsc),
                                 P(dape), 1, P(ws), ws.numel(), s)
        torch.cuda.synchronize()
        res.append((inputs.bits(dkv.cpu()), inputs.bits(dsc.cpu()), dape.cpu().numpy()))
    for x, y, name in zip(res[0], res[1], ("dkv", "dscore", "dape")):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    assert not np.isnan(res[1][2]).any()


def _many_segments(c):
    rng = np.random.default_rng(31)
    lengths = rng.integers(0, 14, size=3000).tolist()
    return inputs.custom("many", lengths, int(sum(lengths)) + 11, 4, c, 32, seed=8)


PAIRS = [
    # (first, second): the second problem is smaller than the first
    ("3x8192_d512_r4_c2", "ragged_d128_r4_c1", True),
    ("ragged_d128_r4_c2", "tiny_r4_c2_d16", False),
    ("3x8192_d512_r2_c2", "1x8192_d128_r2_c2", True),
    ("ragged_d128_r128_c2", "r128_small", False),
    ("many_c2", "many_c1", False),
]


def _wl(name):
    if name == "r128_small":
        return inputs.custom("r128s", [300, 5, 700], 1100, 128, 2, 64, seed=4)
    if name.startswith("many_"):
        return _many_segments(int(name[-1]))
    return inputs.WORKLOADS[name]


@pytest.mark.parametrize("first,second,host", PAIRS, ids=[f"{a}-then-{b}" for a, b, _ in PAIRS])
def test_noalloc_matches_workspace_backward(dev, first, second, host):
    print("noalloc pair", first, second, flush=True)
    _both(dev, _wl(first), host)
    _both(dev, _wl(second), host)


def test_noalloc_refuses_problems_beyond_its_scratch(dev):
    # ten million segments: a 40 MB segment table plus 32 MiB of ratio-128
    # dAPE partials exceed the scratch
    S, T, N, r, c, d = 10_000_000, 65536, 512, 128, 2, 64
    need = G.csa_compressor_bwd_workspace_size(r, c, d, S, T, N)
    assert need > SCRATCH_BYTES
    null = ctypes.c_void_p(0)
    st = G.lib().csa_compressor_bwd_noalloc(null, null, null, null, null, S, T, N, r, c, d, null, null, null, null,
                                            1, null)
    assert st == G.CSA_STATUS_WORKSPACE_TOO_SMALL
    assert "scratch" in G.csa_last_error()

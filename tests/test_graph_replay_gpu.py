"""hipGraph capture / replay with static-capacity buffers [PR5984: zero-init
folding commit (the padding class under graph replay); graph-benchmark
commit].

The forward and the backward are captured once (torch.cuda.graph on the
capture stream; libcsa allocates nothing and issues no memset, so the graph
holds only its kernels) with the device cu_seqlens and no host copy.  Between
replays the pack changes in place -- segment lengths, tails, short and empty
segments, and the amount of padding past cu[S] -- while the number of
segments, total_comp and the token capacity stay fixed.  Every replay starts
from NaN-filled outputs and is checked against the oracle exactly as the
eager parity tests are; eager work and synchronisations run between replays.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_pooling_amd as G
from gated_pooling_amd import inputs
from tests.test_parity_gpu import NAN_BF16, check_against_oracle

pytestmark = pytest.mark.gpu

D = 128
# per ratio: token capacity, total_comp and the packs; the same S = 3 and
# total_comp for every pack of a ratio, while cu[S] and the tails vary
CONFIGS = {
    4: (4608, 1000, [
        [1000, 2000, 1000],
        [1003, 2001, 1002],
        [4, 3996, 2],
        [0, 4000, 0],
        [1, 3, 4003],
        [2001, 1001, 1003],
    ]),
    128: (2048, 12, [
        [512, 768, 256],
        [520, 800, 300],
        [127, 1536, 10],
        [0, 1536, 0],
        [1, 3, 1600],
        [1000, 300, 400],
    ]),
}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("R", [4, 128])
@pytest.mark.parametrize("coff", [1, 2])
def test_graph_replay_with_changing_packs(dev, coff, R):
    T_CAP, N, PACKS = CONFIGS[R]
    W = coff * D
    S = 3
    for lengths in PACKS:
        assert G.csa_compressor_total_comp(np.concatenate([[0], np.cumsum(lengths)]).tolist(), R) == N
    kv = torch.empty(T_CAP, W, dtype=torch.bfloat16, device=dev)
    sc = torch.empty_like(kv)
    ape = torch.empty(R, W, dtype=torch.float32, device=dev)
    dout = torch.empty(N, D, dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(S + 1, dtype=torch.int32, device=dev)
    out = torch.empty(N, D, dtype=torch.bfloat16, device=dev)
    dkv, dsc = torch.empty_like(kv), torch.empty_like(kv)
    dape = torch.empty(R, W, dtype=torch.float32, device=dev)
    fws = G.workspace(G.csa_compressor_fwd_workspace_size(R, coff, D, S, T_CAP, N), dev)
    bws = G.workspace(G.csa_compressor_bwd_workspace_size(R, coff, D, S, T_CAP, N), dev)

    def step():
        G.compressor_fwd(kv, sc, ape, cu, R, coff, N, out=out, ws=fws)
        G.compressor_bwd(kv, sc, ape, cu, R, coff, N, dout, dkv=dkv, dscore=dsc, dape=dape, ws=bws)

    def load(i, lengths):
        wl = inputs.custom(f"g{i}", lengths, T_CAP, R, coff, D, seed=100 + i)
        k, s, a, g = inputs.make_tensors(wl, N)
        kv.copy_(k)
        sc.copy_(s)
        ape.copy_(a)
        dout.copy_(g)
        cu.copy_(torch.tensor(list(wl.cu_seqlens), dtype=torch.int32))
        for t in (out, dkv, dsc):
            t.view(torch.int16).fill_(NAN_BF16)
        dape.fill_(float("nan"))
        return wl, (k, s, a, g)

    # warm up once eagerly on the capture-to-be buffers, then capture
    load(0, PACKS[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for i, lengths in enumerate(PACKS):
            print("replay", rep, "pack", i, lengths, flush=True)
            wl, (k, s, a, g) = load(i, lengths)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = (inputs.bits(out.cpu()), inputs.bits(dkv.cpu()), inputs.bits(dsc.cpu()), dape.cpu().numpy())
            check_against_oracle(list(wl.cu_seqlens), T_CAP, R, coff, D, k, s, a, g, got)

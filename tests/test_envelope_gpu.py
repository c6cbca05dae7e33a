"""GPU tests at the edges of the supported envelope, and of the binding.

* The largest buffer the 32-bit offsets allow at coff 2, head_dim 512:
  total_tokens = 2^21 - 2 rows, so kv/score/dkv/dscore are 2^32 - 4096 bytes
  each.  The pack fills it with one long segment whose last blocks and tail
  sit just below 2^32 bytes, a short first segment, a segment shorter than
  ratio and 4149 padding rows, so the zero workgroups sweep the top 8.5 MB of
  both gradient buffers.  The inputs are drawn on the device (seeded); the
  oracle checks crops of whole blocks copied back to the host (a crop is a
  pack of its own whose inner windows equal the full pack's), the zero
  classes and full overwrite are checked on the device, and dAPE by the
  softmax identity sum_i (dAPE[i, j] + dAPE[i, d + j]) = 0.
* The tensor-level binding on a side stream: outputs and the local workspace
  are allocated on the launch stream, so the caching allocator cannot hand
  them to work on another stream while the kernels still run.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_pooling_amd as G
import oracle
from gated_pooling_amd import inputs
from tests.test_parity_gpu import NAN_BF16, check_against_oracle, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    return torch.device("cuda:0")


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("host", [True, False], ids=["args_table", "device_table"])
def test_largest_buffer_at_the_32bit_edge(dev, host):
    r, c, d = 4, 2, 512
    W = c * d
    T = 2 ** 21 - 2
    lengths = [5001, 3, 2087997]                 # tails 1, 3 (short), 1
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64).tolist()
    assert T * W * 2 == 2 ** 32 - 4096 and cu[-1] == T - 4149
    G.csa_compressor_check_support(r, c, d, 3, T, 0)
    N = G.csa_compressor_total_comp(cu, r)
    print("edge pack", cu, "T", T, "N", N, "host table" if host else "device table", flush=True)

    g = torch.Generator(device=dev)
    g.manual_seed(11)
    kv = torch.randn(T, W, generator=g, device=dev, dtype=torch.bfloat16)
    sc = torch.randn(T, W, generator=g, device=dev, dtype=torch.bfloat16)
    ape = torch.randn(r, W, generator=g, device=dev) * 0.02
    dout = torch.randn(N, d, generator=g, device=dev, dtype=torch.bfloat16)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    out = torch.full((N, d), NAN_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
    dkv = torch.full((T, W), NAN_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
    dsc = torch.full((T, W), NAN_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
    dape = torch.full((r, W), float("nan"), device=dev)
    cu_h = cu if host else None
    G.compressor_fwd(kv, sc, ape, cu_d, r, c, N, out=out, cu_seqlens_host=cu_h)
    G.compressor_bwd(kv, sc, ape, cu_d, r, c, N, dout, dkv=dkv, dscore=dsc, dape=dape, cu_seqlens_host=cu_h)
    torch.cuda.synchronize()

    # full overwrite: no NaN canary left anywhere
    for name, t in (("out", out), ("dkv", dkv), ("dscore", dsc)):
        assert int((t.view(torch.int16) == NAN_BF16).sum()) == 0, name
    # zero classes: rows of the short segment, the tails and the padding rows
    zero_rows = [(cu[0] + 1250 * r, cu[1]), (cu[1], cu[2]), (cu[2] + (lengths[2] // r) * r, cu[3]), (cu[3], T)]
    for a, b in zero_rows:
        for t in (dkv, dsc):
            assert int(t[a:b].view(torch.int16).count_nonzero()) == 0, (a, b)
    # first half of each segment's last block
    for s, L in ((0, lengths[0]), (2, lengths[2])):
        last = cu[s] + (L // r - 1) * r
        for t in (dkv, dsc):
            assert int(t[last:last + r, :d].view(torch.int16).count_nonzero()) == 0, (s, last)

    # crops of whole blocks against the oracle
    off = [0, lengths[0] // r, lengths[0] // r]                 # first output row of each segment
    crops = [(0, 0, 1250, True), (2, 0, 40, False), (2, 260000, 40, False), (2, lengths[2] // r - 40, 40, True)]
    ape_h = ape.cpu().numpy()
    for s, b0, nbk, to_end in crops:
        start = cu[s] + b0 * r
        stop = cu[s + 1] if to_end else start + nbk * r
        L = stop - start
        kvb, scb = _bits(kv[start:stop]), _bits(sc[start:stop])
        gb = _bits(dout[off[s] + b0:off[s] + b0 + nbk])
        ccu = [0, L]
        o_ref = oracle.fwd_f32(kvb, scb, ape_h, ccu, L, r, c, d)
        dkv_ref, dsc_ref, _, _, _ = oracle.bwd_f32(kvb, scb, ape_h, ccu, L, r, c, d, gb)
        first = 0 if b0 == 0 else 1                         # a crop's block 0 is masked unless it starts the segment
        o_got = _bits(out[off[s] + b0 + first:off[s] + b0 + nbk])
        assert np.array_equal(o_got, o_ref[first:]), ("out", s, b0)
        rows_end = L if to_end else (nbk - 1) * r               # the next block's window reads the last first half
        for got, ref, name in ((dkv, dkv_ref, "dkv"), (dsc, dsc_ref, "dscore")):
            gg = _bits(got[start + first * r:start + rows_end])
            assert np.array_equal(gg, ref[first * r:rows_end]), (name, s, b0)
    # dAPE: finite and the softmax identity per column
    dp = dape.cpu().double().numpy()
    assert np.isfinite(dp).all()
    tot = dp[:, :d].sum(axis=0) + dp[:, d:].sum(axis=0)
    assert np.abs(tot).max() <= 1e-3 * np.abs(dp).sum(axis=0).max()
    del kv, sc, dkv, dsc
    torch.cuda.empty_cache()


def test_binding_on_a_side_stream(dev):
    wl = inputs.WORKLOADS["ragged_d128_r4_c2"]
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    N = G.csa_compressor_total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    kv_d, sc_d, ape_d, dout_d = kv.to(dev), sc.to(dev), ape.to(dev), dout.to(dev)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = G.compressor_fwd(kv_d, sc_d, ape_d, cu_d, r, c, N, stream=side)
    dkv, dsc, dape = G.compressor_bwd(kv_d, sc_d, ape_d, cu_d, r, c, N, dout_d, stream=side)
    # meanwhile, the default stream allocates and fills memory of the same sizes
    junk = [torch.full((T, c * d), 7, dtype=torch.int16, device=dev) for _ in range(4)]
    del junk
    side.synchronize()
    torch.cuda.synchronize()
    got = (inputs.bits(out.cpu()), inputs.bits(dkv.cpu()), inputs.bits(dsc.cpu()), dape.cpu().numpy())
    check_against_oracle(cu, T, r, c, d, kv, sc, ape, dout, got)
    ref = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N)
    for x, y in zip(got, ref):
        assert np.array_equal(x, y)

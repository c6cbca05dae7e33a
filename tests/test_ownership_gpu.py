"""Disjoint stores: every dKV/dScore slot is written exactly once.

The backward's contract is that every slot of [0, total_tokens) x [0, W) of
dkv and dscore gets exactly one store -- its gradient from the one window
that reads it, or +0.0 from the one owner of its never-read class -- with no
atomics and no slot written twice [PR5984: zero-init folding commit].  The
NaN-prefill parity tests prove full overwrite; this proves the "exactly once".

libcsa_debug.so is the same library built with -DCSA_DEBUG_OWNERSHIP: every
store to dkv/dscore also adds 1 to a uint32 counter per element it writes
(csa_debug_ownership_counters registers the counter arrays).  After one
backward every counter must be exactly 1.  The debug build's results are
also compared bit for bit with libcsa.so's on the same inputs.  Packs: the
ragged packs at ratio 2, 4 and 128 with coff 1 and 2 (tails, a 1-token and a
(ratio-1)-token segment, an empty segment, padding rows), packs with no output
row at all (only zero workgroups store), odd and padded head_dims (16- and
32-bit stores), a 3000-segment pack (segment table in the workspace), and
long ratio-128 packs with several windows per backward workgroup.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

import gated_pooling_amd as G
from gated_pooling_amd import inputs

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(G.LIB_PATH), "libcsa_debug.so")
NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def dbg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DEBUG_LIB):
        raise RuntimeError(f"{DEBUG_LIB} is not built (gated_pooling_amd.build builds it with libcsa.so)")
    L = ctypes.CDLL(DEBUG_LIB)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.csa_compressor_bwd.restype = ctypes.c_int
    L.csa_compressor_bwd.argtypes = [P, P, P, P, P, i32, i64, i64, i32, i32, i32, P, P, P, P, i32, P, sz, P]
    L.csa_compressor_bwd_workspace_size.restype = ctypes.c_int
    L.csa_compressor_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i64, i64, P]
    L.csa_debug_ownership_counters.restype = ctypes.c_int
    L.csa_debug_ownership_counters.argtypes = [P, P]
    L.csa_last_error.restype = ctypes.c_char_p
    return L


def _ragged(r, c, d=128):
    return inputs.custom(f"ragged_r{r}_c{c}", inputs.ragged_lengths(r), 32768, r, c, d)


def _many(c):
    rng = np.random.default_rng(41)
    lengths = rng.integers(0, 14, size=3000).tolist()
    return inputs.custom("many", lengths, int(sum(lengths)) + 9, 4, c, 64, seed=3)


CASES = {
    "ragged_r4_c2": lambda: _ragged(4, 2),
    "ragged_r4_c1": lambda: _ragged(4, 1),
    "ragged_r2_c2": lambda: _ragged(2, 2),
    "ragged_r2_c1": lambda: _ragged(2, 1),
    "ragged_r128_c2": lambda: _ragged(128, 2),
    "ragged_r128_c1": lambda: _ragged(128, 1, 64),
    "headline_3x8192_d512_r4_c2": lambda: inputs.WORKLOADS["3x8192_d512_r4_c2"],
    "tiny_r4_c2_d16": lambda: inputs.WORKLOADS["tiny_r4_c2_d16"],
    "no_output_rows_c2": lambda: inputs.custom("none", [1, 3, 0, 2], 40, 4, 2, 32),
    "all_padding_r128": lambda: inputs.custom("pad", [100], 700, 128, 2, 64),
    "odd_d65_r4_c2": lambda: inputs.custom("odd", [37, 0, 130, 5, 64], 250, 4, 2, 65, seed=5),
    "odd_d33_r2_c1": lambda: inputs.custom("odd1", [37, 1, 130, 64], 240, 2, 1, 33, seed=6),
    "padded_d192_r4_c2": lambda: inputs.custom("np2", [300, 3, 501], 900, 4, 2, 192, seed=7),
    "many_segments_c2": lambda: _many(2),
    "many_segments_c1": lambda: _many(1),
    # ratio 128, several windows per workgroup (the backward's copy ring in
    # its steady state) with segment tails and padding rows
    "long_r128_c2": lambda: inputs.custom("l2", [15000, 2049, 40000, 777, 30000], 88400, 128, 2, 64, seed=8),
    "long_r128_c1": lambda: inputs.custom("l1", [33333, 129, 20000, 4095], 57900, 128, 1, 128, seed=9),
}


def _run(L, dev, wl, counts):
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    W, S = c * d, len(cu) - 1
    N = G.csa_compressor_total_comp(cu, r)
    kv, sc, ape, dout = (t.to(dev) for t in inputs.make_tensors(wl, N))
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    dkv = torch.full((T, W), NAN_BF16, dtype=torch.int16, device=dev)
    dsc = torch.full((T, W), NAN_BF16, dtype=torch.int16, device=dev)
    dape = torch.empty(r, W, dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    assert L.csa_compressor_bwd_workspace_size(r, c, d, S, T, N, ctypes.byref(nb)) == 0
    ws = G.workspace(nb.value, dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if counts is not None:
        assert L.csa_debug_ownership_counters(P(counts[0]), P(counts[1])) == 0
    st = L.csa_compressor_bwd(P(kv), P(sc), P(ape), P(cu_d), None, S, T, N, r, c, d, P(dout), P(dkv), P(dsc),
                              P(dape), 1, P(ws), ws.numel(), s)
    torch.cuda.synchronize()
    if counts is not None:
        L.csa_debug_ownership_counters(None, None)
    assert st == 0, L.csa_last_error()
    return dkv.cpu().numpy(), dsc.cpu().numpy(), dape.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_every_gradient_slot_is_stored_exactly_once(dbg, name):
    dev = torch.device("cuda:0")
    wl = CASES[name]()
    T, W = wl.total_tokens, wl.coff * wl.head_dim
    print("ownership", name, "T", T, "W", W, flush=True)
    counts = (torch.zeros(T, W, dtype=torch.int32, device=dev), torch.zeros(T, W, dtype=torch.int32, device=dev))
    dkv, dsc, dape = _run(dbg, dev, wl, counts)
    for tname, cnt in (("dkv", counts[0]), ("dscore", counts[1])):
        bad = cnt != 1
        nbad = int(bad.sum())
        if nbad:
            idx = torch.nonzero(bad)[:5].tolist()
            raise AssertionError(f"{tname}: {nbad} slots stored != 1 times (first {idx}: "
                                 f"{[int(cnt[i][j]) for i, j in idx]})")
    # the counting build computes what the library computes
    ref = _run(G.lib(), dev, wl, None)
    assert np.array_equal(dkv, ref[0]) and np.array_equal(dsc, ref[1])
    assert np.array_equal(dape.view(np.uint32), ref[2].view(np.uint32))

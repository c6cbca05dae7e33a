"""The C ABI on the CPU: the library loads, exports every entry point that
include/csa.h declares, and every rejection path returns its status before
any HIP call (so these tests need no GPU).  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import gated_pooling_amd as G
from gated_pooling_amd import inputs
from tests import brute

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

# Fake device addresses: aligned, non-null, never dereferenced (validation
# rejects every call below before anything is enqueued).
A = ctypes.c_void_p(0x100000)
B = ctypes.c_void_p(0x200000)
NULL = ctypes.c_void_p(0)
MISALIGNED = ctypes.c_void_p(0x100002)


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|csa_status_t|int32_t)\s+(csa_\w+)\s*\(", src, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("csa_compressor_fwd", "csa_compressor_bwd", "csa_compressor_check_support",
                 "csa_compressor_total_comp", "csa_compressor_fwd_workspace_size",
                 "csa_compressor_bwd_workspace_size", "csa_compressor_bwd_grads",
                 "csa_compressor_bwd_dape_reduce", "csa_status_string", "csa_last_error", "csa_version"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(G.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_binding_exposes_same_names():
    for name in declared_functions():
        assert callable(getattr(G, name)), name


def test_status_strings():
    for code, name in ((0, "SUCCESS"), (1, "INVALID_VALUE"), (2, "NOT_SUPPORTED"),
                       (3, "WORKSPACE_TOO_SMALL"), (4, "LAUNCH_FAILED"), (5, "DEVICE_ERROR")):
        assert G.csa_status_string(code) == "CSA_STATUS_" + name
    assert "UNKNOWN" in G.csa_status_string(99)
    assert G.csa_version() >= 100


@pytest.mark.parametrize("name", sorted(inputs.WORKLOADS))
def test_workloads_are_supported(name):
    wl = inputs.WORKLOADS[name]
    N = G.csa_compressor_total_comp(wl.cu_seqlens, wl.ratio)
    assert N == brute.count_outputs(wl.cu_seqlens, wl.ratio) if wl.total_tokens <= 64 else N > 0
    G.csa_compressor_check_support(wl.ratio, wl.coff, wl.head_dim, wl.num_segments, wl.total_tokens, N)


@pytest.mark.parametrize("args,exc", [
    ((3, 2, 16, 2, 64, 15), G.CsaNotSupported),       # ratio 3
    ((8, 2, 16, 2, 64, 8), G.CsaNotSupported),        # ratio 8
    ((128, 2, 96, 2, 512, 1), G.CsaNotSupported),     # ratio 128 needs head_dim % 64 == 0
    ((64, 2, 128, 2, 512, 1), G.CsaNotSupported),     # ratio 64
    ((4, 0, 16, 2, 64, 15), G.CsaNotSupported),       # coff 0
    ((4, 3, 16, 2, 64, 15), G.CsaNotSupported),       # coff 3
    ((2, 0, 16, 2, 64, 15), G.CsaNotSupported),       # coff 0 at ratio 2
    ((2, 3, 16, 2, 64, 15), G.CsaNotSupported),       # coff 3 at ratio 2
    ((4, 2, 0, 2, 64, 15), G.CsaNotSupported),        # head_dim 0
    ((4, 2, -8, 2, 64, 15), G.CsaNotSupported),       # negative head_dim
    ((4, 2, 1025, 2, 64, 15), G.CsaNotSupported),     # beyond 1024
    ((4, 2, 2048, 2, 64, 15), G.CsaNotSupported),     # beyond the launch bound
    ((4, 2, 512, 1, 2 ** 21, 1), G.CsaNotSupported),  # total_tokens*W = 2^31
    ((4, 2, 512, 1, 2 ** 21 - 1, 1), G.CsaNotSupported),  # (total_tokens+1)*W = 2^31
    ((4, 1, 16, 1, 100, 26), G.CsaInvalidValue),      # N*ratio > T
    ((4, 2, 16, 1, 3, 1), G.CsaInvalidValue),         # total_comp > 0, total_tokens < ratio
    ((2, 2, 16, 1, 1, 1), G.CsaInvalidValue),         # same at ratio 2
    ((4, 2, 16, -1, 64, 0), G.CsaInvalidValue),
    ((4, 2, 16, 2, -1, 0), G.CsaInvalidValue),
    ((4, 2, 16, 2, 64, -1), G.CsaInvalidValue),
    ((4, 2, 16, 0, 64, 1), G.CsaInvalidValue),        # rows without segments
])
def test_check_support_rejects(args, exc):
    with pytest.raises(exc) as e:
        G.csa_compressor_check_support(*args)
    assert G.csa_last_error() and str(e.value)


def test_check_support_size_limits_are_independent():
    # total_comp*head_dim = 2^31 exactly is rejected even if the rest is small
    with pytest.raises(G.CsaNotSupported):
        G.csa_compressor_check_support(2, 1, 1024, 1, 2 ** 22, 2 ** 21)
    # just below every limit is accepted
    G.csa_compressor_check_support(4, 2, 512, 1, 2 ** 21 - 2, 2 ** 18)
    G.csa_compressor_check_support(2, 2, 2, 1, 4, 2)
    G.csa_compressor_check_support(4, 1, 1024, 3, 0, 0)


@pytest.mark.parametrize("d", [1, 3, 65, 96, 100, 1000, 1023, 1024])
def test_any_head_dim_up_to_1024_is_supported(d):
    for r in (2, 4):
        for c in (1, 2):
            G.csa_compressor_check_support(r, c, d, 2, 64, 15)
            assert G.csa_compressor_bwd_workspace_size(r, c, d, 2, 64, 15) > 0


def test_total_comp():
    assert G.csa_compressor_total_comp([0, 37, 64], 4) == 15
    assert G.csa_compressor_total_comp([0, 1, 4, 4, 9], 2) == 0 + 1 + 0 + 2
    assert G.csa_compressor_total_comp([0], 4) == 0
    with pytest.raises(G.CsaInvalidValue):
        G.csa_compressor_total_comp([1, 5], 4)
    with pytest.raises(G.CsaInvalidValue):
        G.csa_compressor_total_comp([0, 5, 3], 4)
    L = G.lib()
    out = ctypes.c_int64()
    assert L.csa_compressor_total_comp(NULL, 1, 4, ctypes.byref(out)) == G.CSA_STATUS_INVALID_VALUE


def test_total_comp_random_packs():
    rng = np.random.default_rng(3)
    for _ in range(50):
        cu, _ = brute.random_pack(rng, max_segments=8)
        for r in (2, 4):
            assert G.csa_compressor_total_comp(cu, r) == brute.count_outputs(cu, r)


def test_workspace_sizes():
    wl = inputs.WORKLOADS[inputs.HEADLINE]
    N = G.csa_compressor_total_comp(wl.cu_seqlens, wl.ratio)
    fb = G.csa_compressor_fwd_workspace_size(wl.ratio, wl.coff, wl.head_dim, wl.num_segments, wl.total_tokens, N)
    bb = G.csa_compressor_bwd_workspace_size(wl.ratio, wl.coff, wl.head_dim, wl.num_segments, wl.total_tokens, N)
    assert fb == 0 and bb > 256
    # many segments: the offset table moves to the workspace
    fb_big = G.csa_compressor_fwd_workspace_size(4, 2, 16, 5000, 50000, 1000)
    assert fb_big >= 256 + 4 * 5001
    L = G.lib()
    assert L.csa_compressor_fwd_workspace_size(4, 2, 16, 2, 64, 15, NULL) == G.CSA_STATUS_INVALID_VALUE
    with pytest.raises(G.CsaNotSupported):
        G.csa_compressor_bwd_workspace_size(3, 2, 16, 2, 64, 15)


def _fwd(kv=A, score=A, ape=A, cu=B, S=2, T=64, N=15, r=4, c=2, d=16, out=A, ws=NULL, wsb=0, cu_host=NULL):
    return G.lib().csa_compressor_fwd(kv, score, ape, cu, cu_host, S, T, N, r, c, d, out, ws, wsb, NULL)


def _bwd(kv=A, score=A, ape=A, cu=B, S=2, T=64, N=15, r=4, c=2, d=16, dout=A, dkv=A, dsc=A, dape=A,
         ws=A, wsb=None, cu_host=NULL):
    if wsb is None:
        wsb = G.csa_compressor_bwd_workspace_size(r, c, d, max(S, 0), max(T, 0), max(N, 0)) if min(S, T, N) >= 0 else 0
    return G.lib().csa_compressor_bwd(kv, score, ape, cu, cu_host, S, T, N, r, c, d, dout, dkv, dsc, dape, 1, ws, wsb,
                                      NULL)


def test_fwd_rejections_happen_before_any_launch():
    INV, NS, WS = G.CSA_STATUS_INVALID_VALUE, G.CSA_STATUS_NOT_SUPPORTED, G.CSA_STATUS_WORKSPACE_TOO_SMALL
    assert _fwd(kv=NULL) == INV
    assert _fwd(score=NULL) == INV
    assert _fwd(ape=NULL) == INV
    assert _fwd(out=NULL) == INV
    assert _fwd(cu=NULL) == INV
    assert _fwd(kv=MISALIGNED) == INV
    assert _fwd(out=MISALIGNED) == INV
    assert _fwd(cu=ctypes.c_void_p(0x200002)) == INV
    assert _fwd(r=3) == NS
    assert _fwd(c=3) == NS
    assert _fwd(d=2048) == NS
    assert _fwd(T=3, N=1) == INV
    # a pack with many segments needs a workspace for its offset table
    assert _fwd(S=5000, T=50000, N=1000) == WS
    assert "workspace" in G.csa_last_error()
    # no output rows: nothing to do, succeeds without touching the GPU
    assert _fwd(N=0, kv=NULL, score=NULL, ape=NULL, out=NULL) == 0


def test_bwd_rejections_happen_before_any_launch():
    INV, NS, WS = G.CSA_STATUS_INVALID_VALUE, G.CSA_STATUS_NOT_SUPPORTED, G.CSA_STATUS_WORKSPACE_TOO_SMALL
    assert _bwd(dkv=NULL) == INV
    assert _bwd(dsc=NULL) == INV
    assert _bwd(dape=NULL) == INV
    assert _bwd(dout=NULL) == INV
    assert _bwd(kv=NULL) == INV
    assert _bwd(cu=NULL) == INV
    assert _bwd(cu=NULL, N=0) == INV  # the backward always reads cu
    assert _bwd(ws=NULL) == INV
    assert _bwd(dsc=MISALIGNED) == INV
    assert _bwd(r=5, wsb=1 << 20) == NS
    need = G.csa_compressor_bwd_workspace_size(4, 2, 16, 2, 64, 15)
    assert _bwd(wsb=need - 1) == WS
    L = G.lib()
    assert L.csa_compressor_bwd_grads(A, A, A, B, NULL, 2, 64, 15, 4, 2, 16, A, A, A, A, need - 1, NULL) == WS
    assert L.csa_compressor_bwd_dape_reduce(4, 2, 16, 2, 64, 15, NULL, A, need, NULL) == INV
    assert L.csa_compressor_bwd_dape_reduce(4, 2, 16, 2, 64, 15, A, A, need - 1, NULL) == WS
    assert L.csa_compressor_bwd_dape_reduce(3, 2, 16, 2, 64, 15, A, A, need, NULL) == NS


def test_noalloc_rejections_happen_before_any_device_call():
    """The allocation-free backward validates the problem, its scratch need
    and every caller pointer on the host before it looks up the device."""
    INV, NS, WS = G.CSA_STATUS_INVALID_VALUE, G.CSA_STATUS_NOT_SUPPORTED, G.CSA_STATUS_WORKSPACE_TOO_SMALL
    L = G.lib()

    def call(kv=A, dkv=A, dsc=A, dape=A, dout=A, cu=B, r=4, S=2, T=64, N=15, d=16):
        return L.csa_compressor_bwd_noalloc(kv, kv, kv, cu, NULL, S, T, N, r, 2, d, dout, dkv, dsc, dape, 1, NULL)

    assert call(r=5) == NS
    assert call(dkv=NULL) == INV
    assert call(dape=NULL) == INV
    assert call(dout=MISALIGNED) == INV
    assert call(cu=NULL) == INV
    # ten million segments: the segment table alone exceeds the library's scratch
    assert call(S=10_000_000, T=65536, N=512, r=128, d=64) == WS
    assert "scratch" in G.csa_last_error()


def test_host_cu_is_validated_before_any_launch():
    INV = G.CSA_STATUS_INVALID_VALUE
    bad_total = G.host_cu([0, 37, 60])      # 9 + 5 = 14 rows, not 15
    bad_start = G.host_cu([1, 37, 64])
    bad_order = G.host_cu([0, 40, 37])
    past_end = G.host_cu([0, 37, 68])
    for h in (bad_total, bad_start, bad_order, past_end):
        assert _fwd(cu_host=h) == INV
        assert _bwd(cu_host=h) == INV
    assert "cu_seqlens_host" in G.csa_last_error()


def test_tensor_binding_validates_on_host():
    import torch
    kv = torch.zeros(64, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        G.compressor_fwd(kv, kv, torch.zeros(4, 32), torch.tensor([0, 37, 64], dtype=torch.int32), 4, 2, 15)


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "gated_pooling_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "csa_oracle" not in src and "liboracle" not in src, f


def test_consumed_mask_matches_slot_rules():
    rng = np.random.default_rng(11)
    for _ in range(30):
        cu, T = brute.random_pack(rng)
        r, c, d = int(rng.choice([2, 3, 4])), int(rng.choice([1, 2])), int(rng.choice([1, 2, 4]))
        m = brute.consumed_mask(cu, T, r, c, d)
        for t in range(T):
            for col in range(c * d):
                assert m[t, col] == (brute.consumer(cu, r, c, d, t, col) is not None)

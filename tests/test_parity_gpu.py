"""GPU parity: libcsa (HIP, through the C ABI) against the CPU oracle.

Contract (checked element by element on seeded inputs):
  * ratio 2 and 4: out, dKV, dScore bit-identical to the oracle's fp32
    evaluation order (the stated tolerance is 1 bf16 ulp; both sides evaluate
    the same fixed fp32 order, so the expected difference is none);
  * ratio 128: the kernels sum each window in chains (the forward by half
    windows with their own maxima, merged by rescaling), the oracle in one
    chain, so results are compared within 1 bf16 ulp or the error bound of
    that reordering, with the pages' ratio-128 gate as a floor
    (tests/tolerance.py);
  * never-consumed dKV/dScore slots: exactly 0x0000 although the output
    buffers were filled with NaN before the call;
  * dAPE: |gpu - ref| <= 1e-5 * max(|ref|, max|ref|) with ref the double sum
    of the oracle's fp32 ds values;
  * repeated runs are bit-identical (dAPE included).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_pooling_amd as G
import oracle
from gated_pooling_amd import inputs
from tests import brute
from tests.tolerance import check_reordered

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")


def bf16_nan(shape, device):
    return torch.full(shape, NAN_BF16, dtype=torch.int16, device=device).view(torch.bfloat16)


def run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N, stages=False, host=True):
    """Forward and backward on the GPU with NaN-prefilled outputs; returns
    numpy (out bits, dkv bits, dscore bits, dape f32).  host=True also passes
    the host copy of cu_seqlens (small packs then take the segment table from
    the kernel arguments); host=False makes the kernels build it from the
    device copy."""
    W = c * d
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    cu_h = list(cu) if host else None
    kv_d, sc_d, ape_d, dout_d = kv.to(dev), sc.to(dev), ape.to(dev), dout.to(dev)
    out = bf16_nan((N, d), dev)
    G.compressor_fwd(kv_d, sc_d, ape_d, cu_d, r, c, N, out=out, cu_seqlens_host=cu_h)
    dkv, dsc = bf16_nan((T, W), dev), bf16_nan((T, W), dev)
    dape = torch.full((r, W), float("nan"), dtype=torch.float32, device=dev)
    if stages:
        nbytes = G.csa_compressor_bwd_workspace_size(r, c, d, len(cu) - 1, T, N)
        ws = G.workspace(nbytes, dev)
        P = lambda t: t.data_ptr()  # noqa: E731
        s = torch.cuda.current_stream().cuda_stream
        G.csa_compressor_bwd_grads(P(kv_d), P(sc_d), P(ape_d), P(cu_d), G.host_cu(cu_h), len(cu) - 1, T, N, r, c,
                                   d, P(dout_d), P(dkv), P(dsc), P(ws), ws.numel(), s)
        G.csa_compressor_bwd_dape_reduce(r, c, d, len(cu) - 1, T, N, P(dape), P(ws), ws.numel(), s)
    else:
        G.compressor_bwd(kv_d, sc_d, ape_d, cu_d, r, c, N, dout_d, dkv=dkv, dscore=dsc, dape=dape,
                         cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    return (inputs.bits(out.cpu()), inputs.bits(dkv.cpu()), inputs.bits(dsc.cpu()), dape.cpu().numpy())


def ordered(b):
    b = np.asarray(b).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_bits_equal(got, ref, name):
    diff = got != ref
    n = int(np.count_nonzero(diff))
    if n:
        idx = np.argwhere(diff)[:5].tolist()
        dist = np.abs(ordered(got) - ordered(ref))
        raise AssertionError(f"{name}: {n}/{got.size} elements differ (max ordered distance "
                             f"{int(dist.max())}; first at {idx}: got {got[diff][:5]} ref {ref[diff][:5]})")


def assert_dape(got, ref):
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got.astype(np.float64) - ref)
    tol = 1e-5 * np.maximum(np.abs(ref), scale)
    assert np.all(err <= tol), f"dAPE max err {err.max():.3e}, max rel-to-scale {(err / scale).max():.3e}"


def check_against_oracle(cu, T, r, c, d, kv, sc, ape, dout, got, label=""):
    N = oracle.total_comp(cu, r)
    kvb, scb, apen, doutb = inputs.bits(kv), inputs.bits(sc), ape.numpy(), inputs.bits(dout)
    out_ref = oracle.fwd_f32(kvb, scb, apen, cu, T, r, c, d)
    dkv_ref, dsc_ref, dape_ref, _, _ = oracle.bwd_f32(kvb, scb, apen, cu, T, r, c, d, doutb)
    out, dkv, dsc, dape = got
    assert out.shape == (N, d)
    if r == 128:
        unused = ~brute.consumed_mask(cu, T, r, c, d)
        check_reordered(cu, T, r, c, d, kvb, got, (out_ref, dkv_ref, dsc_ref, dape_ref), unused, label=label)
        return out_ref, dkv_ref, dsc_ref, dape_ref
    assert_bits_equal(out, out_ref, "out")
    assert_bits_equal(dkv, dkv_ref, "dkv")
    assert_bits_equal(dsc, dsc_ref, "dscore")
    assert_dape(dape, dape_ref)
    # zero ownership: every never-consumed slot is +0.0 exactly
    unused = ~brute.consumed_mask(cu, T, r, c, d)
    assert np.all(dkv[unused] == 0) and np.all(dsc[unused] == 0)
    return out_ref, dkv_ref, dsc_ref, dape_ref


# ---------------------------------------------------------------------------
# every workload at its full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("host", [True, False], ids=["args_table", "device_table"])
@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_parity(dev, name, host):
    wl = inputs.WORKLOADS[name]
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    N = G.csa_compressor_total_comp(cu, r)
    assert N == oracle.total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    got = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N, host=host)
    check_against_oracle(cu, T, r, c, d, kv, sc, ape, dout, got, label=f"{name}/{'args' if host else 'device'}")


def test_stage_split_equals_full_backward(dev):
    wl = inputs.WORKLOADS["ragged_d128_r4_c2"]
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    N = G.csa_compressor_total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    a = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N)
    b = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N, stages=True)
    c_ = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N, stages=True, host=False)
    for x, y, z in zip(a, b, c_):
        assert np.array_equal(x, y) and np.array_equal(x, z)


@pytest.mark.parametrize("name", ["3x8192_d512_r4_c2", "ragged_d128_r4_c1", "ragged_d128_r4_c2",
                                  "1x8192_d128_r2_c2", "ragged_d128_r128_c2"])
def test_repeat_runs_bit_identical(dev, name):
    wl = inputs.WORKLOADS[name]
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    N = G.csa_compressor_total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    first = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N)
    for _ in range(10):
        again = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N)
        for x, y in zip(first, again):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


# ---------------------------------------------------------------------------
# never-read inputs cannot leak; degenerate packs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_r4_c2_d16", "ragged_d128_r4_c1", "ragged_d128_r4_c2"])
def test_poisoned_unread_inputs_do_not_leak(dev, name):
    """NaN in every kv/score slot no window reads (tails, short segments,
    last-block first halves, padding) changes nothing."""
    wl = inputs.WORKLOADS[name]
    cu, T, r, c, d = list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim
    N = G.csa_compressor_total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    unused = torch.from_numpy(~brute.consumed_mask(cu, T, r, c, d))
    assert int(unused.sum()) > 0
    kvp, scp = kv.clone(), sc.clone()
    kvp[unused] = float("nan")
    scp[unused] = float("nan")
    got = run_gpu(dev, cu, T, r, c, d, kvp, scp, ape, dout, N)
    check_against_oracle(cu, T, r, c, d, kv, sc, ape, dout, got)


@pytest.mark.parametrize("cu,T,r,c,d", [
    ([0, 1, 4, 6, 9], 16, 4, 2, 16),      # every segment shorter than ratio, padding
    ([0, 1, 2, 3], 3, 4, 1, 128),         # no padding, no blocks
    ([0, 1, 1, 2], 8, 2, 2, 8),           # 1-token segments at ratio 2
    ([0], 32, 4, 2, 16),                  # no segments at all: all padding
    ([0, 0, 0], 0, 4, 2, 16),             # empty pack
])
def test_no_output_rows(dev, cu, T, r, c, d):
    """total_comp == 0: the forward does nothing, the backward still writes
    +0.0 everywhere and dAPE = 0."""
    N = G.csa_compressor_total_comp(cu, r)
    assert N == 0
    wl = inputs.custom("deg", np.diff(cu).tolist(), T, r, c, d)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    out, dkv, dsc, dape = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N)
    assert out.shape == (0, d)
    assert np.all(dkv == 0) and np.all(dsc == 0)
    assert np.all(dape.view(np.uint32) == 0)


def test_many_segments_use_workspace_table(dev):
    """More segments than fit the per-workgroup LDS table (the offset scan
    then runs as its own kernel): 5000 short segments of 0..13 tokens."""
    rng = np.random.default_rng(21)
    lengths = rng.integers(0, 14, size=5000).tolist()
    T = int(sum(lengths)) + 37
    for c in (1, 2):
        wl = inputs.custom("many", lengths, T, 4, c, 16, seed=5)
        cu = list(wl.cu_seqlens)
        N = G.csa_compressor_total_comp(cu, 4)
        assert G.csa_compressor_fwd_workspace_size(4, c, 16, 5000, T, N) > 0
        kv, sc, ape, dout = inputs.make_tensors(wl, N)
        got = run_gpu(dev, cu, T, 4, c, 16, kv, sc, ape, dout, N)
        check_against_oracle(cu, T, 4, c, 16, kv, sc, ape, dout, got)


def _random_cases(n=24, seed=77):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        S = int(rng.integers(1, 9))
        lengths = rng.integers(0, 300, size=S).tolist()
        T = int(sum(lengths)) + int(rng.integers(0, 20))
        r = int(rng.choice([2, 4]))
        c = int(rng.choice([1, 2]))
        d = int(rng.choice([2, 4, 8, 16, 32, 64, 256, 1024]))
        if T == 0:
            T = 1
        cases.append((lengths, T, r, c, d, 100 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases())
def test_random_small_packs(dev, case):
    """Ragged packs over head_dim 2..1024 (every lane layout: fewer columns
    than a lane holds, chunks per row below and above a wave and a
    workgroup)."""
    lengths, T, r, c, d, seed = case
    wl = inputs.custom("rand", lengths, T, r, c, d, seed=seed)
    cu = list(wl.cu_seqlens)
    N = G.csa_compressor_total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    got = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N)
    check_against_oracle(cu, T, r, c, d, kv, sc, ape, dout, got)


# head_dims outside the power-of-two lane layout: odd (one column per lane,
# 16-bit accesses) and even with a chunk count that is not a power of two
# (rows padded to a power of two in lanes); below and above one wave of
# chunks (per-lane and wave-uniform paths)
ODD_DIMS = [1, 3, 7, 33, 65, 127, 129, 255, 1023]
EVEN_NONPOW2_DIMS = [6, 12, 96, 100, 192, 258, 320, 1000]


def _nonpow2_cases():
    rng = np.random.default_rng(2024)
    cases = []
    for i, d in enumerate(ODD_DIMS + EVEN_NONPOW2_DIMS):
        nseg = int(rng.integers(1, 6))
        lengths = rng.integers(0, 90, size=nseg).tolist()
        lengths[int(rng.integers(0, nseg))] = int(rng.integers(1, 4))  # a segment shorter than ratio
        T = int(sum(lengths)) + int(rng.integers(1, 12))           # with padding rows
        r = int(rng.choice([2, 4]))
        c = int(rng.choice([1, 2]))
        cases.append((lengths, T, r, c, d, 500 + i))
    # every (ratio, coff) at one odd and one padded head_dim
    for j, (r, c) in enumerate([(2, 1), (2, 2), (4, 1), (4, 2)]):
        for d in (65, 192):
            cases.append(([37, 0, 130, 5, 64], 250, r, c, d, 700 + 10 * j + d))
    return cases


@pytest.mark.parametrize("case", _nonpow2_cases(), ids=lambda c: f"d{c[4]}_r{c[2]}_c{c[3]}_s{c[5]}")
def test_non_power_of_two_head_dims(dev, case):
    lengths, T, r, c, d, seed = case
    wl = inputs.custom("np2", lengths, T, r, c, d, seed=seed)
    cu = list(wl.cu_seqlens)
    N = G.csa_compressor_total_comp(cu, r)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    for host in (True, False):
        got = run_gpu(dev, cu, T, r, c, d, kv, sc, ape, dout, N, host=host)
        check_against_oracle(cu, T, r, c, d, kv, sc, ape, dout, got)


def _r128_cases():
    rng = np.random.default_rng(128)
    cases = []
    for i in range(10):
        nseg = int(rng.integers(1, 6))
        lengths = rng.integers(0, 700, size=nseg).tolist()
        lengths[int(rng.integers(0, nseg))] = int(rng.integers(1, 128))  # shorter than ratio
        T = int(sum(lengths)) + int(rng.integers(1, 300))                # padding rows
        c = int(rng.choice([1, 2]))
        d = int(rng.choice([64, 128, 192, 512]))
        cases.append((lengths, T, c, d, 900 + i, bool(i % 2)))
    lengths = rng.integers(0, 400, size=60).tolist()                     # 60 segments: LDS table
    cases.append((lengths, int(sum(lengths)) + 7, 2, 64, 950, False))
    lengths = rng.integers(0, 260, size=2300).tolist()                   # workspace table
    cases.append((lengths, int(sum(lengths)) + 7, 1, 64, 951, False))
    cases.append(([300, 260, 7], 600, 2, 1024, 952, True))              # largest head_dim: 16 slices
    cases.append(([129, 400], 560, 1, 960, 953, False))                 # 15 slices
    # long segments with tails: several windows per workgroup of the
    # one-workgroup-per-CU backward (the copy ring's steady state), segment
    # ends and their zero tails at every position of the ring
    for i, (c, d) in enumerate([(2, 64), (1, 64), (2, 128), (1, 320), (2, 512), (2, 192)]):
        nseg = int(rng.integers(3, 40))
        lengths = rng.integers(1000, 9000, size=nseg).tolist()
        T = int(sum(lengths)) + int(rng.integers(1, 500))
        cases.append((lengths, T, c, d, 960 + i, bool(i % 2)))
    # the largest segment table kept in LDS (2048 segments) at coff 2: the
    # backward's two window buffers plus the table use nearly all of a CU's
    # 160 KiB of LDS
    lengths = np.random.default_rng(2048).integers(0, 300, size=2048).tolist()
    cases.append((lengths, int(sum(lengths)) + 5, 2, 64, 970, False))
    # segment lengths at and next to multiples of 128 (no tail, a 1-row tail,
    # one row short of a block)
    lengths = [128, 256, 384, 127, 129, 0, 1, 512, 255]
    cases.append((lengths, int(sum(lengths)) + 3, 2, 128, 971, True))
    cases.append((lengths, int(sum(lengths)), 1, 64, 972, False))
    return cases


@pytest.mark.parametrize("case", _r128_cases(), ids=lambda c: f"S{len(c[0])}_c{c[2]}_d{c[3]}_s{c[4]}")
def test_ratio128_packs(dev, case):
    """ratio 128: windows of 128 * coff rows staged through LDS, summed in
    chains (the forward by half windows with their own maxima), compared
    within the reordering tolerance; multi-block
    segments, tails, segments shorter than 128, padding, kernel-argument /
    LDS / workspace segment tables."""
    lengths, T, c, d, seed, host = case
    wl = inputs.custom("r128", lengths, T, 128, c, d, seed=seed)
    cu = list(wl.cu_seqlens)
    N = G.csa_compressor_total_comp(cu, 128)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    got = run_gpu(dev, cu, T, 128, c, d, kv, sc, ape, dout, N, host=host)
    check_against_oracle(cu, T, 128, c, d, kv, sc, ape, dout, got, label=f"r128pack_s{seed}")


def test_extreme_scores_and_subnormals(dev):
    """Score spreads that push EXP to its clamp and products into fp32
    subnormals: still bit-identical (IEEE subnormals on both sides)."""
    wl = inputs.custom("extreme", [64, 40, 7], 128, 4, 2, 64, seed=9)
    cu = list(wl.cu_seqlens)
    N = G.csa_compressor_total_comp(cu, 4)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    g = torch.Generator().manual_seed(4)
    sc = (sc.float() * torch.where(torch.rand(sc.shape, generator=g) < 0.3, 60.0, 1.0)).to(torch.bfloat16)
    dout = (dout.float() * 1e-36).to(torch.bfloat16)
    got = run_gpu(dev, cu, 128, 4, 2, 64, kv, sc, ape, dout, N)
    check_against_oracle(cu, 128, 4, 2, 64, kv, sc, ape, dout, got)


@pytest.mark.parametrize("c", [2, 1])
def test_ratio128_half_windows_far_apart(dev, c):
    """ratio 128: one half of every window about 100 below the other (the
    forward's rescale factor EXP(m_h - M) then underflows to a subnormal or
    to zero) and wide score spreads; compared within the tolerance."""
    d = 64
    lengths = [384, 256, 200, 128, 700]
    wl = inputs.custom("r128far", lengths, sum(lengths) + 9, 128, c, d, seed=13)
    cu = list(wl.cu_seqlens)
    T = wl.total_tokens
    N = G.csa_compressor_total_comp(cu, 128)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    f = sc.float()
    if c == 2:
        f[:, :d] -= 100.0                       # every window's previous-block half
    else:
        pos = torch.zeros(T, dtype=torch.long)
        for s0, s1 in zip(cu[:-1], cu[1:]):
            pos[s0:s1] = torch.arange(s1 - s0) % 128
        f[pos < 64] -= 100.0                    # every window's first 64 rows
    g = torch.Generator().manual_seed(5)
    f = f * torch.where(torch.rand(f.shape, generator=g) < 0.3, 4.0, 1.0)
    sc = f.to(torch.bfloat16)
    for host in (True, False):
        got = run_gpu(dev, cu, T, 128, c, d, kv, sc, ape, dout, N, host=host)
        check_against_oracle(cu, T, 128, c, d, kv, sc, ape, dout, got, label=f"r128far_c{c}")


def test_invalid_device_cu_seqlens_touches_nothing(dev):
    """cu_seqlens that contradicts total_comp (caller error, only detectable
    on the device): the kernels leave every output as it was."""
    cu_true = [0, 37, 64]
    N = 15
    wl = inputs.custom("bad", [37, 27], 64, 4, 2, 16)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    bad = torch.tensor([0, 37, 60], dtype=torch.int32, device=dev)  # implies 9 + 5 = 14 blocks
    out = bf16_nan((N, 16), dev)
    G.compressor_fwd(kv.to(dev), sc.to(dev), ape.to(dev), bad, 4, 2, N, out=out)  # no host copy: device check
    dkv, dsc = bf16_nan((64, 32), dev), bf16_nan((64, 32), dev)
    dape = torch.full((4, 32), float("nan"), device=dev)
    G.compressor_bwd(kv.to(dev), sc.to(dev), ape.to(dev), bad, 4, 2, N, dout.to(dev), dkv=dkv, dscore=dsc, dape=dape)
    torch.cuda.synchronize()
    assert np.all(inputs.bits(out.cpu()) == NAN_BF16)
    assert np.all(inputs.bits(dkv.cpu()) == NAN_BF16)
    assert torch.isnan(dape.cpu()).all()
    del cu_true

"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, not against the oracle's own formulas.

Each test names what it pins and the mistake it would catch.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gated_pooling_amd import inputs
from tests import brute

F32 = np.float32


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def f32_nearest(q: Fraction) -> float:
    """Correctly rounded (nearest-even) fp32 value of an exact rational."""
    x = float(q)  # correctly rounded to double
    c = float(np.float32(x))
    cands = {c, float(np.nextafter(F32(c), F32(np.inf))), float(np.nextafter(F32(c), F32(-np.inf)))}

    def key(v):
        mant = np.array([v], np.float32).view(np.uint32)[0]
        return (abs(Fraction(v) - q), int(mant) & 1)

    return min(cands, key=key)


def ln2_fraction() -> Fraction:
    getcontext().prec = 80
    return Fraction(str(Decimal(2).ln()))


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def bits_to_f64(b):
    return oracle.f64_from_bits(b)


def make_inputs(rng, T, W, r, N, d, spread=1.0):
    kv = torch.from_numpy(rng.standard_normal((T, W)).astype(np.float32)).to(torch.bfloat16)
    sc = torch.from_numpy((spread * rng.standard_normal((T, W))).astype(np.float32)).to(torch.bfloat16)
    ape = (0.02 * rng.standard_normal((r, W))).astype(np.float32)
    dout = torch.from_numpy(rng.standard_normal((N, d)).astype(np.float32)).to(torch.bfloat16)
    return inputs.bits(kv), inputs.bits(sc), ape, inputs.bits(dout)


def random_cases(n_cases=24, seed=1234):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        cu, T = brute.random_pack(rng)
        r = int(rng.choice([1, 2, 3, 4, 8]))
        c = int(rng.choice([1, 2]))
        d = int(rng.choice([1, 2, 3, 8, 16]))
        cases.append((cu, T, r, c, d, 1000 + i))
    # the tiny workload itself, at its own shape
    wl = inputs.WORKLOADS["tiny_r4_c2_d16"]
    cases.append((list(wl.cu_seqlens), wl.total_tokens, wl.ratio, wl.coff, wl.head_dim, 7))
    # ratio 128: windows of 128 or 256 entries (segments with several
    # blocks, a tail, one shorter than ratio, padding)
    cases.append(([0, 300, 320, 680], 700, 128, 2, 3, 51))
    cases.append(([0, 300, 320, 680], 690, 128, 1, 2, 52))
    cases.append(([0, 0, 513], 520, 128, 2, 1, 53))
    return cases


CASES = random_cases()


# --------------------------------------------------------------------------
# EXP and constants
# --------------------------------------------------------------------------

def test_exp_constants_are_their_exact_definitions():
    """L2E, LN2_HI, LN2_LO and the Taylor coefficients are the fp32 numbers
    nearest to log2(e), ln 2, ln 2 - LN2_HI and 1/n!.  Catches a mistyped
    hex digit or a wrong factorial."""
    c = oracle.exp_constants().astype(np.float64)
    ln2 = ln2_fraction()
    assert c[0] == f32_nearest(1 / ln2)
    assert c[1] == f32_nearest(ln2)
    assert c[2] == f32_nearest(ln2 - Fraction(c[1]))
    assert c[3] == -104.0
    for n in range(8):
        assert c[4 + n] == f32_nearest(Fraction(1, math.factorial(n))), n


def _ulp_error(y32: np.ndarray):
    got = oracle.exp_f32_array(y32).astype(np.float64)
    ref = np.exp(y32.astype(np.float64))
    # fp32 spacing at the reference value, subnormal spacing below 2^-126
    spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(ref, 2.0 ** -149))) - 23), 2.0 ** -149)
    return np.abs(got - ref) / spacing


def test_exp_accuracy_over_domain():
    """EXP is within 1 fp32 ulp of e^y on a dense sweep of every fp32 in
    [-104, 0] (every 13th bit pattern, plus the neighbourhoods of each
    rint(y*log2 e) switch point); an exhaustive sweep of every fp32 there
    measured 0.937 ulp at most.  Catches a wrong sign in the reduction, a
    dropped Taylor term (degree 6 alone reaches 2.7 ulp) or a wrong ldexp."""
    lo = np.array([-104.0], np.float32).view(np.uint32)[0]
    # negative floats: bit patterns from 0x80000000 (-0) up to lo
    pats = np.arange(0x80000000, int(lo) + 1, 13, dtype=np.uint64).astype(np.uint32)
    y = pats.view(np.float32)
    err = _ulp_error(y)
    assert err.max() <= 1.0, (float(err.max()), float(y[err.argmax()]))
    # switch points of k = rint(y * log2 e): y ~ (k + 1/2) ln 2
    ks = np.arange(-150, 1)
    centres = ((ks + 0.5) * math.log(2)).astype(np.float32)
    near = []
    for c0 in centres:
        v = c0
        for _ in range(64):
            near.append(v)
            v = np.nextafter(v, np.float32(0))
        v = c0
        for _ in range(64):
            near.append(v)
            v = np.nextafter(v, np.float32(-np.inf))
    near = np.array(near, np.float32)
    near = near[(near <= 0) & (near >= -104)]
    err2 = _ulp_error(near)
    assert err2.max() <= 1.0


def test_exp_special_values():
    """EXP(0) = 1 exactly (so a one-element window has p = 1 exactly);
    EXP(-ln2 * m) = 2^-m for small m; EXP saturates at its value for -104
    below that (~1e-45, under half the smallest subnormal's double)."""
    assert oracle.exp_f32(0.0) == 1.0
    assert oracle.exp_f32(-0.0) == 1.0
    assert oracle.exp_f32(-1e30) == oracle.exp_f32(-104.0)
    assert oracle.exp_f32(-104.0) <= 2.0 ** -149
    assert abs(oracle.exp_f32(-1.0) - math.exp(-1.0)) <= 2 * 2.0 ** -24


def test_bf16_rounding_is_nearest_even():
    """The oracle's fp32->bf16 rounding equals torch's (an independent
    library implementation of round-to-nearest-even) on random bit patterns,
    every tie case and the subnormal range.  Catches truncation or
    ties-away."""
    rng = np.random.default_rng(5)
    pats = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, size=2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    sub = rng.integers(0, 0x00800000, size=2000, dtype=np.uint64).astype(np.uint32)
    allp = np.concatenate([pats, ties, sub, sub | 0x80000000])
    f = allp.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    ref = inputs.bits(torch.from_numpy(f.copy()).to(torch.bfloat16))
    got = np.array([oracle.bf16_from_f32(x) for x in f], np.uint16)
    assert np.array_equal(got, ref)
    # hand cases: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert oracle.bf16_from_f32(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_from_f32(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> even (up)
    assert oracle.f32_from_bf16(0x3F80) == 1.0


# --------------------------------------------------------------------------
# pack bookkeeping
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", CASES[:12])
def test_output_count_matches_block_count(case):
    """N = sum floor(L/r), counted block by block."""
    cu, T, r, c, d, _ = case
    assert oracle.total_comp(cu, r) == brute.count_outputs(cu, r)


def test_tiny_workload_row_count():
    """cu = [0, 37, 64], r = 4: 9 + 6 = 15 output rows (both segments have
    tails: 37 % 4 = 1 and 27 % 4 = 3)."""
    assert oracle.total_comp([0, 37, 64], 4) == 15


# --------------------------------------------------------------------------
# brute force in double, independent window membership
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", CASES)
def test_f64_oracle_matches_slot_side_brute_force(case):
    """The double oracle (window listed block by block) equals a brute-force
    double evaluation whose windows are recovered slot by slot.  Catches a
    wrong row, half, position, masking or output-row order in the oracle."""
    cu, T, r, c, d, seed = case
    rng = np.random.default_rng(seed)
    N = brute.count_outputs(cu, r)
    kv, sc, ape, dout = make_inputs(rng, T, c * d, r, N, d)
    kv64, sc64, ape64, dout64 = bits_to_f64(kv), bits_to_f64(sc), ape.astype(np.float64), bits_to_f64(dout)
    out_o = oracle.fwd_f64(kv64, sc64, ape64, cu, T, r, c, d)
    dkv_o, dsc_o, dape_o = oracle.bwd_f64(kv64, sc64, ape64, cu, T, r, c, d, dout64)
    out_b, dkv_b, dsc_b, dape_b = brute.brute_fwd_bwd_f64(kv64, sc64, ape64, dout64, cu, T, r, c, d)
    np.testing.assert_allclose(out_o, out_b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dkv_o, dkv_b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dsc_o, dsc_b, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dape_o, dape_b, rtol=1e-10, atol=1e-13)


def _torch_reference_f64(kv64, sc64, ape64, dout64, cu, T, r, c, d):
    """Library-routine transcription: gather the slot-side windows into a
    padded [N*d, K] tensor, mask absent entries with -inf, torch.softmax,
    weighted sum; gradients by torch autograd."""
    W = c * d
    N = brute.count_outputs(cu, r)
    win, _ = brute.windows(cu, T, r, c, d)
    K = max((len(m) for m in win.values()), default=1)
    idx = np.zeros((N * d, K), np.int64)
    pidx = np.zeros((N * d, K), np.int64)
    mask = np.zeros((N * d, K), bool)
    for (n, j), members in win.items():
        for k, (t, col, pos) in enumerate(members):
            idx[n * d + j, k] = t * W + col
            pidx[n * d + j, k] = pos * W + col
            mask[n * d + j, k] = True
    kv_t = torch.tensor(kv64, dtype=torch.float64, requires_grad=True)
    sc_t = torch.tensor(sc64, dtype=torch.float64, requires_grad=True)
    ape_t = torch.tensor(ape64, dtype=torch.float64, requires_grad=True)
    ii, pp, mm = torch.from_numpy(idx), torch.from_numpy(pidx), torch.from_numpy(mask)
    x = sc_t.reshape(-1)[ii] + ape_t.reshape(-1)[pp]
    x = x.masked_fill(~mm, float("-inf"))
    p = torch.softmax(x, dim=1)
    v = kv_t.reshape(-1)[ii].masked_fill(~mm, 0.0)
    out = (p * v).sum(dim=1).reshape(N, d)
    out.backward(torch.tensor(dout64, dtype=torch.float64))
    return out.detach().numpy(), kv_t.grad.numpy(), sc_t.grad.numpy(), ape_t.grad.numpy()


@pytest.mark.parametrize("case", CASES[::2])
def test_f64_oracle_matches_torch_autograd(case):
    """The double oracle's gradients equal PyTorch double autograd through
    torch.softmax on the same windows.  Catches a wrong softmax Jacobian
    (e.g. a missing - o term or a sign error) in the oracle's backward."""
    cu, T, r, c, d, seed = case
    rng = np.random.default_rng(seed + 50)
    N = brute.count_outputs(cu, r)
    if N == 0:
        pytest.skip("no output rows")
    kv, sc, ape, dout = make_inputs(rng, T, c * d, r, N, d)
    kv64, sc64, ape64, dout64 = bits_to_f64(kv), bits_to_f64(sc), ape.astype(np.float64), bits_to_f64(dout)
    out_t, dkv_t, dsc_t, dape_t = _torch_reference_f64(kv64, sc64, ape64, dout64, cu, T, r, c, d)
    out_o = oracle.fwd_f64(kv64, sc64, ape64, cu, T, r, c, d)
    dkv_o, dsc_o, dape_o = oracle.bwd_f64(kv64, sc64, ape64, cu, T, r, c, d, dout64)
    np.testing.assert_allclose(out_o, out_t, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dkv_o, dkv_t, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dsc_o, dsc_t, rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(dape_o, dape_t, rtol=1e-9, atol=1e-13)


@pytest.mark.parametrize("case", [CASES[i] for i in (0, 3, 7, len(CASES) - 1)])
def test_f64_backward_matches_finite_differences(case):
    """Central differences of L = sum(dOut * out) with respect to kv, score
    and ape match the double oracle's gradients.  Pins the backward against
    the forward with no formula in common."""
    cu, T, r, c, d, seed = case
    rng = np.random.default_rng(seed + 99)
    N = brute.count_outputs(cu, r)
    if N == 0:
        pytest.skip("no output rows")
    W = c * d
    kv, sc, ape, dout = make_inputs(rng, T, W, r, N, d)
    kv64, sc64, ape64, w = bits_to_f64(kv), bits_to_f64(sc), ape.astype(np.float64), bits_to_f64(dout)
    dkv, dsc, dape = oracle.bwd_f64(kv64, sc64, ape64, cu, T, r, c, d, w)

    def L(kv_, sc_, ape_):
        return float(np.sum(w * oracle.fwd_f64(kv_, sc_, ape_, cu, T, r, c, d)))

    h = 1e-5
    for name, arr, grad in (("kv", kv64, dkv), ("score", sc64, dsc), ("ape", ape64, dape)):
        flat = list(range(arr.size))
        pick = rng.choice(flat, size=min(25, arr.size), replace=False)
        for f in pick:
            i = np.unravel_index(f, arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[i] += h
            am[i] -= h
            args_p = {"kv": (ap, sc64, ape64), "score": (kv64, ap, ape64), "ape": (kv64, sc64, ap)}[name]
            args_m = {"kv": (am, sc64, ape64), "score": (kv64, am, ape64), "ape": (kv64, sc64, am)}[name]
            fd = (L(*args_p) - L(*args_m)) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(grad[i])), (name, i, fd, grad[i])


# --------------------------------------------------------------------------
# closed-form special cases of the fp32 oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", CASES)
def test_one_hot_window_reproduces_kv_bitwise(case):
    """In every (output row, column) one window entry gets score 60 (exact in
    bf16).  In fp32 its weight is exactly 1 and the rest are below 2^-80, so
    out == kv at that slot bit for bit, dKV there == dOut bit for bit and
    dScore there == 0.  The hot slot is chosen from the slot-side windows, so
    this pins every index of the fp32 oracle."""
    cu, T, r, c, d, seed = case
    rng = np.random.default_rng(seed + 7)
    N = brute.count_outputs(cu, r)
    if N == 0:
        pytest.skip("no output rows")
    W = c * d
    kv, sc, ape, dout = make_inputs(rng, T, W, r, N, d)
    kv_f = bits_to_f64(kv)
    # keep kv away from zero so the hot value dominates the tiny others
    kv = np.where(np.abs(kv_f) < 1e-3, np.uint16(0x3F80), kv)
    win, _ = brute.windows(cu, T, r, c, d)
    hot = {}
    sc = sc.copy()
    for (n, j), members in win.items():
        t, col, _ = members[int(rng.integers(len(members)))]
        sc[t, col] = 0x4270  # 60.0
        hot[(n, j)] = (t, col)
    out = oracle.fwd_f32(kv, sc, ape, cu, T, r, c, d)
    dkv, dsc, _, _, _ = oracle.bwd_f32(kv, sc, ape, cu, T, r, c, d, dout)
    for (n, j), (t, col) in hot.items():
        assert out[n, j] == kv[t, col], (n, j, t, col)
        assert dkv[t, col] == dout[n, j], (n, j, t, col)
        assert dsc[t, col] in (0x0000, 0x8000)


@pytest.mark.parametrize("case", CASES)
def test_uniform_scores_give_the_window_mean(case):
    """score = 0 and ape = 0: every weight is 1/K exactly (K = window size,
    a power of two for r in {1, 2, 4, 8}), so out is the mean of the window's
    kv values rounded to bf16.  Pins the normalisation and the first-block
    masking (K = r there, 2r elsewhere at coff = 2)."""
    cu, T, r, c, d, seed = case
    if r not in (1, 2, 4, 8, 128):
        pytest.skip("1/K exact only for powers of two")
    rng = np.random.default_rng(seed + 11)
    N = brute.count_outputs(cu, r)
    if N == 0:
        pytest.skip("no output rows")
    W = c * d
    kv, _, _, _ = make_inputs(rng, T, W, r, N, d)
    sc = np.zeros((T, W), np.uint16)
    ape = np.zeros((r, W), np.float32)
    out = bits_to_f64(oracle.fwd_f32(kv, sc, ape, cu, T, r, c, d))
    kv_f = bits_to_f64(kv)
    win, _ = brute.windows(cu, T, r, c, d)
    for (n, j), members in win.items():
        mean = sum(kv_f[t, col] for t, col, _ in members) / len(members)
        # plus the fp32 error of the K-term sum (at most K u of sum|v| / K)
        sum_err = len(members) * 2.0 ** -24 * sum(abs(kv_f[t, col]) for t, col, _ in members) / len(members)
        assert abs(out[n, j] - mean) <= 0.5 * bf16_ulp(mean) + sum_err + 1e-300, (n, j, out[n, j], mean)


# --------------------------------------------------------------------------
# zero ownership and invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", CASES)
def test_zero_set_is_the_never_consumed_set(case):
    """dKV/dScore are exactly +0.0 (0x0000) on every slot no window reads --
    the seqlen % r tails, segments shorter than r, the first half of each
    segment's last block at coff = 2 and rows past cu[S] -- and dKV is
    nonzero on every consumed slot whose dOut is nonzero."""
    cu, T, r, c, d, seed = case
    rng = np.random.default_rng(seed + 13)
    N = brute.count_outputs(cu, r)
    W = c * d
    kv, sc, ape, dout = make_inputs(rng, T, W, r, N, d)
    dkv, dsc, dape, _, _ = oracle.bwd_f32(kv, sc, ape, cu, T, r, c, d, dout)
    win, unused = brute.windows(cu, T, r, c, d)
    for t, col in unused:
        assert dkv[t, col] == 0 and dsc[t, col] == 0, (t, col)
    for (n, j), members in win.items():
        if dout[n, j] & 0x7FFF:
            for t, col, _ in members:
                assert dkv[t, col] & 0x7FFF, (t, col)
    if N == 0:
        assert not dape.any()


@pytest.mark.parametrize("case", CASES)
def test_backward_invariants(case):
    """Per window and column the ds_k sum to 0 (softmax Jacobian rows sum to
    zero), hence sum_i dAPE[i, j] (+ sum_i dAPE[i, d + j] at coff = 2) = 0;
    and dKV sums to dOut per window (weights sum to 1)."""
    cu, T, r, c, d, seed = case
    rng = np.random.default_rng(seed + 17)
    N = brute.count_outputs(cu, r)
    if N == 0:
        pytest.skip("no output rows")
    W = c * d
    kv, sc, ape, dout = make_inputs(rng, T, W, r, N, d)
    kv64, sc64, ape64, g = bits_to_f64(kv), bits_to_f64(sc), ape.astype(np.float64), bits_to_f64(dout)
    dkv, dsc, dape = oracle.bwd_f64(kv64, sc64, ape64, cu, T, r, c, d, g)
    win, _ = brute.windows(cu, T, r, c, d)
    for (n, j), members in win.items():
        s = sum(dsc[t, col] for t, col, _ in members)
        # rounding in (v - o) scales with |a| (|v| + |o|), not with |ds|
        vmax = max(abs(kv64[t, col]) for t, col, _ in members)
        a = sum(abs(dkv[t, col]) * (abs(kv64[t, col]) + vmax) for t, col, _ in members)
        assert abs(s) <= 1e-12 * a + 1e-300
        sk = sum(dkv[t, col] for t, col, _ in members)
        assert abs(sk - g[n, j]) <= 1e-12 * max(1.0, abs(g[n, j]))
    tot = dape[:, :d].sum(axis=0) + (dape[:, d:].sum(axis=0) if c == 2 else 0)
    assert np.all(np.abs(tot) <= 1e-10 * max(1.0, np.abs(dape).max()))


# --------------------------------------------------------------------------
# fp32 oracle against the double definition
# --------------------------------------------------------------------------

def _ordered(b):
    """bf16 bit patterns -> integers ordered like the values (+0 = -0 = 0)."""
    b = np.asarray(b).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _bf16_neighbours_ok(got_bits, ref64):
    """got is one of the two bf16 numbers bracketing ref (within 1 ulp)."""
    got = bits_to_f64(got_bits)
    return np.abs(got - ref64) <= bf16_ulp(ref64) + 0.0


@pytest.mark.parametrize("case", CASES)
def test_f32_oracle_within_bf16_rounding_of_f64(case):
    """out, dKV within one bf16 ulp of the double result; dScore within one
    ulp or within the fp32 error bound |a| * dO, where dO bounds the fp32
    error of o (cancellation in kv - o); dAPE within 1e-5 of max|dAPE|.
    Catches an fp32-only mistake (e.g. a wrong EXP or a dropped R)."""
    cu, T, r, c, d, seed = case
    rng = np.random.default_rng(seed + 19)
    N = brute.count_outputs(cu, r)
    W = c * d
    kv, sc, ape, dout = make_inputs(rng, T, W, r, N, d, spread=2.0)
    kv64, sc64, ape64, g = bits_to_f64(kv), bits_to_f64(sc), ape.astype(np.float64), bits_to_f64(dout)
    out32 = oracle.fwd_f32(kv, sc, ape, cu, T, r, c, d)
    dkv32, dsc32, dape32, _, _ = oracle.bwd_f32(kv, sc, ape, cu, T, r, c, d, dout)
    out64 = oracle.fwd_f64(kv64, sc64, ape64, cu, T, r, c, d)
    dkv64, dsc64, dape64 = oracle.bwd_f64(kv64, sc64, ape64, cu, T, r, c, d, g)
    assert np.all(_bf16_neighbours_ok(out32, out64))
    assert np.all(_bf16_neighbours_ok(dkv32, dkv64))
    # dScore: error model.  |o32 - o| <= (8 + K) u sum|p v| (u = 2^-24: EXP
    # error, R and the products, plus the K-term chains of additions), so
    # |ds32 - ds| <= |a| * that + 8u|ds|.
    u = 2.0 ** -24
    win, _ = brute.windows(cu, T, r, c, d)
    bound = np.zeros_like(dsc64)
    for (n, j), members in win.items():
        K = len(members)
        chain = K
        spv = sum(abs(dkv64[t, col] / g[n, j] * kv64[t, col]) if g[n, j] else 0 for t, col, _ in members)
        for t, col, _ in members:
            bound[t, col] = abs(dkv64[t, col]) * (8 + max(16, chain)) * u * spv + 8 * u * abs(dsc64[t, col])
    got = bits_to_f64(dsc32)
    ok = np.abs(got - dsc64) <= bf16_ulp(dsc64) + bound
    assert np.all(ok)
    scale = max(np.abs(dape64).max(), 1e-30)
    assert np.all(np.abs(dape32 - dape64) <= 1e-5 * np.maximum(np.abs(dape64), scale))


def test_f32_oracle_deterministic():
    """Two runs (OpenMP threads on) give identical bits and dAPE."""
    wl = inputs.WORKLOADS["ragged_d128_r4_c2"]
    N = oracle.total_comp(wl.cu_seqlens, wl.ratio)
    kv, sc, ape, dout = inputs.make_tensors(wl, N)
    args = (inputs.bits(kv), inputs.bits(sc), ape.numpy(), wl.cu_seqlens, wl.total_tokens,
            wl.ratio, wl.coff, wl.head_dim)
    a = oracle.bwd_f32(*args, inputs.bits(dout))
    b = oracle.bwd_f32(*args, inputs.bits(dout))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_oracle_rejects_bad_packs():
    """Decreasing cu, cu[0] != 0, cu[S] > T_cap and a wrong N are refused."""
    z = np.zeros((8, 4), np.uint16)
    ape = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.fwd_f32(z, z, ape, [0, 5, 3], 8, 2, 2, 2)
    with pytest.raises(ValueError):
        oracle.fwd_f32(z, z, ape, [1, 5], 8, 2, 2, 2)
    with pytest.raises(ValueError):
        oracle.fwd_f32(z, z, ape, [0, 9], 8, 2, 2, 2)

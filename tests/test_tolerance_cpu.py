"""Pins for the ratio-128 tolerance checker (tests/tolerance.py), on the CPU.

A numpy model of the ratio-128 kernels' evaluation order must pass the
checker against the oracle's single-chain results: the forward takes each
half window (coff 2: the previous block's rows, then the own rows; coff 1:
the first and the last 64 rows) with its own maximum, sums 16-entry chains
added in chain order, and merges the halves by rescaling with EXP of the
difference of their maxima; the backward takes the window maximum and sums
8 * coff-entry chains added in chain order.  A planted 2-ulp error in any
output, a lost zero and a wrong dAPE must fail the checker.  The model is
test-side only (it uses the oracle's exponential, so that only the order of
evaluation differs).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import brute
from tests.tolerance import check_reordered

def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _f(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def _fma32(a, b, c):
    # a*b is exact in double for fp32 operands; one rounding of the sum
    return np.float32(np.float64(a) * np.float64(b) + np.float64(c))


def _chains(e, v, L):
    """Z and acc of chains of L consecutive entries, the chain sums added in
    chain order."""
    Z = acc = None
    for c0 in range(0, len(e), L):
        zc, ac = e[c0], np.float32(0)
        for k in range(c0 + 1, min(c0 + L, len(e))):
            zc = np.float32(zc + e[k])
        for k in range(c0, min(c0 + L, len(e))):
            ac = _fma32(e[k], v[k], ac)
        Z, acc = (zc, ac) if Z is None else (np.float32(Z + zc), np.float32(acc + ac))
    return Z, acc


def _exp(y):
    return oracle.exp_f32_array(np.asarray([y], np.float32))[0]


def kernel_order_model(kv, sc, ape, dout, cu, T, r, c, d):
    W = c * d
    N = brute.count_outputs(cu, r)
    out = np.zeros((N, d), np.uint16)
    dkv = np.zeros((T, W), np.uint16)
    dsc = np.zeros((T, W), np.uint16)
    dape = np.zeros((r, W), np.float64)
    win, _ = brute.windows(cu, T, r, c, d)
    for (n, j), members in win.items():
        # window order: previous half (first-half columns) then own half
        members = sorted(members, key=lambda m: (m[1] >= d if c == 2 else 0, m[0]))
        x = np.array([np.float32(_f(sc[t, col])) + np.float32(ape[pos, col]) for t, col, pos in members],
                     np.float32)
        v = np.array([_f(kv[t, col]) for t, col, _ in members], np.float32)
        # forward: half windows with their own maxima, merged by rescaling
        if c == 2:
            cut = sum(1 for _, col, _ in members if col < d)   # the previous block's rows (0 or 128)
        else:
            cut = len(members) // 2
        parts = []
        for lo, hi in ((0, cut), (cut, len(members))):
            if hi > lo:
                mh = x[lo:hi].max()
                eh = oracle.exp_f32_array((x[lo:hi] - mh).astype(np.float32))
                parts.append((mh,) + _chains(eh, v[lo:hi], 16))
        if len(parts) == 1:
            _, Zf, Af = parts[0]
        else:
            (m0, Z0, A0), (m1, Z1, A1) = parts
            M = max(m0, m1)
            s0, s1 = _exp(np.float32(m0 - M)), _exp(np.float32(m1 - M))
            Zf = np.float32(np.float32(Z0 * s0) + np.float32(Z1 * s1))
            Af = np.float32(np.float32(A0 * s0) + np.float32(A1 * s1))
        out[n, j] = _bf16(np.float32(Af * (np.float32(1) / Zf)))
        # backward: the window maximum, 8 * coff-entry chains
        m = x.max()
        e = oracle.exp_f32_array((x - m).astype(np.float32))
        Z, acc = _chains(e, v, 8 * c)
        R = np.float32(1) / Z
        o = np.float32(acc * R)
        G = np.float32(R * _f(dout[n, j]))
        for k, (t, col, pos) in enumerate(members):
            a = np.float32(e[k] * G)
            ds = np.float32(a * np.float32(v[k] - o))
            dkv[t, col] = _bf16(a)
            dsc[t, col] = _bf16(ds)
            dape[pos, col] += float(ds)
    return out, dkv, dsc, dape


PACKS = [
    ([0, 300, 320, 680], 700, 2, 3, 31),
    ([0, 513], 520, 1, 4, 32),
    ([0, 0, 400, 527], 530, 2, 2, 33),
]


@pytest.fixture(scope="module", params=PACKS, ids=lambda p: f"c{p[2]}_d{p[3]}")
def case(request):
    cu, T, c, d, seed = request.param
    r = 128
    rng = np.random.default_rng(seed)
    W = c * d
    N = brute.count_outputs(cu, r)
    kv = _bf16(rng.standard_normal((T, W)))
    sc = _bf16(rng.standard_normal((T, W)))
    ape = (0.02 * rng.standard_normal((r, W))).astype(np.float32)
    dout = _bf16(rng.standard_normal((N, d)))
    ref_out = oracle.fwd_f32(kv, sc, ape, cu, T, r, c, d)
    dkv, dsc, dape, _, _ = oracle.bwd_f32(kv, sc, ape, cu, T, r, c, d, dout)
    got = kernel_order_model(kv, sc, ape, dout, cu, T, r, c, d)
    unused = ~brute.consumed_mask(cu, T, r, c, d)
    return cu, T, r, c, d, kv, got, (ref_out, dkv, dsc, dape), unused


def test_kernel_order_passes(case):
    cu, T, r, c, d, kv, got, ref, unused = case
    st = check_reordered(cu, T, r, c, d, kv, got, ref, unused)
    assert st["out_size"] > 0


@pytest.mark.parametrize("which", [0, 1, 2])
def test_two_ulp_error_fails(case, which):
    cu, T, r, c, d, kv, got, ref, unused = case
    got = [g.copy() for g in got]
    t = got[which]
    idx = np.argwhere((t != 0) & ~(unused if which else np.zeros(t.shape, bool)))[0]
    t[tuple(idx)] = t[tuple(idx)] + 2 if t[tuple(idx)] & 0x7FFF < 0x7F00 else t[tuple(idx)] - 2
    with pytest.raises(AssertionError):
        check_reordered(cu, T, r, c, d, kv, tuple(got), ref, unused)


def test_lost_zero_fails(case):
    cu, T, r, c, d, kv, got, ref, unused = case
    got = [g.copy() for g in got]
    got[1][np.argwhere(unused)[0][0], np.argwhere(unused)[0][1]] = 0x3F80
    with pytest.raises(AssertionError):
        check_reordered(cu, T, r, c, d, kv, tuple(got), ref, unused)


def test_wrong_dape_fails(case):
    cu, T, r, c, d, kv, got, ref, unused = case
    got = list(got)
    got[3] = got[3] * (1 + 1e-4)
    with pytest.raises(AssertionError):
        check_reordered(cu, T, r, c, d, kv, tuple(got), ref, unused)


def test_reordering_is_visible_and_within_tolerance():
    """On a larger pack the kernels' order does change some bf16 results (so
    the checks above are not vacuous), all within the contract."""
    cu, T, c, d, r = [0, 1300, 2000, 4000], 4100, 2, 64, 128
    rng = np.random.default_rng(5)
    W = c * d
    N = brute.count_outputs(cu, r)
    kv = _bf16(rng.standard_normal((T, W)))
    sc = _bf16(rng.standard_normal((T, W)))
    ape = (0.02 * rng.standard_normal((r, W))).astype(np.float32)
    dout = _bf16(rng.standard_normal((N, d)))
    ref = (oracle.fwd_f32(kv, sc, ape, cu, T, r, c, d),) + oracle.bwd_f32(kv, sc, ape, cu, T, r, c, d, dout)[:3]
    got = kernel_order_model(kv, sc, ape, dout, cu, T, r, c, d)
    st = check_reordered(cu, T, r, c, d, kv, got, ref, ~brute.consumed_mask(cu, T, r, c, d))
    assert st["dkv_differ"] + st["dscore_differ"] > 0

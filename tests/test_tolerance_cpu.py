"""Pins for the ratio-128 tolerance checker (tests/tolerance.py), on the CPU.

A numpy model of a reordered evaluation -- every window's Z and acc summed in
64-entry chunks whose sums are then added in chunk order, the order of the
ratio-128 kernels -- must pass the checker against the oracle's single-chain
results; a planted 2-ulp error in any output, a lost zero and a wrong dAPE
must fail it.  The model is test-side only (it uses the oracle's exponential
so that only the summation order differs).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import brute
from tests.tolerance import check_reordered

CHUNK = 64


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _f(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def _fma32(a, b, c):
    # a*b is exact in double for fp32 operands; one rounding of the sum
    return np.float32(np.float64(a) * np.float64(b) + np.float64(c))


def chunked_model(kv, sc, ape, dout, cu, T, r, c, d):
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
        m = x.max()
        e = oracle.exp_f32_array((x - m).astype(np.float32))
        Z = acc = np.float32(0)
        for c0 in range(0, len(e), CHUNK):
            zc, ac = e[c0], np.float32(0)
            for k in range(c0 + 1, min(c0 + CHUNK, len(e))):
                zc = np.float32(zc + e[k])
            for k in range(c0, min(c0 + CHUNK, len(e))):
                ac = _fma32(e[k], v[k], ac)
            Z, acc = (zc, ac) if c0 == 0 else (np.float32(Z + zc), np.float32(acc + ac))
        R = np.float32(1) / Z
        o = np.float32(acc * R)
        out[n, j] = _bf16(o)
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
    got = chunked_model(kv, sc, ape, dout, cu, T, r, c, d)
    unused = ~brute.consumed_mask(cu, T, r, c, d)
    return cu, T, r, c, d, kv, got, (ref_out, dkv, dsc, dape), unused


def test_chunked_order_passes(case):
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
    """On a larger pack the chunked order does change some bf16 results
    (so the checks above are not vacuous), all within the contract."""
    cu, T, c, d, r = [0, 1300, 2000, 4000], 4100, 2, 64, 128
    rng = np.random.default_rng(5)
    W = c * d
    N = brute.count_outputs(cu, r)
    kv = _bf16(rng.standard_normal((T, W)))
    sc = _bf16(rng.standard_normal((T, W)))
    ape = (0.02 * rng.standard_normal((r, W))).astype(np.float32)
    dout = _bf16(rng.standard_normal((N, d)))
    ref = (oracle.fwd_f32(kv, sc, ape, cu, T, r, c, d),) + oracle.bwd_f32(kv, sc, ape, cu, T, r, c, d, dout)[:3]
    got = chunked_model(kv, sc, ape, dout, cu, T, r, c, d)
    st = check_reordered(cu, T, r, c, d, kv, got, ref, ~brute.consumed_mask(cu, T, r, c, d))
    assert st["dkv_differ"] + st["dscore_differ"] > 0

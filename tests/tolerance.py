"""Tolerance comparison of GPU results with the fp32 oracle where the two
evaluate a window in different orders (ratio 128).

The oracle sums every window in one chain in window order after taking the
window maximum.  The ratio-128 backward takes the same maximum and EXP
arguments and sums chains of 8 * coff consecutive entries, then adds the chain
sums [PR5984: ratio=128 commit: per-chunk partials merged in one fixed
order].  The ratio-128 forward takes each half window with its own maximum
m_h, sums 16-entry chains of e = EXP(x - m_h), and merges the halves by
rescaling with EXP(m_h - M) (M the larger maximum), as the pages' forward
merges per-chunk partials that carry their own maxima.  With u = 2^-24 and a
window of K entries, the standard error bound of a K-term fp32 sum, which
holds for any summation order (each term passes through at most K - 1
roundings), gives, between the two fp32 evaluations of Z = sum e and
acc = sum e v:

  |dZ| / Z          <= 2 (K - 1) u
  |d acc|           <= 2 K u sum|e v|
  |d o|             <= (4 K + 2) u sum|p v|          <= (4K + 2) u max|v|
  |d a| / |a|       <= (2 K + 6) u                   (a = e R g)
  |d ds|            <= (2 K + 10) u |ds| + (4 K + 2) u |a| max|v|
                                                       (ds = a (v - o))

The forward's weights also differ from the oracle's: entry i of half h
weighs EXP(x_i - m_h) EXP(m_h - M) instead of EXP(x_i - M).  EXP is within
1 fp32 ulp (2u relative) on [-104, 0] and the rounded differences x_i - m_h,
m_h - M and x_i - M carry relative errors of at most u (M - x_i) in all, so
each weight moves by at most (8 + 2 (M - x_i)) u, counting the rescale's
product and sum; since sum p_i (M - x_i) <= ln K (the softmax entropy is at
most ln K and Z >= 1), out moves by at most a further (16 + 4 ln K) u max|v|.
Each bf16 result moves by at most the fp32 difference plus one bf16 rounding
step.  The contract checked here:

  * out, dKV, dScore: |gpu - ref| <= 1 bf16 ulp, or within the bound above
    (doubled); elements beyond 1 ulp are counted and returned;
  * dKV and dScore on never-consumed slots: exactly 0x0000;
  * the pages' ratio-128 gate as a floor [PR5984: ratio=128 commit]: per
    tensor at most max(1, 0.1 %) of the elements differ at all and the
    largest difference is at most 1.6e-2;
  * dAPE: |gpu - ref| <= 1e-5 * max(|ref|, max|ref|).
"""
from __future__ import annotations

import json
import os

import numpy as np

U = 2.0 ** -24


def bf16_value(bits):
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(x):
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def ordered(b):
    b = np.asarray(b).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def window_stats(cu, T, r, c, d, kv_bits):
    """Per output row and column: the window length K and max|v| over the
    window; per kv slot: the same numbers of the window that consumes it
    (K = 0 for never-consumed slots).  Windows follow the pages' layout:
    block b of a segment takes its own rows in columns [(c-1)d, cd) and, at
    coff 2 and b >= 1, the previous block's rows in columns [0, d)."""
    W = c * d
    v = np.abs(bf16_value(kv_bits)).astype(np.float32)
    out_K, out_m = [], []
    slot_K = np.zeros((T, W), np.int32)
    slot_m = np.zeros((T, W), np.float32)
    for s in range(len(cu) - 1):
        nb = (cu[s + 1] - cu[s]) // r
        if nb == 0:
            continue
        rows = slice(cu[s], cu[s] + nb * r)
        blk = v[rows].reshape(nb, r, W)
        own = blk[:, :, (c - 1) * d:c * d].max(axis=1)          # [nb, d]
        K = np.full((nb, 1), r, np.int32)
        m = own
        if c == 2:
            first = blk[:, :, :d].max(axis=1)
            m = own.copy()
            m[1:] = np.maximum(m[1:], first[:-1])
            K = np.full((nb, 1), 2 * r, np.int32)
            K[0] = r
        out_K.append(np.broadcast_to(K, (nb, d)))
        out_m.append(m)
        # own half of block b -> window b; first half of block b -> window b + 1
        sk = slot_K[rows].reshape(nb, r, W)
        sm = slot_m[rows].reshape(nb, r, W)
        sk[:, :, (c - 1) * d:c * d] = K[:, None, :]
        sm[:, :, (c - 1) * d:c * d] = m[:, None, :]
        if c == 2 and nb > 1:
            sk[:-1, :, :d] = K[1:, None, :]
            sm[:-1, :, :d] = m[1:, None, :]
    if out_K:
        return np.concatenate(out_K), np.concatenate(out_m), slot_K, slot_m
    return np.zeros((0, d), np.int32), np.zeros((0, d), np.float32), slot_K, slot_m


def _gate(name, got, ref, stats):
    diff = np.abs(bf16_value(got) - bf16_value(ref))
    n_diff = int(np.count_nonzero(got != ref))
    limit = max(1, int(0.001 * got.size))
    stats[name + "_differ"] = n_diff
    stats[name + "_size"] = int(got.size)
    stats[name + "_max_abs"] = float(diff.max()) if diff.size else 0.0
    assert n_diff <= limit, f"{name}: {n_diff} of {got.size} elements differ (gate {limit})"
    assert stats[name + "_max_abs"] <= 1.6e-2, f"{name}: max |diff| {stats[name + '_max_abs']}"


def check_reordered(cu, T, r, c, d, kv_bits, got, ref, unused, label=""):
    """got, ref: (out bits, dkv bits, dscore bits, dape).  Returns the
    statistics dict (also appended as a JSON line to $CSA_TOL_REPORT)."""
    out, dkv, dsc, dape = got
    out_r, dkv_r, dsc_r, dape_r = ref
    K_o, m_o, K_s, m_s = window_stats(cu, T, r, c, d, kv_bits)
    stats = {"label": label, "ratio": r, "coff": c, "head_dim": d, "total_tokens": T}

    # never-consumed slots: exact +0.0
    assert np.all(dkv[unused] == 0) and np.all(dsc[unused] == 0), "zero-owned slot not +0.0"

    # out
    g, f = bf16_value(out), bf16_value(out_r)
    dist = np.abs(ordered(out) - ordered(out_r))
    bound = 2 * ((4 * K_o + 2) + 16 + 4 * np.log(np.maximum(K_o, 1))) * U * m_o
    ok = (dist <= 1) | (np.abs(g - f) <= bf16_ulp(np.maximum(np.abs(g), np.abs(f))) + bound)
    assert np.all(ok), f"out: {int((~ok).sum())} elements beyond 1 ulp and the error bound"
    stats["out_beyond_1ulp"] = int(np.count_nonzero(dist > 1))
    _gate("out", out, out_r, stats)

    # dKV: within one bf16 ulp
    cons = ~unused
    dist = np.abs(ordered(dkv) - ordered(dkv_r))
    assert np.all(dist[cons] <= 1), f"dkv: {int((dist[cons] > 1).sum())} elements beyond 1 ulp"
    stats["dkv_beyond_1ulp"] = 0
    _gate("dkv", dkv, dkv_r, stats)

    # dScore: 1 ulp or the error model
    g, f = bf16_value(dsc), bf16_value(dsc_r)
    a = np.abs(bf16_value(dkv_r)) * (1 + 2.0 ** -8)
    bound = 2 * ((2 * K_s + 10) * U * np.abs(f) + (4 * K_s + 2) * U * a * m_s)
    dist = np.abs(ordered(dsc) - ordered(dsc_r))
    ok = (dist <= 1) | (np.abs(g - f) <= bf16_ulp(np.maximum(np.abs(g), np.abs(f))) + bound)
    assert np.all(ok), f"dscore: {int((~ok).sum())} elements beyond 1 ulp and the error bound"
    stats["dscore_beyond_1ulp"] = int(np.count_nonzero(dist > 1))
    _gate("dscore", dsc, dsc_r, stats)

    # dAPE
    scale = max(float(np.abs(dape_r).max()), 1e-30)
    err = np.abs(dape.astype(np.float64) - dape_r)
    assert np.all(err <= 1e-5 * np.maximum(np.abs(dape_r), scale)), f"dAPE max err {err.max():.3e}"
    stats["dape_max_err_rel_to_max"] = float(err.max() / scale)

    path = os.environ.get("CSA_TOL_REPORT")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(stats) + "\n")
    return stats

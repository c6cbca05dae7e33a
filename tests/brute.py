"""Independent brute-force description of the Compressor, for pinning the oracle.

The oracle lists each window in order ("which slots feed block b").  This
module answers the opposite question, from the slot's side, with no offset
scan: for a slot (t, col) of kv/score, which output (row n, column j) consumes
it and at which APE position -- or nobody.  Windows are then recovered by
scanning every slot.  Plain Python; only for tiny packs.

Rules (Megatron-LM PR 5984 page: fused forward+backward commit for the
overlapping window, coff commit for coff=1, zero-init folding commit for the
never-consumed classes):
  * token t belongs to the segment s with cu[s] <= t < cu[s+1]; rows at or past
    cu[S] belong to no segment (static-capacity padding);
  * inside the segment, t is at local offset u = t - cu[s], in block u // r at
    position u % r; blocks past floor(L_s / r) - 1 are the seqlen % r tail;
  * with coff = 1 the slot (t, col) feeds block (s, u // r), column col;
  * with coff = 2 a second-half column (col >= d) feeds block (s, u // r) at
    column col - d; a first-half column feeds the NEXT block (s, u // r + 1) at
    column col, if that block exists;
  * the output row of block (s, b) is the number of blocks in segments before
    s plus b.
"""
from __future__ import annotations

import numpy as np


def segment_of(cu, t):
    for s in range(len(cu) - 1):
        if cu[s] <= t < cu[s + 1]:
            return s
    return None


def blocks_in(cu, s, r):
    return (cu[s + 1] - cu[s]) // r


def output_row(cu, s, b, r):
    return sum(blocks_in(cu, q, r) for q in range(s)) + b


def consumer(cu, r, coff, d, t, col):
    """(n, j, pos) of the window that reads slot (t, col), or None."""
    s = segment_of(cu, t)
    if s is None:
        return None
    u = t - cu[s]
    blk, pos = divmod(u, r)
    nb = blocks_in(cu, s, r)
    if blk >= nb:
        return None  # seqlen % r tail, or a segment shorter than r
    if coff == 1:
        return output_row(cu, s, blk, r), col, pos
    if col >= d:
        return output_row(cu, s, blk, r), col - d, pos
    if blk + 1 < nb:
        return output_row(cu, s, blk + 1, r), col, pos
    return None  # first half of the segment's last block


def windows(cu, T, r, coff, d):
    """dict (n, j) -> list of (t, col, pos) in the order the slots are met
    (row-major), plus the list of never-consumed slots."""
    W = coff * d
    win, unused = {}, []
    for t in range(T):
        for col in range(W):
            c = consumer(cu, r, coff, d, t, col)
            if c is None:
                unused.append((t, col))
            else:
                n, j, pos = c
                win.setdefault((n, j), []).append((t, col, pos))
    return win, unused


def count_outputs(cu, r):
    """Number of output rows, counted block by block."""
    n = 0
    for s in range(len(cu) - 1):
        u = 0
        while u + r <= cu[s + 1] - cu[s]:
            n += 1
            u += r
    return n


def brute_fwd_bwd_f64(kv, score, ape, dout, cu, T, r, coff, d):
    """Plain double evaluation from the slot-side windows.  kv, score: float64
    [T, W]; ape float64 [r, W]; dout float64 [N, d].  Returns out [N, d],
    dkv, dscore [T, W], dape [r, W]."""
    W = coff * d
    N = count_outputs(cu, r)
    win, _ = windows(cu, T, r, coff, d)
    out = np.zeros((N, d))
    dkv = np.zeros((T, W))
    dscore = np.zeros((T, W))
    dape = np.zeros((r, W))
    for (n, j), members in win.items():
        x = np.array([score[t, c] + ape[p, c] for t, c, p in members])
        v = np.array([kv[t, c] for t, c, _ in members])
        e = np.exp(x - x.max())
        p = e / e.sum()
        o = float(np.dot(p, v))
        out[n, j] = o
        g = dout[n, j]
        for (t, c, pos), pk, vk in zip(members, p, v):
            dkv[t, c] = pk * g
            dscore[t, c] = pk * g * (vk - o)
            dape[pos, c] += pk * g * (vk - o)
    return out, dkv, dscore, dape


def random_pack(rng, max_segments=5, max_len=40, max_pad=7):
    S = int(rng.integers(1, max_segments + 1))
    lengths = [int(rng.integers(0, max_len + 1)) for _ in range(S)]
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    T = cu[-1] + int(rng.integers(0, max_pad + 1))
    return cu, T


def consumed_mask(cu, T, r, coff, d):
    """Vectorised slot-side membership: bool [T, coff*d], True where some
    window reads the slot (same rules as `consumer`)."""
    cu = np.asarray(cu, np.int64)
    S = len(cu) - 1
    W = coff * d
    t = np.arange(T, dtype=np.int64)
    s = np.searchsorted(cu, t, side="right") - 1
    inside = (s >= 0) & (s < S) & (t < cu[-1])
    s = np.clip(s, 0, max(S - 1, 0))
    u = t - cu[s] if S else np.zeros_like(t)
    blk = u // r
    nb = (cu[s + 1] - cu[s]) // r if S else np.zeros_like(t)
    in_block = inside & (blk < nb)
    mask = np.zeros((T, W), bool)
    if coff == 1:
        mask[in_block, :] = True
    else:
        mask[in_block, d:] = True
        mask[in_block & (blk + 1 < nb), :d] = True
    return mask

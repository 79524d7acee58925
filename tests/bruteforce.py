"""Unpaged brute-force attention and an independent paging helper (tests only).

Written separately from the oracle: plain Python loops over contiguous
per-request K/V lists that never existed as pages.  Used to pin the oracle on
tiny inputs.
"""

from __future__ import annotations

import math

import numpy as np


def brute_attention(q_rows, K, V, scale, group, window=0):
    """Textbook causal softmax attention for one request.

    q_rows: [n, Hq, D]; K, V: [L, Hkv, D] (contiguous, logical order).
    Row j is the token at position L - n + j and sees keys 0 .. L - n + j
    (with window > 0 only the last `window` of them).
    Returns a nested list [n][Hq][D] of Python floats.
    """
    if len(q_rows) == 0:
        return []
    n, Hq, D = len(q_rows), len(q_rows[0]), len(q_rows[0][0])
    L = len(K)
    out = []
    for j in range(n):
        pos = L - n + j
        keys = [t for t in range(pos + 1) if window <= 0 or pos - t < window]
        row = []
        for h in range(Hq):
            g = h // group
            scores = []
            for t in keys:
                acc = 0.0
                for d in range(D):
                    acc += float(q_rows[j][h][d]) * float(K[t][g][d])
                scores.append(scale * acc)
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            o = []
            for d in range(D):
                acc = 0.0
                for i, t in enumerate(keys):
                    acc += ws[i] * float(V[t][g][d])
                o.append(acc / tot)
            row.append(o)
        out.append(row)
    return out


def page_requests(K_list, V_list, rng, block_size=16, extra_blocks=3, fill=np.nan):
    """Scatter contiguous per-request K/V into a shuffled pool.

    Returns (k_pool, v_pool, block_tables) with pools [NB, Hkv, bs, D]
    of the inputs' dtype and tables padded with an unused block id.  Written independently of the
    oracle's gather.
    """
    Hkv, D = K_list[0].shape[1], K_list[0].shape[2]
    nblk = [-(-len(K) // block_size) for K in K_list]
    NB = sum(nblk) + extra_blocks
    ids = list(rng.permutation(NB))
    dt = K_list[0].dtype
    k_pool = np.full((NB, Hkv, block_size, D), fill, dt)
    v_pool = np.full((NB, Hkv, block_size, D), fill, dt)
    width = max(nblk)
    pad = ids[-1]
    tables = np.full((len(K_list), width), pad, np.int32)
    for b, (K, V) in enumerate(zip(K_list, V_list)):
        mine = [ids.pop(0) for _ in range(nblk[b])]
        tables[b, :nblk[b]] = mine
        for t in range(len(K)):
            blk = mine[t // block_size]
            for h in range(Hkv):
                k_pool[blk, h, t % block_size, :] = K[t, h]
                v_pool[blk, h, t % block_size, :] = V[t, h]
    return k_pool, v_pool, tables

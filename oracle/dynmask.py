"""Content-aware block mask, float64 oracle (test infrastructure only).

The pages do not define a content-based pattern for the Sparse Attention
layers.  The model card's own slug (``full_xattn``, page 1 address) hints at
dynamic block selection, and the "Daily Papers" page (hugingapi.com, search
"Head-Centric Sparse Attention") describes the standard ingredients: block
importance estimated by coarse-grained attention between mean-pooled blocks
(Prism abstract), and an adaptive Top-tau selection of blocks (RRAttention
abstract).  This module is the plainest reading that uses exactly those two
steps, written out one definition at a time:

1. Mean pooling.  For blocks of ``B`` tokens (the last one may be shorter),
   ``qbar[i, h] = mean_{t in block i} q[t, h]`` and likewise ``kbar[j, g]``.
2. Coarse attention.  ``z[h, i, j] = scale * qbar[i, h] . kbar[j, g(h)]`` for
   the causal block pairs ``j <= i`` (query head h reads KV head
   ``g(h) = h // (Hq / Hkv)``), a softmax over ``j`` for every ``(h, i)``, and
   the mean over the query heads: ``P[i, j]`` (one mask per layer, shared by
   all heads, like the static mask).
3. Top-tau.  Row ``i`` always keeps its ``s`` sink blocks and its diagonal
   block.  The other causal blocks are taken in order of decreasing ``P``
   (ties: smaller ``j`` first) while the mass taken so far is below ``tau``
   and the row holds fewer than ``max_blocks`` blocks (0 = no cap).

By linearity, ``qbar[i] . kbar[j]`` is the mean of the token-level products
``q[t] . k[u]`` over the block pair, which the tests check by brute force.
Selection is integer work decided by floating point: the tests compare the
GPU's decision with this one where the margin is clear, and check the
defining properties where it is not.
"""

import numpy as np


def pool_blocks(x, block_size):
    """Mean over each block of ``block_size`` rows: ``x [S, H, d]`` ->
    ``[nb, H, d]`` float64; a partial last block is averaged over its rows."""
    x = np.asarray(x, dtype=np.float64)
    S = x.shape[0]
    nb = (S + block_size - 1) // block_size
    out = np.zeros((nb,) + x.shape[1:], dtype=np.float64)
    for i in range(nb):
        rows = x[i * block_size:min(S, (i + 1) * block_size)]
        out[i] = rows.sum(axis=0) / rows.shape[0]
    return out


def coarse_logits(q, k, block_size, scale=None):
    """``z [Hq, nb, nb]``: scaled dot products of pooled query and key blocks,
    ``-inf`` above the block diagonal (causal)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qb = pool_blocks(q, block_size)
    kb = pool_blocks(k, block_size)
    nb = qb.shape[0]
    group = hq // hkv
    z = np.full((hq, nb, nb), -np.inf)
    for h in range(hq):
        g = h // group
        for i in range(nb):
            for j in range(i + 1):
                z[h, i, j] = scale * float(np.dot(qb[i, h], kb[j, g]))
    return z


def block_probs(q, k, block_size, scale=None):
    """``P [nb, nb]``: per-head softmax of the coarse logits over the causal
    key blocks of each query block, averaged over the query heads."""
    z = coarse_logits(q, k, block_size, scale)
    hq, nb = z.shape[0], z.shape[1]
    P = np.zeros((nb, nb))
    for h in range(hq):
        for i in range(nb):
            row = z[h, i, :i + 1]
            e = np.exp(row - row.max())
            P[i, :i + 1] += e / e.sum()
    return P / hq


def block_probs_rows(q, k, block_size, rows, scale=None):
    """Rows ``rows`` of ``P`` by the same definition with numpy matrix
    products over the pooled blocks (for long sequences; pinned against
    ``block_probs``).  Returns ``[len(rows), nb]``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qb = pool_blocks(q, block_size)  # [nb, hq, d]
    kb = pool_blocks(k, block_size)  # [nb, hkv, d]
    nb = qb.shape[0]
    group = hq // hkv
    out = np.zeros((len(rows), nb))
    for n, i in enumerate(rows):
        for h in range(hq):
            z = scale * (kb[:i + 1, h // group, :] @ qb[i, h])
            e = np.exp(z - z.max())
            out[n, :i + 1] += e / e.sum()
    return out / hq


def select_row(p, i, tau, sink_blocks, max_blocks=0):
    """Blocks kept in row ``i`` given that row's probabilities ``p`` (length
    > i), by the Top-tau rule (module docstring, step 3): a sorted list."""
    mandatory = [j for j in range(i + 1) if j < sink_blocks or j == i]
    keep = list(mandatory)
    mass = sum(p[j] for j in mandatory)
    others = [j for j in range(i + 1) if j not in mandatory]
    others.sort(key=lambda j: (-p[j], j))
    for j in others:
        if mass >= tau or (max_blocks > 0 and len(keep) >= max_blocks):
            break
        keep.append(j)
        mass += p[j]
    return sorted(keep)


def select_blocks(P, tau, sink_blocks, max_blocks=0):
    """Dense uint8 mask ``[nb, nb]``: ``select_row`` for every row of ``P``."""
    P = np.asarray(P, dtype=np.float64)
    nb = P.shape[0]
    m = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        m[i, select_row(P[i], i, tau, sink_blocks, max_blocks)] = 1
    return m


def dynamic_block_mask(q, k, block_size, tau, sink_blocks, max_blocks=0, scale=None):
    """Content-aware mask of one sequence: ``(dense uint8 [nb, nb], P)``."""
    P = block_probs(q, k, block_size, scale)
    return select_blocks(P, tau, sink_blocks, max_blocks), P

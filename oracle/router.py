"""Layer Router, float64 oracle (test infrastructure only).

Source: Flux Attention technical summary (gist.science), section 2
"Methodology": a light router, added to a frozen model, pools the first and
the last 100 prompt tokens, feeds the pooled context to an MLP context
encoder, and decides per layer between Full Attention (FA) and Sparse
Attention (SA).  At inference the soft routing weight is thresholded to a
deterministic 0/1 (same section, "switch to hard routing").

Readings where the pages leave a step open:
* pooling operator = arithmetic mean over the SET of pooled positions (a row
  that is both among the first and the last 100 counts once);
* MLP = Linear(D->H1) -> ReLU -> Linear(H1->L), weights in PyTorch
  ``[out][in]`` layout, one output logit per layer;
* threshold 0.5 on sigmoid(z) is the same decision as z >= 0; an exact tie
  z == 0 routes to FA (1).
"""

import numpy as np

N_POOL = 100  # tokens pooled from each end of the prompt (section 2, Layer Router)


def pool_positions(seqlen):
    """Sorted distinct positions pooled for a prompt of ``seqlen`` tokens:
    the first min(100, S) and the last min(100, S), as a set."""
    seqlen = int(seqlen)
    if seqlen <= 0:
        raise ValueError("empty prompt has nothing to pool")
    first = set(range(0, min(N_POOL, seqlen)))
    last = set(range(max(0, seqlen - N_POOL), seqlen))
    return np.array(sorted(first | last), dtype=np.int64)


def pool_mean(hidden):
    """Mean of the pooled rows of one prompt's hidden states ``[S][D]``."""
    h = np.asarray(hidden, dtype=np.float64)
    pos = pool_positions(h.shape[0])
    total = np.zeros(h.shape[1], dtype=np.float64)
    for p in pos:  # plain sum, then divide: the definition of a mean
        total += h[p]
    return total / len(pos)


def router_mlp(pooled, w1, b1, w2, b2):
    """Two-layer MLP with ReLU: z = W2 relu(W1 x + b1) + b2 (float64)."""
    x = np.asarray(pooled, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    hid = w1 @ x + np.asarray(b1, dtype=np.float64)
    hid = np.maximum(hid, 0.0)
    return w2 @ hid + np.asarray(b2, dtype=np.float64)


def threshold_route(z):
    """Hard route per layer: 1 (FA) where sigmoid(z) >= 0.5, i.e. z >= 0,
    else 0 (SA).  Returns uint8."""
    z = np.asarray(z, dtype=np.float64)
    return (z >= 0.0).astype(np.uint8)


def route_requests(hidden, cu_seqlens, w1, b1, w2, b2):
    """Route every request of a packed batch.

    hidden: ``[T][D]`` rows of all prompts packed back to back;
    cu_seqlens: ``[n_req+1]`` prefix offsets into the rows.
    Returns ``(route uint8 [n_req][L], z float64 [n_req][L])``.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    routes, logits = [], []
    for r in range(len(cu) - 1):
        pooled = pool_mean(hidden[cu[r]:cu[r + 1]])
        z = router_mlp(pooled, w1, b1, w2, b2)
        logits.append(z)
        routes.append(threshold_route(z))
    return np.stack(routes), np.stack(logits)

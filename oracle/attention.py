"""Masked softmax attention, float64 oracle (test infrastructure only).

Full Attention (FA) is causal softmax attention; Sparse Attention (SA) is the
same formula restricted to the active blocks of the block mask (Flux
Attention abstract on arXiv 2604.07394: each layer runs FA or SA; technical
summary on gist.science, section 2).  Block-sparse attention reaches exactly
the masked-softmax definition, so the oracle IS that definition:

    allowed(p, t) = t <= p  and  (layer is FA  or  M[p // B][t // B] == 1)
    O[p] = sum_t softmax_t(scale * q[p].k[t] restricted to allowed) * v[t]

Grouped KV heads: query head h reads KV head h // (Hq / Hkv).  The default
scale is 1/sqrt(d).  Decode: one new token per sequence whose cache already
holds the token itself, so the query sits at position N-1 of N keys and uses
the same rule (the route fixed at prefill is reused for decode: technical
summary, section 2, deployment paragraph).

Soft routing (training-time form; technical summary, section 2: the
Gumbel-softmax relaxation forms a convex combination of the FA and SA branch
with the router's continuous weight r):  O_soft = r * O_FA + (1 - r) * O_SA.

The softmax is taken over a whole row at once (no online rescaling, no
blocking); rows are only chunked to bound memory.
"""

import math

import numpy as np

ROW_CHUNK = 1024


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def allowed_matrix(rows, n_keys, fa, mask, block_size):
    """Boolean ``[len(rows)][n_keys]``: may query position p see key t."""
    rows = np.asarray(rows, dtype=np.int64)
    t = np.arange(n_keys, dtype=np.int64)
    ok = t[None, :] <= rows[:, None]
    if not fa:
        m = np.asarray(mask).astype(bool)
        ok &= m[rows[:, None] // block_size, t[None, :] // block_size]
    return ok


def attention_probs(q_rows, k, rows, fa, mask, block_size, scale):
    """Attention weights ``[len(rows)][n_keys]`` of one head.

    q_rows: ``[len(rows)][d]`` queries at positions ``rows``; k: ``[n_keys][d]``.
    """
    scores = scale * (_as64(q_rows) @ _as64(k).T)
    ok = allowed_matrix(rows, k.shape[0], fa, mask, block_size)
    scores = np.where(ok, scores, -np.inf)
    top = scores.max(axis=1, keepdims=True)
    e = np.where(ok, np.exp(scores - top), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def attention_prefill(q, k, v, fa, mask=None, block_size=None, scale=None,
                      rows=None, heads=None):
    """Prefill attention of one sequence.

    q: ``[S][Hq][d]``; k, v: ``[S][Hkv][d]`` (any float dtype, widened).
    ``fa`` selects Full Attention; otherwise ``mask`` (dense ``[nb][nb]``) and
    ``block_size`` define the SA key set.  ``rows`` / ``heads`` select the
    query positions / heads to evaluate (default: all).
    Returns float64 ``[len(rows)][len(heads)][d]``.
    """
    S, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(hq)) if heads is None else list(heads)
    out = np.zeros((len(rows), len(heads), d), dtype=np.float64)
    for hi, h in enumerate(heads):
        g = h // group
        for c0 in range(0, len(rows), ROW_CHUNK):
            rr = rows[c0:c0 + ROW_CHUNK]
            n_keys = int(rr.max()) + 1  # causal: later keys never contribute
            p = attention_probs(q[rr, h, :], k[:n_keys, g, :], rr, fa, mask,
                                block_size, scale)
            out[c0:c0 + len(rr), hi, :] = p @ _as64(v[:n_keys, g, :])
    return out


def attention_prefill_varlen(q, k, v, cu_seqlens, route, layer, mask, block_size,
                             scale=None, rows_per_req=None, heads=None):
    """Packed variable-length prefill: requests never attend to each other.

    q: ``[T][Hq][d]``, k/v: ``[T][Hkv][d]`` packed by ``cu_seqlens``;
    ``route[r][layer]`` is 1 for FA, 0 for SA.  ``mask`` is one mask big
    enough for the longest request (a shorter request uses its leading
    rows/columns, since an entry does not depend on the length).
    Returns a list with one ``[rows][heads][d]`` array per request.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    outs = []
    for r in range(len(cu) - 1):
        a, b = int(cu[r]), int(cu[r + 1])
        rows = None if rows_per_req is None else rows_per_req[r]
        fa = bool(route[r][layer])
        outs.append(attention_prefill(q[a:b], k[a:b], v[a:b], fa, mask, block_size,
                                      scale, rows, heads))
    return outs


def attention_decode(q, k_cache, v_cache, seqlens, fa, mask=None, block_size=None,
                     scale=None, seqs=None, heads=None):
    """One decode step.

    q: ``[n_seq][Hq][d]`` (the newest token of each sequence);
    k_cache, v_cache: ``[n_seq][Hkv][max_len][d]`` holding ``seqlens[b]`` valid
    keys each, the newest included.  ``fa`` is a bool or one bool per
    sequence.  Returns float64 ``[len(seqs)][len(heads)][d]``.
    """
    n_seq, hq, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqs = list(range(n_seq)) if seqs is None else list(seqs)
    heads = list(range(hq)) if heads is None else list(heads)
    fa_list = [bool(fa)] * n_seq if np.isscalar(fa) or isinstance(fa, bool) else [bool(x) for x in fa]
    out = np.zeros((len(seqs), len(heads), d), dtype=np.float64)
    for si, b in enumerate(seqs):
        n = int(seqlens[b])
        row = np.array([n - 1], dtype=np.int64)
        for hi, h in enumerate(heads):
            g = h // group
            keys = k_cache[b, g, :n, :]
            p = attention_probs(q[b, h, :][None, :], keys, row, fa_list[b], mask,
                                block_size, scale)
            out[si, hi, :] = (p @ _as64(v_cache[b, g, :n, :]))[0]
    return out


def attention_prefill_soft(q, k, v, r, mask, block_size, scale=None, rows=None, heads=None):
    """Soft-routed prefill of one sequence: the convex combination
    ``r * FA + (1 - r) * SA`` of the two branches, each the plain definition
    above (technical summary, section 2, differentiable soft routing).
    Returns float64 ``[len(rows)][len(heads)][d]``."""
    fa = attention_prefill(q, k, v, True, mask, block_size, scale, rows, heads)
    sa = attention_prefill(q, k, v, False, mask, block_size, scale, rows, heads)
    return float(r) * fa + (1.0 - float(r)) * sa

"""Block mask of the Sparse Attention layers, oracle (test infrastructure only).

The pages name block-sparse attention (Block-Sparse-Attention library, on the
Flux Attention Qwen3-4B model card, "Sample Usage") and say SA layers keep
only a minimal KV set and never read the historical KV (technical summary on
gist.science, section 2, deployment paragraph).  The concrete pattern used
here is a reading: ``s`` sink blocks at the start of the sequence plus a
causal local window of ``w`` blocks that includes the diagonal block.

Block (i, j) of an ``nb x nb`` mask over blocks of ``B`` tokens is active iff
``j <= i`` and (``j < s`` or ``j >= i - w + 1``).  Integer work: compared
bit for bit.
"""

import numpy as np


def num_blocks(seqlen, block_size):
    """ceil(S / B): a partial last block still counts as a block."""
    return (int(seqlen) + int(block_size) - 1) // int(block_size)


def block_mask(nb, sink_blocks, local_blocks):
    """Dense uint8 mask ``[nb][nb]`` by the definition, one entry at a time."""
    if local_blocks < 1 or sink_blocks < 0:
        raise ValueError("need local_blocks >= 1 and sink_blocks >= 0")
    m = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        for j in range(nb):
            causal = j <= i
            sink = j < sink_blocks
            local = j >= i - local_blocks + 1
            m[i, j] = 1 if (causal and (sink or local)) else 0
    return m


def mask_to_csr(m):
    """Row-compressed form of a dense mask: ``row_ptr [nb+1]`` and
    ``col_idx [nnz]`` (int32), columns ascending within a row."""
    m = np.asarray(m)
    row_ptr = [0]
    col_idx = []
    for i in range(m.shape[0]):
        for j in range(m.shape[1]):
            if m[i, j]:
                col_idx.append(j)
        row_ptr.append(len(col_idx))
    return np.array(row_ptr, dtype=np.int32), np.array(col_idx, dtype=np.int32)


def mask_row_count(i, sink_blocks, local_blocks):
    """Active blocks in row i, in closed form: the window part
    ``min(i+1, w)`` plus the sink blocks left of the window
    ``max(0, min(s, i-w+1))``."""
    return min(i + 1, local_blocks) + max(0, min(sink_blocks, i - local_blocks + 1))


def mask_nnz(nb, sink_blocks, local_blocks):
    """Total active blocks of an ``nb x nb`` mask (sum of the row counts)."""
    return sum(mask_row_count(i, sink_blocks, local_blocks) for i in range(nb))

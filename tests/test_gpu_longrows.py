"""SA rows with more than 64 blocks, through the C ABI binding, against the
float64 oracle.

The prefill and decode kernels keep the first 64 columns of a mask row in
registers (one per lane) and read later columns from memory; the static sink +
window masks of the bench shapes never reach 64 blocks per row, so these cases
build rows that do: a contiguous window of 70 blocks and a scattered row
(every other block plus the diagonal, up to 76 entries)."""

import numpy as np
import pytest
import torch

import oracle
from tests.flux_testlib import assert_attn_close, ensure_built

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ensure_built()
    import block_sparse_attention_flux_amd as flux
    from tests.test_gpu_parity import f32, make_decode, run_prefill_case, say
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"


def scattered_rows(nb):
    """Row i: every even block up to i, and the diagonal (sorted, unique)."""
    return [sorted({j for j in range(0, i + 1, 2)} | {i}) for i in range(nb)]


def csr_of(rows):
    rp = np.zeros(len(rows) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([c for r in rows for c in r], dtype=np.int32)
    dense = np.zeros((len(rows), len(rows)), dtype=np.uint8)
    for i, r in enumerate(rows):
        dense[i, r] = 1
    return (torch.tensor(rp, device=DEV), torch.tensor(ci, device=DEV), dense)


@pytest.mark.parametrize("pattern,d", [("window70", 64), ("scattered", 128)])
def test_sa_prefill_rows_beyond_64_blocks(pattern, d):
    B, S, hq, hkv = 64, 9600, 4, 2
    nb = S // B
    say(f"SA prefill with long mask rows: {pattern}, d={d}")
    q, k, v, cu, sa, rp, ci, route = run_prefill_case([S], hq, hkv, d, B, 1, 70, [[0]], 4242 + d)
    if pattern == "window70":
        m = oracle.block_mask(nb, 1, 70)
    else:
        rp, ci, m = csr_of(scattered_rows(nb))
    assert int(m.sum(axis=1).max()) > 64
    out = flux.attn_prefill(q, k, v, cu, S, route, 0, rp, ci, sa)
    torch.cuda.synchronize()
    # rows whose mask row holds fewer and more than 64 blocks, block edges, the last row
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, 4095, 4096, 4159, 4160, 8191, 8192, 9000, 9598, 9599}))
    ref = oracle.attention_prefill(f32(q), f32(k), f32(v), False, m, B, rows=rows)
    assert_attn_close(f32(out)[rows], ref, f"long rows {pattern}")


def test_sa_decode_rows_beyond_64_blocks():
    B, max_len, hq, hkv, d = 64, 9600, 8, 2, 128
    nb = max_len // B
    seqlens = [9600, 8193, 4160, 100]
    say("SA decode with long, scattered mask rows")
    qd, kc, vc, sl = make_decode(len(seqlens), max_len, seqlens, hq, hkv, d, 4343)
    rp, ci, m = csr_of(scattered_rows(nb))
    sa = flux.SAParams(B, 1, 3)
    route = torch.tensor([[0]] * len(seqlens), dtype=torch.uint8, device=DEV)
    out = flux.attn_decode(qd, kc, vc, sl, route, 0, rp, ci, sa)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(f32(qd), f32(kc), f32(vc), seqlens, False, m, B)
    assert_attn_close(f32(out), ref, "decode long rows")

"""The attention comparison (allclose atol 2e-2 / rtol 1e-2 AND relative
Frobenius error <= 1e-2) on outputs whose entries are all small, as at long
context (an output averages ~N/e values): the elementwise check alone would
accept an all-zero output, the Frobenius check must reject it, and bf16
rounding of the exact output must pass."""

import numpy as np
import pytest
import torch

import oracle
from tests.flux_testlib import assert_attn_close, attn_errors


def _long_rows():
    r = np.random.default_rng(7)
    S, hq, hkv, d = 4096, 4, 2, 64
    q = r.standard_normal((S, hq, d))
    k = r.standard_normal((S, hkv, d))
    v = 0.15 * r.standard_normal((S, hkv, d))  # keeps every output entry below atol
    rows = list(range(S - 16, S))
    return oracle.attention_prefill(q, k, v, True, rows=rows)


def test_zero_output_is_rejected_at_long_context():
    ref = _long_rows()
    assert np.abs(ref).max() < 0.02
    zeros = np.zeros_like(ref)
    excess, frob, _ = attn_errors(zeros, ref)
    assert excess <= 0.0  # the elementwise check alone passes it
    assert frob == pytest.approx(1.0)
    with pytest.raises(AssertionError, match="Frobenius"):
        assert_attn_close(zeros, ref, "zeros")


def test_bf16_rounding_of_exact_output_passes():
    ref = _long_rows()
    got = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert_attn_close(got, ref, "bf16 rounding")


def test_two_percent_noise_is_rejected():
    ref = _long_rows()
    noisy = ref * (1.0 + 0.02 * np.random.default_rng(8).standard_normal(ref.shape))
    with pytest.raises(AssertionError, match="Frobenius"):
        assert_attn_close(noisy, ref, "noise")

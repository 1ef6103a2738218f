"""Pins of the oracle's base projection and gated LoRA (CPU only)."""

import numpy as np
import torch

from oracle import lora

import workload


def test_matches_brute_force_loops():
    x, W, A, B = (t.double().numpy() for t in workload.lora_case(1, 6, 5, 4, 2, torch.float32))
    mask = np.array([0, 1, 0, 1, 1, 0], bool)
    s = 0.75
    got = lora.gated_lora(x, W, A, B, mask, s)
    for m in range(6):
        for n in range(4):
            base = sum(x[m, k] * W[n, k] for k in range(5))
            if mask[m]:
                t = [sum(x[m, k] * A[j, k] for k in range(5)) for j in range(2)]
                base += s * sum(t[j] * B[n, j] for j in range(2))
            assert abs(got[m, n] - base) < 1e-12


def test_clean_rows_identical_to_base_and_zero_adapter_is_identity():
    x, W, A, B = (t.double().numpy() for t in workload.lora_case(2, 16, 32, 24, 4, torch.float32))
    mask = workload.stride_mask(16, 4)
    base = lora.linear(x, W)
    y = lora.gated_lora(x, W, A, B, mask, 1.0)
    assert np.array_equal(y[~mask], base[~mask])
    assert not np.allclose(y[mask], base[mask])
    assert np.array_equal(lora.gated_lora(x, W, A, np.zeros_like(B), mask, 1.0), base)


def test_delta_has_rank_at_most_r_and_is_linear_in_scale():
    x, W, A, B = (t.double().numpy() for t in workload.lora_case(3, 40, 64, 48, 3, torch.float32))
    mask = workload.stride_mask(40, 4)
    base = lora.linear(x, W)
    d1 = lora.gated_lora(x, W, A, B, mask, 1.0) - base
    d2 = lora.gated_lora(x, W, A, B, mask, 2.5) - base
    assert np.linalg.matrix_rank(d1[mask], tol=1e-10) == 3
    assert np.allclose(d2, 2.5 * d1, rtol=1e-12, atol=1e-15)

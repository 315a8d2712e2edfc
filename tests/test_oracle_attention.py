"""Pins of the oracle's softmax attention: brute force, a library routine, special cases."""
import numpy as np
import pytest
import torch

from oracle.cache import softmax_attention
from oracle.reference import direct_attention

pytestmark = pytest.mark.cpu


def test_matches_scalar_loops_on_tiny_inputs():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((3, 2, 6)) * 2
    k = rng.standard_normal((2, 5, 6)) * 2
    v = rng.standard_normal((2, 5, 6))
    assert np.max(np.abs(softmax_attention(q, k, v) - direct_attention(q, k, v))) < 1e-12


def test_matches_library_sdpa_fp64():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((33, 4, 64)) * 3
    k = rng.standard_normal((4, 517, 64)) * 3
    v = rng.standard_normal((4, 517, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k), torch.from_numpy(v))
    ref = ref.permute(1, 0, 2).numpy()
    assert np.max(np.abs(softmax_attention(q, k, v) - ref)) < 1e-12


def test_special_cases():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 1, 8))
    k1 = rng.standard_normal((1, 1, 8))
    v1 = rng.standard_normal((1, 1, 8))
    assert np.allclose(softmax_attention(q, k1, v1), np.broadcast_to(v1[0, 0], (4, 1, 8)), atol=0, rtol=0)
    keq = np.broadcast_to(k1, (1, 9, 8)).copy()
    v9 = rng.standard_normal((1, 9, 8))
    assert np.max(np.abs(softmax_attention(q, keq, v9) - v9[0].mean(0))) < 1e-14
    # a huge score margin selects one key
    k = np.zeros((1, 3, 8)); k[0, 1, 0] = 1000.0
    qq = np.zeros((1, 1, 8)); qq[0, 0, 0] = 1.0
    v = np.arange(24, dtype=np.float64).reshape(1, 3, 8)
    assert np.array_equal(softmax_attention(qq, k, v)[0, 0], v[0, 1])

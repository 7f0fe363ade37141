"""The parity helper's tolerance checks on planted arrays (CPU)."""
from __future__ import annotations

import numpy as np
import pytest

from parity_util import tol_check


def test_output_bound_is_per_request():
    # request 0: one-row request with large outputs; request 1: long request, small outputs
    ref = np.zeros((2, 3, 8))
    ref[0] = 3.5
    ref[1] = 0.15
    got = ref.copy()
    got[1, 0, 0] += 0.01          # within 1e-2 * 3.5 + 1e-3, not within 1e-2 * 0.15 + 1e-3
    tol_check("global", got, ref, False, "o")               # the whole-tensor bound lets it pass
    with pytest.raises(AssertionError, match="request 1"):
        tol_check("per request", got, ref, False, "o", s_q=1)
    got[1, 0, 0] = ref[1, 0, 0] + 2e-3                      # inside 1e-2 * 0.15 + 1e-3
    tol_check("per request", got, ref, False, "o", s_q=1)


def test_per_request_groups_tokens_by_s_q():
    ref = np.zeros((4, 2, 4))
    ref[:2] = 1.0                  # request 0: tokens 0, 1
    ref[2:] = 0.1                  # request 1: tokens 2, 3
    got = ref.copy()
    got[3, 1, 2] += 0.005          # bound for request 1: 2e-3
    with pytest.raises(AssertionError, match="request 1"):
        tol_check("s_q=2", got, ref, False, "o", s_q=2)


def test_unsampled_entries_are_skipped():
    ref = np.full((3, 2, 4), np.nan)
    ref[1] = 0.2
    got = np.zeros_like(ref)
    got[1] = 0.2
    assert tol_check("sampled", got, ref, False, "o", s_q=1) == 0.0


def test_lse_pattern_and_bound():
    ref = np.array([0.5, -np.inf, 2.0])
    tol_check("lse", np.array([0.5009, -np.inf, 2.0]), ref, False, "lse")
    with pytest.raises(AssertionError, match="-inf pattern"):
        tol_check("lse", np.array([0.5, 0.0, 2.0]), ref, False, "lse")
    with pytest.raises(AssertionError, match="exceeds"):
        tol_check("lse", np.array([0.5, -np.inf, 2.0011]), ref, False, "lse")

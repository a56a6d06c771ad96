"""Pins of the attention oracle against facts other than itself (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle.attention import unmasked_pairs
from tests import pins


@pytest.mark.parametrize("pin", pins.FWD_PINS + pins.BWD_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)


def test_scalar_bruteforce_fwd():
    pins.pin_scalar_bruteforce_fwd(oracle, oracle.scalar_attention_fwd)


def test_scalar_bruteforce_bwd():
    pins.pin_scalar_bruteforce_bwd(oracle, oracle.scalar_attention_bwd)


def test_rows_variant_matches_full():
    c, _ = pins.tiny_case(21, targets=[1, 0, 0, 2])
    O, A = pins.fwd(oracle, c)
    rows = np.array([0, 2, 3, 7, 14])
    O2, A2 = oracle.attention_fwd_rows(c["q"], c["k"], c["v"], c["u"], c["seq_offsets"],
                                       c["max_len"], rows, c["num_targets"], c["timestamps"],
                                       c["rab_pos"], c["rab_time"])
    # one row at a time (matrix-vector) vs blocks of rows: BLAS order may differ
    assert pins.rel(O2, O[rows]) < 1e-13 and pins.rel(A2, A[rows]) < 1e-13


def test_unmasked_pair_count_bruteforce():
    offs = np.array([0, 3, 3, 10, 12])
    nt = np.array([1, 0, 4, 2])
    want = 0
    for b in range(4):
        L = offs[b + 1] - offs[b]
        hist = L - nt[b]
        want += sum(1 for i in range(L) for j in range(L) if (j <= i and j < hist) or j == i)
    assert unmasked_pairs(offs, nt) == want
    assert unmasked_pairs(offs) == sum(int(L) * (int(L) + 1) // 2 for L in np.diff(offs))

"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one plausible slip into the oracle — a wrong table value, a
swapped nibble order, a transposed operand, a wrong scale block width, a dropped
term — and runs the pin that is meant to catch it; the pin must fail.
"""
import numpy as np
import pytest

import oracle
import test_oracle_formats as F
import test_oracle_grouped as G
from oracle import codebooks, grouped, pack


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_swapped_nf4_table_entry_is_caught(monkeypatch):
    bad = oracle.NF4_TABLE_F32.copy()
    bad[[9, 10]] = bad[[10, 9]]
    monkeypatch.setattr(F.oracle, "NF4_TABLE_F32", bad)
    assert _fails(F.test_nf4_table_matches_published_values)


def test_swapped_nibble_order_is_caught(monkeypatch):
    monkeypatch.setattr(pack, "pack_nf4_codes",
                        lambda c: ((np.asarray(c)[..., 1::2] << 4) | np.asarray(c)[..., 0::2]).astype(np.uint8))
    monkeypatch.setattr(F.P, "pack_nf4_codes", pack.pack_nf4_codes)
    assert _fails(F.test_nibble_order_convention)


def test_transposed_operand_is_caught(monkeypatch):
    def bad_grouped(a_bits, sizes, weights, N):
        off = oracle.offsets(sizes)
        out = np.zeros((a_bits.shape[0], N))
        for e in range(len(off) - 1):
            lo, hi = int(off[e]), int(off[e + 1])
            if hi > lo:
                w = weights(e)
                out[lo:hi] = grouped._bf16_to_f64(a_bits[lo:hi]) @ w.reshape(w.shape[1], w.shape[0])[:, :N]
        return out
    monkeypatch.setattr(G.oracle, "grouped_ref", bad_grouped)
    assert _fails(G.test_grouped_matches_brute_force) or _fails(G.test_grouped_is_a_times_w_transposed_nonsquare)


def test_wrong_scale_block_width_is_caught(monkeypatch):
    monkeypatch.setattr(pack, "NF4_BLOCK", 32)
    with pytest.raises(Exception):
        G.test_scale_blocks_are_64_wide_and_row_local()


def test_dropped_e2m1_mantissa_is_caught(monkeypatch):
    monkeypatch.setattr(F.oracle, "e2m1_value", lambda c: codebooks.e2m1_value(int(c) & ~1))
    assert _fails(F.test_e2m1_matches_ocp_table)


def test_wrong_e8m0_bias_is_caught(monkeypatch):
    monkeypatch.setattr(F.oracle, "e8m0_value", lambda x: np.ldexp(1.0, np.asarray(x) - 128))
    assert _fails(F.test_e8m0_all_bytes)


def test_dropped_expert_in_dgrad_is_caught(monkeypatch):
    real = oracle.dgrad_ref
    def bad(dy, sizes, weights, K):
        out = real(dy, sizes, weights, K)
        out[: int(sizes[0])] = 0.0
        return out
    monkeypatch.setattr(G.oracle, "dgrad_ref", bad)
    assert _fails(G.test_dgrad_brute_force_and_adjoint_identity)

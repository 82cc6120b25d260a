"""The oracle's pins have teeth: plausible mistakes planted in the oracle (on
the CPU, through monkeypatch) make at least one pin fail.

Each case replaces one oracle function with a wrong variant, runs the pins
that should catch it, and requires an AssertionError.  The oracle itself is
restored after every case.
"""

import numpy as np
import pytest

import oracle
import oracle.spense as ospense
import test_oracle as pins
from oracle import DT_BF16


def _planted(monkeypatch, name, fn):
    monkeypatch.setattr(ospense, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _expect_caught(checks):
    caught = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught > 0, "no pin caught the planted mistake"


def _golden(dtype):
    return [lambda c=c: pins.test_hand_worked(c) for c in pins._golden_cases() if c["dtype"] == dtype]


def test_signed_bf16_key_is_caught(monkeypatch):
    """The bf16 bit pattern read as a signed integer instead of sign-cleared."""
    good = ospense.magnitude_key

    def signed(bits, dtype):
        if dtype == DT_BF16:
            return np.asarray(bits, dtype=np.uint16).view(np.int16).astype(np.int64)
        return good(bits, dtype)

    _planted(monkeypatch, "magnitude_key", signed)
    _expect_caught(_golden("bf16"))
    _expect_caught([lambda: pins.test_key_order_is_magnitude_order_every_code(DT_BF16)])
    _expect_caught([pins.test_tie_break_exhaustive_small_ints])


def test_unmasked_bf16_key_is_caught(monkeypatch):
    """The bf16 key with the sign bit left in (unsigned 16-bit pattern)."""
    good = ospense.magnitude_key

    def unmasked(bits, dtype):
        if dtype == DT_BF16:
            return np.asarray(bits, dtype=np.uint16).astype(np.int64)
        return good(bits, dtype)

    _planted(monkeypatch, "magnitude_key", unmasked)
    _expect_caught(_golden("bf16"))
    _expect_caught([pins.test_tie_break_exhaustive_small_ints])


def _wrap_bound(monkeypatch, name, change):
    good = getattr(ospense, name)

    def wrong(*a, **k):
        Y, B = good(*a, **k)
        return Y, change(Y, B)

    _planted(monkeypatch, name, wrong)


@pytest.mark.parametrize("change", [lambda Y, B: 3 * B, lambda Y, B: B + 1.0, lambda Y, B: np.abs(Y)],
                         ids=["times3", "plus1", "abs_of_sum"])
def test_wrong_error_scale_is_caught(monkeypatch, change):
    """An inflated or mis-formed error scale B in every function returning one."""
    for name in ("linear_ref", "linear_rows_ref", "down_ref", "linear_w8a8_ref"):
        _wrap_bound(monkeypatch, name, change)
    _expect_caught(_golden("f32") + _golden("fp8") + _golden("bf16"))
    _expect_caught([pins.test_brute_force_e4m3_with_scales_and_bound])
    _expect_caught([pins.test_rows_brute_force_every_dense_row_set_6x8])
    _expect_caught([pins.test_down_ref_brute_force_loops])
    _expect_caught([pins.test_w8a8_tiny_brute_force_loops])


def test_bound_from_unpruned_weights_is_caught(monkeypatch):
    """B taken over the weights before pruning (the pruned positions counted)."""
    good_unpack = ospense.unpack_bits

    def with_pruned(p):
        # put the largest kept value of each group on every pruned slot of the
        # sparse region: a stand-in for magnitudes that pruning removed
        out = good_unpack(p).copy()
        if p.K_s:
            N = out.shape[0]
            mask = p.mask.reshape(N, -1).astype(bool)
            cols = p.pi[: p.K_s]
            fill = np.repeat(p.vals[:, 0::2], 4, axis=1)
            region = out[:, cols]
            region[~mask] = fill[~mask]
            out[:, cols] = region
        return out

    good_linear = ospense.linear_ref

    def wrong(X_bits, xdtype, p, scales=None):
        Y, _ = good_linear(X_bits, xdtype, p, scales)
        Wfull = ospense.decode_values(with_pruned(p), p.dtype)
        X = ospense.decode_values(X_bits, xdtype)
        B = np.abs(X) @ np.abs(Wfull).T
        if scales is not None:
            B = B * np.asarray(scales, dtype=np.float32).astype(np.float64)[None, :]
        return Y, B

    _planted(monkeypatch, "linear_ref", wrong)
    _expect_caught(_golden("f32") + _golden("fp8") + _golden("bf16"))
    _expect_caught([pins.test_brute_force_e4m3_with_scales_and_bound])

"""Pins for the int8 block-quantised state oracle (oracle/mlstm_q8.py).

The encoding is checked on hand-worked blocks (round half to even, the block
maximum mapping to +-127, an all-zero block), against its error bound on
random data (|decode(encode(x)) - x| <= scale / 2 elementwise), and for block
independence.  The quantised step is the float step of the pinned recurrence
followed by the encoding; its readout is checked against the float step from
the decoded state.
"""
import numpy as np
import pytest

from oracle import q8_decode, q8_encode, q8_scaled, recurrent_fw, recurrent_step_q8


def test_hand_worked_block():
    x = np.zeros((1, 64))
    # amax = 127: the scaled values are the values themselves, ties exact
    x[0, :7] = [127.0, -63.5, 31.75, 0.0, 2.5, -3.5, 0.49]
    codes, scales = q8_encode(x)
    # -63.5 -> -64 (even), 31.75 -> 32, 2.5 -> 2 (even), -3.5 -> -4 (even), 0.49 -> 0
    assert codes[0, :7].tolist() == [127, -64, 32, 0, 2, -4, 0]
    assert np.all(codes[0, 7:] == 0)
    assert scales.shape == (1, 1) and scales[0, 0] == 1.0


def test_negative_maximum_and_zero_block():
    x = np.zeros((2, 128))
    x[0, 3] = -8.0
    x[0, 70] = 0.5                  # second block of row 0: its own scale
    codes, scales = q8_encode(x)
    assert codes[0, 3] == -127 and scales[0, 0] == pytest.approx(8.0 / 127)
    assert codes[0, 70] == 127 and scales[0, 1] == pytest.approx(0.5 / 127)
    assert np.all(codes[1] == 0) and np.all(scales[1] == 0)
    np.testing.assert_array_equal(q8_decode(codes, scales)[1], 0.0)


def test_error_bound_and_code_range():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 16, 192)) * rng.uniform(1e-3, 1e3, (3, 16, 1))
    codes, scales = q8_encode(x)
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(q8_decode(codes, scales) - x)
    bound = np.repeat(scales, 64, axis=-1) / 2
    assert np.all(err <= bound * (1 + 1e-12))
    # every block reaches +-127 at its maximum
    blocks = np.abs(codes.reshape(3, 16, 3, 64)).max(axis=-1)
    assert np.all(blocks == 127)


def test_blocks_are_independent():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 128))
    c1, s1 = q8_encode(x)
    y = x.copy()
    y[:, 64:] *= 1000.0
    c2, s2 = q8_encode(y)
    np.testing.assert_array_equal(c1[:, :64], c2[:, :64])
    np.testing.assert_array_equal(s1[:, 0], s2[:, 0])


def test_scaled_values_round_to_codes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    codes, _ = q8_encode(x)
    np.testing.assert_array_equal(np.rint(q8_scaled(x)), codes)


@pytest.mark.parametrize("gate", ["exp", "sig"])
def test_quantised_step_is_the_float_step_then_the_encoding(gate):
    rng = np.random.default_rng(3)
    B, DK, DV = 2, 8, 128
    C = 0.1 * rng.standard_normal((B, DK, DV))
    codes, scales = q8_encode(C)
    q, k = rng.standard_normal((B, DK)), rng.standard_normal((B, DK))
    v = rng.standard_normal((B, DV))
    i, f = rng.standard_normal(B), 2 + rng.random(B)
    n = rng.random((B, DK)) if gate == "exp" else None
    m = rng.standard_normal(B) if gate == "exp" else None
    h, C1, c1, s1, n1, m1 = recurrent_step_q8(q, k, v, i, f, codes, scales, n, m, gate=gate)
    C0 = q8_decode(codes, scales)
    a = [q[:, None], k[:, None], v[:, None], i[:, None], f[:, None]]
    if gate == "exp":
        H, Cr, nr, mr = recurrent_fw(*a, C0, n, m, gate=gate)
        np.testing.assert_allclose(n1, nr, rtol=0, atol=0)
        np.testing.assert_allclose(m1, mr, rtol=0, atol=0)
    else:
        H, Cr, _, _ = recurrent_fw(*a, C0, gate=gate)
    np.testing.assert_array_equal(h, H[:, 0])
    np.testing.assert_array_equal(C1, Cr)
    c2, s2 = q8_encode(Cr)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
    # the quantised state stays within half a quantum of the float state
    assert np.all(np.abs(q8_decode(c1, s1) - Cr) <= np.repeat(s1, 64, axis=-1) / 2 * (1 + 1e-12))


def test_zero_state_step():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((1, 4)), rng.standard_normal((1, 4)), rng.standard_normal((1, 64))
    h, C1, c1, s1, n1, m1 = recurrent_step_q8(q, k, v, np.zeros(1), np.zeros(1), gate="exp")
    H = recurrent_fw(q[:, None], k[:, None], v[:, None], np.zeros((1, 1)), np.zeros((1, 1)), gate="exp")[0]
    np.testing.assert_array_equal(h, H[:, 0])

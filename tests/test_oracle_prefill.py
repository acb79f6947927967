"""Pins of the four-buffer prefill oracle (oracle.prefill)."""
import numpy as np
import pytest

from oracle.formats import decode_bf16
from oracle.prefill import exposed_bound, run, schedule
from synth.gen import f32_to_bf16_bits


def test_fig3_bindings():
    # Fig. 3: H2D loads L1..L5 into B1, B2, B3 and then reuses B1, B2; L0
    # stays in B0.  L4 takes the buffer L1 released, L5 the one L2 released.
    bind, freed_by, trigger = schedule(6)
    assert bind == [0, 1, 2, 3, 1, 2]
    assert freed_by == [-1, -1, -1, -1, 1, 2]
    assert trigger == [-1, -1, -1, -1, 1, 2]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 16, 61, 78])
def test_b0_stays_with_layer_0_and_three_buffers_rotate(n):
    bind, _, _ = schedule(n)
    assert bind[0] == 0 and 0 not in bind[1:]
    assert set(bind[1:]) <= {1, 2, 3}
    # Default map i -> i + 3: layer l >= 1 uses buffer 1 + (l - 1) mod 3.
    assert bind[1:] == [1 + (l - 1) % 3 for l in range(1, n)]


def test_custom_maps():
    # Loads issued one layer later than the default: nothing at layer 1's
    # point, so layer 4 takes the buffer layer 1 released (B1) at layer 2's
    # point, and every later load uses the oldest released buffer.
    m = [-1, -1, 4, 5, 6, 7, -1, -1]
    bind, freed_by, trigger = schedule(8, m)
    assert bind == [0, 1, 2, 3, 1, 2, 3, 1]
    assert freed_by == [-1, -1, -1, -1, 1, 2, 3, 4]
    assert trigger == [-1, -1, -1, -1, 2, 3, 4, 5]
    with pytest.raises(ValueError):
        schedule(6, [-1, 4, 4, -1, -1, -1])      # layer 4 loaded twice
    with pytest.raises(ValueError):
        schedule(6, [-1, 1, -1, -1, -1, -1])     # not a future layer
    with pytest.raises(ValueError):
        schedule(6, [-1, 3, -1, -1, -1, -1])     # layer 3 is already bound
    with pytest.raises(ValueError):
        schedule(6, [-1, -1, -1, -1, -1, -1])    # layers 4, 5 never loaded


def test_exposed_bound_closed_forms():
    assert exposed_bound(3.0, 1.0, 2) == 1.0
    assert exposed_bound(3.0, 1.0, 3) == 0.0
    # One shared copy path: the transfer term is tau_H2D + tau_D2H.
    assert exposed_bound(3.0 + 2.0, 1.0, 2) == 3.0


def test_run_appends_and_sums():
    # Constant rows: a layer whose history rows are all v and new rows all w
    # sums to n_hist * v + n_new * w in every column; the new rows land after
    # the history on host, the rest of host memory is unchanged.
    NL, rows, n_hist, n_new = 3, 20, 12, 5
    host = np.zeros((NL, rows, 576), np.uint16)
    new = np.zeros((NL, n_new, 576), np.uint16)
    for layer in range(NL):
        host[layer, :n_hist] = f32_to_bf16_bits(np.float32([layer + 1]))[0]
        host[layer, n_hist:] = f32_to_bf16_bits(np.float32([-100.0]))[0]   # never read
        new[layer] = f32_to_bf16_bits(np.float32([-2 * layer - 0.5]))[0]
    after, out = run(host, new, n_hist)
    for layer in range(NL):
        assert np.all(out[layer] == n_hist * (layer + 1) + n_new * (-2 * layer - 0.5))
        assert np.array_equal(after[layer, n_hist:n_hist + n_new], new[layer])
        assert np.array_equal(after[layer, :n_hist], host[layer, :n_hist])
        assert np.all(decode_bf16(after[layer, n_hist + n_new:]) == -100.0)

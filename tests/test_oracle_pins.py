"""The oracle against its pins (values the pages print, closed forms, library
routines, brute force).  CPU only."""
import numpy as np
import pytest

import oracle.switch_oracle as so
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: getattr(f, "__name__", "independent_forms_small"))
def test_pin(pin):
    pin(so)


def test_independent_forms_tiny_config_shape():
    """Index form vs dense one-hot form vs per-token loop at the tiny layer's
    shape (T=512, d=64, d_ff=128, E=4, c=1.25, +2 on expert 0's bias)."""
    L = pins.pin_independent_forms(so)
    assert L.C == 160
    assert (~L.slots.keep).sum() > 0


def test_capacity_rejects_bad_arguments():
    for args in [(10, 0, 1.0), (10, 4, -1.0), (10, 4, float("nan")), (10, 4, float("inf"))]:
        with pytest.raises(ValueError):
            so.capacity(*args)


def test_nonfinite_logits_rejected():
    with pytest.raises(ValueError):
        so.softmax_top1(np.array([[0.0, np.nan]]))


def test_backward_weight_gradient_subset():
    """dw_experts only selects which experts' weight gradients are returned:
    the rows equal the full result's, every other output is identical."""
    rng = np.random.default_rng(41)
    T, d, F, E = 96, 8, 12, 5
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((d, E)) * 0.3
    w1 = rng.standard_normal((E, F, d)) * 0.2
    w2 = rng.standard_normal((E, d, F)) * 0.2
    dout = rng.standard_normal((T, d))
    full = so.layer_backward(x, w_r, None, w1, w2, 1.0, 0.01, dout)
    pick = np.array([3, 0])
    part = so.layer_backward(x, w_r, None, w1, w2, 1.0, 0.01, dout, dw_experts=pick)
    np.testing.assert_array_equal(part.dw1, full.dw1[pick])
    np.testing.assert_array_equal(part.dw2, full.dw2[pick])
    for name in ("dx", "dw_r", "db_r", "dz", "dgate"):
        np.testing.assert_array_equal(getattr(part, name), getattr(full, name))

"""The reference oracle checked against facts that do not come from itself."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_append_rejects_out_of_range(orc):
    kc = np.zeros((1, 1, 8, 4), np.uint16)
    kn = np.zeros((1, 2, 1, 4), np.uint16)
    with pytest.raises(ValueError):
        orc.kv_append(kc, kc, kn, kn, [7])
    with pytest.raises(ValueError):
        orc.kv_append(kc, kc, kn, kn, [-1])


def test_attention_rejects_bad_problem(orc):
    q = np.zeros((1, 1, 3, 4), np.uint16)
    kc = np.zeros((1, 2, 8, 4), np.uint16)
    with pytest.raises(ValueError):
        orc.gqa_decode(q, kc, kc, [0], oracle.BF16)  # 3 query heads over 2 KV heads

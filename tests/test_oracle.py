"""The oracle, pinned against the pages and mathematics (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from tests import oracle_pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", oracle_pins.ALL, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_frame(orc):
    c = oracle_pins.Case(5, 2, 1, 8, 4, "f32", 9)
    c.tables[0, 0] = c.NB + 3
    from oracle.oracle import OracleError

    with pytest.raises(OracleError):
        c.decode(orc)


def test_oracle_zero_context_gives_zeros(orc):
    c = oracle_pins.Case(6, 3, 2, 8, 4, "bf16", 9)
    c.ctx[1] = 0
    out = c.decode(orc)
    assert np.all(out[1] == 0)


from tests import blockmgr_pins  # noqa: E402


@pytest.mark.parametrize("pin", blockmgr_pins.ALL, ids=lambda p: p.__name__)
def test_oracle_blockmgr_pin(pin):
    from oracle import blockmgr

    pin(blockmgr)


from tests import dense_pins  # noqa: E402


@pytest.mark.parametrize("pin", dense_pins.ALL, ids=lambda p: p.__name__)
def test_oracle_dense_pin(pin):
    from oracle import dense

    pin(dense)

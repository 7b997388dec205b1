"""The oracle against its pins (library attention, closed forms, golden visibility, invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_malformed(orc):
    import torch

    q = torch.zeros(1, 1, 3, 4, dtype=torch.float64)
    k = torch.zeros(1, 2, 2, 4, dtype=torch.float64)
    with pytest.raises(ValueError):
        orc.attend(q, k, k, scale=1.0)  # 3 query heads over 2 KV heads
    with pytest.raises(ValueError):
        orc.attend(torch.zeros(1, 1, 2, 4, dtype=torch.float64), k, k, scale=1.0, rows=[5])

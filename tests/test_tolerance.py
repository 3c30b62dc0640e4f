"""The parity bar keeps the stated tolerance wherever the output type can meet it."""
import numpy as np
import torch

from tests.tolerance import TOL, bar, half_ulp


def test_half_ulp_matches_torch_rounding():
    # Half the spacing of adjacent representable values, measured with torch's own types.
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16), ("f32", torch.float32)):
        for x in (0.3, 0.75, 1.0, 1.5, 2.37, 5.0):
            t = torch.tensor(x, dtype=tdt)
            nxt = torch.nextafter(t, torch.tensor(100.0, dtype=tdt)).double().item()
            assert half_ulp(np.array([t.double().item()]), dt)[0] == (nxt - t.double().item()) / 2


def test_bar_is_the_stated_tolerance_where_the_output_type_allows():
    x = np.linspace(-1.99, 1.99, 1001)
    assert np.all(bar(x, "bf16") == TOL["bf16"])
    y = np.linspace(-7.9, 7.9, 1001)
    assert np.all(bar(y, "f16") == TOL["f16"])
    assert np.all(bar(y, "f32") == TOL["f32"])
    # Beyond |o| = 2 bf16 storage alone rounds by up to 7.8e-3: the bar follows it.
    assert bar(np.array([2.37]), "bf16")[0] == 2.0 ** -8 * 2 + TOL["bf16"] / 5

"""The CPU oracle against its pins (runs without a GPU)."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_small_configs_run_and_conserve():
    """Per-expert kept counts sum to T*H*k minus the dropped assignments."""
    import numpy as np
    import oracle
    from moe_inputs import SMALL, generate
    for cfg in SMALL:
        out = oracle.forward(cfg, generate(cfg))
        dropped = int((out["row_of"] < 0).sum())
        assert int(out["counts"].sum()) == cfg.T * cfg.k_total - dropped
        assert int(out["demand"].sum()) == cfg.T * cfg.k_total
        assert np.all(np.isfinite(out["y"]))

"""The FP64 oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_run_heads_pool_matches_serial():
    import numpy as np
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((6, 40, 8)) for _ in range(3))

    def unit(u):
        return oracle.attention_head(q[u], k[u], v[u], causal=True, scale=0.3)[0]

    par, workers = oracle.run_heads(unit, range(6), workers=3)
    assert workers == 3
    for u in range(6):
        assert np.array_equal(par[u], unit(u))

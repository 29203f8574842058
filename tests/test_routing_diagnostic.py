"""The routing rationale of the abstract on the CPU oracle: query sharpness
tracks the Taylor route's error, so sending the sharpest blocks to full
attention gives a smaller layer error than random or inverse routing.  A pin
of the routing direction (sharpest blocks -> full) and a check of the Spearman
helper against scipy."""

import numpy as np
import pytest
from scipy.stats import spearmanr

from oracle.isa_diagnostics import routing_diagnostic, spearman
from sparse_attention_context_amd.synth import make_local_inputs


def test_spearman_matches_scipy():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(40)
    y = x + rng.standard_normal(40)
    y[3] = y[7]  # a tie
    assert abs(spearman(x, y) - spearmanr(x, y).correlation) < 1e-12


@pytest.mark.parametrize("sigma", [1.0, 0.5, 0.25])
def test_sharpest_blocks_to_full_route_lower_the_error(sigma):
    Q, K, V = make_local_inputs(1, 2, 32, 1024, 1024, 32, sigma, seed=3)
    rho_s = []
    for h in range(2):
        r = routing_diagnostic(Q[0, h], K[0, h], V[0, h], 32, 0.25, 0.2, seed=h)
        assert r["layer_err_isa"] < r["layer_err_random"] < r["layer_err_inverse"], r
        rho_s.append(r["spearman"])
    assert np.mean(rho_s) > 0.4


def test_locality_lowers_the_taylor_error():
    errs = []
    for sigma in (1.0, 0.25, 0.05):
        Q, K, V = make_local_inputs(1, 1, 32, 512, 512, 32, sigma, seed=5)
        # layer error with every block on the Taylor route
        errs.append(np.linalg.norm(routing_diagnostic(Q[0, 0], K[0, 0], V[0, 0], 32, 0.25, 0.2)["taylor_err"]))
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 0.05

"""CPU checks of the parity comparison itself (tests/parity_util.compare)."""
import numpy as np
import pytest

from tests import parity_util as U


def _ref(n=4096, seed=0):
    return np.random.default_rng(seed).standard_normal(n)


def test_flip_explained_deviation_passes_the_norm_bar():
    ref = _ref()
    gpu = ref.copy()
    gpu[:8] += 0.8                                # a few large deviations ...
    flip = np.zeros_like(ref)
    flip[:8] = 1.0                                # ... each inside its cast-ambiguity radius
    s = U.compare("x", gpu, ref, allow=flip, norm_rel=U.NORM_TOL, flip=flip)
    assert s["norm_rel_err"] > U.NORM_TOL and s["norm_rel_unexplained"] == 0.0


def test_unexplained_deviation_fails_the_norm_bar():
    ref = _ref()
    gpu = ref * (1 + 1e-2)                        # systematic 1% error, inside a loose elementwise allowance
    allow = np.full_like(ref, 1.0)
    with pytest.raises(AssertionError, match="norm-wise"):
        U.compare("x", gpu, ref, allow=allow, norm_rel=U.NORM_TOL, flip=np.zeros_like(ref))


def test_elementwise_bar_catches_an_error_outside_the_allowance():
    ref = _ref()
    gpu = ref.copy()
    gpu[5] += 1.0
    with pytest.raises(AssertionError, match="first bad"):
        U.compare("x", gpu, ref, allow=np.zeros_like(ref))

"""The fp64 oracle against facts outside itself (CPU only)."""
import pytest

import pins

REF, SOL = pins.oracle_namespaces()


@pytest.mark.parametrize("check", pins.ALL_REF_CHECKS, ids=lambda c: c.__name__)
def test_inference_oracle_pins(check):
    check(REF)


@pytest.mark.parametrize("check", pins.ALL_SOL_CHECKS, ids=lambda c: c.__name__)
def test_solver_pins(check):
    check(SOL)


@pytest.mark.parametrize("singular", [False, True])
def test_exact_rank_end_to_end(singular):
    pins.check_exact_rank(REF, SOL, singular=singular)

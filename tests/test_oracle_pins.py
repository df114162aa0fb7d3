"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_checks as oc


@pytest.mark.parametrize("check", oc.DETERMINISTIC_CHECKS, ids=lambda f: f.__name__[6:])
def test_pin(orc, check):
    check(orc)


def test_sd_output_law_chi_square(orc):
    """SD's emitted tokens follow p (chi-square, 1e6 trials at V=5, K=2)."""
    oc.check_sd_statistics(orc, trials=1_000_000, configs=((5, 2),))
    oc.check_sd_statistics(orc, trials=200_000, configs=((2, 1), (3, 4), (8, 1)))


def test_expected_accepted_length(orc):
    oc.check_expected_length(orc, trials=1_000_000)


def test_tree_output_law_chi_square(orc):
    """Tree verification's emitted tokens follow the target (chi-square, depth-2 tree)."""
    oc.check_tree_statistics(orc, trials=200_000)


def test_particle_error_shrinks_like_inverse_sqrt_n(orc):
    """Weighted particles converge to the target at the 1/sqrt(N) rate."""
    oc.check_particle_l1_trend(orc)


def test_power_particles_converge_to_power_target(orc):
    """Power target: weighted (x_0, x_1) particles converge to p^beta at the 1/sqrt(N) rate."""
    oc.check_power_particle_trend(orc)

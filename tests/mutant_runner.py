"""Runs the oracle pins against one (mutated) oracle library, in a process of
its own: exit status 0 when every pin passes (the mutant survived), 1 when a
pin fails; a crash also ends the process with a non-zero status."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import oracle_checks as oc  # noqa: E402


def main(path):
    lib = oracle.load(path)
    for check in oc.DETERMINISTIC_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError, StopIteration, ZeroDivisionError, FloatingPointError, IndexError) as e:
            print(f"caught by {check.__name__}: {type(e).__name__} {str(e)[:200]}")
            return 1
    try:
        oc.check_sd_statistics(lib, trials=100_000, configs=((5, 2),))
        oc.check_expected_length(lib, trials=100_000)
    except AssertionError as e:
        print(f"caught by the statistics: {str(e)[:200]}")
        return 1
    print("survived")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))

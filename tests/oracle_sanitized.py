"""Runs every oracle pin against a sanitizer build of the oracle (argv[1]).
Started by tests/test_host.py in a subprocess with the address sanitizer's
runtime preloaded; any out-of-bounds access or undefined behaviour in the C
oracle aborts it."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import oracle_pins  # noqa: E402


def main() -> int:
    orc = oracle.Oracle(sys.argv[1])
    for pin in oracle_pins.ALL_PINS:
        pin(orc)
        print("ok", pin.__name__, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

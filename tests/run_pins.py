"""Run every oracle pin against one oracle library; exit 1 if any pin fails.

usage: python tests/run_pins.py /path/to/libpkv_oracle.so
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import oracle_pins  # noqa: E402


def main(path):
    orc = oracle.Oracle(path)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # a mutant may fail by assertion or by a rejected call
            failed.append(f"{pin.__name__}: {type(e).__name__}")
    print("FAILED:", ", ".join(failed) if failed else "none", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))

"""Runs every oracle pin against one oracle build given on the command line.

Exit status 0: all pins passed.  Exit status 1: some pin failed (the name of
the first failing pin is printed).  Used by the planted-mistake test, which
runs broken copies of the oracle in a child process so that a copy that
crashes cannot take the test session down.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import oracle_pins  # noqa: E402
import oracle_pool_pins  # noqa: E402


def main(path):
    lib = oracle.load(path)

    def topk(scores, k, lengths):
        return oracle.topk(scores, k, lengths, threads=2, lib=lib)

    def pool(scores, group, keep, pinned, lengths):
        return oracle.block_pool(scores, group, keep, pinned, lengths, lib=lib)

    def pooled(pool_scores, pool_idx, group, k, n, lengths):
        return oracle.pooled_topk(pool_scores, pool_idx, group, k, n, lengths, lib=lib)

    for pin, fn in [(p, topk) for p in oracle_pins.ALL_PINS] + \
                   [(p, pool) for p in oracle_pool_pins.POOL_PINS] + \
                   [(p, pooled) for p in oracle_pool_pins.POOLED_PINS]:
        try:
            pin(fn)
        except (AssertionError, oracle.OracleNaN, RuntimeError) as e:
            print(f"FAILED {pin.__name__}: {str(e)[:200]}")
            return 1
    print("ALL PINS PASSED")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))

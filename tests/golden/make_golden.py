"""Writes the stored expected values under tests/golden/ from the oracle only.

skip_sets.txt: the layer-skip draft's skip set (MLX layer-skip blog, "Code")
for the layer counts and skip fractions of the sweep workloads.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import skip_layers  # noqa: E402


def main():
    with open(os.path.join(HERE, "skip_sets.txt"), "w") as f:
        f.write("# n_layers skip_frac first_skipped last_skipped  (written by make_golden.py from oracle.skip)\n")
        for n in (4, 32, 36):
            for frac in (0.1, 0.2, 0.3, 0.4, 0.5):
                s = skip_layers(n, frac)
                f.write(f"{n} {frac} {s[0]} {s[-1]}\n")


if __name__ == "__main__":
    main()

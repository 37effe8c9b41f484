"""Write tests/golden/brute_force_sha256.txt: SHA-256 digests of the CPU oracle's
outputs over the two exhaustive row domains of tests/brute_domains.py (every row of
8 values over {0, +-0.5, +-1, +-2, 3}; every row of 16 values over {-1, 0, 1}), for
LayerNorm+modulate and RMSNorm+scale/shift with a weight, the modulation vectors
being seeded draws.  The values come from oracle/ alone.

    python tests/golden/make_brute_force_sha256.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from tests import brute_domains as D  # noqa: E402


def main():
    lines = ["# SHA-256 of the CPU oracle's bf16 outputs (row-major, little-endian halfwords)",
             "# over the exhaustive row domains of tests/brute_domains.py, rows in index order;",
             "# written by tests/golden/make_brute_force_sha256.py, which calls only oracle/.",
             "# domain op sha256"]
    for name in D.DOMAINS:
        d_ln, d_rms, _ = D.oracle_digests(name, check=False)
        lines += [f"{name} ln {d_ln}", f"{name} rms {d_rms}"]
        print(name, d_ln, d_rms, flush=True)
    path = os.path.join(ROOT, "tests", "golden", "brute_force_sha256.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()

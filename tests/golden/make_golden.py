"""Write tests/golden/codebooks.json from the CPU oracle (and nothing else).

The fp32 Lloyd-Max tables are stored as raw IEEE bit patterns so a later change
of the oracle's codebook arithmetic shows up as a failing regression test.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import ref  # noqa: E402


def main():
    tables = {}
    for d in (8, 16, 32, 64, 128):
        for bits in (1, 2, 3, 4):
            c, t, _ = ref.codebook(d, bits)
            tables[f"{d},{bits}"] = {
                "centroid_bits": [int(v) for v in c.view("uint32")],
                "threshold_bits": [int(v) for v in t.view("uint32")],
                "centroid": [float(v) for v in c],
            }
    out = {"_about": "fp32 sphere-marginal Lloyd-Max tables written by make_golden.py from oracle/ only",
           "tables": tables}
    with open(os.path.join(HERE, "codebooks.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()

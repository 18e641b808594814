"""Writes tests/golden/unmasked_pairs.json from the oracle alone.

The stored numbers are the block-causal mask areas per query head of the five
benchmark layouts: the area that the forward FLOP count is taken over
(MAGI-1 paperlayer summary §B.2.1: forward FLOPs are two matrix products over
the mask area, following Flash-Attention). Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def main():
    pairs = {c.name: oracle.unmasked_pairs(c.layout) for c in CONFIGS}
    doc = {
        "source": "oracle.unmasked_pairs over the dense block-causal mask (tests/golden/make_golden.py)",
        "citation": "MAGI-1 paperlayer summary §B.2.1 (FLOPs over the mask area); paperlayer §2 / Figure 1 (mask)",
        "pairs_per_head": pairs,
    }
    with open(os.path.join(os.path.dirname(__file__), "unmasked_pairs.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(json.dumps(pairs))


if __name__ == "__main__":
    main()

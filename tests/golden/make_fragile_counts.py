"""Write tests/golden/fragile_counts.json: the number of fragile commit decisions
(within 1e-4 of a tie in the oracle's fp64 values; see tests/acceptance.py) in
the first step and in the whole block loop of configs 1, 2, 3 and 5.  Calls only
the oracle and the seeded input generator.

    python tests/golden/make_fragile_counts.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import acceptance  # noqa: E402

CONFIGS = (1, 2, 3, 5)


def main():
    out = {"rule": "fragile = within 1e-4 of a tie in the oracle's fp64 confidences; excluded = rank | tau "
                   "(tests/acceptance.py)",
           "configs": {str(c): acceptance.summarize(c) for c in CONFIGS}}
    path = os.path.join(HERE, "fragile_counts.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out, indent=1, sort_keys=True))


if __name__ == "__main__":
    main()

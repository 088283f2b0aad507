"""Write oracle_tiny.json from the CPU oracle (and nothing else).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from swa_inputs import PrefillConfig, prefill_inputs  # noqa: E402

CASES = [
    PrefillConfig("golden_swa", 1, 12, 2, 1, 4, 3, "f32", seed=101),
    PrefillConfig("golden_ga", 1, 9, 4, 2, 4, 0, "f32", seed=102, Sk=11),
]


def main():
    out = {}
    for cfg in CASES:
        q, k, v, sinks = prefill_inputs(cfg)
        o = oracle.prefill(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale)
        out[cfg.name] = {"config": cfg.__dict__, "o": o.round(15).tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()

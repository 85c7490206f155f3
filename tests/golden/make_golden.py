"""Write the oracle's outputs on the tiny fp32 head (B=1, d=256, V=4096, r=32,
k=8) to ``c1_oracle.json``. Calls only ``gen`` (inputs) and ``oracle``.

The EAGLE-4 pages print no worked numeric example of the head, so this file
is a regression snapshot of the oracle, not a value from the pages.
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import gen      # noqa: E402
import oracle   # noqa: E402


def main() -> None:
    inp = gen.make(1)
    lr = oracle.lowrank_head(inp["Q"], inp["P"], inp["W"], inp["H"], 8, "fp32")
    fh = oracle.full_head(inp["W"], inp["H"], 8, "fp32")
    snap = {
        "config": "tiny fp32 head: B=1, d=256, V=4096, r=32, k=8, seed 1001",
        "lowrank_idx": lr["idx"].tolist(),
        "lowrank_score": lr["score"].tolist(),
        "lowrank_logits": lr["logits"].tolist(),
        "gap": lr["gap"].tolist(), "tau": lr["tau"].tolist(),
        "full_idx": fh["idx"].tolist(),
        "full_logits": fh["logits"].tolist(),
    }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_oracle.json")
    with open(out, "w") as f:
        json.dump(snap, f, indent=1)


if __name__ == "__main__":
    main()

"""Screen seeds of the 4096-token prefill routing workload (Zipf logit bias)
for near ties at the top-8 boundary, using the oracle only.

A token whose exact 8th and 9th largest logits differ by less than the
fp32 accumulation error of the GPU router could legitimately be routed
either way.  The parity tests bound that error by 2e-5 (they assert it);
a seed is kept when every token's 8th/9th gap exceeds 4e-5, so that no
routing decision of a kept seed can flip.

Writes prefill_seeds.json next to this file:
    python tests/golden/screen_prefill_seeds.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

GAP = 4e-5
WEIGHT_SEED = 0


def main():
    w = synth.moe_weights(WEIGHT_SEED)
    rows = []
    for seed in range(40):
        tok = synth.moe_tokens(seed, 4096, skewed=True)
        L = oracle.router_logits(tok["H"], w["Wr"], tok["logit_bias"])
        srt = -np.sort(-L, axis=1)
        gap = float((srt[:, 7] - srt[:, 8]).min())
        rows.append((seed, gap))
    kept = sorted([s for s, g in rows if g > GAP], key=lambda s: -dict(rows)[s])
    out = {
        "source": "written by tests/golden/screen_prefill_seeds.py from the oracle only",
        "weight_seed": WEIGHT_SEED,
        "tokens": 4096,
        "min_gap_required": GAP,
        "kept_seeds_by_gap": kept,
        "min_gap_per_seed": {str(s): g for s, g in rows},
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "prefill_seeds.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("kept", kept)


if __name__ == "__main__":
    main()

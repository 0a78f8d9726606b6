"""Screen seeds of the 4096-token prefill routing workload (Zipf logit bias)
for near ties, using the oracle only.

A token whose exact 8th and 9th largest logits differ by less than the
fp32 accumulation error of the GPU router could legitimately be routed
either way.  Two lists are written:

* kept_seeds_by_gap (seeds 0..39): every token's 8th/9th gap exceeds 4e-5;
  the parity tests assert the fp32 logit error stays below 2e-5, so no
  token's expert set can differ from the oracle's;
* kept_seeds_full_order (seeds 0..199): every gap between adjacent logits
  among each token's 9 largest exceeds 2e-5; the tests that use these seeds
  assert an fp32 logit error below 1e-5, so neither the set nor the order
  of any token's experts (which fixes the ids, the permutation and its
  inverse) can differ from the oracle's.

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
GAP_FULL = 2e-5
WEIGHT_SEED = 0
SEEDS_BOUNDARY = 40
SEEDS_FULL = 200


def main():
    w = synth.moe_weights(WEIGHT_SEED)
    rows, full = [], []
    for seed in range(SEEDS_FULL):
        tok = synth.moe_tokens(seed, 4096, skewed=True)
        L = oracle.router_logits(tok["H"], w["Wr"], tok["logit_bias"])
        srt = -np.sort(-L, axis=1)[:, :9]
        if seed < SEEDS_BOUNDARY:
            rows.append((seed, float((srt[:, 7] - srt[:, 8]).min())))
        full.append((seed, float((srt[:, :8] - srt[:, 1:9]).min())))
    kept = sorted([s for s, g in rows if g > GAP], key=lambda s: -dict(rows)[s])
    kept_full = sorted([s for s, g in full if g > GAP_FULL], key=lambda s: -dict(full)[s])
    out = {
        "source": "written by tests/golden/screen_prefill_seeds.py from the oracle only",
        "weight_seed": WEIGHT_SEED,
        "tokens": 4096,
        "min_gap_required": GAP,
        "kept_seeds_by_gap": kept,
        "min_gap_per_seed": {str(s): g for s, g in rows},
        "min_gap_full_order_required": GAP_FULL,
        "kept_seeds_full_order": kept_full,
        "min_gap_full_order_per_kept_seed": {str(s): g for s, g in full if g > GAP_FULL},
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "prefill_seeds.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("kept", kept)
    print("kept (full order)", kept_full)


if __name__ == "__main__":
    main()

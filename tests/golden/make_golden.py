"""Writes tests/golden/tiny_fp32_L512.json: the oracle's results for a small seeded fp32 case
(one sequence of 512 raw tokens, 4 decode queries at t = 508..511, 4 heads, D = 32 + 16,
CSA m = 4, w = 8, top-k 16, HCA m' = 32, window 16; indexer 4 heads x 64).

The pages print no worked example, so this fixture is a regression pin of the oracle itself
(tests/test_oracle_golden.py) and a second, stored reference for the GPU library
(tests/test_gpu_golden.py). It calls only oracle/ and the seeded generators in synth/:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import indexer, pipeline  # noqa: E402

PARAMS = dict(seed=2024, L=512, n_queries=4, heads=4, d_nope=32, d_rope=16, m=4, w=8, topk=16,
              n_idx_heads=4, d_idx=64, m_prime=32, W=16)
PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_L512.json")


def case():
    return synth.tiny_fp32(**PARAMS)


def well_separated(c):
    """Every query's k-th and (k+1)-th indexer scores differ by more than 1e-3 of the largest
    score, so float32 scoring on the GPU cannot reorder them."""
    p, a = c.params, {k: v.numpy().astype(np.float64) for k, v in c.t.items()}
    for i, t in enumerate(c.t["q_pos"].tolist()):
        n = indexer.n_visible(t, p["m"])
        if n <= p["topk"]:
            continue
        s = np.sort(indexer.scores(a["q_idx"][i], a["w_idx"][i], a["k_idx"][:n]))[::-1]
        if s[p["topk"] - 1] - s[p["topk"]] <= 1e-3 * np.abs(s).max():
            return False
    return True


def compute():
    c = case()
    a = {k: v.numpy() for k, v in c.t.items()}
    r = pipeline.tiny_fp32(c.params, a)
    return {
        "params": PARAMS,
        "idx": [np.asarray(i).tolist() for i in r["idx"]],
        "csa_entries_first4": np.asarray(r["y_csa"][:4]).tolist(),
        "hca_entries_first2": np.asarray(r["y_hca"][:2]).tolist(),
        "o_csa": np.asarray(r["o_csa"]).tolist(),
        "lse_csa": np.asarray(r["lse_csa"]).tolist(),
        "o_hca": np.asarray(r["o_hca"]).tolist(),
        "lse_hca": np.asarray(r["lse_hca"]).tolist(),
    }


if __name__ == "__main__":
    while not well_separated(case()):
        PARAMS["seed"] += 1
    with open(PATH, "w") as f:
        json.dump(compute(), f, indent=0, sort_keys=True)
    print("wrote", PATH)

"""Writes oracle_small.json: a regression fixture of the CPU oracle.

Calls only the oracle and the shared input generator. Rerun after a change to
the oracle's arithmetic that a passage of the pages justifies, and name that
passage in the commit.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synthgen  # noqa: E402


def main():
    w = {"lengths": [300, 97, 1], "Hq": 8, "Hkv": 2, "d": 128, "K": 48, "W": 16, "seed": 4242}
    T = sum(w["lengths"])
    cu = np.concatenate([[0], np.cumsum(w["lengths"])]).astype(np.int32)
    q = synthgen.normal_bf16(w["seed"], 1, (T, w["Hq"], w["d"]))
    k = synthgen.normal_bf16(w["seed"], 2, (T, w["Hkv"], w["d"]))
    v = synthgen.normal_bf16(w["seed"], 3, (T, w["Hkv"], w["d"]))
    idx, kth = oracle.select(q, k, cu, w["Hq"], w["Hkv"], w["K"], w["W"])
    o64, _ = oracle.sparse_attn(q, k, v, cu, w["Hq"], w["Hkv"], idx.reshape(T, w["Hkv"], -1))
    rows = [0, 1, 63, 64, 65, 200, 399, 400, 599, 600, 700, 795]
    out = {
        "workload": w,
        "idx_rows": {str(r): idx[r].tolist() for r in rows},
        "kth": {str(r): float(kth[r]) for r in rows},
        "o_token_sums": o64.sum(axis=(1, 2)).tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print("wrote", path)


if __name__ == "__main__":
    main()

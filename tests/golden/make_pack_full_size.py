"""Writes pack_full_size.json: SHA-256 digests of the oracle's packed
qweight, scales and qzeros (little-endian bytes, row-major) for whole
sweep-shaped groups packed with the oracle's chosen scale row: the MLP
gate/up pair (24576 x 4096, G = 128) and down_proj (4096 x 12288, G = 64) of
tests/golden/make_weight_score_full_size.py, symmetric and asymmetric.
A GPU pack of the same inputs must hash to the same digests (bit-exact codes,
fp16 scales and zero points over every weight).  Calls only oracle/ and the
seeded input generators.

    python3 tests/golden/make_pack_full_size.py
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import awq_oracle as O  # noqa: E402
from make_weight_score_full_size import CASES, inputs  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main() -> None:
    out = {"about": "sha256 of oracle.quantize_pack(_asym)(W, S[k], G) outputs, W the concatenated parts and "
                    "S[k] the oracle's chosen weight-score candidate; written by make_pack_full_size.py",
           "cases": []}
    for rows, d_in, G in CASES:
        t0 = time.time()
        parts, X = inputs(rows, d_in)
        xm = O.act_stats(X)
        _, k, s = O.search_scales(parts, xm, G, 20)
        W = np.concatenate(parts, axis=0)
        for asym in (False, True):
            qw, sc, qz = (O.quantize_pack_asym(W, s, G) if asym else O.quantize_pack(W, s, G))[:3]
            out["cases"].append({"rows": rows, "d_in": d_in, "group_size": G, "asym": asym, "best_idx": int(k),
                                 "qweight": digest(qw.astype("<u4")), "scales": digest(sc.astype("<f2")),
                                 "qzeros": digest(qz.astype("<u4"))})
        print(f"rows {rows} d_in {d_in} G {G}: {time.time() - t0:.0f} s", flush=True)
    with open(os.path.join(HERE, "pack_full_size.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

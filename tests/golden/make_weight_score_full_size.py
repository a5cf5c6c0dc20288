"""Writes weight_score_full_size.json: the oracle's weight-score errors of the
20 alpha candidates over every row of two sweep-shaped groups, the MLP
gate/up pair (2 x 12288 x 4096, G = 128) and down_proj (4096 x 12288,
G = 64), on the seeded inputs the sweep-shape test draws (2048 calibration
tokens, bf16), and the gate/up pair again with duo scaling and with
asymmetric INT4.  Calls only oracle/ (act_stats, search_scales) and the seeded
input generators.

    python3 tests/golden/make_weight_score_full_size.py
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import awq_oracle as O  # noqa: E402
import workloads as WL  # noqa: E402

# (rows of the parts, d_in, group size): the shapes of one sweep block's gate/up and down
CASES = [([12288, 12288], 4096, 128), ([4096], 12288, 64)]
# the gate/up shape again with duo scaling and with asymmetric INT4: (case, duo, asym)
VARIANTS = [(CASES[0], True, False), (CASES[0], False, True)]


def inputs(rows, d_in):
    """The parts and calibration input of tests/test_gpu_full_size.py's sweep-shape test."""
    parts = [WL.make_weight(9100 + 31 * i + d_in, r, d_in) for i, r in enumerate(rows)]
    X = WL.make_activations(9200 + d_in, 2048, d_in, "bf16")
    return parts, X


def main() -> None:
    out = {"about": "oracle.search_scales(score='weight', n_grid=20) over every row of the sweep-shape test's "
                    "seeded parts and inputs; written by make_weight_score_full_size.py", "cases": []}
    for (rows, d_in, G), duo, asym in [(c, False, False) for c in CASES] + VARIANTS:
        t0 = time.time()
        parts, X = inputs(rows, d_in)
        xm = O.act_stats(X)
        errs, k, _ = O.search_scales(parts, xm, G, 20, duo=duo, asym=asym)
        out["cases"].append({"rows": rows, "d_in": d_in, "group_size": G, "duo": duo, "asym": asym,
                             "tokens": int(X.shape[0]), "errors": [float(e) for e in errs], "best_idx": int(k)})
        print(f"rows {rows} d_in {d_in} G {G} duo={duo} asym={asym}: best {k}, {time.time() - t0:.0f} s",
              flush=True)
    with open(os.path.join(HERE, "weight_score_full_size.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

"""Writes output_score_full_size.json: the oracle's output-score errors of the
20 alpha candidates for the fused QKV group (6144 x 4096, 16384 tokens; plain,
with duo scaling and with asymmetric INT4) and the MLP gate/up group
(2 x 12288 x 4096, 16384 tokens) at their full calibration sizes, G = 128, on
the seeded inputs of the workloads module.

Calls only oracle/ (act_stats, search_scales) and the seeded input
generators; the down projection is left out because its input is a float32
matrix product whose bits depend on the host's BLAS.  Takes a few minutes
(about 4 TFLOP of fp64 products per candidate set).

    python3 tests/golden/make_output_score_full_size.py
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import awq_oracle as O  # noqa: E402
import workloads as WL  # noqa: E402

# (workload, group, duo scaling, asymmetric INT4)
CASES = [("qkv_6144x4096_output", 0, False, False), ("mlp_output_clip", 0, False, False),
         ("qkv_6144x4096_output", 0, True, False), ("qkv_6144x4096_output", 0, False, True)]


def main() -> None:
    out = {"about": "oracle.search_scales(score='output', n_grid=20, G=128, duo, asym) over every row and token of "
                     "workloads.host_group_inputs(WORKLOADS[workload], 0, group); written by "
                     "make_output_score_full_size.py", "cases": []}
    for name, gi, duo, asym in CASES:
        wl = WL.WORKLOADS[name]
        t0 = time.time()
        parts, X = WL.host_group_inputs(wl, 0, gi)
        xm = O.act_stats(X)
        errs, k, _ = O.search_scales(parts, xm, 128, 20, "output", X=X, duo=duo, asym=asym)
        out["cases"].append({"workload": name, "group": gi, "group_size": 128, "duo": duo, "asym": asym,
                             "rows": [int(p.shape[0]) for p in parts], "d_in": int(X.shape[1]),
                             "tokens": int(X.shape[0]), "errors": [float(e) for e in errs], "best_idx": int(k)})
        print(f"{name} group {gi} duo={duo} asym={asym}: best {k}, {time.time() - t0:.0f} s", flush=True)
    with open(os.path.join(HERE, "output_score_full_size.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

"""Writes pair_counts.json: the attended block-0 pair count P0 of every
workload, computed by the CPU oracle's row-by-row visibility rule. It calls
only the oracle and the seeded workload definitions; rerun it if a workload
definition changes."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth   # noqa: E402


def main():
    res = {}
    for name in synth.WORKLOADS:
        w = synth.workload(name)
        res[name] = {
            "layout": w.layout, "S": w.S, "T": w.T, "cp": w.cp, "rank": w.rank,
            "doc_lens": w.doc_lens,
            "P0": oracle.pair_count(w.layout, w.T, w.cp, w.rank, w.cu_seqlens()),
        }
    with open(os.path.join(HERE, "pair_counts.json"), "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

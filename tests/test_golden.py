"""Stored pair counts agree with closed forms and with the oracle."""
import json
import os

import oracle
import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load():
    with open(os.path.join(HERE, "pair_counts.json")) as f:
        return json.load(f)


def test_pair_counts_closed_forms():
    g = load()
    assert g["tiny"]["P0"] == 256 * 257 // 2
    assert g["dense"]["P0"] == 4096 * 4097 // 2
    assert g["ulysses"]["P0"] == 4 * (8192 * 8193 // 2)
    c = 8192
    assert g["zigzag"]["P0"] == 2 * 8 * c * c + c == 1_073_750_016
    lens = g["packed"]["doc_lens"]
    assert sum(lens) == 16384 and all(1 <= n <= 4096 for n in lens)
    assert all(256 <= n for n in lens[:-1])
    assert g["packed"]["P0"] == sum(n * (n + 1) // 2 for n in lens)


def test_pair_counts_match_current_workloads():
    g = load()
    for name in synth.WORKLOADS:
        w = synth.workload(name)
        assert g[name]["doc_lens"] == w.doc_lens
        assert g[name]["P0"] == oracle.pair_count(w.layout, w.T, w.cp, w.rank, w.cu_seqlens())

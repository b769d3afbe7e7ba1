"""Seeded random shapes on the GPU against the CPU oracle: lengths that are not
multiples of any tile size, both head dims and dtypes, batch rows, random
document splits (empty and one-row documents included) and every layout with
random degree and rank. Same tolerances as the fixed parity cases."""
import random

import pytest

import synth
from tests.parity import assert_within, compare, inputs, run_hip, run_oracle, say

pytestmark = pytest.mark.gpu

N_CASES = 32


def _docs(rng, total):
    lens, acc = [], 0
    while acc < total:
        n = rng.choice([0, 1, rng.randint(1, 64), rng.randint(32, 400)])
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def _zigzag_docs(rng, cp, ndocs):
    """Document lengths that are multiples of 2cp (some empty, some one chunk row)."""
    return [2 * cp * rng.choice([0, 1, rng.randint(1, 8), rng.randint(5, 60)]) for _ in range(ndocs)]


def fuzz_case_docs(i):
    """Cases 24..31: zig-zag shares of several documents, every degree and rank."""
    rng = random.Random(5000 + i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    D = rng.choice([64, 128])
    cp = rng.randint(1, 4)
    lens = _zigzag_docs(rng, cp, rng.randint(2, 6))
    if sum(lens) == 0:
        lens[0] = 2 * cp
    return synth.small_workload(f"fuzz{i}", dtype=dtype, D=D, H=rng.randint(1, 4),
                                num_blocks=rng.randint(1, 9), seed=i, layout="zigzag",
                                S=sum(lens), cp=cp, rank=rng.randrange(cp), doc_lens=lens)


def fuzz_case(i):
    if i >= 24:
        return fuzz_case_docs(i)
    rng = random.Random(1000 + i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    D = rng.choice([64, 128])
    H = rng.randint(1, 3) if i < 12 else rng.randint(1, 6)
    nb = rng.randint(1, 5) if i < 12 else rng.randint(1, 9)
    layout = ["full", "full", "headshard", "contiguous", "zigzag"][i % 5]
    kw = dict(dtype=dtype, D=D, H=H, num_blocks=nb, seed=i, layout=layout)
    if layout == "zigzag":
        cp = rng.randint(1, 4)
        c = rng.randint(17, 150)                       # chunk rows
        kw.update(S=2 * cp * c, cp=cp, rank=rng.randrange(cp))
    elif layout == "contiguous":
        cp = rng.randint(1, 4)
        t = rng.randint(33, 300)
        kw.update(S=cp * t, cp=cp, rank=rng.randrange(cp), chunk=t)
        if rng.random() < 0.5:
            kw["doc_lens"] = _docs(rng, cp * t)
    elif layout == "headshard":
        cp = rng.randint(1, 4)
        S = cp * rng.randint(40, 200)
        kw.update(S=S, cp=cp, rank=rng.randrange(cp), doc_lens=_docs(rng, S))
    else:
        S = rng.randint(1, 700)
        if rng.random() < 0.5:
            kw.update(S=S, doc_lens=_docs(rng, S))
        else:
            kw.update(S=S, B=rng.randint(1, 2))
    return synth.small_workload(f"fuzz{i}", **kw)


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_parity(i):
    w = fuzz_case(i)
    say(f"[fuzz] {i}: {w}")
    inp = inputs(w)
    hip = run_hip(w, inp)
    ref = run_oracle(w, inp)
    m = compare(w, hip, ref)
    say(f"[fuzz] {i}: {m}")
    assert_within(w, m)

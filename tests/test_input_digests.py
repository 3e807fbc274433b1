"""The seeded input recipe reproduces the recorded tensors: the SHA-256 of
every tensor each workload draws with the CPU generator at seed 0 matches
tests/golden/input_sha256.json (written by make_input_sha256.py beside it).
A failure means torch's random stream or the recipe changed, so every
stored expectation drawn from these inputs must be looked at again."""
import json
import os

import pytest

from dilated_sparse_attention_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "input_sha256.json")
WORKLOADS = [(w, inputs.make_prefill) for w in inputs.PREFILL_WORKLOADS] + \
            [(w, inputs.make_decode) for w in inputs.DECODE_WORKLOADS]


@pytest.mark.parametrize("case", WORKLOADS, ids=lambda c: c[0].name)
def test_input_sha256(case):
    w, make = case
    with open(GOLDEN) as f:
        want = json.load(f)["workloads"][w.name]
    got = inputs.sha256_of(make(w, seed=0))
    assert got == want


def test_digest_sees_one_flipped_bit():
    x = inputs.make_prefill(inputs.TINY_FP32, seed=0)
    a = inputs.sha256_of(x)
    x["k"].view(-1)[17] = -x["k"].view(-1)[17]
    b = inputs.sha256_of(x)
    assert a["q"] == b["q"] and a["k"] != b["k"]

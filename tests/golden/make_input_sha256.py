"""Write input_sha256.json: the SHA-256 of every tensor the seed-0 recipe of
each workload draws (dilated_sparse_attention_amd.inputs, CPU generator), so
that a change in torch's random stream shows up as a failed digest check
rather than as silently different inputs.  Run from the repository root:

    python3 tests/golden/make_input_sha256.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from dilated_sparse_attention_amd import inputs  # noqa: E402


def main():
    out = {"torch_generator": "torch.Generator('cpu'), seed 0", "workloads": {}}
    for w in inputs.PREFILL_WORKLOADS:
        out["workloads"][w.name] = inputs.sha256_of(inputs.make_prefill(w, seed=0))
    for w in inputs.DECODE_WORKLOADS:
        out["workloads"][w.name] = inputs.sha256_of(inputs.make_decode(w, seed=0))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_sha256.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()

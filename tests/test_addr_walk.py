"""Host walk of the kernels' global addresses (no GPU): the history-writing
scan's stores and final state, the raw-ring fill, the band pass's and the
dilated kernel's ring copies (history and plain layouts), their (m, l) side
loads and output rows, over whole launch grids of the one-call layer
prefill's cases and the full-size workloads.  The harness calls the same
address functions the kernels call (csrc/rat_plan.h), compiled for the host,
and fails on any access outside its buffer; a planted undersized history
must be caught."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "harness", "addr_walk.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def walker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    exe = str(tmp_path_factory.mktemp("addr") / "addr_walk")
    subprocess.run([HIPCC, "-std=c++17", "-O2", "--cuda-host-only", "-x", "hip",
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "dilated_sparse_attention_amd", "csrc"), SRC, "-o", exe],
                   check=True, capture_output=True)
    return exe


def history_rows(T, D):
    return max(Dh * ((T - 1) // Dh + 1) for Dh in D)


def run(exe, B, T, H, d, L, mode, dtype, n_cap, w_cap, fin, D, W):
    args = [exe] + [str(x) for x in (B, T, H, d, L, mode, dtype, n_cap, w_cap, int(fin))]
    args += [",".join(map(str, D)), ",".join(map(str, W))]
    return subprocess.run(args, capture_output=True, text=True, timeout=300)


# the one-call layer prefill's parity cases: (B, T, H, d, D, W, L, mode, bf16)
LAYER_CASES = [
    (1, 300, 3, 128, [1, 4, 16], [0, 8, 0], None, 0, 1),
    (2, 257, 2, 64, [16, 7], [16, 5], 64, 0, 1),
    (1, 700, 2, 128, [64, 20], [128, 33], 64, 1, 1),
    (1, 200, 2, 64, [3, 5], [0, 4], 50, 1, 1),
    (1, 2048, 4, 128, [1, 1, 64, 64], [0, 0, 256, 256], None, 0, 1),
    (1, 40, 2, 128, [64, 100], [0, 3], None, 0, 1),
    (2, 1, 2, 128, [1, 16], [4, 0], None, 0, 1),
    (1, 256, 2, 64, [4, 4], [0, 0], None, 0, 0),
    (2, 1000, 4, 128, [16, 16, 1, 64], [0, 64, 0, 128], None, 0, 1),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}D{c[4]}W{c[5]}")
def test_layer_prefill_addresses(walker, case):
    B, T, H, d, D, W, L, mode, dtype = case
    n_cap = history_rows(T, D) + 2 * max(D)
    w_cap = max(W) + 3 if any(W) else 0
    r = run(walker, B, T, H, d, T if L is None else L, mode, dtype, n_cap, w_cap, mode == 0, D, W)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK" in r.stdout


WORKLOADS = [
    # (B, T, H, d, D, W, L): the 1.5B, long and 7.6B hybrid prefill shapes
    (4, 4096, 16, 128, [16] * 16, [0] * 16, 4096),
    (1, 16384, 16, 128, [64] * 16, [128] * 16, 64),
    (1, 32768, 32, 128, [1] * 8 + [64] * 24, [0] * 8 + [256] * 24, 32768),
]


@pytest.mark.parametrize("history", [False, True])
@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: f"T{w[1]}H{w[2]}")
def test_full_size_addresses(walker, w, history):
    B, T, H, d, D, W, L = w
    n_cap = history_rows(T, D) if history else 0
    r = run(walker, B, T, H, d, L, 0, 1, n_cap, max(W), True, D, W)
    assert r.returncode == 0, r.stdout + r.stderr


def test_walk_catches_an_undersized_history(walker):
    """A history of 200 rows where D = 16 needs 304 at T = 300: the walk
    reports the stores past its end."""
    r = run(walker, 1, 300, 3, 128, 300, 0, 1, 200, 11, True, [1, 4, 16], [0, 8, 0])
    assert r.returncode == 1 and "out of range" in r.stdout

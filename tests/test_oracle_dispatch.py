"""Pins for the oracle's dispatch (CPU only): a hand-worked example, a library
stable sort as an independent construction, and the pool invariants."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_tiny():
    d = {}
    with open(os.path.join(GOLDEN, "dispatch_tiny.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line and not line.startswith("T="):
                k, *v = line.split()
                d[k] = np.array([int(x) for x in v], dtype=np.int64)
    return d


def test_dispatch_hand_worked_example():
    g = _load_tiny()
    r = oracle.route(g["topk_idx"].reshape(4, 2), 3)
    for key in ("count", "offset", "src", "pos"):
        assert np.array_equal(r[key], g[key]), key
    assert r["num_invalid"] == int(g["num_invalid"][0])


def _by_stable_sort(idx, E):
    """Independent construction: a stable library sort of pair ids by expert id."""
    flat = idx.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    pairs = np.nonzero(valid)[0]
    order = np.argsort(flat[pairs], kind="stable")
    src = pairs[order]
    count = np.bincount(flat[pairs], minlength=E)
    return src, count


def check_invariants(idx, E, r):
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    n_valid = int(valid.sum())
    assert r["count"].sum() == n_valid
    assert np.array_equal(np.diff(r["offset"]), r["count"])
    assert r["offset"][0] == 0 and r["offset"][-1] == n_valid
    # each valid pair exactly once
    assert np.array_equal(np.sort(r["src"]), np.nonzero(valid)[0])
    # pos is the inverse of src, -1 elsewhere
    assert np.array_equal(r["pos"][r["src"]], np.arange(n_valid))
    assert np.all(r["pos"][~valid] == -1)
    for e in range(E):
        seg = r["src"][r["offset"][e]:r["offset"][e + 1]]
        assert np.all(np.diff(seg) > 0)                    # stable row-major order
        assert np.all(flat[seg] == e)
    assert r["num_invalid"] == int((flat >= E).sum())


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_dispatch_configs_match_stable_sort(cfg):
    spec = synth.CONFIGS[cfg]
    idx, _ = synth.make_routing(spec)
    idx = idx.numpy()
    r = oracle.route(idx, spec.E)
    src, count = _by_stable_sort(idx, spec.E)
    assert np.array_equal(r["src"], src)
    assert np.array_equal(r["count"], count)
    check_invariants(idx, spec.E, r)
    assert r["count"].sum() == spec.T * spec.k         # configs never mask


@pytest.mark.parametrize("case", ["one_expert", "empty_T", "T1", "E1", "k1", "masked_invalid", "skewed"])
def test_dispatch_edge_cases(case):
    rng = np.random.default_rng(5)
    if case == "one_expert":
        E, idx = 16, np.full((37, 4), 9)
    elif case == "empty_T":
        E, idx = 8, np.zeros((0, 2), dtype=np.int64)
    elif case == "T1":
        E, idx = 8, np.array([[3, 1]])
    elif case == "E1":
        E, idx = 1, np.zeros((13, 1), dtype=np.int64)
    elif case == "k1":
        E, idx = 5, rng.integers(0, 5, (29, 1))
    elif case == "masked_invalid":
        E, idx = 6, rng.integers(-2, 9, (41, 3))
    else:
        E, idx = 32, np.minimum(rng.zipf(1.5, (300, 4)) - 1, 31)
    r = oracle.route(idx, E)
    src, count = _by_stable_sort(idx, E)
    assert np.array_equal(r["src"], src)
    assert np.array_equal(r["count"], count)
    check_invariants(idx, E, r)

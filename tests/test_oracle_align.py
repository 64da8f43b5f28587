"""Pins for the oracle's align step (stable group-by-expert, per-expert padding)."""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(ids, E, bm):
    T, k = ids.shape
    A = T * k
    flat = [(int(ids[a // k, a % k]), a) for a in range(A)]
    out, be = [], []
    for e in range(E):
        group = [a for (ee, a) in flat if ee == e]     # ascending a
        while len(group) % bm:
            group.append(A)
        be += [e] * (len(group) // bm)
        out += group
    return out, be


@pytest.mark.parametrize("T,k,E,bm", [(64, 2, 8, 16), (33, 8, 128, 32), (7, 10, 512, 16),
                                      (100, 3, 5, 64), (1, 8, 128, 16)])
def test_matches_brute_force(orc, T, k, E, bm):
    rng = np.random.default_rng(T + k + E + bm)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)   # duplicates allowed
    s, be, n = orc.align(ids, E, bm)
    bs, bbe = _brute(ids, E, bm)
    assert list(s) == bs and list(be) == bbe and n == len(bs)


def test_invariants(orc):
    rng = np.random.default_rng(7)
    T, k, E, bm = 333, 8, 128, 32
    ids = rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)   # some invalid
    s, be, n = orc.align(ids, E, bm)
    A = T * k
    valid = [(a, int(ids[a // k, a % k])) for a in range(A) if 0 <= ids[a // k, a % k] < E]
    got = [a for a in s if a != A]
    assert sorted(got) == [a for a, _ in valid]              # each valid once, invalid never
    counts = np.bincount([e for _, e in valid], minlength=E)
    assert n == int(sum(-(-c // bm) * bm for c in counts))
    assert n % bm == 0 and len(be) == n // bm
    for b in range(n // bm):                                  # block -> expert is right
        blk = s[b * bm:(b + 1) * bm]
        real = [a for a in blk if a != A]
        assert all(ids[a // k, a % k] == be[b] for a in real)
        assert list(blk[:len(real)]) == real                  # sentinels only at the tail
    assert list(be) == sorted(be)


def test_empty_and_all_invalid(orc):
    ids = np.full((4, 2), -1, dtype=np.int32)
    s, be, n = orc.align(ids, 8, 16)
    assert n == 0 and s.size == 0 and be.size == 0
    s, be, n = orc.align(np.zeros((0, 8), dtype=np.int32), 8, 16)
    assert n == 0


def test_replay_slice_stride_and_equal_to_contiguous(orc):
    g = json.load(open(os.path.join(GOLDEN, "prime_rl_routed_experts_slice.json")))
    L, k = g["layers"], g["top_k"]
    T = 50
    rng = np.random.default_rng(8)
    full = rng.integers(0, 128, size=(1, T, L, k)).astype(np.int32)
    sl = full[:, :, 7, :][0]
    assert sl.strides[0] // sl.itemsize == g["slice_token_stride"] == L * k
    a = orc.align(sl, 128, 32)
    b = orc.align(np.ascontiguousarray(sl), 128, 32)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all() and a[2] == b[2]

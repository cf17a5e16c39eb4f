"""Pins of the oracle's dispatch layout: a brute-force sort of (expert,
token) pairs written with Python's sorted(), the invariants every
expert-major permutation must satisfy, and the tile count by enumeration."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def brute_layout(ids, e_lo, E_L):
    T, k = ids.shape
    pairs = [(int(ids[t, s]) - e_lo, t, s) for t in range(T) for s in range(k)
             if 0 <= int(ids[t, s]) - e_lo < E_L]
    pairs = sorted(pairs)          # by (local expert, token, slot)
    counts = [0] * E_L
    for e, _, _ in pairs:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    tsr = np.full((T, k), -1)
    for j, (_, t, s) in enumerate(pairs):
        tsr[t, s] = j
    return (np.array(counts), np.array(offsets), np.array([p[1] for p in pairs]),
            np.array([p[2] for p in pairs]), tsr)


def random_ids(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("T,E,k,e_lo,E_L", [
    (50, 8, 2, 0, 8), (64, 16, 4, 4, 8), (33, 32, 8, 24, 8), (10, 6, 6, 0, 1),
    (1, 8, 3, 5, 3), (0, 8, 2, 0, 8), (40, 64, 8, 60, 4)])
def test_layout_matches_sorted_pairs(seed, T, E, k, e_lo, E_L):
    rng = np.random.default_rng(seed)
    ids = random_ids(rng, T, E, k) if T else np.zeros((0, k), np.int32)
    got = O.index_build(ids, e_lo, E_L)
    c, o, rt, rs, tsr = brute_layout(ids, e_lo, E_L)
    np.testing.assert_array_equal(got["counts"], c)
    np.testing.assert_array_equal(got["offsets"], o)
    np.testing.assert_array_equal(got["row_token"], rt)
    np.testing.assert_array_equal(got["row_slot"], rs)
    np.testing.assert_array_equal(got["token_slot_row"], tsr)


@pytest.mark.parametrize("e_lo,E_L", [(0, 64), (16, 16), (48, 16)])
def test_layout_invariants(e_lo, E_L):
    rng = np.random.default_rng(11)
    T, E, k = 500, 64, 8
    ids = random_ids(rng, T, E, k)
    L = O.index_build(ids, e_lo, E_L)
    N = int(L["offsets"][-1])
    # counts sum to N and offsets are their exclusive scan
    assert L["counts"].sum() == N
    np.testing.assert_array_equal(np.diff(L["offsets"]), L["counts"])
    # each token appears once per local slot (k times when all are local)
    local = (ids >= e_lo) & (ids < e_lo + E_L)
    np.testing.assert_array_equal(np.bincount(L["row_token"], minlength=T), local.sum(1))
    if E_L == E:
        assert np.all(local.sum(1) == k)
    # inverse map round trip and slot consistency
    tsr = L["token_slot_row"]
    for t in range(T):
        for s in range(k):
            r = tsr[t, s]
            if local[t, s]:
                assert L["row_token"][r] == t and L["row_slot"][r] == s
                e = ids[t, s] - e_lo
                assert L["offsets"][e] <= r < L["offsets"][e + 1]
            else:
                assert r == -1
    # segments are strictly ascending in token
    for e in range(E_L):
        seg = L["row_token"][L["offsets"][e]:L["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_all_tokens_on_one_expert_and_empty_experts():
    T, k = 37, 2
    ids = np.stack([np.zeros(T), np.arange(T) % 3 + 1], 1).astype(np.int32)
    L = O.index_build(ids, 0, 8)
    assert L["counts"][0] == T and L["counts"][4:].sum() == 0
    np.testing.assert_array_equal(L["row_token"][:T], np.arange(T))


def test_tile_count_by_enumeration():
    rng = np.random.default_rng(3)
    for _ in range(20):
        counts = rng.integers(0, 300, size=rng.integers(1, 40))
        counts[rng.random(len(counts)) < 0.3] = 0
        for tm in (16, 64, 128, 256):
            tiles = []
            for e, m in enumerate(counts):
                r = 0
                while r < m:
                    tiles.append((e, r))
                    r += tm
            assert O.tile_count(counts, tm) == len(tiles)

"""Pins for the oracle's align (sort tokens to experts, pad to block_m): brute force
with numpy's stable argsort + bincount, and the invariants every output must meet."""
import numpy as np
import pytest


def brute_align(ids, E, B):
    """Written independently of the oracle: stable argsort by expert id."""
    flat = ids.reshape(-1)
    P = flat.size
    valid = (flat >= 0) & (flat < E)
    L = P + E * (B - 1)
    NB = -(-L // B)
    counts = np.bincount(flat[valid], minlength=E)
    padded = -(-counts // B) * B
    off = np.concatenate([[0], np.cumsum(padded)])
    sorted_ids = np.full(L, P, np.int32)
    order = np.argsort(np.where(valid, flat, E), kind="stable")
    pos = 0
    for e in range(E):
        sel = order[pos:pos + counts[e]]
        sorted_ids[off[e]:off[e] + counts[e]] = sel
        pos += counts[e]
    expert_ids = np.full(NB, -1, np.int32)
    for e in range(E):
        expert_ids[off[e] // B:off[e + 1] // B] = e
    return sorted_ids, expert_ids, int(off[-1]), off.astype(np.int32)


def check_invariants(ids, E, B, sorted_ids, expert_ids, ntp, offs):
    flat = ids.reshape(-1)
    P = flat.size
    valid_idx = np.nonzero((flat >= 0) & (flat < E))[0]
    real = sorted_ids[sorted_ids < P]
    # every valid (token, slot) appears exactly once, invalid ones never
    assert np.array_equal(np.sort(real), valid_idx)
    assert np.all((sorted_ids >= 0) & (sorted_ids <= P))
    assert ntp % B == 0 and np.all(np.diff(offs) % B == 0) and offs[0] == 0 and offs[-1] == ntp
    # each segment holds only its expert's pairs, ascending, then sentinels
    for e in range(E):
        seg = sorted_ids[offs[e]:offs[e + 1]]
        r = seg[seg < P]
        assert np.all(flat[r] == e) and np.all(np.diff(r) > 0)
        assert np.all(seg[len(r):] == P)
        assert np.all(expert_ids[offs[e] // B:offs[e + 1] // B] == e)
    assert np.all(sorted_ids[ntp:] == P) and np.all(expert_ids[ntp // B:] == -1)
    # sentinel count inside the padded region
    assert np.sum(sorted_ids[:ntp] == P) == ntp - valid_idx.size


@pytest.mark.parametrize("T,k,E,B", [
    (16, 2, 8, 16), (32, 8, 48, 16), (37, 3, 5, 4), (1, 1, 1, 1), (256, 8, 384, 16),
    (300, 8, 48, 128), (64, 4, 4, 256), (8, 8, 8, 32),
])
def test_align_matches_stable_sort(oracle_mod, T, k, E, B):
    rng = np.random.default_rng(T * 1000 + E + B)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    got = oracle_mod.moe_align(ids, E, B)
    exp = brute_align(ids, E, B)
    assert np.array_equal(got[0], exp[0]) and np.array_equal(got[1], exp[1])
    assert got[2] == exp[2] and np.array_equal(got[3], exp[3])
    check_invariants(ids, E, B, *got)


def test_align_skewed_repeated_and_invalid_ids(oracle_mod):
    rng = np.random.default_rng(5)
    E, B = 6, 8
    ids = rng.integers(-2, E + 2, size=(200, 3)).astype(np.int32)  # repeats and out-of-range
    ids[:50] = 0  # heavy expert
    got = oracle_mod.moe_align(ids, E, B)
    exp = brute_align(ids, E, B)
    for a, b in zip(got, exp):
        assert np.array_equal(np.asarray(a), np.asarray(b))
    check_invariants(ids, E, B, *got)


def test_align_empty_and_all_invalid(oracle_mod):
    for ids in (np.zeros((0, 4), np.int32), np.full((5, 2), 99, np.int32)):
        s, eids, ntp, offs = oracle_mod.moe_align(ids, 3, 16)
        assert ntp == 0 and np.all(offs == 0)
        assert np.all(s == ids.size) and np.all(eids == -1)
        assert s.size == ids.size + 3 * 15

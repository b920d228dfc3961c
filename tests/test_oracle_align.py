"""Pins of the oracle's align step: brute force by a Python stable sort,
invariants, adversarial id patterns via hypothesis."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def _brute_align(ids, E, BM):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    n = len(flat)
    order = sorted(range(n), key=lambda i: flat[i])          # Python's sort is stable
    segs = {e: [i for i in order if flat[i] == e] for e in range(E)}
    sorted_ids, blocks, offs = [], [], [0]
    for e in range(E):
        seg = segs[e]
        padded = -(-len(seg) // BM) * BM
        sorted_ids += seg + [n] * (padded - len(seg))
        blocks += [e] * (padded // BM)
        offs.append(offs[-1] + padded)
    cap, nblk = oracle.align_capacity(len(ids), np.asarray(ids).shape[1], E, BM)
    sorted_ids += [n] * (cap - len(sorted_ids))
    blocks += [-1] * (nblk - len(blocks))
    return sorted_ids, blocks, offs, [len(segs[e]) for e in range(E)]


def _check(ids, E, BM):
    ids = np.asarray(ids, dtype=np.int32)
    out = oracle.align(ids, E, BM)
    s, b, o, c = _brute_align(ids, E, BM)
    assert out["sorted_token_ids"].tolist() == s
    assert out["block_expert_ids"].tolist() == b
    assert out["expert_offsets"].tolist() == o
    assert out["expert_counts"].tolist() == c
    n = ids.size
    assert out["num_tokens_post_padded"][0] == o[-1]
    # invariants
    assert sum(c) == n
    assert all(v % BM == 0 for v in o)
    real = out["sorted_token_ids"][out["sorted_token_ids"] != n]
    assert sorted(real.tolist()) == list(range(n))
    for e in range(E):
        seg = out["sorted_token_ids"][o[e]:o[e + 1]]
        seg = seg[seg != n]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ids.reshape(-1)[seg] == e)


@pytest.mark.parametrize("T,k,E,BM", [(16, 2, 8, 16), (301, 2, 8, 64), (203, 8, 32, 16),
                                      (157, 1, 16, 128), (1, 2, 8, 16), (0, 2, 8, 16)])
def test_align_random(T, k, E, BM):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k))
    _check(ids.reshape(T, k), E, BM)


def test_align_all_on_one_expert_and_empty_experts():
    _check(np.full((50, 1), 3), 8, 16)
    ids = np.array([[255, 0]] * 33 + [[0, 255]] * 2)
    _check(ids, 256, 32)


def test_align_capacity_bound_is_tight_for_one_row_per_expert():
    ids = np.arange(8).reshape(8, 1)
    out = oracle.align(ids, 8, 16)
    cap, nblk = oracle.align_capacity(8, 1, 8, 16)
    assert out["num_tokens_post_padded"][0] == cap == 8 * 16
    assert nblk == 8


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 40), st.integers(1, 4), st.sampled_from([1, 2, 3, 8, 16, 256]),
       st.sampled_from([16, 32, 64, 128]), st.integers(0, 2 ** 31 - 1))
def test_align_hypothesis(T, k, E, BM, seed):
    k = min(k, E)
    rng = np.random.default_rng(seed)
    hot = rng.integers(0, E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if seed % 3 == 0:      # adversarial: force most rows to contain one hot expert
        ids[:, 0] = hot
        for t in range(T):
            rest = [e for e in rng.permutation(E) if e != hot][:k - 1]
            ids[t, 1:] = rest
    _check(ids, E, BM)

"""Pins of the oracle routing tables: naive loops vs the vectorised twin, the
practice page's invariants (bijection, padded ranges, slack identity), the pool
capacity formula and exhaustive brute force over tiny shapes."""
import itertools
import os

import numpy as np
import pytest

from oracle.routing import capacity_rows, plan_naive, plan_ref

FIELDS = ["counts", "offsets", "slot", "row_token", "row_topk", "block_expert", "slack", "pull_order"]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def assert_same(a, b):
    for f in FIELDS:
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert (a.num_valid, a.r_pad, a.n_pull, a.n_blocks, a.capacity) == \
        (b.num_valid, b.r_pad, b.n_pull, b.n_blocks, b.capacity)


def check_invariants(p, ids, E, begin, bm):
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    local = ids - begin
    valid = (local >= 0) & (local < E)
    # counts and padded ranges
    assert p.counts.sum() == valid.sum() == p.num_valid
    assert np.array_equal(p.counts, np.bincount(local[valid], minlength=E))
    pad = np.diff(p.offsets)
    assert np.all(pad % bm == 0) and np.all(pad >= p.counts) and np.all(pad - p.counts < bm)
    assert p.offsets[0] == 0 and p.offsets[-1] == p.r_pad <= p.capacity
    # bijection: valid hits <-> non-padding rows, with inverse tables
    s = p.slot
    assert np.all((s >= 0) == valid)
    used = s[valid]
    assert np.unique(used).size == used.size
    assert set(used.tolist()) == set(np.nonzero(p.row_token >= 0)[0].tolist())
    tt, jj = np.nonzero(valid)
    assert np.array_equal(p.row_token[s[tt, jj]], tt) and np.array_equal(p.row_topk[s[tt, jj]], jj)
    assert np.all((p.row_token < 0) == (p.row_topk < 0))
    # each expert's rows: [offsets[e], offsets[e]+counts[e]) filled in ascending flat order, rest padding
    for e in range(E):
        r0, n, r1 = p.offsets[e], p.counts[e], p.offsets[e + 1]
        rows = np.arange(r0, r0 + n)
        assert np.all(p.row_token[rows] >= 0) and np.all(p.row_token[r0 + n:r1] < 0)
        flat = p.row_token[rows] * k + p.row_topk[rows]
        assert np.all(np.diff(flat) > 0)
        assert np.all(local[p.row_token[rows], p.row_topk[rows]] == e)
    # block tables and the slack identity: slack + real rows = block_m; sum slack = R_pad - N
    assert p.n_blocks * bm == p.r_pad
    for b in range(p.n_blocks):
        e = p.block_expert[b]
        assert p.offsets[e] <= b * bm < p.offsets[e + 1]
        assert p.slack[b] + (p.row_token[b * bm:(b + 1) * bm] >= 0).sum() == bm
    assert p.slack.sum() == p.r_pad - p.num_valid
    # pull order: every token with a hit once, ascending by smallest slot
    has = valid.any(axis=1)
    assert sorted(p.pull_order.tolist()) == np.nonzero(has)[0].tolist() and p.n_pull == has.sum()
    mins = [s[t][s[t] >= 0].min() for t in p.pull_order]
    assert np.all(np.diff(mins) > 0)


def random_ids(rng, T, k, E, begin, span, dup=False):
    ids = rng.integers(begin - span, begin + E + span, size=(T, k))
    if not dup:
        for t in range(T):   # mostly distinct per token, like top-k
            ids[t] = rng.permutation(np.arange(begin - span, begin + E + span))[:k]
    return ids


@pytest.mark.parametrize("seed", range(6))
def test_naive_vs_vectorised_random(seed):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(1, 60)), int(rng.integers(1, 9)), int(rng.integers(1, 17))
    begin = int(rng.integers(0, 40))
    bm = int(2 ** rng.integers(0, 6))
    ids = random_ids(rng, T, k, E, begin, span=max(E, k), dup=bool(seed % 2))
    a, b = plan_naive(ids, E, begin, bm), plan_ref(ids, E, begin, bm)
    assert_same(a, b)
    check_invariants(b, ids, E, begin, bm)


def test_exhaustive_tiny_shapes():
    # every routing of T<=3 tokens, k<=2, E<=3 experts with ids in [-1, E] (one invalid id each side)
    n = 0
    for T, k, E, bm in itertools.product([1, 2, 3], [1, 2], [1, 2, 3], [1, 2, 4]):
        vals = list(range(-1, E + 1))
        for combo in itertools.product(vals, repeat=T * k):
            ids = np.array(combo, np.int64).reshape(T, k)
            a, b = plan_naive(ids, E, 0, bm), plan_ref(ids, E, 0, bm)
            assert_same(a, b)
            check_invariants(b, ids, E, 0, bm)
            n += 1
    assert n > 5000


def test_empty_and_all_invalid():
    ids = np.zeros((0, 4), np.int64)
    p = plan_ref(ids, 8, 0, 16)
    assert p.r_pad == 0 and p.num_valid == 0 and p.n_pull == 0 and p.n_blocks == 0
    ids = np.full((5, 2), -3, np.int64)
    p = plan_ref(ids, 8, 0, 16)
    assert p.r_pad == 0 and np.all(p.slot == -1) and p.n_pull == 0
    assert_same(p, plan_naive(ids, 8, 0, 16))


def test_capacity_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "pool_capacity.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) >= 5
    for tok, k, e, bm, want in (map(int, r) for r in rows):
        assert capacity_rows(tok, k, e, bm) == want


def test_capacity_bounds_worst_case():
    # R_pad <= capacity for adversarial routings, and the bound is reached
    rng = np.random.default_rng(5)
    for _ in range(200):
        T, k, E = int(rng.integers(1, 20)), int(rng.integers(1, 6)), int(rng.integers(1, 9))
        bm = int(2 ** rng.integers(0, 5))
        ids = random_ids(rng, T, k, E, 0, span=0, dup=False) if k <= E else rng.integers(0, E, (T, k))
        p = plan_ref(ids, E, 0, bm)
        assert p.r_pad <= capacity_rows(T, k, E, bm)
    # tight case: T = E*bm... every expert with counts == 1 mod bm and each token k distinct hits
    E, bm, k = 4, 8, 2
    T = (E * (bm + 1)) // k + 2
    best = 0
    for seed in range(50):
        r = np.random.default_rng(seed)
        ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
        best = max(best, plan_ref(ids, E, 0, bm).r_pad)
    assert best <= capacity_rows(T, k, E, bm)


def test_pull_order_tie_free_and_single_expert():
    ids = np.array([[0, 1], [1, 0], [2, 2], [1, 1]], np.int64)   # duplicates inside a token
    p = plan_ref(ids, 3, 0, 2)
    assert_same(p, plan_naive(ids, 3, 0, 2))
    check_invariants(p, ids, 3, 0, 2)
    # both hits of token 2 on expert 2 get consecutive rows in j order
    assert p.slot[2, 1] == p.slot[2, 0] + 1

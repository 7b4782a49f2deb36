"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to a library routine, a closed form, exact
rational arithmetic, exhaustive enumeration or hand-computed values, chosen so
that a plausible slip (dropped term, wrong sign or index, transposed operand,
off-by-one count) fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from tests import brute

RNG = np.random.default_rng(12345)


def bf16_bits(x):
    """torch's own fp32 -> bf16 rounding (RNE), as uint16 bit patterns."""
    t = torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------- Philox
@pytest.mark.parametrize("ctr,key", [
    ([1, 0, 0, 0], [0, 0]),
    ([5, 0, 0, 0], [7, 0]),
    ([1, 2, 3, 4], [5, 6]),
    ([2**63 + 11, 2**40 + 3, 99, 2**64 - 5], [2**64 - 1, 2**33]),
    ([123456789, 0, (7 << 32) | 5, 42], [0xDEADBEEF, 0]),
])
def test_philox_matches_numpy(ctr, key):
    # numpy's Philox (Philox-4x64-10) increments its counter before each block,
    # so numpy seeded with c - 1 produces the block of counter c (no carry here).
    mine = oracle.philox4x64_10(ctr, key)
    c = list(ctr)
    c[0] -= 1
    ref = np.random.Philox(counter=np.array(c, np.uint64),
                              key=np.array(key, np.uint64)).random_raw(4).astype(np.uint64)
    assert np.array_equal(mine, ref)


def test_philox_grid_matches_numpy():
    for i in range(64):
        ctr = [int(v) for v in RNG.integers(1, 2**63, 4, dtype=np.uint64)]
        key = [int(v) for v in RNG.integers(0, 2**63, 2, dtype=np.uint64)]
        c = list(ctr)
        c[0] -= 1
        ref = np.random.Philox(counter=np.array(c, np.uint64),
                              key=np.array(key, np.uint64)).random_raw(4).astype(np.uint64)
        assert np.array_equal(oracle.philox4x64_10(ctr, key), ref), i


def test_random_score_counter_layout_matches_numpy():
    seed, req, pss, layer, head, N, P = 0x1234_5678_9ABC, 77, 5, 3, 6, 203, 37
    u = oracle.random_score(seed, req, pss, layer, head, N, P)
    assert u.shape == (N - P,) and u.dtype == np.uint32
    for n in [P, P + 1, P + 2, 40, 41, 42, 43, 100, N - 1]:
        ctr = [n // 4 - 1, pss, (layer << 32) | head, req]
        if ctr[0] < 0:
            continue
        words = np.random.Philox(counter=np.array(ctr, np.uint64),
                                key=np.array([seed, 0], np.uint64)).random_raw(4)
        assert int(u[n - P]) == int(words[n % 4]) >> 32, n


def test_random_score_uniform_and_fresh_per_pass_and_head():
    N, P = 40000, 0
    u = oracle.random_score(9, 1, 0, 0, 0, N, P).astype(np.float64) / 2**32
    hist, _ = np.histogram(u, bins=50, range=(0, 1))
    expected = N / 50
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 100, chi2          # 49 dof; p ~ 5e-5 at 100
    a = oracle.random_score(9, 1, 0, 0, 0, 4096, 0)
    assert not np.array_equal(a, oracle.random_score(9, 1, 1, 0, 0, 4096, 0))   # new pass
    assert not np.array_equal(a, oracle.random_score(9, 1, 0, 0, 1, 4096, 0))   # other head
    assert not np.array_equal(a, oracle.random_score(9, 1, 0, 1, 0, 4096, 0))   # other layer
    assert not np.array_equal(a, oracle.random_score(9, 2, 0, 0, 0, 4096, 0))   # other request
    # slot-addressed: prompt length only changes which slots are scored
    b = oracle.random_score(9, 1, 0, 0, 0, 4096, 100)
    assert np.array_equal(a[100:], b)


# --------------------------------------------------------------- maintenance
def test_bf16_round_matches_torch():
    x = np.concatenate([RNG.standard_normal(5000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 1 + 2**-8, 1 + 3 * 2**-9, 1 + 2**-9,
                                  -(1 + 2**-9), 3.0 + 2**-7], np.float32)])
    mine = np.array([oracle.bf16_round(v) for v in x], np.uint16)
    assert np.array_equal(mine, bf16_bits(x))


def test_macqueen_fill_is_exact():
    T, G, d, K = 5, 2, 16, 12
    q = bf16_bits(RNG.standard_normal((T, G, d)))
    b, c, a = oracle.beacon_update(q, np.full((K, d), 7.0, np.float32), np.zeros(K, np.int32))
    assert list(a) == list(range(10))
    assert np.array_equal(c, np.array([1] * 10 + [0] * 2, np.int32))
    assert np.array_equal(b[:10], bf16_values(q.reshape(10, d)))
    assert np.all(b[10:] == 7.0)


def test_fills_first_empty_slot_even_when_not_leading():
    d, K = 8, 4
    b0 = RNG.standard_normal((K, d)).astype(np.float32)
    c0 = np.array([3, 0, 5, 0], np.int32)
    q = bf16_bits(RNG.standard_normal((2, 1, d)))
    b, c, a = oracle.beacon_update(q, b0, c0)
    assert list(a) == [1, 3]
    assert list(c) == [3, 1, 5, 1]
    assert np.array_equal(b[[0, 2]], b0[[0, 2]])


def test_update_hand_computed_values():
    # b = 0, count 1; query 3.0 -> count 2, b = 0 + (3 - 0)/2 = 1.5;
    # query 1.5 -> count 3, b = 1.5 + 0/3 = 1.5; query -4.5 -> count 4,
    # b = 1.5 + (-6)/4 = 0.
    d = 2
    q = bf16_bits(np.array([[[3.0, 1.0]], [[1.5, 1.0]], [[-4.5, 1.0]]]))
    b, c, _ = oracle.beacon_update(q, np.array([[0.0, 1.0]], np.float32),
                                   np.array([1], np.int32))
    assert c[0] == 4
    assert b[0, 0] == 0.0 and b[0, 1] == 1.0
    # a non-representable step rounds once per IEEE fp32 operation:
    # b = 1, count 2 -> x = 2: b = 1 + (2 - 1)/3 = 1 + fl32(1/3)
    q = bf16_bits(np.array([[[2.0, 0.0]]]))
    b, c, _ = oracle.beacon_update(q, np.array([[1.0, 0.0]], np.float32), np.array([2], np.int32))
    assert b[0, 0] == np.float32(np.float32(1.0) + np.float32(np.float32(1.0) / np.float32(3.0)))


def test_running_mean_tracks_exact_mean():
    T, G, d, K = 40, 4, 32, 6
    q = bf16_bits(RNG.standard_normal((T, G, d)) + 0.5)
    b0 = RNG.standard_normal((K, d)).astype(np.float32)
    c0 = RNG.integers(1, 9, K).astype(np.int32)
    b, c, a = oracle.beacon_update(q, b0, c0)
    assert c.sum() == c0.sum() + T * G
    xs = bf16_values(q.reshape(T * G, d)).astype(np.float64)
    for j in range(K):
        m = np.flatnonzero(a == j)
        assert c[j] == c0[j] + len(m)
        mean = (c0[j] * b0[j].astype(np.float64) + xs[m].sum(0)) / (c0[j] + len(m))
        # each fp32 update adds at most a few ulps of max(|x|, |b|)
        scale = max(np.abs(xs).max(), np.abs(b0[j]).max())
        tol = 4 * (len(m) + 1) * 2**-24 * scale
        assert np.max(np.abs(b[j] - mean)) <= tol, (j, np.max(np.abs(b[j] - mean)), tol)


# ---------------------------------------------- capped count (beacon forgetting)
def test_cap_at_least_the_counts_reached_is_the_plain_mean():
    T, G, d, K = 16, 4, 32, 6
    q = bf16_bits(RNG.standard_normal((T, G, d)))
    b0 = RNG.standard_normal((K, d)).astype(np.float32)
    c0 = np.array([0, 3, 1, 7, 0, 2], np.int32)
    b, c, a = oracle.beacon_update(q, b0, c0)
    bc, cc, ac = oracle.beacon_update(q, b0, c0, cap=int(c0.max()) + T * G)
    assert np.array_equal(a, ac) and np.array_equal(c, cc)
    assert np.array_equal(b.view(np.int32), bc.view(np.int32))


def test_cap_hand_computed_values():
    # count 5 above a cap of 2: the next observation uses c = 2, the count
    # becomes 2: b = 1 + (4 - 1)/2 = 2.5; the next: b = 2.5 + (0 - 2.5)/2 = 1.25
    q = bf16_bits(np.array([[[4.0, 1.0]], [[0.0, 1.0]]]))
    b, c, _ = oracle.beacon_update(q, np.array([[1.0, 1.0]], np.float32),
                                   np.array([5], np.int32), cap=2)
    assert c[0] == 2 and b[0, 0] == 1.25 and b[0, 1] == 1.0
    # an empty row is still filled exactly, whatever the cap
    b, c, _ = oracle.beacon_update(q[:1], np.array([[9.0, 9.0]], np.float32),
                                   np.array([0], np.int32), cap=1)
    assert c[0] == 1 and b[0, 0] == 4.0 and b[0, 1] == 1.0
    # cap 1 on a filled row: b + (x - b) / 1, one IEEE operation each
    b, c, _ = oracle.beacon_update(q[:1], np.array([[0.3, 0.7]], np.float32),
                                   np.array([4], np.int32), cap=1)
    f = np.float32
    assert c[0] == 1
    assert b[0, 0] == f(f(0.3) + f(f(4.0) - f(0.3))) and b[0, 1] == f(f(0.7) + f(f(1.0) - f(0.7)))


def test_capped_row_decays_geometrically_toward_a_repeated_query():
    # a full row (count == cap C) fed m copies of x: b_m - x = (1 - 1/C)^m (b_0 - x)
    d, C, m = 16, 4, 30
    x = bf16_bits(RNG.standard_normal(d))
    b0 = RNG.standard_normal((1, d)).astype(np.float32)
    q = np.tile(x, (m, 1, 1))
    b, c, a = oracle.beacon_update(q, b0, np.array([C], np.int32), cap=C)
    assert c[0] == C and (a == 0).all()
    xv = bf16_values(x).astype(np.float64)
    want = xv + (1 - 1 / C) ** m * (b0[0].astype(np.float64) - xv)
    scale = max(np.abs(xv).max(), np.abs(b0).max())
    assert np.max(np.abs(b[0] - want)) <= 4 * m * 2**-24 * scale


def test_counts_never_exceed_the_cap():
    T, G, d, K, C = 32, 4, 16, 5, 6
    q = bf16_bits(RNG.standard_normal((T, G, d)))
    b0 = RNG.standard_normal((K, d)).astype(np.float32)
    c0 = np.array([0, 2, 9, 6, 1], np.int32)
    _, c, a = oracle.beacon_update(q, b0, c0, cap=C)
    for j in range(K):
        hits = int((a == j).sum())
        want = c0[j] if hits == 0 else min(c0[j] + hits, C) if c0[j] < C else C
        assert c[j] == want, (j, c[j], want)


def test_assignment_is_exact_argmax_on_tiny_inputs():
    for trial in range(6):
        T, G, d, K = 6, 2, 6, 5
        q = bf16_bits(RNG.standard_normal((T, G, d)))
        b0 = RNG.standard_normal((K, d)).astype(np.float32)
        if trial == 0:
            b0[2] = 0.0                       # a zero-norm beacon counts as cosine 0
        c0 = RNG.integers(1, 5, K).astype(np.int32)
        _, _, a = oracle.beacon_update(q, b0, c0)
        flat = q.reshape(T * G, d)
        for s in range(T * G):
            if s == 0:
                bs = b0
            else:
                bs, _, _ = oracle.beacon_update(flat[:s].reshape(s, 1, d), b0, c0)
            assert a[s] == brute.exact_nearest(flat[s], bs), (trial, s)


def test_zero_query_goes_to_row_zero():
    d, K = 8, 3
    b0 = RNG.standard_normal((K, d)).astype(np.float32)
    q = np.zeros((1, 1, d), np.uint16)
    _, _, a = oracle.beacon_update(q, b0, np.ones(K, np.int32))
    assert a[0] == 0


def test_forced_replay_gap_and_rules():
    T, G, d, K = 20, 2, 16, 4
    q = bf16_bits(RNG.standard_normal((T, G, d)))
    b0 = np.zeros((K, d), np.float32)
    c0 = np.zeros(K, np.int32)
    b1, c1, a = oracle.beacon_update(q, b0, c0)
    b2, c2, gap = oracle.beacon_update_forced(q, b0, c0, a)
    assert np.array_equal(b1, b2) and np.array_equal(c1, c2)
    assert np.all(gap == 0.0)
    bad = a.copy()
    bad[0] = 1                                    # breaks the empty-slot rule
    _, _, gap = oracle.beacon_update_forced(q, b0, c0, bad)
    assert np.isinf(gap[0])
    bad = a.copy()
    s = K + 3
    bad[s] = (a[s] + 1) % K                       # a worse row after the fill
    _, _, gap = oracle.beacon_update_forced(q, b0, c0, bad)
    assert gap[s] > 0


# --------------------------------------------------------------- scoring
def _keys(N, d, scale=1.0):
    return bf16_bits(RNG.standard_normal((N, d)) * scale)


def test_single_beacon_score_is_torch_softmax():
    N, P, d, W = 300, 40, 128, 64
    k = _keys(N, d)
    b = RNG.standard_normal((1, d)).astype(np.float32)
    s, lse = oracle.beacon_score(k, b, np.array([3], np.int32), P, W=W, bonus=0.0)
    kv = torch.tensor(bf16_values(k), dtype=torch.float64)
    bv = torch.tensor(bf16_values(bf16_bits(b)), dtype=torch.float64)    # torch's bf16 RNE
    logits = (kv @ bv[0]) / math.sqrt(d)
    ref = torch.softmax(logits, 0).numpy()
    assert np.allclose(s, ref[P:], rtol=1e-12, atol=0)
    assert abs(lse[0] - torch.logsumexp(logits, 0).item()) < 1e-12


def test_window_bonus_and_max_over_beacons():
    N, P, d, K, W = 260, 20, 128, 3, 64
    k = _keys(N, d)
    b = RNG.standard_normal((K, d)).astype(np.float32)
    c = np.array([1, 2, 3], np.int32)
    s0, _ = oracle.beacon_score(k, b, c, P, W=W, bonus=0.0)
    s1, _ = oracle.beacon_score(k, b, c, P, W=W, bonus=1.0)
    diff = s1 - s0
    n = np.arange(P, N)
    assert np.allclose(diff[n >= N - W], 1.0, atol=1e-15)
    assert np.all(diff[n < N - W] == 0.0)
    singles = [oracle.beacon_score(k, b[j:j + 1], c[j:j + 1], P, W=W, bonus=0.0)[0]
               for j in range(K)]
    assert np.array_equal(s0, np.maximum.reduce(singles))


def test_lse_normalises_every_live_beacon():
    N, P, d, K = 500, 0, 128, 5
    k = _keys(N, d, 2.0)
    b = (RNG.standard_normal((K, d)) * 1.5).astype(np.float32)
    c = np.array([2, 0, 5, 1, 9], np.int32)
    s, lse = oracle.beacon_score(k, b, c, P, W=0, bonus=0.0)
    assert np.isnan(lse[1]) and not np.isnan(lse[[0, 2, 3, 4]]).any()
    kv = bf16_values(k).astype(np.float64)
    bv = bf16_values(bf16_bits(b)).astype(np.float64)
    logits = bv @ kv.T / math.sqrt(d)                      # [K, N]
    for j in (0, 2, 3, 4):
        assert abs(np.exp(logits[j] - lse[j]).sum() - 1.0) < 1e-12
    assert np.all(s > 0) and np.all(s <= 1.0)


def test_identical_keys_give_uniform_sigma():
    N, P, d, K = 128, 16, 128, 4
    row = _keys(1, d)
    k = np.repeat(row, N, axis=0)
    b = RNG.standard_normal((K, d)).astype(np.float32)
    s, _ = oracle.beacon_score(k, b, np.ones(K, np.int32), P, W=0, bonus=0.0)
    assert np.allclose(s, 1.0 / N, rtol=1e-13)


def test_dead_beacons_are_ignored_and_empty_set_scores_zero():
    N, P, d, W = 200, 50, 128, 64
    k = _keys(N, d)
    b = RNG.standard_normal((3, d)).astype(np.float32)
    s_all, _ = oracle.beacon_score(k, b, np.array([4, 0, 1], np.int32), P, W=W)
    s_sub, _ = oracle.beacon_score(k, b[[0, 2]], np.array([4, 1], np.int32), P, W=W)
    assert np.array_equal(s_all, s_sub)
    s_none, lse = oracle.beacon_score(k, b, np.zeros(3, np.int32), P, W=W, bonus=1.0)
    n = np.arange(P, N)
    assert np.array_equal(s_none, np.where(n >= N - W, 1.0, 0.0))
    assert np.isnan(lse).all()


def test_more_beacons_never_lower_sigma():
    N, P, d = 300, 0, 128
    k = _keys(N, d)
    b = RNG.standard_normal((6, d)).astype(np.float32)
    prev = np.zeros(N)
    for K in range(1, 7):
        s, _ = oracle.beacon_score(k, b[:K], np.ones(K, np.int32), P, W=0, bonus=0.0)
        assert np.all(s >= prev)
        prev = s


def test_beacons_are_rounded_to_bf16_once():
    N, P, d = 100, 0, 128
    k = _keys(N, d)
    b = RNG.standard_normal((2, d)).astype(np.float32)
    b_rounded = bf16_values(bf16_bits(b))
    s1, l1 = oracle.beacon_score(k, b, np.ones(2, np.int32), P, W=0, bonus=0.0)
    s2, l2 = oracle.beacon_score(k, b_rounded, np.ones(2, np.int32), P, W=0, bonus=0.0)
    assert np.array_equal(s1, s2) and np.array_equal(l1, l2)


# --------------------------------------------------------------- selection
def test_topk_matches_exhaustive_dominance_search():
    for trial in range(30):
        P = int(RNG.integers(0, 4))
        m = int(RNG.integers(1, 10))
        B = P + int(RNG.integers(0, m))          # N > B so a real choice is made
        N = P + m
        if trial % 3 == 0:
            scores = RNG.integers(0, 3, m).astype(np.float64)     # many ties
        else:
            scores = RNG.random(m)
        keep = oracle.topk_select(scores, N, P, B)
        found = brute.topk_by_dominance(list(scores), P, B)
        assert len(found) == 1
        assert list(keep) == list(range(P)) + found[0], (trial, keep, found)


def test_topk_invariants_on_larger_inputs():
    for N, P, B in [(2112, 1024, 2048), (4096, 512, 1024), (3136, 1500, 3072), (700, 0, 64)]:
        s = RNG.random(N - P)
        s[::7] = 0.5                                   # plant ties
        keep = oracle.topk_select(s, N, P, B)
        assert keep.shape == (B,)
        assert np.array_equal(keep[:P], np.arange(P))
        assert np.all(np.diff(keep) > 0)
        mask = np.zeros(N, bool)
        mask[keep] = True
        kept, evicted = np.flatnonzero(mask[P:]), np.flatnonzero(~mask[P:])
        lo = s[kept].min()
        hi = s[evicted].max()
        assert lo >= hi
        if lo == hi:   # ties at the boundary go to the lower slots
            assert kept[s[kept] == lo].max() < evicted[s[evicted] == hi].min()


def test_topk_edge_cases():
    assert list(oracle.topk_select(np.ones(5), 8, 3, 10)) == list(range(8))    # N <= B
    assert list(oracle.topk_select(np.ones(5), 8, 3, 8)) == list(range(8))     # N == B
    assert list(oracle.topk_select(np.ones(5), 8, 3, 3)) == [0, 1, 2]         # P == B
    assert list(oracle.topk_select(np.ones(5), 8, 3, 5)) == [0, 1, 2, 3, 4]   # all tied
    assert list(oracle.topk_select(np.zeros(0), 0, 0, 4)) == []               # empty
    with pytest.raises(ValueError):
        oracle.topk_select(np.ones(5), 8, 3, 2)                                # P > B


def test_topk_on_uint32_draws_is_exact():
    u = np.array([5, 2**32 - 1, 2**32 - 2, 7, 2**32 - 1, 0], np.uint32)
    keep = oracle.topk_select(u, 8, 2, 5)
    # best three: slot 3 (2^32-1), slot 6 (2^32-1, later), slot 4 (2^32-2)
    assert list(keep) == [0, 1, 3, 4, 6]


# --------------------------------------------------------------- shared positions
def test_shared_select_hand_computed_merge():
    # Two heads disagree on slots 1 and 2 and agree on a middling slot 3.  The
    # largest per-head score keeps 1 and 2; a mean would keep 3 and 1, a
    # minimum 3 and 4, and reading the [H][m] rows transposed keeps 1 and 3.
    s = np.array([[0.9, 0.1, 0.6, 0.2],
                  [0.1, 0.9, 0.6, 0.3]])
    assert list(oracle.shared_select(s, 5, 1, 3)) == [0, 1, 2]
    # three heads, uint32 draws: merged = [7, 9, 4, 9, 2] -> keep slots 2+1, 2+3 and 2+0
    u = np.array([[7, 1, 4, 0, 2], [0, 9, 0, 0, 0], [3, 0, 0, 9, 1]], np.uint32)
    assert list(oracle.shared_select(u, 7, 2, 5)) == [0, 1, 2, 3, 5]


def test_shared_select_matches_exhaustive_dominance_on_merged_scores():
    for trial in range(30):
        H = int(RNG.integers(1, 5))
        P = int(RNG.integers(0, 4))
        m = int(RNG.integers(1, 10))
        B = P + int(RNG.integers(0, m))
        N = P + m
        s = RNG.integers(0, 4, (H, m)).astype(np.float64) if trial % 2 else RNG.random((H, m))
        merged = [max(s[h][i] for h in range(H)) for i in range(m)]
        found = brute.topk_by_dominance(merged, P, B)
        assert len(found) == 1
        assert list(oracle.shared_select(s, N, P, B)) == list(range(P)) + found[0], trial


def test_shared_select_reduces_to_per_head_selection():
    N, P, B = 2112, 1024, 2048
    s = RNG.random(N - P)
    per_head = oracle.topk_select(s, N, P, B)
    assert np.array_equal(oracle.shared_select(s[None], N, P, B), per_head)      # one head
    assert np.array_equal(oracle.shared_select(np.stack([s] * 8), N, P, B), per_head)  # equal heads
    assert list(oracle.shared_select(np.ones((3, 5)), 8, 3, 10)) == list(range(8))   # N <= B
    with pytest.raises(ValueError):
        oracle.shared_select(np.ones((3, 5)), 8, 3, 2)                             # P > B


# --------------------------------------------------------------- page retention
def test_page_select_hand_computed():
    # page 4, N 18, P 5: pages [0,4) [4,8) [8,12) [12,16) [16,18).  Pages 0 and 1
    # hold prompt slots and page 4 is a partial last page: all three are kept.
    # B 16 -> 4 pages, so one of pages 2 and 3 survives.  Row 0 peaks in page 2
    # at 0.7, row 1 in page 3 at 0.8: the largest slot score over both rows
    # keeps page 3 (a page mean, or row 0 alone, would keep page 2).
    N, P = 18, 5
    s = np.zeros((2, N - P))
    s[0, 8 - P:12 - P] = [0.1, 0.7, 0.1, 0.1]
    s[0, 12 - P:16 - P] = [0.2, 0.2, 0.2, 0.2]
    s[1, 8 - P:12 - P] = [0.3, 0.3, 0.3, 0.3]
    s[1, 12 - P:16 - P] = [0.0, 0.0, 0.8, 0.0]
    s[0, 16 - P] = 0.99
    kp = oracle.page_select(s, N, P, 16, page=4)
    assert list(kp) == [0, 1, 3, 4]
    row, freed, n = oracle.page_remap([40, 41, 42, 43, 44], N, kp, page=4)
    assert list(row) == [40, 41, 43, 44] and list(freed) == [42] and n == 4 + 4 + 4 + 2
    # equal page scores: the earlier page wins
    s[1, 12 - P:16 - P] = [0.0, 0.0, 0.7, 0.0]
    assert list(oracle.page_select(s, N, P, 16, page=4)) == [0, 1, 2, 4]


def test_page_select_with_unit_pages_is_the_shared_selection():
    for trial in range(10):
        H, N, P = int(RNG.integers(1, 4)), int(RNG.integers(50, 300)), int(RNG.integers(0, 40))
        B = int(RNG.integers(P, N))
        s = RNG.random((H, N - P))
        assert np.array_equal(oracle.page_select(s, N, P, B, page=1),
                              oracle.shared_select(s, N, P, B)), trial


def test_page_select_matches_exhaustive_dominance():
    for trial in range(40):
        page = int(RNG.choice([2, 3, 4]))
        rows = int(RNG.integers(1, 4))
        N = int(RNG.integers(6, 30))
        P = int(RNG.integers(0, N // 2))
        npages = -(-N // page)
        forced = [j for j in range(npages) if j * page < P or (j == npages - 1 and N % page)]
        cands = [j for j in range(npages) if j not in forced]
        if not cands:
            continue
        Bp = len(forced) + int(RNG.integers(0, len(cands)))
        s = RNG.integers(0, 3, (rows, N - P)).astype(np.float64) if trial % 2 else \
            RNG.random((rows, N - P))
        # page score written out: max over rows and the page's candidate slots
        ps = []
        for j in cands:
            ps.append(max(s[r][n - P] for r in range(rows)
                          for n in range(j * page, min((j + 1) * page, N))))
        k = Bp - len(forced)
        found = []
        for S in itertools.combinations(range(len(cands)), k):
            inside = set(S)
            beats = lambda a, b: ps[a] > ps[b] or (ps[a] == ps[b] and a < b)   # noqa: E731
            if all(beats(a, b) for a in S for b in range(len(cands)) if b not in inside):
                found.append(sorted(forced + [cands[i] for i in S]))
        assert len(found) == 1
        kp = oracle.page_select(s, N, P, Bp * page, page=page)
        assert list(kp) == found[0], (trial, list(kp), found)


def test_page_select_edge_cases_and_remap_invariants():
    s = RNG.random((3, 100 - 20))
    # everything fits: all pages kept, nothing released
    kp = oracle.page_select(s, 100, 20, 112, page=16)
    assert list(kp) == list(range(7))
    # prompt pages plus the partial last page exceed the budget: refused
    with pytest.raises(ValueError):
        oracle.page_select(s, 100, 20, 32, page=16)      # 2 prompt + 1 partial > 2
    assert list(oracle.page_select(s, 100, 20, 48, page=16)) == [0, 1, 6]
    # steady state of the serving shape: 132 pages, 128 kept
    N, P, B = 2112, 1024, 2048
    s = RNG.random((288, N - P))
    kp = oracle.page_select(s, N, P, B, page=16)
    assert len(kp) == B // 16 and np.all(np.diff(kp) > 0)
    assert np.array_equal(kp[:64], np.arange(64))
    block_row = RNG.permutation(5000)[:132].astype(np.int32)
    row, freed, n = oracle.page_remap(block_row, N, kp, page=16)
    assert n == B and len(freed) == 4
    assert sorted(np.concatenate([row, freed]).tolist()) == sorted(block_row.tolist())
    assert np.array_equal(row, block_row[kp])


def test_random_page_retention_is_uniform_over_pages():
    # one shared draw row per request: the page score is the largest of 16
    # independent uniform draws, so every candidate page is equally likely
    # to survive ((Bp - forced) / candidates each)
    N, P, B, trials = 512, 64, 256, 4000
    hits = np.zeros(N // 16)
    for t in range(trials):
        u = oracle.random_score(3, t, 0, 0, 0, N, P)
        hits[oracle.page_select(u[None], N, P, B, page=16)] += 1
    cand = hits[P // 16:] / trials
    expect = (B // 16 - P // 16) / (N // 16 - P // 16)
    sd = math.sqrt(expect * (1 - expect) / trials)
    assert np.all(hits[:P // 16] == trials)
    assert np.all(np.abs(cand - expect) < 5 * sd), (cand, expect)


# --------------------------------------------------------------- decode attention
def _bf16_rows(shape, scale=1.0):
    return bf16_bits(RNG.standard_normal(shape).astype(np.float32) * scale)


def test_decode_attention_matches_torch_sdpa():
    for G, N in [(4, 37), (1, 1), (8, 300)]:
        q, k, v = _bf16_rows((G, 128)), _bf16_rows((N, 128), 2.0), _bf16_rows((N, 128))
        qf, kf, vf = (torch.from_numpy(bf16_values(x).astype(np.float64)) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qf[None], kf[None], vf[None])[0]
        out = oracle.decode_attention(q, k, v)
        assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12), (G, N)


def test_decode_attention_closed_forms():
    q, k, v = _bf16_rows((4, 128)), _bf16_rows((1, 128)), _bf16_rows((1, 128))
    assert np.array_equal(oracle.decode_attention(q, k, v), np.tile(bf16_values(v), (4, 1)))
    k = np.tile(_bf16_rows((1, 128)), (50, 1))                 # identical keys -> mean of values
    v = _bf16_rows((50, 128))
    mean = bf16_values(v).astype(np.float64).mean(0)
    assert np.allclose(oracle.decode_attention(q, k, v), np.tile(mean, (4, 1)), rtol=1e-13,
                       atol=1e-13)
    k, v = _bf16_rows((20, 128)), _bf16_rows((20, 128))          # huge scale -> the best key
    best = (bf16_values(q).astype(np.float64) @ bf16_values(k).astype(np.float64).T).argmax(1)
    hard = oracle.decode_attention(q, k, v, scale=1e6)
    assert np.allclose(hard, bf16_values(v)[best], atol=1e-9)
    assert np.all(oracle.decode_attention(q, k[:0], v[:0]) == 0)  # empty cache


def test_decode_attention_ignores_slot_order():
    q, k, v = _bf16_rows((4, 128)), _bf16_rows((200, 128), 1.5), _bf16_rows((200, 128))
    perm = RNG.permutation(200)
    a = oracle.decode_attention(q, k, v)
    b = oracle.decode_attention(q, k[perm], v[perm])
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------- compaction
def test_compaction_is_numpy_gather():
    rows = RNG.integers(0, 2**16, (300, 128), dtype=np.uint16)
    keep = np.sort(RNG.choice(300, 120, replace=False)).astype(np.int32)
    out = oracle.kv_compact(rows, keep)
    assert np.array_equal(out, rows[keep])
    assert oracle.kv_compact(rows, np.zeros(0, np.int32)).shape == (0, 128)


def test_evict_batch_is_the_per_head_steps_composed():
    """The whole-pass oracle (the CPU baseline's timed routine) equals the
    pinned per-head steps called one head-cache at a time: update, score,
    select, compact, bit for bit, with its own strides over a padded batch."""
    H, T, G, d, K, B, W, bonus = 9, 5, 3, 128, 40, 48, 8, 1.0
    Nmax = 83
    N = np.array([80, 70, 49, 48, 33, 64, 77, 56, 83], np.int32)
    P = np.array([10, 0, 20, 5, 33, 50, 47, 3, 12], np.int32)   # head 5: P > B, refused
    rng = np.random.default_rng(2024)
    q = bf16_bits(rng.normal(size=(H, T, G, d)))
    keys = bf16_bits(rng.normal(size=(H, Nmax, d)) * rng.uniform(0.5, 2, (H, 1, d)))
    vals = bf16_bits(rng.normal(size=(H, Nmax, d)))
    beacons = rng.normal(size=(H, K, d)).astype(np.float32)
    counts = rng.integers(1, 9, (H, K)).astype(np.int32)
    counts[1, [3, 17, 39]] = 0          # rows still to be filled (MacQueen)
    counts[4] = 0                       # a fresh beacon set: every step fills
    beacons[counts == 0] = 0.0
    b2, c2, keep, ko, vo, fails = oracle.evict_batch(q, beacons, counts, keys, vals, N, P, B,
                                                     W, bonus, strict=False)
    assert fails == 1
    for h in range(H):
        rb, rc, _ = oracle.beacon_update(q[h], beacons[h], counts[h])
        assert np.array_equal(b2[h].view(np.int32), rb.view(np.int32)), h
        assert np.array_equal(c2[h], rc), h
        n, p = int(N[h]), int(P[h])
        sc, _ = oracle.beacon_score(keys[h, :n], rb, rc, p, W, bonus)
        if p > B:
            with pytest.raises(ValueError):
                oracle.topk_select(sc, n, p, B)
            assert np.all(keep[h] == -1) and not ko[h].any() and not vo[h].any(), h
            continue
        rk = oracle.topk_select(sc, n, p, B)
        nk = len(rk)
        assert np.array_equal(keep[h, :nk], rk) and np.all(keep[h, nk:] == -1), h
        assert np.array_equal(ko[h, :nk], oracle.kv_compact(keys[h, :n], rk)), h
        assert np.array_equal(vo[h, :nk], oracle.kv_compact(vals[h, :n], rk)), h
        assert not ko[h, nk:].any() and not vo[h, nk:].any(), h
    with pytest.raises(ValueError):
        oracle.evict_batch(q, beacons, counts, keys, vals, N, P, B, W, bonus)


def test_gather_paged_reads_block_table():
    pool = RNG.integers(0, 2**16, (10, 2, 16, 4), dtype=np.uint16)
    table = np.array([7, 2, 9], np.int32)
    dense = oracle.gather_paged(pool, table, 1, 40)
    assert np.array_equal(dense[:16], pool[7, 1])
    assert np.array_equal(dense[16:32], pool[2, 1])
    assert np.array_equal(dense[32:40], pool[9, 1, :8])


# --------------------------------------------------------------- random retention
def test_random_retention_survival_decays_geometrically():
    """A generated token must survive every eviction, so under the random
    selector its survival falls geometrically.  In steady state with budget B,
    prompt P and T new slots per pass, each candidate is kept with probability
    (B-P)/(B-P+T) per pass, independently across passes (fresh draws)."""
    P, B, T = 8, 72, 16                  # keep 64 of 80 -> p = 0.8
    p = (B - P) / (B - P + T)
    heads, passes, cohorts, ages = 24, 40, 28, 12
    alive_at_age = np.zeros(ages)
    for h in range(heads):
        pos = list(range(B))             # token ids in slot order
        birth = {}
        nxt = B
        for ps in range(passes):
            new = list(range(nxt, nxt + T))
            nxt += T
            for t in new:
                birth[t] = ps
            pos = pos + new
            u = oracle.random_score(2024, h, ps, 0, h, len(pos), P)
            keep = oracle.topk_select(u, len(pos), P, B)
            pos = [pos[i] for i in keep]
            for t in pos:
                b = birth.get(t)
                if b is not None and b < cohorts and ps - b < ages:
                    alive_at_age[ps - b] += 1
    n = heads * cohorts * T
    for m in range(ages):
        rate = alive_at_age[m] / n
        expect = p ** (m + 1)
        sd = math.sqrt(expect * (1 - expect) / n)
        assert abs(rate - expect) < 5 * sd, (m, rate, expect)

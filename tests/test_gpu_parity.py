"""GPU parity: every kernel behind the C ABI against the CPU oracle, on the same
seeded inputs (sizes the oracle finishes in seconds; several MFMA tiles and a
ragged tail).  Bit-exact for draws, keep lists and moved bytes; 1e-3 relative
for float scores; teacher-forced for beacon assignment."""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_beacon_amd import synth
from tests.gpu_util import (ASSIGN_TOL, ATT_TOL, INEXACT_LIMIT, bf16_values, check_scores, check_selection,
                            device_cache, hc_index, host_pools, keep_rows)

pytestmark = pytest.mark.gpu

bk = None


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global bk
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from decode_kv_cache_beacon_amd import beaconkv
    bk = beaconkv
    torch.cuda.init()
    yield


def say(*a):
    print("[case]", *a, flush=True)


def small(name="serving_r128", **kw):
    return synth.WORKLOADS[name].with_(**kw)


def head_iter(cache):
    L, R, H = cache.n_layers, cache.n_requests, cache.n_kv_heads
    for layer in range(L):
        for r in range(R):
            for h in range(H):
                yield hc_index(R, H, layer, r, h), layer, r, h


def random_keep(cache, B, N, P, seed=7):
    """Keep lists chosen by the oracle's random selector (inputs for compaction)."""
    keep = np.full((cache.n_head_caches, B), -1, np.int32)
    for hc, layer, r, h in head_iter(cache):
        u = oracle.random_score(seed, r, 0, layer, h, N[r], P[r])
        k = oracle.topk_select(u, N[r], P[r], B)
        keep[hc, :len(k)] = k
    return keep


# ------------------------------------------------------------------ compaction
@pytest.mark.parametrize("case", ["paged", "dense", "ragged"])
def test_compact_matches_oracle_gather(case):
    say("compact", case)
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, budget=512, prompt_len=200, seq_len=576,
               paged=case != "dense")
    batch = synth.make_batch(wl)
    N = [576, 555, 301] if case == "ragged" else [576] * 3
    P = [200, 200, 37] if case == "ragged" else [200] * 3
    B = 512
    cache = device_cache(batch, N, P)
    k_in, v_in = host_pools(cache)
    bt = batch.block_table.numpy()
    keep = random_keep(cache, B, N, P)
    HC, S = cache.n_head_caches, cache.max_slots
    pos = (np.arange(HC * S, dtype=np.int32).reshape(HC, S) * 7 + 3).astype(np.int32)
    pos_dev = torch.from_numpy(pos).cuda()
    bk.bkv_kv_compact(cache, torch.from_numpy(keep).cuda(), B, pos_ids=pos_dev)
    k_out, v_out = host_pools(cache)
    pos_out = pos_dev.cpu().numpy()
    for hc, layer, r, h in head_iter(cache):
        kp = keep_rows(keep[hc])
        nk = len(kp)
        for src, dst in ((k_in, k_out), (v_in, v_out)):
            dense_in = oracle.gather_paged(src[layer], bt[r], h, N[r])
            dense_out = oracle.gather_paged(dst[layer], bt[r], h, N[r])
            assert np.array_equal(dense_out[:nk], oracle.kv_compact(dense_in, kp)), (hc, case)
            assert np.array_equal(dense_out[nk:], dense_in[nk:]), (hc, "tail changed")
        assert np.array_equal(pos_out[hc, :nk], pos[hc][kp])
        assert np.array_equal(pos_out[hc, nk:], pos[hc, nk:])


def test_compact_rejects_bad_keep_lists():
    say("compact bad keep")
    wl = small(n_layers=1, n_requests=2, n_kv_heads=2, budget=64, prompt_len=16, seq_len=128)
    batch = synth.make_batch(wl)
    cache = device_cache(batch)
    k_in, _ = host_pools(cache)
    keep = np.tile(np.arange(64, dtype=np.int32), (cache.n_head_caches, 1)) + 1
    keep[0, 5], keep[0, 6] = keep[0, 6], keep[0, 5]      # not ascending
    keep[3, 63] = 128                                      # outside [0, N)
    st = bk.bkv_kv_compact(cache, torch.from_numpy(keep).cuda(), 64, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 1 << bk.BKV_ERR_INVALID
    k_out, _ = host_pools(cache)
    bt = batch.block_table.numpy()
    for hc, layer, r, h in head_iter(cache):
        a = oracle.gather_paged(k_in[layer], bt[r], h, 128)
        b = oracle.gather_paged(k_out[layer], bt[r], h, 128)
        if hc in (0, 3):
            assert np.array_equal(a, b), hc                # refused: untouched
        else:
            assert np.array_equal(b[:64], a[1:65]), hc     # valid lists still applied


# ------------------------------------------------------------------ random scores
def test_random_scores_bit_exact():
    say("philox")
    wl = small(n_layers=2, n_requests=3, n_kv_heads=4, budget=512, prompt_len=200, seq_len=576)
    batch = synth.make_batch(wl)
    N, P = [576, 555, 301], [200, 203, 0]
    cache = device_cache(batch, N, P)
    seed = 0xC0FFEE_1234_5678
    rid = torch.tensor([11, 2**40 + 5, 3], dtype=torch.int64).cuda()
    pss = torch.tensor([0, 7, 123456], dtype=torch.int32).cuda()
    stride = 600
    sc = torch.full((cache.n_head_caches, stride), -1, dtype=torch.int32).cuda()
    bk.bkv_random_score(cache, seed, rid, pss, sc)
    got = sc.cpu().numpy().view(np.uint32)
    for hc, layer, r, h in head_iter(cache):
        ref = oracle.random_score(seed, int(rid[r]), int(pss[r]), layer, h, N[r], P[r])
        assert np.array_equal(got[hc, :N[r] - P[r]], ref), hc
        assert np.all(got[hc, N[r] - P[r]:] == 0xFFFFFFFF), hc


# ------------------------------------------------------------------ selection
def test_select_bit_exact_on_draws_and_tied_floats():
    say("select u32/f32")
    wl = small(n_layers=1, n_requests=4, n_kv_heads=4, budget=512, prompt_len=200, seq_len=1500)
    batch = synth.make_batch(wl)
    N, P, B = [576, 1500, 700, 513], [200, 0, 511, 100], 512
    cache = device_cache(batch, N, P)
    stride = 1500
    rid = torch.arange(4, dtype=torch.int64).cuda()
    pss = torch.zeros(4, dtype=torch.int32).cuda()
    u = torch.zeros((cache.n_head_caches, stride), dtype=torch.int32).cuda()
    bk.bkv_random_score(cache, 99, rid, pss, u)
    keep = torch.full((cache.n_head_caches, B), -7, dtype=torch.int32).cuda()
    bk.bkv_topk_select(cache, u, B, keep)
    un = u.cpu().numpy().view(np.uint32)
    kn = keep.cpu().numpy()
    for hc, layer, r, h in head_iter(cache):
        ref = oracle.topk_select(un[hc, :N[r] - P[r]], N[r], P[r], B)
        assert np.array_equal(keep_rows(kn[hc]), ref), hc
    # fp32 scores with heavy ties (few distinct values) and window-like values
    rng = np.random.default_rng(5)
    f = (np.round(rng.random((cache.n_head_caches, stride)) * 6) / 6).astype(np.float32)
    f[:, ::5] += 1.0
    f[:, 7] = 0.0
    fs = torch.from_numpy(f).cuda()
    bk.bkv_topk_select(cache, fs, B, keep)
    kn = keep.cpu().numpy()
    for hc, layer, r, h in head_iter(cache):
        ref = oracle.topk_select(f[hc, :N[r] - P[r]].astype(np.float64), N[r], P[r], B)
        assert np.array_equal(keep_rows(kn[hc]), ref), hc


def test_select_edge_cases():
    say("select edges")
    wl = small(n_layers=1, n_requests=5, n_kv_heads=2, budget=512, prompt_len=200, seq_len=608)
    batch = synth.make_batch(wl)
    # (N, P): normal, N <= B, P == B, P > B (refused), empty
    N, P, B = [576, 300, 576, 600, 0], [200, 100, 512, 600, 0], 512
    cache = device_cache(batch, N, P)
    stride = 608
    rng = np.random.default_rng(3)
    f = rng.random((cache.n_head_caches, stride)).astype(np.float32)
    keep = torch.full((cache.n_head_caches, B), -7, dtype=torch.int32).cuda()
    st = bk.bkv_topk_select(cache, torch.from_numpy(f).cuda(), B, keep, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 1 << bk.BKV_ERR_BUDGET
    kn = keep.cpu().numpy()
    for hc, layer, r, h in head_iter(cache):
        if r == 3:
            assert np.all(kn[hc] == -7), "refused request must stay untouched"
            continue
        ref = oracle.topk_select(f[hc, :N[r] - P[r]].astype(np.float64), N[r], P[r], B)
        assert np.array_equal(keep_rows(kn[hc]), ref), (hc, r)
        assert np.all(kn[hc, len(ref):] == -1), (hc, r)


def test_select_one_shot_32k_candidates():
    say("select 32k")
    wl = small(n_layers=1, n_requests=1, n_kv_heads=2, budget=2048, prompt_len=512,
               seq_len=32768, n_clusters=4)
    batch = synth.make_batch(wl)
    cache = device_cache(batch)
    stride = 32768
    rid = torch.tensor([5], dtype=torch.int64).cuda()
    pss = torch.tensor([3], dtype=torch.int32).cuda()
    u = torch.zeros((cache.n_head_caches, stride), dtype=torch.int32).cuda()
    bk.bkv_random_score(cache, 1, rid, pss, u)
    keep = torch.zeros((cache.n_head_caches, 2048), dtype=torch.int32).cuda()
    bk.bkv_topk_select(cache, u, 2048, keep)
    un, kn = u.cpu().numpy().view(np.uint32), keep.cpu().numpy()
    for hc in range(cache.n_head_caches):
        ref = oracle.topk_select(un[hc, :32768 - 512], 32768, 512, 2048)
        assert np.array_equal(kn[hc], ref), hc


# ------------------------------------------------------------------ maintenance
@pytest.mark.parametrize("K,prewarm,G,T,cap", [
    (5, False, 4, 16, 0), (64, True, 4, 64, 0), (128, True, 4, 64, 0), (256, True, 8, 64, 0),
    (64, False, 1, 256, 0), (40, True, 2, 33, 0),
    # a final chunk of one step; every step of a K = 256 set filling empty rows
    (64, True, 1, 33, 0), (256, False, 8, 5, 0),
    # capped counts (moving average once a row is full)
    (128, True, 4, 64, 16), (64, True, 4, 64, 8), (5, False, 4, 16, 1), (40, True, 2, 33, 3)])
def test_beacon_update_teacher_forced(K, prewarm, G, T, cap):
    say("update", K, prewarm, G, T, "cap", cap)
    wl = small(n_layers=1, n_requests=2, n_kv_heads=2, n_beacons=K, group=G, steps=T,
               prewarm=prewarm, budget=512, prompt_len=200, seq_len=576)
    batch = synth.make_batch(wl)
    q = batch.queries.cuda()
    b = batch.beacons.cuda()
    c = batch.counts.cuda()
    HC = q.shape[0]
    assign = torch.full((HC, T * G), -1, dtype=torch.int32).cuda()
    bk.bkv_beacon_update(q, b, c, assign, count_cap=cap)
    torch.cuda.synchronize()
    qb = synth.bits(batch.queries)
    bg, cg, ag = b.cpu().numpy(), c.cpu().numpy(), assign.cpu().numpy()
    inexact, worst = 0, 0.0
    for hc in range(HC):
        ob, oc, gap = oracle.beacon_update_forced(qb[hc], batch.beacons[hc].numpy(),
                                                  batch.counts[hc].numpy(), ag[hc], cap=cap)
        assert np.all(np.isfinite(gap)) and gap.max() <= ASSIGN_TOL, (hc, gap.max())
        inexact += int((gap > 0).sum())
        worst = max(worst, float(gap.max()))
        assert np.array_equal(oc, cg[hc]), hc
        assert np.array_equal(ob.view(np.int32), bg[hc].view(np.int32)), hc
    say("update", K, "picks below the oracle's best cosine:", inexact, "largest gap:", worst)
    assert inexact <= INEXACT_LIMIT, (inexact, worst)


def _near_tie_rows(b, c, rng):
    """Every other row a near copy of its neighbour (a relative change of about
    1e-6, inside the chain's error bound) and some rows exact copies, so
    queries meet near ties and exact ties over and over."""
    K = b.shape[1]
    for j in range(0, K - 1, 2):
        b[:, j + 1] = b[:, j] * (1 + torch.from_numpy(rng.normal(0, 1e-6, (b.shape[0], 128))).float())
        c[:, j + 1] = c[:, j]
    b[:, K - 1] = b[:, 0]
    c[:, K - 1] = c[:, 0]


@pytest.mark.parametrize("case,K,G,T,cap", [
    ("near_ties", 64, 4, 64, 0), ("near_ties", 128, 4, 64, 0), ("near_ties", 256, 8, 32, 0),
    ("near_ties", 40, 2, 33, 3), ("zero_queries", 64, 4, 16, 0), ("opposed", 5, 4, 16, 0),
    ("opposed", 128, 2, 32, 0), ("cap_one", 64, 4, 16, 1), ("extreme_norms", 128, 4, 64, 0),
    ("extreme_norms", 256, 2, 48, 0), ("garbage_unfilled", 64, 4, 32, 0),
    ("garbage_unfilled", 128, 2, 48, 2)])
def test_beacon_update_teacher_forced_adversarial(case, K, G, T, cap):
    """Near ties, exact ties, zero queries, queries opposed to every beacon
    (all cosines negative, where the chain's error bound does not hold and its
    rows are re-ranked exactly), row and query norms far outside the bound's
    range (2^+-35 and beyond), and never-filled rows holding NaN and infinity:
    every pick must still be the oracle's argmax."""
    say("update adversarial", case, K, G, T, "cap", cap)
    wl = small(n_layers=1, n_requests=2, n_kv_heads=2, n_beacons=K, group=G, steps=T,
               prewarm=True, budget=512, prompt_len=200, seq_len=576)
    batch = synth.make_batch(wl)
    rng = np.random.default_rng(K * 7 + T)
    b, c, qv = batch.beacons.clone(), batch.counts.clone(), batch.queries.float().clone()
    if case == "near_ties":
        _near_tie_rows(b, c, rng)
        # queries aimed at the tied rows themselves
        pick = torch.from_numpy(rng.integers(0, K, qv.shape[:3]))
        aim = torch.gather(b, 1, pick.reshape(pick.shape[0], -1, 1).expand(-1, -1, 128))
        qv = torch.where(torch.from_numpy(rng.random(qv.shape[:3]) < 0.5)[..., None],
                         aim.reshape(qv.shape), qv)
    elif case == "zero_queries":
        qv[:, ::3] = 0.0
    elif case in ("opposed", "cap_one"):
        # every query points away from the mean of the beacons
        qv = -b.mean(1, keepdim=True)[:, :, None, :].expand_as(qv) * 3 + 0.1 * qv
    elif case == "extreme_norms":
        # rows and queries scaled far above and below the covered norm range
        b[:, 0::3] *= 2.0 ** 35
        b[:, 1::5] *= 2.0 ** -40
        flat = qv.reshape(qv.shape[0], -1, 128)
        flat[:, 0::4] *= 2.0 ** 36
        flat[:, 1::7] *= 2.0 ** -38
        qv = flat.reshape(qv.shape)
    elif case == "garbage_unfilled":
        # never-filled rows whose stored values are NaN and infinity: the fill
        # replaces them, and nothing may read them before
        dead = torch.from_numpy(rng.choice(K, size=K // 6, replace=False))
        c[:, dead] = 0
        b[:, dead] = float("nan")
        b[:, dead[::2], ::3] = float("inf")
    q = qv.to(torch.bfloat16)
    HC = q.shape[0]
    qd, bd, cd = q.cuda(), b.cuda(), c.cuda()
    assign = torch.full((HC, T * G), -1, dtype=torch.int32).cuda()
    bk.bkv_beacon_update(qd, bd, cd, assign, count_cap=cap)
    torch.cuda.synchronize()
    qb = synth.bits(q)
    bg, cg, ag = bd.cpu().numpy(), cd.cpu().numpy(), assign.cpu().numpy()
    inexact, worst = 0, 0.0
    for hc in range(HC):
        ob, oc, gap = oracle.beacon_update_forced(qb[hc], b[hc].numpy(), c[hc].numpy(), ag[hc],
                                                  cap=cap)
        assert np.all(np.isfinite(gap)) and gap.max() <= ASSIGN_TOL, (hc, gap.max())
        inexact += int((gap > 0).sum())
        worst = max(worst, float(gap.max()))
        assert np.array_equal(oc, cg[hc]), hc
        assert np.array_equal(ob.view(np.int32), bg[hc].view(np.int32)), hc
    say("update adversarial", case, K, "picks below the oracle's best cosine:", inexact,
        "largest gap:", worst)
    assert inexact <= INEXACT_LIMIT, (inexact, worst)


@pytest.mark.parametrize("seed", range(8))
def test_beacon_update_random_shapes(seed):
    """Seeded random maintenance shapes beside the hand-picked ones: K on and
    off the 32-row blocks, G, T (ragged last chunks), the count cap (1
    included), an empty or prewarmed state and, half the time, rows pushed
    into near and exact ties.  Teacher-forced against the oracle: every pick
    its argmax, counts and beacons bit for bit."""
    rng = np.random.default_rng(5000 + seed)
    K = int(rng.choice([1, 3, 31, 32, 33, 64, 65, 100, 128, 129, 200, 256]))
    G, T = int(rng.choice([1, 2, 3, 4, 8])), int(rng.integers(1, 50))
    cap = int(rng.choice([0, 0, 1, 2, 7, 64]))
    R, H = int(rng.integers(1, 4)), int(rng.integers(1, 3))
    prewarm, ties = bool(rng.integers(0, 2)), bool(rng.integers(0, 2)) and K >= 2
    say("update random shape", seed, dict(K=K, G=G, T=T, cap=cap, R=R, H=H, prewarm=prewarm,
                                          ties=ties))
    wl = small(n_layers=1, n_requests=R, n_kv_heads=H, n_beacons=K, group=G, steps=T,
               prewarm=prewarm, budget=512, prompt_len=100, seq_len=300, seed=90 + seed)
    batch = synth.make_batch(wl)
    b, c = batch.beacons.clone(), batch.counts.clone()
    if ties:
        _near_tie_rows(b, c, rng)
    HC = b.shape[0]
    qd, bd, cd = batch.queries.cuda(), b.cuda(), c.cuda()
    assign = torch.full((HC, T * G), -1, dtype=torch.int32).cuda()
    bk.bkv_beacon_update(qd, bd, cd, assign, count_cap=cap)
    torch.cuda.synchronize()
    qb = synth.bits(batch.queries)
    bg, cg, ag = bd.cpu().numpy(), cd.cpu().numpy(), assign.cpu().numpy()
    inexact = 0
    for hc in range(HC):
        ob, oc, gap = oracle.beacon_update_forced(qb[hc], b[hc].numpy(), c[hc].numpy(), ag[hc],
                                                  cap=cap)
        assert np.all(np.isfinite(gap)) and gap.max() <= ASSIGN_TOL, (hc, gap.max())
        inexact += int((gap > 0).sum())
        assert np.array_equal(oc, cg[hc]), hc
        assert np.array_equal(ob.view(np.int32), bg[hc].view(np.int32)), hc
    assert inexact <= INEXACT_LIMIT, inexact


# ------------------------------------------------------------------ scoring
def _score_case(wl, N, P, kill=(), window=64, bonus=1.0, mutate=None):
    batch = synth.make_batch(wl)
    if mutate:
        mutate(batch)
    cache = device_cache(batch, N, P)
    b = batch.beacons.clone()
    c = batch.counts.clone()
    for hc, j in kill:
        c[hc, j] = 0
    K = b.shape[1]
    stride = max(n - p for n, p in zip(N, P)) + 3
    sc = torch.full((cache.n_head_caches, stride), float("nan")).cuda()
    lse = torch.zeros((cache.n_head_caches, K)).cuda()
    bk.bkv_beacon_score(cache, b.cuda(), c.cuda(), sc, window=window, bonus=bonus, lse=lse)
    k_in, _ = host_pools(cache)
    bt = batch.block_table.numpy()
    scn, lsen = sc.cpu().numpy(), lse.cpu().numpy()
    for hc, layer, r, h in head_iter(cache):
        keys = oracle.gather_paged(k_in[layer], bt[r], h, N[r])
        os_, ol = oracle.beacon_score(keys, b[hc].numpy(), c[hc].numpy(), P[r], window, bonus)
        check_scores(scn[hc, :N[r] - P[r]], os_, f"hc {hc}")
        assert np.all(np.isnan(scn[hc, N[r] - P[r]:])), "wrote past N - P"
        live = c[hc].numpy() > 0
        assert np.all(np.isnan(lsen[hc][~live]))
        if live.any() and N[r] > 0:
            assert np.max(np.abs(lsen[hc][live] - ol[live])) <= 1e-3, hc
    return batch


@pytest.mark.parametrize("K", [1, 5, 64, 128, 256])
def test_beacon_score_parity(K):
    say("score", K)
    wl = small(n_layers=1, n_requests=3, n_kv_heads=2, n_beacons=K, budget=512, prompt_len=200,
               seq_len=1040)
    _score_case(wl, N=[1040, 577, 31], P=[200, 576, 0], kill=[(0, 0), (3, K - 1)])


def test_beacon_score_prompt_boundaries():
    """Phase 2 starts at the tile holding slot P: no candidates (P = N, with N
    on and off a tile boundary), and P on a tile boundary."""
    say("score prompt boundaries")
    wl = small(n_layers=1, n_requests=4, n_kv_heads=2, n_beacons=128, budget=1024,
               prompt_len=200, seq_len=640)
    _score_case(wl, N=[640, 333, 128, 97], P=[640, 333, 96, 32])


def test_beacon_score_no_live_beacons():
    say("score empty J")
    wl = small(n_layers=1, n_requests=1, n_kv_heads=2, n_beacons=64, prewarm=False,
               budget=512, prompt_len=100, seq_len=300)
    _score_case(wl, N=[300], P=[100])


def test_beacon_score_extreme_logit_spread_uses_exact_fallback():
    say("score rescue")
    wl = small(n_layers=1, n_requests=2, n_kv_heads=2, n_beacons=64, budget=512, prompt_len=100,
               seq_len=600)

    def mutate(batch):
        k = batch.k_pools[0].float()
        bt = batch.block_table
        # request 0: one late block of huge keys -> overflow of the running sum
        k[bt[0, 30]] *= 40.0
        batch.k_pools[0] = k.to(torch.bfloat16)
        # request 1: beacon 0 enormous, beacon 1 tiny -> underflow of beacon 1
        for h in range(2):
            hc = 1 * 2 + h
            batch.beacons[hc, 0] *= 60.0
            batch.beacons[hc, 1] *= 1e-4
    _score_case(wl, N=[600, 600], P=[100, 100], mutate=mutate)


def test_beacon_score_one_shot_long():
    say("score one-shot 4096")
    _score_case(synth.WORKLOADS["tiny"].with_(prewarm=True), N=[4096], P=[512])


# ------------------------------------------------------------------ whole pass
def _pass_case(wl, N, P, B, selector, seed=17, shared=False, separate=False, mutate=None):
    """One bkv_evict_pass against the oracle.  shared=True: one selection per
    (layer, request) for all its heads (beacon: merged per-head scores;
    random: one draw row with the head field 0).  separate=True: score,
    select and compact as three kernels instead of the fused one.  The beacon
    selector's lse output is checked too."""
    batch = synth.make_batch(wl)
    if mutate:
        mutate(batch)
    cache = device_cache(batch, N, P)
    k_in, v_in = host_pools(cache)
    bt = batch.block_table.numpy()
    L, R, H = cache.n_layers, cache.n_requests, cache.n_kv_heads
    HC, S = cache.n_head_caches, cache.max_slots
    pos = np.tile(np.arange(S, dtype=np.int32), (HC, 1))
    pos_dev = torch.from_numpy(pos).cuda()
    keep = torch.full((L * R if shared else HC, B), -7, dtype=torch.int32).cuda()
    if selector == "beacon":
        q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
        T, G = q.shape[1], q.shape[2]
        assign = torch.zeros((HC, T * G), dtype=torch.int32).cuda()
        sc = torch.zeros((HC, S)).cuda()
        lse = torch.zeros((HC, b.shape[1])).cuda()
        bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                          window=64, bonus=1.0, assign=assign, pos_ids=pos_dev, scores_out=sc,
                          keep_out=keep, shared_positions=shared, separate_steps=separate,
                          lse=lse)
    else:
        rid = torch.arange(100, 100 + cache.n_requests, dtype=torch.int64).cuda()
        pss = torch.full((cache.n_requests,), 4, dtype=torch.int32).cuda()
        sc = torch.zeros((L * R if shared else HC, S), dtype=torch.int32).cuda()
        bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=seed, request_ids=rid,
                          pass_idx=pss, pos_ids=pos_dev, scores_out=sc, keep_out=keep,
                          shared_positions=shared, separate_steps=separate)
    torch.cuda.synchronize()
    k_out, v_out = host_pools(cache)
    kn, scn, posn = keep.cpu().numpy(), sc.cpu().numpy(), pos_dev.cpu().numpy()
    qb = synth.bits(batch.queries)
    mism = 0
    keys, vals, kept = {}, {}, {}
    for layer in range(L):
        for r in range(R):
            n, p = N[r], P[r]
            hcs = [hc_index(R, H, layer, r, h) for h in range(H)]
            for h, hc in enumerate(hcs):
                keys[hc] = oracle.gather_paged(k_in[layer], bt[r], h, n)
                vals[hc] = oracle.gather_paged(v_in[layer], bt[r], h, n)
            if selector == "beacon":
                os_, gs = [], []
                for hc in hcs:
                    ob, oc, gap = oracle.beacon_update_forced(qb[hc], batch.beacons[hc].numpy(),
                                                              batch.counts[hc].numpy(),
                                                              assign[hc].cpu().numpy())
                    assert gap.max() <= ASSIGN_TOL, hc
                    assert np.array_equal(ob.view(np.int32), b[hc].cpu().numpy().view(np.int32))
                    assert np.array_equal(oc, c[hc].cpu().numpy()), hc
                    o, ol = oracle.beacon_score(keys[hc], ob, oc, p, 64, 1.0)
                    check_scores(scn[hc, :n - p], o, f"pass hc {hc}")
                    live, ln = oc > 0, lse[hc].cpu().numpy()
                    assert np.all(np.isnan(ln[~live])), hc
                    if live.any() and n > 0:
                        assert np.max(np.abs(ln[live] - ol[live])) <= 1e-3, hc
                    os_.append(o)
                    gs.append(scn[hc, :n - p].astype(np.float64))
                if shared:
                    u = layer * R + r
                    kp = keep_rows(kn[u])
                    ref = oracle.shared_select(np.stack(os_), n, p, B)
                    merged = np.max(np.stack(os_), axis=0)
                    mism += check_selection(kp, ref, merged, n, p, B, f"shared pass {u}")
                    assert np.array_equal(kp, oracle.shared_select(np.stack(gs), n, p, B)), u
                    for hc in hcs:
                        kept[hc] = kp
                else:
                    for hc, o, g in zip(hcs, os_, gs):
                        kp = keep_rows(kn[hc])
                        ref = oracle.topk_select(o, n, p, B)
                        mism += check_selection(kp, ref, o, n, p, B, f"pass hc {hc}")
                        assert np.array_equal(kp, oracle.topk_select(g, n, p, B)), hc
                        kept[hc] = kp
            else:
                if shared:
                    u = layer * R + r
                    draw = oracle.random_score(seed, 100 + r, 4, layer, 0, n, p)
                    assert np.array_equal(scn[u, :n - p].view(np.uint32), draw), u
                    kp = keep_rows(kn[u])
                    assert np.array_equal(kp, oracle.shared_select(draw[None], n, p, B)), u
                    for hc in hcs:
                        kept[hc] = kp
                else:
                    for h, hc in enumerate(hcs):
                        draw = oracle.random_score(seed, 100 + r, 4, layer, h, n, p)
                        assert np.array_equal(scn[hc, :n - p].view(np.uint32), draw), hc
                        kp = keep_rows(kn[hc])
                        assert np.array_equal(kp, oracle.topk_select(draw, n, p, B)), hc
                        kept[hc] = kp
    for hc, layer, r, h in head_iter(cache):
        kp = kept[hc]
        nk = len(kp)
        ko = oracle.gather_paged(k_out[layer], bt[r], h, N[r])
        vo = oracle.gather_paged(v_out[layer], bt[r], h, N[r])
        assert np.array_equal(ko[:nk], oracle.kv_compact(keys[hc], kp)), hc
        assert np.array_equal(vo[:nk], oracle.kv_compact(vals[hc], kp)), hc
        assert np.array_equal(posn[hc, :nk], kp), hc
    say(selector, "shared" if shared else "per head", "selection differences at boundary ties:",
        mism)


@pytest.mark.parametrize("selector,separate", [("beacon", False), ("beacon", True),
                                               ("random", False), ("random", True)])
def test_evict_pass_end_to_end(selector, separate):
    say("pass", selector, "separate" if separate else "fused")
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, budget=512, prompt_len=200, seq_len=576)
    _pass_case(wl, N=[576, 541, 400], P=[200, 333, 100], B=512, selector=selector,
               separate=separate)


@pytest.mark.parametrize("seed", range(10))
def test_evict_pass_random_shapes(seed):
    """A seeded sweep of small shapes beside the hand-picked ones: K, G, T,
    the layer, request and head counts, the budget, paged or dense pools, a
    prewarmed or empty beacon state, ragged lengths and prompts per request
    (some at or under the budget, some prompts equal to it, empty caches),
    either selector, per head or shared, fused or separate; every output
    checked against the oracle as in the end-to-end test."""
    rng = np.random.default_rng(2000 + seed)
    K = int(rng.choice([1, 7, 32, 33, 64, 100, 128, 200, 256]))
    G, T = int(rng.choice([1, 2, 4, 8])), int(rng.integers(1, 41))
    L, R, H = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 3))
    B = int(rng.choice([64, 128, 256, 384]))
    S = B + int(rng.integers(1, 300))
    # request 0 always evicts; the others may be empty, full or anywhere between
    N = [S] + [0 if u < 0.1 else S if u < 0.4 else int(rng.integers(1, S + 1))
               for u in rng.random(R - 1)]
    P = [0 if u < 0.2 else min(n, B) if u < 0.35 else int(rng.integers(0, min(n, B) + 1))
         for n, u in zip(N, rng.random(R))]
    selector = "beacon" if seed % 3 else "random"
    shared, separate = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    paged, prewarm = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    say("random shape", seed, dict(K=K, G=G, T=T, L=L, R=R, H=H, B=B, N=N, P=P, sel=selector,
                                   shared=shared, separate=separate, paged=paged,
                                   prewarm=prewarm))
    wl = small(n_layers=L, n_requests=R, n_kv_heads=H, n_beacons=K, group=G, steps=T,
               budget=B, prompt_len=max(P), seq_len=S, paged=paged, prewarm=prewarm,
               seed=30 + seed)
    _pass_case(wl, N=N, P=P, B=B, selector=selector, seed=5 + seed, shared=shared,
               separate=separate)


@pytest.mark.parametrize("selector,K", [("beacon", 64), ("beacon", 128), ("beacon", 256),
                                        ("random", 128), ("shared", 128), ("shared", 256)])
def test_fused_pass_matches_separate_steps(selector, K):
    """The fused score-select-compact kernel leaves every output byte for byte
    as the three separate kernels do, with and without the optional keep and
    pos outputs, at lengths that exercise each branch: eviction, N <= B (no
    move), B == P (only the prompt survives), an empty cache, one eviction
    without a prompt, and a ragged last tile."""
    say("fused vs separate,", selector, "K", K)
    wl = small(n_layers=2, n_requests=6, n_kv_heads=2, budget=512, prompt_len=200, seq_len=608,
               n_beacons=K, steps=8)
    N, P, B = [576, 400, 600, 0, 513, 607], [200, 100, 512, 0, 0, 31], 512
    batch = synth.make_batch(wl)
    outs = []
    for separate, optional in ((True, True), (False, True), (False, False)):
        cache = device_cache(batch, N, P)
        HC, S = cache.n_head_caches, cache.max_slots
        q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
        pos = torch.arange(S, dtype=torch.int32).repeat(HC, 1).cuda() if optional else None
        rows = HC if selector != "shared" else cache.n_layers * cache.n_requests
        keep = torch.full((rows, B), -7, dtype=torch.int32).cuda() if optional else None
        if selector == "shared":
            sc = torch.zeros((HC, S)).cuda()
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                              pos_ids=pos, keep_out=keep, scores_out=sc, separate_steps=separate,
                              shared_positions=True)
        elif selector == "beacon":
            sc = torch.zeros((HC, S)).cuda()
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                              pos_ids=pos, keep_out=keep, scores_out=sc, separate_steps=separate)
        else:
            sc = torch.zeros((HC, S), dtype=torch.int32).cuda()
            rid = torch.arange(40, 40 + cache.n_requests, dtype=torch.int64).cuda()
            pss = torch.arange(cache.n_requests, dtype=torch.int32).cuda()
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=11, request_ids=rid,
                              pass_idx=pss, pos_ids=pos, keep_out=keep, scores_out=sc,
                              separate_steps=separate)
        torch.cuda.synchronize()
        k_out, v_out = host_pools(cache)
        outs.append(dict(b=b.cpu().numpy().view(np.int32), c=c.cpu().numpy(),
                         sc=sc.cpu().numpy().view(np.int32), k=k_out, v=v_out,
                         keep=None if keep is None else keep.cpu().numpy(),
                         pos=None if pos is None else pos.cpu().numpy()))
    ref = outs[0]
    for got in outs[1:]:
        for name in ("b", "c", "sc", "keep", "pos"):
            if got[name] is not None:
                assert np.array_equal(got[name], ref[name]), name
        for layer in range(wl.n_layers):
            assert np.array_equal(got["k"][layer], ref["k"][layer]), ("k", layer)
            assert np.array_equal(got["v"][layer], ref["v"][layer]), ("v", layer)
    # the separate path itself is pinned to the oracle elsewhere; here also
    # check the branches' keep lists directly
    kn = ref["keep"]
    for hc, layer, r, h in head_iter(cache):
        row = keep_rows(kn[layer * cache.n_requests + r if selector == "shared" else hc])
        if N[r] <= B:
            assert np.array_equal(row, np.arange(N[r])), hc
        elif B == P[r]:
            assert np.array_equal(row, np.arange(P[r])), hc
        else:
            assert len(row) == B and np.all(np.diff(row) > 0), hc


@pytest.mark.parametrize("selector,separate", [("beacon", False), ("beacon", True),
                                               ("random", False)])
def test_evict_pass_shared_positions(selector, separate):
    say("pass shared", selector, "separate" if separate else "default")
    wl = small(n_layers=2, n_requests=3, n_kv_heads=4, budget=512, prompt_len=200, seq_len=576)
    _pass_case(wl, N=[576, 541, 400], P=[200, 333, 100], B=512, selector=selector, shared=True,
               separate=separate)


def test_shared_select_standalone_entry_points():
    """bkv_random_score(shared) -> bkv_topk_select_shared -> bkv_kv_compact(keep_shared),
    and per-head fp32 scores merged over heads, with ties and the N <= B / P == B cases."""
    say("shared standalone")
    wl = small(n_layers=2, n_requests=4, n_kv_heads=4, budget=512, prompt_len=200, seq_len=700)
    batch = synth.make_batch(wl)
    N, P, B = [700, 512, 600, 300], [200, 512, 0, 100], 512
    cache = device_cache(batch, N, P)
    L, R, H = cache.n_layers, cache.n_requests, cache.n_kv_heads
    stride = 700
    rid = torch.arange(4, dtype=torch.int64).cuda() * 3 + 1
    pss = torch.tensor([2, 0, 9, 4], dtype=torch.int32).cuda()
    u = torch.full((L * R, stride), -1, dtype=torch.int32).cuda()
    bk.bkv_random_score(cache, 77, rid, pss, u, rows=bk.BKV_ROWS_PER_LAYER_REQUEST)
    keep = torch.full((L * R, B), -7, dtype=torch.int32).cuda()
    bk.bkv_topk_select_shared(cache, u, B, keep)
    un, kn = u.cpu().numpy().view(np.uint32), keep.cpu().numpy()
    for layer in range(L):
        for r in range(R):
            i = layer * R + r
            draw = oracle.random_score(77, int(rid[r]), int(pss[r]), layer, 0, N[r], P[r])
            assert np.array_equal(un[i, :N[r] - P[r]], draw), i
            assert np.array_equal(keep_rows(kn[i]), oracle.shared_select(draw[None], N[r], P[r],
                                                                          B)), i
    # per-head fp32 scores with heavy ties, merged by their maximum over the heads
    rng = np.random.default_rng(11)
    f = (np.round(rng.random((cache.n_head_caches, stride)) * 5) / 5).astype(np.float32)
    f[:, ::9] += 1.0
    bk.bkv_topk_select_shared(cache, torch.from_numpy(f).cuda(), B, keep)
    kn = keep.cpu().numpy()
    for layer in range(L):
        for r in range(R):
            i = layer * R + r
            rows = f[i * H:(i + 1) * H, :N[r] - P[r]].astype(np.float64)
            assert np.array_equal(keep_rows(kn[i]), oracle.shared_select(rows, N[r], P[r], B)), i
    # compaction applies the one list to every head
    k_in, v_in = host_pools(cache)
    bk.bkv_kv_compact(cache, keep, B, keep_shared=True)
    k_out, v_out = host_pools(cache)
    bt = batch.block_table.numpy()
    for hc, layer, r, h in head_iter(cache):
        kp = keep_rows(kn[layer * R + r])
        a = oracle.gather_paged(k_in[layer], bt[r], h, N[r])
        o = oracle.gather_paged(k_out[layer], bt[r], h, N[r])
        assert np.array_equal(o[:len(kp)], oracle.kv_compact(a, kp)), hc
        a = oracle.gather_paged(v_in[layer], bt[r], h, N[r])
        o = oracle.gather_paged(v_out[layer], bt[r], h, N[r])
        assert np.array_equal(o[:len(kp)], oracle.kv_compact(a, kp)), hc


def _page_outputs(cache, B):
    R, M = cache.n_requests, cache.max_blocks
    dev = torch.device("cuda")
    return (torch.full((R, B // 16), -7, dtype=torch.int32, device=dev),
            torch.full((R, M), -7, dtype=torch.int32, device=dev),
            torch.full((R,), -7, dtype=torch.int32, device=dev),
            torch.full((R, M), -7, dtype=torch.int32, device=dev))


def _check_pages(where, r, kp_row, bt_row_in, bt_row_out, n_out, fr_row, ref_pages, N, M):
    """GPU page outputs of request r against the oracle's pages and block-table rewrite."""
    kp = keep_rows(kp_row)
    assert np.array_equal(kp, ref_pages), (where, r, kp, ref_pages)
    row, freed, new_n = oracle.page_remap(bt_row_in, N, ref_pages)
    npages = -(-N // 16)
    assert np.array_equal(bt_row_out[:len(row)], row), (where, r)
    assert np.all(bt_row_out[len(row):npages] == -1), (where, r)
    assert np.array_equal(bt_row_out[npages:], bt_row_in[npages:]), (where, r)  # untouched
    assert n_out == new_n, (where, r, n_out, new_n)
    assert np.array_equal(fr_row[:len(freed)], freed), (where, r)
    assert np.all(fr_row[len(freed):] == -1), (where, r)


def test_page_retain_standalone():
    """bkv_random_score(rows per request) -> bkv_page_retain in place, and per-head fp32
    scores merged over every layer and head out of place; partial pages, unaligned
    prompts, nothing to evict and a refused request."""
    say("page retain standalone")
    wl = small(n_layers=3, n_requests=5, n_kv_heads=2, budget=512, prompt_len=200, seq_len=700)
    batch = synth.make_batch(wl)
    # (N, P): partial last page + unaligned prompt; aligned; N <= B; prompt fills the
    # budget exactly; too many forced pages (refused)
    N, P, B = [700, 640, 500, 688, 700], [201, 64, 100, 512, 510], 512
    cache = device_cache(batch, N, P)
    R, M, L, H = cache.n_requests, cache.max_blocks, cache.n_layers, cache.n_kv_heads
    stride = 700
    k_in, v_in = host_pools(cache)
    bt_in = batch.block_table.numpy().copy()
    rid = torch.arange(R, dtype=torch.int64).cuda() + 40
    pss = torch.tensor([1, 2, 3, 4, 5], dtype=torch.int32).cuda()
    u = torch.full((R, stride), -1, dtype=torch.int32).cuda()
    bk.bkv_random_score(cache, 5, rid, pss, u, rows=bk.BKV_ROWS_PER_REQUEST)
    kp, _, _, fr = _page_outputs(cache, B)
    st = bk.bkv_page_retain(cache, u, B, kp, cache.block_table, cache.seq_len, fr,
                            rows=bk.BKV_ROWS_PER_REQUEST, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 1 << bk.BKV_ERR_BUDGET       # request 4: 32 prompt pages + 1 partial
    un = u.cpu().numpy().view(np.uint32)
    kpn, btn, sln, frn = (kp.cpu().numpy(), cache.block_table.cpu().numpy(),
                          cache.seq_len.cpu().numpy(), fr.cpu().numpy())
    for r in range(R):
        draw = oracle.random_score(5, int(rid[r]), int(pss[r]), 0, 0, N[r], P[r])
        assert np.array_equal(un[r, :N[r] - P[r]], draw), r
        if r == 4:
            assert np.all(kpn[r] == -7) and np.array_equal(btn[r], bt_in[r]) and sln[r] == N[r]
            assert np.all(frn[r] == -7)
            continue
        ref = oracle.page_select(draw[None], N[r], P[r], B)
        _check_pages("random", r, kpn[r], bt_in[r], btn[r], sln[r], frn[r], ref, N[r], M)
    k_out, v_out = host_pools(cache)
    for layer in range(L):                       # no K/V row moved
        assert np.array_equal(k_in[layer], k_out[layer]) and np.array_equal(v_in[layer], v_out[layer])

    # per-head fp32 scores (heavy ties), out of place, on a fresh copy of the cache
    cache = device_cache(batch, N, P)
    rng = np.random.default_rng(21)
    f = (np.round(rng.random((cache.n_head_caches, stride)) * 7) / 7).astype(np.float32)
    kp, bto, slo, fr = _page_outputs(cache, B)
    st = bk.bkv_page_retain(cache, torch.from_numpy(f).cuda(), B, kp, bto, slo, fr, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 1 << bk.BKV_ERR_BUDGET
    kpn, bton, slon, frn = kp.cpu().numpy(), bto.cpu().numpy(), slo.cpu().numpy(), fr.cpu().numpy()
    for r in range(R):
        if r == 4:
            assert np.all(bton[r] == -7) and slon[r] == -7
            continue
        rows = np.stack([f[hc_index(R, H, layer, r, h), :N[r] - P[r]]
                         for layer in range(L) for h in range(H)]).astype(np.float64)
        ref = oracle.page_select(rows, N[r], P[r], B)
        row_out = bton[r].copy()
        row_out[row_out == -7] = bt_in[r][row_out == -7]   # entries the kernel leaves alone
        _check_pages("f32", r, kpn[r], bt_in[r], row_out, slon[r], frn[r], ref, N[r], M)
        assert np.all(bton[r][-(-N[r] // 16):] == -7), r   # beyond the old pages: untouched
    assert np.array_equal(cache.block_table.cpu().numpy(), bt_in)   # input table unchanged


def test_page_retain_edge_lengths():
    """Lengths at page boundaries: an empty request, a single slot, one partial page,
    no prompt with a partial last page, the prompt ending exactly on a page boundary,
    and a cache of whole pages with exactly one page over the budget."""
    say("page retain edges")
    wl = small(n_layers=1, n_requests=7, n_kv_heads=2, budget=64, prompt_len=0, seq_len=96)
    batch = synth.make_batch(wl)
    N = [0, 1, 15, 83, 96, 80, 96]
    P = [0, 0, 3, 0, 32, 16, 64]
    B = 64
    cache = device_cache(batch, N, P)
    R, M = cache.n_requests, cache.max_blocks
    bt_in = batch.block_table.numpy().copy()
    stride = 96
    rng = np.random.default_rng(8)
    f = rng.random((cache.n_head_caches, stride)).astype(np.float32)
    kp, _, _, fr = _page_outputs(cache, B)
    bk.bkv_page_retain(cache, torch.from_numpy(f).cuda(), B, kp, cache.block_table,
                       cache.seq_len, fr)
    torch.cuda.synchronize()
    kpn, btn, sln, frn = (kp.cpu().numpy(), cache.block_table.cpu().numpy(),
                          cache.seq_len.cpu().numpy(), fr.cpu().numpy())
    H = cache.n_kv_heads
    for r in range(R):
        rows = np.stack([f[hc_index(R, H, 0, r, h), :N[r] - P[r]] for h in range(H)])
        ref = oracle.page_select(rows.astype(np.float64), N[r], P[r], B)
        _check_pages("edges", r, kpn[r], bt_in[r], btn[r], sln[r], frn[r], ref, N[r], M)


def test_decode_attention_tiny_lengths():
    """N = 1, 2, 3, 4, 5 and 16, 17 slots with 8 query heads: the masking of the rows
    of the first and the last page."""
    say("attention tiny lengths")
    wl = small("qwen3_32b_r32", n_layers=1, n_requests=7, n_kv_heads=1, budget=64, seq_len=32,
               prompt_len=0)
    batch = synth.make_batch(wl)
    N = [1, 2, 3, 4, 5, 16, 17]
    cache = device_cache(batch, N, [0] * 7)
    k_in, v_in = host_pools(cache)
    bt = batch.block_table.numpy()
    q = batch.queries[:, 0].contiguous().cuda()
    out = torch.full((cache.n_head_caches, q.shape[1], 128), float("nan")).cuda()
    bk.bkv_decode_attention(cache, q, out)
    on, qn = out.cpu().numpy(), synth.bits(q)
    for hc, layer, r, h in head_iter(cache):
        keys = oracle.gather_paged(k_in[layer], bt[r], h, N[r])
        vals = oracle.gather_paged(v_in[layer], bt[r], h, N[r])
        _check_attention(on[hc], qn[hc], keys, vals, f"tiny N {N[r]}")


def _page_pass_case(wl, N, P, B, selector, seed=23):
    """bkv_evict_pass with page retention, in place on the cache's block table."""
    batch = synth.make_batch(wl)
    cache = device_cache(batch, N, P)
    k_in, v_in = host_pools(cache)
    bt_in = batch.block_table.numpy().copy()
    L, R, H = cache.n_layers, cache.n_requests, cache.n_kv_heads
    HC, S, M = cache.n_head_caches, cache.max_slots, cache.max_blocks
    kp, _, _, fr = _page_outputs(cache, B)
    outs = (cache.block_table, cache.seq_len, fr)
    if selector == "beacon":
        q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
        T, G = q.shape[1], q.shape[2]
        assign = torch.zeros((HC, T * G), dtype=torch.int32).cuda()
        sc = torch.zeros((HC, S)).cuda()
        bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                          window=64, bonus=1.0, assign=assign, scores_out=sc, keep_out=kp,
                          page_retention=outs)
    else:
        rid = torch.arange(100, 100 + R, dtype=torch.int64).cuda()
        pss = torch.full((R,), 4, dtype=torch.int32).cuda()
        sc = torch.zeros((R, S), dtype=torch.int32).cuda()
        bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=seed, request_ids=rid,
                          pass_idx=pss, scores_out=sc, keep_out=kp, page_retention=outs)
    torch.cuda.synchronize()
    k_out, v_out = host_pools(cache)
    for layer in range(L):                       # no K/V row moved
        assert np.array_equal(k_in[layer], k_out[layer]) and np.array_equal(v_in[layer], v_out[layer])
    scn = sc.cpu().numpy()
    kpn, btn, sln, frn = (kp.cpu().numpy(), cache.block_table.cpu().numpy(),
                          cache.seq_len.cpu().numpy(), fr.cpu().numpy())
    qb = synth.bits(batch.queries)
    for r in range(R):
        n, p = N[r], P[r]
        if selector == "beacon":
            rows = []
            for layer in range(L):
                for h in range(H):
                    hc = hc_index(R, H, layer, r, h)
                    ob, oc, gap = oracle.beacon_update_forced(qb[hc], batch.beacons[hc].numpy(),
                                                              batch.counts[hc].numpy(),
                                                              assign[hc].cpu().numpy())
                    assert gap.max() <= ASSIGN_TOL, hc
                    assert np.array_equal(ob.view(np.int32), b[hc].cpu().numpy().view(np.int32))
                    keys = oracle.gather_paged(k_in[layer], bt_in[r], h, n)
                    o, _ = oracle.beacon_score(keys, ob, oc, p, 64, 1.0)
                    check_scores(scn[hc, :n - p], o, f"page pass hc {hc}")
                    rows.append(scn[hc, :n - p].astype(np.float64))
            ref = oracle.page_select(np.stack(rows), n, p, B)
        else:
            draw = oracle.random_score(seed, 100 + r, 4, 0, 0, n, p)
            assert np.array_equal(scn[r, :n - p].view(np.uint32), draw), r
            ref = oracle.page_select(draw[None], n, p, B)
        _check_pages(selector, r, kpn[r], bt_in[r], btn[r], sln[r], frn[r], ref, n, M)


@pytest.mark.parametrize("selector", ["beacon", "random"])
def test_evict_pass_page_retention(selector):
    say("pass pages", selector)
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, budget=512, prompt_len=200, seq_len=584)
    _page_pass_case(wl, N=[584, 541, 400], P=[200, 333, 100], B=512, selector=selector)


@pytest.mark.parametrize("seed", range(6))
def test_evict_pass_page_retention_random_shapes(seed):
    """Page-retention passes over seeded random small shapes: the budget any
    multiple of 16, lengths on and off page boundaries (empty caches
    included), prompts up to a page under the budget, paged or dense pools,
    either selector; pages, the rewritten table, lengths and released blocks
    against the oracle."""
    rng = np.random.default_rng(3000 + seed)
    K = int(rng.choice([1, 33, 64, 128, 256]))
    G, T = int(rng.choice([1, 4, 8])), int(rng.integers(1, 33))
    L, R, H = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 3))
    B = 16 * int(rng.integers(2, 25))
    S = B + int(rng.integers(1, 300))
    N = [S] + [0 if u < 0.1 else S if u < 0.4 else int(rng.integers(1, S + 1))
               for u in rng.random(R - 1)]
    P = [int(rng.integers(0, max(0, min(n, B - 16)) + 1)) for n in N]
    selector = "beacon" if seed % 2 else "random"
    paged, prewarm = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    say("random page shape", seed, dict(K=K, G=G, T=T, L=L, R=R, H=H, B=B, N=N, P=P,
                                        sel=selector, paged=paged, prewarm=prewarm))
    wl = small(n_layers=L, n_requests=R, n_kv_heads=H, n_beacons=K, group=G, steps=T,
               budget=B, prompt_len=max(P), seq_len=S, paged=paged, prewarm=prewarm,
               seed=60 + seed)
    _page_pass_case(wl, N=N, P=P, B=B, selector=selector, seed=40 + seed)


# ------------------------------------------------------------------ decode attention
def _check_attention(out, q, keys, vals, where):
    ref = oracle.decode_attention(q, keys, vals)
    vmax = float(np.abs(bf16_values(vals)).max()) if len(vals) else 1.0
    err = np.abs(np.asarray(out, np.float64) - ref).max()
    assert err <= ATT_TOL * vmax, (where, err, vmax)


@pytest.mark.parametrize("G", [1, 3, 4, 8])
def test_decode_attention_parity(G):
    say("attention G", G)
    wl = small(n_layers=2, n_requests=6, n_kv_heads=2, budget=512, prompt_len=100, seq_len=576,
               group=G)
    batch = synth.make_batch(wl)
    N = [576, 0, 1, 5, 17, 331]
    cache = device_cache(batch, N, [0] * 6)
    k_in, v_in = host_pools(cache)
    bt = batch.block_table.numpy()
    q = batch.queries[:, -1].contiguous().cuda()         # the last buffered decode step
    out = torch.full((cache.n_head_caches, G, 128), float("nan")).cuda()
    bk.bkv_decode_attention(cache, q, out)
    on, qn = out.cpu().numpy(), synth.bits(q)
    for hc, layer, r, h in head_iter(cache):
        keys = oracle.gather_paged(k_in[layer], bt[r], h, N[r])
        vals = oracle.gather_paged(v_in[layer], bt[r], h, N[r])
        _check_attention(on[hc], qn[hc], keys, vals, f"G {G} hc {hc} N {N[r]}")


@pytest.mark.parametrize("seed", range(6))
def test_decode_attention_random_shapes(seed):
    """Seeded random attention shapes: G from 1 to 8, the layer, request and
    head counts, lengths from empty through one slot, page boundaries and
    ragged, paged or dense pools, the default scale or another; every output
    against the oracle."""
    rng = np.random.default_rng(6000 + seed)
    G = int(rng.integers(1, 9))
    L, R, H = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 3))
    S = int(rng.integers(1, 700))
    N = [S] + [int(rng.choice([0, 1, S, 16 * (S // 16), int(rng.integers(0, S + 1))]))
               for _ in range(R - 1)]
    paged = bool(rng.integers(0, 2))
    scale = [None, 0.05, 0.12][seed % 3]
    say("attention random shape", seed, dict(G=G, L=L, R=R, H=H, N=N, paged=paged,
                                             scale=scale))
    wl = small(n_layers=L, n_requests=R, n_kv_heads=H, group=G, steps=2, seq_len=S,
               prompt_len=0, budget=512, paged=paged, seed=120 + seed)
    batch = synth.make_batch(wl)
    cache = device_cache(batch, N, [0] * R)
    k_in, v_in = host_pools(cache)
    bt = batch.block_table.numpy()
    q = batch.queries[:, -1].contiguous().cuda()
    out = torch.full((cache.n_head_caches, G, 128), float("nan")).cuda()
    bk.bkv_decode_attention(cache, q, out, scale=scale)
    on, qn = out.cpu().numpy(), synth.bits(q)
    for hc, layer, r, h in head_iter(cache):
        keys = oracle.gather_paged(k_in[layer], bt[r], h, N[r])
        vals = oracle.gather_paged(v_in[layer], bt[r], h, N[r])
        ref = oracle.decode_attention(qn[hc], keys, vals, scale)
        vmax = float(np.abs(bf16_values(vals)).max()) if len(vals) else 1.0
        err = np.abs(np.asarray(on[hc], np.float64) - ref).max()
        assert err <= ATT_TOL * vmax, (hc, N[r], err, vmax)


def test_decode_attention_after_compaction():
    """The consumer of the pass: attention over the compacted cache (length set to the
    kept count) equals attention over the kept rows in their original slots."""
    say("attention after compaction")
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, budget=512, prompt_len=200, seq_len=576)
    batch = synth.make_batch(wl)
    N, P, B = [576, 541, 400], [200, 333, 100], 512
    cache = device_cache(batch, N, P)
    k_in, v_in = host_pools(cache)
    bt = batch.block_table.numpy()
    q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
    keep = torch.full((cache.n_head_caches, B), -7, dtype=torch.int32).cuda()
    bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                      keep_out=keep)
    cache.seq_len.copy_(torch.tensor([min(n, B) for n in N], dtype=torch.int32))
    ql = batch.queries[:, -1].contiguous().cuda()
    out = torch.zeros((cache.n_head_caches, ql.shape[1], 128)).cuda()
    bk.bkv_decode_attention(cache, ql, out)
    on, qn, kn = out.cpu().numpy(), synth.bits(ql), keep.cpu().numpy()
    for hc, layer, r, h in head_iter(cache):
        kp = keep_rows(kn[hc])
        keys = oracle.gather_paged(k_in[layer], bt[r], h, N[r])[kp]
        vals = oracle.gather_paged(v_in[layer], bt[r], h, N[r])[kp]
        _check_attention(on[hc], qn[hc], keys, vals, f"compacted hc {hc}")


def test_evict_pass_tiny_one_shot():
    say("pass tiny")
    _pass_case(synth.WORKLOADS["tiny"], N=[4096], P=[512], B=1024, selector="beacon")


@pytest.mark.parametrize("case", ["k256", "k64-rescue", "k128-sparse", "k256-shared", "k5-edges"])
def test_evict_pass_split_scoring(case):
    """More candidates and keep entries than a fused kernel holds, and few
    head-caches: the pass splits each head-cache's keys over several
    workgroups (partial log-sum-exps, merged, then each part's share of the
    candidates).  Covered: a request whose candidates span fewer tiles than
    there are parts, one with no prompt, a logit spread that overflows one
    part's running sum (its exact fallback), mostly never-filled beacons, and
    shared positions."""
    say("pass split", case)
    N, P, B = [12288, 4200, 9001], [512, 4090, 0], 4096
    assert max(N) + B > bk.FUSED_MAX_ENTRIES
    if case.startswith("k256"):
        wl = small("qwen3_32b_r32", n_layers=1, n_requests=3, n_kv_heads=2, budget=B,
                   seq_len=max(N), steps=8)
        _pass_case(wl, N, P, B, selector="beacon", shared=case == "k256-shared")
    elif case == "k64-rescue":
        wl = small(n_layers=1, n_requests=3, n_kv_heads=2, n_beacons=64, budget=B,
                   seq_len=max(N), steps=4)

        def mutate(batch):
            k = batch.k_pools[0].float()
            k[batch.block_table[0, 500]] *= 40.0   # a late block of huge keys, request 0
            batch.k_pools[0] = k.to(torch.bfloat16)
        _pass_case(wl, N, P, B, selector="beacon", mutate=mutate)
    elif case == "k128-sparse":
        wl = small(n_layers=1, n_requests=3, n_kv_heads=2, n_beacons=128, budget=B,
                   seq_len=max(N), steps=2, prewarm=False)
        _pass_case(wl, N, P, B, selector="beacon")
    else:
        # K = 5 (one 32-row block, so some row groups hold no beacons), an
        # empty request, and one whose 10 candidates sit in a single tile
        wl = small(n_layers=1, n_requests=3, n_kv_heads=2, n_beacons=5, budget=B,
                   seq_len=max(N), steps=2)
        _pass_case(wl, [12288, 0, 4100], [0, 0, 4090], B, selector="beacon")


def test_evict_pass_k256_group8():
    say("pass K=256")
    wl = small("qwen3_32b_r32", n_layers=1, n_requests=2, n_kv_heads=2, budget=1024,
               seq_len=1088)
    _pass_case(wl, N=[1088, 1000], P=[512, 512], B=1024, selector="beacon")


@pytest.mark.parametrize("selector", ["beacon", "random"])
def test_fused_kernels_at_their_lds_capacity(selector):
    """score_stride + budget exactly at the fused limit: the candidate keys and
    the keep list fill the LDS the fused kernels hold them in (more head-caches
    than CUs, so the standard layout runs), and the result equals the separate
    kernels'; one entry more and the pass runs the separate kernels."""
    say("fused at LDS capacity", selector)
    B, P, N = 4096, 0, 11776
    assert (N - P) + B == bk.FUSED_MAX_ENTRIES
    wl = small(n_layers=1, n_requests=33, n_kv_heads=8, n_beacons=64, budget=B, prompt_len=0,
               seq_len=N, steps=2)
    batch = synth.make_batch(wl)
    R = wl.n_requests
    outs = []
    for stride, separate in ((N - P, False), (N - P, True), (N - P + 1, False)):
        cache = device_cache(batch, [N] * R, [P] * R)
        HC = cache.n_head_caches
        assert HC > 256
        keep = torch.full((HC, B), -7, dtype=torch.int32).cuda()
        pos = torch.arange(cache.max_slots, dtype=torch.int32).repeat(HC, 1).cuda()
        if selector == "beacon":
            sc = torch.zeros((HC, stride)).cuda()
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=batch.queries.cuda(),
                              beacons=batch.beacons.cuda(), counts=batch.counts.cuda(),
                              keep_out=keep, scores_out=sc, pos_ids=pos, score_stride=stride,
                              separate_steps=separate)
        else:
            sc = torch.zeros((HC, stride), dtype=torch.int32).cuda()
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=3,
                              request_ids=torch.arange(R, dtype=torch.int64).cuda(),
                              pass_idx=torch.ones(R, dtype=torch.int32).cuda(), keep_out=keep,
                              scores_out=sc, pos_ids=pos, score_stride=stride,
                              separate_steps=separate)
        torch.cuda.synchronize()
        outs.append((keep.cpu(), pos.cpu(), sc[:, :N - P].cpu(),
                     cache.k_pools[0].view(torch.int16).cpu(),
                     cache.v_pools[0].view(torch.int16).cpu()))
    for got in outs[1:]:
        for x, y in zip(got, outs[0]):
            assert torch.equal(x, y)
    kn = outs[0][0].numpy()
    assert all(len(keep_rows(r)) == B and np.all(np.diff(keep_rows(r)) > 0) for r in kn)


@pytest.mark.parametrize("mode", ["beacon", "beacon-separate", "shared", "random"])
def test_evict_pass_skips_invalid_request_entirely(mode):
    """A request that fails a device check is left untouched by every kernel
    of the pass (fused or separate, per head or shared), and the others
    proceed."""
    say("pass atomic skip", mode)
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, budget=256, prompt_len=100, seq_len=320)
    batch = synth.make_batch(wl)
    bt = batch.block_table.clone()
    bt[2, 3] = wl.num_blocks + 5                         # request 2: bad block id
    batch.block_table = bt
    cache = device_cache(batch, [320, 320, 320], [100, 300, 100])   # request 1: P > B
    k_in, v_in = host_pools(cache)
    q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
    if mode == "random":
        rid = torch.arange(3, dtype=torch.int64).cuda()
        pss = torch.zeros(3, dtype=torch.int32).cuda()
        st = bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, 256, seed=5, request_ids=rid,
                               pass_idx=pss, check=False)
    else:
        st = bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, 256, queries=q, beacons=b, counts=c,
                               check=False, separate_steps=mode == "beacon-separate",
                               shared_positions=mode == "shared")
    torch.cuda.synchronize()
    assert int(st.item()) == (1 << bk.BKV_ERR_BUDGET) | (1 << bk.BKV_ERR_BLOCK_TABLE)
    k_out, v_out = host_pools(cache)
    bn = b.cpu().numpy()
    cn = c.cpu().numpy()
    btn = batch.block_table.numpy()
    if mode != "random":
        for hc, layer, r, h in head_iter(cache):
            if r in (1, 2):
                assert np.array_equal(bn[hc].view(np.int32),
                                      batch.beacons[hc].numpy().view(np.int32))
                assert np.array_equal(cn[hc], batch.counts[hc].numpy())
            else:
                assert cn[hc].sum() == batch.counts[hc].numpy().sum() + q.shape[1] * q.shape[2]
    # request 1's blocks and request 2's valid blocks are untouched; request 0 was compacted
    for layer in range(2):
        for blk in list(btn[1]) + [x for x in btn[2] if x < wl.num_blocks]:
            assert np.array_equal(k_in[layer][blk], k_out[layer][blk])
            assert np.array_equal(v_in[layer][blk], v_out[layer][blk])
    assert any(not np.array_equal(k_in[0][blk], k_out[0][blk]) for blk in btn[0])


@pytest.mark.parametrize("mode", ["split", "head_pages", "pages"])
def test_split_and_head_page_passes_replay_from_a_hip_graph(mode):
    """The same for a pass whose scoring splits each head-cache's keys over
    several workgroups (its partial log-sum-exps in the workspace), for a
    per-head page pass rewriting per-head rows in place, and for a
    per-request beacon page pass (its page keys formed in the workspace after
    a fill kernel zeroes them) rewriting the block table and lengths in place:
    three replays from restored inputs, each byte for byte the eager pass."""
    say("graph replay", mode)
    if mode == "split":
        N, P, B = [12288, 5000, 9001], [512, 100, 0], 4096
    else:
        N, P, B = [576, 541, 400], [200, 333, 100], 384
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, n_beacons=64, budget=B,
               prompt_len=max(P), seq_len=max(N), steps=4)
    batch = synth.make_batch(wl)
    cache = device_cache(batch, N, P)
    HC, S, M = cache.n_head_caches, cache.max_slots, cache.max_blocks
    q = batch.queries.cuda()
    b0, c0 = batch.beacons.cuda(), batch.counts.cuda()
    k0 = [k.clone() for k in cache.k_pools]
    v0 = [v.clone() for v in cache.v_pools]
    b, c = b0.clone(), c0.clone()
    sc = torch.zeros((HC, S)).cuda()
    st = torch.zeros(1, dtype=torch.int32).cuda()
    ws = torch.empty(4 << 20, dtype=torch.uint8).cuda()
    H, L = cache.n_kv_heads, cache.n_layers
    hrow0 = cache.block_table.repeat_interleave(H, 0).repeat(L, 1).contiguous()
    hlen0 = cache.seq_len.repeat_interleave(H).repeat(L).contiguous()
    hrow, hlen = hrow0.clone(), hlen0.clone()
    dropped = torch.zeros((HC, M), dtype=torch.int32).cuda()
    bt0, sl0 = cache.block_table.clone(), cache.seq_len.clone()
    freed = torch.zeros((cache.n_requests, M), dtype=torch.int32).cuda()
    pc = cache
    if mode == "head_pages":
        pc = bk.PagedCache(cache.k_pools, cache.v_pools, cache.block_table, cache.seq_len,
                           cache.prompt_len, head_block_table=hrow, head_seq_len=hlen)
        keep = torch.zeros((HC, B // 16), dtype=torch.int32).cuda()
    elif mode == "pages":
        keep = torch.zeros((cache.n_requests, B // 16), dtype=torch.int32).cuda()
    else:
        keep = torch.zeros((HC, B), dtype=torch.int32).cuda()

    def restore():
        b.copy_(b0)
        c.copy_(c0)
        hrow.copy_(hrow0)
        hlen.copy_(hlen0)
        cache.block_table.copy_(bt0)
        cache.seq_len.copy_(sl0)
        for dst, src in zip(cache.k_pools + cache.v_pools, k0 + v0):
            dst.copy_(src)

    def run():
        kw = {}
        if mode == "head_pages":
            kw = dict(page_retention=(hrow, hlen, dropped), page_heads=True)
        elif mode == "pages":
            kw = dict(page_retention=(cache.block_table, cache.seq_len, freed))
        bk.bkv_evict_pass(pc, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                          scores_out=sc, keep_out=keep, status=st, check=False, workspace=ws,
                          **kw)

    run()                                   # eager reference
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    outs = (b, c, sc, keep, hrow, hlen, dropped, cache.block_table, cache.seq_len, freed,
            *cache.k_pools, *cache.v_pools)
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on the capture stream
        restore()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        restore()
        if mode == "head_pages":
            dropped.fill_(-3)               # every entry is written again
        if mode == "pages":
            freed.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        for i, (x, y) in enumerate(zip(outs, ref)):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), (rep, i)


@pytest.mark.parametrize("mode", ["beacon", "shared", "random"])
def test_evict_pass_replays_from_a_hip_graph(mode):
    """The pass allocates nothing and sets no memory, so it can be captured: a
    captured pass (each fused kernel: per-head beacon, shared beacon, random),
    replayed several times from restored inputs (eager copies and
    synchronisations between replays), matches the eager pass byte for byte
    every time."""
    say("graph replay", mode)
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, budget=512, prompt_len=200, seq_len=576)
    batch = synth.make_batch(wl)
    N, P, B = [576, 541, 400], [200, 333, 100], 512
    cache = device_cache(batch, N, P)
    HC, S = cache.n_head_caches, cache.max_slots
    q = batch.queries.cuda()
    b0, c0 = batch.beacons.cuda(), batch.counts.cuda()
    k0 = [k.clone() for k in cache.k_pools]
    v0 = [v.clone() for v in cache.v_pools]
    b, c = b0.clone(), c0.clone()
    sc = torch.zeros((HC, S), dtype=torch.int32 if mode == "random" else torch.float32).cuda()
    rows = cache.n_layers * cache.n_requests if mode == "shared" else HC
    keep = torch.zeros((rows, B), dtype=torch.int32).cuda()
    st = torch.zeros(1, dtype=torch.int32).cuda()
    ws = torch.empty(1 << 20, dtype=torch.uint8).cuda()
    rid = torch.arange(7, 7 + cache.n_requests, dtype=torch.int64).cuda()
    pss = torch.full((cache.n_requests,), 3, dtype=torch.int32).cuda()

    def restore():
        b.copy_(b0)
        c.copy_(c0)
        for dst, src in zip(cache.k_pools + cache.v_pools, k0 + v0):
            dst.copy_(src)

    def run():
        if mode == "random":
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=9, request_ids=rid,
                              pass_idx=pss, scores_out=sc, keep_out=keep, status=st, check=False,
                              workspace=ws)
        else:
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                              scores_out=sc, keep_out=keep, status=st, check=False,
                              workspace=ws, shared_positions=mode == "shared")

    run()                                   # eager reference
    torch.cuda.synchronize()
    ref = [t.clone() for t in (b, c, sc, keep, *cache.k_pools, *cache.v_pools)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on the capture stream
        restore()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        got = (b, c, sc, keep, *cache.k_pools, *cache.v_pools)
        for i, (x, y) in enumerate(zip(got, ref)):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), (rep, i)

"""Per-head page retention (bkv_page_retain_heads, page_heads passes) and a
cache read through per-head page tables, against the oracle on the GPU.

Each head-cache keeps its own whole pages (Random Attention article, section
"发现二": contiguous blocks of up to 64 tokens keep accuracy; the selection
here is per head, the case the article compares common positions against).
The oracle of one head-cache's selection is the pinned page selection over
its one score row, and the rewrite of its row the pinned page remap."""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_beacon_amd import synth
from tests.gpu_util import ASSIGN_TOL, check_scores, device_cache, host_pools, keep_rows
from tests.test_gpu_parity import _check_attention, small

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


def _outputs(HC, M, B):
    dev = torch.device("cuda")
    return (torch.full((HC, B // 16), -7, dtype=torch.int32, device=dev),
            torch.full((HC, M), -7, dtype=torch.int32, device=dev),
            torch.full((HC,), -7, dtype=torch.int32, device=dev),
            torch.full((HC, M), -7, dtype=torch.int32, device=dev))


def _check_head(where, hc, kp_row, row_in, row_out, n_out, dr_row, ref_pages, N):
    """One head-cache's outputs against the oracle's pages and row rewrite."""
    kp = keep_rows(kp_row)
    assert np.array_equal(kp, ref_pages), (where, hc, kp, ref_pages)
    row, dropped, new_n = oracle.page_remap(row_in, N, ref_pages)
    npages = -(-N // 16)
    assert np.array_equal(row_out[:len(row)], row), (where, hc)
    assert np.all(row_out[len(row):npages] == -1), (where, hc)
    assert n_out == new_n, (where, hc, n_out, new_n)
    assert np.array_equal(dr_row[:len(dropped)], dropped), (where, hc)
    assert np.all(dr_row[len(dropped):] == -1), (where, hc)


def _head_rows(cache, bt, N):
    """Request rows and lengths repeated for every head-cache (the per-head
    tables a cache starts from)."""
    L, R, H = cache.n_layers, cache.n_requests, cache.n_kv_heads
    rows = np.stack([bt[(hc // H) % R] for hc in range(L * R * H)]).astype(np.int32)
    lens = np.array([N[(hc // H) % R] for hc in range(L * R * H)], np.int32)
    return rows, lens


def test_page_retain_heads_then_read_through_rows():
    """Per-head selection from the request rows (out of place; a partial last
    page, an unaligned prompt, nothing to evict, a refused request), then a
    second, smaller selection in place on the per-head rows, then decode
    attention, beacon scoring and row compaction read through those rows."""
    say("head pages: select, select again, read")
    wl = small(n_layers=2, n_requests=5, n_kv_heads=2, n_beacons=64, budget=512, prompt_len=200,
               seq_len=700)
    batch = synth.make_batch(wl)
    N, P, B = [700, 640, 500, 688, 700], [201, 64, 100, 512, 510], 512
    cache = device_cache(batch, N, P)
    L, R, H, M = cache.n_layers, cache.n_requests, cache.n_kv_heads, cache.max_blocks
    HC = cache.n_head_caches
    k_in, v_in = host_pools(cache)
    bt = batch.block_table.numpy().copy()
    stride = 700
    rng = np.random.default_rng(31)
    f = (np.round(rng.random((HC, stride)) * 7) / 7).astype(np.float32)   # heavy ties
    kp, hto, hlo, dr = _outputs(HC, M, B)
    st = bk.bkv_page_retain_heads(cache, torch.from_numpy(f).cuda(), B, kp, hto, hlo, dr,
                                  check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 1 << bk.BKV_ERR_BUDGET   # request 4: 32 prompt pages + 1 partial
    kpn, hton, hlon, drn = kp.cpu().numpy(), hto.cpu().numpy(), hlo.cpu().numpy(), dr.cpu().numpy()
    for hc in range(HC):
        r = (hc // H) % R
        if r == 4:
            assert np.all(kpn[hc] == -7) and np.all(hton[hc] == -7) and hlon[hc] == -7
            continue
        ref = oracle.page_select(f[hc, :N[r] - P[r]][None].astype(np.float64), N[r], P[r], B)
        _check_head("first", hc, kpn[hc], bt[r], hton[hc], hlon[hc], drn[hc], ref, N[r])
        assert np.all(hton[hc][-(-N[r] // 16):] == -7), hc   # beyond the old pages: untouched
    k_out, v_out = host_pools(cache)
    for layer in range(L):                                     # no K/V row moved
        assert np.array_equal(k_in[layer], k_out[layer]) and np.array_equal(v_in[layer], v_out[layer])
    # the heads of one request chose different pages somewhere (the point of the mode)
    assert any(not np.array_equal(kpn[hc], kpn[hc + 1]) for hc in range(0, HC, H)
               if (hc // H) % R != 4)

    # the per-head cache: the refused request keeps its request rows
    rows0, lens0 = _head_rows(cache, bt, N)
    for hc in range(HC):
        if (hc // H) % R != 4:
            rows0[hc] = np.where(hton[hc] == -7, rows0[hc], hton[hc])
            lens0[hc] = hlon[hc]
    hcache = bk.PagedCache(cache.k_pools, cache.v_pools, cache.block_table, cache.seq_len,
                           cache.prompt_len, head_block_table=torch.from_numpy(rows0).cuda(),
                           head_seq_len=torch.from_numpy(lens0).cuda())

    # second selection, in place, smaller budget (request 4 now fits: 512 slots... its
    # 33 forced pages still exceed 256 // 16, so it is refused again)
    B2 = 256
    P2 = [201, 64, 100, 240, 510]
    hcache.prompt_len.copy_(torch.tensor(P2, dtype=torch.int32))
    f2 = rng.random((HC, stride)).astype(np.float32)
    kp2, _, _, dr2 = _outputs(HC, M, B2)
    st = bk.bkv_page_retain_heads(hcache, torch.from_numpy(f2).cuda(), B2, kp2,
                                  hcache.head_block_table, hcache.head_seq_len, dr2, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 1 << bk.BKV_ERR_BUDGET
    kp2n, rows1, lens1, dr2n = (kp2.cpu().numpy(), hcache.head_block_table.cpu().numpy(),
                                hcache.head_seq_len.cpu().numpy(), dr2.cpu().numpy())
    for hc in range(HC):
        r = (hc // H) % R
        if r == 4:
            assert np.array_equal(rows1[hc], rows0[hc]) and lens1[hc] == lens0[hc]
            continue
        n = int(lens0[hc])
        ref = oracle.page_select(f2[hc, :n - P2[r]][None].astype(np.float64), n, P2[r], B2)
        _check_head("in place", hc, kp2n[hc], rows0[hc], rows1[hc], lens1[hc], dr2n[hc], ref, n)

    # decode attention through the per-head rows
    G = 4
    q = torch.randn((HC, G, 128), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    out = torch.full((HC, G, 128), float("nan")).cuda()
    bk.bkv_decode_attention(hcache, q.cuda(), out)
    torch.cuda.synchronize()
    on, qn = out.cpu().numpy(), synth.bits(q)
    for hc in range(HC):
        layer, h = hc // (R * H), hc % H
        n = int(lens1[hc])
        keys = oracle.gather_paged(k_in[layer], rows1[hc], h, n)
        vals = oracle.gather_paged(v_in[layer], rows1[hc], h, n)
        _check_attention(on[hc], qn[hc], keys, vals, f"head rows hc {hc}")

    # beacon scores through the per-head rows
    b, c = batch.beacons.cuda(), batch.counts.cuda()
    sst = max(int(lens1[hc]) - P2[(hc // H) % R] for hc in range(HC))
    sc = torch.full((HC, sst), float("nan")).cuda()
    bk.bkv_beacon_score(hcache, b, c, sc, window=64, bonus=1.0)
    torch.cuda.synchronize()
    scn = sc.cpu().numpy()
    for hc in range(HC):
        layer, r, h = hc // (R * H), (hc // H) % R, hc % H
        n = int(lens1[hc])
        keys = oracle.gather_paged(k_in[layer], rows1[hc], h, n)
        o, _ = oracle.beacon_score(keys, batch.beacons[hc].numpy(), batch.counts[hc].numpy(),
                                   P2[r], 64, 1.0)
        check_scores(scn[hc, :n - P2[r]], o, f"head rows score hc {hc}")

    # row compaction inside each head-cache's own pages
    Bc = 160
    keep = np.full((HC, Bc), -1, np.int32)
    for hc in range(HC):
        r = (hc // H) % R
        n = int(lens1[hc])
        nk = min(n, Bc)
        pr = min(P2[r], nk)
        rest = np.sort(rng.choice(np.arange(pr, n), nk - pr, replace=False)) if nk > pr else []
        keep[hc, :nk] = np.concatenate([np.arange(pr), rest]).astype(np.int32)
    bk.bkv_kv_compact(hcache, torch.from_numpy(keep).cuda(), Bc, check=False)
    torch.cuda.synchronize()
    k_c, v_c = host_pools(hcache)
    for hc in range(HC):
        layer, r, h = hc // (R * H), (hc // H) % R, hc % H
        n = int(lens1[hc])
        if P2[r] > Bc:
            continue      # refused (prompt over the budget): untouched, checked below
        kk = keep_rows(keep[hc])
        a = oracle.gather_paged(k_in[layer], rows1[hc], h, n)
        o = oracle.gather_paged(k_c[layer], rows1[hc], h, n)
        assert np.array_equal(o[:len(kk)], oracle.kv_compact(a, kk)), hc
        a = oracle.gather_paged(v_in[layer], rows1[hc], h, n)
        o = oracle.gather_paged(v_c[layer], rows1[hc], h, n)
        assert np.array_equal(o[:len(kk)], oracle.kv_compact(a, kk)), hc


def _head_page_pass_case(wl, N, P, B, B2, selector):
    """A whole pass with per-head page retention at budget B, each head-cache's
    pages from its own scores (beacon: after maintenance; random: its own draw
    row) written to per-head rows, then a second pass at budget B2 on the
    cache read through those rows; every output against the oracle."""
    batch = synth.make_batch(wl)
    cache = device_cache(batch, N, P)
    L, R, H, M, HC = (cache.n_layers, cache.n_requests, cache.n_kv_heads, cache.max_blocks,
                      cache.n_head_caches)
    bt = batch.block_table.numpy().copy()
    q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
    rid = torch.arange(R, dtype=torch.int64).cuda() + 7
    pss = torch.full((R,), 3, dtype=torch.int32).cuda()
    qb = synth.bits(batch.queries)
    k_in, _ = host_pools(cache)

    def run(pc, budget, rows_in, lens_in, b_in, c_in, seed):
        kp, hto, hlo, dr = _outputs(HC, M, budget)
        stride = M * 16
        sc = torch.zeros((HC, stride), dtype=torch.float32 if selector == "beacon" else torch.int32).cuda()
        assign = torch.zeros((HC, q.shape[1] * q.shape[2]), dtype=torch.int32).cuda()
        if selector == "beacon":
            bk.bkv_evict_pass(pc, bk.BKV_SELECT_BEACON, budget, queries=q, beacons=b, counts=c,
                              assign=assign, scores_out=sc, keep_out=kp,
                              page_retention=(hto, hlo, dr), page_heads=True)
        else:
            bk.bkv_evict_pass(pc, bk.BKV_SELECT_RANDOM, budget, seed=seed, request_ids=rid,
                              pass_idx=pss, scores_out=sc, keep_out=kp,
                              page_retention=(hto, hlo, dr), page_heads=True)
        torch.cuda.synchronize()
        kpn, hton, hlon, drn, scn = (kp.cpu().numpy(), hto.cpu().numpy(), hlo.cpu().numpy(),
                                     dr.cpu().numpy(), sc.cpu().numpy())
        for hc in range(HC):
            layer, r, h = hc // (R * H), (hc // H) % R, hc % H
            n = int(lens_in[hc])
            if selector == "beacon":
                ob, oc, gap = oracle.beacon_update_forced(qb[hc], b_in[hc], c_in[hc],
                                                          assign[hc].cpu().numpy())
                assert gap.max() <= ASSIGN_TOL, hc
                keys = oracle.gather_paged(k_in[layer], rows_in[hc], h, n)
                o, _ = oracle.beacon_score(keys, ob, oc, P[r], 64, 1.0)
                check_scores(scn[hc, :n - P[r]], o, f"pass scores hc {hc}")
                row = scn[hc, :n - P[r]].astype(np.float64)
            else:
                row = oracle.random_score(seed, 7 + r, 3, layer, h, n, P[r])
                assert np.array_equal(scn[hc, :n - P[r]].view(np.uint32), row), hc
            ref = oracle.page_select(row[None], n, P[r], budget)
            _check_head(selector, hc, kpn[hc], rows_in[hc], hton[hc], hlon[hc], drn[hc], ref, n)
        rows = rows_in.copy()
        for hc in range(HC):
            rows[hc] = np.where(hton[hc] == -7, rows[hc], hton[hc])
        return rows, hlon.copy()

    rows0, lens0 = _head_rows(cache, bt, N)
    b0, c0 = batch.beacons.numpy().copy(), batch.counts.numpy().copy()
    rows1, lens1 = run(cache, B, rows0, lens0, b0, c0, 11)
    # the second pass reads the cache through the per-head rows the first wrote
    hcache = bk.PagedCache(cache.k_pools, cache.v_pools, cache.block_table, cache.seq_len,
                           cache.prompt_len, head_block_table=torch.from_numpy(rows1).cuda(),
                           head_seq_len=torch.from_numpy(lens1).cuda())
    b1, c1 = b.cpu().numpy().copy(), c.cpu().numpy().copy()
    run(hcache, B2, rows1, lens1, b1, c1, 12)


@pytest.mark.parametrize("selector", ["beacon", "random"])
def test_evict_pass_per_head_pages(selector):
    """A whole pass with per-head page retention, then a second pass on the
    per-head cache."""
    say("pass head pages", selector)
    wl = small(n_layers=2, n_requests=3, n_kv_heads=2, n_beacons=64, budget=512, prompt_len=100,
               seq_len=900, steps=4)
    _head_page_pass_case(wl, N=[900, 777, 400], P=[100, 37, 64], B=512, B2=256,
                         selector=selector)


@pytest.mark.parametrize("seed", range(6))
def test_evict_pass_per_head_pages_random_shapes(seed):
    """The same over seeded random small shapes: K, G, T, the counts, both
    budgets (multiples of 16, the second at most the first), lengths on and
    off page boundaries with empty caches, prompts up to a page under the
    second budget, paged or dense pools, either selector."""
    rng = np.random.default_rng(4000 + seed)
    K = int(rng.choice([1, 33, 64, 128, 256]))
    G, T = int(rng.choice([1, 4, 8])), int(rng.integers(1, 33))
    L, R, H = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 3))
    B = 16 * int(rng.integers(3, 25))
    B2 = 16 * int(rng.integers(2, B // 16 + 1))
    S = B + int(rng.integers(1, 300))
    N = [S] + [0 if u < 0.1 else S if u < 0.4 else int(rng.integers(1, S + 1))
               for u in rng.random(R - 1)]
    P = [int(rng.integers(0, max(0, min(n, B2 - 16)) + 1)) for n in N]
    selector = "beacon" if seed % 2 else "random"
    paged, prewarm = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    say("random head-page shape", seed, dict(K=K, G=G, T=T, L=L, R=R, H=H, B=B, B2=B2, N=N,
                                             P=P, sel=selector, paged=paged, prewarm=prewarm))
    wl = small(n_layers=L, n_requests=R, n_kv_heads=H, n_beacons=K, group=G, steps=T,
               budget=B, prompt_len=max(P), seq_len=S, paged=paged, prewarm=prewarm,
               seed=80 + seed)
    _head_page_pass_case(wl, N=N, P=P, B=B, B2=B2, selector=selector)


def test_per_head_tables_skip_only_the_failing_head_cache():
    """With per-head page tables a device check fails for one head-cache only:
    a block id outside the pool in one row and a length past the table in
    another.  Those two head-caches are left untouched by every kernel of a
    per-head page pass (beacons, counts, rows, lengths); the others match a
    pass over the same cache without the faults."""
    say("head pages: per-head skip")
    wl = small(n_layers=1, n_requests=2, n_kv_heads=4, n_beacons=64, budget=256, prompt_len=64,
               seq_len=400, steps=4)
    batch = synth.make_batch(wl)
    N, P, B = [400, 333], [64, 40], 256
    cache = device_cache(batch, N, P)
    HC, M = cache.n_head_caches, cache.max_blocks
    bt = batch.block_table.numpy().copy()
    rows0, lens0 = _head_rows(cache, bt, N)
    bad_block, bad_len = 1, 6                    # head-cache 1: bad block id; 6: bad length
    faulty_rows, faulty_lens = rows0.copy(), lens0.copy()
    faulty_rows[bad_block, 3] = wl.num_blocks + 9
    faulty_lens[bad_len] = M * 16 + 5
    q = batch.queries.cuda()
    outs = {}
    for name, rows, lens in (("clean", rows0, lens0), ("faulty", faulty_rows, faulty_lens)):
        hc_ = bk.PagedCache(cache.k_pools, cache.v_pools, cache.block_table, cache.seq_len,
                            cache.prompt_len, head_block_table=torch.from_numpy(rows).cuda(),
                            head_seq_len=torch.from_numpy(lens).cuda())
        b, c = batch.beacons.cuda(), batch.counts.cuda()
        kp, _, _, dr = _outputs(HC, M, B)
        st = bk.bkv_evict_pass(hc_, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                               keep_out=kp, page_retention=(hc_.head_block_table,
                                                            hc_.head_seq_len, dr),
                               page_heads=True, check=False)
        torch.cuda.synchronize()
        outs[name] = (int(st.item()), b.cpu().numpy(), c.cpu().numpy(),
                      hc_.head_block_table.cpu().numpy(), hc_.head_seq_len.cpu().numpy(),
                      kp.cpu().numpy())
    st_c, b_c, c_c, r_c, l_c, k_c = outs["clean"]
    st_f, b_f, c_f, r_f, l_f, k_f = outs["faulty"]
    assert st_c == 0
    assert st_f == (1 << bk.BKV_ERR_BLOCK_TABLE) | (1 << bk.BKV_ERR_LENGTH), st_f
    b0, c0 = batch.beacons.numpy(), batch.counts.numpy()
    for hc in range(HC):
        if hc in (bad_block, bad_len):
            assert np.array_equal(b_f[hc].view(np.int32), b0[hc].view(np.int32)), hc
            assert np.array_equal(c_f[hc], c0[hc]), hc
            assert np.array_equal(r_f[hc], faulty_rows[hc]) and l_f[hc] == faulty_lens[hc], hc
            assert np.all(k_f[hc] == -7), hc
        else:
            assert np.array_equal(b_f[hc].view(np.int32), b_c[hc].view(np.int32)), hc
            assert np.array_equal(c_f[hc], c_c[hc]), hc
            assert np.array_equal(r_f[hc], r_c[hc]) and l_f[hc] == l_c[hc], hc
            assert np.array_equal(k_f[hc], k_c[hc]), hc

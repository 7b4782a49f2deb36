"""The HIP path against the golden files of tests/golden/ (oracle outputs on
seeded inputs, written by tests/golden/make_golden.py): a beacon pass, a
random pass and the page-retention passes on the same small paged batch.
Integer outputs (assignments, counts, keep lists, draws, pages, block rows,
lengths) and the updated beacons and compacted rows (by digest) must match
exactly; scores and log-sum-exps within the parity tolerances."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.golden import make_golden as G
from tests.gpu_util import check_scores, check_selection, device_cache, host_pools, keep_rows

pytestmark = pytest.mark.gpu

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
bk = None


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global bk
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from decode_kv_cache_beacon_amd import beaconkv
    bk = beaconkv
    yield


def say(*a):
    print("[case]", *a, flush=True)


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def golden_inputs(g):
    """The seeded batch, checked against the digests the file was written from."""
    x = G.inputs()
    assert G.input_digests(x) == g["inputs_sha256"], "the input generator changed"
    return x


def compacted_digests(cache, x, layer, r, h, n_keep):
    k_out, v_out = host_pools(cache)
    bt = x["bt"][r]
    ko = oracle.gather_paged(k_out[layer], bt, h, G.N[r])[:n_keep]
    vo = oracle.gather_paged(v_out[layer], bt, h, G.N[r])[:n_keep]
    return G.sha(ko), G.sha(vo)


def test_beacon_pass_matches_golden():
    say("golden beacon pass")
    g = load("beacon_pass.json")
    x = golden_inputs(g)
    batch = x["batch"]
    cache = device_cache(batch, G.N, G.P)
    wl = G.workload()
    HC, S, K = cache.n_head_caches, cache.max_slots, wl.n_beacons
    q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
    assign = torch.zeros((HC, wl.steps * wl.group), dtype=torch.int32).cuda()
    sc = torch.zeros((HC, S)).cuda()
    lse = torch.zeros((HC, K)).cuda()
    keep = torch.full((HC, G.B), -7, dtype=torch.int32).cuda()
    bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, G.B, queries=q, beacons=b, counts=c,
                      window=G.WINDOW, bonus=G.BONUS, assign=assign, scores_out=sc, lse=lse,
                      keep_out=keep)
    torch.cuda.synchronize()
    an, bn, cn = assign.cpu().numpy(), b.cpu().numpy(), c.cpu().numpy()
    scn, lsen, kn = sc.cpu().numpy(), lse.cpu().numpy(), keep.cpu().numpy()
    R, H = wl.n_requests, wl.n_kv_heads
    for d in g["head_caches"]:
        hc = d["hc"]
        layer, r, h = hc // (R * H), (hc // H) % R, hc % H
        n, p = G.N[r], G.P[r]
        assert an[hc].tolist() == G.parse_ints(d["assign"]), hc
        assert cn[hc].tolist() == G.parse_ints(d["counts"]), hc
        assert G.sha(bn[hc]) == d["beacons_sha256"], hc
        ref = G.parse_floats(d["scores"])
        check_scores(scn[hc, :n - p], ref, f"golden hc {hc}")
        ol = G.parse_floats(d["lse"])
        live = ~np.isnan(ol)
        assert np.all(np.isnan(lsen[hc][~live])), hc
        assert np.max(np.abs(lsen[hc][live] - ol[live])) <= 1e-3, hc
        kp, ref_keep = keep_rows(kn[hc]), np.array(G.parse_ints(d["keep"]), np.int32)
        # kept sets may differ only at slots tied with the boundary score
        if check_selection(kp, ref_keep, ref, n, p, G.B, f"golden hc {hc}") == 0:
            assert compacted_digests(cache, x, layer, r, h, len(kp)) == (
                d["k_compacted_sha256"], d["v_compacted_sha256"]), hc


def test_random_pass_matches_golden():
    say("golden random pass")
    g = load("random_pass.json")
    x = golden_inputs(g)
    cache = device_cache(x["batch"], G.N, G.P)
    wl = G.workload()
    HC, S = cache.n_head_caches, cache.max_slots
    rnd = g["random"]
    rid = torch.tensor(rnd["request_ids"], dtype=torch.int64).cuda()
    pss = torch.tensor(rnd["pass_idx"], dtype=torch.int32).cuda()
    sc = torch.zeros((HC, S), dtype=torch.int32).cuda()
    keep = torch.full((HC, G.B), -7, dtype=torch.int32).cuda()
    bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, G.B, seed=rnd["seed"], request_ids=rid,
                      pass_idx=pss, scores_out=sc, keep_out=keep)
    torch.cuda.synchronize()
    scn, kn = sc.cpu().numpy().view(np.uint32), keep.cpu().numpy()
    R, H = wl.n_requests, wl.n_kv_heads
    for d in g["head_caches"]:
        hc = d["hc"]
        layer, r, h = hc // (R * H), (hc // H) % R, hc % H
        n, p = G.N[r], G.P[r]
        assert scn[hc, :n - p].tolist() == G.parse_ints(d["draws"]), hc
        kp = keep_rows(kn[hc])
        assert kp.tolist() == G.parse_ints(d["keep"]), hc
        assert compacted_digests(cache, x, layer, r, h, len(kp)) == (
            d["k_compacted_sha256"], d["v_compacted_sha256"]), hc


@pytest.mark.parametrize("mode", ["beacon_per_request", "beacon_per_head", "random_per_request"])
def test_page_passes_match_golden(mode):
    say("golden pages", mode)
    g = load("page_retention.json")
    x = golden_inputs(g)
    batch = x["batch"]
    cache = device_cache(batch, G.N, G.P)
    wl = G.workload()
    L, R, H = wl.n_layers, wl.n_requests, wl.n_kv_heads
    HC, S, M = cache.n_head_caches, cache.max_slots, cache.max_blocks
    Bp = g["budget"]
    per_head = mode == "beacon_per_head"
    rows_n = HC if per_head else R
    kp = torch.full((rows_n, Bp // 16), -7, dtype=torch.int32).cuda()
    row_out = torch.full((rows_n, M), -7, dtype=torch.int32).cuda()
    len_out = torch.full((rows_n,), -7, dtype=torch.int32).cuda()
    freed = torch.full((rows_n, M), -7, dtype=torch.int32).cuda()
    if mode == "random_per_request":
        rnd = g["random"]
        rid = torch.tensor(rnd["request_ids"], dtype=torch.int64).cuda()
        pss = torch.tensor(rnd["pass_idx"], dtype=torch.int32).cuda()
        sc = torch.zeros((R, S), dtype=torch.int32).cuda()
        bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, Bp, seed=rnd["seed"], request_ids=rid,
                          pass_idx=pss, scores_out=sc, keep_out=kp,
                          page_retention=(row_out, len_out, freed))
    else:
        pc = cache
        if per_head:   # per-head tables starting from the request rows
            hrow = cache.block_table.repeat_interleave(H, 0).repeat(L, 1).contiguous()
            hlen = cache.seq_len.repeat_interleave(H).repeat(L).contiguous()
            pc = bk.PagedCache(cache.k_pools, cache.v_pools, cache.block_table, cache.seq_len,
                               cache.prompt_len, head_block_table=hrow, head_seq_len=hlen)
        q, b, c = batch.queries.cuda(), batch.beacons.cuda(), batch.counts.cuda()
        sc = torch.zeros((HC, S)).cuda()
        bk.bkv_evict_pass(pc, bk.BKV_SELECT_BEACON, Bp, queries=q, beacons=b, counts=c,
                          window=G.WINDOW, bonus=G.BONUS, scores_out=sc, keep_out=kp,
                          page_retention=(row_out, len_out, freed), page_heads=per_head)
    torch.cuda.synchronize()
    kpn, rown, lenn, frn = (kp.cpu().numpy(), row_out.cpu().numpy(), len_out.cpu().numpy(),
                            freed.cpu().numpy())
    released = "dropped" if per_head else "freed"
    for i, d in enumerate(g[mode]):
        u = d["hc"] if per_head else d["request"]
        assert i == u
        r = (u // H) % R if per_head else u
        pages = G.parse_ints(d["pages"])
        assert keep_rows(kpn[u]).tolist() == pages, (mode, u)
        npages = -(-G.N[r] // 16)
        assert rown[u][:len(pages)].tolist() == G.parse_ints(d["block_row"]), (mode, u)
        assert np.all(rown[u][len(pages):npages] == -1), (mode, u)
        assert int(lenn[u]) == d["seq_len"], (mode, u)
        rel = G.parse_ints(d[released])
        assert frn[u][:len(rel)].tolist() == rel, (mode, u)
        assert np.all(frn[u][len(rel):] == -1), (mode, u)

"""Writes the golden files of this folder.

The pages print no worked example of the method's arithmetic (their numbers
are end-to-end memory, throughput and accuracy claims), so every value stored
here is an output of the fp64 oracle (`oracle/`) on seeded synthetic inputs
from `decode_kv_cache_beacon_amd.synth`.  This script calls nothing else for
any stored value.  Small outputs are stored in full (assignments, counts,
scores and log-sum-exps as exact float hex, keep lists, draws, pages); large
arrays (updated beacons, compacted K/V rows, the inputs themselves) as SHA-256
digests of their bytes.

    python tests/golden/make_golden.py        # rewrites the *.json files

`tests/test_golden.py` regenerates every value on the CPU and requires the
files bit for bit; `tests/test_gpu_golden.py` checks the HIP path against them.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from decode_kv_cache_beacon_amd import synth  # noqa: E402

# One small paged batch serves every case: 2 layers x 2 requests x 2 KV heads,
# K = 16 beacons (prewarmed), G = 2 query heads, T = 16 buffered steps; the
# requests have ragged lengths and prompts.
WORKLOAD = dict(base="serving_r128", n_layers=2, n_requests=2, n_kv_heads=2, n_beacons=16,
                group=2, steps=16, budget=200, prompt_len=40, seq_len=300, prewarm=True,
                seed=11)
N = [300, 251]
P = [40, 17]
B = 200            # row compaction budget
B_PAGES = 160      # page-retention budget (a multiple of the 16-slot page)
WINDOW, BONUS = 64, 1.0
RANDOM = dict(seed=7, request_ids=[3, 4], pass_idx=[5, 6])


def workload():
    kw = dict(WORKLOAD)
    return synth.WORKLOADS[kw.pop("base")].with_(**kw)


def sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def fhex(xs):
    """Floats as exact hex, space-separated."""
    return " ".join(float(x).hex() for x in np.asarray(xs, np.float64))


def ints(xs):
    return " ".join(str(int(v)) for v in xs)


def parse_ints(s):
    return [int(v) for v in s.split()]


def parse_floats(s):
    return np.array([float.fromhex(v) for v in s.split()], np.float64)


def hc_index(R, H, layer, req, head):
    return (layer * R + req) * H + head


def inputs():
    """The batch and its host copies (bf16 as uint16 bits)."""
    batch = synth.make_batch(workload())
    return dict(batch=batch, q=synth.bits(batch.queries), b=batch.beacons.numpy(),
                c=batch.counts.numpy(), k=[synth.bits(k) for k in batch.k_pools],
                v=[synth.bits(v) for v in batch.v_pools], bt=batch.block_table.numpy())


def input_digests(x):
    return dict(queries=sha(x["q"]), beacons=sha(x["b"]), counts=sha(x["c"]),
                block_table=sha(x["bt"]), k_pools=[sha(k) for k in x["k"]],
                v_pools=[sha(v) for v in x["v"]])


def beacon_case(x):
    """Maintenance, scoring, selection and compaction of every head-cache."""
    wl = workload()
    L, R, H = wl.n_layers, wl.n_requests, wl.n_kv_heads
    heads = []
    for layer in range(L):
        for r in range(R):
            for h in range(H):
                hc = hc_index(R, H, layer, r, h)
                ob, oc, asg = oracle.beacon_update(x["q"][hc], x["b"][hc], x["c"][hc])
                keys = oracle.gather_paged(x["k"][layer], x["bt"][r], h, N[r])
                vals = oracle.gather_paged(x["v"][layer], x["bt"][r], h, N[r])
                sc, lse = oracle.beacon_score(keys, ob, oc, P[r], WINDOW, BONUS)
                keep = oracle.topk_select(sc, N[r], P[r], B)
                heads.append(dict(
                    hc=hc, assign=ints(asg), counts=ints(oc), beacons_sha256=sha(ob),
                    scores=fhex(sc), lse=fhex(lse), keep=ints(keep),
                    k_compacted_sha256=sha(oracle.kv_compact(keys, keep)),
                    v_compacted_sha256=sha(oracle.kv_compact(vals, keep))))
    return heads


def random_case(x):
    """Per-head Philox draws, selection and compaction of every head-cache."""
    wl = workload()
    L, R, H = wl.n_layers, wl.n_requests, wl.n_kv_heads
    heads = []
    for layer in range(L):
        for r in range(R):
            for h in range(H):
                hc = hc_index(R, H, layer, r, h)
                draws = oracle.random_score(RANDOM["seed"], RANDOM["request_ids"][r],
                                            RANDOM["pass_idx"][r], layer, h, N[r], P[r])
                keep = oracle.topk_select(draws, N[r], P[r], B)
                keys = oracle.gather_paged(x["k"][layer], x["bt"][r], h, N[r])
                vals = oracle.gather_paged(x["v"][layer], x["bt"][r], h, N[r])
                heads.append(dict(
                    hc=hc, draws=ints(draws), keep=ints(keep),
                    k_compacted_sha256=sha(oracle.kv_compact(keys, keep)),
                    v_compacted_sha256=sha(oracle.kv_compact(vals, keep))))
    return heads


def page_case(x, beacon_heads):
    """Page retention at B_PAGES from the beacon scores above: one selection
    per request over all its score rows, and one per head-cache from its own
    row; each with the rewritten block-table row, released blocks and length.
    Plus the random selector's per-request draws (layer and head fields 0)."""
    wl = workload()
    L, R, H = wl.n_layers, wl.n_requests, wl.n_kv_heads
    rows = {d["hc"]: parse_floats(d["scores"]) for d in beacon_heads}
    per_request, per_head, random_request = [], [], []
    for r in range(R):
        mine = np.stack([rows[hc_index(R, H, layer, r, h)] for layer in range(L)
                         for h in range(H)])
        pages = oracle.page_select(mine, N[r], P[r], B_PAGES)
        new_row, freed, new_n = oracle.page_remap(x["bt"][r], N[r], pages)
        per_request.append(dict(request=r, pages=ints(pages), block_row=ints(new_row),
                                freed=ints(freed), seq_len=new_n))
        draws = oracle.random_score(RANDOM["seed"], RANDOM["request_ids"][r],
                                    RANDOM["pass_idx"][r], 0, 0, N[r], P[r])
        rpages = oracle.page_select(draws[None], N[r], P[r], B_PAGES)
        rrow, rfreed, rn = oracle.page_remap(x["bt"][r], N[r], rpages)
        random_request.append(dict(request=r, pages=ints(rpages), block_row=ints(rrow),
                                   freed=ints(rfreed), seq_len=rn))
        for layer in range(L):
            for h in range(H):
                hc = hc_index(R, H, layer, r, h)
                hp = oracle.page_select(rows[hc][None], N[r], P[r], B_PAGES)
                hrow, hdrop, hn = oracle.page_remap(x["bt"][r], N[r], hp)
                per_head.append(dict(hc=hc, pages=ints(hp), block_row=ints(hrow),
                                     dropped=ints(hdrop), seq_len=hn))
    per_head.sort(key=lambda d: d["hc"])
    return dict(beacon_per_request=per_request, beacon_per_head=per_head,
                random_per_request=random_request)


def compute():
    """Every golden file's contents, keyed by file name."""
    x = inputs()
    common = dict(workload=WORKLOAD, N=N, P=P, window=WINDOW, bonus=BONUS,
                  inputs_sha256=input_digests(x),
                  source="fp64 oracle (oracle/beacon_oracle.c) on seeded synthetic inputs; "
                         "the pages print no worked example of the method's arithmetic")
    beacon = beacon_case(x)
    return {
        "beacon_pass.json": dict(common, budget=B, head_caches=beacon),
        "random_pass.json": dict(common, budget=B, random=RANDOM, head_caches=random_case(x)),
        "page_retention.json": dict(common, budget=B_PAGES, random=RANDOM,
                                    **page_case(x, beacon)),
    }


def main():
    for name, content in compute().items():
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(content, f, indent=1)
            f.write("\n")
        print("wrote", name)


if __name__ == "__main__":
    main()

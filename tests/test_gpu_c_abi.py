"""libbeaconkv.so called from plain C: tests/probes/c_abi_driver (built by
build(), from c_abi_driver.c) runs a random-selector pass through
bkv_workspace_size and bkv_evict_pass on a small paged cache it fills from an
integer hash, and one pass the library must refuse.  Its printed keep lists,
draw digests and compacted-row digests are checked against the oracle on the
same cache, rebuilt here from the same hash."""
import os
import subprocess

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "probes", "c_abi_driver")

# the driver's cache (c_abi_driver.c)
R, H, NBLK, MAXB, D, BS = 2, 2, 40, 20, 128, 16
SEQ, PROMPT, BUDGET = [300, 213], [40, 7], 128
SEED, RIDS, PASSES = 99, [11, 12], [2, 3]
BKV_ERR_WORKSPACE = 5


def pool_values(salt):
    """The driver's pool_value() over every flat index, as uint16 [NBLK, H, BS, D]."""
    idx = np.arange(NBLK * H * BS * D, dtype=np.uint64)
    m = np.uint64(0xFFFFFFFF)
    x = (idx * np.uint64(2654435761) + np.uint64(salt)) & m
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(2246822519)) & m
    x ^= x >> np.uint64(13)
    return (x & np.uint64(0xFFFF)).astype(np.uint16).reshape(NBLK, H, BS, D)


def fnv1a(data: bytes) -> int:
    h = 14695981039346656037
    for byte in data:
        h = ((h ^ byte) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def test_c_caller_random_pass_matches_the_oracle():
    assert os.path.exists(DRIVER), "build() builds tests/probes/c_abi_driver"
    print("[case] C caller, random pass", flush=True)
    run = subprocess.run([DRIVER], capture_output=True, text=True, timeout=120)
    print(run.stdout + run.stderr, flush=True)
    assert run.returncode == 0, run.stderr
    lines = [ln.split() for ln in run.stdout.splitlines()]
    head = {ln[0]: ln[1:] for ln in lines if ln[0] != "hc"}
    from decode_kv_cache_beacon_amd import beaconkv as bk
    assert int(head["abi"][0]) == bk.BKV_ABI_VERSION
    assert int(head["workspace"][0]) >= 0
    assert int(head["refused"][0]) == BKV_ERR_WORKSPACE       # nothing enqueued
    assert head["pass"] == ["0", "0"]                          # returned OK, no device error
    per_hc = {}
    for ln in lines:
        if ln[0] == "hc":
            per_hc.setdefault(int(ln[1]), {})[ln[2]] = ln[3:]
    kpool, vpool = pool_values(1), pool_values(2)
    bt = np.array([[20 * r + (7 * i) % 20 for i in range(MAXB)] for r in range(R)], np.int32)
    assert sorted(per_hc) == list(range(R * H))
    for hc, got in per_hc.items():
        r, h = (hc // H) % R, hc % H
        n, p = SEQ[r], PROMPT[r]
        draws = oracle.random_score(SEED, RIDS[r], PASSES[r], 0, h, n, p)
        assert int(got["draws"][0], 16) == fnv1a(draws.astype("<u4").tobytes()), hc
        keep = oracle.topk_select(draws, n, p, BUDGET)
        assert [int(v) for v in got["keep"]] == keep.tolist(), hc
        keys = oracle.kv_compact(oracle.gather_paged(kpool, bt[r], h, n), keep)
        vals = oracle.kv_compact(oracle.gather_paged(vpool, bt[r], h, n), keep)
        assert int(got["rows"][0], 16) == fnv1a(keys.astype("<u2").tobytes()), hc
        assert int(got["rows"][1], 16) == fnv1a(vals.astype("<u2").tobytes()), hc

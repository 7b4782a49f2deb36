"""The golden files under tests/golden/ are oracle outputs on seeded inputs,
written by tests/golden/make_golden.py.  Regenerating them here must give the
stored files bit for bit, so a change to the oracle's arithmetic or to the
input generator cannot pass unnoticed (the GPU path is checked against the
same files in tests/test_gpu_golden.py)."""
import json
import os

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_golden_files_regenerate_bit_for_bit():
    for name, content in make_golden.compute().items():
        with open(os.path.join(HERE, name)) as f:
            stored = json.load(f)
        assert json.loads(json.dumps(content)) == stored, name


def test_golden_files_cover_every_head_cache_and_request():
    wl = make_golden.workload()
    hcs = list(range(wl.n_layers * wl.n_requests * wl.n_kv_heads))
    for name in ("beacon_pass.json", "random_pass.json"):
        with open(os.path.join(HERE, name)) as f:
            assert [d["hc"] for d in json.load(f)["head_caches"]] == hcs, name
    with open(os.path.join(HERE, "page_retention.json")) as f:
        pages = json.load(f)
    assert [d["hc"] for d in pages["beacon_per_head"]] == hcs
    for key in ("beacon_per_request", "random_per_request"):
        assert [d["request"] for d in pages[key]] == list(range(wl.n_requests)), key

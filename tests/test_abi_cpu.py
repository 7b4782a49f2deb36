"""The C ABI without a GPU: exports match the header, and host-side
validation rejects bad arguments before anything is launched (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

from decode_kv_cache_beacon_amd import beaconkv as bk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "beaconkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(bkv_\w+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 14, names
    lib = ctypes.CDLL(bk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bk.EXPORTS) == names


def test_binding_constants_match_the_header():
    src = open(os.path.join(ROOT, "include", "beaconkv.h")).read()
    macros = dict(re.findall(r"^#define (BKV_\w+) (\d+)", src, re.M))
    assert int(macros["BKV_ABI_VERSION"]) == bk.BKV_ABI_VERSION
    assert int(macros["BKV_FUSED_MAX_ENTRIES"]) == bk.FUSED_MAX_ENTRIES
    assert int(macros["BKV_MAX_BEACONS"]) == bk.BKV_MAX_BEACONS
    assert int(macros["BKV_NOALLOC_SCRATCH_BYTES"]) == bk.NOALLOC_SCRATCH_BYTES


def test_version_and_status_strings():
    assert bk.bkv_abi_version() == bk.BKV_ABI_VERSION == 8
    for code in range(0, 10):
        s = bk.bkv_status_string(code)
        assert s and s != "unknown status code"
    assert bk.bkv_status_string(99) == "unknown status code"


@pytest.mark.parametrize("struct", [bk.bkv_cache, bk.bkv_pass_args])
def test_binding_structs_match_the_header(struct, tmp_path):
    """Every field of the ctypes mirror sits at the offset the C compiler
    gives it in include/beaconkv.h, and the sizes agree."""
    name = struct.__name__
    fields = [f[0] for f in struct._fields_]
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "beaconkv.h"',
             "int main(void) {", f'  printf("size %zu\\n", sizeof({name}));']
    lines += [f'  printf("{f} %zu\\n", offsetof({name}, {f}));' for f in fields]
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True,
                                                 text=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(struct)
    for f in fields:
        assert int(out[f]) == getattr(struct, f).offset, f
    # the header declares no field the mirror lacks
    body = open(os.path.join(ROOT, "include", "beaconkv.h")).read()
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    decl = re.search(r"typedef struct\s+" + name + r"\s*\{(.*?)\}\s*" + name + ";", body,
                     re.S).group(1)
    declared = re.findall(r"(\w+)\s*(?:,|;)", decl)
    assert sorted(declared) == sorted(fields)


FAKE = 0x100000  # never dereferenced: validation fails before any launch


def _cache(**kw):
    c = dict(n_layers=2, n_requests=3, n_kv_heads=8, head_dim=128, block_size=16, max_blocks=10,
             num_blocks=30, k_pools=FAKE, v_pools=FAKE, block_table=FAKE, seq_len=FAKE,
             prompt_len=FAKE)
    c.update(kw)
    return bk.bkv_cache(**c)


def _score(cache, K=64, stride=160, beacons=FAKE, counts=FAKE, scores=FAKE, window=64):
    return bk._lib.bkv_beacon_score(ctypes.byref(cache), beacons, counts, K, window, 1.0, scores,
                                    stride, None, None, None)


def test_beacon_update_validation():
    f = bk._lib.bkv_beacon_update
    assert f(4, 8, 2, 64, 16, FAKE, FAKE, FAKE, None, 0, None) == bk.BKV_ERR_UNSUPPORTED
    assert f(4, 8, 2, 128, 0, FAKE, FAKE, FAKE, None, 0, None) == bk.BKV_ERR_INVALID
    assert f(4, 8, 2, 128, 257, FAKE, FAKE, FAKE, None, 0, None) == bk.BKV_ERR_INVALID
    assert f(4, 0, 2, 128, 16, FAKE, FAKE, FAKE, None, 0, None) == bk.BKV_ERR_INVALID
    assert f(-1, 8, 2, 128, 16, FAKE, FAKE, FAKE, None, 0, None) == bk.BKV_ERR_INVALID
    assert f(4, 8, 2, 128, 16, FAKE, FAKE, FAKE, None, -1, None) == bk.BKV_ERR_INVALID  # cap < 0
    assert f(4, 8, 2, 128, 16, None, FAKE, FAKE, None, 0, None) == bk.BKV_ERR_NULL
    assert f(4, 8, 2, 128, 16, FAKE + 4, FAKE, FAKE, None, 0, None) == bk.BKV_ERR_INVALID  # misaligned
    assert f(0, 8, 2, 128, 16, None, None, None, None, 0, None) == bk.BKV_OK   # nothing to do


def test_cache_validation():
    assert _score(_cache(head_dim=64)) == bk.BKV_ERR_UNSUPPORTED
    assert _score(_cache(block_size=32)) == bk.BKV_ERR_UNSUPPORTED
    assert _score(_cache(k_pools=None)) == bk.BKV_ERR_NULL
    assert _score(_cache(block_table=None)) == bk.BKV_ERR_NULL
    assert _score(_cache(n_layers=0)) == bk.BKV_ERR_INVALID
    assert _score(_cache(num_blocks=0)) == bk.BKV_ERR_INVALID
    assert _score(_cache(seq_len=FAKE + 2)) == bk.BKV_ERR_INVALID
    assert _score(_cache(n_layers=2**16, n_requests=2**12, n_kv_heads=8)) == bk.BKV_ERR_INVALID
    # a head-cache count whose product overflows 64 bits is refused, not wrapped
    m = 2**31 - 1
    assert _score(_cache(n_layers=m, n_requests=m, n_kv_heads=m)) == bk.BKV_ERR_INVALID
    assert _score(_cache(n_layers=2**21, n_requests=2**21, n_kv_heads=2**21)) == \
        bk.BKV_ERR_INVALID
    assert bk._lib.bkv_beacon_score(None, FAKE, FAKE, 8, 64, 1.0, FAKE, 16, None, None,
                                    None) == bk.BKV_ERR_NULL


def test_score_argument_validation():
    c = _cache()
    assert _score(c, K=0) == bk.BKV_ERR_INVALID
    assert _score(c, K=300) == bk.BKV_ERR_INVALID
    assert _score(c, stride=0) == bk.BKV_ERR_INVALID
    assert _score(c, window=-1) == bk.BKV_ERR_INVALID
    assert _score(c, beacons=None) == bk.BKV_ERR_NULL
    assert _score(c, beacons=FAKE + 8) == bk.BKV_ERR_INVALID
    assert _score(_cache(max_blocks=4096)) == bk.BKV_ERR_INVALID   # > 32768 slots


def test_select_compact_random_validation():
    c = _cache()
    sel = bk._lib.bkv_topk_select
    assert sel(ctypes.byref(c), FAKE, 7, 160, 64, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert sel(ctypes.byref(c), FAKE, 0, 0, 64, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert sel(ctypes.byref(c), FAKE, 0, 40000, 64, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert sel(ctypes.byref(c), FAKE, 0, 160, 0, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert sel(ctypes.byref(c), None, 0, 160, 64, FAKE, None, None) == bk.BKV_ERR_NULL
    cmp_ = bk._lib.bkv_kv_compact
    assert cmp_(ctypes.byref(c), None, 64, 0, None, 0, None, None) == bk.BKV_ERR_NULL
    assert cmp_(ctypes.byref(c), FAKE, 0, 0, None, 0, None, None) == bk.BKV_ERR_INVALID
    assert cmp_(ctypes.byref(c), FAKE, 64, 0, FAKE, 100, None, None) == bk.BKV_ERR_INVALID  # pos stride < 160
    assert cmp_(ctypes.byref(c), FAKE, 64, 2, None, 0, None, None) == bk.BKV_ERR_INVALID   # keep_shared
    rnd = bk._lib.bkv_random_score
    assert rnd(ctypes.byref(c), 1, None, FAKE, 0, FAKE, 160, None, None) == bk.BKV_ERR_NULL
    assert rnd(ctypes.byref(c), 1, FAKE, FAKE, 0, FAKE, 0, None, None) == bk.BKV_ERR_INVALID
    assert rnd(ctypes.byref(c), 1, FAKE, FAKE, -1, FAKE, 160, None, None) == bk.BKV_ERR_INVALID
    assert rnd(ctypes.byref(c), 1, FAKE, FAKE, 3, FAKE, 160, None, None) == bk.BKV_ERR_INVALID


def test_decode_attention_validation():
    c = _cache()
    f = bk._lib.bkv_decode_attention
    assert f(ctypes.byref(c), FAKE, 0, 0.1, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert f(ctypes.byref(c), FAKE, 9, 0.1, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert f(ctypes.byref(c), None, 4, 0.1, FAKE, None, None) == bk.BKV_ERR_NULL
    assert f(ctypes.byref(c), FAKE, 4, 0.1, None, None, None) == bk.BKV_ERR_NULL
    assert f(ctypes.byref(c), FAKE + 8, 4, 0.1, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert f(ctypes.byref(c), FAKE, 4, 0.1, FAKE + 4, None, None) == bk.BKV_ERR_INVALID
    assert f(ctypes.byref(_cache(head_dim=64)), FAKE, 4, 0.1, FAKE, None, None) == \
        bk.BKV_ERR_UNSUPPORTED


def test_page_retain_validation():
    c = _cache()
    f = bk._lib.bkv_page_retain
    ok = dict(scores=FAKE, kind=0, stride=160, rows=bk.BKV_ROWS_PER_HEAD, budget=64, keep=FAKE,
              bt=FAKE, sl=FAKE, fr=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(c), a["scores"], a["kind"], a["stride"], a["rows"], a["budget"],
                 a["keep"], a["bt"], a["sl"], a["fr"], None, None)

    assert call(budget=40) == bk.BKV_ERR_INVALID          # not a whole number of pages
    assert call(budget=0) == bk.BKV_ERR_INVALID
    assert call(rows=bk.BKV_ROWS_PER_LAYER_REQUEST) == bk.BKV_ERR_INVALID
    assert call(kind=2) == bk.BKV_ERR_INVALID
    assert call(stride=0) == bk.BKV_ERR_INVALID
    assert call(bt=None) == bk.BKV_ERR_NULL
    assert call(fr=None) == bk.BKV_ERR_NULL
    assert call(sl=FAKE + 2) == bk.BKV_ERR_INVALID


def test_per_head_tables_validation():
    """Per-head page tables come as an aligned pair, and the calls that share
    one selection across a request's heads refuse a cache read through them."""
    assert _score(_cache(head_block_table=FAKE)) == bk.BKV_ERR_INVALID        # without lengths
    assert _score(_cache(head_seq_len=FAKE)) == bk.BKV_ERR_INVALID            # without rows
    assert _score(_cache(head_block_table=FAKE + 2, head_seq_len=FAKE)) == bk.BKV_ERR_INVALID
    hc = _cache(head_block_table=FAKE, head_seq_len=FAKE)
    sh = bk._lib.bkv_topk_select_shared
    assert sh(ctypes.byref(hc), FAKE, 0, 160, 8, 64, FAKE, None, None) == bk.BKV_ERR_INVALID
    cmp_ = bk._lib.bkv_kv_compact
    assert cmp_(ctypes.byref(hc), FAKE, 64, 1, None, 0, None, None) == bk.BKV_ERR_INVALID
    rnd = bk._lib.bkv_random_score
    for rows in (bk.BKV_ROWS_PER_LAYER_REQUEST, bk.BKV_ROWS_PER_REQUEST):
        assert rnd(ctypes.byref(hc), 1, FAKE, FAKE, rows, FAKE, 160, None, None) == \
            bk.BKV_ERR_INVALID
    pr = bk._lib.bkv_page_retain
    assert pr(ctypes.byref(hc), FAKE, 0, 160, bk.BKV_ROWS_PER_HEAD, 64, FAKE, FAKE, FAKE, FAKE,
              None, None) == bk.BKV_ERR_INVALID
    a = bk.bkv_pass_args()
    a.selector, a.budget = bk.BKV_SELECT_RANDOM, 64
    n = ctypes.c_size_t(0)
    ws = bk._lib.bkv_workspace_size
    assert ws(ctypes.byref(hc), ctypes.byref(a), ctypes.byref(n)) == 0
    a.shared_positions = 1
    assert ws(ctypes.byref(hc), ctypes.byref(a), ctypes.byref(n)) == bk.BKV_ERR_INVALID
    a.shared_positions, a.page_retention = 0, bk.BKV_PAGES_PER_REQUEST
    assert ws(ctypes.byref(hc), ctypes.byref(a), ctypes.byref(n)) == bk.BKV_ERR_INVALID
    a.page_retention = bk.BKV_PAGES_PER_HEAD   # per-head pages: draws and page lists per head
    assert ws(ctypes.byref(hc), ctypes.byref(a), ctypes.byref(n)) == 0
    HC = 2 * 3 * 8
    assert HC * 160 * 4 + HC * 4 * 4 <= n.value <= HC * 160 * 4 + HC * 4 * 4 + 512
    a.page_retention = 3
    assert ws(ctypes.byref(hc), ctypes.byref(a), ctypes.byref(n)) == bk.BKV_ERR_INVALID


def test_page_retain_heads_validation():
    c = _cache()
    f = bk._lib.bkv_page_retain_heads
    ok = dict(scores=FAKE, kind=0, stride=160, budget=64, keep=FAKE, bt=FAKE, sl=FAKE, dr=FAKE)

    def call(cache=c, **kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(cache), a["scores"], a["kind"], a["stride"], a["budget"],
                 a["keep"], a["bt"], a["sl"], a["dr"], None, None)

    assert call(budget=40) == bk.BKV_ERR_INVALID          # not a whole number of pages
    assert call(budget=0) == bk.BKV_ERR_INVALID
    assert call(kind=2) == bk.BKV_ERR_INVALID
    assert call(stride=0) == bk.BKV_ERR_INVALID
    assert call(scores=None) == bk.BKV_ERR_NULL
    assert call(bt=None) == bk.BKV_ERR_NULL
    assert call(dr=None) == bk.BKV_ERR_NULL
    assert call(sl=FAKE + 2) == bk.BKV_ERR_INVALID
    assert call(cache=_cache(head_dim=64)) == bk.BKV_ERR_UNSUPPORTED


def test_shared_select_validation():
    c = _cache()   # 8 KV heads
    f = bk._lib.bkv_topk_select_shared
    assert f(ctypes.byref(c), FAKE, 0, 160, 0, 64, FAKE, None, None) == bk.BKV_ERR_INVALID  # S < 1
    assert f(ctypes.byref(c), FAKE, 0, 160, 9, 64, FAKE, None, None) == bk.BKV_ERR_INVALID  # S > H
    assert f(ctypes.byref(c), FAKE, 3, 160, 8, 64, FAKE, None, None) == bk.BKV_ERR_INVALID  # kind
    assert f(ctypes.byref(c), FAKE, 0, 40000, 8, 64, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert f(ctypes.byref(c), FAKE, 0, 160, 8, 0, FAKE, None, None) == bk.BKV_ERR_INVALID
    assert f(ctypes.byref(c), None, 0, 160, 8, 64, FAKE, None, None) == bk.BKV_ERR_NULL
    assert f(ctypes.byref(c), FAKE, 0, 160, 8, 64, FAKE + 2, None, None) == bk.BKV_ERR_INVALID
    assert f(None, FAKE, 0, 160, 8, 64, FAKE, None, None) == bk.BKV_ERR_NULL


def test_workspace_and_pass_validation():
    c = _cache()
    a = bk.bkv_pass_args()
    a.selector, a.budget = bk.BKV_SELECT_RANDOM, 64
    n = ctypes.c_size_t(0)
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    HC = 2 * 3 * 8
    # per-head random pass: the fused kernel keeps the keep lists on chip
    assert HC * 160 * 4 <= n.value < HC * 160 * 4 + 256
    a.separate_steps = 1          # three kernels: the keep lists go through the workspace
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    assert HC * 160 * 4 + HC * 64 * 4 <= n.value < HC * 160 * 4 + HC * 64 * 4 + 512
    a.separate_steps = 0
    a.budget = 15872 - 160 + 1    # past the fused kernel's LDS: keep lists in the workspace
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value >= HC * 160 * 4 + HC * a.budget * 4
    a.budget = 64
    a.shared_positions = 1        # random + shared: one score row and one keep row per (layer, request)
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    assert HC // 8 * (160 + 64) * 4 <= n.value < HC * 64 * 4
    a.selector = bk.BKV_SELECT_BEACON   # beacon + shared (fused): per-head scores only
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    assert HC * 160 * 4 <= n.value < HC * 160 * 4 + 256
    a.separate_steps = 1               # separate kernels: plus the shared keep rows
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    assert HC * 160 * 4 + HC // 8 * 64 * 4 <= n.value < HC * 160 * 4 + HC * 64 * 4
    a.separate_steps = 0
    a.shared_positions = 2
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == \
        bk.BKV_ERR_INVALID
    a.shared_positions, a.selector = 0, bk.BKV_SELECT_RANDOM
    a.page_retention = 1           # random + pages: one draw row and one page list per request
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    assert 3 * 160 * 4 + 3 * 4 * 4 <= n.value <= 3 * 160 * 4 + 3 * 4 * 4 + 512
    a.shared_positions = 1         # pages exclude shared positions
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == \
        bk.BKV_ERR_INVALID
    a.shared_positions, a.budget = 0, 72   # pages need a whole number of pages
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == \
        bk.BKV_ERR_INVALID
    a.page_retention, a.budget = 0, 64
    a.scores_out, a.keep_out = FAKE, FAKE
    assert bk._lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value == 0
    a.scores_out, a.keep_out = None, None
    ev = bk._lib.bkv_evict_pass
    assert ev(ctypes.byref(c), ctypes.byref(a), None, 0, None, None) == bk.BKV_ERR_WORKSPACE
    a.request_ids = None
    a.pass_idx = FAKE
    big = 1 << 40
    assert ev(ctypes.byref(c), ctypes.byref(a), FAKE, big, None, None) == bk.BKV_ERR_NULL
    a.selector = 5
    assert ev(ctypes.byref(c), ctypes.byref(a), FAKE, big, None, None) == bk.BKV_ERR_INVALID
    a.selector = bk.BKV_SELECT_BEACON
    a.queries = a.beacons = a.counts = FAKE
    a.n_beacons, a.T, a.G = 0, 64, 4
    assert ev(ctypes.byref(c), ctypes.byref(a), FAKE, big, None, None) == bk.BKV_ERR_INVALID
    a.n_beacons = 64
    a.budget = 0
    assert ev(ctypes.byref(c), ctypes.byref(a), FAKE, big, None, None) == bk.BKV_ERR_INVALID
    a.budget = 64
    assert ev(ctypes.byref(c), ctypes.byref(a), FAKE + 16, big, None, None) == bk.BKV_ERR_INVALID


def test_noalloc_pass_validation():
    """The allocation-free pass validates like bkv_evict_pass and refuses a
    pass whose buffers exceed its scratch before any HIP call."""
    ev = bk._lib.bkv_evict_pass_noalloc
    a = bk.bkv_pass_args()
    a.selector, a.budget = bk.BKV_SELECT_RANDOM, 64
    a.request_ids = a.pass_idx = FAKE
    assert ev(None, ctypes.byref(a), None, None) == bk.BKV_ERR_NULL
    assert ev(ctypes.byref(_cache()), None, None, None) == bk.BKV_ERR_NULL
    assert ev(ctypes.byref(_cache(head_dim=64)), ctypes.byref(a), None, None) == \
        bk.BKV_ERR_UNSUPPORTED
    a.selector = 5
    assert ev(ctypes.byref(_cache()), ctypes.byref(a), None, None) == bk.BKV_ERR_INVALID
    a.selector = bk.BKV_SELECT_RANDOM
    # 64 layers x 512 requests x 8 heads x 2048 candidates x 4 B = 2 GiB > 256 MiB
    big = _cache(n_layers=64, n_requests=512, n_kv_heads=8, max_blocks=128)
    n = ctypes.c_size_t(0)
    assert bk._lib.bkv_workspace_size(ctypes.byref(big), ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value > bk.NOALLOC_SCRATCH_BYTES
    assert ev(ctypes.byref(big), ctypes.byref(a), None, None) == bk.BKV_ERR_SCRATCH
    # given its own score and keep buffers the same pass needs no scratch; the
    # remaining checks still run before anything is enqueued
    a.scores_out, a.keep_out = FAKE, FAKE
    assert bk._lib.bkv_workspace_size(ctypes.byref(big), ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value == 0
    a.pass_idx = None
    assert ev(ctypes.byref(big), ctypes.byref(a), None, None) == bk.BKV_ERR_NULL
    assert "scratch" in bk.bkv_status_string(bk.BKV_ERR_SCRATCH)


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(2, 4, 1, 128, dtype=torch.bfloat16)
    b = torch.zeros(2, 8, 128)
    c = torch.zeros(2, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        bk.bkv_beacon_update(q, b, c)

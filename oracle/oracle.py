"""Python face of the CPU oracle (test infrastructure only).

Plain, slow, obviously-correct reference of the decode-time KV eviction pass.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product library never does, and this module imports nothing
from the product package.  The arithmetic lives in ``beacon_oracle.c``
(double precision, plain loops); this file only marshals numpy arrays and reads
the paged cache layout with its own numpy indexing.

Pages followed: the BeaconKV explainer (papers.ananclaw.com), section 3.2, for
nearest-beacon assignment and incremental beacon update; the Random Attention
article (aiinking.com), section "Random Attention: 不判断重要性, 只随机保留",
for prompt protection and per-head top-K of random scores, section "发现四"
for the shared compaction step, and section "发现二" for one common set of
positions shared by all heads, and for retaining contiguous blocks (pages).
Where the pages leave a rule open, each function states the rule it applies.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "beacon_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_BUILD_CMD = [
    "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
    _SRC, "-o", _LIB, "-lm",
]


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = list(_BUILD_CMD)
        cmd[cmd.index(_LIB)] = tmp
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_beacon_update.argtypes = [i32, i32, i32, i32, P, P, P, P, i32]
        L.oracle_beacon_update.restype = None
        L.oracle_beacon_update_forced.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i32]
        L.oracle_beacon_update_forced.restype = i32
        L.oracle_beacon_score.argtypes = [i32, i32, i32, i32, P, P, P, i32, f64, P, P]
        L.oracle_beacon_score.restype = None
        L.oracle_philox4x64_10.argtypes = [P, P, P]
        L.oracle_philox4x64_10.restype = None
        L.oracle_random_score.argtypes = [u64, u64, i32, i32, i32, i32, i32, P]
        L.oracle_random_score.restype = None
        L.oracle_topk_select.argtypes = [i32, i32, i32, P, P]
        L.oracle_topk_select.restype = i32
        L.oracle_shared_select.argtypes = [i32, i32, i32, i32, P, P]
        L.oracle_shared_select.restype = i32
        L.oracle_page_select.argtypes = [i32, i32, i32, i32, i32, P, P]
        L.oracle_page_select.restype = i32
        L.oracle_page_remap.argtypes = [i32, i32, P, i32, P, P, P, P]
        L.oracle_page_remap.restype = i32
        L.oracle_decode_attention.argtypes = [i32, i32, i32, P, P, P, f64, P]
        L.oracle_decode_attention.restype = None
        L.oracle_kv_compact.argtypes = [i32, P, i64, P, P]
        L.oracle_kv_compact.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = i32
        L.oracle_evict_batch.argtypes = [i32, i32, i32, i32, i32, i32, i32, f64, i32,
                                         P, P, P, P, P, P, P, P, P, P]
        L.oracle_evict_batch.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- conversions
def bf16_round(x: float) -> int:
    """fp32 value -> bf16 bit pattern, round to nearest even (oracle's own)."""
    return int(lib().oracle_bf16_round(float(np.float32(x))))


# ---------------------------------------------------------------- maintenance
def beacon_update(q_bits, beacons, counts, cap=0):
    """Absorb queries q[T][G][d] (bf16 bits) in (t, g) order.

    cap > 0 clamps every incremented count to cap (exponential moving average
    once a row is full); 0 is the plain running mean.
    Returns (beacons', counts', assign[T*G]); inputs are not modified.
    """
    q = _c(q_bits, np.uint16)
    T, G, d = q.shape
    b = _c(beacons, np.float32).copy()
    c = _c(counts, np.int32).copy()
    K = b.shape[0]
    assert b.shape == (K, d) and c.shape == (K,)
    a = np.zeros(T * G, np.int32)
    lib().oracle_beacon_update(T, G, d, K, _ptr(q), _ptr(b), _ptr(c), _ptr(a), int(cap))
    return b, c, a


def beacon_update_forced(q_bits, beacons, counts, forced, cap=0):
    """Replay a given assignment sequence; returns (beacons', counts', gap).

    gap[s] = best cosine - cosine of the forced row (0 for an exact argmax,
    +inf when the forced row breaks the empty-slot rule, NaN when out of range).
    """
    q = _c(q_bits, np.uint16)
    T, G, d = q.shape
    b = _c(beacons, np.float32).copy()
    c = _c(counts, np.int32).copy()
    K = b.shape[0]
    f = _c(forced, np.int32).reshape(-1)
    assert f.shape == (T * G,)
    gap = np.zeros(T * G, np.float64)
    lib().oracle_beacon_update_forced(T, G, d, K, _ptr(q), _ptr(b), _ptr(c), _ptr(f), _ptr(gap),
                                      int(cap))
    return b, c, gap


# ---------------------------------------------------------------- scoring
def beacon_score(keys_bits, beacons, counts, P, W=64, bonus=1.0):
    """keys[N][d] bf16 bits of one head-cache -> (scores[N-P] f64, lse[K] f64)."""
    k = _c(keys_bits, np.uint16)
    N, d = k.shape
    b = _c(beacons, np.float32)
    c = _c(counts, np.int32)
    K = b.shape[0]
    assert 0 <= P <= N
    s = np.zeros(max(N - P, 1), np.float64)
    lse = np.zeros(K, np.float64)
    lib().oracle_beacon_score(N, P, d, K, _ptr(k), _ptr(b), _ptr(c), int(W), float(bonus),
                              _ptr(s), _ptr(lse))
    return s[: N - P], lse


def philox4x64_10(counter, key):
    ctr = np.array(counter, dtype=np.uint64)
    k = np.array(key, dtype=np.uint64)
    out = np.zeros(4, np.uint64)
    lib().oracle_philox4x64_10(_ptr(ctr), _ptr(k), _ptr(out))
    return out


def random_score(seed, request_id, pass_idx, layer, head, N, P):
    out = np.zeros(max(N - P, 1), np.uint32)
    lib().oracle_random_score(int(seed) & (2**64 - 1), int(request_id) & (2**64 - 1),
                              int(pass_idx), int(layer), int(head), int(N), int(P), _ptr(out))
    return out[: N - P]


# ---------------------------------------------------------------- selection
def topk_select(scores, N, P, B):
    """scores[N-P] (any real dtype; uint32 draws are exact in double)."""
    s = _c(np.asarray(scores).astype(np.float64), np.float64)
    assert s.shape == (N - P,)
    keep = np.zeros(max(min(N, B), 1), np.int32)
    n = lib().oracle_topk_select(int(N), int(P), int(B), _ptr(s) if s.size else None, _ptr(keep))
    if n < 0:
        raise ValueError(f"selection refused: P={P} exceeds budget B={B} or bad lengths")
    return keep[:n]


def shared_select(scores, N, P, B):
    """One selection for all heads of a (layer, request).

    scores[H][N-P]: per-head candidate scores (H = 1 for one shared random
    draw).  The merged score of a candidate is its largest per-head score; the
    prompt-protected top-B then runs once on the merged scores.
    """
    s = np.asarray(scores).astype(np.float64)
    if s.ndim == 1:
        s = s[None, :]
    s = _c(s, np.float64)
    H = s.shape[0]
    assert s.shape == (H, N - P)
    keep = np.zeros(max(min(N, B), 1), np.int32)
    n = lib().oracle_shared_select(H, int(N), int(P), int(B), _ptr(s) if s.size else None,
                                   _ptr(keep))
    if n < 0:
        raise ValueError(f"selection refused: P={P} exceeds budget B={B} or bad lengths")
    return keep[:n]


def page_select(scores, N, P, B, page=16):
    """Pages kept for one request: scores[n_rows][N-P] are all its score rows
    (every layer and head, or one shared draw row).  Prompt pages and a partial
    last page are always kept; a page's score is the largest of its slots'
    scores over all rows; B // page pages survive."""
    s = np.asarray(scores).astype(np.float64)
    if s.ndim == 1:
        s = s[None, :]
    s = _c(s, np.float64)
    assert s.shape[1] == N - P
    npages = (N + page - 1) // page
    keep = np.zeros(max(npages, 1), np.int32)
    n = lib().oracle_page_select(s.shape[0], int(N), int(P), int(B), int(page),
                                 _ptr(s) if s.size else None, _ptr(keep))
    if n < 0:
        raise ValueError(f"page selection refused: forced pages exceed B // page (P={P}, B={B})")
    return keep[:n]


def page_remap(block_row, N, keep_pages, page=16):
    """(new block row, released blocks, new N) after keeping keep_pages."""
    row = _c(block_row, np.int32)
    kp = _c(keep_pages, np.int32)
    npages = (N + page - 1) // page
    new_row = np.zeros(max(len(kp), 1), np.int32)
    freed = np.zeros(max(npages, 1), np.int32)
    nf = ctypes.c_int32(0)
    new_n = lib().oracle_page_remap(int(N), int(page), _ptr(row), len(kp),
                                    _ptr(kp) if len(kp) else None, _ptr(new_row), _ptr(freed),
                                    ctypes.byref(nf))
    return new_row[:len(kp)], freed[:nf.value], int(new_n)


# ---------------------------------------------------------------- compaction
def kv_compact(rows, keep):
    """rows[N][...] (any dtype) -> rows[keep] via a byte-wise gather."""
    r = np.ascontiguousarray(rows)
    kp = _c(keep, np.int32)
    row_bytes = r[0].nbytes if r.shape[0] else 0
    out = np.zeros((kp.shape[0],) + r.shape[1:], r.dtype)
    if kp.shape[0]:
        assert kp.min() >= 0 and kp.max() < r.shape[0]
        lib().oracle_kv_compact(int(kp.shape[0]), _ptr(kp), int(row_bytes), _ptr(r), _ptr(out))
    return out


# ---------------------------------------------------------------- attention
def decode_attention(q_bits, keys_bits, vals_bits, scale=None):
    """Single-query softmax attention of q[G][d] over keys/vals[N][d] (bf16 bits) in
    double; scale defaults to 1/sqrt(d).  Returns out[G][d] (float64)."""
    q = _c(q_bits, np.uint16)
    k = _c(keys_bits, np.uint16)
    v = _c(vals_bits, np.uint16)
    G, d = q.shape
    N = k.shape[0]
    assert k.shape == (N, d) and v.shape == (N, d)
    out = np.zeros((G, d), np.float64)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    lib().oracle_decode_attention(N, d, G, _ptr(q), _ptr(k) if N else None,
                                  _ptr(v) if N else None, sc, _ptr(out))
    return out


# ---------------------------------------------------------------- paged reads
def gather_paged(pool, block_row, head, n_slots, block_size=16):
    """Dense rows [n_slots][d] of one head from a paged pool [blocks][H][bs][d]."""
    pool = np.asarray(pool)
    slots = np.arange(n_slots)
    blocks = np.asarray(block_row, np.int64)[slots // block_size]
    return np.ascontiguousarray(pool[blocks, head, slots % block_size])


# ---------------------------------------------------------------- whole pass
def num_threads() -> int:
    return int(lib().oracle_num_threads())


def evict_batch(q, beacons, counts, keys, vals, N, P, B, W=64, bonus=1.0, strict=True):
    """Beacon eviction pass over H independent dense head-caches (OpenMP).

    q[H][T][G][d] bf16 bits, beacons[H][K][d] f32, counts[H][K] i32,
    keys/vals[H][Nmax][d] bf16 bits, N/P[H] i32.  Returns
    (beacons', counts', keep[H][B], kout[H][B][d], vout[H][B][d]); keep rows
    are -1 past the kept count and kout/vout rows past it stay zero.  A
    head-cache whose prompt exceeds the budget is refused: its keep row stays
    -1 and nothing is compacted (its beacons are still updated).  strict=True
    raises on any refusal; strict=False appends the number of refusals to the
    returned tuple.
    """
    q = _c(q, np.uint16)
    H, T, G, d = q.shape
    b = _c(beacons, np.float32).copy()
    c = _c(counts, np.int32).copy()
    K = b.shape[1]
    k = _c(keys, np.uint16)
    v = _c(vals, np.uint16)
    Nmax = k.shape[1]
    n = _c(N, np.int32)
    p = _c(P, np.int32)
    keep = np.full((H, B), -1, np.int32)
    ko = np.zeros((H, B, d), np.uint16)
    vo = np.zeros((H, B, d), np.uint16)
    fails = lib().oracle_evict_batch(H, T, G, d, K, int(B), int(W), float(bonus), Nmax,
                                     _ptr(n), _ptr(p), _ptr(q), _ptr(b), _ptr(c), _ptr(k),
                                     _ptr(v), _ptr(keep), _ptr(ko), _ptr(vo))
    if strict:
        if fails:
            raise ValueError(f"{fails} head-caches refused (prompt exceeds budget)")
        return b, c, keep, ko, vo
    return b, c, keep, ko, vo, int(fails)

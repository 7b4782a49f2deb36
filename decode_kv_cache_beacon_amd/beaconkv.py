"""ctypes binding of libbeaconkv.so (the C ABI in include/beaconkv.h).

Argument marshalling only: every step of the eviction pass runs in the HIP
kernels of the library.  Functions carry the C names; tensors are torch
tensors on the GPU (torch provides device memory and the current stream).
Importing this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbeaconkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m decode_kv_cache_beacon_amd.build` "
        "(the eviction pass has no CPU fallback)")
_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- constants
BKV_ABI_VERSION = 8
# bkv_evict_pass fuses score, select and compact (row compaction with per-head
# selection, or shared positions for the beacon selector) when score_stride +
# budget is at most this
FUSED_MAX_ENTRIES = 15872
# bytes of the scratch array bkv_evict_pass_noalloc holds on each GPU
NOALLOC_SCRATCH_BYTES = 268435456
BKV_OK, BKV_ERR_NULL, BKV_ERR_INVALID, BKV_ERR_BUDGET, BKV_ERR_UNSUPPORTED = 0, 1, 2, 3, 4
BKV_ERR_WORKSPACE, BKV_ERR_HIP, BKV_ERR_LENGTH, BKV_ERR_BLOCK_TABLE = 5, 6, 7, 8
BKV_ERR_SCRATCH = 9
BKV_SCORE_F32, BKV_SCORE_U32 = 0, 1
BKV_SELECT_BEACON, BKV_SELECT_RANDOM = 0, 1
BKV_ROWS_PER_HEAD, BKV_ROWS_PER_LAYER_REQUEST, BKV_ROWS_PER_REQUEST = 0, 1, 2
BKV_PAGES_OFF, BKV_PAGES_PER_REQUEST, BKV_PAGES_PER_HEAD = 0, 1, 2
BKV_MAX_BEACONS = 256
BKV_MAX_CANDIDATES = 32768
BKV_MAX_QUERY_HEADS = 8
HEAD_DIM = 128
BLOCK_SIZE = 16

_P = ctypes.c_void_p
_i32, _i64, _u64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t


class bkv_cache(ctypes.Structure):
    _fields_ = [
        ("n_layers", _i32), ("n_requests", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
        ("block_size", _i32), ("max_blocks", _i32), ("num_blocks", _i64),
        ("k_pools", _P), ("v_pools", _P), ("block_table", _P), ("seq_len", _P),
        ("prompt_len", _P), ("head_block_table", _P), ("head_seq_len", _P),
    ]


class bkv_pass_args(ctypes.Structure):
    _fields_ = [
        ("selector", _i32), ("budget", _i32), ("score_stride", _i32), ("shared_positions", _i32),
        ("page_retention", _i32), ("block_table_out", _P), ("seq_len_out", _P),
        ("freed_blocks", _P),
        ("n_beacons", _i32), ("T", _i32), ("G", _i32), ("window", _i32), ("bonus", _f32),
        ("queries", _P), ("beacons", _P), ("counts", _P), ("assign", _P), ("count_cap", _i32),
        ("lse", _P),
        ("seed", _u64), ("request_ids", _P), ("pass_idx", _P),
        ("pos_ids", _P), ("pos_stride", _i32), ("scores_out", _P), ("keep_out", _P),
        ("timing_events", _P), ("n_timing_events", _i32), ("separate_steps", _i32),
    ]


_lib.bkv_abi_version.argtypes = []
_lib.bkv_abi_version.restype = _i32
_lib.bkv_status_string.argtypes = [_i32]
_lib.bkv_status_string.restype = ctypes.c_char_p
_lib.bkv_beacon_update.argtypes = [_i32, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _i32, _P]
_lib.bkv_beacon_update.restype = _i32
_lib.bkv_beacon_score.argtypes = [ctypes.POINTER(bkv_cache), _P, _P, _i32, _i32, _f32, _P, _i32,
                                  _P, _P, _P]
_lib.bkv_beacon_score.restype = _i32
_lib.bkv_random_score.argtypes = [ctypes.POINTER(bkv_cache), _u64, _P, _P, _i32, _P, _i32, _P,
                                  _P]
_lib.bkv_random_score.restype = _i32
_lib.bkv_topk_select.argtypes = [ctypes.POINTER(bkv_cache), _P, _i32, _i32, _i32, _P, _P, _P]
_lib.bkv_topk_select.restype = _i32
_lib.bkv_topk_select_shared.argtypes = [ctypes.POINTER(bkv_cache), _P, _i32, _i32, _i32, _i32, _P,
                                        _P, _P]
_lib.bkv_topk_select_shared.restype = _i32
_lib.bkv_kv_compact.argtypes = [ctypes.POINTER(bkv_cache), _P, _i32, _i32, _P, _i32, _P, _P]
_lib.bkv_kv_compact.restype = _i32
_lib.bkv_page_retain.argtypes = [ctypes.POINTER(bkv_cache), _P, _i32, _i32, _i32, _i32, _P, _P, _P,
                                 _P, _P, _P]
_lib.bkv_page_retain.restype = _i32
_lib.bkv_page_retain_heads.argtypes = [ctypes.POINTER(bkv_cache), _P, _i32, _i32, _i32, _P, _P,
                                       _P, _P, _P, _P]
_lib.bkv_page_retain_heads.restype = _i32
_lib.bkv_decode_attention.argtypes = [ctypes.POINTER(bkv_cache), _P, _i32, _f32, _P, _P, _P]
_lib.bkv_decode_attention.restype = _i32
_lib.bkv_workspace_size.argtypes = [ctypes.POINTER(bkv_cache), ctypes.POINTER(bkv_pass_args),
                                    ctypes.POINTER(_sz)]
_lib.bkv_workspace_size.restype = _i32
_lib.bkv_evict_pass.argtypes = [ctypes.POINTER(bkv_cache), ctypes.POINTER(bkv_pass_args), _P, _sz,
                                _P, _P]
_lib.bkv_evict_pass.restype = _i32
_lib.bkv_evict_pass_noalloc.argtypes = [ctypes.POINTER(bkv_cache), ctypes.POINTER(bkv_pass_args),
                                        _P, _P]
_lib.bkv_evict_pass_noalloc.restype = _i32

EXPORTS = ("bkv_abi_version", "bkv_status_string", "bkv_beacon_update", "bkv_beacon_score",
           "bkv_random_score", "bkv_topk_select", "bkv_topk_select_shared", "bkv_kv_compact",
           "bkv_page_retain", "bkv_page_retain_heads", "bkv_decode_attention", "bkv_workspace_size", "bkv_evict_pass",
           "bkv_evict_pass_noalloc")


class BkvError(RuntimeError):
    def __init__(self, code: int, where: str, device: bool = False):
        self.code = code
        self.device = device
        if device:
            names = [bkv_status_string(b) for b in range(1, 31) if code & (1 << b)]
            msg = f"{where}: device-detected error bits {code:#x}: " + "; ".join(names)
        else:
            msg = f"{where}: {bkv_status_string(code)} (code {code})"
        super().__init__(msg)


def bkv_abi_version() -> int:
    return int(_lib.bkv_abi_version())


def bkv_status_string(code: int) -> str:
    return _lib.bkv_status_string(int(code)).decode()


# ---------------------------------------------------------------- helpers
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape: Optional[Sequence[int]] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _check(code: int, where: str):
    if code != BKV_OK:
        raise BkvError(code, where)


def _for_stream(t: torch.Tensor, stream) -> torch.Tensor:
    """A tensor this module created on the current stream and hands to kernels
    on `stream`: its initialisation is ordered before `stream`'s later work, and
    the caching allocator does not reuse its memory until that work is done."""
    if stream is not None and stream != torch.cuda.current_stream():
        stream.wait_stream(torch.cuda.current_stream())
        t.record_stream(stream)
    return t


def _status(status: Optional[torch.Tensor], device, stream=None):
    if status is None:
        return _for_stream(torch.zeros(1, dtype=torch.int32, device=device), stream), True
    _need(status, "status", torch.int32)
    return status, False


def check_status(status: torch.Tensor, where: str = "eviction pass", stream=None):
    """Synchronise the stream and raise if the kernels flagged an error."""
    (stream or torch.cuda.current_stream()).synchronize()
    v = int(status.view(-1)[0].item())
    if v:
        raise BkvError(v, where, device=True)


@dataclasses.dataclass
class PagedCache:
    """A paged bf16 KV cache: per-layer pools [num_blocks, H, 16, 128].  With
    head_block_table int32 [HC, max_blocks] and head_seq_len int32 [HC] (both
    or neither), every head-cache reads its slots through its own row (what
    bkv_page_retain_heads writes)."""
    k_pools: list
    v_pools: list
    block_table: torch.Tensor   # int32 [R, max_blocks]
    seq_len: torch.Tensor       # int32 [R]
    prompt_len: torch.Tensor    # int32 [R]
    head_block_table: Optional[torch.Tensor] = None   # int32 [HC, max_blocks]
    head_seq_len: Optional[torch.Tensor] = None       # int32 [HC]
    _k_addr: torch.Tensor = None
    _v_addr: torch.Tensor = None

    def __post_init__(self):
        if len(self.k_pools) != len(self.v_pools) or not self.k_pools:
            raise ValueError("need one K and one V pool per layer")
        shape = tuple(self.k_pools[0].shape)
        if len(shape) != 4 or shape[2] != BLOCK_SIZE or shape[3] != HEAD_DIM:
            raise ValueError(f"pools must be [num_blocks, H, {BLOCK_SIZE}, {HEAD_DIM}] (got {shape})")
        for i, (k, v) in enumerate(zip(self.k_pools, self.v_pools)):
            _need(k, f"k_pools[{i}]", torch.bfloat16, shape)
            _need(v, f"v_pools[{i}]", torch.bfloat16, shape)
        R = self.block_table.shape[0]
        _need(self.block_table, "block_table", torch.int32)
        if self.block_table.dim() != 2:
            raise ValueError("block_table must be [R, max_blocks]")
        _need(self.seq_len, "seq_len", torch.int32, (R,))
        _need(self.prompt_len, "prompt_len", torch.int32, (R,))
        if (self.head_block_table is None) != (self.head_seq_len is None):
            raise ValueError("head_block_table and head_seq_len come together")
        if self.head_block_table is not None:
            HC = len(self.k_pools) * R * shape[1]
            _need(self.head_block_table, "head_block_table", torch.int32,
                  (HC, self.block_table.shape[1]))
            _need(self.head_seq_len, "head_seq_len", torch.int32, (HC,))
        dev = self.k_pools[0].device
        self._k_addr = torch.tensor([t.data_ptr() for t in self.k_pools], dtype=torch.int64,
                                    device=dev)
        self._v_addr = torch.tensor([t.data_ptr() for t in self.v_pools], dtype=torch.int64,
                                    device=dev)

    @property
    def n_layers(self):
        return len(self.k_pools)

    @property
    def n_requests(self):
        return self.block_table.shape[0]

    @property
    def n_kv_heads(self):
        return self.k_pools[0].shape[1]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    @property
    def num_blocks(self):
        return self.k_pools[0].shape[0]

    @property
    def n_head_caches(self):
        return self.n_layers * self.n_requests * self.n_kv_heads

    @property
    def max_slots(self):
        return self.max_blocks * BLOCK_SIZE

    @property
    def device(self):
        return self.k_pools[0].device

    def struct(self) -> bkv_cache:
        return bkv_cache(self.n_layers, self.n_requests, self.n_kv_heads, HEAD_DIM, BLOCK_SIZE,
                         self.max_blocks, self.num_blocks, self._k_addr.data_ptr(),
                         self._v_addr.data_ptr(), self.block_table.data_ptr(),
                         self.seq_len.data_ptr(), self.prompt_len.data_ptr(),
                         None if self.head_block_table is None
                         else self.head_block_table.data_ptr(),
                         None if self.head_seq_len is None else self.head_seq_len.data_ptr())


# ---------------------------------------------------------------- entry points
def bkv_beacon_update(queries, beacons, counts, assign=None, count_cap=0, stream=None):
    """queries bf16 [HC,T,G,128]; beacons fp32 [HC,K,128]; counts int32 [HC,K] (in place);
    count_cap > 0 clamps the counts (moving average once a row is full)."""
    _need(queries, "queries", torch.bfloat16)
    if queries.dim() != 4 or queries.shape[3] != HEAD_DIM:
        raise ValueError("queries must be [HC, T, G, 128]")
    HC, T, G, _ = queries.shape
    if beacons.dim() != 3:
        raise ValueError("beacons must be [HC, K, 128]")
    K = beacons.shape[1]
    _need(beacons, "beacons", torch.float32, (HC, K, HEAD_DIM))
    _need(counts, "counts", torch.int32, (HC, K))
    if assign is not None:
        _need(assign, "assign", torch.int32, (HC, T * G))
    code = _lib.bkv_beacon_update(HC, T, G, HEAD_DIM, K, _ptr(queries), _ptr(beacons),
                                  _ptr(counts), _ptr(assign), int(count_cap), _stream(stream))
    _check(code, "bkv_beacon_update")


def bkv_beacon_score(cache: PagedCache, beacons, counts, scores, window=64, bonus=1.0, lse=None,
                     status=None, check=True, stream=None):
    """scores fp32 [HC, stride] receives score(n) at column n - P."""
    HC = cache.n_head_caches
    if beacons.dim() != 3:
        raise ValueError("beacons must be [HC, K, 128]")
    K = beacons.shape[1]
    _need(beacons, "beacons", torch.float32, (HC, K, HEAD_DIM))
    _need(counts, "counts", torch.int32, (HC, K))
    _need(scores, "scores", torch.float32)
    if scores.dim() != 2 or scores.shape[0] != HC:
        raise ValueError("scores must be [HC, stride]")
    if lse is not None:
        _need(lse, "lse", torch.float32, (HC, K))
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_beacon_score(ctypes.byref(c), _ptr(beacons), _ptr(counts), K, int(window),
                                 float(bonus), _ptr(scores), scores.shape[1], _ptr(lse), _ptr(st),
                                 _stream(stream))
    _check(code, "bkv_beacon_score")
    if own and check:
        check_status(st, "bkv_beacon_score", stream)
    return st


def _layout_rows(cache: PagedCache, rows):
    return {BKV_ROWS_PER_HEAD: cache.n_head_caches,
            BKV_ROWS_PER_LAYER_REQUEST: cache.n_layers * cache.n_requests,
            BKV_ROWS_PER_REQUEST: cache.n_requests}[rows]


def bkv_random_score(cache: PagedCache, seed, request_ids, pass_idx, scores,
                     rows=BKV_ROWS_PER_HEAD, status=None, check=True, stream=None):
    """scores uint32 draws (stored in an int32 tensor) [n_rows, stride]: one row per
    head-cache, per (layer, request) (shared positions) or per request (page retention)."""
    R = cache.n_requests
    layout = int(rows)
    rows = _layout_rows(cache, layout)
    _need(request_ids, "request_ids", torch.int64, (R,))
    _need(pass_idx, "pass_idx", torch.int32, (R,))
    _need(scores, "scores", torch.int32)
    if scores.dim() != 2 or scores.shape[0] != rows:
        raise ValueError(f"scores must be [{rows}, stride]")
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_random_score(ctypes.byref(c), int(seed) & (2**64 - 1), _ptr(request_ids),
                                 _ptr(pass_idx), layout, _ptr(scores),
                                 scores.shape[1], _ptr(st), _stream(stream))
    _check(code, "bkv_random_score")
    if own and check:
        check_status(st, "bkv_random_score", stream)
    return st


def _score_kind(scores):
    if scores.dtype == torch.float32:
        return BKV_SCORE_F32
    if scores.dtype == torch.int32:
        return BKV_SCORE_U32
    raise ValueError("scores must be float32 or int32 (uint32 bit patterns)")


def bkv_topk_select(cache: PagedCache, scores, budget, keep, status=None, check=True,
                    stream=None):
    """scores fp32 (beacon) or int32-stored uint32 (random) [HC, stride]; keep int32 [HC, budget]."""
    HC = cache.n_head_caches
    kind = _score_kind(scores)
    _need(scores, "scores", scores.dtype)
    if scores.dim() != 2 or scores.shape[0] != HC:
        raise ValueError("scores must be [HC, stride]")
    _need(keep, "keep", torch.int32, (HC, budget))
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_topk_select(ctypes.byref(c), _ptr(scores), kind, scores.shape[1], int(budget),
                                _ptr(keep), _ptr(st), _stream(stream))
    _check(code, "bkv_topk_select")
    if own and check:
        check_status(st, "bkv_topk_select", stream)
    return st


def bkv_topk_select_shared(cache: PagedCache, scores, budget, keep, status=None, check=True,
                           stream=None):
    """One selection per (layer, request) for all its heads.

    scores [n_layers * n_requests * S, stride] with S = n_kv_heads (per-head
    scores, merged by their maximum) or S = 1 (one shared draw row);
    keep int32 [n_layers * n_requests, budget]."""
    LR = cache.n_layers * cache.n_requests
    kind = _score_kind(scores)
    _need(scores, "scores", scores.dtype)
    if scores.dim() != 2 or scores.shape[0] % LR:
        raise ValueError("scores must be [n_layers * n_requests * S, stride]")
    S = scores.shape[0] // LR
    _need(keep, "keep", torch.int32, (LR, budget))
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_topk_select_shared(ctypes.byref(c), _ptr(scores), kind, scores.shape[1], S,
                                       int(budget), _ptr(keep), _ptr(st), _stream(stream))
    _check(code, "bkv_topk_select_shared")
    if own and check:
        check_status(st, "bkv_topk_select_shared", stream)
    return st


def bkv_kv_compact(cache: PagedCache, keep, budget, pos_ids=None, status=None, check=True,
                   stream=None, keep_shared=False):
    """In-place compaction of every layer pool; pos_ids int32 [HC, >= max_slots] optional.
    keep int32 [HC, budget], or [n_layers * n_requests, budget] with keep_shared=True."""
    HC = cache.n_head_caches
    rows = cache.n_layers * cache.n_requests if keep_shared else HC
    _need(keep, "keep", torch.int32, (rows, budget))
    pos_stride = 0
    if pos_ids is not None:
        _need(pos_ids, "pos_ids", torch.int32)
        if pos_ids.dim() != 2 or pos_ids.shape[0] != HC:
            raise ValueError("pos_ids must be [HC, stride]")
        pos_stride = pos_ids.shape[1]
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_kv_compact(ctypes.byref(c), _ptr(keep), int(budget), int(bool(keep_shared)),
                               _ptr(pos_ids), pos_stride, _ptr(st), _stream(stream))
    _check(code, "bkv_kv_compact")
    if own and check:
        check_status(st, "bkv_kv_compact", stream)
    return st


def bkv_page_retain(cache: PagedCache, scores, budget, keep_pages, block_table_out, seq_len_out,
                    freed_blocks, rows=BKV_ROWS_PER_HEAD, status=None, check=True, stream=None):
    """Whole-page retention, one selection per request for every layer and head.

    scores: fp32 per-head beacon scores [HC, stride] (rows=BKV_ROWS_PER_HEAD) or int32-stored
    uint32 draws [n_requests, stride] (rows=BKV_ROWS_PER_REQUEST).  keep_pages int32
    [n_requests, budget // 16]; block_table_out int32 [n_requests, max_blocks] and seq_len_out
    int32 [n_requests] (either may be the cache's own tensor: rewritten in place);
    freed_blocks int32 [n_requests, max_blocks]."""
    R = cache.n_requests
    kind = _score_kind(scores)
    _need(scores, "scores", scores.dtype)
    if scores.dim() != 2 or scores.shape[0] != _layout_rows(cache, rows):
        raise ValueError("scores rows do not match the row layout")
    _need(keep_pages, "keep_pages", torch.int32, (R, budget // BLOCK_SIZE))
    _need(block_table_out, "block_table_out", torch.int32, (R, cache.max_blocks))
    _need(seq_len_out, "seq_len_out", torch.int32, (R,))
    _need(freed_blocks, "freed_blocks", torch.int32, (R, cache.max_blocks))
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_page_retain(ctypes.byref(c), _ptr(scores), kind, scores.shape[1], int(rows),
                                int(budget), _ptr(keep_pages), _ptr(block_table_out),
                                _ptr(seq_len_out), _ptr(freed_blocks), _ptr(st), _stream(stream))
    _check(code, "bkv_page_retain")
    if own and check:
        check_status(st, "bkv_page_retain", stream)
    return st


def bkv_page_retain_heads(cache: PagedCache, scores, budget, keep_pages, head_table_out,
                          head_seq_len_out, dropped_blocks, status=None, check=True, stream=None):
    """Whole-page retention per head-cache: each head-cache keeps budget // 16
    pages chosen from its own score row.

    scores: fp32 beacon scores or int32-stored uint32 draws, [HC, stride].
    keep_pages int32 [HC, budget // 16]; head_table_out int32 [HC, max_blocks] and
    head_seq_len_out int32 [HC] (either may be the cache's own per-head tensor:
    rewritten in place); dropped_blocks int32 [HC, max_blocks].  Reading the cache
    afterwards: PagedCache(..., head_block_table=head_table_out,
    head_seq_len=head_seq_len_out)."""
    HC = cache.n_head_caches
    kind = _score_kind(scores)
    _need(scores, "scores", scores.dtype)
    if scores.dim() != 2 or scores.shape[0] != HC:
        raise ValueError("scores must be [HC, stride]")
    _need(keep_pages, "keep_pages", torch.int32, (HC, budget // BLOCK_SIZE))
    _need(head_table_out, "head_table_out", torch.int32, (HC, cache.max_blocks))
    _need(head_seq_len_out, "head_seq_len_out", torch.int32, (HC,))
    _need(dropped_blocks, "dropped_blocks", torch.int32, (HC, cache.max_blocks))
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_page_retain_heads(ctypes.byref(c), _ptr(scores), kind, scores.shape[1],
                                      int(budget), _ptr(keep_pages), _ptr(head_table_out),
                                      _ptr(head_seq_len_out), _ptr(dropped_blocks), _ptr(st),
                                      _stream(stream))
    _check(code, "bkv_page_retain_heads")
    if own and check:
        check_status(st, "bkv_page_retain_heads", stream)
    return st


def bkv_decode_attention(cache: PagedCache, queries, out, scale=None, status=None, check=True,
                         stream=None):
    """queries bf16 [HC, G, 128] -> out fp32 [HC, G, 128]: softmax attention of every query
    head over the slots [0, seq_len) of its head-cache; scale defaults to 1/sqrt(128)."""
    HC = cache.n_head_caches
    _need(queries, "queries", torch.bfloat16)
    if queries.dim() != 3 or queries.shape[0] != HC or queries.shape[2] != HEAD_DIM:
        raise ValueError("queries must be [HC, G, 128]")
    G = queries.shape[1]
    _need(out, "out", torch.float32, (HC, G, HEAD_DIM))
    sc = HEAD_DIM ** -0.5 if scale is None else float(scale)
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_decode_attention(ctypes.byref(c), _ptr(queries), G, sc, _ptr(out), _ptr(st),
                                     _stream(stream))
    _check(code, "bkv_decode_attention")
    if own and check:
        check_status(st, "bkv_decode_attention", stream)
    return st


def _pass_args(cache: PagedCache, selector, budget, queries, beacons, counts, window, bonus,
               assign, lse, seed, request_ids, pass_idx, pos_ids, scores_out, keep_out,
               score_stride, count_cap=0, shared_positions=False, page_retention=None,
               separate_steps=False, page_heads=False):
    HC, R = cache.n_head_caches, cache.n_requests
    LR = cache.n_layers * R
    a = bkv_pass_args()
    a.selector = selector
    a.budget = int(budget)
    a.score_stride = int(score_stride)
    a.shared_positions = int(bool(shared_positions))
    a.separate_steps = int(bool(separate_steps))
    if page_retention is not None:
        bto, slo, fr = page_retention
        U = HC if page_heads else R
        _need(bto, "block_table_out", torch.int32, (U, cache.max_blocks))
        _need(slo, "seq_len_out", torch.int32, (U,))
        _need(fr, "freed_blocks", torch.int32, (U, cache.max_blocks))
        a.page_retention = BKV_PAGES_PER_HEAD if page_heads else BKV_PAGES_PER_REQUEST
        a.block_table_out, a.seq_len_out, a.freed_blocks = bto.data_ptr(), slo.data_ptr(), fr.data_ptr()
    if selector == BKV_SELECT_BEACON:
        _need(queries, "queries", torch.bfloat16)
        if queries.dim() != 4 or queries.shape[0] != HC or queries.shape[3] != HEAD_DIM:
            raise ValueError("queries must be [HC, T, G, 128]")
        K = beacons.shape[1]
        _need(beacons, "beacons", torch.float32, (HC, K, HEAD_DIM))
        _need(counts, "counts", torch.int32, (HC, K))
        a.n_beacons, a.T, a.G = K, queries.shape[1], queries.shape[2]
        a.window, a.bonus = int(window), float(bonus)
        a.count_cap = int(count_cap)
        a.queries, a.beacons, a.counts = queries.data_ptr(), beacons.data_ptr(), counts.data_ptr()
        if assign is not None:
            _need(assign, "assign", torch.int32, (HC, a.T * a.G))
            a.assign = assign.data_ptr()
        if lse is not None:
            _need(lse, "lse", torch.float32, (HC, K))
            a.lse = lse.data_ptr()
    elif selector == BKV_SELECT_RANDOM:
        _need(request_ids, "request_ids", torch.int64, (R,))
        _need(pass_idx, "pass_idx", torch.int32, (R,))
        a.seed = int(seed) & (2**64 - 1)
        a.request_ids, a.pass_idx = request_ids.data_ptr(), pass_idx.data_ptr()
    else:
        raise ValueError("selector must be BKV_SELECT_BEACON or BKV_SELECT_RANDOM")
    if pos_ids is not None:
        _need(pos_ids, "pos_ids", torch.int32)
        a.pos_ids, a.pos_stride = pos_ids.data_ptr(), pos_ids.shape[1]
    stride = score_stride if score_stride > 0 else cache.max_slots
    if scores_out is not None:
        want = torch.float32 if selector == BKV_SELECT_BEACON else torch.int32
        rows = HC
        if selector == BKV_SELECT_RANDOM and page_retention is not None and not page_heads:
            rows = R
        elif selector == BKV_SELECT_RANDOM and shared_positions:
            rows = LR
        _need(scores_out, "scores_out", want, (rows, stride))
        a.scores_out = scores_out.data_ptr()
    if keep_out is not None:
        if page_retention is not None:
            shape = (HC if page_heads else R, budget // BLOCK_SIZE)
        else:
            shape = (LR if shared_positions else HC, budget)
        _need(keep_out, "keep_out", torch.int32, shape)
        a.keep_out = keep_out.data_ptr()
    return a


def _timing_args(a: bkv_pass_args, timing_events, stream):
    """Puts the HIP handles of torch timing events into the pass arguments;
    returns the handle array, which must outlive the call."""
    if timing_events is None:
        return None
    handles = []
    for e in timing_events:
        if e.cuda_event == 0:            # torch creates the HIP event lazily
            e.record(stream or torch.cuda.current_stream())
        handles.append(e.cuda_event)
    ev_arr = (ctypes.c_void_p * len(handles))(*handles)
    a.timing_events = ctypes.cast(ev_arr, ctypes.c_void_p)
    a.n_timing_events = len(handles)
    return ev_arr


def bkv_workspace_size(cache: PagedCache, args: bkv_pass_args) -> int:
    n = _sz(0)
    c = cache.struct()
    _check(_lib.bkv_workspace_size(ctypes.byref(c), ctypes.byref(args), ctypes.byref(n)),
           "bkv_workspace_size")
    return int(n.value)


def bkv_evict_pass(cache: PagedCache, selector, budget, *, queries=None, beacons=None,
                   counts=None, window=64, bonus=1.0, assign=None, lse=None, seed=0,
                   request_ids=None, pass_idx=None, pos_ids=None, scores_out=None,
                   keep_out=None, score_stride=0, workspace=None, status=None, check=True,
                   stream=None, timing_events=None, count_cap=0, shared_positions=False,
                   page_retention=None, separate_steps=False, page_heads=False):
    """One whole eviction pass (beacon: update -> score -> select -> compact;
    random: score -> select -> compact), every layer/request/head at once.
    shared_positions: one selection per (layer, request) for all its heads.
    page_retention: (block_table_out, seq_len_out, freed_blocks) to keep whole
    pages per request instead (no rows move; keep_out is then the kept pages);
    with page_heads=True every head-cache keeps its own pages and the three
    outputs are per head-cache ([HC, max_blocks], [HC], [HC, max_blocks]).

    separate_steps: run score, select and compact as three kernels even where
    a fused kernel applies (row compaction with per-head selection for either
    selector, or with shared positions for the beacon selector).

    timing_events: optional list of torch.cuda.Event(enable_timing=True), 5 for
    the beacon selector and 4 for the random one, recorded around each step
    (with the fused kernel the score interval covers score, select and
    compact, and the other two are empty)."""
    a = _pass_args(cache, selector, budget, queries, beacons, counts, window, bonus, assign, lse,
                   seed, request_ids, pass_idx, pos_ids, scores_out, keep_out, score_stride,
                   count_cap, shared_positions, page_retention, separate_steps, page_heads)
    ev_arr = _timing_args(a, timing_events, stream)  # noqa: F841 (kept alive for the call)
    need = bkv_workspace_size(cache, a)
    if workspace is None and need:
        workspace = _for_stream(torch.empty(need, dtype=torch.uint8, device=cache.device), stream)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    st, own = _status(status, cache.device, stream)
    c = cache.struct()
    code = _lib.bkv_evict_pass(ctypes.byref(c), ctypes.byref(a), _ptr(workspace),
                               0 if workspace is None else workspace.numel(), _ptr(st),
                               _stream(stream))
    _check(code, "bkv_evict_pass")
    if own and check:
        check_status(st, "bkv_evict_pass", stream)
    return st


def bkv_evict_pass_noalloc(cache: PagedCache, selector, budget, *, queries=None, beacons=None,
                           counts=None, window=64, bonus=1.0, assign=None, lse=None, seed=0,
                           request_ids=None, pass_idx=None, pos_ids=None, scores_out=None,
                           keep_out=None, score_stride=0, status=None, stream=None,
                           timing_events=None, count_cap=0, shared_positions=False,
                           page_retention=None, separate_steps=False, page_heads=False):
    """bkv_evict_pass for callers that cannot allocate device memory: the
    score and keep buffers it is not given live in the library's per-GPU
    scratch array (NOALLOC_SCRATCH_BYTES; larger passes raise BKV_ERR_SCRATCH).
    Nothing is allocated here either: `status` (int32 [1], caller-zeroed) is
    optional and is not checked (call check_status to see device-detected
    errors).  Calls whose work overlaps on one GPU share the scratch and race."""
    a = _pass_args(cache, selector, budget, queries, beacons, counts, window, bonus, assign, lse,
                   seed, request_ids, pass_idx, pos_ids, scores_out, keep_out, score_stride,
                   count_cap, shared_positions, page_retention, separate_steps, page_heads)
    ev_arr = _timing_args(a, timing_events, stream)  # noqa: F841 (kept alive for the call)
    if status is not None:
        _need(status, "status", torch.int32)
    c = cache.struct()
    code = _lib.bkv_evict_pass_noalloc(ctypes.byref(c), ctypes.byref(a), _ptr(status),
                                       _stream(stream))
    _check(code, "bkv_evict_pass_noalloc")

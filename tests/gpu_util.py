"""Host-side helpers shared by the GPU parity tests (no method arithmetic).

They move synthetic batches to the GPU, cut per-head dense views out of host
copies for the oracle, and implement the comparison rules:
  * Philox draws, keep lists and compacted K/V bytes: bit-exact;
  * float scores: |gpu - oracle| <= 1e-3 |oracle| + 1e-30;
  * beacon selection: a slot may differ from the oracle's choice only if its
    oracle score is within 1e-3 (relative) of the oracle's boundary score;
  * beacon assignment (teacher-forced): the GPU's row must be the oracle's
    cosine argmax to within ASSIGN_TOL (fp64 rounding), and the replayed state
    must match bit for bit.
"""
import numpy as np
import torch

from decode_kv_cache_beacon_amd import beaconkv as bk
from decode_kv_cache_beacon_amd import synth

SCORE_RTOL = 1e-3
SCORE_ATOL = 1e-30
# Beacon assignment: the GPU picks a row whose cosine lies within a rigorous
# bound of the best, and re-ranks every such near tie in fp64 from the actual
# fp32 rows; the oracle ranks in fp64 too.  Each side's cosine is a sum of 128
# exact products (bf16 x fp32 fits a double) with at most 127 roundings,
# norms alike, then a square root and a divide: within about 3e-14 of the
# exact cosine.  Two rows can therefore be ranked differently only when their
# cosines lie within about 6e-14, so every pick is the oracle's argmax to
# within 1e-12; picks with a positive gap at all (INEXACT_LIMIT) need such a
# near tie, which the seeded inputs do not contain.
ASSIGN_TOL = 1e-12
INEXACT_LIMIT = 0
# Decode attention, |gpu - oracle| <= ATT_TOL * max |v| of the head-cache: the
# fp32 logit (128 exact bf16 products, fp32 sums) is off by at most ~128 u |q||k|
# scale, at most ~3e-4 in log units for these inputs; a weight p = exp(s - m)
# then carries that relative error, plus ~1e-6 from exp2 and the rescalings,
# and sum_n p_n v_n / sum_n p_n inherits it times max |v|.  1e-3 leaves a
# margin of three over that worst case.
ATT_TOL = 1e-3


def hc_index(R, H, layer, req, head):
    return (layer * R + req) * H + head


def device_cache(batch, seq_len=None, prompt_len=None):
    dev = torch.device("cuda")
    kp = [k.to(dev) for k in batch.k_pools]
    vp = [v.to(dev) for v in batch.v_pools]
    N = batch.seq_len if seq_len is None else torch.as_tensor(seq_len, dtype=torch.int32)
    P = batch.prompt_len if prompt_len is None else torch.as_tensor(prompt_len, dtype=torch.int32)
    return bk.PagedCache(kp, vp, batch.block_table.to(dev).contiguous(), N.to(dev).contiguous(),
                         P.to(dev).contiguous())


def host_pools(cache):
    """uint16 numpy copies of every layer's K and V pool."""
    ks = [synth.bits(k) for k in cache.k_pools]
    vs = [synth.bits(v) for v in cache.v_pools]
    return ks, vs


def check_scores(gpu, ref, where=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, where
    err = np.abs(gpu - ref)
    bound = SCORE_RTOL * np.abs(ref) + SCORE_ATOL
    bad = np.flatnonzero(~(err <= bound))
    assert bad.size == 0, (f"{where}: {bad.size} scores off, worst rel "
                           f"{np.max(err / np.maximum(np.abs(ref), 1e-30)):.3e} at {bad[:5]}")


def check_selection(gpu_keep, ref_keep, ref_scores, N, P, B, where=""):
    """Kept sets may differ only at slots whose oracle score ties the boundary
    to within SCORE_RTOL."""
    g = set(int(v) for v in gpu_keep if v >= 0)
    o = set(int(v) for v in ref_keep)
    assert len(g) == len(o) == min(N, B), where
    assert all(i in g for i in range(min(P, B))), f"{where}: prompt not kept"
    diff = g ^ o
    if not diff:
        return 0
    k = B - P
    boundary = np.sort(np.asarray(ref_scores, np.float64))[::-1][k - 1]
    for n in diff:
        s = ref_scores[n - P]
        assert abs(s - boundary) <= SCORE_RTOL * abs(boundary) + SCORE_ATOL, (
            f"{where}: slot {n} differs with oracle score {s} vs boundary {boundary}")
    return len(diff)


def bf16_values(bits):
    """float32 values of bf16 bit patterns."""
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def keep_rows(keep_row):
    """Valid entries of one GPU keep row (drops the -1 padding)."""
    k = np.asarray(keep_row)
    return k[k >= 0]

"""Seeded synthetic inputs for the eviction pass (no method arithmetic here).

This module only draws data: Gaussian-mixture keys and decode queries, values,
a warmed-up beacon state, paged block tables and sequence/prompt lengths.  It
computes nothing the eviction pass computes, so both the HIP path and the CPU
oracle can be fed from it.

Recipe (one seed drives everything; draws are made with ``torch.Generator`` on
the device asked for, so a given seed reproduces exactly on the same device
type):
  * per (layer, KV head): channel scales sigma_c ~ U(0.5, 2) and C cluster
    centres mu_m ~ N(0, I_d);
  * keys of one head-cache: sigma * z with z ~ N(0, I_d); C planted spans of 16
    slots each (one 16-slot aligned window per span, windows chosen without
    replacement in [P, N - W)) hold sigma * z + mu_m instead;
  * values: N(0, 1);
  * decode queries [T][G][d]: with probability p_revisit the centre of a span
    that starts in the first 5% of the generated part, with probability
    p_centre a random centre, each plus 0.3 * N(0, I); otherwise N(0, I);
  * warmed beacon state (when asked for): count c_j ~ U{4..64};
    b_j = mu_j + 0.3 / sqrt(c_j) * z for the first C rows, z / sqrt(c_j) for
    the rest (the spread of a mean of c_j such queries); otherwise all zero;
  * block tables: dense caches use the identity map, paged caches a seeded
    random permutation of all physical blocks;
  * everything stored as bf16 is drawn in fp32 and rounded by torch.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

BLOCK = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_requests: int
    n_kv_heads: int
    group: int            # query heads per KV head (G)
    n_beacons: int        # K
    budget: int           # B (prompt included)
    prompt_len: int       # P (or the low end when prompt_range is set)
    seq_len: int          # N at the pass
    steps: int            # T decode steps buffered since the last pass
    n_clusters: int       # C
    paged: bool
    prewarm: bool
    head_dim: int = 128
    window: int = 64      # W
    bonus: float = 1.0
    p_centre: float = 0.2
    p_revisit: float = 0.0
    noise_std: float = 0.3
    prompt_range: Optional[tuple] = None   # (lo, hi) inclusive, per request
    seed: int = 1

    @property
    def n_head_caches(self) -> int:
        return self.n_layers * self.n_requests * self.n_kv_heads

    @property
    def blocks_per_request(self) -> int:
        return (self.seq_len + BLOCK - 1) // BLOCK

    @property
    def num_blocks(self) -> int:
        return self.n_requests * self.blocks_per_request

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Synthetic stand-ins for the pages' workload shapes.
WORKLOADS = {
    # one head, one layer; one-shot pass over a 4096-slot cache
    "tiny": Workload("tiny", 1, 1, 1, 1, 64, 1024, 512, 4096, 256, 8,
                     paged=False, prewarm=False, seed=1),
    # Qwen3-4B-like GQA batch, 16 requests, steady state N = B + 64
    "qwen3_4b_r16": Workload("qwen3_4b_r16", 36, 16, 8, 4, 64, 2048, 1024, 2112, 64, 16,
                             paged=False, prewarm=True, seed=2),
    # serving scale: 128 requests, paged 16-token blocks, permuted tables
    "serving_r128": Workload("serving_r128", 36, 128, 8, 4, 128, 2048, 1024, 2112, 64, 16,
                             paged=True, prewarm=True, seed=3),
    # Qwen3-32B-like, K = 256 beacons, revisiting queries (B = 2048 variant)
    "qwen3_32b_r32": Workload("qwen3_32b_r32", 64, 32, 8, 8, 256, 2048, 512, 2112, 64, 32,
                              paged=True, prewarm=True, p_revisit=0.1, seed=4),
    # serving shape with long, varying prompts
    "long_prompt_r128": Workload("long_prompt_r128", 36, 128, 8, 4, 128, 3072, 256, 3136, 64, 16,
                                 paged=True, prewarm=True, prompt_range=(256, 1536), seed=6),
}


def _gen(device, seed: int, *salt: int) -> torch.Generator:
    g = torch.Generator(device=device)
    s = seed
    for v in salt:
        s = (s * 1000003 + v + 1) % (2**63 - 1)
    g.manual_seed(s)
    return g


def prompt_lengths(wl: Workload) -> torch.Tensor:
    """int32 [R] prompt lengths (drawn on the CPU so they match on any device)."""
    if wl.prompt_range is None:
        return torch.full((wl.n_requests,), wl.prompt_len, dtype=torch.int32)
    lo, hi = wl.prompt_range
    g = _gen("cpu", wl.seed, 7)
    return torch.randint(lo, hi + 1, (wl.n_requests,), generator=g, dtype=torch.int32)


def block_table(wl: Workload) -> torch.Tensor:
    """int32 [R, blocks_per_request] logical -> physical block ids."""
    nb = wl.blocks_per_request
    if wl.paged:
        g = _gen("cpu", wl.seed, 11)
        perm = torch.randperm(wl.num_blocks, generator=g).to(torch.int32)
    else:
        perm = torch.arange(wl.num_blocks, dtype=torch.int32)
    return perm.reshape(wl.n_requests, nb).contiguous()


def layer_params(wl: Workload, layer: int, device="cpu"):
    """(scales [H, d], centres [H, C, d]) fp32 for one layer."""
    g = _gen(device, wl.seed, 13, layer)
    H, d, C = wl.n_kv_heads, wl.head_dim, wl.n_clusters
    scales = torch.rand(H, d, generator=g, device=device) * 1.5 + 0.5
    centres = torch.randn(H, C, d, generator=g, device=device)
    return scales, centres


def span_windows(wl: Workload, layer: int, prompt_len: torch.Tensor):
    """int64 [R, H, C] span start slots (multiples of 16; -1 when none fit).

    Block-aligned windows of 16 slots inside [P, N - W) are chosen without
    replacement, so every span fills exactly one cache block.  With
    p_revisit > 0 the first span of every head-cache starts inside the first
    5% of the generated part [P, N).
    """
    R, H, C = wl.n_requests, wl.n_kv_heads, wl.n_clusters
    g = _gen("cpu", wl.seed, 17, layer)
    starts = torch.zeros(R, H, C, dtype=torch.int64)
    for r in range(R):
        P = int(prompt_len[r])
        p0 = (P + BLOCK - 1) // BLOCK * BLOCK        # first block boundary >= P
        n_win = max((wl.seq_len - wl.window - p0) // BLOCK, 0)
        take = min(C, n_win)
        if take == 0:
            starts[r] = -1
            continue
        order = torch.argsort(torch.rand(H, n_win, generator=g), dim=1)[:, :take]
        if wl.p_revisit > 0:
            early = max(int(0.05 * (wl.seq_len - P)) // BLOCK, 1)
            first = torch.randint(0, min(early, n_win), (H,), generator=g)
            # put an early window first, keep the rest distinct from it
            rest = []
            for h in range(H):
                row = [int(w) for w in order[h] if int(w) != int(first[h])][: take - 1]
                rest.append([int(first[h])] + row)
            order = torch.tensor(rest, dtype=torch.int64)
        s = p0 + order * BLOCK
        if take < C:
            pad = torch.full((H, C - take), -1, dtype=torch.int64)
            s = torch.cat([s, pad], dim=1)
        starts[r] = s
    return starts


def layer_kv(wl: Workload, layer: int, table: torch.Tensor, prompt_len: torch.Tensor,
             device="cpu"):
    """Paged K and V pools of one layer: bf16 [num_blocks, H, 16, d] each."""
    H, d = wl.n_kv_heads, wl.head_dim
    scales, centres = layer_params(wl, layer, device)
    g = _gen(device, wl.seed, 19, layer)
    nblk = wl.num_blocks
    k = torch.randn(nblk, H, BLOCK, d, generator=g, device=device)
    k.mul_(scales.view(1, H, 1, d))
    starts = span_windows(wl, layer, prompt_len)               # [R, H, C]
    R, C = wl.n_requests, wl.n_clusters
    r_idx = torch.arange(R).view(R, 1, 1).expand(R, H, C)
    h_idx = torch.arange(H).view(1, H, 1).expand(R, H, C)
    m_idx = torch.arange(C).view(1, 1, C).expand(R, H, C)
    ok = starts >= 0
    if bool(ok.any()):
        rr, hh, mm, ss = r_idx[ok], h_idx[ok], m_idx[ok], starts[ok]
        blk = table[rr, ss // BLOCK].long().to(device)
        k[blk, hh.to(device)] += centres[hh.to(device), mm.to(device)].unsqueeze(1)
    kb = k.to(torch.bfloat16)
    del k
    v = torch.randn(nblk, H, BLOCK, d, generator=g, device=device).to(torch.bfloat16)
    return kb, v


def _query_draws(wl: Workload, layer: int, device="cpu"):
    """The random draws behind one layer's queries: noise z [R, H, T, G, d],
    uniform u [R, H, T, G] (which kind of query) and cluster m [R, H, T, G]."""
    R, H, T, G, d, C = (wl.n_requests, wl.n_kv_heads, wl.steps, wl.group, wl.head_dim,
                        wl.n_clusters)
    g = _gen(device, wl.seed, 23, layer)
    z = torch.randn(R, H, T, G, d, generator=g, device=device)
    u = torch.rand(R, H, T, G, generator=g, device=device)
    m = torch.randint(0, C, (R, H, T, G), generator=g, device=device)
    return z, u, m


def query_clusters(wl: Workload, layer: int) -> torch.Tensor:
    """int64 [R, H, T, G]: the cluster each decode query of one layer aims at
    (the span planted on that cluster's centre), or -1 for a plain N(0, I)
    query.  Revisiting queries aim at cluster 0."""
    _, u, m = _query_draws(wl, layer, "cpu")
    is_centre = (u >= wl.p_revisit) & (u < wl.p_revisit + wl.p_centre)
    out = torch.where(is_centre, m, torch.full_like(m, -1))
    if wl.p_revisit > 0:
        out = torch.where(u < wl.p_revisit, torch.zeros_like(m), out)
    return out


def layer_queries(wl: Workload, layer: int, prompt_len: torch.Tensor, device="cpu"):
    """bf16 decode queries [R, H, T, G, d] of one layer."""
    H, d = wl.n_kv_heads, wl.head_dim
    _, centres = layer_params(wl, layer, device)
    z, u, m = _query_draws(wl, layer, device)
    cen = centres[torch.arange(H, device=device).view(1, H, 1, 1), m]   # [R,H,T,G,d]
    is_centre = (u >= wl.p_revisit) & (u < wl.p_revisit + wl.p_centre)
    q = torch.where(is_centre.unsqueeze(-1), cen + wl.noise_std * z, z)
    if wl.p_revisit > 0:
        # revisiting queries aim at the early span of their head-cache (cluster 0)
        early = centres[:, 0].view(1, H, 1, 1, d)
        q = torch.where((u < wl.p_revisit).unsqueeze(-1), early + wl.noise_std * z, q)
    return q.to(torch.bfloat16)


def layer_beacons(wl: Workload, layer: int, device="cpu"):
    """(beacons fp32 [R, H, K, d], counts int32 [R, H, K]) of one layer."""
    R, H, K, d, C = wl.n_requests, wl.n_kv_heads, wl.n_beacons, wl.head_dim, wl.n_clusters
    if not wl.prewarm:
        return (torch.zeros(R, H, K, d, device=device),
                torch.zeros(R, H, K, dtype=torch.int32, device=device))
    _, centres = layer_params(wl, layer, device)
    g = _gen(device, wl.seed, 29, layer)
    counts = torch.randint(4, 65, (R, H, K), generator=g, device=device, dtype=torch.int32)
    z = torch.randn(R, H, K, d, generator=g, device=device)
    spread = counts.to(torch.float32).rsqrt().unsqueeze(-1)
    b = z * spread
    nc = min(K, C)
    b[:, :, :nc] = centres[:, :nc].unsqueeze(0) + wl.noise_std * b[:, :, :nc]
    return b.contiguous(), counts


def fresh_tail(wl: Workload, layer: int, step: int, device="cpu"):
    """New K/V rows for the W slots appended between two passes: bf16 [R, H, W, d]."""
    R, H, W, d = wl.n_requests, wl.n_kv_heads, wl.window, wl.head_dim
    scales, _ = layer_params(wl, layer, device)
    g = _gen(device, wl.seed, 31, layer, step)
    k = (torch.randn(R, H, W, d, generator=g, device=device)
         * scales.view(1, H, 1, d)).to(torch.bfloat16)
    v = torch.randn(R, H, W, d, generator=g, device=device).to(torch.bfloat16)
    return k, v


@dataclasses.dataclass
class Batch:
    """All inputs of one pass.  Layer-major head-cache order hc = (l*R + r)*H + h."""
    wl: Workload
    k_pools: list          # L x bf16 [num_blocks, H, 16, d]
    v_pools: list
    block_table: torch.Tensor   # int32 [R, blocks_per_request]
    seq_len: torch.Tensor       # int32 [R]
    prompt_len: torch.Tensor    # int32 [R]
    queries: torch.Tensor       # bf16 [HC, T, G, d]
    beacons: torch.Tensor       # fp32 [HC, K, d]
    counts: torch.Tensor        # int32 [HC, K]


def make_batch(wl: Workload, device="cpu") -> Batch:
    table = block_table(wl)
    P = prompt_lengths(wl)
    N = torch.full((wl.n_requests,), wl.seq_len, dtype=torch.int32)
    kp, vp, qs, bs, cs = [], [], [], [], []
    for layer in range(wl.n_layers):
        k, v = layer_kv(wl, layer, table, P, device)
        kp.append(k)
        vp.append(v)
        qs.append(layer_queries(wl, layer, P, device).reshape(-1, wl.steps, wl.group, wl.head_dim))
        b, c = layer_beacons(wl, layer, device)
        bs.append(b.reshape(-1, wl.n_beacons, wl.head_dim))
        cs.append(c.reshape(-1, wl.n_beacons))
    dev = torch.device(device)
    return Batch(wl, kp, vp, table.to(dev), N.to(dev), P.to(dev),
                 torch.cat(qs).contiguous(), torch.cat(bs).contiguous(),
                 torch.cat(cs).contiguous())


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def max_slots(wl: Workload) -> int:
    return wl.blocks_per_request * BLOCK


__all__ = ["Workload", "WORKLOADS", "Batch", "make_batch", "block_table", "prompt_lengths",
           "layer_kv", "layer_queries", "layer_beacons", "fresh_tail", "bits", "max_slots",
           "span_windows", "layer_params", "BLOCK"]

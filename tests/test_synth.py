"""The seeded input generator: determinism, shapes and layout validity (CPU)."""
import numpy as np
import torch

from decode_kv_cache_beacon_amd import synth


def test_deterministic_per_seed():
    wl = synth.WORKLOADS["serving_r128"].with_(n_layers=1, n_requests=2)
    a = synth.make_batch(wl)
    b = synth.make_batch(wl)
    assert torch.equal(a.k_pools[0].view(torch.int16), b.k_pools[0].view(torch.int16))
    assert torch.equal(a.queries.view(torch.int16), b.queries.view(torch.int16))
    assert torch.equal(a.beacons, b.beacons) and torch.equal(a.counts, b.counts)
    c = synth.make_batch(wl.with_(seed=99))
    assert not torch.equal(a.k_pools[0].view(torch.int16), c.k_pools[0].view(torch.int16))


def test_block_tables_are_permutations():
    for name in ("serving_r128", "qwen3_4b_r16"):
        wl = synth.WORKLOADS[name].with_(n_requests=5)
        t = synth.block_table(wl)
        assert t.shape == (5, wl.blocks_per_request)
        assert sorted(t.flatten().tolist()) == list(range(wl.num_blocks))
    dense = synth.block_table(synth.WORKLOADS["qwen3_4b_r16"].with_(n_requests=3))
    assert torch.equal(dense.flatten(), torch.arange(dense.numel(), dtype=torch.int32))


def test_shapes_of_tiny():
    wl = synth.WORKLOADS["tiny"]
    b = synth.make_batch(wl)
    assert b.k_pools[0].shape == (256, 1, 16, 128) and b.k_pools[0].dtype == torch.bfloat16
    assert b.queries.shape == (1, 256, 1, 128)
    assert int(b.counts.sum()) == 0 and float(b.beacons.abs().sum()) == 0.0
    assert int(b.seq_len[0]) == 4096 and int(b.prompt_len[0]) == 512


def test_planted_spans_sit_on_centres():
    wl = synth.WORKLOADS["tiny"]
    b = synth.make_batch(wl)
    scales, centres = synth.layer_params(wl, 0)
    starts = synth.span_windows(wl, 0, b.prompt_len)[0, 0]
    keys = b.k_pools[0][:, 0].reshape(-1, 128).float()
    for m, s in enumerate(starts.tolist()):
        assert s % 16 == 0 and 512 <= s and s + 16 <= 4096 - 64
        span = keys[s:s + 16]
        # mean over the span approaches the centre (noise sd ~ scale / 4)
        err = (span.mean(0) - centres[0, m]).abs().mean()
        assert err < 0.6, (m, float(err))
    assert len(set(starts.tolist())) == wl.n_clusters


def test_long_prompt_lengths_in_range():
    wl = synth.WORKLOADS["long_prompt_r128"]
    P = synth.prompt_lengths(wl)
    assert P.shape == (128,) and int(P.min()) >= 256 and int(P.max()) <= 1536
    assert len(set(P.tolist())) > 50


def test_revisit_first_span_is_early():
    wl = synth.WORKLOADS["qwen3_32b_r32"].with_(n_layers=1, n_requests=3)
    P = synth.prompt_lengths(wl)
    s = synth.span_windows(wl, 0, P)
    early_end = 512 + int(0.05 * (2112 - 512))
    assert bool((s[:, :, 0] < early_end).all())
    for r in range(3):
        for h in range(8):
            assert len(set(s[r, h].tolist())) == wl.n_clusters


def test_bits_roundtrip():
    x = torch.randn(7, 5).to(torch.bfloat16)
    u = synth.bits(x)
    assert u.dtype == np.uint16
    back = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16)
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))

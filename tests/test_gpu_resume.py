"""Checkpoint and resume of a decode loop around the pass.

Everything a pass carries to the next lives in the caller's buffers: the K/V
pools, the beacons and counts (BeaconKV explainer, section 3.3: the beacon
state is O(K)), the position ids, and for the random selector the per-request
pass index that makes every pass draw afresh (Random Attention article,
section "Random Attention").  So 2m passes run straight through must equal m
passes, a save of that state to host memory, a restore into freshly allocated
device tensors, and m more passes -- byte for byte, for both selectors.
Between passes the 64 tail slots receive fresh rows (the tokens decoded since
the last pass) and every pass absorbs fresh decode queries."""
import numpy as np
import pytest
import torch

from decode_kv_cache_beacon_amd import synth

pytestmark = pytest.mark.gpu

bk = None
M = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global bk
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from decode_kv_cache_beacon_amd import beaconkv
    bk = beaconkv
    torch.cuda.init()
    yield


WL = synth.WORKLOADS["serving_r128"].with_(n_layers=2, n_requests=3, n_kv_heads=2, budget=256,
                                          prompt_len=100, seq_len=320, n_beacons=40)


class State:
    """The decode loop's device state; `save` returns host copies, and a State
    built from them allocates new device tensors."""
    FIELDS = ("k", "v", "beacons", "counts", "pos", "pass_idx")

    def __init__(self, host):
        dev = torch.device("cuda")
        self.k = [torch.from_numpy(a).to(dev).view(torch.bfloat16) for a in host["k"]]
        self.v = [torch.from_numpy(a).to(dev).view(torch.bfloat16) for a in host["v"]]
        self.beacons = torch.from_numpy(host["beacons"]).to(dev)
        self.counts = torch.from_numpy(host["counts"]).to(dev)
        self.pos = torch.from_numpy(host["pos"]).to(dev)
        self.pass_idx = torch.from_numpy(host["pass_idx"]).to(dev)
        self.table = torch.from_numpy(host["table"]).to(dev)
        self.seq = torch.from_numpy(host["seq"]).to(dev)
        self.prompt = torch.from_numpy(host["prompt"]).to(dev)
        self.cache = bk.PagedCache(self.k, self.v, self.table, self.seq, self.prompt)

    def save(self):
        torch.cuda.synchronize()
        return {"k": [t.view(torch.int16).cpu().numpy().copy() for t in self.k],
                "v": [t.view(torch.int16).cpu().numpy().copy() for t in self.v],
                "beacons": self.beacons.cpu().numpy().copy(),
                "counts": self.counts.cpu().numpy().copy(),
                "pos": self.pos.cpu().numpy().copy(),
                "pass_idx": self.pass_idx.cpu().numpy().copy(),
                "table": self.table.cpu().numpy().copy(),
                "seq": self.seq.cpu().numpy().copy(),
                "prompt": self.prompt.cpu().numpy().copy()}


def initial_state():
    batch = synth.make_batch(WL)
    HC = WL.n_head_caches
    return {"k": [synth.bits(t).view(np.int16).copy() for t in batch.k_pools],
            "v": [synth.bits(t).view(np.int16).copy() for t in batch.v_pools],
            "beacons": batch.beacons.numpy().copy(), "counts": batch.counts.numpy().copy(),
            "pos": np.tile(np.arange(WL.seq_len, dtype=np.int32), (HC, 1)),
            "pass_idx": np.zeros(WL.n_requests, np.int32),
            "table": batch.block_table.numpy().copy(), "seq": batch.seq_len.numpy().copy(),
            "prompt": batch.prompt_len.numpy().copy()}


def step(st, i, selector):
    """Pass i of the loop: append the tokens decoded since the last pass, then
    evict back to the budget."""
    B, W, R, H = WL.budget, WL.window, WL.n_requests, WL.n_kv_heads
    tail = st.table[:, B // 16:(B + W) // 16].long()
    for layer in range(WL.n_layers):
        fk, fv = synth.fresh_tail(WL, layer, i, "cpu")          # [R, H, W, d]
        shp = (R, H, W // 16, 16, WL.head_dim)
        st.k[layer][tail] = fk.reshape(shp).permute(0, 2, 1, 3, 4).cuda()
        st.v[layer][tail] = fv.reshape(shp).permute(0, 2, 1, 3, 4).cuda()
    st.pos[:, B:B + W] = WL.seq_len + i * W + torch.arange(W, dtype=torch.int32).cuda()
    status = torch.zeros(1, dtype=torch.int32).cuda()
    if selector == "beacon":
        g = torch.Generator().manual_seed(5000 + i)
        q = torch.randn(WL.n_head_caches, WL.steps, WL.group, WL.head_dim, generator=g)
        bk.bkv_evict_pass(st.cache, bk.BKV_SELECT_BEACON, B, queries=q.to(torch.bfloat16).cuda(),
                          beacons=st.beacons, counts=st.counts, pos_ids=st.pos, status=status)
    else:
        rid = torch.arange(40, 40 + R, dtype=torch.int64).cuda()
        bk.bkv_evict_pass(st.cache, bk.BKV_SELECT_RANDOM, B, seed=77, request_ids=rid,
                          pass_idx=st.pass_idx, pos_ids=st.pos, status=status)
        st.pass_idx += 1


@pytest.mark.parametrize("selector", ["beacon", "random"])
def test_resume_from_a_saved_state_matches_a_straight_run(selector):
    print(f"[case] resume {selector}: {2 * M} passes straight vs {M} + save/restore + {M}",
          flush=True)
    h0 = initial_state()
    straight = State(h0)
    for i in range(2 * M):
        step(straight, i, selector)
    end_straight = straight.save()
    first = State(h0)
    for i in range(M):
        step(first, i, selector)
    saved = first.save()
    del first
    resumed = State(saved)              # new device tensors from the host copy
    for i in range(M, 2 * M):
        step(resumed, i, selector)
    end_resumed = resumed.save()
    for key in State.FIELDS:
        a, b = end_straight[key], end_resumed[key]
        a = a if isinstance(a, list) else [a]
        b = b if isinstance(b, list) else [b]
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (selector, key)
    # the loop did evict: positions past the prompt are no longer 0..B-1
    assert not np.array_equal(end_straight["pos"][:, :WL.budget],
                              h0["pos"][:, :WL.budget]), "nothing was compacted"
    if selector == "beacon":
        assert not np.array_equal(end_straight["counts"], h0["counts"])

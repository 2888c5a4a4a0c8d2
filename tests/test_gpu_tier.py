"""GPU parity of the HBM / host expert tier: the layer read through the
expert table, with every routed expert in pinned host memory or some of them
in HBM slots after a repin, equals moe_layer_forward on the same weights in
HBM bit for bit, and the oracle within the layer tolerance.  The selection
counts equal the routing's own.  A decode-width layer (hidden 6144,
inter 2048, int4) with 16 routed experts keeps the host copy small."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DevLayer, assert_close
from test_gpu_layer import forward, reference

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


def pinned_copy(w):
    return synth.DeviceWeights(*[getattr(w, f).cpu().pin_memory() for f in
                                 ("gate", "up", "down", "gate_s", "up_s", "down_s")])


def tiered(m, L, tier, T):
    wl = L.wl
    sh = m.shape_of(wl)
    dev = L.x.device
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    ws = m.workspace(m.moe_workspace_bytes(sh, T, m.MOE_PATH_GEMV), dev)
    m.moe_layer_forward_tiered(sh, L.x[:T], L.gate_w, L.bias, tier, L.shared, y, ws, idx, w)
    torch.cuda.synchronize()
    return y, idx.cpu().numpy(), w.cpu().numpy()


@pytest.fixture(scope="module")
def layer(dev):
    wl = synth.workload("decode_int4", n_experts=16, n_group=4, topk_group=2, top_k=4, T=8)
    L = DevLayer(wl, dev)
    return L, pinned_copy(L.routed)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_all_experts_on_the_host(m, layer, T):
    L, host = layer
    tier = m.Tier(m.shape_of(L.wl), host, 4)
    try:
        print("tier parity: all on host, T=%d" % T, flush=True)
        y, idx, w = tiered(m, L, tier, T)
        y0, idx0, w0 = forward(m, L, T)
        assert np.array_equal(idx, idx0) and np.array_equal(w, w0)
        assert torch.equal(y, y0)
        counts = tier.counts()
        assert counts == list(np.bincount(idx.ravel(), minlength=L.wl.n_experts))
        y_ref, idx_ref, _ = reference(L, T)
        assert np.array_equal(idx, idx_ref)
        assert_close(y.cpu().numpy(), y_ref)
    finally:
        tier.close()


def test_repin_moves_the_hot_experts(m, layer):
    L, host = layer
    E, C = L.wl.n_experts, 5
    tier = m.Tier(m.shape_of(L.wl), host, C)
    try:
        y0, _, _ = forward(m, L, 8)
        for step in range(3):
            print("tier parity: repin round %d" % step, flush=True)
            yt, idx, _ = tiered(m, L, tier, 8)
            assert torch.equal(yt, y0)
            heat = tier.counts()
            before = tier.resident()
            n_exp, after_exp = m.moe_tier_plan(heat, C, before)
            n = tier.repin()
            assert n == n_exp and tier.resident() == after_exp
            assert tier.counts() == [h >> 1 for h in heat]
        assert sum(s >= 0 for s in tier.resident()) == C   # 32 selections a round fill every slot
        for T in (1, 8):
            yt, _, _ = tiered(m, L, tier, T)
            y0, _, _ = forward(m, L, T)
            assert torch.equal(yt, y0)
    finally:
        tier.close()


def test_repin_on_two_streams(m, layer):
    """Two repins back to back on different streams: the second reads the
    heat the first one halved and uploaded, and the results stay exact."""
    L, host = layer
    tier = m.Tier(m.shape_of(L.wl), host, 5)
    try:
        print("tier parity: repins on two streams", flush=True)
        y0, _, _ = forward(m, L, 8)
        yt, _, _ = tiered(m, L, tier, 8)
        assert torch.equal(yt, y0)
        heat = np.array(tier.counts(), dtype=np.uint32)
        assert heat.sum() > 0
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        tier.repin(stream=a)
        tier.repin(stream=b)
        torch.cuda.synchronize()
        assert tier.counts() == list(heat >> 2)
        yt, _, _ = tiered(m, L, tier, 8)
        assert torch.equal(yt, y0)
    finally:
        tier.close()


@pytest.mark.parametrize("T", [1, 5])
def test_tiered_top_p_and_accumulate(m, layer, dev, T):
    """adaptive top-p and MOE_ACCUMULATE through the table: equal to the HBM layer"""
    L, host = layer
    sh = m.shape_of(L.wl, top_p=0.7)
    tier = m.Tier(sh, host, 6)
    try:
        ws = m.workspace(m.moe_workspace_bytes(sh, T, m.MOE_PATH_GEMV), dev)
        y0 = torch.randn((T, L.wl.hidden), dtype=torch.float32, device=dev)
        ya, yb = y0.clone(), y0.clone()
        for rnd in range(2):
            print("tier parity: top-p 0.7, accumulate, T=%d, round %d" % (T, rnd), flush=True)
            m.moe_layer_forward_tiered(sh, L.x[:T], L.gate_w, L.bias, tier, L.shared, ya, ws,
                                       flags=m.MOE_ACCUMULATE)
            m.moe_layer_forward(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, yb, ws,
                                flags=m.MOE_PATH_GEMV | m.MOE_ACCUMULATE)
            torch.cuda.synchronize()
            assert torch.equal(ya, yb)
            tier.repin()
    finally:
        tier.close()


def test_prefetch_keeps_results_and_fills_the_ring(m, layer, dev):
    """prefetched experts are read from their prefetch slots, results unchanged;
    the ring holds min(16, E) experts; a repin that pins one frees its slot"""
    L, host = layer
    E = L.wl.n_experts
    tier = m.Tier(m.shape_of(L.wl), host, 2)
    try:
        y0, idx0, _ = forward(m, L, 4)
        side = torch.cuda.Stream()
        print("tier prefetch: the routed experts of 4 tokens", flush=True)
        want = list(dict.fromkeys(int(e) for e in idx0.ravel()))
        with torch.cuda.stream(side):
            n = tier.prefetch(want, stream=side)
        side.synchronize()
        assert n == len(want)
        res = tier.resident()
        assert all(res[e] == -2 for e in want) and sum(r == -2 for r in res) == len(want)
        yt, idx, _ = tiered(m, L, tier, 4)
        assert torch.equal(yt, y0) and np.array_equal(idx, idx0)
        assert tier.prefetch(want) == 0          # already there
        print("tier prefetch: every expert, the ring keeps 16", flush=True)
        n = tier.prefetch(list(range(E)) * 2)
        torch.cuda.synchronize()
        assert n == min(16, E) - len(want) or n == min(16, E)
        assert sum(r == -2 for r in tier.resident()) == min(16, E)
        yt, _, _ = tiered(m, L, tier, 4)
        assert torch.equal(yt, y0)
        tier.repin()
        torch.cuda.synchronize()
        res = tier.resident()
        assert sum(r >= 0 for r in res) == 2 and sum(r == -2 for r in res) == min(16, E) - 2
        yt, _, _ = tiered(m, L, tier, 4)
        assert torch.equal(yt, y0)
    finally:
        tier.close()


def test_tier_argument_errors(m, layer, dev):
    L, host = layer
    sh = m.shape_of(L.wl)
    with pytest.raises(ValueError):
        m.Tier(sh, L.routed, 2)                       # device tensors, not pinned host memory
    with pytest.raises(m.MoeError):
        m.Tier(sh, host, L.wl.n_experts + 1)          # more slots than experts
    tiny = synth.workload("tiny")
    Lt = DevLayer(tiny, dev)
    with pytest.raises(m.MoeError):
        m.Tier(m.shape_of(tiny), pinned_copy(Lt.routed), 2)   # row widths without the table kernels
    tier = m.Tier(sh, host, 2)
    try:
        ws = m.workspace(m.moe_workspace_bytes(sh, 9, m.MOE_PATH_GEMV), dev)
        y = torch.empty((9, L.wl.hidden), dtype=torch.float32, device=dev)
        x9 = torch.zeros((9, L.wl.hidden), dtype=torch.float32, device=dev)
        with pytest.raises(m.MoeError):
            m.moe_layer_forward_tiered(sh, x9, L.gate_w, L.bias, tier, L.shared, y, ws)   # T > 8
    finally:
        tier.close()

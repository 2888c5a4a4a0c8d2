"""Workspaces need no initial contents: every path run on a workspace filled
with 0xFF bytes (NaN as fp32, -1 as int32) gives the same results, bit for
bit, as on a zero-filled one.  A kernel that read a workspace word before
writing it (a plan entry, a count, a staged row) would see different values
in the two runs.  Covered: the one-token and batch GEMV paths (also with
adaptive top-p, whose dropped pairs are staged and never used), the grouped
path, a two-layer decode stack, the tiered layer, the router, the
permutation, the single-expert call and the draft acceptance."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DevLayer, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


def ws_pair(n, dev):
    a = torch.zeros(max(int(n), 1), dtype=torch.uint8, device=dev)
    b = torch.full((max(int(n), 1),), 0xFF, dtype=torch.uint8, device=dev)
    return a, b


def layer_run(m, L, T, flags, ws, top_p=None):
    wl = L.wl
    sh = m.shape_of(wl, top_p=top_p)
    dev = L.x.device
    y = torch.full((T, wl.hidden), 7.0, dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    m.moe_layer_forward(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, y, ws, idx, w, flags=flags)
    torch.cuda.synchronize()
    return y, idx, w


def same(a, b):
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.fixture(scope="module")
def decode(dev):
    return DevLayer(synth.workload("decode_int4"), dev, T=100)


@pytest.mark.parametrize("T,flags,top_p", [(1, 1, None), (5, 1, None), (1, 1, 0.6), (5, 1, 0.6),
                                           (100, 2, None), (100, 2, 0.6)])
def test_layer_paths(m, decode, T, flags, top_p):
    print("workspace fill: decode_int4 T=%d path=%d top_p=%s" % (T, flags, top_p), flush=True)
    sh = m.shape_of(decode.wl, top_p=top_p)
    z, f = ws_pair(m.moe_workspace_bytes(sh, T, flags), decode.x.device)
    a = layer_run(m, decode, T, flags, z, top_p)
    b = layer_run(m, decode, T, flags, f, top_p)
    same(a, b)
    assert torch.isfinite(a[0]).all()


def test_stack_two_layers(m, dev):
    wl = synth.workload("stack_int2", layers=2)
    print("workspace fill: 2-layer int2 stack", flush=True)
    hosts, layers = synth.device_stack(wl, dev)
    arr = m.layers(layers)
    sh = m.shape_of(wl)
    x0 = to_dev(hosts[0].x, dev)
    z, f = ws_pair(m.moe_stack_workspace_bytes(sh, 1), dev)
    outs = []
    for ws in (z, f):
        x = x0.clone()
        idx = torch.empty((2, 1, wl.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((2, 1, wl.top_k), dtype=torch.float32, device=dev)
        m.moe_stack_forward(sh, x, arr, 1e-6, ws, idx, w)
        torch.cuda.synchronize()
        outs.append((x, idx, w))
    same(*outs)


def test_tiered_layer(m, dev):
    wl = synth.workload("decode_int4", n_experts=16, n_group=4, topk_group=2, top_k=4, T=8)
    L = DevLayer(wl, dev)
    host = synth.DeviceWeights(*[getattr(L.routed, f).cpu().pin_memory() for f in
                                 ("gate", "up", "down", "gate_s", "up_s", "down_s")])
    sh = m.shape_of(wl)
    tier = m.Tier(sh, host, 4)
    try:
        for T in (1, 3):
            print("workspace fill: tiered layer T=%d" % T, flush=True)
            z, f = ws_pair(m.moe_workspace_bytes(sh, T, m.MOE_PATH_GEMV), dev)
            outs = []
            for ws in (z, f):
                y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
                idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
                w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
                m.moe_layer_forward_tiered(sh, L.x[:T], L.gate_w, L.bias, tier, L.shared, y, ws, idx, w)
                torch.cuda.synchronize()
                outs.append((y, idx, w))
            same(*outs)
    finally:
        tier.close()


def test_route_permute_expert_and_accept(m, dev):
    wl = synth.workload("prefill_int4", T=300)
    L = DevLayer(wl, dev)
    sh = m.shape_of(wl)
    T = 300
    print("workspace fill: route, permute, expert_ffn, mtp_accept", flush=True)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((m.moe_route_workspace_bytes(sh, T),), fill, dtype=torch.uint8, device=dev)
        idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
        m.moe_route(sh, L.x, L.gate_w, L.bias, idx, w, ws)
        pws = torch.full((m.moe_permute_workspace_bytes(T, wl.top_k, wl.n_experts),), fill, dtype=torch.uint8,
                         device=dev)
        perm = torch.empty(T * wl.top_k, dtype=torch.int32, device=dev)
        off = torch.empty(wl.n_experts + 1, dtype=torch.int32, device=dev)
        inv = torch.empty(T * wl.top_k, dtype=torch.int32, device=dev)
        m.moe_permute(idx, wl.n_experts, perm, off, inv, pws)
        q = torch.empty((3, wl.hidden), dtype=torch.int8, device=dev)
        d = torch.empty((3, wl.hidden // 32), dtype=torch.float32, device=dev)
        m.moe_quant_act(L.x[:3], q, d)
        ews = torch.full((m.moe_workspace_bytes(sh, 3, m.MOE_PATH_GEMV),), fill, dtype=torch.uint8, device=dev)
        y = torch.empty((3, wl.hidden), dtype=torch.float32, device=dev)
        m.moe_expert_ffn(sh, L.routed, 5, q, d, y, ews)
        dr, p, qq, u = synth.mtp_inputs(4, 3, 2, 5000, 0.7)
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
        n = torch.empty(3, dtype=torch.int32, device=dev)
        nx = torch.empty(3, dtype=torch.int32, device=dev)
        aws = torch.full((m.moe_mtp_accept_workspace_bytes(3, 2, 5000),), fill, dtype=torch.uint8, device=dev)
        m.moe_mtp_accept(t(dr, np.int32), t(p, np.float32), t(qq, np.float32), 0.7, t(u, np.float64), n, nx, aws)
        torch.cuda.synchronize()
        outs.append((idx, w, perm, off, inv, y, n, nx))
    same(*outs)

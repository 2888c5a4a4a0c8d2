"""GPU parity of the whole MoE layer (and the single-expert entry point)
against the CPU oracle, through the C ABI.  Expert indices are bit-exact;
float outputs are held to max-abs error <= 1e-3 x max|ref|."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DevLayer, assert_close, dev_expert, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


def forward(m, L, T=None, flags=0, y=None, rsf=None):
    wl = L.wl
    T = L.x.shape[0] if T is None else T
    sh = m.shape_of(wl, rsf=rsf)
    dev = L.x.device
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev) if y is None else y
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    ws = m.workspace(m.moe_workspace_bytes(sh, T, flags), dev)
    m.moe_layer_forward(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, y, ws, idx, w, flags=flags)
    torch.cuda.synchronize()
    return y, idx.cpu().numpy(), w.cpu().numpy()


def reference(L, T=None, rsf=None):
    wl, H = L.wl, L.host
    T = H.x.shape[0] if T is None else T
    sh = oracle.shape_of(wl, rsf=rsf)
    idx, _ = oracle.route(sh, H.x[:T], H.gate_w, H.bias)
    return oracle.layer_forward(sh, H.x[:T], H.gate_w, H.bias, oracle.layer_experts(H, idx), H.shared)


def check(m, L, T=None, flags=0):
    y, idx, w = forward(m, L, T, flags)
    y_ref, idx_ref, w_ref = reference(L, T)
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6)
    return assert_close(y.cpu().numpy(), y_ref)


# ---------------------------------------------------------------- tiny layer
@pytest.mark.parametrize("wbits", [4, 8, 2])
def test_tiny_layer(dev, m, wbits):
    L = DevLayer(synth.workload("tiny", wbits=wbits), dev)
    for T in (8, 1, 3, 5):
        check(m, L, T)


def test_tiny_layer_no_shared(dev, m):
    L = DevLayer(synth.workload("tiny", n_shared=0), dev)
    check(m, L)


def test_tiny_layer_chunked_tokens(dev, m):
    # more tokens than one batch-union chunk: the GEMV path runs in chunks of 8
    wl = synth.workload("tiny", T=21)
    L = DevLayer(wl, dev)
    assert m.moe_layer_stage_count(m.shape_of(wl), 21, m.MOE_PATH_GEMV) == 2 + 3 * 3
    check(m, L, flags=m.MOE_PATH_GEMV)


# ---------------------------------------------------------------- full-size layers
def test_decode_int4_full(dev, m):
    L = DevLayer(synth.workload("decode_int4"), dev)
    rel = check(m, L)
    print("decode_int4: max rel err %.3g" % rel)


def test_decode_int4_other_tokens(dev, m):
    # a few more seeds of the decode token through the same weights
    wl = synth.workload("decode_int4")
    L = DevLayer(wl, dev)
    for s in (1, 2, 3):
        xs = synth.host_normals(s, synth.stream_id(0, synth.X), wl.hidden, 1.0).reshape(1, -1)
        L.host.x = xs
        L.x = to_dev(xs, dev)
        check(m, L)


def test_verify_int8_full(dev, m):
    L = DevLayer(synth.workload("verify_int8"), dev)
    rel = check(m, L)
    print("verify_int8: max rel err %.3g" % rel)


@pytest.mark.parametrize("name,wbits,T", [("decode_int4", 4, 2), ("decode_int4", 4, 5), ("decode_int4", 4, 8),
                                          ("stack_int2", 2, 6), ("verify_int8", 8, 7)])
def test_verify_batches_full_size(dev, m, name, wbits, T):
    """MTP verify batches (1 + drafts) at the full shapes: one batch-union
    chunk whatever T (the down kernel stages the pairs in slot batches when
    they exceed its LDS), the gate/up and down kernels at the exact token
    count; every token compared with the oracle."""
    wl = synth.workload(name, T=T)
    sh = m.shape_of(wl)
    assert m.moe_layer_stage_count(sh, T, m.MOE_PATH_GEMV) == 4   # router, plan, gate/up, down
    print("verify batch: %s T=%d" % (name, T), flush=True)
    L = DevLayer(wl, dev, layer=3 if wl.layers > 1 else 0)
    rel = check(m, L)
    print("verify batch %s T=%d: max rel err %.3g" % (name, T, rel))


def test_stack_int2_layer(dev, m):
    L = DevLayer(synth.workload("stack_int2"), dev, layer=5)
    check(m, L)


# ---------------------------------------------------------------- semantics
def test_accumulate_flag(dev, m):
    L = DevLayer(synth.workload("tiny"), dev)
    y0 = torch.randn((8, 256), dtype=torch.float32, device=dev)
    y_plain, _, _ = forward(m, L)
    y_acc, _, _ = forward(m, L, flags=m.MOE_ACCUMULATE, y=y0.clone())
    assert torch.equal(y_acc, y0 + y_plain)


def test_deterministic(dev, m):
    L = DevLayer(synth.workload("verify_int8"), dev)
    a, ia, wa = forward(m, L)
    b, ib, wb = forward(m, L)
    assert torch.equal(a, b) and np.array_equal(ia, ib) and np.array_equal(wa, wb)


def test_stages_one_by_one(dev, m):
    wl = synth.workload("decode_int4")
    L = DevLayer(wl, dev)
    sh = m.shape_of(wl)
    y_full, _, _ = forward(m, L)
    n = m.moe_layer_stage_count(sh, 1)
    ws = m.workspace(m.moe_workspace_bytes(sh, 1), dev)
    y = torch.empty_like(y_full)
    for s in range(n):
        m.moe_layer_forward(sh, L.x, L.gate_w, L.bias, L.routed, L.shared, y, ws, flags=m.MOE_STAGE(s))
    torch.cuda.synchronize()
    assert torch.equal(y, y_full)


def test_rsf_zero_is_shared_expert(dev, m):
    wl = synth.workload("tiny")
    L = DevLayer(wl, dev)
    y0, _, _ = forward(m, L, rsf=0.0)
    q, d = oracle.quant_act(L.host.x)
    ysh = oracle.expert_ffn(oracle.shape_of(wl), L.host.shared, q, d)
    assert_close(y0.cpu().numpy(), ysh)


# ---------------------------------------------------------------- single expert
@pytest.mark.parametrize("name,T", [("tiny", 8), ("decode_int4", 1), ("verify_int8", 3), ("tiny", 13)])
def test_expert_ffn(dev, m, name, T):
    wl = synth.workload(name)
    H = synth.HostLayer(wl, T=T)
    e = 3
    ex = H.expert(e)
    sh = m.shape_of(wl)
    w = dev_expert(synth.HostExpert(*[getattr(ex, f)[None] for f in
                                      ("gate", "up", "down", "gate_s", "up_s", "down_s")]), dev)
    q, d = oracle.quant_act(H.x)
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    ws = m.workspace(m.moe_workspace_bytes(sh, T), dev)
    shape1 = m.shape(wl.hidden, wl.inter, 1, 1, 1, 1, 0, wl.wbits, 1.0)
    m.moe_expert_ffn(shape1, w, 0, to_dev(q, dev), to_dev(d, dev), y, ws)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.expert_ffn(oracle.shape_of(wl), ex, q, d))


# ---------------------------------------------------------------- graph replay
@pytest.mark.parametrize("name,T,path", [("decode_int4", 1, "gemv"), ("verify_int8", 8, "gemv"),
                                         ("tiny", 100, "grouped")])
def test_layer_graph_replay(dev, m, name, T, path):
    """A captured layer call replays the eager result exactly, on several
    inputs in turn, with eager work and synchronisations between replays."""
    wl = synth.workload(name)
    L = DevLayer(wl, dev, T=T)
    flags = m.MOE_PATH_GROUPED if path == "grouped" else m.MOE_PATH_GEMV
    sh = m.shape_of(wl)
    ws = m.workspace(m.moe_workspace_bytes(sh, T, flags), dev)
    xs = [L.x] + [torch.from_numpy(synth.host_normals(s, synth.stream_id(0, synth.X), T * wl.hidden, 1.0)
                                   .reshape(T, wl.hidden)).to(dev) for s in (21, 22)]
    outs = []
    for x in xs:
        y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
        idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
        m.moe_layer_forward(sh, x, L.gate_w, L.bias, L.routed, L.shared, y, ws, idx, w, flags=flags)
        outs.append((y, idx, w))
    torch.cuda.synchronize()
    x_s = torch.empty_like(L.x)
    y_s = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    i_s = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    w_s = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        m.moe_layer_forward(sh, x_s, L.gate_w, L.bias, L.routed, L.shared, y_s, ws, i_s, w_s, flags=flags)
    torch.cuda.synchronize()
    for rep in range(2):
        for x, (y, idx, w) in zip(xs, outs):
            x_s.copy_(x)
            g.replay()
            torch.cuda.synchronize()
            _ = (x * 2).sum().item()
            assert torch.equal(y_s, y) and torch.equal(i_s, idx) and torch.equal(w_s, w), \
                "replay %d differs from the eager call" % rep


# ---------------------------------------------------------------- adaptive expert top-p
@pytest.mark.parametrize("name,T,p", [("tiny", 8, 0.5), ("tiny", 5, 0.8), ("decode_int4", 1, 0.7),
                                      ("decode_int4", 1, 0.3), ("verify_int8", 3, 0.7), ("tiny", 20, 0.6)])
def test_layer_top_p(dev, m, name, T, p):
    """Top-p keeps a per-token prefix of each selection: indices and weights
    match the oracle's (dropped slots -1 / 0), the output within tolerance.
    T = 20 runs on the GEMV path in chunks (AUTO does not take the grouped
    kernels with top-p on)."""
    wl = synth.workload(name, top_p=p)
    L = DevLayer(wl, dev, T=T)
    rel = check(m, L, T)
    idx, _ = oracle.route(oracle.shape_of(wl), L.host.x[:T], L.host.gate_w, L.host.bias)
    print("%s T=%d p=%.1f: experts kept per token %.2f, max rel err %.3g" %
          (name, T, p, (idx >= 0).sum(1).mean(), rel))


# ---------------------------------------------------------------- largest shapes the ABI takes
@pytest.mark.parametrize("E,G,tg,k,T,path", [(512, 8, 4, 32, 1, "gemv"), (512, 8, 4, 32, 8, "gemv"),
                                             (512, 64, 8, 32, 5, "gemv"), (512, 64, 8, 32, 40, "grouped"),
                                             (512, 8, 4, 32, 100, "grouped")])
def test_largest_routing_shapes(dev, m, E, G, tg, k, T, path):
    """E = 512 experts, up to G = 64 groups, top_k = 32: the plan holds up to
    8 * 32 + 1 slots; both paths match the oracle."""
    wl = synth.workload("tiny", n_experts=E, n_group=G, topk_group=tg, top_k=k)
    L = DevLayer(wl, dev, T=T)
    flags = m.MOE_PATH_GROUPED if path == "grouped" else m.MOE_PATH_GEMV
    rel = check(m, L, T, flags)
    print("E=%d G=%d tg=%d k=%d T=%d %s: max rel err %.3g" % (E, G, tg, k, T, path, rel))

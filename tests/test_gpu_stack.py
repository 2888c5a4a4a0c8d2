"""GPU parity of the 75-layer int2 decode stack x <- x + MoE_l(RMSNorm(x))
(moe_stack_forward) against the CPU oracle.

The oracle runs the whole chain for one token: per layer, RMSNorm with unit
weight and eps 1e-6, the layer forward, and the fp32 residual add.  Two
checks follow the method's own validation by teacher forcing:
  - teacher forced: every layer on the GPU gets the oracle's normalised
    input; its routing must be bit-exact and its output within tolerance;
  - free running: the GPU runs the whole stack from the same token; every
    layer's routing must match the oracle chain's, and the final residual
    must be within tolerance of the oracle's.
A graph capture of the stack call is replayed on several tokens and checked
against eager runs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


@pytest.fixture(scope="module")
def stack(dev):
    wl = synth.workload("stack_int2")
    print("stack: generating %d layers in HBM" % wl.layers, flush=True)
    hosts, layers = synth.device_stack(wl, dev)
    torch.cuda.synchronize()
    return wl, hosts, layers


@pytest.fixture(scope="module")
def chain(stack):
    """The oracle's chain for the stack's token: per layer the normalised
    input, the routing (with margins) and the residual after the layer."""
    wl, hosts, _ = stack
    sh = oracle.shape_of(wl)
    ones = np.ones(wl.hidden, np.float32)
    x = hosts[0].x.copy()
    out = []
    print("stack: oracle chain over %d layers" % wl.layers, flush=True)
    for l, H in enumerate(hosts):
        n = oracle.rmsnorm(x, ones, EPS)
        idx, w, marg = oracle.route(sh, n, H.gate_w, H.bias, margins=True)
        y, _, _ = oracle.layer_forward(sh, n, H.gate_w, H.bias, oracle.layer_experts(H, idx), H.shared)
        H._experts = {}
        x = (x + y).astype(np.float32)
        out.append(dict(n=n, idx=idx, w=w, margins=marg, y=y, x=x.copy()))
    return out


def test_stack_teacher_forced(dev, m, stack, chain):
    wl, hosts, layers = stack
    sh = m.shape_of(wl)
    ws = m.workspace(m.moe_workspace_bytes(sh, 1), dev)
    idx = torch.empty((1, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((1, wl.top_k), dtype=torch.float32, device=dev)
    worst = 0.0
    y = torch.empty((1, wl.hidden), dtype=torch.float32, device=dev)
    for l, (L, ref) in enumerate(zip(layers, chain)):
        n = to_dev(ref["n"], dev)
        m.moe_layer_forward(sh, n, L.gate_w, L.bias, L.routed, L.shared, y, ws, idx, w)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref["idx"]), "layer %d routing" % l
        np.testing.assert_allclose(w.cpu().numpy(), ref["w"], rtol=1e-6)
        worst = max(worst, assert_close(y.cpu().numpy(), ref["y"], what="layer %d output" % l))
    print("teacher forced: 75 layers, routing bit-exact, max rel err %.3g" % worst)


def test_rmsnorm_along_the_chain(dev, m, stack, chain):
    wl, hosts, layers = stack
    out = torch.empty((1, wl.hidden), dtype=torch.float32, device=dev)
    for l in (0, 1, 37, 74):
        x = to_dev(chain[l - 1]["x"] if l else hosts[0].x, dev)
        m.moe_rmsnorm(x, layers[l].norm_g, EPS, out)
        torch.cuda.synchronize()
        np.testing.assert_allclose(out.cpu().numpy(), chain[l]["n"], rtol=2e-7, atol=0)


def run_stack(m, wl, layers, x0, dev):
    sh = m.shape_of(wl)
    arr = m.layers(layers)
    ws = m.workspace(m.moe_stack_workspace_bytes(sh, 1), dev)
    x = x0.clone()
    idx = torch.empty((wl.layers, 1, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((wl.layers, 1, wl.top_k), dtype=torch.float32, device=dev)
    m.moe_stack_forward(sh, x, arr, EPS, ws, idx, w)
    torch.cuda.synchronize()
    return x, idx.cpu().numpy(), w.cpu().numpy()


def test_stack_free_running(dev, m, stack, chain):
    wl, hosts, layers = stack
    x, idx, w = run_stack(m, wl, layers, to_dev(hosts[0].x, dev), dev)
    flips = [l for l in range(wl.layers) if not np.array_equal(idx[l], chain[l]["idx"])]
    if flips:
        l = flips[0]
        pytest.fail("free-running routing departs from the oracle at layer %d (oracle margins %s)" %
                    (l, chain[l]["margins"].tolist()))
    rel = assert_close(x.cpu().numpy(), chain[-1]["x"], what="final residual")
    print("free running: 75 layers, routing identical, final residual max rel err %.3g" % rel)


def test_stack_graph_replay(dev, m, stack):
    wl, hosts, layers = stack
    sh = m.shape_of(wl)
    arr = m.layers(layers)
    ws = m.workspace(m.moe_stack_workspace_bytes(sh, 1), dev)
    tokens = [torch.from_numpy(synth.host_normals(s, synth.stream_id(0, synth.X), wl.hidden, 1.0)
                               .reshape(1, -1)).to(dev) for s in (11, 12, 13)]
    eager = []
    for t in tokens:
        x = t.clone()
        m.moe_stack_forward(sh, x, arr, EPS, ws)
        eager.append(x)
    torch.cuda.synchronize()
    x_static = torch.empty_like(tokens[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        m.moe_stack_forward(sh, x_static, arr, EPS, ws)
    torch.cuda.synchronize()
    for rep in range(2):
        for t, ref in zip(tokens, eager):
            x_static.copy_(t)
            g.replay()
            torch.cuda.synchronize()
            # eager work between replays
            _ = (t * 2).sum().item()
            assert torch.equal(x_static, ref), "graph replay %d differs from the eager stack" % rep


def test_stack_matches_separate_norm_launches(dev, m, stack):
    """The stack's router launch forms each layer's RMSNorm itself; the result
    must equal, bit for bit, RMSNorm launches followed by layer calls that add
    into the residual, through the public entry points."""
    wl, hosts, layers = stack
    sh = m.shape_of(wl)
    n_l = 6
    x0 = to_dev(hosts[0].x, dev)
    x_fused, idx_f, w_f = run_stack(m, wl, layers[:n_l], x0, dev)
    x = x0.clone()
    n = torch.empty_like(x)
    ws = m.workspace(m.moe_workspace_bytes(sh, 1), dev)
    idx = torch.empty((n_l, 1, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((n_l, 1, wl.top_k), dtype=torch.float32, device=dev)
    for l, L in enumerate(layers[:n_l]):
        m.moe_rmsnorm(x, L.norm_g, EPS, n)
        m.moe_layer_forward(sh, n, L.gate_w, L.bias, L.routed, L.shared, x, ws, idx[l], w[l],
                            flags=m.MOE_ACCUMULATE)
    torch.cuda.synchronize()
    assert np.array_equal(idx_f[:n_l], idx.cpu().numpy())
    assert np.array_equal(w_f[:n_l], w.cpu().numpy())
    assert torch.equal(x_fused, x)


def test_stack_stages_one_by_one(dev, m, stack):
    wl, hosts, layers = stack
    sh = m.shape_of(wl)
    arr = m.layers(layers[:1])
    ws = m.workspace(m.moe_stack_workspace_bytes(sh, 1), dev)
    x0 = to_dev(hosts[0].x, dev)
    ref = x0.clone()
    m.moe_stack_forward(sh, ref, arr, EPS, ws)
    n = m.moe_layer_stage_count(sh, 1)
    x = x0.clone()
    for s in range(n):
        m.moe_stack_forward(sh, x, arr, EPS, ws, flags=m.MOE_STAGE(s))
    torch.cuda.synchronize()
    assert torch.equal(x, ref)


@pytest.mark.parametrize("wgs", [1, 8, 32])
def test_stack_lookahead_identical(dev, m, stack, wgs):
    """The router lookahead only prefetches: with it on, every layer's
    routing and the final residual are bit-identical to the stack without
    it, through eager runs and a replayed graph capture."""
    wl, hosts, layers = stack
    sh = m.shape_of(wl)
    x0 = to_dev(hosts[0].x, dev)
    ref, idx_r, w_r = run_stack(m, wl, layers, x0, dev)
    arr = m.layers(layers)
    flags = m.MOE_LOOKAHEAD(wgs)
    ws = m.workspace(m.moe_stack_workspace_bytes(sh, 1, flags), dev)
    assert m.moe_stack_workspace_bytes(sh, 1, flags) > m.moe_stack_workspace_bytes(sh, 1)
    x = x0.clone()
    idx = torch.empty((wl.layers, 1, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((wl.layers, 1, wl.top_k), dtype=torch.float32, device=dev)
    m.moe_stack_forward(sh, x, arr, EPS, ws, idx, w, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx_r)
    assert np.array_equal(w.cpu().numpy(), w_r)
    assert torch.equal(x, ref)
    x_static = x0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        m.moe_stack_forward(sh, x_static, arr, EPS, ws, flags=flags)
    torch.cuda.synchronize()
    for rep in range(2):
        x_static.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        _ = (x0 * 2).sum().item()
        assert torch.equal(x_static, ref), "lookahead graph replay %d" % rep


def test_stack_lookahead_prediction(dev, m, stack, chain):
    """The logits the lookahead predicts with: after a stack call the
    workspace holds those of the last prediction, layer L-1's router on the
    normalised residual before layer L-2.  Their sigmoid must match the
    oracle's router scores on the oracle's RMSNorm of the GPU's own residual
    there (the two norms agree to a few fp32 ulps, hence the tolerance).
    The recall of the prediction (the predicted top-k among the experts the
    next layer then selects) along the oracle chain is printed."""
    wl, hosts, layers = stack
    sh = m.shape_of(wl)
    flags = m.MOE_LOOKAHEAD(8)
    ws = m.workspace(m.moe_stack_workspace_bytes(sh, 1, flags), dev)
    x = to_dev(hosts[0].x, dev)
    m.moe_stack_forward(sh, x, m.layers(layers), EPS, ws, flags=flags)
    torch.cuda.synchronize()
    nb = (4 * wl.hidden + 255) // 256 * 256
    logits = ws[nb:nb + 8 * wl.n_experts].view(torch.float64).cpu().numpy()
    L = wl.layers
    xp, _, _ = run_stack(m, wl, layers[:L - 2], to_dev(hosts[0].x, dev), dev)
    n = oracle.rmsnorm(xp.cpu().numpy(), np.ones(wl.hidden, np.float32), EPS)
    s, _ = oracle.router_scores(sh, n[0], hosts[L - 1].gate_w, hosts[L - 1].bias)
    np.testing.assert_allclose(1.0 / (1.0 + np.exp(-logits)), s, rtol=0, atol=1e-6)
    hits = 0
    for l in range(L - 1):
        pred, _ = oracle.route(sh, chain[l]["n"], hosts[l + 1].gate_w, hosts[l + 1].bias)
        hits += len(set(pred[0].tolist()) & set(chain[l + 1]["idx"][0].tolist()))
    print("lookahead recall along the chain: %.1f%% of %d selections" %
          (100.0 * hits / ((L - 1) * wl.top_k), (L - 1) * wl.top_k))


@pytest.mark.parametrize("H", [8192, 8448])
def test_stack_norm_paths_at_the_width_limit(dev, m, H):
    """The router launch forms RMSNorm(x) itself up to H = 8192; above, the
    stack runs a separate RMSNorm launch.  A 3-layer stack of 2 tokens with
    non-unit norm weights at H = 8192 (fused) and H = 8448 (separate): equal,
    bit for bit, to moe_rmsnorm + moe_layer_forward launches adding into the
    residual, with every layer's routing equal to the oracle chain's and the
    final residual within tolerance of it."""
    import types
    wl = synth.workload("tiny", hidden=H, layers=3, T=2)
    hosts, base = synth.device_stack(wl, dev)
    rng = np.random.default_rng(H)
    gs = [(1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32) for _ in range(wl.layers)]
    layers = [types.SimpleNamespace(gate_w=L.gate_w, bias=L.bias, norm_g=to_dev(g, dev), routed=L.routed,
                                    shared=L.shared) for L, g in zip(base, gs)]
    sh = m.shape_of(wl)
    T = wl.T
    x0 = to_dev(hosts[0].x, dev)
    x = x0.clone()
    idx = torch.empty((wl.layers, T, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((wl.layers, T, wl.top_k), dtype=torch.float32, device=dev)
    ws = m.workspace(m.moe_stack_workspace_bytes(sh, T), dev)
    m.moe_stack_forward(sh, x, m.layers(layers), EPS, ws, idx, w)
    xm = x0.clone()
    n = torch.empty_like(xm)
    lws = m.workspace(m.moe_workspace_bytes(sh, T), dev)
    im = torch.empty_like(idx)
    wm = torch.empty_like(w)
    for l, L in enumerate(layers):
        m.moe_rmsnorm(xm, L.norm_g, EPS, n)
        m.moe_layer_forward(sh, n, L.gate_w, L.bias, L.routed, L.shared, xm, lws, im[l], wm[l],
                            flags=m.MOE_ACCUMULATE)
    torch.cuda.synchronize()
    assert torch.equal(x, xm) and torch.equal(idx, im) and torch.equal(w, wm)
    osh = oracle.shape_of(wl)
    xr = hosts[0].x.copy()
    for l, Hl in enumerate(hosts):
        nr = oracle.rmsnorm(xr, gs[l], EPS)
        ir, _ = oracle.route(osh, nr, Hl.gate_w, Hl.bias)
        assert np.array_equal(idx[l].cpu().numpy(), ir), "layer %d routing" % l
        yr, _, _ = oracle.layer_forward(osh, nr, Hl.gate_w, Hl.bias, oracle.layer_experts(Hl, ir), Hl.shared)
        xr = (xr + yr).astype(np.float32)
    assert_close(x.cpu().numpy(), xr, what="final residual at H=%d" % H)


@pytest.mark.parametrize("top_p", [0.0, 0.7])
def test_stack_lookahead_identical_with_top_p_and_batches(dev, m, stack, top_p):
    """The lookahead fetches every predicted rank whatever the adaptive
    top-p keeps, and is ignored for batches of more than one token: with
    top-p 0.7 on one token, and for a batch of 3 tokens, the first 8 layers
    give bit-identical routing and residuals with and without it."""
    wl, hosts, layers = stack
    sh = m.shape_of(synth.workload("stack_int2", top_p=top_p))
    arr = m.layers(layers[:8])
    for T in (1, 3):
        x0 = torch.from_numpy(np.stack([synth.host_normals(50 + t, synth.stream_id(0, synth.X), wl.hidden, 1.0)
                                        for t in range(T)])).to(dev)
        outs = []
        for flags in (0, m.MOE_LOOKAHEAD(8)):
            ws = m.workspace(m.moe_stack_workspace_bytes(sh, T, flags), dev)
            x = x0.clone()
            idx = torch.empty((8, T, wl.top_k), dtype=torch.int32, device=dev)
            w = torch.empty((8, T, wl.top_k), dtype=torch.float32, device=dev)
            m.moe_stack_forward(sh, x, arr, EPS, ws, idx, w, flags=flags)
            torch.cuda.synchronize()
            outs.append((x, idx, w))
        (xa, ia, wa), (xb, ib, wb) = outs
        assert torch.equal(xa, xb) and torch.equal(ia, ib) and torch.equal(wa, wb), "T=%d top_p=%.1f" % (T, top_p)
        if top_p:
            assert (ia < 0).any(), "top-p dropped no slot"

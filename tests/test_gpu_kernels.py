"""GPU parity of the individual kernels against the CPU oracle, through the
C ABI: bit-exact where the result is integer (codes, block sums, expert
indices, permutation) or fixed by IEEE fp32 division (activation scales)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DevLayer, assert_close, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


# ---------------------------------------------------------------- generator
@pytest.mark.parametrize("wbits", [2, 4, 8])
def test_device_generator_matches_host(dev, wbits):
    wl = synth.workload("tiny", wbits=wbits)
    L = synth.HostLayer(wl, layer=3)
    d = synth.device_weights(wl, 3, 0, wl.n_experts, dev)
    ds = synth.device_weights(wl, 3, wl.n_experts, 1, dev)
    torch.cuda.synchronize()
    for e in (0, 7, wl.n_experts - 1):
        for f in ("gate", "up", "down", "gate_s", "up_s", "down_s"):
            assert np.array_equal(getattr(d, f)[e].cpu().numpy(), getattr(L.expert(e), f)), (e, f)
    for f in ("gate", "down", "up_s"):
        assert np.array_equal(getattr(ds, f)[0].cpu().numpy(), getattr(L.shared, f))


# ---------------------------------------------------------------- quantiser
def special_rows(D):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, D)).astype(np.float32) * np.float32(3.0)
    x[0, :32] = 0.0                                              # zero block
    x[1, :10] = [127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5, -126.5, 4.4999995]  # half-way cases
    x[1, 10:32] = 0.25
    x[2, :32] = np.float32(1e-40) * np.sign(rng.standard_normal(32))   # subnormal scale
    x[3, :32] = np.float32(3e38) * np.sign(rng.standard_normal(32))    # near fp32 max
    x[4, 32:64] = -7.0                                           # constant negative block
    v = np.zeros(32, np.uint32)
    v[0], v[1] = 0x3FA3D70A, 0x3D107D23                          # x/d just below a half-way point
    x[5, 64:96] = v.view(np.float32)
    return x


@pytest.mark.parametrize("T,D", [(1, 32), (3, 6144), (5, 2048), (2048, 6144), (6, 256)])
def test_quant_act_bit_exact(dev, m, T, D):
    rng = np.random.default_rng(T * 7 + D)
    x = (rng.standard_normal((T, D)) * rng.uniform(0.01, 50, (T, 1))).astype(np.float32)
    if T >= 6:
        x[:6] = special_rows(D)
    xd = to_dev(x, dev)
    q = torch.empty((T, D), dtype=torch.int8, device=dev)
    d = torch.empty((T, D // 32), dtype=torch.float32, device=dev)
    m.moe_quant_act(xd, q, d)
    torch.cuda.synchronize()
    q_ref, d_ref = oracle.quant_act(x)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


# ---------------------------------------------------------------- block dots
@pytest.mark.parametrize("wbits,D,rows,T", [(4, 6144, 40, 2), (4, 2048, 33, 1), (8, 6144, 17, 3),
                                            (8, 256, 64, 8), (2, 6144, 24, 1), (2, 128, 80, 5)])
def test_block_dots_bit_exact(dev, m, wbits, D, rows, T):
    codes = (synth.host_int8(5, 77, rows * D).view(np.uint8) if wbits == 8
             else synth.host_bytes(5, 77, rows * D * wbits // 8)).reshape(rows, -1)
    x = synth.host_normals(5, 78, T * D, 1.0).reshape(T, D)
    q, _ = oracle.quant_act(x)
    out = torch.empty((T, rows, D // 32), dtype=torch.int32, device=dev)
    m.moe_block_dots(wbits, to_dev(codes, dev), D, to_dev(q, dev), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.block_dots(wbits, codes, D, q))


@pytest.mark.parametrize("wbits,byte,bound", [(8, 0x81, 516128), (4, 0x88, 32512), (2, 0xAA, 8128)])
def test_block_dots_extremes(dev, m, wbits, byte, bound):
    D = 256
    codes = np.full((2, D * wbits // 8), byte, np.uint8)
    q = np.full((1, D), -127, np.int8)
    out = torch.empty((1, 2, D // 32), dtype=torch.int32, device=dev)
    m.moe_block_dots(wbits, to_dev(codes, dev), D, to_dev(q, dev), out)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == bound)


# ---------------------------------------------------------------- router
def run_route(m, dev, wl, x, gate_w, bias):
    sh = m.shape_of(wl)
    T = x.shape[0]
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    ws = m.workspace(m.moe_route_workspace_bytes(sh, T), dev)
    m.moe_route(sh, to_dev(x, dev), to_dev(gate_w, dev), to_dev(bias, dev), idx, w, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name,T", [("tiny", 8), ("decode_int4", 1), ("decode_int4", 64),
                                    ("prefill_int4", 2048)])
def test_route_bit_exact(dev, m, name, T):
    wl = synth.workload(name)
    L = synth.HostLayer(wl, T=T)
    idx, w = run_route(m, dev, wl, L.x, L.gate_w, L.bias)
    idx_ref, w_ref, margins = oracle.route(oracle.shape_of(wl), L.x, L.gate_w, L.bias, margins=True)
    print("%s T=%d: smallest selection margin %.3g, group margin %.3g" %
          (name, T, margins[:, 0].min(), margins[:, 1].min()))
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6, atol=0)


@pytest.mark.parametrize("E,G,tg,k,H", [(12, 3, 1, 4, 64), (32, 8, 3, 5, 96), (8, 8, 8, 3, 32),
                                        (512, 8, 4, 8, 128), (160, 5, 2, 6, 64), (24, 8, 2, 2, 32),
                                        (1, 1, 1, 1, 32),
                                        # experts per lane 2, 6 and 2 with 16-lane groups; one 64-lane group
                                        (128, 8, 4, 8, 64), (384, 8, 4, 8, 64), (96, 3, 2, 4, 32),
                                        (64, 1, 1, 6, 32)])
def test_route_other_shapes(dev, m, E, G, tg, k, H):
    wl = synth.workload("tiny", n_experts=E, n_group=G, topk_group=tg, top_k=k, hidden=H)
    L = synth.HostLayer(wl, T=37)
    idx, w = run_route(m, dev, wl, L.x, L.gate_w, L.bias)
    idx_ref, w_ref = oracle.route(oracle.shape_of(wl), L.x, L.gate_w, L.bias)
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6)


def test_route_ties_lower_index(dev, m):
    # W = 0: every sigmoid is 1/2; equal biases make exact ties everywhere
    wl = synth.workload("tiny")
    E, H = wl.n_experts, wl.hidden
    x = np.ones((3, H), np.float32)
    W = np.zeros((E, H), np.float32)
    bias = np.zeros(E, np.float32)
    bias[[5, 6, 13]] = 0.25            # groups 1 and 3 lead; ties among the rest
    idx, w = run_route(m, dev, wl, x, W, bias)
    idx_ref, w_ref = oracle.route(oracle.shape_of(wl), x, W, bias)
    assert np.array_equal(idx, idx_ref)
    assert list(idx[0]) == [5, 6, 13, 4]


@pytest.mark.parametrize("name,T", [("tiny", 8), ("decode_int4", 64), ("prefill_int4", 2048)])
@pytest.mark.parametrize("p", [0.3, 0.7, 0.9])
def test_route_top_p_bit_exact(dev, m, name, T, p):
    wl = synth.workload(name, top_p=p)
    L = synth.HostLayer(wl, T=T)
    idx, w = run_route(m, dev, wl, L.x, L.gate_w, L.bias)
    idx_ref, w_ref = oracle.route(oracle.shape_of(wl), L.x, L.gate_w, L.bias)
    kept = (idx_ref >= 0).sum(1)
    print("%s T=%d p=%.1f: experts kept per token %.2f (min %d, max %d)" % (name, T, p, kept.mean(), kept.min(),
                                                                           kept.max()))
    assert 1 <= kept.min() and kept.max() <= wl.top_k
    if p <= 0.7:
        assert kept.min() < wl.top_k                     # the cut drops experts here
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6, atol=0)


# ---------------------------------------------------------------- permutation
@pytest.mark.parametrize("T,k,E,skew", [(2048, 8, 256, True), (2048, 8, 256, False), (3, 8, 256, False),
                                        (1, 1, 16, False), (0, 8, 256, False), (777, 4, 16, True)])
def test_permute_bit_exact(dev, m, T, k, E, skew):
    rng = np.random.default_rng(T + k + E)
    p = rng.dirichlet(np.full(E, 0.05 if skew else 5.0))
    idx = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(T)], np.int32).reshape(T, k)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ws = m.workspace(m.moe_permute_workspace_bytes(T, k, E), dev)
    m.moe_permute(to_dev(idx, dev), E, perm, off, inv, ws)
    torch.cuda.synchronize()
    perm_ref, off_ref, inv_ref = oracle.permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), off_ref)
    assert np.array_equal(perm.cpu().numpy(), perm_ref)
    assert np.array_equal(inv.cpu().numpy(), inv_ref.reshape(-1))


@pytest.mark.parametrize("T,k,E", [(2048, 8, 256), (37, 4, 16)])
def test_permute_with_dropped_slots(dev, m, T, k, E):
    # adaptive top-p leaves a per-token prefix; the dropped slots (-1) get no row
    rng = np.random.default_rng(T + E)
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32).reshape(T, k)
    kept = rng.integers(1, k + 1, T)
    for t in range(T):
        idx[t, kept[t]:] = -1
    perm = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ws = m.workspace(m.moe_permute_workspace_bytes(T, k, E), dev)
    m.moe_permute(to_dev(idx, dev), E, perm, off, inv, ws)
    torch.cuda.synchronize()
    perm_ref, off_ref, inv_ref = oracle.permute(idx, E)
    R = int(off_ref[E])
    assert R == int(kept.sum())
    assert np.array_equal(off.cpu().numpy(), off_ref)
    assert np.array_equal(perm.cpu().numpy()[:R], perm_ref[:R])
    assert np.array_equal(inv.cpu().numpy(), inv_ref.reshape(-1))


# ---------------------------------------------------------------- rmsnorm
@pytest.mark.parametrize("T,H", [(1, 6144), (5, 256), (3, 100)])
def test_rmsnorm(dev, m, T, H):
    rng = np.random.default_rng(H)
    x = (rng.standard_normal((T, H)) * 30).astype(np.float32)
    g = rng.uniform(0.5, 2, H).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    m.moe_rmsnorm(to_dev(x, dev), to_dev(g, dev), 1e-6, out)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), oracle.rmsnorm(x, g, 1e-6), rtol=2e-7, atol=0)

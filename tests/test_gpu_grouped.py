"""GPU parity of the expert-grouped path (MOE_PATH_GROUPED: token permutation
and int8 MFMA grouped GEMMs) against the CPU oracle, through the C ABI.

Expert indices are bit-exact; float outputs are held to max-abs error
<= 1e-3 x max|ref|.  At the full prefill size (2048 tokens, every tile of
every expert the skewed routing loads) the routing and the whole [2048][6144]
output are compared with the oracle element by element, and with the GEMV
path.  At the decode shape, batches of 3, 8, 16 and 64 independent tokens
run on both paths and against the oracle (the two paths are the forced
equivalence of the batch-union GEMV and the grouped GEMM)."""
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


def forward(m, L, flags, T=None, y=None):
    wl = L.wl
    T = L.x.shape[0] if T is None else T
    sh = m.shape_of(wl)
    dev = L.x.device
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev) if y is None else y
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    ws = m.workspace(m.moe_workspace_bytes(sh, T, flags), dev)
    m.moe_layer_forward(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, y, ws, idx, w, flags=flags)
    torch.cuda.synchronize()
    return y, idx.cpu().numpy(), w.cpu().numpy()


def reference(L, rows):
    wl, H = L.wl, L.host
    sh = oracle.shape_of(wl)
    x = H.x[rows]
    idx, _ = oracle.route(sh, x, H.gate_w, H.bias)
    return oracle.layer_forward(sh, x, H.gate_w, H.bias, oracle.layer_experts(H, idx), H.shared)


def check(m, L, T, flags):
    print("grouped parity: %s T=%d wbits=%d" % (L.wl.name, T, L.wl.wbits), flush=True)
    y, idx, w = forward(m, L, flags, T)
    y_ref, idx_ref, w_ref = reference(L, np.arange(T))
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6)
    return assert_close(y.cpu().numpy(), y_ref)


# ---------------------------------------------------------------- tiny layer
@pytest.mark.parametrize("wbits", [4, 8, 2])
def test_tiny_grouped(dev, m, wbits):
    # T=1..200: one tile, several tiles per expert, ragged last tiles
    wl = synth.workload("tiny", wbits=wbits, T=200)
    L = DevLayer(wl, dev)
    for T in (8, 1, 3, 21, 64, 65, 200):
        check(m, L, T, m.MOE_PATH_GROUPED)


def test_tiny_grouped_no_shared(dev, m):
    L = DevLayer(synth.workload("tiny", n_shared=0, T=70), dev)
    check(m, L, 70, m.MOE_PATH_GROUPED)


def test_auto_takes_grouped_above_eight_tokens(dev, m):
    wl = synth.workload("tiny", T=9)
    sh = m.shape_of(wl)
    assert m.moe_layer_stage_count(sh, 9) == 7
    assert m.moe_layer_stage_count(sh, 8) == 1 + 3
    L = DevLayer(wl, dev)
    check(m, L, 9, m.MOE_PATH_AUTO)


def test_grouped_matches_gemv_path(dev, m):
    # the two paths compute the same layer; both within tolerance of the oracle
    L = DevLayer(synth.workload("verify_int8"), dev)
    yg, ig, wg = forward(m, L, m.MOE_PATH_GROUPED)
    yv, iv, wv = forward(m, L, m.MOE_PATH_GEMV)
    assert np.array_equal(ig, iv) and np.array_equal(wg, wv)
    assert_close(yg.cpu().numpy(), yv.cpu().numpy().astype(np.float64), what="grouped vs gemv")
    check(m, L, 3, m.MOE_PATH_GROUPED)


def test_decode_shape_grouped(dev, m):
    L = DevLayer(synth.workload("decode_int4"), dev)
    check(m, L, 1, m.MOE_PATH_GROUPED)


# ---------------------------------------------------------------- semantics
def test_grouped_accumulate_and_determinism(dev, m):
    wl = synth.workload("tiny", T=40)
    L = DevLayer(wl, dev)
    G = m.MOE_PATH_GROUPED
    y0 = torch.randn((40, wl.hidden), dtype=torch.float32, device=dev)
    a, ia, wa = forward(m, L, G)
    b, ib, wb = forward(m, L, G)
    assert torch.equal(a, b) and np.array_equal(ia, ib) and np.array_equal(wa, wb)
    c, _, _ = forward(m, L, G | m.MOE_ACCUMULATE, y=y0.clone())
    assert torch.equal(c, y0 + a)


def test_grouped_stages_one_by_one(dev, m):
    wl = synth.workload("tiny", T=100)
    L = DevLayer(wl, dev)
    G = m.MOE_PATH_GROUPED
    sh = m.shape_of(wl)
    y_full, _, _ = forward(m, L, G)
    n = m.moe_layer_stage_count(sh, 100, G)
    assert n == 7
    ws = m.workspace(m.moe_workspace_bytes(sh, 100, G), dev)
    y = torch.empty_like(y_full)
    for s in range(n):
        m.moe_layer_forward(sh, L.x, L.gate_w, L.bias, L.routed, L.shared, y, ws, flags=G | m.MOE_STAGE(s))
    torch.cuda.synchronize()
    assert torch.equal(y, y_full)


# ---------------------------------------------------------------- full prefill size
@pytest.fixture(scope="module")
def prefill(dev):
    return DevLayer(synth.workload("prefill_int4"), dev)


def test_prefill_routing_full(dev, m, prefill):
    L = prefill
    print("prefill routing: T=2048", flush=True)
    _, idx, w = forward(m, L, m.MOE_PATH_AUTO)
    idx_ref, w_ref = oracle.route(oracle.shape_of(L.wl), L.host.x, L.host.gate_w, L.host.bias)
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6)
    # the skewed bias concentrates the load: some expert takes hundreds of tokens
    assert np.bincount(idx.ravel(), minlength=256).max() > 256


@pytest.mark.timeout(900)
def test_prefill_full_output(dev, m, prefill):
    """Every one of the 2048 tokens against the oracle (about a minute of
    oracle time on 16 host threads), and against the GEMV path."""
    L = prefill
    T = L.wl.T
    print("prefill output: T=%d, all rows, grouped path" % T, flush=True)
    y, idx, w = forward(m, L, m.MOE_PATH_AUTO)
    yv, idxv, wv = forward(m, L, m.MOE_PATH_GEMV)
    assert np.array_equal(idx, idxv) and np.array_equal(w, wv)
    y = y.cpu().numpy()
    print("prefill output: oracle on %d tokens (%d threads)" % (T, oracle.num_threads()), flush=True)
    y_ref, idx_ref, w_ref = reference(L, np.arange(T))
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6)
    rel = assert_close(y, y_ref)
    print("prefill full output: max err %.3g of max|ref|" % rel)
    assert_close(yv.cpu().numpy(), y_ref, what="GEMV path at T=2048")
    # rows of every tile: the busiest experts span several 128-row tiles
    counts = np.bincount(idx.ravel(), minlength=L.wl.n_experts)
    assert counts.max() > 2 * 128


@pytest.fixture(scope="module")
def decode_batch(dev):
    return DevLayer(synth.workload("decode_int4"), dev, T=64)


@pytest.mark.parametrize("T", [3, 8, 16, 64])
def test_decode_shape_batches_both_paths(dev, m, decode_batch, T):
    L = decode_batch
    print("decode shape batch: T=%d, GEMV and grouped" % T, flush=True)
    yg, ig, wg = forward(m, L, m.MOE_PATH_GROUPED, T)
    yv, iv, wv = forward(m, L, m.MOE_PATH_GEMV, T)
    assert np.array_equal(ig, iv) and np.array_equal(wg, wv)
    y_ref, idx_ref, w_ref = reference(L, np.arange(T))
    assert np.array_equal(ig, idx_ref)
    np.testing.assert_allclose(wg, w_ref, rtol=1e-6)
    assert_close(yg.cpu().numpy(), y_ref, what="grouped")
    assert_close(yv.cpu().numpy(), y_ref, what="gemv")
    assert_close(yg.cpu().numpy(), yv.cpu().numpy().astype(np.float64), what="grouped vs gemv")


# ---------------------------------------------------------------- adaptive expert top-p
@pytest.mark.parametrize("wbits,T,p", [(4, 100, 0.6), (8, 40, 0.8), (2, 70, 0.5)])
def test_grouped_top_p(dev, m, wbits, T, p):
    """Top-p on the grouped path: the permutation gives dropped slots no row
    and the combine skips them; indices, weights and outputs match the
    oracle, and the GEMV path's routing bit for bit."""
    wl = synth.workload("tiny", wbits=wbits, top_p=p)
    L = DevLayer(wl, dev, T=T)
    y, idx, w = forward(m, L, m.MOE_PATH_GROUPED, T)
    y_ref, idx_ref, w_ref = reference(L, np.arange(T))
    assert (idx_ref < 0).any()
    assert np.array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=1e-6)
    assert_close(y.cpu().numpy(), y_ref)
    yg, idxg, _ = forward(m, L, m.MOE_PATH_GEMV, T)
    assert np.array_equal(idxg, idx)


# ---------------------------------------------------------------- full-size int8 and int2
@pytest.mark.parametrize("name,T", [("verify_int8", 16), ("stack_int2", 64)])
def test_full_size_int8_int2_both_paths(dev, m, name, T):
    """The grouped GEMMs' int8 (weights copied into LDS as they are) and
    int2 (four 2-bit fields expanded per byte) forms at the full H = 6144,
    I = 2048, next to the int4 cases above: T independent tokens of the
    verify_int8 layer and of layer 0 of the int2 stack, on the grouped and
    the GEMV path, each against the oracle (routing bit-exact)."""
    wl = synth.workload(name)
    L = DevLayer(wl, dev, T=T)
    print("full-size grouped parity: %s T=%d" % (name, T), flush=True)
    yg, ig, wg = forward(m, L, m.MOE_PATH_GROUPED, T)
    yv, iv, wv = forward(m, L, m.MOE_PATH_GEMV, T)
    y_ref, idx_ref, w_ref = reference(L, np.arange(T))
    assert np.array_equal(ig, idx_ref) and np.array_equal(iv, idx_ref)
    np.testing.assert_allclose(wg, w_ref, rtol=1e-6)
    assert_close(yg.cpu().numpy(), y_ref, what="grouped")
    assert_close(yv.cpu().numpy(), y_ref, what="gemv")

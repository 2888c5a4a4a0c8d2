"""Forced equivalence of the weight encodings on the GPU.

The same weight codes written in two layouts (int4 codes as int8 bytes; int2
codes as int4) are the same integers, so (GeekNews #31297, implemented
features: a fast path forced to coincide with a plain one must give the
same result):
  - moe_block_dots gives identical int32 block sums from either encoding;
  - the layer's routing is identical (the router never reads the experts);
  - the layer outputs agree within the layer tolerance, and each matches the
    oracle, whose own output is identical for both encodings (CPU pin in
    test_equivalence.py).
The int8 and int4 kernels are different code (no nibble unpacking, another
chunking of the rows), so their float sums may round differently, and the
h quantisation after g and u may then move one code; the outputs are held
to the benchmark spec's bound rather than bit equality.  Full decode-size layers,
one token (GEMV, routed inside the gate/up launch), a verify batch of 3
(GEMV batch plan) and 64 tokens (grouped GEMMs)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from codes import reencode_torch
from gpu_util import DevLayer, assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


def reencoded(w, wfrom, wto):
    # codes re-encoded tensor by tensor (one expert stack at a time keeps
    # the int16 temporaries small)
    out = []
    for f in ("gate", "up", "down"):
        t = getattr(w, f)
        out.append(torch.stack([reencode_torch(t[e], wfrom, wto) for e in range(t.shape[0])]))
    return synth.DeviceWeights(*out, w.gate_s, w.up_s, w.down_s)


def run(m, wl, L, routed, shared, T, flags):
    sh = m.shape_of(wl)
    dev = L.x.device
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    ws = m.workspace(m.moe_workspace_bytes(sh, T, flags), dev)
    m.moe_layer_forward(sh, L.x[:T], L.gate_w, L.bias, routed, shared, y, ws, idx, w, flags=flags)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name,wfrom,wto", [("decode_int4", 4, 8), ("stack_int2", 2, 4)])
def test_encodings_agree(dev, m, name, wfrom, wto):
    wl = synth.workload(name, layers=1, T=64)
    L = DevLayer(wl, dev)
    print("encoding equivalence: int%d codes as int%d, generating" % (wfrom, wto), flush=True)
    routed2 = reencoded(L.routed, wfrom, wto)
    shared2 = reencoded(L.shared, wfrom, wto)
    wl2 = synth.workload(name, layers=1, T=64, wbits=wto)
    torch.cuda.synchronize()

    # block dots: identical int32 sums from both encodings
    q = torch.empty((4, wl.hidden), dtype=torch.int8, device=dev)
    d = torch.empty((4, wl.hidden // 32), dtype=torch.float32, device=dev)
    m.moe_quant_act(L.x[:4], q, d)
    rows = 96
    a = torch.empty((4, rows, wl.hidden // 32), dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    m.moe_block_dots(wfrom, L.routed.gate[7, :rows].contiguous(), wl.hidden, q, a)
    m.moe_block_dots(wto, routed2.gate[7, :rows].contiguous(), wl.hidden, q, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

    for T, flags in ((1, m.MOE_PATH_GEMV), (3, m.MOE_PATH_GEMV), (64, m.MOE_PATH_GROUPED)):
        print("encoding equivalence: int%d vs int%d, T=%d path=%d" % (wfrom, wto, T, flags), flush=True)
        y1, i1, w1 = run(m, wl, L, L.routed, L.shared, T, flags)
        y2, i2, w2 = run(m, wl2, L, routed2, shared2, T, flags)
        assert np.array_equal(i1, i2) and np.array_equal(w1, w2)
        H = L.host
        sh = oracle.shape_of(wl)
        y_ref, idx_ref, _ = oracle.layer_forward(sh, H.x[:T], H.gate_w, H.bias, oracle.layer_experts(H, i1),
                                                 H.shared)
        assert np.array_equal(i1, idx_ref)
        assert_close(y1, y_ref, what="int%d" % wfrom)
        assert_close(y2, y_ref, what="int%d encoding of the same codes" % wto)
        rel = assert_close(y2, y1.astype(np.float64), what="int%d vs int%d" % (wto, wfrom))
        print("  max diff between encodings: %.3g of max|y|" % rel)

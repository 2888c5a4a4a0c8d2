"""moe_layer_forward_noalloc (the entry point for callers that cannot
allocate) against moe_layer_forward on a workspace of its own, through the
C ABI: bit-identical outputs and routing on two calls in a row, the second
smaller than the first (the fixed buffer keeps the first call's contents),
on the grouped path and both GEMV paths; a call larger than the fixed buffer
is refused with MOE_ESCRATCH before anything runs (its output untouched)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DevLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


def outputs(m, wl, dev, T):
    return (torch.full((T, wl.hidden), 3.0, dtype=torch.float32, device=dev),
            torch.empty((T, wl.top_k), dtype=torch.int32, device=dev),
            torch.empty((T, wl.top_k), dtype=torch.float32, device=dev))


def test_noalloc_matches_layer_forward(m, dev):
    wl = synth.workload("decode_int4", T=64)
    L = DevLayer(wl, dev)
    sh = m.shape_of(wl)
    for T, flags in ((64, m.MOE_PATH_GROUPED), (5, m.MOE_PATH_GEMV), (1, m.MOE_PATH_AUTO)):
        print("noalloc: decode_int4 T=%d path=%d" % (T, flags), flush=True)
        assert m.moe_workspace_bytes(sh, T, flags) <= m.MOE_NOALLOC_SCRATCH_BYTES
        y0, i0, w0 = outputs(m, wl, dev, T)
        ws = m.workspace(m.moe_workspace_bytes(sh, T, flags), dev)
        m.moe_layer_forward(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, y0, ws, i0, w0, flags=flags)
        y1, i1, w1 = outputs(m, wl, dev, T)
        m.moe_layer_forward_noalloc(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, y1, i1, w1, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(w0, w1)
        assert torch.equal(y0, y1)
        assert torch.isfinite(y1).all()


def test_noalloc_tiny_layers_and_accumulate(m, dev):
    # grouped then GEMV on a small layer, each also with MOE_ACCUMULATE
    wl = synth.workload("tiny", T=40)
    L = DevLayer(wl, dev)
    sh = m.shape_of(wl)
    for T in (40, 8):
        print("noalloc: tiny T=%d" % T, flush=True)
        base = torch.randn((T, wl.hidden), dtype=torch.float32, device=dev)
        y0, i0, w0 = outputs(m, wl, dev, T)
        y0.copy_(base)
        ws = m.workspace(m.moe_workspace_bytes(sh, T, 0), dev)
        m.moe_layer_forward(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, y0, ws, i0, w0,
                            flags=m.MOE_ACCUMULATE)
        y1, i1, w1 = outputs(m, wl, dev, T)
        y1.copy_(base)
        m.moe_layer_forward_noalloc(sh, L.x[:T], L.gate_w, L.bias, L.routed, L.shared, y1, i1, w1,
                                    flags=m.MOE_ACCUMULATE)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(w0, w1)


def test_noalloc_refuses_calls_beyond_its_buffer(m, dev):
    wl = synth.workload("prefill_int4", T=512)
    L = DevLayer(wl, dev)
    sh = m.shape_of(wl)
    assert m.moe_workspace_bytes(sh, 512, 0) > m.MOE_NOALLOC_SCRATCH_BYTES
    y, i, w = outputs(m, wl, dev, 512)
    with pytest.raises(m.MoeError) as e:
        m.moe_layer_forward_noalloc(sh, L.x, L.gate_w, L.bias, L.routed, L.shared, y, i, w)
    assert e.value.code == m.MOE_ESCRATCH
    torch.cuda.synchronize()
    assert (y == 3.0).all()
    # argument errors are those of moe_layer_forward
    with pytest.raises(m.MoeError) as e:
        m.moe_layer_forward_noalloc(sh, L.x[:4], L.gate_w, L.bias, L.routed, L.shared, y[:4], i[:4], w[:4],
                                    flags=3)
    assert e.value.code == m.MOE_EINVAL

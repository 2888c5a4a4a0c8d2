"""Forced equivalence of the weight encodings in the oracle (CPU).

The pages validate fast paths by forcing them to coincide with plain ones
(GeekNews #31297, implemented features: MLA absorption forced on still
matches the reference token for token).  Here: int4 codes written as int8
bytes, and int2 codes written as int4 or int8, are the same integers, so
the oracle's block dots are identical and its layer output is identical bit
for bit, whatever the encoding.  A mistake in the oracle's unpacking of one
layout (a nibble order, a sign extension, a field shift) breaks this."""
import numpy as np
import pytest

import oracle
import synth
from codes import pack, reencode, unpack


def test_pack_roundtrip_and_layout():
    rng = np.random.default_rng(3)
    for w in (2, 4, 8):
        lo, hi = -(1 << (w - 1)), (1 << (w - 1)) - 1
        c = rng.integers(lo, hi + 1, (5, 64)).astype(np.int8)
        assert np.array_equal(unpack(pack(c, w), w), c)
    # element 2m in the low nibble; element 4m+i at bits 2i; two's complement
    assert list(unpack(np.array([[0x8F]], np.uint8), 4)[0]) == [-1, -8]
    assert list(unpack(np.array([[0b01101100]], np.uint8), 2)[0]) == [0, -1, -2, 1]
    # the oracle's own code reader agrees with the helper on every element
    row = rng.integers(0, 256, 32, dtype=np.uint8)
    for w in (2, 4, 8):
        n = 32 * 8 // w
        assert [oracle.code(w, row, j) for j in range(n)] == list(unpack(row[None], w)[0])


def as_encoding(ex, wfrom, wto):
    return synth.HostExpert(reencode(ex.gate, wfrom, wto), reencode(ex.up, wfrom, wto),
                            reencode(ex.down, wfrom, wto), ex.gate_s, ex.up_s, ex.down_s)


@pytest.mark.parametrize("wfrom,wto", [(4, 8), (2, 4), (2, 8)])
def test_block_dots_identical(wfrom, wto):
    wl = synth.workload("tiny", wbits=wfrom)
    L = synth.HostLayer(wl)
    q, _ = oracle.quant_act(L.x)
    ex = L.expert(3)
    a = oracle.block_dots(wfrom, ex.gate, wl.hidden, q)
    b = oracle.block_dots(wto, reencode(ex.gate, wfrom, wto), wl.hidden, q)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("wfrom,wto", [(4, 8), (2, 4), (2, 8)])
def test_layer_identical_across_encodings(wfrom, wto):
    wl = synth.workload("tiny", wbits=wfrom, T=8)
    L = synth.HostLayer(wl)
    sh_from, sh_to = oracle.shape_of(wl), oracle.shape_of(synth.workload("tiny", wbits=wto))
    experts = {e: L.expert(e) for e in range(wl.n_experts)}
    y0, i0, w0 = oracle.layer_forward(sh_from, L.x, L.gate_w, L.bias, experts, L.shared)
    conv = {e: as_encoding(x, wfrom, wto) for e, x in experts.items()}
    y1, i1, w1 = oracle.layer_forward(sh_to, L.x, L.gate_w, L.bias, conv, as_encoding(L.shared, wfrom, wto))
    assert np.array_equal(i0, i1) and np.array_equal(w0, w1)
    assert np.array_equal(y0, y1)

"""The seeded input generator (no GPU): published sequence, layouts, distributions."""
import json
import math
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_sequence():
    g = json.load(open(os.path.join(GOLD, "splitmix64_seed1234567.json")))
    assert [synth.word(g["state"], i) for i in range(len(g["outputs"]))] == g["outputs"]


def test_bytes_are_little_endian_words():
    k = synth.key(0, 77)
    b = synth.host_bytes(0, 77, 24)
    for i in range(3):
        assert int.from_bytes(b[8 * i:8 * i + 8].tobytes(), "little") == synth.word(k, i)


def test_int8_codes_range_and_balance():
    c = synth.host_int8(0, 5, 1 << 20).astype(np.int64)
    assert c.min() == -127 and c.max() == 127
    assert abs(c.mean()) < 0.5
    counts = np.bincount(c + 127, minlength=255)
    assert counts.min() > 0.8 * counts.mean()


def test_packed_codes_uniform():
    b = synth.host_bytes(0, 9, 1 << 20)
    nib = np.concatenate([b & 15, b >> 4]).astype(np.int64)
    cnt = np.bincount(nib, minlength=16)
    assert np.all(np.abs(cnt / cnt.mean() - 1) < 0.02)


def test_scales_and_normals():
    s = synth.host_scales(0, 3, 100000, 6144)
    assert s.min() >= 0.5 / math.sqrt(6144) and s.max() < 1.5 / math.sqrt(6144)
    n = synth.host_normals(0, 4, 200000, 2.0)
    assert abs(n.mean()) < 0.02 and abs(n.std() - 2.0) < 0.02


def test_layer_streams_distinct_and_reproducible():
    wl = synth.workload("tiny")
    a, b = synth.HostLayer(wl), synth.HostLayer(wl)
    assert np.array_equal(a.expert(3).gate, b.expert(3).gate)
    assert not np.array_equal(a.expert(3).gate, a.expert(4).gate)
    assert not np.array_equal(a.expert(3).gate, a.expert(3).up)
    assert not np.array_equal(synth.HostLayer(wl, layer=1).x, a.x)
    assert a.shared.gate.shape == (wl.inter, wl.hidden // 2)


def test_shape_closure_against_pages():
    g = json.load(open(os.path.join(GOLD, "shape_closure.json")))
    wl = synth.WORKLOADS["decode_int4"]
    mb = wl.expert_bytes / 1e6
    assert abs(mb / g["expert_mb_int4"]["value"] - 1) < g["expert_mb_int4"]["rel_tol"]
    per_tok = g["moe_layers"] * g["active_routed"] * wl.expert_bytes / 1e9
    assert abs(per_tok / g["routed_gb_per_token"]["value"] - 1) < g["routed_gb_per_token"]["rel_tol"]
    disk = (g["moe_layers"] + 1) * g["experts_per_layer"] * wl.expert_bytes / 1e9
    assert abs(disk / g["disk_gb_int4"]["value"] - 1) < g["disk_gb_int4"]["rel_tol"]
    params = g["moe_layers"] * (g["experts_per_layer"] + g["shared"]) * 3 * wl.hidden * wl.inter
    total = params / 1e9 + g["total_params_b"]["dense_params_b"]
    assert abs(total / g["total_params_b"]["value"] - 1) < g["total_params_b"]["rel_tol"]

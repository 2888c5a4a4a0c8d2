"""Helpers for the GPU parity tests: device copies of synthetic layers and
the tolerance the float outputs are held to (max-abs error <= 1e-3 of the
reference's largest magnitude)."""
import numpy as np
import torch

import synth

REL_TOL = 1e-3


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def dev_expert(ex, dev):
    """DeviceWeights from a HostExpert (a single expert or a stack)."""
    return synth.DeviceWeights(*[to_dev(getattr(ex, f), dev) for f in
                                 ("gate", "up", "down", "gate_s", "up_s", "down_s")])


def assert_close(got, ref, rel=REL_TOL, what="output"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return
    err = np.abs(got - ref).max()
    tol = rel * np.abs(ref).max()
    assert err <= tol, "%s: max abs err %.4g > %.4g (= %g x max|ref|)" % (what, err, tol, rel)
    return err / max(np.abs(ref).max(), 1e-30)


class DevLayer:
    """One synthetic layer with its routed stack and shared expert in HBM
    (weights drawn on the device; the host regenerates any expert)."""

    def __init__(self, wl, dev, layer=0, T=None, host=None):
        self.wl = wl
        self.host = host if host is not None else synth.HostLayer(wl, layer=layer, T=T)
        self.x = to_dev(self.host.x, dev)
        self.gate_w = to_dev(self.host.gate_w, dev)
        self.bias = to_dev(self.host.bias, dev)
        self.routed = synth.device_weights(wl, layer, 0, wl.n_experts, dev)
        self.shared = synth.device_weights(wl, layer, wl.n_experts, 1, dev) if wl.n_shared else None

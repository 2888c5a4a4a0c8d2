"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package generates tensors only; it contains none of the MoE layer's
arithmetic.  Every tensor is a pure function of (seed, stream, index) through
SplitMix64 (see synth.c for the exact definitions), so the device twin can
fill multi-gigabyte weight stacks in HBM while the host regenerates any
single expert bit for bit for the oracle.

Workloads follow the shapes and distributions of the GLM-5.2 MoE layer the
pages describe (GeekNews #31297 "Show HN: running GLM 5.2 on a slow
computer", disk-streaming and implemented-features sections; wpnews.pro
"Colibri - GLM-5.2 744B MoE on 25GB RAM", spec table: 75 MoE layers, 256
experts, 8 active + 1 shared).  Hidden 6144 and intermediate 2048 are the
dims that reproduce the pages' ~19 MB int4 expert.
"""
import ctypes
import math
import os
from dataclasses import dataclass, replace

import numpy as np

from . import _build

# tensor kinds (bits 32..39 of the stream id)
X, GATE_W, BIAS, W_GATE, W_UP, W_DOWN, S_GATE, S_UP, S_DOWN = range(9)
# draft verification: target logits, draft-logit noise, draft draws, uniforms
MTP_P, MTP_Q, MTP_G, MTP_U = range(9, 13)


def stream_id(layer, kind, expert=0):
    """Stream of one tensor: layer in bits 40.., kind in 32..39, expert in 0..31.

    The shared expert uses expert index n_experts."""
    return (int(layer) << 40) | (int(kind) << 32) | int(expert)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    hidden: int
    inter: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    n_shared: int
    wbits: int
    rsf: float
    bias_sigma: float
    layers: int = 1
    seed: int = 0
    top_p: float = 0.0      # adaptive expert top-p (0: off)

    def rowbytes(self, in_dim):
        return in_dim * self.wbits // 8

    @property
    def gate_bytes(self):  # one expert's gate (or up) matrix: [inter][hidden]
        return self.inter * self.rowbytes(self.hidden)

    @property
    def down_bytes(self):  # one expert's down matrix: [hidden][inter]
        return self.hidden * self.rowbytes(self.inter)

    @property
    def expert_bytes(self):
        """Packed codes plus fp32 per-row scales of one SwiGLU expert."""
        return 2 * self.gate_bytes + self.down_bytes + 4 * (2 * self.inter + self.hidden)


# Sizes and distributions of the five workloads.  Router gate weights are
# N(0, 1/hidden); the correction bias N(0, v) is read with v a variance.
WORKLOADS = {
    "tiny": Workload("tiny", T=8, hidden=256, inter=128, n_experts=16, n_group=4, topk_group=2,
                     top_k=4, n_shared=1, wbits=4, rsf=2.5, bias_sigma=0.1),
    "decode_int4": Workload("decode_int4", T=1, hidden=6144, inter=2048, n_experts=256, n_group=8,
                            topk_group=4, top_k=8, n_shared=1, wbits=4, rsf=2.5, bias_sigma=0.1),
    "verify_int8": Workload("verify_int8", T=3, hidden=6144, inter=2048, n_experts=256, n_group=8,
                            topk_group=4, top_k=8, n_shared=1, wbits=8, rsf=2.5, bias_sigma=0.1),
    "prefill_int4": Workload("prefill_int4", T=2048, hidden=6144, inter=2048, n_experts=256, n_group=8,
                             topk_group=4, top_k=8, n_shared=1, wbits=4, rsf=2.5,
                             bias_sigma=math.sqrt(0.5)),
    "stack_int2": Workload("stack_int2", T=1, hidden=6144, inter=2048, n_experts=256, n_group=8,
                           topk_group=4, top_k=8, n_shared=1, wbits=2, rsf=2.5, bias_sigma=0.1,
                           layers=75),
}


def workload(name, **over):
    return replace(WORKLOADS[name], **over)


# ----------------------------------------------------------------------------
# host generator (ctypes over libsynth.so)

_host = None


def _host_lib():
    global _host
    if _host is None:
        # SYNTH_HOST_LIB names a sanitizer build of synth.c to load in place of HOST_LIB
        path = os.environ.get("SYNTH_HOST_LIB") or _build.HOST_LIB
        if path == _build.HOST_LIB and not os.path.exists(path):
            _build.build_host()
        lib = ctypes.CDLL(path)
        u64 = ctypes.c_uint64
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_word.restype = u64
        lib.synth_word.argtypes = [u64, u64]
        lib.synth_bytes.argtypes = [u64, u64, u64, ctypes.c_void_p]
        lib.synth_int8_codes.argtypes = [u64, u64, u64, ctypes.c_void_p]
        lib.synth_scales.argtypes = [u64, u64, u64, ctypes.c_double, ctypes.c_void_p]
        lib.synth_normals.argtypes = [u64, u64, u64, ctypes.c_double, ctypes.c_void_p]
        lib.synth_uniforms.argtypes = [u64, u64, u64, ctypes.c_void_p]
        _host = lib
    return _host


def key(seed, stream):
    return _host_lib().synth_key(seed, stream)


def word(k, i):
    return _host_lib().synth_word(k, i)


def host_bytes(seed, stream, n):
    out = np.empty(n, np.uint8)
    _host_lib().synth_bytes(key(seed, stream), 0, n, out.ctypes.data)
    return out


def host_int8(seed, stream, n):
    out = np.empty(n, np.int8)
    _host_lib().synth_int8_codes(key(seed, stream), 0, n, out.ctypes.data)
    return out


def host_scales(seed, stream, n, in_dim):
    out = np.empty(n, np.float32)
    _host_lib().synth_scales(key(seed, stream), 0, n, 1.0 / math.sqrt(in_dim), out.ctypes.data)
    return out


def host_normals(seed, stream, n, sigma):
    out = np.empty(n, np.float32)
    _host_lib().synth_normals(key(seed, stream), 0, n, float(sigma), out.ctypes.data)
    return out


def host_uniforms(seed, stream, n):
    out = np.empty(n, np.float64)
    _host_lib().synth_uniforms(key(seed, stream), 0, n, out.ctypes.data)
    return out


def mtp_inputs(seed, B, D, V, tau, sigma_p=3.0, sigma_n=1.0):
    """Synthetic inputs of one draft-verification step for B sequences.

    Target logits N(0, sigma_p^2) per token; the draft model's logits are the
    target's plus N(0, sigma_n^2) noise (a draft head that mostly agrees with
    the model); draft i of sequence b is drawn from the draft distribution at
    temperature tau by the Gumbel-max trick (its argmax when tau = 0), with
    uniforms of its own stream; u [B][D+1] are the uniforms the acceptance
    step consumes.  Returns (draft [B][D] int32, p_logits [B][D+1][V] f32,
    q_logits [B][D][V] f32, u [B][D+1] f64)."""
    p = np.empty((B, D + 1, V), np.float32)
    q = np.empty((B, D, V), np.float32)
    draft = np.empty((B, D), np.int32)
    u = np.empty((B, D + 1), np.float64)
    for b in range(B):
        p[b] = host_normals(seed, stream_id(0, MTP_P, b), (D + 1) * V, sigma_p).reshape(D + 1, V)
        if D:
            q[b] = p[b, :D] + host_normals(seed, stream_id(0, MTP_Q, b), D * V, sigma_n).reshape(D, V)
            if tau > 0:
                g = host_uniforms(seed, stream_id(0, MTP_G, b), D * V).reshape(D, V)
                g = -np.log(-np.log(g + 2.0 ** -54))  # Gumbel(0, 1); the offset keeps log(0) out
                draft[b] = np.argmax(q[b].astype(np.float64) / tau + g, axis=1)
            else:
                draft[b] = np.argmax(q[b], axis=1)
        u[b] = host_uniforms(seed, stream_id(0, MTP_U, b), D + 1)
    return draft, p, q, u


def _codes(wl, seed, stream, rows, in_dim):
    if wl.wbits == 8:
        return host_int8(seed, stream, rows * in_dim).reshape(rows, in_dim).view(np.uint8)
    return host_bytes(seed, stream, rows * wl.rowbytes(in_dim)).reshape(rows, wl.rowbytes(in_dim))


@dataclass
class HostExpert:
    """Packed codes (row-major [rows][rowbytes] uint8) and fp32 per-row scales."""
    gate: np.ndarray
    up: np.ndarray
    down: np.ndarray
    gate_s: np.ndarray
    up_s: np.ndarray
    down_s: np.ndarray


class HostLayer:
    """One layer's inputs on the host.  Experts are generated on demand."""

    def __init__(self, wl, layer=0, seed=None, T=None):
        self.wl = wl
        self.layer = layer
        self.seed = wl.seed if seed is None else seed
        self.T = wl.T if T is None else T
        H, E = wl.hidden, wl.n_experts
        self.x = host_normals(self.seed, stream_id(layer, X), self.T * H, 1.0).reshape(self.T, H)
        self.gate_w = host_normals(self.seed, stream_id(layer, GATE_W), E * H,
                                   1.0 / math.sqrt(H)).reshape(E, H)
        self.bias = host_normals(self.seed, stream_id(layer, BIAS), E, wl.bias_sigma)
        self._experts = {}

    def expert(self, e):
        """Expert e in [0, n_experts); e == n_experts is the shared expert."""
        if e not in self._experts:
            wl, s, l = self.wl, self.seed, self.layer
            H, I = wl.hidden, wl.inter
            self._experts[e] = HostExpert(
                gate=_codes(wl, s, stream_id(l, W_GATE, e), I, H),
                up=_codes(wl, s, stream_id(l, W_UP, e), I, H),
                down=_codes(wl, s, stream_id(l, W_DOWN, e), H, I),
                gate_s=host_scales(s, stream_id(l, S_GATE, e), I, H),
                up_s=host_scales(s, stream_id(l, S_UP, e), I, H),
                down_s=host_scales(s, stream_id(l, S_DOWN, e), H, I),
            )
        return self._experts[e]

    @property
    def shared(self):
        return self.expert(self.wl.n_experts)

    def stacked(self):
        """All routed experts stacked: codes [E][rows][rowbytes], scales [E][rows]."""
        ex = [self.expert(e) for e in range(self.wl.n_experts)]
        return HostExpert(*[np.stack([getattr(x, f) for x in ex]) for f in
                            ("gate", "up", "down", "gate_s", "up_s", "down_s")])


# ----------------------------------------------------------------------------
# device generator (ctypes over libsynth_dev.so; tensors from torch)

_dev = None


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(_build.DEV_LIB):
            raise RuntimeError("libsynth_dev.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_build.DEV_LIB)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_dev_bytes.argtypes = [u64, u64, i64, u64, vp, vp]
        lib.synth_dev_int8.argtypes = [u64, u64, i64, u64, vp, vp]
        lib.synth_dev_scales.argtypes = [u64, u64, i64, u64, ctypes.c_double, vp, vp]
        _dev = lib
    return _dev


def _stream_handle(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed with code %d" % (what, rc))


class DeviceWeights:
    """Stacked expert weights in device memory (torch uint8 / float32 tensors)."""

    def __init__(self, gate, up, down, gate_s, up_s, down_s):
        self.gate, self.up, self.down = gate, up, down
        self.gate_s, self.up_s, self.down_s = gate_s, up_s, down_s


def device_weights(wl, layer, e0, n_exp, device="cuda", seed=None):
    """Experts e0 .. e0+n_exp-1 of `layer`, generated directly in HBM.

    Expert e0 + j of the stack is drawn from stream_id(layer, kind, e0 + j), so
    the host can regenerate it bit for bit with HostLayer(...).expert(e0 + j)."""
    import torch
    seed = wl.seed if seed is None else seed
    lib, st = _dev_lib(), _stream_handle(torch)
    H, I = wl.hidden, wl.inter

    def fill(fn, kind, t, per, *extra):
        if e0 == 0:  # stream_base | e == stream_id(layer, kind, e) for the whole stack
            _check(fn(seed, stream_id(layer, kind, 0), n_exp, per, *extra, t.data_ptr(), st), fn.__name__)
        else:
            for j in range(n_exp):
                _check(fn(seed, stream_id(layer, kind, e0 + j), 1, per, *extra, t[j].data_ptr(), st),
                       fn.__name__)
        return t

    def codes(kind, rows, in_dim):
        t = torch.empty((n_exp, rows, wl.rowbytes(in_dim)), dtype=torch.uint8, device=device)
        per = rows * wl.rowbytes(in_dim)
        return fill(lib.synth_dev_int8 if wl.wbits == 8 else lib.synth_dev_bytes, kind, t, per)

    def scales(kind, rows, in_dim):
        t = torch.empty((n_exp, rows), dtype=torch.float32, device=device)
        return fill(lib.synth_dev_scales, kind, t, rows, 1.0 / math.sqrt(in_dim))

    return DeviceWeights(codes(W_GATE, I, H), codes(W_UP, I, H), codes(W_DOWN, H, I),
                         scales(S_GATE, I, H), scales(S_UP, I, H), scales(S_DOWN, H, I))


class StackLayer:
    """One layer of a device-resident decode stack: router weights, correction
    bias, RMSNorm weight (ones) and expert stacks, all in HBM."""

    def __init__(self, gate_w, bias, norm_g, routed, shared):
        self.gate_w, self.bias, self.norm_g = gate_w, bias, norm_g
        self.routed, self.shared = routed, shared


def device_stack(wl, device="cuda", layers=None):
    """Every layer of a stack workload generated in HBM (about 2.4 GB per int2
    layer of the GLM-5.2 shape), plus the host copies of the router weights
    (HostLayer per layer, experts regenerated on demand)."""
    import torch
    n = wl.layers if layers is None else layers
    hosts, dev_layers = [], []
    ones = torch.ones(wl.hidden, dtype=torch.float32, device=device)
    for l in range(n):
        h = HostLayer(wl, layer=l)
        hosts.append(h)
        dev_layers.append(StackLayer(torch.from_numpy(h.gate_w).to(device), torch.from_numpy(h.bias).to(device),
                                     ones, device_weights(wl, l, 0, wl.n_experts, device),
                                     device_weights(wl, l, wl.n_experts, 1, device) if wl.n_shared else None))
    return hosts, dev_layers

"""ctypes binding of libmoe.so (include/moe.h), same names as the C ABI.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  Tensors are torch tensors on the GPU (PyTorch provides device
memory and streams); each wrapper checks dtype / device / contiguity, passes
data_ptr()s and the current HIP stream, and raises MoeError on a non-zero
return code.  If libmoe.so is missing the import fails loudly: there is no
fallback implementation.
"""
import ctypes
import os

import torch

from . import _build

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = range(6)
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_GROUPED, MOE_ACCUMULATE = 0, 1, 2, 4


def MOE_LOOKAHEAD(n):
    """moe_stack_forward: router lookahead with n workgroups per prefetched expert."""
    if not 0 <= n <= 63:
        raise ValueError("lookahead workgroups must be in 0 .. 63")
    return n << 16


def MOE_STAGE(n):
    return 1 << (8 + n)


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s failed: %s (%d)" % (fn, strerror(code), code))
        self.code = code


class moe_layer_t(ctypes.Structure):
    pass


class moe_shape_t(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("wbits", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("routed_top_p", ctypes.c_float)]


class moe_weights_t(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


moe_layer_t._fields_ = [("gate_w", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("norm_g", ctypes.c_void_p),
                        ("routed", moe_weights_t), ("shared", moe_weights_t)]


def _load():
    # MOE_LIB names another build of the same sources to load in place of the
    # in-tree library (the sanitizer build of the host code, for CPU-only tests)
    path = os.environ.get("MOE_LIB") or _build.LIB
    if not os.path.exists(path):
        raise ImportError("libmoe.so is not built (%s); run __graft_entry__.build()" % path)
    L = ctypes.CDLL(path)
    L.path = path
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_route": (ctypes.c_int, [P(moe_shape_t), vp, i32, vp, vp, vp, vp, vp, sz, vp]),
        "moe_route_workspace_bytes": (sz, [P(moe_shape_t), i32]),
        "moe_quant_act": (ctypes.c_int, [vp, i32, i32, vp, vp, vp]),
        "moe_block_dots": (ctypes.c_int, [i32, vp, i32, i32, vp, i32, vp, vp]),
        "moe_stream_read": (ctypes.c_int, [vp, sz, vp, vp]),
        "moe_expert_ffn": (ctypes.c_int, [P(moe_shape_t), P(moe_weights_t), i32, vp, vp, i32, vp, vp, sz, vp]),
        "moe_layer_forward": (ctypes.c_int, [P(moe_shape_t), vp, i32, vp, vp, P(moe_weights_t),
                                             P(moe_weights_t), vp, vp, vp, u32, vp, sz, vp]),
        "moe_workspace_bytes": (sz, [P(moe_shape_t), i32, u32]),
        "moe_layer_forward_noalloc": (ctypes.c_int, [P(moe_shape_t), vp, i32, vp, vp, P(moe_weights_t),
                                                     P(moe_weights_t), vp, vp, vp, u32, vp]),
        "moe_layer_stage_count": (ctypes.c_int, [P(moe_shape_t), i32, u32]),
        "moe_rmsnorm": (ctypes.c_int, [vp, vp, ctypes.c_double, i32, i32, vp, vp]),
        "moe_permute": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "moe_permute_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_mtp_accept": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]),
        "moe_mtp_accept_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_stack_forward": (ctypes.c_int, [P(moe_shape_t), vp, i32, P(moe_layer_t), i32, ctypes.c_double,
                                             vp, vp, u32, vp, sz, vp]),
        "moe_stack_workspace_bytes": (sz, [P(moe_shape_t), i32, u32]),
        "moe_tier_create": (ctypes.c_int, [P(moe_shape_t), P(moe_weights_t), i32, P(vp)]),
        "moe_tier_repin": (ctypes.c_int, [vp, P(i32), vp]),
        "moe_tier_plan": (ctypes.c_int, [P(u32), i32, i32, P(i32), P(i32), i32]),
        "moe_tier_prefetch": (ctypes.c_int, [vp, P(i32), i32, P(i32), vp]),
        "moe_tier_resident": (ctypes.c_int, [vp, P(i32)]),
        "moe_tier_counts": (ctypes.c_int, [vp, P(u32), vp]),
        "moe_layer_forward_tiered": (ctypes.c_int, [P(moe_shape_t), vp, i32, vp, vp, vp, P(moe_weights_t), vp, vp,
                                                    vp, u32, vp, sz, vp]),
        "moe_tier_destroy": (None, [vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


lib = _load()


def strerror(code):
    return lib.moe_strerror(code).decode()


def _chk(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def _ptr(t, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError("expected %s, got %s" % (dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def shape(hidden, inter, n_experts, n_group, topk_group, top_k, n_shared, wbits, rsf, top_p=0.0):
    return moe_shape_t(hidden, inter, n_experts, n_group, topk_group, top_k, n_shared, wbits, rsf, top_p)


def shape_of(wl, rsf=None, top_p=None):
    """moe_shape_t from an object with the workload fields (hidden, inter, ...)."""
    return shape(wl.hidden, wl.inter, wl.n_experts, wl.n_group, wl.topk_group, wl.top_k,
                 wl.n_shared, wl.wbits, wl.rsf if rsf is None else rsf,
                 getattr(wl, "top_p", 0.0) if top_p is None else top_p)


def weights(w):
    """moe_weights_t from an object with gate/up/down (uint8) and *_s (float32) tensors."""
    return moe_weights_t(_ptr(w.gate, torch.uint8), _ptr(w.up, torch.uint8), _ptr(w.down, torch.uint8),
                         _ptr(w.gate_s, torch.float32), _ptr(w.up_s, torch.float32),
                         _ptr(w.down_s, torch.float32))


def workspace(nbytes, device="cuda"):
    """A device buffer for the *_workspace_bytes sizes (torch's allocations
    are 256-byte aligned; the calls need no initial contents)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moe_route_workspace_bytes(sh, T):
    return lib.moe_route_workspace_bytes(ctypes.byref(sh), T)


def moe_route(sh, x, gate_w, bias, idx, w, ws, stream=None):
    _chk("moe_route", lib.moe_route(ctypes.byref(sh), _ptr(x, torch.float32), x.shape[0],
                                    _ptr(gate_w, torch.float32), _ptr(bias, torch.float32),
                                    _ptr(idx, torch.int32), _ptr(w, torch.float32),
                                    _ptr(ws), ws.numel(), _stream(stream)))


def moe_quant_act(x, q, d, stream=None):
    T, D = x.shape
    _chk("moe_quant_act", lib.moe_quant_act(_ptr(x, torch.float32), T, D, _ptr(q, torch.int8),
                                            _ptr(d, torch.float32), _stream(stream)))


MOE_STREAM_SINK_WORDS = 2048 * 256


def moe_stream_read(src, sink, stream=None):
    """Reads every byte of the device tensor src once (measurement aid);
    sink: MOE_STREAM_SINK_WORDS int32 words of XORs."""
    if sink.numel() < MOE_STREAM_SINK_WORDS:
        raise ValueError("sink needs %d words" % MOE_STREAM_SINK_WORDS)
    _chk("moe_stream_read", lib.moe_stream_read(_ptr(src), src.numel() * src.element_size(),
                                                _ptr(sink, torch.int32), _stream(stream)))


def moe_block_dots(wbits, codes, D, q, out, stream=None):
    _chk("moe_block_dots", lib.moe_block_dots(wbits, _ptr(codes, torch.uint8), codes.shape[0], D,
                                              _ptr(q, torch.int8), q.shape[0], _ptr(out, torch.int32),
                                              _stream(stream)))


def moe_expert_ffn(sh, w, expert, q, d, y, ws, stream=None):
    wt = weights(w)
    _chk("moe_expert_ffn", lib.moe_expert_ffn(ctypes.byref(sh), ctypes.byref(wt), expert,
                                              _ptr(q, torch.int8), _ptr(d, torch.float32), q.shape[0],
                                              _ptr(y, torch.float32), _ptr(ws), ws.numel(), _stream(stream)))


def moe_workspace_bytes(sh, T, flags=0):
    return lib.moe_workspace_bytes(ctypes.byref(sh), T, flags)


def moe_layer_stage_count(sh, T, flags=0):
    return lib.moe_layer_stage_count(ctypes.byref(sh), T, flags)


def moe_layer_forward(sh, x, gate_w, bias, routed, shared, y, ws, idx_out=None, w_out=None, flags=0,
                      stream=None):
    rw = weights(routed)
    sw = weights(shared) if shared is not None else None
    _chk("moe_layer_forward", lib.moe_layer_forward(
        ctypes.byref(sh), _ptr(x, torch.float32), x.shape[0], _ptr(gate_w, torch.float32),
        _ptr(bias, torch.float32), ctypes.byref(rw), ctypes.byref(sw) if sw is not None else None,
        _ptr(y, torch.float32), _ptr(idx_out, torch.int32), _ptr(w_out, torch.float32), flags,
        _ptr(ws), ws.numel(), _stream(stream)))


def moe_layer_forward_noalloc(sh, x, gate_w, bias, routed, shared, y, idx_out=None, w_out=None, flags=0,
                              stream=None):
    """moe_layer_forward on the library's fixed scratch buffer (no workspace)."""
    rw = weights(routed)
    sw = weights(shared) if shared is not None else None
    _chk("moe_layer_forward_noalloc", lib.moe_layer_forward_noalloc(
        ctypes.byref(sh), _ptr(x, torch.float32), x.shape[0], _ptr(gate_w, torch.float32),
        _ptr(bias, torch.float32), ctypes.byref(rw), ctypes.byref(sw) if sw is not None else None,
        _ptr(y, torch.float32), _ptr(idx_out, torch.int32), _ptr(w_out, torch.float32), flags,
        _stream(stream)))


def moe_rmsnorm(x, g, eps, out, stream=None):
    T, H = x.shape
    _chk("moe_rmsnorm", lib.moe_rmsnorm(_ptr(x, torch.float32), _ptr(g, torch.float32), eps, T, H,
                                        _ptr(out, torch.float32), _stream(stream)))


def moe_permute_workspace_bytes(T, k, E):
    return lib.moe_permute_workspace_bytes(T, k, E)


def moe_permute(idx, E, perm, off, inv, ws, stream=None):
    T, k = idx.shape
    _chk("moe_permute", lib.moe_permute(_ptr(idx, torch.int32), T, k, E, _ptr(perm, torch.int32),
                                        _ptr(off, torch.int32), _ptr(inv, torch.int32), _ptr(ws),
                                        ws.numel(), _stream(stream)))


def layers(descs):
    """Host array of moe_layer_t from objects with gate_w, bias, norm_g tensors
    and routed / shared weight objects (shared may be None)."""
    arr = (moe_layer_t * len(descs))()
    for i, d in enumerate(descs):
        arr[i].gate_w = _ptr(d.gate_w, torch.float32)
        arr[i].bias = _ptr(d.bias, torch.float32)
        arr[i].norm_g = _ptr(d.norm_g, torch.float32)
        arr[i].routed = weights(d.routed)
        if d.shared is not None:
            arr[i].shared = weights(d.shared)
    return arr


def moe_stack_workspace_bytes(sh, T, flags=0):
    return lib.moe_stack_workspace_bytes(ctypes.byref(sh), T, flags)


def moe_stack_forward(sh, x, layer_array, eps, ws, idx_out=None, w_out=None, flags=0, stream=None):
    """x [T][H] fp32 updated in place; layer_array from layers()."""
    _chk("moe_stack_forward", lib.moe_stack_forward(
        ctypes.byref(sh), _ptr(x, torch.float32), x.shape[0], layer_array, len(layer_array), eps,
        _ptr(idx_out, torch.int32), _ptr(w_out, torch.float32), flags, _ptr(ws), ws.numel(), _stream(stream)))


def moe_mtp_accept_workspace_bytes(B, D, V):
    return lib.moe_mtp_accept_workspace_bytes(B, D, V)


def moe_mtp_accept(draft, p_logits, q_logits, tau, u, n_acc, next_tok, ws, stream=None):
    """draft [B][D] int32, p_logits [B][D+1][V] and q_logits [B][D][V] float32,
    u [B][D+1] float64 (device tensors); writes n_acc and next_tok [B] int32."""
    B, D1, V = p_logits.shape
    D = D1 - 1
    _chk("moe_mtp_accept", lib.moe_mtp_accept(
        B, D, V, _ptr(draft, torch.int32) if D else None, _ptr(p_logits, torch.float32),
        _ptr(q_logits, torch.float32) if D else None, float(tau), _ptr(u, torch.float64),
        _ptr(n_acc, torch.int32), _ptr(next_tok, torch.int32), _ptr(ws), ws.numel(), _stream(stream)))


# ---------------------------------------------------------------- expert tier
def _host_ptr(t, dtype):
    """pinned host tensor -> its address (the tier maps it for the device)"""
    if t.is_cuda or not t.is_pinned():
        raise ValueError("tier host tensors must be pinned host memory")
    if not t.is_contiguous() or t.dtype != dtype:
        raise ValueError("expected a contiguous %s tensor" % dtype)
    return ctypes.c_void_p(t.data_ptr())


class Tier:
    """One layer's HBM / host expert tier (moe_tier_*).  host_w: the routed
    stacks as pinned host tensors (kept referenced here)."""

    def __init__(self, sh, host_w, slots):
        self._host = host_w
        hw = moe_weights_t(_host_ptr(host_w.gate, torch.uint8), _host_ptr(host_w.up, torch.uint8),
                           _host_ptr(host_w.down, torch.uint8), _host_ptr(host_w.gate_s, torch.float32),
                           _host_ptr(host_w.up_s, torch.float32), _host_ptr(host_w.down_s, torch.float32))
        self.h = ctypes.c_void_p()
        self.E = sh.n_experts
        _chk("moe_tier_create", lib.moe_tier_create(ctypes.byref(sh), ctypes.byref(hw), slots, ctypes.byref(self.h)))

    def repin(self, stream=None):
        n = ctypes.c_int32(0)
        _chk("moe_tier_repin", lib.moe_tier_repin(self.h, ctypes.byref(n), _stream(stream)))
        return n.value

    def prefetch(self, experts, stream=None):
        ids = [int(e) for e in experts]
        arr = (ctypes.c_int32 * max(1, len(ids)))(*ids)
        n = ctypes.c_int32(0)
        _chk("moe_tier_prefetch", lib.moe_tier_prefetch(self.h, arr, len(ids), ctypes.byref(n), _stream(stream)))
        return n.value

    def resident(self):
        out = (ctypes.c_int32 * self.E)()
        _chk("moe_tier_resident", lib.moe_tier_resident(self.h, out))
        return list(out)

    def counts(self, stream=None):
        out = (ctypes.c_uint32 * self.E)()
        _chk("moe_tier_counts", lib.moe_tier_counts(self.h, out, _stream(stream)))
        return list(out)

    def close(self):
        if self.h:
            lib.moe_tier_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_tier_plan(heat, C, slot_in, max_swaps=4):
    """The repin decision (host only): returns (copies, slot_out)."""
    E = len(heat)
    h = (ctypes.c_uint32 * E)(*heat)
    si = (ctypes.c_int32 * E)(*slot_in)
    so = (ctypes.c_int32 * E)()
    n = lib.moe_tier_plan(h, E, C, si, so, max_swaps)
    if n < 0:
        raise MoeError("moe_tier_plan", -n)
    return n, list(so)


def moe_layer_forward_tiered(sh, x, gate_w, bias, tier, shared, y, ws, idx_out=None, w_out=None, flags=0,
                             stream=None):
    sw = weights(shared) if shared is not None else None
    _chk("moe_layer_forward_tiered", lib.moe_layer_forward_tiered(
        ctypes.byref(sh), _ptr(x, torch.float32), x.shape[0], _ptr(gate_w, torch.float32),
        _ptr(bias, torch.float32), tier.h, ctypes.byref(sw) if sw is not None else None,
        _ptr(y, torch.float32), _ptr(idx_out, torch.int32), _ptr(w_out, torch.float32), flags,
        _ptr(ws), ws.numel(), _stream(stream)))

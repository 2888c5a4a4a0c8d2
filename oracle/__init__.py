"""CPU oracle of the quantised MoE layer -- TEST INFRASTRUCTURE ONLY.

Thin ctypes marshalling over liboracle.so (oracle.c, plain C99, fp64).  Only
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the product library and its Python binding never do.

Every function here converts numpy arrays and calls the C function of the
same name; the arithmetic and its citations live in oracle.c.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build():
    """Compile oracle.c with gcc (no fast-math: IEEE division and rintf hold)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "oracle.c", "-o", LIB, "-lm"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n%s%s" % (r.stdout, r.stderr))


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("wbits", ctypes.c_int32),
                ("rsf", ctypes.c_double), ("top_p", ctypes.c_double)]


class Expert(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB names a sanitizer build of oracle.c to load in place of LIB
        path = os.environ.get("ORACLE_LIB") or LIB
        if path == LIB and not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(path)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.oracle_num_threads.restype = i32
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_code.restype = i32
        L.oracle_code.argtypes = [i32, vp, i32]
        L.oracle_route.restype = i32
        L.oracle_route.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp]
        L.oracle_router_scores.argtypes = [vp, vp, vp, vp, vp, vp]
        L.oracle_quant_act.argtypes = [vp, i32, i32, vp, vp]
        L.oracle_block_dots.argtypes = [i32, vp, i32, i32, vp, i32, vp]
        L.oracle_matvec.argtypes = [i32, vp, vp, i32, i32, vp, vp, i32, vp]
        L.oracle_dequant_matmul.argtypes = [i32, vp, vp, i32, i32, vp, vp, i32, vp]
        L.oracle_expert_ffn.restype = i32
        L.oracle_expert_ffn.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp]
        L.oracle_layer_forward.restype = i32
        L.oracle_layer_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_combine.restype = i32
        L.oracle_combine.argtypes = [vp, i32, vp, vp, vp, vp]
        L.oracle_rmsnorm.argtypes = [vp, vp, dbl, i32, i32, vp]
        L.oracle_permute.restype = i32
        L.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.oracle_mtp_accept.restype = i32
        L.oracle_mtp_accept.argtypes = [i32, i32, i32, vp, vp, vp, dbl, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def shape_of(wl, rsf=None, top_p=None):
    # top_p as the fp32 value the GPU library receives
    p = getattr(wl, "top_p", 0.0) if top_p is None else top_p
    return Shape(wl.hidden, wl.inter, wl.n_experts, wl.n_group, wl.topk_group, wl.top_k,
                 wl.n_shared, wl.wbits, wl.rsf if rsf is None else rsf, float(np.float32(p)))


def _expert_struct(ex):
    arrs = [_c(ex.gate, np.uint8), _c(ex.up, np.uint8), _c(ex.down, np.uint8),
            _c(ex.gate_s, np.float32), _c(ex.up_s, np.float32), _c(ex.down_s, np.float32)]
    return Expert(*[a.ctypes.data for a in arrs]), arrs


def num_threads():
    return lib().oracle_num_threads()


def set_num_threads(n):
    lib().oracle_set_num_threads(int(n))


def code(wbits, row, j):
    row = _c(row, np.uint8)
    return lib().oracle_code(wbits, _p(row), j)


def route(sh, x, gate_w, bias, margins=False):
    x, gate_w, bias = _c(x, np.float32), _c(gate_w, np.float32), _c(bias, np.float32)
    T = x.shape[0]
    idx = np.empty((T, sh.top_k), np.int32)
    w = np.empty((T, sh.top_k), np.float32)
    m = np.empty((T, 2), np.float64) if margins else None
    rc = lib().oracle_route(ctypes.byref(sh), _p(x), T, _p(gate_w), _p(bias), _p(idx), _p(w), _p(m))
    if rc:
        raise ValueError("oracle_route failed: %d" % rc)
    return (idx, w, m) if margins else (idx, w)


def router_scores(sh, x_row, gate_w, bias):
    x_row, gate_w, bias = _c(x_row, np.float32), _c(gate_w, np.float32), _c(bias, np.float32)
    s = np.empty(sh.n_experts, np.float64)
    c = np.empty(sh.n_experts, np.float64)
    lib().oracle_router_scores(ctypes.byref(sh), _p(x_row), _p(gate_w), _p(bias), _p(s), _p(c))
    return s, c


def quant_act(x):
    x = _c(x, np.float32)
    T, D = x.shape
    q = np.empty((T, D), np.int8)
    d = np.empty((T, D // 32), np.float32)
    lib().oracle_quant_act(_p(x), T, D, _p(q), _p(d))
    return q, d


def block_dots(wbits, codes, D, q):
    codes, q = _c(codes, np.uint8), _c(q, np.int8)
    rows, T = codes.shape[0], q.shape[0]
    out = np.empty((T, rows, D // 32), np.int32)
    lib().oracle_block_dots(wbits, _p(codes), rows, D, _p(q), T, _p(out))
    return out


def matvec(wbits, codes, s_w, D, q, d):
    codes, s_w, q, d = _c(codes, np.uint8), _c(s_w, np.float32), _c(q, np.int8), _c(d, np.float32)
    rows, T = codes.shape[0], q.shape[0]
    y = np.empty((T, rows), np.float32)
    lib().oracle_matvec(wbits, _p(codes), _p(s_w), rows, D, _p(q), _p(d), T, _p(y))
    return y


def dequant_matmul(wbits, codes, s_w, D, q, d):
    codes, s_w, q, d = _c(codes, np.uint8), _c(s_w, np.float32), _c(q, np.int8), _c(d, np.float32)
    rows, T = codes.shape[0], q.shape[0]
    y = np.empty((T, rows), np.float64)
    lib().oracle_dequant_matmul(wbits, _p(codes), _p(s_w), rows, D, _p(q), _p(d), T, _p(y))
    return y


def expert_ffn(sh, ex, q, d, with_h=False):
    q, d = _c(q, np.int8), _c(d, np.float32)
    T = q.shape[0]
    y = np.empty((T, sh.hidden), np.float32)
    qh = np.empty((T, sh.inter), np.int8)
    dh = np.empty((T, sh.inter // 32), np.float32)
    st, keep = _expert_struct(ex)
    rc = lib().oracle_expert_ffn(ctypes.byref(sh), ctypes.byref(st), _p(q), _p(d), T, _p(y),
                                 _p(qh), _p(dh))
    del keep
    if rc:
        raise RuntimeError("oracle_expert_ffn failed: %d" % rc)
    return (y, qh, dh) if with_h else y


def layer_forward(sh, x, gate_w, bias, experts, shared):
    """experts: mapping e -> HostExpert (only the experts the tokens select are needed)."""
    x, gate_w, bias = _c(x, np.float32), _c(gate_w, np.float32), _c(bias, np.float32)
    T = x.shape[0]
    keep = []
    ptrs = (ctypes.c_void_p * sh.n_experts)()
    structs = {}
    for e, ex in experts.items():
        st, arrs = _expert_struct(ex)
        keep.append(arrs)
        structs[e] = st
        ptrs[e] = ctypes.addressof(st)
    sh_st = None
    if shared is not None:
        sh_st, arrs = _expert_struct(shared)
        keep.append(arrs)
    y = np.empty((T, sh.hidden), np.float32)
    idx = np.empty((T, sh.top_k), np.int32)
    w = np.empty((T, sh.top_k), np.float32)
    rc = lib().oracle_layer_forward(ctypes.byref(sh), _p(x), T, _p(gate_w), _p(bias), ptrs,
                                    ctypes.byref(sh_st) if sh_st is not None else None,
                                    _p(y), _p(idx), _p(w))
    if rc:
        raise RuntimeError("oracle_layer_forward failed: %d" % rc)
    return y, idx, w


def combine(sh, w, y_slots, y_shared):
    w, y_slots = _c(w, np.float32), _c(y_slots, np.float32)
    T = w.shape[0]
    ys = _c(y_shared, np.float32) if y_shared is not None else None
    out = np.empty((T, sh.hidden), np.float32)
    lib().oracle_combine(ctypes.byref(sh), T, _p(w), _p(y_slots), _p(ys), _p(out))
    return out


def rmsnorm(x, g, eps=1e-6):
    x, g = _c(x, np.float32), _c(g, np.float32)
    T, H = x.shape
    out = np.empty((T, H), np.float32)
    lib().oracle_rmsnorm(_p(x), _p(g), eps, T, H, _p(out))
    return out


def permute(idx, E):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    perm = np.empty(T * k, np.int32)
    off = np.empty(E + 1, np.int32)
    inv = np.empty(T * k, np.int32)
    rc = lib().oracle_permute(_p(idx), T, k, E, _p(perm), _p(off), _p(inv))
    if rc:
        raise ValueError("oracle_permute failed: %d" % rc)
    return perm, off, inv.reshape(T, k)


def layer_experts(layer, idx):
    """HostExpert objects for the routed experts that idx selects."""
    return {int(e): layer.expert(int(e)) for e in np.unique(idx) if e >= 0}


def mtp_accept(draft, p_logits, q_logits, tau, u):
    """Draft verification: draft [B][D] int32, p_logits [B][D+1][V],
    q_logits [B][D][V] float32, uniforms u [B][D+1] float64.  Returns
    (n_acc [B], next [B], margins [B])."""
    p_logits = _c(p_logits, np.float32)
    B, D1, V = p_logits.shape
    D = D1 - 1
    draft = _c(np.asarray(draft).reshape(B, D), np.int32)
    q_logits = _c(np.asarray(q_logits).reshape(B, D, V), np.float32)
    u = _c(np.asarray(u).reshape(B, D + 1), np.float64)
    n_acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    mg = np.empty(B, np.float64)
    rc = lib().oracle_mtp_accept(B, D, V, _p(draft), _p(p_logits), _p(q_logits), float(tau), _p(u),
                                 _p(n_acc), _p(nxt), _p(mg))
    if rc:
        raise ValueError("oracle_mtp_accept failed: %d" % rc)
    return n_acc, nxt, mg

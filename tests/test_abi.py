"""The C ABI library without a GPU: it loads, exports what include/moe.h
declares, sizes workspaces, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def m():
    from quantized_moe_noaux_amd import moe
    return moe


def test_header_declares_the_boundary():
    names = header_functions()
    for f in ("moe_route", "moe_quant_act", "moe_expert_ffn", "moe_layer_forward", "moe_workspace_bytes",
              "moe_rmsnorm", "moe_block_dots", "moe_permute", "moe_strerror"):
        assert f in names


def test_library_exports_every_declared_symbol(m):
    lib = ctypes.CDLL(m.lib.path)
    missing = [f for f in header_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_strerror(m):
    assert m.strerror(0) == "success"
    assert m.strerror(m.MOE_EWORKSPACE) == "workspace too small"
    assert m.strerror(99) == "unknown error"


def big_shape(m, **kw):
    d = dict(hidden=6144, inter=2048, n_experts=256, n_group=8, topk_group=4, top_k=8, n_shared=1,
             wbits=4, rsf=2.5)
    d.update(kw)
    return m.shape(**d)


def test_workspace_sizes(m):
    sh = big_shape(m)
    ws1 = m.moe_workspace_bytes(sh, 1)
    assert ws1 > 0 and ws1 % 256 == 0
    assert m.moe_workspace_bytes(sh, 3) > ws1
    # fp64 partial logits of the K-split router (8 slices at this size)
    assert m.moe_route_workspace_bytes(sh, 2048) == 8 * 2048 * 256 * 8
    assert m.moe_route_workspace_bytes(sh, 8) == 8 * 256 * 8
    assert m.moe_workspace_bytes(big_shape(m, wbits=3), 1) == 0          # unsupported shape
    assert m.moe_workspace_bytes(big_shape(m, n_group=7), 1) == 0        # E % G != 0
    assert m.moe_permute_workspace_bytes(2048, 8, 256) == 64 * 256 * 4


def test_stage_count(m):
    sh = big_shape(m)
    # one token: router+quant, gate/up (which routes the token itself), down
    assert m.moe_layer_stage_count(sh, 1) == 3
    assert m.moe_layer_stage_count(big_shape(m, wbits=2), 1) == 3
    # a row width without a row-sweep kernel keeps the plan launch
    assert m.moe_layer_stage_count(big_shape(m, hidden=4096), 1) == 4
    assert m.moe_layer_stage_count(sh, 2) == 4          # router+quant, plan, gate/up, down
    assert m.moe_layer_stage_count(sh, 0) == 0
    assert m.moe_layer_stage_count(big_shape(m, top_k=40), 1) < 0
    # grouped path: logits, top-k, quant, permute, gate/up, down, combine
    assert m.moe_layer_stage_count(sh, 2048) == 7
    assert m.moe_layer_stage_count(sh, 1, m.MOE_PATH_GROUPED) == 7
    assert m.moe_layer_stage_count(sh, 2048, m.MOE_PATH_GEMV) == 2 + 3 * 256  # chunks of 8 tokens
    assert m.moe_layer_stage_count(sh, 1, 3) < 0


def test_top_p_shape_and_path(m):
    # the shape struct carries routed_top_p at the end, as include/moe.h lays it out
    assert ctypes.sizeof(m.moe_shape_t) == 9 * 4 + 4
    sh = big_shape(m)
    sh.routed_top_p = 0.7
    # both paths take top-p; the workspace and stages do not change
    assert m.moe_layer_stage_count(sh, 2048) == 7
    assert m.moe_layer_stage_count(sh, 1) == 3
    sh0 = big_shape(m)
    assert m.moe_workspace_bytes(sh, 2048) == m.moe_workspace_bytes(sh0, 2048)
    assert m.moe_workspace_bytes(sh, 1) == m.moe_workspace_bytes(sh0, 1)
    for bad in (-0.1, float("nan")):
        sh.routed_top_p = bad
        assert m.moe_layer_stage_count(sh, 1) < 0
    for off in (0.0, 1.0, 2.0):                         # off: the plain selection and paths
        sh.routed_top_p = off
        assert m.moe_layer_stage_count(sh, 2048) == 7


def test_grouped_workspace(m):
    sh = big_shape(m)
    G = m.MOE_PATH_GROUPED
    ws = m.moe_workspace_bytes(sh, 2048)                 # AUTO -> grouped
    assert ws == m.moe_workspace_bytes(sh, 2048, G)
    rows = 2048 * 9
    assert ws > rows * 6144 * 4 + rows * 2048            # expert outputs + int8 h
    assert ws % 256 == 0
    assert m.moe_workspace_bytes(sh, 1, G) > 0
    assert m.moe_workspace_bytes(big_shape(m, hidden=6080), 2048, G) == 0   # 6080 % 256 != 0
    # AUTO falls back to the GEMV path where the grouped kernels do not fit
    assert m.moe_workspace_bytes(big_shape(m, hidden=6080), 2048) > 0


NULL = None


def call_layer(m, sh, T=1, flags=0, ws_bytes=1 << 20, x=1 << 12, y=2 << 12, shared=True, gate_w=3 << 12,
               bias=4 << 12):
    w = m.moe_weights_t(16, 32, 48, 64, 80, 96)
    sw = m.moe_weights_t(16, 32, 48, 64, 80, 96) if shared else None
    return m.lib.moe_layer_forward(ctypes.byref(sh), x, T, gate_w, bias, ctypes.byref(w),
                                   ctypes.byref(sw) if sw else None, y, None, None, flags, 1 << 20,
                                   ws_bytes, None)


def test_layer_argument_errors_launch_nothing(m):
    sh = big_shape(m)
    assert call_layer(m, sh, T=-1) == m.MOE_EINVAL
    assert call_layer(m, sh, ws_bytes=16) == m.MOE_EWORKSPACE
    assert call_layer(m, sh, x=0) == m.MOE_EINVAL
    assert call_layer(m, sh, x=(1 << 12) + 4) == m.MOE_EINVAL              # x not 16-byte aligned
    assert call_layer(m, sh, x=1 << 12, y=1 << 12) == m.MOE_EINVAL         # y aliases x
    assert call_layer(m, sh, shared=False) == m.MOE_EINVAL                 # n_shared = 1 needs it
    assert call_layer(m, sh, flags=3) == m.MOE_EINVAL
    assert call_layer(m, sh, flags=1 << 20) == m.MOE_EINVAL
    assert call_layer(m, big_shape(m, wbits=3)) == m.MOE_EUNSUPPORTED
    assert call_layer(m, big_shape(m, n_shared=2)) == m.MOE_EUNSUPPORTED
    assert call_layer(m, big_shape(m, hidden=6000)) == m.MOE_EINVAL       # not a multiple of 32
    assert call_layer(m, big_shape(m, top_k=33, topk_group=8)) == m.MOE_EUNSUPPORTED
    assert call_layer(m, big_shape(m, n_experts=1024, n_group=8)) == m.MOE_EUNSUPPORTED
    assert call_layer(m, sh, T=0) == m.MOE_OK                               # no-op
    assert call_layer(m, big_shape(m, hidden=6080), flags=m.MOE_PATH_GROUPED) == m.MOE_EUNSUPPORTED
    assert call_layer(m, sh, T=2048, ws_bytes=1 << 20) == m.MOE_EWORKSPACE  # grouped sizes


def test_other_entry_point_errors(m):
    L = m.lib
    assert L.moe_quant_act(1 << 12, 4, 48, 2 << 12, 3 << 12, None) == m.MOE_EINVAL   # D % 32
    assert L.moe_quant_act(None, 4, 64, 2 << 12, 3 << 12, None) == m.MOE_EINVAL
    assert L.moe_quant_act(None, 0, 64, None, None, None) == m.MOE_OK
    assert L.moe_block_dots(3, 1 << 12, 4, 64, 2 << 12, 1, 3 << 12, None) == m.MOE_EUNSUPPORTED
    assert L.moe_block_dots(2, 1 << 12, 4, 32, 2 << 12, 1, 3 << 12, None) == m.MOE_EUNSUPPORTED  # 8-byte rows
    assert L.moe_rmsnorm(1 << 12, 2 << 12, -1.0, 1, 64, 3 << 12, None) == m.MOE_EINVAL
    sh = big_shape(m)
    assert L.moe_route(ctypes.byref(sh), 1 << 12, 1, 2 << 12, 3 << 12, 4 << 12, 5 << 12, 1 << 20, 8,
                       None) == m.MOE_EWORKSPACE
    w = m.moe_weights_t(16, 32, 48, 64, 80, 96)
    assert L.moe_expert_ffn(ctypes.byref(sh), ctypes.byref(w), 256, 1 << 12, 2 << 12, 1, 3 << 12,
                            1 << 20, 1 << 30, None) == m.MOE_EINVAL      # expert out of range
    assert L.moe_permute(1 << 12, 4, 8, 600, 1 << 13, 1 << 14, 1 << 15, 1 << 20, 1 << 20,
                         None) == m.MOE_EUNSUPPORTED


def test_mtp_accept_argument_checks(m):
    """moe_mtp_accept rejects bad arguments before any launch (no GPU)."""
    L = m.lib
    P, Q, U, N, X, D_, WS = (k << 16 for k in range(1, 8))
    need = L.moe_mtp_accept_workspace_bytes(2, 4, 320000)
    assert need >= 16 * 2 * 9 * 79 + 16 * 2 * 79 and need % 256 == 0
    assert L.moe_mtp_accept_workspace_bytes(-1, 4, 10) == 0
    assert L.moe_mtp_accept(-1, 4, 100, D_, P, Q, 0.7, U, N, X, WS, need, None) == m.MOE_EINVAL
    assert L.moe_mtp_accept(2, 4, 0, D_, P, Q, 0.7, U, N, X, WS, need, None) == m.MOE_EINVAL
    assert L.moe_mtp_accept(2, 4, 100, D_, P, Q, -0.5, U, N, X, WS, need, None) == m.MOE_EINVAL
    assert L.moe_mtp_accept(2, 4, 100, D_, P, Q, float("nan"), U, N, X, WS, need, None) == m.MOE_EINVAL
    assert L.moe_mtp_accept(2, 17, 100, D_, P, Q, 0.7, U, N, X, WS, need, None) == m.MOE_EUNSUPPORTED
    assert L.moe_mtp_accept(2, 4, 4096 * 256 + 1, D_, P, Q, 0.7, U, N, X, WS, 1 << 40, None) == m.MOE_EUNSUPPORTED
    assert L.moe_mtp_accept(2, 4, 100, None, P, Q, 0.7, U, N, X, WS, need, None) == m.MOE_EINVAL
    assert L.moe_mtp_accept(2, 4, 100, D_, P, None, 0.7, U, N, X, WS, need, None) == m.MOE_EINVAL
    assert L.moe_mtp_accept(2, 4, 100, D_, P + 2, Q, 0.7, U, N, X, WS, need, None) == m.MOE_EINVAL  # misaligned
    assert L.moe_mtp_accept(2, 4, 320000, D_, P, Q, 0.7, U, N, X, WS, need - 1, None) == m.MOE_EWORKSPACE
    assert L.moe_mtp_accept(0, 4, 100, None, None, None, 0.7, None, None, None, None, 0, None) == m.MOE_OK


def test_stack_lookahead_workspace_and_flag(m):
    """MOE_LOOKAHEAD(n) adds the predicted logits (E fp64) and one sink word
    per wave of the n (k + 1) lookahead workgroups (4 words each), each part
    256-byte aligned; the helper refuses n outside 0 .. 63."""
    sh = big_shape(m)
    base = m.moe_stack_workspace_bytes(sh, 1)
    for n in (1, 8, 32, 63):
        got = m.moe_stack_workspace_bytes(sh, 1, m.MOE_LOOKAHEAD(n))
        sink = 4 * 4 * n * (8 + 1)
        assert got == base + 256 * 8 + (sink + 255) // 256 * 256
    assert m.moe_stack_workspace_bytes(sh, 1, m.MOE_LOOKAHEAD(0)) == base
    for bad in (-1, 64):
        with pytest.raises(ValueError):
            m.MOE_LOOKAHEAD(bad)


def test_stream_read_rejects_misuse_before_any_launch(m):
    f = m.lib.moe_stream_read
    assert f(None, 16, None, None) == m.MOE_EINVAL
    assert f(ctypes.c_void_p(16), 20, ctypes.c_void_p(16), None) == m.MOE_EINVAL   # not a multiple of 16
    assert f(ctypes.c_void_p(20), 16, ctypes.c_void_p(16), None) == m.MOE_EINVAL   # misaligned source
    assert f(None, 0, None, None) == m.MOE_OK                                       # nothing to read

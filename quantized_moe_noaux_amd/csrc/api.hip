// extern "C" entry points of libmoe: argument checks, workspace layout and
// the launch sequences.  Declarations and contracts: include/moe.h.
#include "moe_internal.h"

#include <algorithm>
#include <vector>

using namespace moe;

namespace {

bool al(const void *p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Router-level checks (all that moe_route needs).
int check_router_shape(const moe_shape_t *s)
{
    if (!s) return MOE_EINVAL;
    if (s->hidden <= 0 || s->inter <= 0 || s->hidden % 32 || s->inter % 32) return MOE_EINVAL;
    if (s->n_experts <= 0 || s->n_group <= 0 || s->n_experts % s->n_group) return MOE_EINVAL;
    if (s->topk_group < 1 || s->topk_group > s->n_group) return MOE_EINVAL;
    if (s->top_k < 1 || s->top_k > s->topk_group * (s->n_experts / s->n_group)) return MOE_EINVAL;
    if (s->n_shared < 0) return MOE_EINVAL;
    if (!(s->routed_scaling_factor == s->routed_scaling_factor)) return MOE_EINVAL;  // NaN
    if (!(s->routed_top_p >= 0.f)) return MOE_EINVAL;                                 // negative or NaN
    if (s->n_experts > kMaxExperts || s->n_group > kMaxGroups || s->top_k > kMaxTopK) return MOE_EUNSUPPORTED;
    RouteCfg rc;
    if (!route_cfg(*s, rc)) return MOE_EUNSUPPORTED;
    return MOE_OK;
}

// Full layer checks: router plus the expert weight layout.
int check_shape(const moe_shape_t *s)
{
    int rc = check_router_shape(s);
    if (rc) return rc;
    if (s->wbits != 2 && s->wbits != 4 && s->wbits != 8) return MOE_EUNSUPPORTED;
    if (s->n_shared > 1) return MOE_EUNSUPPORTED;
    ChunkCfg cc;
    if (!chunk_cfg(s->hidden, s->wbits, cc) || !chunk_cfg(s->inter, s->wbits, cc)) return MOE_EUNSUPPORTED;
    return MOE_OK;
}

int check_weights(const moe_weights_t *w)
{
    if (!w || !w->gate || !w->up || !w->down || !w->gate_s || !w->up_s || !w->down_s) return MOE_EINVAL;
    if (!al(w->gate, 16) || !al(w->up, 16) || !al(w->down, 16)) return MOE_EINVAL;
    if (!al(w->gate_s, 4) || !al(w->up_s, 4) || !al(w->down_s, 4)) return MOE_EINVAL;
    return MOE_OK;
}

inline int hip_rc(int e) { return e ? MOE_EHIP : MOE_OK; }

size_t route_ws(const moe_shape_t &s, int T) { return align256(router_logit_bytes(s, T)); }

// The stage list of the GEMV path for T tokens: the router / quantiser
// launch(es), then (plan, gate/up, down) for every chunk of Tc tokens; a
// token routed inside the gate/up launch has no plan launch.
int gemv_stage_count(const moe_shape_t &s, int T, int Tc)
{
    if (gemv_inline_route(s, T)) return 3;
    return (T <= kGemvMaxT ? 1 : 2) + 3 * ((T + Tc - 1) / Tc);
}

// The grouped path's stages: router logits, top-k, quantiser, permutation
// (three launches), gate/up, down, combine.
constexpr int kGgStages = 7;

// Which path serves a call: GEMV / GROUPED as asked; AUTO takes the grouped
// path above kGemvMaxT tokens when its kernels take the shape.
bool use_grouped(const moe_shape_t &s, int T, uint32_t flags)
{
    const uint32_t path = flags & 3u;
    if (path == MOE_PATH_GROUPED) return true;
    if (path == MOE_PATH_GEMV) return false;
    return T > kGemvMaxT && gg_shape_ok(s);
}

// moe_layer_forward on the expert-grouped path (arguments already checked)
int layer_grouped(const moe_shape_t &s, const float *x, int T, const float *gate_w, const float *bias,
                  const moe_weights_t &routed, const moe_weights_t *shared, float *y, int32_t *idx_out,
                  float *w_out, uint32_t flags, void *ws, size_t ws_bytes, hipStream_t st)
{
    const GgWs L = gg_ws(s, T);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    const uint32_t sel = (flags & MOE_STAGE_MASK) >> 8;
    auto run = [&](int stage) { return sel == 0 || ((sel >> stage) & 1u); };
    char *base = static_cast<char *>(ws);
    auto at = [&](size_t o) { return static_cast<void *>(base + o); };
    const int H = s.hidden, E = s.n_experts, k = s.top_k;
    RouteCfg rc;
    route_cfg(s, rc);
    double *logits = static_cast<double *>(at(L.logits));
    int32_t *idx = idx_out ? idx_out : static_cast<int32_t *>(at(L.idx));
    float *w = w_out ? w_out : static_cast<float *>(at(L.w));
    GgArgs a{};
    a.T = T; a.H = H; a.I = s.inter; a.E = E; a.k = k; a.n_shared = s.n_shared; a.wbits = s.wbits;
    a.Tk = T * k;
    a.tiles = static_cast<const int4 *>(at(L.tiles));
    a.perm = static_cast<const int32_t *>(at(L.perm));
    a.inv = static_cast<const int32_t *>(at(L.inv));
    a.w = w;
    a.routed = routed;
    if (shared) a.shared = *shared;
    a.xq = static_cast<const int8_t *>(at(L.xq));
    a.xd = static_cast<const float *>(at(L.xd));
    a.qh = static_cast<int8_t *>(at(L.qh));
    a.dh = static_cast<float *>(at(L.dh));
    a.yrows = static_cast<float *>(at(L.y));
    a.y = y;
    a.accumulate = (flags & MOE_ACCUMULATE) ? 1 : 0;
    const int max_tiles = gg_max_tiles(s, T);
    const int ksplit = router_ksplit(T, H, E);
    if (run(0) && launch_router_logits_mfma(x, T, H, gate_w, E, ksplit, logits, st)) return MOE_EHIP;
    if (run(1) && launch_topk(rc, logits, ksplit, bias, T, idx, w, st)) return MOE_EHIP;
    if (run(2) && launch_gg_quant(x, T, H, s.wbits, const_cast<int8_t *>(a.xq), const_cast<float *>(a.xd), st))
        return MOE_EHIP;
    if (run(3) && launch_permute(idx, T, k, E, const_cast<int32_t *>(a.perm), static_cast<int32_t *>(at(L.off)),
                                 const_cast<int32_t *>(a.inv), static_cast<int32_t *>(at(L.pscr)),
                                 const_cast<int4 *>(a.tiles), s.n_shared, st))
        return MOE_EHIP;
    if (run(4) && launch_gg_gate_up(a, max_tiles, st)) return MOE_EHIP;
    if (run(5) && launch_gg_down(a, max_tiles, st)) return MOE_EHIP;
    if (run(6) && launch_gg_combine(a, st)) return MOE_EHIP;
    return MOE_OK;
}

} // namespace

extern "C" {

const char *moe_strerror(int code)
{
    switch (code) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or parameter";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failed";
    case MOE_ESCRATCH: return "call exceeds the fixed scratch buffer of moe_layer_forward_noalloc";
    default: return "unknown error";
    }
}

size_t moe_route_workspace_bytes(const moe_shape_t *shape, int32_t T)
{
    if (check_router_shape(shape) || T < 0) return 0;
    return route_ws(*shape, T);
}

int moe_route(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w, const float *bias,
              int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int rc = check_router_shape(shape);
    if (rc) return rc;
    if (T < 0) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !gate_w || !bias || !topk_idx || !topk_w || !ws) return MOE_EINVAL;
    if (!al(x, 16) || !al(gate_w, 16) || !al(ws, 256)) return MOE_EINVAL;
    if (ws_bytes < route_ws(*shape, T)) return MOE_EWORKSPACE;
    RouteCfg rcfg;
    route_cfg(*shape, rcfg);
    double *logits = static_cast<double *>(ws);
    const int ksplit = router_ksplit(T, shape->hidden, shape->n_experts);
    int e = (T <= kGemvMaxT)
                ? launch_router_logits(x, T, shape->hidden, gate_w, shape->n_experts, logits, nullptr, nullptr,
                                       nullptr, 0.0, stream)
                : launch_router_logits_mfma(x, T, shape->hidden, gate_w, shape->n_experts, ksplit, logits, stream);
    if (e) return MOE_EHIP;
    return hip_rc(launch_topk(rcfg, logits, ksplit, bias, T, topk_idx, topk_w, stream));
}

int moe_quant_act(const float *x, int32_t T, int32_t D, int8_t *q, float *d, hipStream_t stream)
{
    if (T < 0 || D <= 0 || D % 32) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !q || !d || !al(x, 16) || !al(q, 4) || !al(d, 4)) return MOE_EINVAL;
    return hip_rc(launch_quant(x, T, D, q, d, stream));
}

int moe_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (bytes % 16) return MOE_EINVAL;
    if (bytes == 0) return MOE_OK;
    if (!src || !sink || !al(src, 16) || !al(sink, 4)) return MOE_EINVAL;
    return hip_rc(launch_stream_read(src, bytes, sink, stream));
}

int moe_block_dots(int32_t wbits, const uint8_t *codes, int32_t rows, int32_t D, const int8_t *q, int32_t T,
                   int32_t *out, hipStream_t stream)
{
    if (wbits != 2 && wbits != 4 && wbits != 8) return MOE_EUNSUPPORTED;
    if (rows < 0 || T < 0 || D <= 0 || D % 32) return MOE_EINVAL;
    if ((D * wbits / 8) % 16) return MOE_EUNSUPPORTED;
    if (T == 0 || rows == 0) return MOE_OK;
    if (!codes || !q || !out || !al(codes, 16) || !al(q, 16)) return MOE_EINVAL;
    return hip_rc(launch_block_dots(wbits, codes, rows, D, q, T, out, stream));
}

size_t moe_workspace_bytes(const moe_shape_t *shape, int32_t T, uint32_t flags)
{
    if (check_shape(shape) || T < 0 || (flags & 3u) == 3u) return 0;
    if (use_grouped(*shape, T, flags)) return gg_shape_ok(*shape) ? gg_ws(*shape, T > 0 ? T : 1).total : 0;
    const int Tc = gemv_chunk_tokens(*shape, T > 0 ? T : 1);
    if (!Tc) return 0;
    return gemv_ws(*shape, T, Tc, false).total;
}

int moe_layer_stage_count(const moe_shape_t *shape, int32_t T, uint32_t flags)
{
    if (check_shape(shape) || T < 0) return -MOE_EINVAL;
    if (T == 0) return 0;
    if ((flags & 3u) == 3u) return -MOE_EINVAL;
    if (use_grouped(*shape, T, flags)) return gg_shape_ok(*shape) ? kGgStages : -MOE_EUNSUPPORTED;
    const int Tc = gemv_chunk_tokens(*shape, T);
    if (!Tc) return -MOE_EUNSUPPORTED;
    return gemv_stage_count(*shape, T, Tc);
}

int moe_expert_ffn(const moe_shape_t *shape, const moe_weights_t *w, int32_t expert, const int8_t *q,
                   const float *d, int32_t T, float *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_weights(w))) return rc;
    if (T < 0 || expert < 0 || expert >= shape->n_experts) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!q || !d || !y || !ws || !al(q, 16) || !al(d, 4) || !al(y, 4) || !al(ws, 256)) return MOE_EINVAL;
    // single-expert mode stages at most Tc tokens per chunk, like the layer
    const int Tc = gemv_chunk_tokens(*shape, T);
    if (!Tc) return MOE_EUNSUPPORTED;
    const GemvWs L = gemv_ws(*shape, T, Tc, true);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    char *base = static_cast<char *>(ws);
    const int H = shape->hidden, nb = H / 32;
    for (int c0 = 0; c0 < T; c0 += Tc) {
        GemvArgs a{};
        a.T = (T - c0 < Tc) ? T - c0 : Tc;
        a.H = H; a.I = shape->inter; a.E = shape->n_experts; a.wbits = shape->wbits; a.n_shared = 0;
        route_cfg(*shape, a.rc);
        a.logits = nullptr; a.bias = nullptr; a.single = expert;
        a.routed = *w; a.shared = *w;
        a.xq = q + (size_t)c0 * H; a.xd = d + (size_t)c0 * nb;
        a.plan = reinterpret_cast<int *>(base + L.plan);
        a.qh = reinterpret_cast<int8_t *>(base + L.qh);
        a.dh = reinterpret_cast<float *>(base + L.dh);
        a.y = y + (size_t)c0 * H;
        a.accumulate = 0;
        if (launch_plan(a, stream) || launch_gate_up(a, stream) || launch_down(a, stream)) return MOE_EHIP;
    }
    return MOE_OK;
}

// The next layer of a decode stack, for the router lookahead: its router
// weights, norm weight, correction bias and experts, the workgroups per
// prefetched expert, and workspace for its predicted logits and the sink.
struct Lookahead {
    const float *gate_w, *ng, *bias;
    moe_weights_t routed, shared;
    int wgs;
    double *logits;
    uint32_t *sink;
};

static int layer_gemv(const moe_shape_t &sh, const float *x, int T, const float *gate_w, const float *bias,
                      const moe_weights_t *routed, const moe_weights_t *shared, float *y, int32_t *idx_out,
                      float *w_out, uint32_t flags, void *ws, size_t ws_bytes, const float *ng, double eps,
                      hipStream_t stream, const int64_t *toff = nullptr, uint32_t *counts = nullptr,
                      const Lookahead *la = nullptr);

int moe_layer_forward(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w, const float *bias,
                      const moe_weights_t *routed, const moe_weights_t *shared, float *y, int32_t *idx_out,
                      float *w_out, uint32_t flags, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_weights(routed))) return rc;
    if (shape->n_shared && (rc = check_weights(shared))) return rc;
    if (!shape->n_shared && shared) return MOE_EINVAL;
    if (T < 0) return MOE_EINVAL;
    if (flags & ~(3u | MOE_ACCUMULATE | MOE_STAGE_MASK)) return MOE_EINVAL;
    const uint32_t path = flags & 3u;
    if (path == 3u) return MOE_EINVAL;
    if (path == MOE_PATH_GROUPED && !gg_shape_ok(*shape)) return MOE_EUNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !gate_w || !bias || !y || !ws) return MOE_EINVAL;
    if ((idx_out == nullptr) != (w_out == nullptr)) return MOE_EINVAL;
    if (!al(x, 16) || !al(gate_w, 16) || !al(y, 4) || !al(ws, 256)) return MOE_EINVAL;
    if (x == y) return MOE_EINVAL;
    if (use_grouped(*shape, T, flags))
        return layer_grouped(*shape, x, T, gate_w, bias, *routed, shared, y, idx_out, w_out, flags, ws, ws_bytes,
                             stream);
    return layer_gemv(*shape, x, T, gate_w, bias, routed, shared, y, idx_out, w_out, flags, ws, ws_bytes, nullptr,
                      0.0, stream);
}

// moe_layer_forward on the GEMV path (arguments already checked).  With
// ng != nullptr the layer input is RMSNorm(x) with weight ng, formed by the
// router launch (router_norms_input must hold); y may then be x itself with
// MOE_ACCUMULATE, since x is read by the router launch only.  With la (one
// token, routed inside the gate/up launch, ng given) the router launch also
// computes the next layer's logits on the same input and the gate/up launch
// prefetches the experts they select; the layer's results do not change.
static int layer_gemv(const moe_shape_t &sh, const float *x, int T, const float *gate_w, const float *bias,
                      const moe_weights_t *routed, const moe_weights_t *shared, float *y, int32_t *idx_out,
                      float *w_out, uint32_t flags, void *ws, size_t ws_bytes, const float *ng, double eps,
                      hipStream_t stream, const int64_t *toff, uint32_t *counts, const Lookahead *la)
{
    const moe_shape_t *shape = &sh;
    if (shape->hidden % kGemvDownRows) return MOE_EUNSUPPORTED;
    const int Tc = gemv_chunk_tokens(*shape, T);
    if (!Tc) return MOE_EUNSUPPORTED;
    const GemvWs L = gemv_ws(*shape, T, Tc, false);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    const int nstages = gemv_stage_count(*shape, T, Tc);
    const uint32_t sel = (flags & MOE_STAGE_MASK) >> 8;
    if (sel && nstages > 8) return MOE_EINVAL;
    auto run = [&](int s) { return sel == 0 || ((sel >> s) & 1u); };

    char *base = static_cast<char *>(ws);
    double *logits = reinterpret_cast<double *>(base + L.logits);
    int8_t *xq = reinterpret_cast<int8_t *>(base + L.xq);
    float *xd = reinterpret_cast<float *>(base + L.xd);
    const int H = shape->hidden, nb = H / 32, E = shape->n_experts, k = shape->top_k;
    const int ksplit = router_ksplit(T, H, E);
    auto args = [&](int c0, int tc) {
        GemvArgs a{};
        a.T = tc;
        a.H = H; a.I = shape->inter; a.E = E; a.wbits = shape->wbits; a.n_shared = shape->n_shared;
        route_cfg(*shape, a.rc);
        a.logits = logits + (size_t)c0 * E; a.bias = bias; a.single = -1;
        a.lstride = (size_t)T * E; a.lparts = ksplit;
        a.routed = *routed;
        if (shared) a.shared = *shared;
        a.xq = xq + (size_t)c0 * H; a.xd = xd + (size_t)c0 * nb;
        a.plan = reinterpret_cast<int *>(base + L.plan);
        a.qh = reinterpret_cast<int8_t *>(base + L.qh);
        a.dh = reinterpret_cast<float *>(base + L.dh);
        a.y = y + (size_t)c0 * H;
        a.idx_out = idx_out ? idx_out + (size_t)c0 * k : nullptr;
        a.w_out = w_out ? w_out + (size_t)c0 * k : nullptr;
        a.accumulate = (flags & MOE_ACCUMULATE) ? 1 : 0;
        a.toff = toff;
        a.counts = counts;
        return a;
    };
    const bool here = gemv_inline_route(*shape, T);
    if (la && (!here || !ng || toff || la->wgs <= 0)) la = nullptr;
    int stage = 0;
    if (T <= kGemvMaxT) {
        if (run(stage) && launch_router_logits(x, T, H, gate_w, E, logits, xq, xd, ng, eps, stream,
                                               la ? la->gate_w : nullptr, la ? la->ng : nullptr,
                                               la ? la->logits : nullptr))
            return MOE_EHIP;
        stage++;
    } else {
        if (ng) return MOE_EINVAL;
        if (run(stage) && launch_router_logits_mfma(x, T, H, gate_w, E, ksplit, logits, stream)) return MOE_EHIP;
        stage++;
        if (run(stage) && launch_quant(x, T, H, xq, xd, stream)) return MOE_EHIP;
        stage++;
    }
    for (int c0 = 0; c0 < T; c0 += Tc) {
        GemvArgs a = args(c0, (T - c0 < Tc) ? T - c0 : Tc);
        a.inline_route = here ? 1 : 0;
        if (la) {
            a.la_logits = la->logits; a.la_bias = la->bias;
            a.la_routed = la->routed; a.la_shared = la->shared;
            a.la_wgs = la->wgs; a.la_sink = la->sink;
        }
        if (!here) {
            if (run(stage) && launch_plan(a, stream)) return MOE_EHIP;
            stage++;
        }
        if (run(stage) && launch_gate_up(a, stream)) return MOE_EHIP;
        stage++;
        if (run(stage) && launch_down(a, stream)) return MOE_EHIP;
        stage++;
    }
    return MOE_OK;
}

// ---------------------------------------------------------------- expert tier
} // extern "C"

// prefetch slots per tier (router lookahead)
constexpr int kTierPrefetch = 16;

struct moe_tier {
    moe_shape_t shape;
    int E, C;
    size_t bytes[6];        // one expert's gate, up, down codes and their scales
    uintptr_t hdev[6];      // device addresses of the pinned host stacks
    const uint8_t *hsrc[6]; // host addresses of the same stacks (copy sources)
    uint8_t *pool[6];       // HBM slots [C][expert bytes]
    moe_weights_t base;     // the base pointers the table's offsets refer to
    int64_t *dtab, *htab;   // expert table (device) and its pinned host mirror
    uint32_t *dcounts, *hcounts;
    std::vector<int> slot_of, expert_in;
    // prefetch slots (a ring): experts brought in ahead of use by the
    // router lookahead, apart from the pinned slots
    int P = 0, pnext = 0;
    uint8_t *ppool[6] = {};
    std::vector<int> pslot_of, pexpert;
    // the last host-to-device copy of the table's host mirror: the mirror
    // is changed only once it has completed
    hipEvent_t uploaded = nullptr;
};

namespace {

void tier_free(moe_tier *t)
{
    for (int i = 0; i < 6; i++) {
        if (t->pool[i]) (void)hipFree(t->pool[i]);
        if (t->ppool[i]) (void)hipFree(t->ppool[i]);
    }
    if (t->uploaded) (void)hipEventDestroy(t->uploaded);
    if (t->dtab) (void)hipFree(t->dtab);
    if (t->dcounts) (void)hipFree(t->dcounts);
    if (t->htab) (void)hipHostFree(t->htab);
    if (t->hcounts) (void)hipHostFree(t->hcounts);
    delete t;
}

uintptr_t base_addr(const moe_tier *t, int i)
{
    const void *p = i == 0 ? (const void *)t->base.gate : i == 1 ? (const void *)t->base.up
                  : i == 2 ? (const void *)t->base.down : i == 3 ? (const void *)t->base.gate_s
                  : i == 4 ? (const void *)t->base.up_s : (const void *)t->base.down_s;
    return (uintptr_t)p;
}

// the host mirror's entry of expert e: its pinned slot, else its prefetch
// slot, else the host stack
void tier_entry(moe_tier *t, int e)
{
    const int s = t->slot_of[e], q = t->pslot_of[e];
    for (int i = 0; i < 6; i++) {
        const uintptr_t a = (s >= 0)   ? (uintptr_t)t->pool[i] + (uintptr_t)s * t->bytes[i]
                            : (q >= 0) ? (uintptr_t)t->ppool[i] + (uintptr_t)q * t->bytes[i]
                                       : t->hdev[i] + (uintptr_t)e * t->bytes[i];
        t->htab[(size_t)e * 6 + i] = (int64_t)(a - base_addr(t, i));
    }
}

// the table's host mirror (and the host counts) may change: their last
// upload has completed
int tier_mirror_free(moe_tier *t)
{
    return hipEventSynchronize(t->uploaded) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int tier_upload(moe_tier *t, hipStream_t stream)
{
    if (hipMemcpyAsync(t->dtab, t->htab, sizeof(int64_t) * 6 * t->E, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipEventRecord(t->uploaded, stream) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

// experts by (count desc, index asc)
std::vector<int> by_count(const uint32_t *c, int E)
{
    std::vector<int> o(E);
    for (int e = 0; e < E; e++) o[e] = e;
    std::stable_sort(o.begin(), o.end(), [&](int a, int b) { return c[a] > c[b]; });
    return o;
}

} // namespace

extern "C" {

int moe_tier_plan(const uint32_t *heat, int32_t E, int32_t C, const int32_t *slot_in, int32_t *slot_out,
                  int32_t max_swaps)
{
    if (!heat || !slot_in || !slot_out || E <= 0 || C < 0 || C > E || max_swaps < 0) return -MOE_EINVAL;
    std::vector<int> expert_in(C, -1);
    for (int e = 0; e < E; e++) {
        const int s = slot_in[e];
        if (s < -1 || s >= C || (s >= 0 && expert_in[s] >= 0)) return -MOE_EINVAL;
        if (s >= 0) expert_in[s] = e;
        slot_out[e] = s;
    }
    // streamed experts, hottest first (ties: lower index)
    std::vector<int> hot;
    for (int e : by_count(heat, E))
        if (slot_in[e] < 0 && heat[e] > 0) hot.push_back(e);
    size_t h = 0;
    int copies = 0;
    // free slots take the hottest streamed experts, lowest slot first
    for (int s = 0; s < C && h < hot.size(); s++)
        if (expert_in[s] < 0) {
            slot_out[hot[h]] = s;
            expert_in[s] = hot[h++];
            copies++;
        }
    // then up to max_swaps replacements: the hottest streamed expert against
    // the coldest pinned one (ties: higher index), while the first is more
    // than 25% hotter
    std::vector<int> cold;
    for (int s = 0; s < C; s++)
        if (expert_in[s] >= 0 && slot_in[expert_in[s]] >= 0) cold.push_back(expert_in[s]);
    std::stable_sort(cold.begin(), cold.end(),
                     [&](int a, int b) { return heat[a] != heat[b] ? heat[a] < heat[b] : a > b; });
    for (size_t c = 0; c < cold.size() && h < hot.size() && c < (size_t)max_swaps; c++, h++) {
        const int in = hot[h], out = cold[c];
        if (!(4ull * heat[in] > 5ull * heat[out])) break;
        slot_out[in] = slot_out[out];
        slot_out[out] = -1;
        copies++;
    }
    return copies;
}

int moe_tier_create(const moe_shape_t *shape, const moe_weights_t *host, int32_t slots, moe_tier_t **out)
{
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_weights(host))) return rc;
    if (!gemv_table_ok(*shape)) return MOE_EUNSUPPORTED;
    const int E = shape->n_experts;
    if (slots < 0 || slots > E) return MOE_EINVAL;
    moe_tier *t = new moe_tier();
    t->shape = *shape;
    t->E = E;
    t->C = slots;
    const size_t H = shape->hidden, I = shape->inter, cb = H * I * shape->wbits / 8;
    const size_t bytes[6] = {cb, cb, cb, 4 * I, 4 * I, 4 * H};
    const void *hp[6] = {host->gate, host->up, host->down, host->gate_s, host->up_s, host->down_s};
    for (int i = 0; i < 6; i++) {
        t->bytes[i] = bytes[i];
        t->hsrc[i] = static_cast<const uint8_t *>(hp[i]);
        void *d = nullptr;
        if (hipHostGetDevicePointer(&d, const_cast<void *>(hp[i]), 0) != hipSuccess || !d) {
            (void)hipGetLastError();
            tier_free(t);
            return MOE_EINVAL;  // not pinned, device-mapped host memory
        }
        t->hdev[i] = (uintptr_t)d;
        if (slots > 0 && hipMalloc(reinterpret_cast<void **>(&t->pool[i]), bytes[i] * slots) != hipSuccess) {
            tier_free(t);
            return MOE_EHIP;
        }
    }
    const bool hbm = slots > 0;
    t->base.gate = hbm ? t->pool[0] : reinterpret_cast<const uint8_t *>(t->hdev[0]);
    t->base.up = hbm ? t->pool[1] : reinterpret_cast<const uint8_t *>(t->hdev[1]);
    t->base.down = hbm ? t->pool[2] : reinterpret_cast<const uint8_t *>(t->hdev[2]);
    t->base.gate_s = reinterpret_cast<const float *>(hbm ? (uintptr_t)t->pool[3] : t->hdev[3]);
    t->base.up_s = reinterpret_cast<const float *>(hbm ? (uintptr_t)t->pool[4] : t->hdev[4]);
    t->base.down_s = reinterpret_cast<const float *>(hbm ? (uintptr_t)t->pool[5] : t->hdev[5]);
    if (hipMalloc(reinterpret_cast<void **>(&t->dtab), sizeof(int64_t) * 6 * E) != hipSuccess ||
        hipMalloc(reinterpret_cast<void **>(&t->dcounts), sizeof(uint32_t) * E) != hipSuccess ||
        hipHostMalloc(reinterpret_cast<void **>(&t->htab), sizeof(int64_t) * 6 * E, 0) != hipSuccess ||
        hipHostMalloc(reinterpret_cast<void **>(&t->hcounts), sizeof(uint32_t) * E, 0) != hipSuccess) {
        tier_free(t);
        return MOE_EHIP;
    }
    t->slot_of.assign(E, -1);
    t->expert_in.assign(slots, -1);
    t->P = E < kTierPrefetch ? E : kTierPrefetch;
    t->pslot_of.assign(E, -1);
    t->pexpert.assign(t->P, -1);
    for (int i = 0; i < 6; i++)
        if (hipMalloc(reinterpret_cast<void **>(&t->ppool[i]), t->bytes[i] * t->P) != hipSuccess) {
            tier_free(t);
            return MOE_EHIP;
        }
    if (hipEventCreateWithFlags(&t->uploaded, hipEventDisableTiming) != hipSuccess) {
        tier_free(t);
        return MOE_EHIP;
    }
    for (int e = 0; e < E; e++) tier_entry(t, e);
    for (int e = 0; e < E; e++) t->hcounts[e] = 0;
    if (hipMemcpy(t->dtab, t->htab, sizeof(int64_t) * 6 * E, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(t->dcounts, t->hcounts, sizeof(uint32_t) * E, hipMemcpyHostToDevice) != hipSuccess ||
        hipEventRecord(t->uploaded, nullptr) != hipSuccess) {
        tier_free(t);
        return MOE_EHIP;
    }
    *out = t;
    return MOE_OK;
}

void moe_tier_destroy(moe_tier_t *t)
{
    if (t) tier_free(t);
}

// replacements of pinned experts per repin (the four-swap limit)
constexpr int kTierSwaps = 4;

int moe_tier_repin(moe_tier_t *t, int32_t *copied, hipStream_t stream)
{
    if (!t) return MOE_EINVAL;
    const int E = t->E, C = t->C;
    if (copied) *copied = 0;
    // the host counts are overwritten below: the last repin's upload of
    // them (possibly on another stream) must have completed
    if (tier_mirror_free(t)) return MOE_EHIP;
    if (hipMemcpyAsync(t->hcounts, t->dcounts, sizeof(uint32_t) * E, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return MOE_EHIP;
    std::vector<int32_t> next(E);
    const int nc = moe_tier_plan(t->hcounts, E, C, t->slot_of.data(), next.data(), kTierSwaps);
    if (nc < 0) return -nc;
    for (int e = 0; e < E; e++)  // experts leaving HBM first: their entries point to the host again
        if (t->slot_of[e] >= 0 && next[e] < 0) {
            t->expert_in[t->slot_of[e]] = -1;
            t->slot_of[e] = -1;
            tier_entry(t, e);
        }
    for (int e = 0; e < E; e++)
        if (next[e] >= 0 && t->slot_of[e] < 0) {
            const int s = next[e];
            for (int k = 0; k < 6; k++)
                if (hipMemcpyAsync(t->pool[k] + (size_t)s * t->bytes[k], t->hsrc[k] + (size_t)e * t->bytes[k],
                                   t->bytes[k], hipMemcpyHostToDevice, stream) != hipSuccess)
                    return MOE_EHIP;
            t->slot_of[e] = s;
            t->expert_in[s] = e;
            if (t->pslot_of[e] >= 0) {  // a prefetched expert now pinned: its prefetch slot is free
                t->pexpert[t->pslot_of[e]] = -1;
                t->pslot_of[e] = -1;
            }
            tier_entry(t, e);
        }
    for (int e = 0; e < E; e++) t->hcounts[e] >>= 1;  // usage decays by half per repin
    // the counts first: the upload event then covers both host buffers
    if (hipMemcpyAsync(t->dcounts, t->hcounts, sizeof(uint32_t) * E, hipMemcpyHostToDevice, stream) != hipSuccess ||
        tier_upload(t, stream))
        return MOE_EHIP;
    if (copied) *copied = nc;
    return MOE_OK;
}

int moe_tier_prefetch(moe_tier_t *t, const int32_t *experts, int32_t n, int32_t *copied, hipStream_t stream)
{
    if (!t || n < 0 || (n > 0 && !experts)) return MOE_EINVAL;
    if (copied) *copied = 0;
    if (tier_mirror_free(t)) return MOE_EHIP;
    int nc = 0;
    for (int i = 0; i < n && nc < t->P; i++) {
        const int e = experts[i];
        if (e < 0 || e >= t->E || t->slot_of[e] >= 0 || t->pslot_of[e] >= 0) continue;
        const int p = t->pnext;
        t->pnext = (t->pnext + 1) % t->P;
        const int old = t->pexpert[p];
        if (old >= 0) {  // the ring's oldest prefetch goes back to the host stack
            t->pslot_of[old] = -1;
            tier_entry(t, old);
        }
        for (int k = 0; k < 6; k++)
            if (hipMemcpyAsync(t->ppool[k] + (size_t)p * t->bytes[k], t->hsrc[k] + (size_t)e * t->bytes[k],
                               t->bytes[k], hipMemcpyHostToDevice, stream) != hipSuccess)
                return MOE_EHIP;
        t->pexpert[p] = e;
        t->pslot_of[e] = p;
        tier_entry(t, e);
        nc++;
    }
    if (nc && tier_upload(t, stream)) return MOE_EHIP;
    if (copied) *copied = nc;
    return MOE_OK;
}

int moe_tier_resident(const moe_tier_t *t, int32_t *slot_of)
{
    if (!t || !slot_of) return MOE_EINVAL;
    for (int e = 0; e < t->E; e++) slot_of[e] = t->slot_of[e] >= 0 ? t->slot_of[e] : t->pslot_of[e] >= 0 ? -2 : -1;
    return MOE_OK;
}

int moe_tier_counts(const moe_tier_t *t, uint32_t *counts, hipStream_t stream)
{
    if (!t || !counts) return MOE_EINVAL;
    if (hipMemcpyAsync(counts, t->dcounts, sizeof(uint32_t) * t->E, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

int moe_layer_forward_tiered(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w,
                             const float *bias, const moe_tier_t *tier, const moe_weights_t *shared, float *y,
                             int32_t *idx_out, float *w_out, uint32_t flags, void *ws, size_t ws_bytes,
                             hipStream_t stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!tier) return MOE_EINVAL;
    const moe_shape_t &ts = tier->shape;
    if (ts.hidden != shape->hidden || ts.inter != shape->inter || ts.n_experts != shape->n_experts ||
        ts.wbits != shape->wbits)
        return MOE_EINVAL;
    if (shape->n_shared && (rc = check_weights(shared))) return rc;
    if (!shape->n_shared && shared) return MOE_EINVAL;
    if (T < 0) return MOE_EINVAL;
    if (flags & ~(3u | MOE_ACCUMULATE | MOE_STAGE_MASK)) return MOE_EINVAL;
    const uint32_t path = flags & 3u;
    if (path == 3u) return MOE_EINVAL;
    if (path == MOE_PATH_GROUPED || T > kGemvMaxT) return MOE_EUNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !gate_w || !bias || !y || !ws) return MOE_EINVAL;
    if ((idx_out == nullptr) != (w_out == nullptr)) return MOE_EINVAL;
    if (!al(x, 16) || !al(gate_w, 16) || !al(y, 4) || !al(ws, 256)) return MOE_EINVAL;
    if (x == y) return MOE_EINVAL;
    return layer_gemv(*shape, x, T, gate_w, bias, &tier->base, shared, y, idx_out, w_out, flags & ~3u, ws,
                      ws_bytes, nullptr, 0.0, stream, tier->dtab, tier->dcounts);
}

int moe_rmsnorm(const float *x, const float *g, double eps, int32_t T, int32_t H, float *out, hipStream_t stream)
{
    if (T < 0 || H <= 0 || !(eps >= 0.0)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !g || !out) return MOE_EINVAL;
    return hip_rc(launch_rmsnorm(x, g, eps, T, H, out, stream));
}

// the lookahead's part of a stack's workspace: the next layer's logits of
// the one token, then the sink words of its workgroups
static size_t lookahead_bytes(const moe_shape_t &s, uint32_t flags)
{
    const int wgs = (int)((flags & MOE_LOOKAHEAD_MASK) >> 16);
    if (!wgs) return 0;
    return align256(sizeof(double) * s.n_experts) +
           align256(sizeof(uint32_t) * kLookaheadSinkWords * wgs * (s.top_k + (s.n_shared ? 1 : 0)));
}

size_t moe_stack_workspace_bytes(const moe_shape_t *shape, int32_t T, uint32_t flags)
{
    const size_t layer = moe_workspace_bytes(shape, T, flags & 3u);
    if (!layer) return 0;
    return align256(sizeof(float) * (size_t)(T > 0 ? T : 1) * shape->hidden) + lookahead_bytes(*shape, flags) +
           layer;
}

int moe_stack_forward(const moe_shape_t *shape, float *x, int32_t T, const moe_layer_t *layers, int32_t n_layers,
                      double eps, int32_t *idx_out, float *w_out, uint32_t flags, void *ws, size_t ws_bytes,
                      hipStream_t stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (T < 0 || n_layers < 0 || !(eps >= 0.0)) return MOE_EINVAL;
    if (flags & ~(3u | MOE_STAGE_MASK | MOE_LOOKAHEAD_MASK)) return MOE_EINVAL;
    if ((flags & 3u) == 3u) return MOE_EINVAL;
    if ((idx_out == nullptr) != (w_out == nullptr)) return MOE_EINVAL;
    if (T == 0 || n_layers == 0) return MOE_OK;
    if (!x || !layers || !ws || !al(ws, 256)) return MOE_EINVAL;
    for (int l = 0; l < n_layers; l++) {
        const moe_layer_t &L = layers[l];
        if (!L.gate_w || !L.bias || !L.norm_g) return MOE_EINVAL;
        if ((rc = check_weights(&L.routed))) return rc;
        if (shape->n_shared && (rc = check_weights(&L.shared))) return rc;
    }
    const size_t need = moe_stack_workspace_bytes(shape, T, flags);
    if (!need) return MOE_EUNSUPPORTED;
    if (ws_bytes < need) return MOE_EWORKSPACE;
    const size_t nb = align256(sizeof(float) * (size_t)T * shape->hidden);
    const size_t lab = lookahead_bytes(*shape, flags);
    float *n = static_cast<float *>(ws);
    char *lap = static_cast<char *>(ws) + nb;
    void *lws = lap + lab;
    const size_t lws_bytes = ws_bytes - nb - lab;
    const uint32_t lflags = flags & (3u | MOE_STAGE_MASK);
    const size_t tk = (size_t)T * shape->top_k;
    const uint32_t sel = (flags & MOE_STAGE_MASK) >> 8;
    for (int l = 0; l < n_layers; l++) {
        const moe_layer_t &L = layers[l];
        const moe_weights_t *sw = shape->n_shared ? &L.shared : nullptr;
        int32_t *il = idx_out ? idx_out + l * tk : nullptr;
        float *wl = w_out ? w_out + l * tk : nullptr;
        if (!use_grouped(*shape, T, lflags) && T <= kGemvMaxT && router_norms_input(x, L.norm_g, shape->hidden)) {
            // the router launch normalises the residual itself; the layer
            // adds its output to the residual in place
            Lookahead la{};
            const bool look = lab && l + 1 < n_layers && router_norms_input(x, layers[l + 1].norm_g, shape->hidden);
            if (look) {
                const moe_layer_t &N = layers[l + 1];
                la.gate_w = N.gate_w; la.ng = N.norm_g; la.bias = N.bias;
                la.routed = N.routed;
                if (shape->n_shared) la.shared = N.shared;
                la.wgs = (int)((flags & MOE_LOOKAHEAD_MASK) >> 16);
                la.logits = reinterpret_cast<double *>(lap);
                la.sink = reinterpret_cast<uint32_t *>(lap + align256(sizeof(double) * shape->n_experts));
            }
            rc = layer_gemv(*shape, x, T, L.gate_w, L.bias, &L.routed, sw, x, il, wl, lflags | MOE_ACCUMULATE, lws,
                            lws_bytes, L.norm_g, eps, stream, nullptr, nullptr, look ? &la : nullptr);
        } else {
            if ((sel == 0 || (sel & 1u)) && launch_rmsnorm(x, L.norm_g, eps, T, shape->hidden, n, stream))
                return MOE_EHIP;
            rc = moe_layer_forward(shape, n, T, L.gate_w, L.bias, &L.routed, sw, x, il, wl, lflags | MOE_ACCUMULATE,
                                   lws, lws_bytes, stream);
        }
        if (rc) return rc;
    }
    return MOE_OK;
}

size_t moe_permute_workspace_bytes(int32_t T, int32_t k, int32_t E)
{
    if (T < 0 || k <= 0 || E <= 0) return 0;
    const size_t tiles = ((size_t)T * k + 255) / 256;
    return align256(sizeof(int32_t) * (tiles ? tiles : 1) * E);
}

int moe_permute(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *perm, int32_t *off, int32_t *inv,
                void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (T < 0 || k <= 0 || E <= 0) return MOE_EINVAL;
    if (E > kMaxExperts) return MOE_EUNSUPPORTED;
    if (!off || !ws || (T > 0 && (!idx || !perm || !inv))) return MOE_EINVAL;
    if (ws_bytes < moe_permute_workspace_bytes(T, k, E)) return MOE_EWORKSPACE;
    return hip_rc(launch_permute(idx, T, k, E, perm, off, inv, static_cast<int32_t *>(ws), nullptr, 0, stream));
}

size_t moe_mtp_accept_workspace_bytes(int32_t B, int32_t D, int32_t V)
{
    if (B < 0 || D < 0 || V < 1) return 0;
    return mtp_workspace_bytes(B, D, V);
}

int moe_mtp_accept(int32_t B, int32_t D, int32_t V, const int32_t *draft, const float *p_logits,
                   const float *q_logits, float tau, const double *u, int32_t *n_acc, int32_t *next, void *ws,
                   size_t ws_bytes, hipStream_t stream)
{
    if (B < 0 || D < 0 || V < 1 || !(tau >= 0.f) || !(tau < INFINITY)) return MOE_EINVAL;
    if (D > kMtpMaxDraft || mtp_chunks(V) > kMtpMaxChunks) return MOE_EUNSUPPORTED;
    if (B == 0) return MOE_OK;
    if (!p_logits || !u || !n_acc || !next || !ws || (D > 0 && (!draft || !q_logits))) return MOE_EINVAL;
    if (!al(p_logits, 4) || !al(u, 8) || !al(ws, 256) || (D > 0 && !al(q_logits, 4))) return MOE_EINVAL;
    if (ws_bytes < mtp_workspace_bytes(B, D, V)) return MOE_EWORKSPACE;
    return hip_rc(launch_mtp_accept(B, D, V, draft, p_logits, D > 0 ? q_logits : p_logits, (double)tau, u, n_acc,
                                    next, ws, stream));
}

} // extern "C"

// Batch-union GEMV path of the MoE layer (decode and small verify batches).
//
// GeekNews #31297, implemented features: batch-union MoE reads each unique
// expert of a batch once and applies it to every position routed to it; the
// experts are SwiGLU FFNs over int8 / packed int4 / packed int2 codes with
// per-row scales, evaluated as integer dots on Q8_0-style int8 activations.
// wpnews.pro spec table: 8 routed + 1 shared expert per token.
//
// Per chunk of tokens, three launches after the router:
//  k_plan       one workgroup routes the chunk's tokens (fp64 noaux_tc top-k,
//               one wave per token) and publishes the batch-union plan:
//               slots = the union of the selected experts in ascending
//               order, then the shared expert; each slot lists its tokens
//               (pairs) and their combine weights.
//  k_gate_up_*  one workgroup per (slot, 32-row tile) of the intermediate
//               dimension: g = W_gate x, u = W_up x as integer block dots,
//               h = silu(g) * u, h quantised to int8 in blocks of 32 rows
//               (one tile = one block).
//  k_down_*     one workgroup per tile of output rows: for each row, the down
//               rows of all slots dotted with the slots' int8 h, scaled by
//               combine weight x row scale and summed per token in a fixed
//               order.  The combine is fused; no float atomics, so results
//               are run-to-run identical.
// The *_sw ("row-sweep") kernels serve the production shapes; the *_rg
// ("row-group") kernels take any other shape the ABI accepts.  A single
// token on the row-sweep kernels has no plan launch: its gate/up workgroups
// run the selection themselves (slot u as far as rank u) while the shared
// expert's workgroups, which need no routing, already stream their rows.
#include "moe_dev.h"
#include "moe_internal.h"
#include "slot_record.h"
#include "topk_dev.h"

namespace moe {

bool chunk_cfg(int in_dim, int wbits, ChunkCfg &cc)
{
    const int rowbytes = in_dim * wbits / 8;
    if (rowbytes % 16) return false;
    cc.cpr = rowbytes / 16;
    return true;
}

GemvWs gemv_ws(const moe_shape_t &s, int T, int Tc, bool single)
{
    GemvWs w;
    const int H = s.hidden, I = s.inter;
    // plan and h buffers hold one chunk of Tc tokens
    PlanDims pd = plan_dims(Tc, s.top_k, s.n_shared, single);
    size_t o = 0;
    w.logits = o; o = align256(o + router_logit_bytes(s, T));
    w.xq = o;     o = align256(o + (size_t)T * H);
    w.xd = o;     o = align256(o + sizeof(float) * (size_t)T * (H / 32));
    w.plan = o;   o = align256(o + sizeof(int) * (size_t)pd.words);
    w.qh = o;     o = align256(o + (size_t)pd.P * I);
    w.dh = o;     o = align256(o + sizeof(float) * (size_t)pd.P * (I / 32));
    w.total = o;
    return w;
}

// Range check of a plan read back from the workspace: every slot names a
// valid expert (or -1 = shared) and its pairs stay inside the buffers.
__device__ __forceinline__ bool plan_ok(const int *plan, const PlanDims &pd, int T, int E)
{
    const int S = plan[0];
    if (S < 0 || S > pd.S) return false;
    for (int u = 0; u < S; u++) {
        const int e = plan[pd.o_e + u], n = plan[pd.o_n + u], p0 = plan[pd.o_p0 + u];
        if (e < -1 || e >= E || n < 0 || n > T || p0 < 0 || p0 + n > pd.P) return false;
    }
    return true;
}

// The pairs a plan uses: the routed slots' pairs are 0 .. R-1 (pairs are
// numbered by (expert, token) order), the shared slot's (the last slot,
// expert -1) start at its own first pair, T * k, which top-p can leave
// apart from R.  Staged pair i of the (R + ns) is pair i for i < R, else
// p0s + (i - R).
struct PlanPairs {
    int R, p0s, ns;
    __device__ int operator()(int i) const { return i < R ? i : p0s + (i - R); }
    __device__ int count() const { return R + ns; }
};
__device__ __forceinline__ PlanPairs plan_pairs(const int *plan, const PlanDims &pd)
{
    const int S = plan[0];
    const bool sh = S > 0 && plan[pd.o_e + S - 1] == -1;
    PlanPairs q;
    q.R = 0;
    for (int u = 0; u < S - (sh ? 1 : 0); u++) q.R += plan[pd.o_n + u];
    q.p0s = sh ? plan[pd.o_p0 + S - 1] : 0;
    q.ns = sh ? plan[pd.o_n + S - 1] : 0;
    return q;
}

// Expert e's tensors through the expert table: the routed base pointers
// plus e's byte offsets (the offsets are workgroup-uniform scalar loads, and
// the pointers stay derived from the kernel's own arguments, so every access
// through them is a global one)
__device__ __forceinline__ moe_weights_t table_view(const GemvArgs &a, int e)
{
    const int64_t *o = a.toff + (size_t)e * 6;
    moe_weights_t v;
    v.gate = a.routed.gate + o[0];
    v.up = a.routed.up + o[1];
    v.down = a.routed.down + o[2];
    v.gate_s = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(a.routed.gate_s) + o[3]);
    v.up_s = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(a.routed.up_s) + o[4]);
    v.down_s = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(a.routed.down_s) + o[5]);
    return v;
}

// The plan of one token (slots = its kept experts in rank order, slot r
// taking pair r, then the shared expert; a batch of one needs no union).  Kept apart from the batch plan so that a caller that
// only ever routes one token compiles no access through generic pointers: a
// pending flat access anywhere in a kernel makes the compiler wait for all
// outstanding loads wherever it waits for one.
__device__ __forceinline__ void build_plan_one(const GemvArgs &a, const PlanDims &pd, int *plan, int *s_idx,
                                               float *s_w)
{
    const int tid = threadIdx.x, k = a.rc.k;
    int *slot_e = plan + pd.o_e, *slot_n = plan + pd.o_n, *slot_p0 = plan + pd.o_p0;
    int *pair_t = plan + pd.o_t;
    float *pair_w = reinterpret_cast<float *>(plan + pd.o_w);
    // one token: slots are its kept experts in rank order, then the shared
    // expert; the pair of a routed slot is the slot itself, the shared
    // expert's pair is k (also when top-p keeps fewer experts)
    if (__builtin_amdgcn_readfirstlane(wave_id()) == 0) {  // the first wave routes the token
        const WaveSel ws = wave_topk(a.rc, a.logits, a.lstride, a.lparts, a.bias, k);
        if (tid < k) { s_idx[tid] = ws.e; s_w[tid] = ws.w; }
    }
    __syncthreads();
    if (tid < k) {
        const int e = s_idx[tid];
        if (e >= 0) {  // top-p keeps a prefix of the ranks
            slot_e[tid] = e;
            slot_n[tid] = 1;
            slot_p0[tid] = tid;
            pair_t[tid] = 0;
            pair_w[tid] = s_w[tid];
        }
    }
    if (tid == 0) {
        int kept = 0;
        for (int j = 0; j < k; j++) kept += (s_idx[j] >= 0);
        plan[0] = kept + a.n_shared;
        if (a.n_shared) {
            slot_e[kept] = -1; slot_n[kept] = 1; slot_p0[kept] = k;
            pair_t[k] = 0; pair_w[k] = 1.0f;
        }
    }
    __syncthreads();
}

// Builds the batch-union plan in LDS (all threads of the block take part).
// Slots hold the union of the routed experts in ascending expert order, then
// the shared expert; pairs of a slot list its tokens in ascending order.
// Everything follows from one bitmap of selected experts per token:
//   slot(e)       = number of union experts below e
//   first pair(e) = number of (token, expert) selections with expert below e
//   pair of (t,e) = first pair(e) + number of tokens before t selecting e
// tokbits: LDS scratch of kGemvMaxT x 16 words (E <= 512).  Each wave of the
// block routes every nw-th token (nw waves), so up to nw tokens route at once.
__device__ __forceinline__ void build_plan(const GemvArgs &a, const PlanDims &pd, int *plan, int *s_idx, float *s_w,
                           uint32_t (*tokbits)[16])
{
    const int tid = threadIdx.x, nt = blockDim.x, T = a.T, k = a.rc.k;
    int *slot_e = plan + pd.o_e, *slot_n = plan + pd.o_n, *slot_p0 = plan + pd.o_p0;
    int *pair_t = plan + pd.o_t;
    float *pair_w = reinterpret_cast<float *>(plan + pd.o_w);
    if (!a.logits) {  // single expert, all tokens, weight 1
        if (tid == 0) { plan[0] = 1; slot_e[0] = a.single; slot_n[0] = T; slot_p0[0] = 0; }
        for (int t = tid; t < T; t += nt) { pair_t[t] = t; pair_w[t] = 1.0f; }
        __syncthreads();
        return;
    }
    if (T == 1) {
        build_plan_one(a, pd, plan, s_idx, s_w);
        return;
    }
    // each wave routes every nw-th token and writes that token's bitmap
    // (lane w < 16 ORs together the selections that fall in word w)
    {
        const int nw = nt >> 6, wv = __builtin_amdgcn_readfirstlane(wave_id()), lane = lane_id();
        for (int t = wv; t < T; t += nw) {
            const WaveSel ws = wave_topk(a.rc, a.logits + (size_t)t * a.E, a.lstride, a.lparts, a.bias, k);
            if (lane < k) { s_idx[t * k + lane] = ws.e; s_w[t * k + lane] = ws.w; }
            if (a.counts && lane < k && ws.e >= 0) atomicAdd(&a.counts[ws.e], 1u);
            uint32_t word = 0u;
            for (int i = 0; i < k; i++) {
                const int e = __builtin_amdgcn_readlane(ws.e, i);  // e < 0: dropped by top-p
                if (e >= 0 && (e >> 5) == lane) word |= 1u << (e & 31);
            }
            if (lane < 16) tokbits[t][lane] = word;
        }
    }
    __syncthreads();
    // per bitmap word: union experts and selections below it (exclusive
    // prefix sums over the words, one wave), and the union's size
    __shared__ int upre[16], cpre[16], s_u;
    const int nwd = (a.E + 31) >> 5;
    if (tid < kWave) {
        uint32_t un = 0u;
        int cnt = 0;
        for (int tt = 0; tt < T; tt++) {
            const uint32_t v = tokbits[tt][tid & 15];
            un |= v;
            cnt += __popc(v);
        }
        const bool live = tid < nwd;
        const int uc = live ? __popc(un) : 0;
        cnt = live ? cnt : 0;
        int us = uc, cs = cnt;
        for (int o = 1; o < 16; o <<= 1) {
            const int ua = __shfl_up(us, o), ca = __shfl_up(cs, o);
            if (tid >= o) { us += ua; cs += ca; }
        }
        if (tid < 16) { upre[tid] = us - uc; cpre[tid] = cs - cnt; }
        if (tid == 15) s_u = us;
    }
    __syncthreads();
    for (int i = tid; i < T * k; i += nt) {
        if (s_idx[i] < 0) continue;
        const int t = i / k, e = s_idx[i], wi = e >> 5;
        const uint32_t bit = 1u << (e & 31), below = bit - 1u;
        int slot = upre[wi], p0 = cpre[wi], n = 0, rank = 0;
        uint32_t un = 0u;
        for (int tt = 0; tt < T; tt++) {
            const uint32_t v = tokbits[tt][wi];
            un |= v;
            p0 += __popc(v & below);
            if (v & bit) { n++; rank += (tt < t); }
        }
        slot += __popc(un & below);
        slot_e[slot] = e;
        slot_n[slot] = n;
        slot_p0[slot] = p0;
        pair_t[p0 + rank] = t;
        pair_w[p0 + rank] = s_w[i];
    }
    if (tid == 0) {
        const int U = s_u;
        plan[0] = U + a.n_shared;
        if (a.n_shared) { slot_e[U] = -1; slot_n[U] = T; slot_p0[U] = T * k; }
    }
    if (a.n_shared)
        for (int t = tid; t < T; t += nt) {
            pair_t[T * k + t] = t;
            pair_w[T * k + t] = 1.0f;
        }
    __syncthreads();
}

// ---------------------------------------------------------------- plan kernel
// One workgroup routes the chunk's tokens and publishes the plan (and the
// routing, when asked): for several tokens, measured on MI355X, one such
// launch costs less than every gate/up workgroup re-deriving the union plan,
// or than cross-workgroup signalling through a shared atomic counter.
// One wave per token routes every token of the chunk at once.
constexpr int kPlanThreads = kWave * kGemvMaxT;
__global__ __launch_bounds__(kPlanThreads) void k_plan(const GemvArgs a, const PlanDims pd)
{
    __shared__ int plan[1 + 3 * (kGemvMaxT * kMaxTopK + 1) + 2 * kGemvMaxT * (kMaxTopK + 1)];
    __shared__ int s_idx[kGemvMaxT * kMaxTopK];
    __shared__ float s_w[kGemvMaxT * kMaxTopK];
    __shared__ uint32_t tokbits[kGemvMaxT][16];
    build_plan(a, pd, plan, s_idx, s_w, tokbits);
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int i = tid; i < pd.words; i += nt) a.plan[i] = plan[i];
    if (a.logits && a.idx_out)
        for (int i = tid; i < a.T * a.rc.k; i += nt) { a.idx_out[i] = s_idx[i]; a.w_out[i] = s_w[i]; }
}

int launch_plan(const GemvArgs &a, hipStream_t st)
{
    const PlanDims pd = plan_dims(a.T, a.rc.k, a.n_shared, a.logits == nullptr);
    k_plan<<<1, kPlanThreads, 0, st>>>(a, pd);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- activations in LDS
// Per token, the activation operand of every chunk position of a row (nch
// positions), laid out for act_from_lds: A [NA / 4][nch] 16-byte pieces
// (already permuted for the weight packing; piece i of consecutive
// positions is contiguous, so the lanes of a read take consecutive 16-byte
// words, free of bank conflicts), then per block its scale (int8: D
// [blocks]) or its scale and code sum (int4 / int2: {d, qs} [blocks]).
template <int WB> struct ActShape;
template <> struct ActShape<8> { static constexpr int NA = 4; };
template <> struct ActShape<4> { static constexpr int NA = 8; };
template <> struct ActShape<2> { static constexpr int NA = 16; };

// chunks per thread staged in one batch of loads by the down kernel (one
// token's pairs fit one batch at the production shapes)
constexpr int stage_batch(int wb) { return wb == 8 ? 5 : wb == 4 ? 3 : 2; }

template <int WB>
__device__ __forceinline__ void store_act(const Act<WB> &A, int pos, int nch, uint32_t *la, float *ld)
{
    uint4 *dst = reinterpret_cast<uint4 *>(la);
#pragma unroll
    for (int i = 0; i < ActShape<WB>::NA / 4; i++)
        dst[i * nch + pos] = make_uint4(A.a[4 * i], A.a[4 * i + 1], A.a[4 * i + 2], A.a[4 * i + 3]);
    if constexpr (WB == 8) {
        ld[pos >> 1] = A.d;  // both chunks of a block store the block's scale
    } else if constexpr (WB == 4) {
        reinterpret_cast<float2 *>(ld)[pos] = make_float2(A.d, __int_as_float(A.qs));
    } else {
        reinterpret_cast<float4 *>(ld)[pos] =
            make_float4(A.d0, __int_as_float(A.qs0), A.d1, __int_as_float(A.qs1));
    }
}

template <int WB>
__device__ __forceinline__ void stage_act(const int8_t *q, const float *d, int pos, int nch, uint32_t *la, float *ld)
{
    Act<WB> A;
    A.load(q, d, pos);
    store_act<WB>(A, pos, nch, la, ld);
}

template <int WB>
__device__ __forceinline__ void act_from_lds(Act<WB> &A, const uint32_t *la, const float *ld, int pos, int nch)
{
    const uint4 *src = reinterpret_cast<const uint4 *>(la);
#pragma unroll
    for (int i = 0; i < ActShape<WB>::NA / 4; i++) {
        const uint4 v = src[i * nch + pos];
        A.a[4 * i] = v.x; A.a[4 * i + 1] = v.y; A.a[4 * i + 2] = v.z; A.a[4 * i + 3] = v.w;
    }
    if constexpr (WB == 8) {
        A.d = ld[pos >> 1];
    } else if constexpr (WB == 4) {
        const float2 v = reinterpret_cast<const float2 *>(ld)[pos];
        A.set_scale(v.x);
        A.qs = __float_as_int(v.y);
    } else {
        const float4 v = reinterpret_cast<const float4 *>(ld)[pos];
        A.set_scale(v.x, v.z);
        A.qs0 = __float_as_int(v.y); A.qs1 = __float_as_int(v.w);
    }
}

// A 16-byte weight load, marked non-temporal: every weight byte of a GEMV
// launch is read once, so the request asks the caches not to keep it
// (global_load_dwordx4 ... nt), which leaves L2 to the activations, plans
// and h rows that are read again.
typedef unsigned v4u_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const uint8_t *p)
{
    const v4u_nt v = __builtin_nontemporal_load(reinterpret_cast<const v4u_nt *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- gate / up
constexpr int kGuLanes = 8;   // lanes per row in k_gate_up
constexpr int kGuBatch = 4;   // chunks per lane per prefetch batch

template <int WB, int TT>
__global__ __launch_bounds__(256) void k_gate_up_rg(const GemvArgs a, const ChunkCfg cc, const PlanDims pd)
{
    __shared__ int plan[1 + 3 * (kGemvMaxT * kMaxTopK + 1) + 2 * kGemvMaxT * (kMaxTopK + 1)];
    __shared__ float s_h[TT][32];
    extern __shared__ __align__(16) unsigned char lds_act[];
    static_assert(sizeof(plan) + sizeof(s_h) <= kGateUpStaticLds, "static LDS of k_gate_up");

    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    for (int i = tid; i < pd.words; i += 256) plan[i] = a.plan[i];
    __syncthreads();
    if (!plan_ok(plan, pd, a.T, a.E)) return;
    const int tiles = a.I / 32;
    const int u = blockIdx.x / tiles, row0 = (blockIdx.x % tiles) * 32;
    if (u >= plan[0]) return;
    const int e = plan[pd.o_e + u];
    const moe_weights_t &W = (e >= 0) ? a.routed : a.shared;
    const int ee = (e >= 0) ? e : 0;
    const int cpr = cc.cpr, H = a.H, nb = H / 32;
    const size_t rowbytes = (size_t)cpr * 16;
    const int n_u = plan[pd.o_n + u], p0 = plan[pd.o_p0 + u];

    // stage the slot's token activations (n_u <= TT)
    const size_t tok_bytes = act_lds_bytes(WB, H);
    auto la_of = [&](int tt) { return reinterpret_cast<uint32_t *>(lds_act + tt * tok_bytes); };
    auto ld_of = [&](int tt) { return reinterpret_cast<float *>(lds_act + tt * tok_bytes + H); };
    for (int c = tid; c < n_u * cpr; c += 256) {
        const int tt = c / cpr, pos = c - tt * cpr;
        const int t = plan[pd.o_t + p0 + tt];
        stage_act<WB>(a.xq + (size_t)t * H, a.xd + (size_t)t * nb, pos, cpr, la_of(tt), ld_of(tt));
    }
    __syncthreads();

    // 8 lanes per row: this lane's row and its chunk positions sub, sub+8, ...
    const int sub = lane & (kGuLanes - 1);
    const int rloc = wv * (64 / kGuLanes) + (lane / kGuLanes);
    const int row = row0 + rloc;
    const uint8_t *grow = W.gate + ((size_t)ee * a.I + row) * rowbytes;
    const uint8_t *urow = W.up + ((size_t)ee * a.I + row) * rowbytes;
    const int niter = (cpr + kGuLanes - 1) / kGuLanes;
    const int nbatch = (niter + kGuBatch - 1) / kGuBatch;

    float accg[TT], accu[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) { accg[tt] = 0.f; accu[tt] = 0.f; }

    uint4 bg[2][kGuBatch], bu[2][kGuBatch];
    auto load_batch = [&](int b, uint4 *g, uint4 *v) {
#pragma unroll
        for (int j = 0; j < kGuBatch; j++) {
            const int pos = sub + kGuLanes * (b * kGuBatch + j);
            if (pos < cpr) {
                g[j] = ld16(grow + (size_t)pos * 16);
                v[j] = ld16(urow + (size_t)pos * 16);
            } else {
                g[j] = make_uint4(0, 0, 0, 0);
                v[j] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto use_batch = [&](int b, const uint4 *g, const uint4 *v) {
#pragma unroll
        for (int j = 0; j < kGuBatch; j++) {
            const int pos = sub + kGuLanes * (b * kGuBatch + j);
            if (pos < cpr) {
#pragma unroll
                for (int tt = 0; tt < TT; tt++) {
                    if (tt < n_u) {
                        Act<WB> A;
                        act_from_lds<WB>(A, la_of(tt), ld_of(tt), pos, cpr);
                        accg[tt] += A.dot(g[j]);
                        accu[tt] += A.dot(v[j]);
                    }
                }
            }
        }
    };
    load_batch(0, bg[0], bu[0]);
    for (int b = 0; b < nbatch; b += 2) {
        if (b + 1 < nbatch) load_batch(b + 1, bg[1], bu[1]);
        use_batch(b, bg[0], bu[0]);
        if (b + 1 < nbatch) {
            if (b + 2 < nbatch) load_batch(b + 2, bg[0], bu[0]);
            use_batch(b + 1, bg[1], bu[1]);
        }
    }
    const float sg = W.gate_s[(size_t)ee * a.I + row], su = W.up_s[(size_t)ee * a.I + row];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        if (tt < n_u) {
            float g = accg[tt], v = accu[tt];
#pragma unroll
            for (int o = 1; o < kGuLanes; o <<= 1) {
                g += __shfl_xor(g, o);
                v += __shfl_xor(v, o);
            }
            if (sub == 0) s_h[tt][rloc] = silu_mul(g * sg, v * su);
        }
    }
    __syncthreads();
    // quantise h per token: one block of 32 rows, lanes 0..31 of a wave
    for (int tt = wv; tt < n_u; tt += 4) {
        const int p = p0 + tt;
        const float h = s_h[tt][lane & 31];
        float amax = fabsf(h);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float d = amax / 127.0f;
        float r = (d == 0.0f) ? 0.0f : rintf(h / d);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        if (lane < 32) a.qh[(size_t)p * a.I + row0 + lane] = (int8_t)(int)r;
        if (lane == 0) a.dh[(size_t)p * (a.I / 32) + row0 / 32] = d;
    }
}

// ---------------------------------------------------------------- down / combine
constexpr int kDnLanes = 16;  // lanes per row in k_down
constexpr int kDnRows = 16;   // rows per workgroup (4 waves x 4 rows)
constexpr int kDnBatch = 4;   // chunks per lane per prefetch batch

template <int WB, int TT>
__global__ __launch_bounds__(256) void k_down_rg(const GemvArgs a, const ChunkCfg cc, const PlanDims pd)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int I = a.I, nbh = I / 32, cpr = cc.cpr;
    int *plan = reinterpret_cast<int *>(lds);
    const int plan_words = (pd.words + 3) & ~3;
    unsigned char *act = lds + sizeof(int) * plan_words;
    const size_t pair_bytes = act_lds_bytes(WB, I);
    auto la_of = [&](int p) { return reinterpret_cast<uint32_t *>(act + p * pair_bytes); };
    auto ld_of = [&](int p) { return reinterpret_cast<float *>(act + p * pair_bytes + I); };

    for (int i = tid; i < pd.words; i += 256) plan[i] = a.plan[i];
    __syncthreads();
    if (!plan_ok(plan, pd, a.T, a.E)) return;
    const int S = plan[0];
    const PlanPairs pp = plan_pairs(plan, pd);
    for (int c = tid; c < pp.count() * cpr; c += 256) {
        const int i = c / cpr, pos = c - i * cpr, p = pp(i);
        stage_act<WB>(a.qh + (size_t)p * I, a.dh + (size_t)p * nbh, pos, cpr, la_of(p), ld_of(p));
    }
    __syncthreads();

    const int sub = lane & (kDnLanes - 1);
    const int row = blockIdx.x * kDnRows + wv * (64 / kDnLanes) + lane / kDnLanes;
    const size_t rowbytes = (size_t)cpr * 16;
    const int niter = (cpr + kDnLanes - 1) / kDnLanes;
    const int nbatch = (niter + kDnBatch - 1) / kDnBatch;  // batches per slot
    const int total = S * nbatch;                           // (slot, batch) steps

    float acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) acc[tt] = 0.f;

    uint4 buf[2][kDnBatch];
    auto slot_row = [&](int u) {
        const int e = plan[pd.o_e + u];
        const moe_weights_t &W = (e >= 0) ? a.routed : a.shared;
        return W.down + ((size_t)((e >= 0) ? e : 0) * a.H + row) * rowbytes;
    };
    auto load_step = [&](int s, uint4 *w) {
        const int u = s / nbatch, b = s - u * nbatch;
        const uint8_t *src = slot_row(u);
#pragma unroll
        for (int j = 0; j < kDnBatch; j++) {
            const int pos = sub + kDnLanes * (b * kDnBatch + j);
            w[j] = (pos < cpr) ? ld16(src + (size_t)pos * 16) : make_uint4(0, 0, 0, 0);
        }
    };
    auto use_step = [&](int s, const uint4 *w) {
        const int u = s / nbatch, b = s - u * nbatch;
        const int e = plan[pd.o_e + u];
        const float sr = ((e >= 0) ? a.routed.down_s + (size_t)e * a.H : a.shared.down_s)[row];
        const int n = plan[pd.o_n + u], p0 = plan[pd.o_p0 + u];
        for (int j2 = 0; j2 < n; j2++) {
            const int p = p0 + j2;
            const int t = plan[pd.o_t + p];
            const float coef = __int_as_float(plan[pd.o_w + p]) * sr;
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < kDnBatch; j++) {
                const int pos = sub + kDnLanes * (b * kDnBatch + j);
                if (pos < cpr) {
                    Act<WB> A;
                    act_from_lds<WB>(A, la_of(p), ld_of(p), pos, cpr);
                    part += A.dot(w[j]);
                }
            }
#pragma unroll
            for (int tt = 0; tt < TT; tt++)
                if (tt == t) acc[tt] += coef * part;
        }
    };
    load_step(0, buf[0]);
    for (int s = 0; s < total; s += 2) {
        if (s + 1 < total) load_step(s + 1, buf[1]);
        use_step(s, buf[0]);
        if (s + 1 < total) {
            if (s + 2 < total) load_step(s + 2, buf[0]);
            use_step(s + 1, buf[1]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        if (tt < a.T) {
            float v = acc[tt];
#pragma unroll
            for (int o = 1; o < kDnLanes; o <<= 1) v += __shfl_xor(v, o);
            if (sub == 0) {
                float *dst = a.y + (size_t)tt * a.H + row;
                *dst = a.accumulate ? *dst + v : v;
            }
        }
    }
}


// ---------------------------------------------------------------- row-sweep kernels
// Measured on MI355X: streaming reads reach ~6.4 TB/s only when each step of
// a workgroup reads one contiguous window of a few KB; workgroups whose waves
// walk separate rows (even 1 KB contiguous per wave) stall near 2.5 TB/s.  So
// in these kernels the workgroup reads whole consecutive rows per step, each
// thread owns fixed chunk positions of the row (its int8 activation operand
// then lives in registers), per-row partial sums accumulate in registers, and
// rows are finished by a reduce-scatter over 32-lane groups plus a
// fixed-order combine of the groups in LDS.

// Reduce-scatter of N partials (N a power of two <= 32) over a 32-lane
// group: afterwards lane l of the group holds, for slot j = (l % 32) / (32/N),
// the sum of v[j] over the 32 lanes (valid where (l % 32) % (32/N) == 0).
// One level of the reduce-scatter: lanes exchange the half of their NA live
// values they do not keep with the lane O apart and add the received half.
// NA and O are compile-time, so every register index is static (a runtime
// width would turn v[j + NA/2] into compare/select ladders).
// The partner of a lane at level O: a lane whose bit O differs and whose
// bits above O agree.  With DPP, inside a row of 16 that is a DPP move in
// the VALU (lane ^ 1, lane ^ 2, then the mirror of 8 and of 16, which flip
// bit 2 and bit 3 together with the bits below) and only level 16 crosses
// rows; without, every level is a swap through the LDS crossbar.  Measured
// on MI355X: DPP pays where a workgroup reduces several token rows at once
// (verify batches of 3 and 5 tokens, 3-4% faster); one token keeps the
// crossbar, which leaves its VALU-heavy int2 sweep to the VALU.
template <int O, bool DPP> __device__ __forceinline__ float rs_partner(float v)
{
    if constexpr (O == 16 || !DPP) {
        return __shfl_xor(v, O);
    } else {
        constexpr int CTRL = O == 1 ? 0xB1 : O == 2 ? 0x4E : O == 4 ? 0x141 : 0x140;
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
    }
}

template <int N, int O, int NA, bool DPP>
__device__ __forceinline__ void reduce_scatter_level(float (&v)[N], int lane)
{
    if constexpr (NA > 1) {
        constexpr int HALF = NA / 2;
        const bool upper = (lane & O) != 0;
#pragma unroll
        for (int j = 0; j < HALF; j++) {
            const float send = upper ? v[j] : v[j + HALF];
            const float keep = upper ? v[j + HALF] : v[j];
            v[j] = keep + rs_partner<O, DPP>(send);
        }
    } else {
        v[0] += rs_partner<O, DPP>(v[0]);
    }
    if constexpr (O > 1) reduce_scatter_level<N, O / 2, (NA > 1 ? NA / 2 : 1), DPP>(v, lane);
}

// Sum of N values over the 32 lanes of a half-wave, scattered: lane l ends
// with the total of value j = l / (32 / N) (fixed pairing and order, so the
// result is run-to-run identical).
template <int N, bool DPP = false>
__device__ __forceinline__ float group32_reduce_scatter(float (&v)[N])
{
    reduce_scatter_level<N, 16, N, DPP>(v, lane_id());
    return v[0];
}

constexpr int kSwThreads = 192;  // gate/up row-sweep block
static_assert(kSwThreads % 32 == 0, "row r of a tile is handled by threads r mod 32");
constexpr int kSwGroups = kSwThreads / 32;
constexpr int kSwDepth = 11;     // steps of prefetch in flight (<= 168 VGPRs: 3 waves per SIMD)
// Batches of 2-8 tokens: per-token accumulators and activations are live
// registers, so a batch kernel takes passes of 4 rows (one token: 8) and,
// with one chunk per thread, 4 steps of prefetch: at most ~200 VGPRs, two or
// three waves per SIMD.  With the one-token settings the batch kernels held
// 256 VGPRs plus AGPR spills, one wave per SIMD (measured on MI355X: verify
// batches of 2, 3, 5 and 8 tokens 6%, 9%, 14% and 22% faster this way).
constexpr int kSwDepthBatch = 4;
constexpr int kSwPassRowsBatch = 4;

// gate/up of one 32-row tile of one expert for the n_u tokens of a slot: a
// step reads RPS rows of gate and of up (kSwThreads * CPT chunks each,
// contiguous), in passes of 8 rows (4 for batches).  toks lists the slot's tokens; pair
// p_first + tt receives token tt's quantised h.  All threads of the block
// must call it.
template <int WB, int CPT, int RPS, int TT>
__device__ __forceinline__ void gate_up_tile_sw(const GemvArgs &a, const moe_weights_t &W, int ee, int row0,
                                                int n_u, const int *toks, int p_first, float (*s_h)[32],
                                                float (*part)[TT][kSwGroups][32])
{
    static_assert(CPT == 1 || RPS == 1, "chunks of one thread stay in one row");
    // batches of tokens: shorter passes (fewer live accumulators) and, with
    // one chunk per thread, a shallower prefetch (each step's dots are TT
    // times the work)
    constexpr int PASS_ROWS = TT > 1 ? kSwPassRowsBatch : 8;
    constexpr int NSTEP = 32 / RPS, PS = PASS_ROWS / RPS;
    constexpr int PF = (CPT == 1) ? (TT > 1 ? kSwDepthBatch : kSwDepth) : kSwDepth / 2;
    const int tid = threadIdx.x, lane = lane_id();
    const int cpr = (kSwThreads * CPT) / RPS, H = a.H, nb = H / 32;
    const size_t rowbytes = (size_t)cpr * 16;
    const int rowoff = (RPS == 1) ? 0 : tid / cpr;
    const int grp = tid >> 5;

    const uint8_t *gb = W.gate + ((size_t)ee * a.I + row0) * rowbytes + (size_t)tid * 16;
    const uint8_t *ub = W.up + ((size_t)ee * a.I + row0) * rowbytes + (size_t)tid * 16;
    // the row scales this thread applies at the end (row tid % 32; kSwThreads
    // is a multiple of 32), requested now so the epilogue does not wait on them
    const float sg_r = W.gate_s[(size_t)ee * a.I + row0 + (tid & 31)];
    const float su_r = W.up_s[(size_t)ee * a.I + row0 + (tid & 31)];
    const size_t step_bytes = (size_t)kSwThreads * CPT * 16;
    // Activation loads first, then PF steps of weight rows: the vector memory
    // counter retires loads in issue order, so the first dot then waits for
    // the activations only, not for the whole prefetch.
    Act<WB> act[TT][CPT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        if (tt < n_u) {
            const int t = toks[tt];
#pragma unroll
            for (int k = 0; k < CPT; k++) {
                const int pos = (tid + kSwThreads * k) % cpr;
                act[tt][k].load_raw(a.xq + (size_t)t * H, a.xd + (size_t)t * nb, pos);
            }
        }
    }
    uint4 bg[PF][CPT], bu[PF][CPT];
#pragma unroll
    for (int s = 0; s < PF; s++)
#pragma unroll
        for (int k = 0; k < CPT; k++) {
            bg[s][k] = ld16(gb + s * step_bytes + (size_t)k * kSwThreads * 16);
            bu[s][k] = ld16(ub + s * step_bytes + (size_t)k * kSwThreads * 16);
        }
#pragma unroll
    for (int tt = 0; tt < TT; tt++)
        if (tt < n_u)
#pragma unroll
            for (int k = 0; k < CPT; k++) act[tt][k].finish();
    float accg[TT][PS], accu[TT][PS];
    // issue priority falls as the sweep advances, so that on a CU the waves
    // of a workgroup that is behind are served first and the workgroups
    // finish closer together (measured on MI355X: the older of two
    // workgroups on a CU otherwise finishes ~3 us earlier)
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int s = 0; s < NSTEP; s++) {
        const int slot = s % PF, j = s % PS;
        if (s == NSTEP / 4) __builtin_amdgcn_s_setprio(2);
        if (s == NSTEP / 2) __builtin_amdgcn_s_setprio(1);
        if (s == 3 * NSTEP / 4) __builtin_amdgcn_s_setprio(0);
        if (j == 0) {
#pragma unroll
            for (int tt = 0; tt < TT; tt++)
#pragma unroll
                for (int q = 0; q < PS; q++) { accg[tt][q] = 0.f; accu[tt][q] = 0.f; }
        }
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
            if (tt < n_u) {
#pragma unroll
                for (int k = 0; k < CPT; k++) {
                    accg[tt][j] += act[tt][k].dot(bg[slot][k]);
                    accu[tt][j] += act[tt][k].dot(bu[slot][k]);
                }
            }
        }
        if (s + PF < NSTEP) {
#pragma unroll
            for (int k = 0; k < CPT; k++) {
                bg[slot][k] = ld16(gb + (s + PF) * step_bytes + (size_t)k * kSwThreads * 16);
                bu[slot][k] = ld16(ub + (s + PF) * step_bytes + (size_t)k * kSwThreads * 16);
            }
        }
        // keep one step's loads and dots together: without this the
        // scheduler gathers the unrolled steps' loads into bursts and lets the
        // number in flight drain between them
        __builtin_amdgcn_sched_barrier(0);
        if (j == PS - 1) {
            const int pass = s / PS;
            const int l32 = lane & 31;
            const int jj = l32 / (32 / PS);
            const bool writer = (l32 % (32 / PS)) == 0;
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                if (tt < n_u) {
                    const float g = group32_reduce_scatter<PS, (TT > 1)>(accg[tt]);
                    const float v = group32_reduce_scatter<PS, (TT > 1)>(accu[tt]);
                    if (writer) {
                        part[0][tt][grp][pass * PASS_ROWS + jj * RPS + rowoff] = g;
                        part[1][tt][grp][pass * PASS_ROWS + jj * RPS + rowoff] = v;
                    }
                }
            }
        }
    }
    __syncthreads();
    // combine the groups of each row in a fixed order, then SwiGLU
    const int groups_per_row = kSwGroups / RPS;
    for (int i = tid; i < n_u * 32; i += kSwThreads) {
        const int tt = i >> 5, r = i & 31, g0 = (r % RPS) * groups_per_row;
        float g = 0.f, v = 0.f;
        for (int q = 0; q < groups_per_row; q++) { g += part[0][tt][g0 + q][r]; v += part[1][tt][g0 + q][r]; }
        s_h[tt][r] = silu_mul(g * sg_r, v * su_r);  // r == tid % 32
    }
    __syncthreads();
    // quantise h per token: one block of 32 rows, lanes 0..31 of a wave
    for (int tt = wave_id(); tt < n_u; tt += kSwThreads / 64) {
        const int p = p_first + tt;
        const float h = s_h[tt][lane & 31];
        float amax = fabsf(h);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float d = amax / 127.0f;
        float r = (d == 0.0f) ? 0.0f : rintf(h / d);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        if (lane < 32) a.qh[(size_t)p * a.I + row0 + lane] = (int8_t)(int)r;
        if (lane == 0) a.dh[(size_t)p * (a.I / 32) + row0 / 32] = d;
    }
}

// Every slot of a chunk, with the plan the plan kernel published.  The plan
// is range-checked, so a corrupt plan can only skip work, never steer a load
// out of the weight tensors.
// One token, no plan launch: the shared expert's workgroups need no routing
// and start streaming at once; the workgroups of routed slot u take the
// expert of rank u, found by the first
// u + 1 rounds of the selection in their first wave (the same inputs in the
// same order, so every workgroup reaches the same ranking), so a slot's
// stream starts as soon as its own rank is known.  Workgroup (u = 0, tile 0)
// runs the whole selection and publishes the plan for the down kernel, and
// the routing when asked; with adaptive top-p every workgroup does, since
// whether rank u is kept depends on all the weights.
// Dispatch order: the routed slots in rank order, then the shared expert.
// The launch has more workgroups than two per CU, and the last dispatched
// land on CUs that already stream two; there a selection runs slowest (it
// shares the SIMDs with the streaming waves), so those places go to the
// workgroups that select nothing.
template <int WB, int CPT, int RPS, bool TAB>
__device__ void gate_up_sw_routed_here(const GemvArgs &a, const PlanDims &pd, int tiles, float (*s_h)[32],
                                       float (*part)[1][kSwGroups][32])
{
    __shared__ int plan[1 + 5 * (kMaxTopK + 1)];
    __shared__ int s_idx[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    const int b = blockIdx.x / tiles, tile = blockIdx.x % tiles, row0 = tile * 32;
    const int nr = pd.S - a.n_shared;  // routed slots
    // slot v: 0 .. n_shared - 1 the shared experts, then rank v - n_shared
    const int v = b < nr ? b + a.n_shared : b - nr;
    if (v < a.n_shared) {
        if (threadIdx.x == 0) plan[0] = 0;  // the token list of the shared slot: token 0
        __syncthreads();
        gate_up_tile_sw<WB, CPT, RPS, 1>(a, a.shared, 0, row0, 1, plan, a.rc.k, s_h, part);
        return;
    }
    const int u = v - a.n_shared;
    int e;
    if ((u == 0 && tile == 0) || a.rc.top_p > 0.f) {
        build_plan_one(a, pd, plan, s_idx, s_w);
        if (u >= plan[0] - a.n_shared) return;  // a slot top-p dropped (uniform in the workgroup)
        if (u == 0 && tile == 0) {
            for (int i = threadIdx.x; i < pd.words; i += kSwThreads) a.plan[i] = plan[i];
            if (a.idx_out && threadIdx.x < a.rc.k) {
                a.idx_out[threadIdx.x] = s_idx[threadIdx.x];
                a.w_out[threadIdx.x] = s_w[threadIdx.x];
            }
            if (a.counts && threadIdx.x < a.rc.k && s_idx[threadIdx.x] >= 0)
                atomicAdd(&a.counts[s_idx[threadIdx.x]], 1u);
        }
        e = plan[pd.o_e + u];
        __syncthreads();  // plan[0] becomes the slot's token list below
    } else {
        if (__builtin_amdgcn_readfirstlane(wave_id()) == 0) {
            const WaveSel ws = wave_topk(a.rc, a.logits, a.lstride, a.lparts, a.bias, u + 1);
            if (threadIdx.x == 0) s_idx[0] = ws.last;
        }
        __syncthreads();
        e = s_idx[0];
    }
    if (e < 0 || e >= a.E || u >= pd.P) return;
    if (threadIdx.x == 0) plan[0] = 0;  // the slot's token list: token 0
    __syncthreads();
    if constexpr (TAB) {
        const moe_weights_t V = table_view(a, e);
        gate_up_tile_sw<WB, CPT, RPS, 1>(a, V, 0, row0, 1, plan, u, s_h, part);
    } else {
        gate_up_tile_sw<WB, CPT, RPS, 1>(a, a.routed, e, row0, 1, plan, u, s_h, part);
    }
}

// Router lookahead (wpnews.pro "Colibri -- GLM-5.2 (744B MoE) on 25GB RAM in
// one pure C file", paragraph "Router-lookahead prefetch (PILOT=1)": layer
// L+1's router, run on layer L's state, predicts the experts layer L+1 will
// select, and those are fetched while layer L computes).
// Lookahead workgroup j of unit j / la_wgs: units 0 .. k-1 are the experts of
// ranks 0 .. k-1 of the next layer's selection (the full noaux_tc selection
// on la_logits, the same wave-level routine as the routing itself; top-p is
// ignored: every rank the prediction names is fetched), unit k is the next
// layer's shared expert.  The workgroup streams slice j % la_wgs of the
// expert's gate, up and down codes (and, slice 0, its row scales) with
// non-temporal loads: they bypass the L2s and fill the memory-side cache,
// from which that layer's kernels then read them.  The loaded data only
// feeds an XOR stored to la_sink, which keeps the loads.
template <int WB>
__device__ void gate_up_lookahead(const GemvArgs &a, int j)
{
    __shared__ int s_e;
    const int unit = j / a.la_wgs, slice = j % a.la_wgs, tid = threadIdx.x;
    const moe_weights_t *W = &a.la_shared;
    size_t e = 0;
    if (unit < a.rc.k) {
        RouteCfg rc = a.rc;
        rc.top_p = 0.f;
        if (__builtin_amdgcn_readfirstlane(wave_id()) == 0) {
            const WaveSel ws = wave_topk(rc, a.la_logits, (size_t)a.E, 1, a.la_bias, unit + 1);
            if (tid == 0) s_e = ws.last;
        }
        __syncthreads();
        const int pe = s_e;
        if (pe < 0 || pe >= a.E) return;
        e = (size_t)pe;
        W = &a.la_routed;
    }
    const size_t cb = (size_t)a.I * a.H * WB / 8;        // code bytes of each of gate, up, down
    const size_t per = ((cb / 16) + a.la_wgs - 1) / a.la_wgs;  // 16-byte chunks per slice
    const size_t c0 = (size_t)slice * per, c1 = min(c0 + per, cb / 16);
    const uint8_t *src[3] = {W->gate + e * cb, W->up + e * cb, W->down + e * cb};
    typedef unsigned v4u_nt __attribute__((ext_vector_type(4)));
    uint32_t acc = 0;
    constexpr int U = 8;  // loads in flight per thread
#pragma unroll
    for (int m = 0; m < 3; m++) {
        const v4u_nt *p = reinterpret_cast<const v4u_nt *>(src[m]);
        for (size_t c = c0 + tid; c < c1; c += (size_t)kSwThreads * U) {
            v4u_nt v[U];
#pragma unroll
            for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(p + min(c + (size_t)kSwThreads * u, c1 - 1));
#pragma unroll
            for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    if (slice == 0) {
        const float *sc[3] = {W->gate_s + e * a.I, W->up_s + e * a.I, W->down_s + e * a.H};
        const int n[3] = {a.I, a.I, a.H};
#pragma unroll
        for (int m = 0; m < 3; m++)
            for (int i = tid; i < n[m]; i += kSwThreads) acc ^= __float_as_uint(__builtin_nontemporal_load(sc[m] + i));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    static_assert(kSwThreads / 64 <= kLookaheadSinkWords, "sink words per workgroup");
    if (lane_id() == 0) a.la_sink[(size_t)j * kLookaheadSinkWords + wave_id()] = acc;
}

// TAB: routed experts through the expert table (a.toff)
template <int WB, int CPT, int RPS, int TT, bool TAB = false>
__global__ __launch_bounds__(kSwThreads) void k_gate_up_sw(const GemvArgs a, const ChunkCfg cc, const PlanDims pd)
{
    __shared__ float s_h[TT][32];
    __shared__ float part[2][TT][kSwGroups][32];
    const int tiles = a.I / 32;
    if constexpr (TT == 1) {
        if (a.inline_route) {
            if constexpr (!TAB) {
                // the workgroups past the layer's own run the router lookahead
                if ((int)blockIdx.x >= pd.S * tiles) {
                    gate_up_lookahead<WB>(a, (int)blockIdx.x - pd.S * tiles);
                    return;
                }
            }
            gate_up_sw_routed_here<WB, CPT, RPS, TAB>(a, pd, tiles, s_h, part);
            return;
        }
    }
    const int u = blockIdx.x / tiles, row0 = (blockIdx.x % tiles) * 32;
    // the slot count and the slot's entries in one round trip (u < pd.S, so
    // every entry read lies inside the plan; a stale entry of an unused slot
    // is discarded by the checks below)
    const int S = a.plan[0];
    const int e = a.plan[pd.o_e + u], n_u = a.plan[pd.o_n + u], p0 = a.plan[pd.o_p0 + u];
    if (S > pd.S || u >= S) return;
    if (e < -1 || e >= a.E || n_u < 1 || n_u > a.T || p0 < 0 || p0 + n_u > pd.P) return;
    if constexpr (TAB) {
        if (e >= 0) {
            const moe_weights_t V = table_view(a, e);
            gate_up_tile_sw<WB, CPT, RPS, TT>(a, V, 0, row0, n_u, a.plan + pd.o_t + p0, p0, s_h, part);
            return;
        }
    }
    gate_up_tile_sw<WB, CPT, RPS, TT>(a, (e >= 0) ? a.routed : a.shared, (e >= 0) ? e : 0, row0, n_u,
                                      a.plan + pd.o_t + p0, p0, s_h, part);
}

constexpr int kDsThreads = 256;  // down row-sweep block
constexpr int kDsGroups = kDsThreads / 32;
constexpr int kDsRows = 16;      // output rows per workgroup
static_assert(kDsRows == kGemvDownRows, "rows per down workgroup (LDS sizing)");

// slot buffers of the down kernel's ring: two slots of rows in flight ahead
// of the one in use (measured on MI355X: a ring that holds every slot of a
// one-token plan at once ran ~1.5 us slower, its first use waiting for all)
constexpr int kDownRing = 3;

// down/combine: a step reads RPS consecutive down rows of one slot (4 KB);
// kDsRows rows per workgroup, every slot in turn through a ring of NB slot
// buffers.  MB: the plan's pairs take more than one staging batch.
// EARLY (one routed token with a shared expert): nothing the shared slot and
// the staging read depends on the plan (every pair is staged, pair p at
// LDS index p, and the shared expert's rows are known), so they are
// requested together with the plan, one dependent round trip fewer, and
// the shared slot is combined first.
// TAB: routed experts through the expert table (a.toff).
template <int WB, int RPS, int TT, int NB, bool MB, bool EARLY = false, bool TAB = false>
__global__ __launch_bounds__(kDsThreads) void k_down_sw(const GemvArgs a, const ChunkCfg cc, const PlanDims pd)
{
    static_assert(!(EARLY && (MB || TT != 1)), "the early prologue is for one token, one batch");
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ float part[TT][kDsGroups][kDsRows];
    // EARLY: one record per slot (slot_record.h), formed once after the
    // plan barrier
    static_assert(kMaxTopK + 1 <= kRecordMaxPair, "a record's staged pair index");
    __shared__ int4 sdesc[EARLY ? kMaxTopK + 1 : 1];
    constexpr int NSTEP = kDsRows / RPS;
    const int tid = threadIdx.x, lane = lane_id();
    const int I = a.I, nbh = I / 32, cpr = cc.cpr;
    int *plan = reinterpret_cast<int *>(lds);
    const int plan_words = (pd.words + 3) & ~3;
    unsigned char *act = lds + sizeof(int) * plan_words;
    const size_t pair_bytes = act_lds_bytes(WB, I);
    auto la_of = [&](int p) { return reinterpret_cast<uint32_t *>(act + p * pair_bytes); };
    auto ld_of = [&](int p) { return reinterpret_cast<float *>(act + p * pair_bytes + I); };
    // every slot's kDsRows row scales, [slot][row], after a.down_pmax pairs
    float *lsc = reinterpret_cast<float *>(act + (size_t)a.down_pmax * pair_bytes);

    int pv = 0;
    if constexpr (EARLY) {
        pv = a.plan[min(tid, pd.words - 1)];  // pd.words <= kDsThreads (checked on the host)
    } else {
        for (int i = tid; i < pd.words; i += kDsThreads) plan[i] = a.plan[i];
        __syncthreads();
        if (!plan_ok(plan, pd, a.T, a.E) || plan[0] < 1) return;
    }
    // with EARLY, S and every plan entry are read only after the plan
    // barrier further down
    int S = EARLY ? 1 : plan[0];
    // every slot's pairs must fit one staging batch (the host sizes
    // a.down_pmax >= T; a plan that breaks it writes nothing)
    if constexpr (MB) {
        for (int u = 0; u < S; u++)
            if (plan[pd.o_n + u] > a.down_pmax) return;
    }
    // thread i < T * kDsRows writes output (token i / kDsRows, row i % kDsRows);
    // with MOE_ACCUMULATE it adds to the value read here, at the start
    static_assert(kGemvMaxT * kDsRows <= kDsThreads, "one output per thread");
    const float y_old = [&] {
        const int i = min(tid, a.T * kDsRows - 1);
        return a.y[(size_t)(i / kDsRows) * a.H + blockIdx.x * kDsRows + i % kDsRows];
    }();
    // processing order of the slots: the shared (last) slot first with EARLY
    auto slot_at = [&](int v) { return EARLY ? (v == 0 ? S - 1 : v - 1) : v; };

    const int rowoff = tid / cpr, pos = tid % cpr, grp = tid >> 5;
    const int row_base = blockIdx.x * kDsRows;
    const size_t rowbytes = (size_t)cpr * 16;
    const size_t step_bytes = (size_t)kDsThreads * 16;
    auto slot_w = [&](int u) -> const moe_weights_t & { return plan[pd.o_e + u] >= 0 ? a.routed : a.shared; };
    auto slot_ee = [&](int u) { return max(plan[pd.o_e + u], 0); };
    // the first of the workgroup's rows of slot u
    auto slot_rows = [&](int u) {
        if constexpr (TAB) {
            const int e = plan[pd.o_e + u];
            const int64_t off = a.toff[(size_t)max(e, 0) * 6 + 2];
            const uint8_t *b = (e >= 0) ? a.routed.down + off : a.shared.down;
            return b + (size_t)row_base * rowbytes;
        }
        return slot_w(u).down + ((size_t)slot_ee(u) * a.H + row_base) * rowbytes;
    };
    // the slot's base address is workgroup-uniform (scalar registers): the
    // loads then take a fixed per-lane offset
    auto slot_src = [&](int u) { return slot_rows(__builtin_amdgcn_readfirstlane(u)) + (size_t)tid * 16; };
    float acc[TT][NSTEP];
#pragma unroll
    for (int tt = 0; tt < TT; tt++)
#pragma unroll
        for (int j = 0; j < NSTEP; j++) acc[tt][j] = 0.f;

    // a ring of NB slot buffers, NB - 1 slots of rows in flight ahead of use
    // (every index into the ring is static once the loops are unrolled, so
    // the buffers stay in registers)
    uint4 wr[NB][NSTEP];
    auto load_rows = [&](const uint8_t *src, uint4 (&wb)[NSTEP]) {
#pragma unroll
        for (int j = 0; j < NSTEP; j++) wb[j] = ld16(src + j * step_bytes);
    };
    auto load_slot = [&](int u, uint4 (&wb)[NSTEP]) { load_rows(slot_src(u), wb); };
    constexpr int SB = stage_batch(WB);
    const int pmax = a.down_pmax;
    int nsc = S * kDsRows;
    int p0s = EARLY ? 0x7fffffff : (plan[pd.o_e + S - 1] == -1) ? plan[pd.o_p0 + S - 1] : 0x7fffffff;
    int bend = 0, rbase = 0, rcount = 0, nst = 0;  // the batch: slots .. bend - 1
    auto batch_from = [&](int s0) {
        int np = 0, nr = 0, s1 = s0;
        while (s1 < S) {
            const int n = plan[pd.o_n + s1];
            if (np + n > pmax) break;
            np += n;
            if (plan[pd.o_e + s1] != -1) nr += n;
            s1++;
        }
        bend = s1;
        rbase = plan[pd.o_p0 + s0];
        rcount = nr;
        nst = np * cpr;
    };
    // staged index of pair p of the current batch
    auto lidx = [&](int p) { return p >= p0s ? rcount + (p - p0s) : p - rbase; };
    auto pair_of = [&](int i) { return i < rcount ? rbase + i : p0s + (i - rcount); };
    // a slot's pairs list its tokens in ascending order: walk the tokens in
    // compile-time order so every accumulator index is static
    auto use_slot = [&](int u, const uint4 (&wb)[NSTEP]) {
        const int n = plan[pd.o_n + u], p0 = plan[pd.o_p0 + u];
        float sb[NSTEP];
#pragma unroll
        for (int j = 0; j < NSTEP; j++) sb[j] = lsc[u * kDsRows + j * RPS + rowoff];
        int q = 0;
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
            if (q < n && plan[pd.o_t + p0 + q] == tt) {
                const int p = p0 + q, li = lidx(p);
                const float pw = __int_as_float(plan[pd.o_w + p]);
                Act<WB> A;
                act_from_lds<WB>(A, la_of(li), ld_of(li), pos, cpr);
#pragma unroll
                for (int j = 0; j < NSTEP; j++) acc[tt][j] += A.dot(wb[j]) * (pw * sb[j]);
                q++;
            }
        }
    };
    // the same for one token from the slot's record (li: staged pair, -1 for none)
    auto use_slot1 = [&](int u, const uint4 (&wb)[NSTEP], int li, float pw) {
        float sb[NSTEP];
#pragma unroll
        for (int j = 0; j < NSTEP; j++) sb[j] = lsc[u * kDsRows + j * RPS + rowoff];
        if (li >= 0) {
            Act<WB> A;
            act_from_lds<WB>(A, la_of(li), ld_of(li), pos, cpr);
#pragma unroll
            for (int j = 0; j < NSTEP; j++) acc[0][j] += A.dot(wb[j]) * (pw * sb[j]);
        }
    };
    // Staging.  Every slot's row scales go to LDS once.  The pairs' int8 h
    // go in batches of consecutive slots whose pairs fit the LDS pair space
    // (a.down_pmax pairs): the whole plan at one token, a few batches for
    // larger verify batches, so every routed expert of the batch is read
    // once whatever its size.  A batch holds the routed pairs of its slots
    // (consecutive pair numbers from rbase) and, when it reaches the last
    // slot, the shared expert's pairs after them.  SB chunks (and one scale)
    // per thread per round of loads; spare lanes of the last round take the
    // last chunk or scale again (same value, same place), so no load or
    // store sits under a per-lane branch.
    Act<WB> sa[SB];
    int scs[SB];
    float scv;
    int sci;
    auto stage_issue = [&](int c0) {
#pragma unroll
        for (int b = 0; b < SB; b++) {
            scs[b] = min(c0 + b * kDsThreads + tid, nst - 1);
            const int i = scs[b] / cpr, pp = scs[b] - i * cpr, p = pair_of(i);
            sa[b].load_raw(a.qh + (size_t)p * I, a.dh + (size_t)p * nbh, pp);
        }
    };
    auto stage_store = [&]() {
#pragma unroll
        for (int b = 0; b < SB; b++) {
            const int i = scs[b] / cpr, pp = scs[b] - i * cpr;
            sa[b].finish();
            store_act<WB>(sa[b], pp, cpr, la_of(i), ld_of(i));
        }
    };
    auto scale_issue = [&](int i0) {
        sci = min(i0 + tid, nsc - 1);
        const int u = sci / kDsRows;
        if constexpr (TAB) {
            const int e = plan[pd.o_e + u];
            const int64_t off = a.toff[(size_t)max(e, 0) * 6 + 5];
            const float *b = (e >= 0) ? reinterpret_cast<const float *>(
                                            reinterpret_cast<const uint8_t *>(a.routed.down_s) + off)
                                      : a.shared.down_s;
            scv = b[row_base + sci % kDsRows];
        } else {
            scv = slot_w(u).down_s[(size_t)slot_ee(u) * a.H + row_base + sci % kDsRows];
        }
    };
    auto stage_rest = [&](int c0) {
        for (; c0 < nst; c0 += SB * kDsThreads) {
            stage_issue(c0);
            stage_store();
        }
    };
    // The first round of the first batch, the first scales and then the
    // first NB - 1 slots' rows are requested together, one plan round trip
    // into the kernel; the staging stores wait for the staging loads only
    // (the vector memory counter retires loads in issue order).  A plan with
    // fewer slots requests its last slot again: straight-line code, so that
    // wait counts exactly the loads issued after the staging.
    if constexpr (EARLY) {
        // every pair at its own index (pairs a top-p drop leaves are staged
        // and never read), the shared expert's rows, then the plan itself
        rbase = 0; rcount = pd.P; nst = pd.P * cpr;
        stage_issue(0);
        load_rows(a.shared.down + (size_t)row_base * rowbytes + (size_t)tid * 16, wr[0]);
        __builtin_amdgcn_sched_barrier(0);
        if (tid < pd.words) plan[tid] = pv;
        __syncthreads();
        if (!plan_ok(plan, pd, a.T, a.E) || plan[0] < 1) return;
        S = plan[0];
        if (plan[pd.o_e + S - 1] != -1) return;  // the shared slot is last
        nsc = S * kDsRows;
        bend = S;
        if (tid < S) {  // the slot records (a pair is used when its token is 0)
            const int n = plan[pd.o_n + tid], p0 = plan[pd.o_p0 + tid];
            const bool sh = plan[pd.o_e + tid] < 0;
            const bool use = n > 0 && plan[pd.o_t + p0] == 0;
            SlotRecord rec;
            rec.off = slot_rows(tid) - (sh ? a.shared.down : a.routed.down);
            rec.pair = use ? lidx(p0) : -1;
            rec.shared = sh;
            rec.w_bits = use ? plan[pd.o_w + p0] : 0;
            int w[4];
            record_pack(rec, w);
            sdesc[tid] = make_int4(w[0], w[1], w[2], w[3]);
        }
        scale_issue(0);
#pragma unroll
        for (int b = 1; b < NB - 1; b++) load_slot(slot_at(min(b, S - 1)), wr[b]);
    } else {
        if constexpr (MB) {
            batch_from(0);
        } else {  // one batch: every pair (no data-dependent walk before the first loads)
            const PlanPairs pq = plan_pairs(plan, pd);
            bend = S; rbase = 0; rcount = pq.R; nst = pq.count() * cpr;
        }
        stage_issue(0);
        scale_issue(0);
#pragma unroll
        for (int b = 0; b < NB - 1; b++) load_slot(min(b, S - 1), wr[b]);
    }
    // keep every load above issued before the first use of any of them
    __builtin_amdgcn_sched_barrier(0);
    stage_store();
    lsc[sci] = scv;
    for (int i0 = kDsThreads; i0 < nsc; i0 += kDsThreads) {
        scale_issue(i0);
        lsc[sci] = scv;
    }
    stage_rest(SB * kDsThreads);
    __syncthreads();
    // EARLY: the record fields of the ring's slots (scalar registers)
    int dli[NB];
    float dpw[NB];
    auto take_record = [&](int u, int r) {
        const int4 d = sdesc[u];
        const SlotRecord rec = record_unpack(__builtin_amdgcn_readfirstlane(d.x), __builtin_amdgcn_readfirstlane(d.y),
                                             __builtin_amdgcn_readfirstlane(d.z), __builtin_amdgcn_readfirstlane(d.w));
        dli[r] = rec.pair;
        dpw[r] = __int_as_float(rec.w_bits);
        // from the weights' own base pointers, so the loads stay global ones
        return (rec.shared ? a.shared.down : a.routed.down) + rec.off;
    };
    if constexpr (EARLY) {
#pragma unroll
        for (int b = 0; b < NB - 1; b++) take_record(slot_at(min(b, S - 1)), b);
    }
    for (int u0 = 0; u0 < S; u0 += NB) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int u = u0 + b;
            // unconditional (past the end: the last slot again, an L2 hit),
            // so the ring's registers carry no merge of loaded and unloaded
            // values and every wait counts the ring's loads exactly
            if constexpr (EARLY) {
                const int r = (b + NB - 1) % NB;
                load_rows(take_record(slot_at(min(u + NB - 1, S - 1)), r) + (size_t)tid * 16, wr[r]);
            } else {
                load_slot(slot_at(min(u + NB - 1, S - 1)), wr[(b + NB - 1) % NB]);
            }
            if (MB && u < S && u == bend) {  // next batch of pairs (uniform)
                __syncthreads();
                batch_from(u);
                stage_rest(0);
                __syncthreads();
            }
            // issue priority falls over the slots (as in the gate/up sweep)
            if (u == 0) __builtin_amdgcn_s_setprio(3);
            if (u == S / 4) __builtin_amdgcn_s_setprio(2);
            if (u == S / 2) __builtin_amdgcn_s_setprio(1);
            if (u == (3 * S) / 4) __builtin_amdgcn_s_setprio(0);
            if (u < S) {
                if constexpr (EARLY) use_slot1(slot_at(u), wr[b], dli[b], dpw[b]);
                else use_slot(slot_at(u), wr[b]);
            }
        }
    }
    const int l32 = lane & 31;
    const int jj = l32 / (32 / NSTEP);
    const bool writer = (l32 % (32 / NSTEP)) == 0;
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        if (tt < a.T) {
            const float v = group32_reduce_scatter<NSTEP>(acc[tt]);
            if (writer) part[tt][grp][jj * RPS + rowoff] = v;
        }
    }
    __syncthreads();
    const int groups_per_row = cpr / 32;
    if (tid < a.T * kDsRows) {
        const int tt = tid / kDsRows, r = tid % kDsRows, g0 = (r % RPS) * groups_per_row;
        float v = 0.f;
        for (int q = 0; q < groups_per_row; q++) v += part[tt][g0 + q][r];
        a.y[(size_t)tt * a.H + row_base + r] = a.accumulate ? y_old + v : v;
    }
}

// lookahead workgroups of a launch: la_wgs per predicted rank, and per
// shared expert of the next layer (one-token launches that route inline)
static int lookahead_wgs(const GemvArgs &a)
{
    if (!a.la_logits || a.la_wgs <= 0 || !a.inline_route || a.toff) return 0;
    return a.la_wgs * (a.rc.k + (a.la_shared.gate ? 1 : 0));
}

template <int WB, int CPT, int RPS, int TT, bool TAB = false>
static int run_gate_up_sw(const GemvArgs &a, const ChunkCfg &cc, const PlanDims &pd, hipStream_t st)
{
    // the sweep's row width (kSwThreads * CPT / RPS chunks) must be the row's
    if (cc.cpr * RPS != kSwThreads * CPT) return (int)hipErrorInvalidValue;
    k_gate_up_sw<WB, CPT, RPS, TT, TAB><<<pd.S * (a.I / 32) + lookahead_wgs(a), kSwThreads, 0, st>>>(a, cc, pd);
    return (int)hipGetLastError();
}

template <int WB, int RPS, int TT, bool TAB = false>
static int run_down_sw(const GemvArgs &a, const ChunkCfg &cc, const PlanDims &pd, hipStream_t st)
{
    constexpr int NB = kDownRing;
    // a step covers RPS whole rows: a row of cc.cpr chunks must tile the block
    if (cc.cpr * RPS != kDsThreads) return (int)hipErrorInvalidValue;
    const size_t lds = down_sw_lds_bytes(WB, a.I, pd, a.down_pmax);
    // one staging batch holds every pair (one token at the production
    // shapes): the kernel without the batch switch in its slot loop
    if constexpr (TT == 1) {
        if (a.T == 1 && a.logits && a.n_shared == 1 && pd.words <= kDsThreads && a.down_pmax >= pd.P) {
            k_down_sw<WB, RPS, TT, NB, false, true, TAB><<<a.H / kDsRows, kDsThreads, lds, st>>>(a, cc, pd);
            return (int)hipGetLastError();
        }
    }
    if (a.down_pmax >= pd.P)
        k_down_sw<WB, RPS, TT, NB, false, false, TAB><<<a.H / kDsRows, kDsThreads, lds, st>>>(a, cc, pd);
    else k_down_sw<WB, RPS, TT, NB, true, false, TAB><<<a.H / kDsRows, kDsThreads, lds, st>>>(a, cc, pd);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- dispatch
static int tt_for(int T) { return T <= 1 ? 1 : (T <= 4 ? 4 : 8); }

// which row-sweep variant a row of cpr chunks takes (0: none, use the
// row-group kernels)
static int gate_up_sw_kind(int cpr) { return cpr == 192 ? 1 : cpr == 384 ? 2 : cpr == 96 ? 3 : 0; }
static int down_sw_kind(int cpr) { return cpr == 64 ? 1 : cpr == 128 ? 2 : cpr == 32 ? 3 : 0; }

template <int WB, int TT>
static int run_gate_up(const GemvArgs &a, const ChunkCfg &cc, const PlanDims &pd, hipStream_t st)
{
    const int grid = pd.S * (a.I / 32);
    const size_t lds = a.T * act_lds_bytes(WB, a.H);
    k_gate_up_rg<WB, TT><<<grid, 256, lds, st>>>(a, cc, pd);
    return (int)hipGetLastError();
}

template <int WB, int TT>
static int run_down(const GemvArgs &a, const ChunkCfg &cc, const PlanDims &pd, hipStream_t st)
{
    static_assert(kDnRows == kGemvDownRows, "rows per down workgroup");
    k_down_rg<WB, TT><<<a.H / kDnRows, 256, down_lds_bytes(WB, a.I, pd), st>>>(a, cc, pd);
    return (int)hipGetLastError();
}

#define MOE_DISPATCH(FN)                                                        \
    switch (a.wbits * 16 + tt_for(a.T)) {                                       \
    case 2 * 16 + 1: return FN<2, 1>(a, cc, pd, st);                            \
    case 2 * 16 + 4: return FN<2, 4>(a, cc, pd, st);                            \
    case 2 * 16 + 8: return FN<2, 8>(a, cc, pd, st);                            \
    case 4 * 16 + 1: return FN<4, 1>(a, cc, pd, st);                            \
    case 4 * 16 + 4: return FN<4, 4>(a, cc, pd, st);                            \
    case 4 * 16 + 8: return FN<4, 8>(a, cc, pd, st);                            \
    case 8 * 16 + 1: return FN<8, 1>(a, cc, pd, st);                            \
    case 8 * 16 + 4: return FN<8, 4>(a, cc, pd, st);                            \
    default: return FN<8, 8>(a, cc, pd, st);                                    \
    }

#define MOE_SW_TT(FN, ...)                                                      \
    switch (tt_for(a.T)) {                                                      \
    case 1: return FN<__VA_ARGS__, 1>(a, cc, pd, st);                           \
    case 4: return FN<__VA_ARGS__, 4>(a, cc, pd, st);                           \
    default: return FN<__VA_ARGS__, 8>(a, cc, pd, st);                          \
    }

// The production row widths take the token count of the chunk exactly (up
// to 6; 7 and 8 share 8): per-token accumulators and activations are live
// registers, and a kernel sized for 8 tokens runs one wave per SIMD.
#define MOE_SW_TTX(FN, ...)                                                     \
    switch (a.T <= 6 ? a.T : 8) {                                               \
    case 1: return FN<__VA_ARGS__, 1>(a, cc, pd, st);                           \
    case 2: return FN<__VA_ARGS__, 2>(a, cc, pd, st);                           \
    case 3: return FN<__VA_ARGS__, 3>(a, cc, pd, st);                           \
    case 4: return FN<__VA_ARGS__, 4>(a, cc, pd, st);                           \
    case 5: return FN<__VA_ARGS__, 5>(a, cc, pd, st);                           \
    case 6: return FN<__VA_ARGS__, 6>(a, cc, pd, st);                           \
    default: return FN<__VA_ARGS__, 8>(a, cc, pd, st);                          \
    }

bool gemv_gate_up_sw(const moe_shape_t &s)
{
    ChunkCfg cc;
    return chunk_cfg(s.hidden, s.wbits, cc) && gate_up_sw_kind(cc.cpr) != 0;
}

bool gemv_down_sw(const moe_shape_t &s)
{
    ChunkCfg cc;
    return s.hidden % kDsRows == 0 && chunk_cfg(s.inter, s.wbits, cc) && down_sw_kind(cc.cpr) != 0;
}

bool gemv_table_ok(const moe_shape_t &s)
{
    ChunkCfg cg, cd;
    return s.wbits == 4 && s.hidden % kDsRows == 0 && chunk_cfg(s.hidden, 4, cg) && gate_up_sw_kind(cg.cpr) == 1 &&
           chunk_cfg(s.inter, 4, cd) && down_sw_kind(cd.cpr) == 1;
}

bool gemv_inline_route(const moe_shape_t &s, int T)
{
    ChunkCfg cc;
    return T == 1 && chunk_cfg(s.hidden, s.wbits, cc) && gate_up_sw_kind(cc.cpr) != 0;
}

int launch_gate_up(const GemvArgs &a, hipStream_t st)
{
    ChunkCfg cc;
    if (!chunk_cfg(a.H, a.wbits, cc)) return (int)hipErrorInvalidValue;
    const PlanDims pd = plan_dims(a.T, a.rc.k, a.n_shared, a.logits == nullptr);
    const int kind = gate_up_sw_kind(cc.cpr);
    if (a.toff) {  // expert table: the int4 production row widths (checked by the caller)
        if (kind != 1 || a.wbits != 4) return (int)hipErrorInvalidValue;
        return a.T == 1 ? run_gate_up_sw<4, 1, 1, 1, true>(a, cc, pd, st)
                        : run_gate_up_sw<4, 1, 1, 8, true>(a, cc, pd, st);
    }
    if (kind == 1 && a.wbits == 4) { MOE_SW_TTX(run_gate_up_sw, 4, 1, 1) }
    if (kind == 1 && a.wbits == 8) { MOE_SW_TT(run_gate_up_sw, 8, 1, 1) }
    if (kind == 1 && a.wbits == 2) { MOE_SW_TT(run_gate_up_sw, 2, 1, 1) }
    if (kind == 2 && a.wbits == 8) { MOE_SW_TTX(run_gate_up_sw, 8, 2, 1) }
    if (kind == 2 && a.wbits == 4) { MOE_SW_TT(run_gate_up_sw, 4, 2, 1) }
    if (kind == 3 && a.wbits == 2) { MOE_SW_TTX(run_gate_up_sw, 2, 1, 2) }
    if (kind == 3 && a.wbits == 4) { MOE_SW_TT(run_gate_up_sw, 4, 1, 2) }
    MOE_DISPATCH(run_gate_up)
}

int launch_down(const GemvArgs &args, hipStream_t st)
{
    ChunkCfg cc;
    if (!chunk_cfg(args.I, args.wbits, cc)) return (int)hipErrorInvalidValue;
    const PlanDims pd = plan_dims(args.T, args.rc.k, args.n_shared, args.logits == nullptr);
    GemvArgs a = args;
    a.down_pmax = down_pair_cap(a.wbits, a.I, pd);
    const int kind = down_sw_kind(cc.cpr);
    if (a.toff) {
        if (kind != 1 || a.wbits != 4 || a.H % kDsRows) return (int)hipErrorInvalidValue;
        return a.T == 1 ? run_down_sw<4, kDsThreads / 64, 1, true>(a, cc, pd, st)
                        : run_down_sw<4, kDsThreads / 64, 8, true>(a, cc, pd, st);
    }
    if (a.H % kDsRows == 0) {
        if (kind == 1 && a.wbits == 4) { MOE_SW_TTX(run_down_sw, 4, kDsThreads / 64) }
        if (kind == 1 && a.wbits == 8) { MOE_SW_TT(run_down_sw, 8, kDsThreads / 64) }
        if (kind == 1 && a.wbits == 2) { MOE_SW_TT(run_down_sw, 2, kDsThreads / 64) }
        if (kind == 2 && a.wbits == 8) { MOE_SW_TTX(run_down_sw, 8, kDsThreads / 128) }
        if (kind == 2 && a.wbits == 4) { MOE_SW_TT(run_down_sw, 4, kDsThreads / 128) }
        if (kind == 3 && a.wbits == 2) { MOE_SW_TTX(run_down_sw, 2, kDsThreads / 32) }
        if (kind == 3 && a.wbits == 4) { MOE_SW_TT(run_down_sw, 4, kDsThreads / 32) }
    }
    MOE_DISPATCH(run_down)
}

} // namespace moe

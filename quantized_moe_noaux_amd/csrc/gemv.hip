// Batch-union GEMV path of the MoE layer (decode and small verify batches).
//
// GeekNews #31297, implemented features: batch-union MoE reads each unique
// expert of a batch once and applies it to every position routed to it; the
// experts are SwiGLU FFNs over int8 / packed int4 / packed int2 codes with
// per-row scales, evaluated as integer dots on Q8_0-style int8 activations.
// wpnews.pro spec table: 8 routed + 1 shared expert per token.
//
// Two kernels:
//  k_gate_up  one workgroup per (slot, 32-row tile) of the intermediate
//             dimension, slot = one expert of the batch union (or the shared
//             expert).  Every workgroup re-derives the routing of the batch
//             from the fp64 logits (a few hundred instructions per token), so
//             no extra launch or inter-workgroup counter is needed; block 0
//             publishes it.  Per row: g and u as integer block dots streamed
//             with 16-byte loads, h = silu(g) * u, and h quantised to int8 in
//             blocks of 32 rows (one workgroup tile = one block).
//  k_down     one workgroup per tile of output rows; for each row it streams
//             the down rows of all slots, dots them with the slots' int8 h
//             (staged once in LDS), scales by combine weight x row scale and
//             sums per token in a fixed order: the combine is fused, no float
//             atomics, results are run-to-run identical.
#include "moe_dev.h"
#include "moe_internal.h"
#include "topk_dev.h"

namespace moe {

bool chunk_cfg(int in_dim, int wbits, ChunkCfg &cc)
{
    int rowbytes = in_dim * wbits / 8;
    if (rowbytes % 16) return false;
    cc.cpr = rowbytes / 16;
    int g = 64, a = cc.cpr;
    while (a % g) g >>= 1;  // gcd(cpr, 64)
    cc.rw = 64 / g;
    cc.cpl = cc.rw * cc.cpr / 64;
    return cc.rw <= 32 && (cc.cpl == 1 || cc.cpl == 2 || cc.cpl == 3 || cc.cpl == 6);
}

GemvWs gemv_ws(const moe_shape_t &s, int T, bool single)
{
    GemvWs w;
    const int H = s.hidden, I = s.inter, E = s.n_experts;
    // plan and h buffers hold one chunk of at most kGemvMaxT tokens
    PlanDims pd = plan_dims(T < kGemvMaxT ? T : kGemvMaxT, s.top_k, s.n_shared, single);
    size_t o = 0;
    w.logits = o; o = align256(o + sizeof(double) * (size_t)T * E);
    w.xq = o;     o = align256(o + (size_t)T * H);
    w.xd = o;     o = align256(o + sizeof(float) * (size_t)T * (H / 32));
    w.plan = o;   o = align256(o + sizeof(int) * (size_t)pd.words);
    w.qh = o;     o = align256(o + (size_t)pd.P * I);
    w.dh = o;     o = align256(o + sizeof(float) * (size_t)pd.P * (I / 32));
    w.total = o;
    return w;
}

// ---------------------------------------------------------------- block scan
// Exclusive scan of up to 512 ints, two per thread of a 256-thread block.
__device__ int block_scan2(int v0, int v1, int &o0, int &o1, int *tmp /*[4]*/)
{
    const int lane = lane_id(), wv = wave_id();
    int s = v0 + v1, inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(inc, o);
        if (lane >= o) inc += n;
    }
    if (lane == 63) tmp[wv] = inc;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        if (w < wv) base += tmp[w];
        total += tmp[w];
    }
    __syncthreads();
    o0 = base + inc - s;
    o1 = o0 + v0;
    return total;
}

// Builds the batch-union plan in LDS (all threads of the block take part).
// Slots hold the union of the routed experts in ascending expert order, then
// the shared expert; pairs of a slot list its tokens in ascending order.
__device__ void build_plan(const GemvArgs &a, const PlanDims &pd, int *plan, int *s_idx, float *s_w,
                           int *s_slot, int *tmp)
{
    const int tid = threadIdx.x, T = a.T, k = a.rc.k;
    int *slot_e = plan + pd.o_e, *slot_n = plan + pd.o_n, *slot_p0 = plan + pd.o_p0;
    int *pair_t = plan + pd.o_t;
    float *pair_w = reinterpret_cast<float *>(plan + pd.o_w);
    if (!a.logits) {  // single expert, all tokens, weight 1
        if (tid == 0) { plan[0] = 1; slot_e[0] = a.single; slot_n[0] = T; slot_p0[0] = 0; }
        for (int t = tid; t < T; t += 256) { pair_t[t] = t; pair_w[t] = 1.0f; }
        __syncthreads();
        return;
    }
    for (int t = wave_id(); t < T; t += 4)
        wave_topk(a.rc, a.logits + (size_t)t * a.E, a.bias, s_idx + t * k, s_w + t * k);
    for (int e = tid; e < kMaxExperts; e += 256) s_slot[e] = 0;
    __syncthreads();
    for (int i = tid; i < T * k; i += 256) s_slot[s_idx[i]] = 1;
    __syncthreads();
    int f0 = s_slot[2 * tid], f1 = s_slot[2 * tid + 1], o0, o1;
    const int U = block_scan2(f0, f1, o0, o1, tmp);
    __syncthreads();
    if (f0) { s_slot[2 * tid] = o0; slot_e[o0] = 2 * tid; }
    if (f1) { s_slot[2 * tid + 1] = o1; slot_e[o1] = 2 * tid + 1; }
    const int S = U + a.n_shared;
    for (int u = tid; u < S; u += 256) slot_n[u] = (u < U) ? 0 : T;
    if (tid == 0) {
        plan[0] = S;
        if (a.n_shared) slot_e[U] = -1;
    }
    __syncthreads();
    for (int i = tid; i < T * k; i += 256) atomicAdd(&slot_n[s_slot[s_idx[i]]], 1);
    __syncthreads();
    int n0 = (2 * tid < S) ? slot_n[2 * tid] : 0, n1 = (2 * tid + 1 < S) ? slot_n[2 * tid + 1] : 0;
    block_scan2(n0, n1, o0, o1, tmp);
    if (2 * tid < S) slot_p0[2 * tid] = o0;
    if (2 * tid + 1 < S) slot_p0[2 * tid + 1] = o1;
    __syncthreads();
    for (int i = tid; i < T * k; i += 256) {
        const int t = i / k, e = s_idx[i];
        int r = 0;
        for (int j = 0; j < t * k; j++) r += (s_idx[j] == e);
        const int p = slot_p0[s_slot[e]] + r;
        pair_t[p] = t;
        pair_w[p] = s_w[i];
    }
    if (a.n_shared)
        for (int t = tid; t < T; t += 256) {
            pair_t[slot_p0[U] + t] = t;
            pair_w[slot_p0[U] + t] = 1.0f;
        }
    __syncthreads();
}

// ---------------------------------------------------------------- gate / up
template <int WB, int CPL, int TT>
__global__ __launch_bounds__(256) void k_gate_up(const GemvArgs a, const ChunkCfg cc, const PlanDims pd)
{
    __shared__ int plan[1 + 3 * (kGemvMaxT * kMaxTopK + 1) + 2 * kGemvMaxT * (kMaxTopK + 1)];
    __shared__ int s_idx[kGemvMaxT * kMaxTopK];
    __shared__ float s_w[kGemvMaxT * kMaxTopK];
    __shared__ int s_slot[kMaxExperts];
    __shared__ int tmp[4];
    __shared__ float s_h[TT][32];

    build_plan(a, pd, plan, s_idx, s_w, s_slot, tmp);
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    if (blockIdx.x == 0) {
        for (int i = tid; i < pd.words; i += 256) a.plan[i] = plan[i];
        if (a.logits && a.idx_out)
            for (int i = tid; i < a.T * a.rc.k; i += 256) { a.idx_out[i] = s_idx[i]; a.w_out[i] = s_w[i]; }
    }
    const int tiles = a.I / 32;
    const int u = blockIdx.x / tiles, row0 = (blockIdx.x % tiles) * 32;
    if (u >= plan[0]) return;
    const int e = plan[pd.o_e + u];
    const moe_weights_t &W = (e >= 0) ? a.routed : a.shared;
    const int ee = (e >= 0) ? e : 0;
    const size_t rowbytes = (size_t)cc.cpr * 16;
    const uint8_t *gate = W.gate + (size_t)ee * a.I * rowbytes;
    const uint8_t *up = W.up + (size_t)ee * a.I * rowbytes;
    const float *gs = W.gate_s + (size_t)ee * a.I, *us = W.up_s + (size_t)ee * a.I;
    const int n_u = plan[pd.o_n + u], p0 = plan[pd.o_p0 + u];
    const int nb = a.H / 32;

    // lane's chunks inside a wave tile: row offset and position in the row
    int crow[CPL], cpos[CPL];
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        int g = lane + 64 * i;
        crow[i] = g / cc.cpr;
        cpos[i] = g - crow[i] * cc.cpr;
    }

    for (int j0 = 0; j0 < n_u; j0 += TT) {
        const int nt = min(TT, n_u - j0);
        Act<WB> act[TT][CPL];
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
            if (tt < nt) {
                const int t = plan[pd.o_t + p0 + j0 + tt];
#pragma unroll
                for (int i = 0; i < CPL; i++) {
                    act[tt][i].load(a.xq + (size_t)t * a.H, a.xd + (size_t)t * nb, cpos[i]);
                }
            }
        }
        for (int tile = wv; tile < 32 / cc.rw; tile += 4) {
            const int rb = row0 + tile * cc.rw;
            uint4 wg[CPL], wu[CPL];
#pragma unroll
            for (int i = 0; i < CPL; i++) {
                const size_t off = (size_t)(rb + crow[i]) * rowbytes + (size_t)cpos[i] * 16;
                wg[i] = *reinterpret_cast<const uint4 *>(gate + off);
                wu[i] = *reinterpret_cast<const uint4 *>(up + off);
            }
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                if (tt < nt) {
                    float pg[CPL], pu[CPL];
#pragma unroll
                    for (int i = 0; i < CPL; i++) {
                        pg[i] = act[tt][i].dot(wg[i]);
                        pu[i] = act[tt][i].dot(wu[i]);
                    }
                    for (int r = 0; r < cc.rw; r++) {
                        float vg = 0.f, vu = 0.f;
#pragma unroll
                        for (int i = 0; i < CPL; i++)
                            if (crow[i] == r) { vg += pg[i]; vu += pu[i]; }
                        vg = wave_sum(vg) * gs[rb + r];
                        vu = wave_sum(vu) * us[rb + r];
                        if (lane == 0) s_h[tt][tile * cc.rw + r] = silu_mul(vg, vu);
                    }
                }
            }
        }
        __syncthreads();
        // quantise h per token: one block of 32 rows, lanes 0..31 of a wave
        for (int tt = wv; tt < nt; tt += 4) {
            const int p = p0 + j0 + tt;
            float h = s_h[tt][lane & 31];
            float amax = fabsf(h);
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
            float d = amax / 127.0f;
            float r = (d == 0.0f) ? 0.0f : rintf(h / d);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            if (lane < 32) a.qh[(size_t)p * a.I + row0 + lane] = (int8_t)(int)r;
            if (lane == 0) a.dh[(size_t)p * (a.I / 32) + row0 / 32] = d;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- down / combine
template <int WB> struct ActShape;
template <> struct ActShape<8> { static constexpr int NA = 4, NB = 1; };   // dwords, blocks per chunk (x2 chunks per block)
template <> struct ActShape<4> { static constexpr int NA = 8, NB = 1; };
template <> struct ActShape<2> { static constexpr int NA = 16, NB = 2; };

template <int WB>
__device__ __forceinline__ void act_from_lds(Act<WB> &A, const uint32_t *la, const float *ld, const int *lq, int pos)
{
    const uint32_t *src = la + pos * ActShape<WB>::NA;
    if constexpr (WB == 8) {
        uint4 v = *reinterpret_cast<const uint4 *>(src);
        A.a[0] = v.x; A.a[1] = v.y; A.a[2] = v.z; A.a[3] = v.w;
        A.d = ld[pos >> 1];
    } else if constexpr (WB == 4) {
        uint4 v0 = reinterpret_cast<const uint4 *>(src)[0], v1 = reinterpret_cast<const uint4 *>(src)[1];
        A.a[0] = v0.x; A.a[1] = v0.y; A.a[2] = v0.z; A.a[3] = v0.w;
        A.a[4] = v1.x; A.a[5] = v1.y; A.a[6] = v1.z; A.a[7] = v1.w;
        A.d = ld[pos];
        A.qs = lq[pos];
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint4 v = reinterpret_cast<const uint4 *>(src)[i];
            A.a[4 * i] = v.x; A.a[4 * i + 1] = v.y; A.a[4 * i + 2] = v.z; A.a[4 * i + 3] = v.w;
        }
        A.d0 = ld[2 * pos]; A.d1 = ld[2 * pos + 1];
        A.qs0 = lq[2 * pos]; A.qs1 = lq[2 * pos + 1];
    }
}

template <int WB, int CPL, int TT>
__global__ __launch_bounds__(256) void k_down(const GemvArgs a, const ChunkCfg cc, const PlanDims pd,
                                              int rows_per_wg)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int I = a.I, nbh = I / 32;
    int *plan = reinterpret_cast<int *>(lds);
    const int plan_words = (pd.words + 3) & ~3;
    uint32_t *la = reinterpret_cast<uint32_t *>(plan + plan_words);  // [P][I/4] permuted codes
    float *ld = reinterpret_cast<float *>(la + (size_t)pd.P * (I / 4)); // [P][I/32] scales
    int *lq = reinterpret_cast<int *>(ld + (size_t)pd.P * nbh);         // [P][I/32] block sums

    for (int i = tid; i < pd.words; i += 256) plan[i] = a.plan[i];
    __syncthreads();
    const int S = plan[0];
    int npairs = 0;
    for (int u = 0; u < S; u++) npairs += plan[pd.o_n + u];
    // stage every pair's h codes in LDS, permuted for the weight layout
    const int cpr = cc.cpr;
    for (int c = tid; c < npairs * cpr; c += 256) {
        const int p = c / cpr, pos = c - p * cpr;
        const int8_t *q = a.qh + (size_t)p * I;
        Act<WB> A;
        if constexpr (WB == 8) {
            A.load(q, a.dh + (size_t)p * nbh, pos);
            *reinterpret_cast<uint4 *>(la + (size_t)p * (I / 4) + pos * 4) = make_uint4(A.a[0], A.a[1], A.a[2], A.a[3]);
        } else if constexpr (WB == 4) {
            A.load(q, a.dh + (size_t)p * nbh, pos);
            uint4 *dst = reinterpret_cast<uint4 *>(la + (size_t)p * (I / 4) + pos * 8);
            dst[0] = make_uint4(A.a[0], A.a[1], A.a[2], A.a[3]);
            dst[1] = make_uint4(A.a[4], A.a[5], A.a[6], A.a[7]);
            lq[(size_t)p * nbh + pos] = A.qs;
        } else {
            A.load(q, a.dh + (size_t)p * nbh, pos);
            uint4 *dst = reinterpret_cast<uint4 *>(la + (size_t)p * (I / 4) + pos * 16);
#pragma unroll
            for (int i = 0; i < 4; i++) dst[i] = make_uint4(A.a[4 * i], A.a[4 * i + 1], A.a[4 * i + 2], A.a[4 * i + 3]);
            lq[(size_t)p * nbh + 2 * pos] = A.qs0;
            lq[(size_t)p * nbh + 2 * pos + 1] = A.qs1;
        }
    }
    for (int c = tid; c < npairs * nbh; c += 256) ld[c] = a.dh[c];
    __syncthreads();

    int crow[CPL], cpos[CPL];
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        int g = lane + 64 * i;
        crow[i] = g / cpr;
        cpos[i] = g - crow[i] * cpr;
    }
    const size_t rowbytes = (size_t)cpr * 16;
    const int row_base = blockIdx.x * rows_per_wg;
    constexpr int UB = (CPL == 1) ? 8 : 4;  // slots whose rows are in flight together

    for (int tile = wv; tile < rows_per_wg / cc.rw; tile += 4) {
        const int rb = row_base + tile * cc.rw;
        float acc[TT][CPL];
#pragma unroll
        for (int tt = 0; tt < TT; tt++)
#pragma unroll
            for (int i = 0; i < CPL; i++) acc[tt][i] = 0.f;

        for (int u0 = 0; u0 < S; u0 += UB) {
            uint4 wd[UB][CPL];
            float sr[UB][CPL];
#pragma unroll
            for (int b = 0; b < UB; b++) {
                const int u = u0 + b;
                if (u < S) {
                    const int e = plan[pd.o_e + u];
                    const moe_weights_t &W = (e >= 0) ? a.routed : a.shared;
                    const int ee = (e >= 0) ? e : 0;
                    const uint8_t *down = W.down + (size_t)ee * a.H * rowbytes;
                    const float *ds = W.down_s + (size_t)ee * a.H;
#pragma unroll
                    for (int i = 0; i < CPL; i++) {
                        wd[b][i] = *reinterpret_cast<const uint4 *>(down + (size_t)(rb + crow[i]) * rowbytes +
                                                                    (size_t)cpos[i] * 16);
                        sr[b][i] = ds[rb + crow[i]];
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < UB; b++) {
                const int u = u0 + b;
                if (u < S) {
                    const int n = plan[pd.o_n + u], p0 = plan[pd.o_p0 + u];
                    for (int j = 0; j < n; j++) {
                        const int p = p0 + j;
                        const int t = plan[pd.o_t + p];
                        const float pw = __int_as_float(plan[pd.o_w + p]);
#pragma unroll
                        for (int i = 0; i < CPL; i++) {
                            Act<WB> A;
                            act_from_lds<WB>(A, la + (size_t)p * (I / 4), ld + (size_t)p * nbh, lq + (size_t)p * nbh, cpos[i]);
                            const float v = A.dot(wd[b][i]) * (pw * sr[b][i]);
#pragma unroll
                            for (int tt = 0; tt < TT; tt++)
                                if (tt == t) acc[tt][i] += v;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
            if (tt < a.T) {
                for (int r = 0; r < cc.rw; r++) {
                    float v = 0.f;
#pragma unroll
                    for (int i = 0; i < CPL; i++)
                        if (crow[i] == r) v += acc[tt][i];
                    v = wave_sum(v);
                    if (lane == 0) {
                        float *dst = a.y + (size_t)tt * a.H + rb + r;
                        *dst = a.accumulate ? *dst + v : v;
                    }
                }
            }
        }
    }
}

size_t down_lds_bytes(const GemvArgs &a, const PlanDims &pd)
{
    const size_t nbh = a.I / 32;
    return sizeof(int) * (size_t)((pd.words + 3) & ~3) + (size_t)pd.P * a.I +
           2 * sizeof(float) * (size_t)pd.P * nbh;
}

// ---------------------------------------------------------------- dispatch
template <int WB, int CPL, int TT>
static int run_gate_up(const GemvArgs &a, const ChunkCfg &cc, const PlanDims &pd, hipStream_t st)
{
    const int grid = pd.S * (a.I / 32);
    k_gate_up<WB, CPL, TT><<<grid, 256, 0, st>>>(a, cc, pd);
    return (int)hipGetLastError();
}

template <int WB, int CPL, int TT>
static int run_down(const GemvArgs &a, const ChunkCfg &cc, const PlanDims &pd, hipStream_t st)
{
    const int rows = cc.rw > 16 ? cc.rw : 16;
    const size_t lds = down_lds_bytes(a, pd);
    k_down<WB, CPL, TT><<<a.H / rows, 256, lds, st>>>(a, cc, pd, rows);
    return (int)hipGetLastError();
}

#define MOE_TT_SWITCH(FN, WB, CPL)                          \
    switch (tt) {                                           \
    case 1: return FN<WB, CPL, 1>(a, cc, pd, st);           \
    case 4: return FN<WB, CPL, 4>(a, cc, pd, st);           \
    default: return FN<WB, CPL, 8>(a, cc, pd, st);          \
    }
#define MOE_CPL_SWITCH(FN, WB)                              \
    switch (cc.cpl) {                                       \
    case 1: MOE_TT_SWITCH(FN, WB, 1)                        \
    case 2: MOE_TT_SWITCH(FN, WB, 2)                        \
    case 3: MOE_TT_SWITCH(FN, WB, 3)                        \
    default: MOE_TT_SWITCH(FN, WB, 6)                       \
    }
#define MOE_WB_SWITCH(FN)                                   \
    switch (a.wbits) {                                      \
    case 2: MOE_CPL_SWITCH(FN, 2)                           \
    case 4: MOE_CPL_SWITCH(FN, 4)                           \
    default: MOE_CPL_SWITCH(FN, 8)                          \
    }

static int tt_for(int T) { return T <= 1 ? 1 : (T <= 4 ? 4 : 8); }

int launch_gate_up(const GemvArgs &a, hipStream_t st)
{
    ChunkCfg cc;
    if (!chunk_cfg(a.H, a.wbits, cc)) return (int)hipErrorInvalidValue;
    const PlanDims pd = plan_dims(a.T, a.rc.k, a.n_shared, a.logits == nullptr);
    const int tt = tt_for(a.T);
    MOE_WB_SWITCH(run_gate_up)
}

int launch_down(const GemvArgs &a, hipStream_t st)
{
    ChunkCfg cc;
    if (!chunk_cfg(a.I, a.wbits, cc)) return (int)hipErrorInvalidValue;
    const PlanDims pd = plan_dims(a.T, a.rc.k, a.n_shared, a.logits == nullptr);
    const int tt = tt_for(a.T);
    MOE_WB_SWITCH(run_down)
}

} // namespace moe

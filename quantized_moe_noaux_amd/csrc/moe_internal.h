// Host-side internals shared by the MoE entry points and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kMaxGroups = 64;
constexpr int kMaxTopK = 32;
constexpr int kGemvMaxT = 8;          // the batch-union GEMV path takes T <= 8
constexpr int kGemvMaxLdsAct = 64 * 1024;

// Router layout: each lane of a wave holds `epl` consecutive experts and a
// group spans `lpg` lanes (a power of two), so group top-2 sums are lane
// butterflies.  Chosen on the host by route_cfg().
struct RouteCfg {
    int E, G, tg, k, epl, lpg;
    float rsf;
    float top_p;  // adaptive expert top-p; active in (0, 1)
};
inline bool top_p_on(const moe_shape_t &s) { return s.routed_top_p > 0.f && s.routed_top_p < 1.f; }

bool route_cfg(const moe_shape_t &s, RouteCfg &rc);

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// A weight row is read as `cpr` 16-byte chunks.
struct ChunkCfg {
    int cpr;  // chunks per row
};
bool chunk_cfg(int in_dim, int wbits, ChunkCfg &cc);

// Plan of the batch-union GEMV path (written to the workspace by the
// gate/up kernel, read by the down/combine kernel).  Flat int32 array:
//   [0]                n_slots
//   [1 ..]             slot_e[S]    expert of slot (-1 = shared)
//                      slot_n[S]    tokens routed to slot
//                      slot_p0[S]   first pair of slot
//                      pair_t[P]    token of pair
//                      pair_w[P]    combine weight of pair (fp32 bits)
struct PlanDims {
    int S, P;
    int o_e, o_n, o_p0, o_t, o_w, words;
};
inline PlanDims plan_dims(int T, int k, int n_shared, bool single)
{
    PlanDims d;
    d.S = single ? 1 : T * k + n_shared;
    d.P = single ? T : T * (k + n_shared);
    d.o_e = 1;
    d.o_n = d.o_e + d.S;
    d.o_p0 = d.o_n + d.S;
    d.o_t = d.o_p0 + d.S;
    d.o_w = d.o_t + d.P;
    d.words = d.o_w + d.P;
    return d;
}

// LDS bytes of one token's staged activations over `in` elements: the int8
// codes, one fp32 scale per block and (int4 / int2 only: the XOR offset
// needs them) one int32 block sum per block, rounded up to 16 bytes.
__host__ __device__ inline size_t act_lds_bytes(int wbits, int in)
{
    return ((size_t)in + (size_t)(in / 32) * (wbits == 8 ? 4 : 8) + 15) & ~(size_t)15;
}
constexpr int kGemvDownRows = 16;  // rows per down/combine workgroup
// LDS of the down/combine kernel: the plan, every pair's activations, then
// every slot's row scales of the workgroup's rows.
inline size_t down_lds_bytes(int wbits, int I, const PlanDims &pd)
{
    return sizeof(int) * (size_t)((pd.words + 3) & ~3) + (size_t)pd.P * act_lds_bytes(wbits, I) +
           sizeof(float) * (size_t)pd.S * kGemvDownRows;
}
// The row-sweep down kernel stages the pairs' h in batches of whole slots:
// the pairs that fit the LDS left by the plan and the slots' row scales
// (at least kGemvMaxT, the most pairs one slot can have).
inline int down_pair_cap(int wbits, int I, const PlanDims &pd)
{
    const size_t fixed = sizeof(int) * (size_t)((pd.words + 3) & ~3) + sizeof(float) * (size_t)pd.S * kGemvDownRows;
    const size_t per = act_lds_bytes(wbits, I);
    const int cap = fixed < (size_t)kGemvMaxLdsAct ? (int)(((size_t)kGemvMaxLdsAct - fixed) / per) : 0;
    return cap < pd.P ? cap : pd.P;
}
inline size_t down_sw_lds_bytes(int wbits, int I, const PlanDims &pd, int pmax)
{
    return sizeof(int) * (size_t)((pd.words + 3) & ~3) + (size_t)pmax * act_lds_bytes(wbits, I) +
           sizeof(float) * (size_t)pd.S * kGemvDownRows;
}
bool gemv_gate_up_sw(const moe_shape_t &s);
bool gemv_down_sw(const moe_shape_t &s);
// LDS of the gate/up kernel: static plan / routing scratch plus Tc tokens of
// staged activations over H.
constexpr size_t kGateUpStaticLds = 12 * 1024;
inline size_t gate_up_lds_bytes(int wbits, int H, int Tc) { return kGateUpStaticLds + Tc * act_lds_bytes(wbits, H); }
// tokens per batch-union chunk: the largest count <= kGemvMaxT whose LDS fits
// (0 if not even one token fits)
// (the row-sweep kernels read x directly and stage h in batches, so only
// the other kernels' full staging bounds the chunk)
inline int gemv_chunk_tokens(const moe_shape_t &s, int T)
{
    const bool gsw = gemv_gate_up_sw(s), dsw = gemv_down_sw(s);
    for (int tc = (T < kGemvMaxT ? T : kGemvMaxT); tc >= 1; tc--) {
        const PlanDims pd = plan_dims(tc, s.top_k, s.n_shared, false);
        const bool down_ok = dsw ? down_pair_cap(s.wbits, s.inter, pd) >= (tc < pd.P ? tc : pd.P)
                                 : down_lds_bytes(s.wbits, s.inter, pd) <= (size_t)kGemvMaxLdsAct;
        if (down_ok && (gsw || gate_up_lds_bytes(s.wbits, s.hidden, tc) <= (size_t)kGemvMaxLdsAct))
            return tc;
    }
    return 0;
}

// ---------------------------------------------------------------- MTP draft verification
constexpr int kMtpMaxDraft = 16;   // drafts per sequence
constexpr int kMtpChunk = 4096;    // tokens per chunk of a logit row
constexpr int kMtpMaxChunks = 256; // chunks per row: vocabularies up to 1,048,576 tokens
inline int mtp_chunks(int V) { return (V + kMtpChunk - 1) / kMtpChunk; }
constexpr int kMtpDrawChunk = 1024;  // tokens per chunk of the draw
inline int mtp_draw_chunks(int V) { return (V + kMtpDrawChunk - 1) / kMtpDrawChunk; }
// workspace: per-(row, chunk) stats (16 B, rows = B * (2D + 1)), the
// decisions (64 B per sequence), per-draw-chunk masses (16 B) and every
// token's draw weight (8 B, whole chunks)
struct MtpWs {
    size_t stats, dec, mass, w, total;
};
inline MtpWs mtp_ws(int B, int D, int V)
{
    MtpWs L;
    size_t o = 0;
    L.stats = o; o = align256(o + (size_t)16 * B * (2 * D + 1) * mtp_chunks(V));
    L.dec = o;   o = align256(o + (size_t)64 * B);
    L.mass = o;  o = align256(o + (size_t)16 * B * mtp_draw_chunks(V));
    L.w = o;     o = align256(o + (size_t)8 * B * mtp_draw_chunks(V) * kMtpDrawChunk);
    L.total = o;
    return L;
}
inline size_t mtp_workspace_bytes(int B, int D, int V) { return mtp_ws(B, D, V).total; }
int launch_mtp_accept(int B, int D, int V, const int32_t *draft, const float *p, const float *q, double tau,
                      const double *u, int32_t *n_acc, int32_t *next, void *ws, hipStream_t st);

struct GemvWs {
    size_t logits, xq, xd, plan, qh, dh, total;
};
GemvWs gemv_ws(const moe_shape_t &s, int T, int Tc, bool single);

// ---------------------------------------------------------------- launchers
// (each returns hipGetLastError() as an int after its launch)
// Router logits (and the quantised x) of T <= kGemvMaxT tokens; with
// ng != nullptr the input is RMSNorm(x) with weight ng, formed in the launch.
int launch_router_logits(const float *x, int T, int H, const float *gate_w, int E, double *logits,
                         int8_t *xq, float *xd, const float *ng, double eps, hipStream_t st,
                         const float *la_gate_w = nullptr, const float *la_ng = nullptr,
                         double *la_logits = nullptr);
// whether the router launch can normalise its own input for this row width
inline bool router_norms_input(const float *x, const float *ng, int H)
{
    return H % 4 == 0 && H <= 8192 && ((((uintptr_t)x) | ((uintptr_t)ng)) & 15) == 0;
}
// Router logits of more than kGemvMaxT tokens: fp64 MFMA over `ksplit`
// slices of the hidden dimension, partial sums in part[ksplit][T][E]
// (router_ksplit picks the slice count; 1 for T <= kGemvMaxT).
int router_ksplit(int T, int H, int E);
inline size_t router_logit_bytes(const moe_shape_t &s, int T)
{
    return sizeof(double) * (size_t)router_ksplit(T, s.hidden, s.n_experts) * T * s.n_experts;
}
int launch_router_logits_mfma(const float *x, int T, int H, const float *gate_w, int E, int ksplit, double *part,
                              hipStream_t st);
int launch_topk(const RouteCfg &rc, const double *logits, int nparts, const float *bias, int T, int32_t *idx,
                float *w, hipStream_t st);
int launch_quant(const float *x, int T, int D, int8_t *q, float *d, hipStream_t st);

struct GemvArgs {
    // shape
    int T, H, I, E, wbits, n_shared;
    RouteCfg rc;
    // routing (logits == nullptr: single-expert mode on expert `single`);
    // a token's logits are the sum of lparts slices lstride apart
    const double *logits;
    size_t lstride;
    int lparts;
    const float *bias;
    int single;
    // weights
    moe_weights_t routed, shared;
    // int8 activations of x (natural order) and their block scales
    const int8_t *xq;
    const float *xd;
    // workspace: plan and the quantised h of every (slot, token) pair
    int *plan;
    int8_t *qh;
    float *dh;
    // layer outputs
    float *y;
    int32_t *idx_out;
    float *w_out;
    int accumulate;
    // one token, routed by the gate/up workgroups themselves (no plan launch)
    int inline_route;
    // pairs the row-sweep down kernel stages at a time (down_pair_cap)
    int down_pmax;
    // expert table (tiered weights): expert e's six tensors are at the
    // routed base pointers plus the byte offsets toff[6e .. 6e+5] (gate, up,
    // down, gate_s, up_s, down_s); nullptr: the stacks [E][rows][bytes]
    const int64_t *toff;
    // per-expert selection counts, incremented by the routing (or nullptr)
    uint32_t *counts;
    // router lookahead (one token routed inside the gate/up launch): the
    // next layer's logits (computed by this layer's router launch), its
    // correction bias and experts; la_wgs workgroups per prefetched expert
    // (the k ranks the next layer's router predicts, then its shared
    // expert) stream their share of its weights so that they are in the
    // memory-side cache when that layer runs; 0 = no lookahead
    const double *la_logits;
    const float *la_bias;
    moe_weights_t la_routed, la_shared;
    int la_wgs;
    uint32_t *la_sink;  // one word per lookahead workgroup (the loaded data's XOR; keeps the loads)
};
constexpr int kLookaheadSinkWords = 4;  // la_sink words per lookahead workgroup (>= its waves)
// Whether a T-token call of this shape routes inside the gate/up launch
// (one token, row-sweep gate/up kernel) instead of in a plan launch.
// Whether the expert-table (tiered) GEMV kernels take this shape: int4
// weights at the production row widths.
bool gemv_table_ok(const moe_shape_t &s);
bool gemv_inline_route(const moe_shape_t &s, int T);
// one workgroup: routing of the chunk and its batch-union plan
int launch_plan(const GemvArgs &a, hipStream_t st);
// gate/up + SwiGLU + h quantisation of every slot of the published plan
int launch_gate_up(const GemvArgs &a, hipStream_t st);
int launch_down(const GemvArgs &a, hipStream_t st);

// ---------------------------------------------------------------- grouped path
constexpr int kGgTN = 128;  // rows (token, expert assignments) per grouped-GEMM tile

// 256-assignment tiles of the permutation's counting sort
inline int perm_tiles(int n) { return (n + 255) / 256; }
// rows of the grouped problem: T*k routed assignments, then T shared rows
inline size_t gg_rows(const moe_shape_t &s, int T) { return (size_t)T * s.top_k + (size_t)s.n_shared * T; }
// upper bound of the tile count: sum_e ceil(n_e / TN) <= T*k/TN + (experts used)
inline int gg_max_tiles(const moe_shape_t &s, int T)
{
    const long tk = (long)T * s.top_k;
    const long used = tk < s.n_experts ? tk : s.n_experts;
    return (int)(tk / kGgTN + used + 1 + (s.n_shared ? (T + kGgTN - 1) / kGgTN : 0));
}
// shapes the grouped kernels take: gate/up workgroups of 128 intermediate
// channels, down workgroups of 256 hidden channels, K in steps of 128
inline bool gg_shape_ok(const moe_shape_t &s) { return s.hidden % 256 == 0 && s.inter % 128 == 0; }

struct GgWs {
    size_t logits, idx, w, xq, xd, perm, off, inv, pscr, tiles, qh, dh, y, total;
};
GgWs gg_ws(const moe_shape_t &s, int T);

struct GgArgs {
    int T, H, I, E, k, n_shared, wbits, Tk;
    const int4 *tiles;      // [0].x = count, then {expert (E = shared), first row, rows, 0}
    const int32_t *perm;    // row -> assignment t*k + slot
    const int32_t *inv;     // assignment -> row
    const float *w;         // combine weight of each assignment
    moe_weights_t routed, shared;
    const int8_t *xq;       // [T][H] int8 x in the weights' code order (gg_act_pos), block scales xd
    const float *xd;
    int8_t *qh;             // [rows][I] int8 h in the same order, block scales dh
    float *dh;
    float *yrows;           // [rows][H] weighted expert outputs
    float *y;               // [T][H] layer output
    int accumulate;
};
int launch_gg_quant(const float *x, int T, int D, int wbits, int8_t *q, float *d, hipStream_t st);
int launch_gg_gate_up(const GgArgs &a, int max_tiles, hipStream_t st);
int launch_gg_down(const GgArgs &a, int max_tiles, hipStream_t st);
int launch_gg_combine(const GgArgs &a, hipStream_t st);

int launch_rmsnorm(const float *x, const float *g, double eps, int T, int H, float *out, hipStream_t st);
int launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st);
int launch_block_dots(int wbits, const uint8_t *codes, int rows, int D, const int8_t *q, int T,
                      int32_t *out, hipStream_t st);
// Stable counting sort of the T*k assignments by expert.  With tiles != null
// it also writes the grouped path's tile list (kGgTN rows per tile, then the
// n_shared * T shared rows).
int launch_permute(const int32_t *idx, int T, int k, int E, int32_t *perm, int32_t *off, int32_t *inv,
                   int32_t *scratch, int4 *tiles, int n_shared, hipStream_t st);

} // namespace moe

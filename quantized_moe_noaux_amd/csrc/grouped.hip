// Expert-grouped path of the MoE layer (prefill and other large batches).
//
// GeekNews #31297, implemented features: batch-union MoE applies each
// selected expert once to every position routed to it; the expert FFNs are
// SwiGLU over packed int4 / int8 / int2 codes with per-row scales, evaluated
// as integer dots on Q8_0-style int8 activations in blocks of 32.
// wpnews.pro spec table: 8 routed + 1 shared expert per token.
//
// After routing, the T*k (token, slot) assignments are sorted by expert
// (stable counting sort, moe_permute's kernels) into "rows", followed by T
// rows for the shared expert.  Rows are cut into tiles of kGgTN = 128 rows
// that never straddle two experts; every tile is a small GEMM against its
// expert's weights, on v_mfma_i32_32x32x32_i8: one MFMA is exactly one
// activation block of 32, so its int32 result is that block's exact integer
// dot for 32 x 32 (channel, row) pairs, scaled by the row's block scale and
// summed in fp32.
//   k_gg_gate_up  workgroup = (tile, 128 intermediate channels): 256 weight
//                 rows (the channels' gate and up rows) against the tile's
//                 128 activation rows; then g, u -> h = silu(g) u -> int8 h
//                 in blocks of 32 channels.
//   k_gg_down     workgroup = (tile, 256 hidden channels), over the int8 h
//                 rows; the result is scaled by the row's combine weight and
//                 written to the row's output slot.
//   k_gg_combine  out[t] = t's k routed slots in slot order, then the shared
//                 row.
// No float atomics anywhere: results are run-to-run identical.
//
// Code forms.  A packed weight code is masked in place into the top bits of
// its byte, where the byte reads as the signed value 16c (int4) or 64c
// (int2): two's-complement codes keep their sign there, so the MFMA gives
// 16 (or 64) times the exact block dot, |16 I| <= 520192, and the power of
// two is folded into the row scale.  The two halves of a wave's MFMA operand
// (lanes 0-31 and 32-63 hold K = 0-15 and 16-31 of the block) take
// different fields of the same packed bytes (int4: lanes 0-31 the low
// nibbles, lanes 32-63 the high ones), so the activation codes of every
// block are stored once in that code order (gg_act_src below): by the row
// quantiser for x, by the gate/up epilogue for h.
//
// Work order.  The 1-D grid is dealt round-robin over the 8 XCDs (each with
// its own L2).  XCD x takes the channel groups [x cpx, (x+1) cpx) of every
// tile, and its workgroups walk tile by tile with a tile's channel groups
// back to back, so a tile's activation rows are fetched once per XCD and the
// tiles of one expert run at about the same time on the same XCD.  (The
// L2-to-fabric counters show those tiles re-fetching most of their weight
// slices rather than sharing them: the kernels are bound by the VALU, not
// by this traffic, and an expert-contiguous order measured slower.)
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGgThreads = 512;
constexpr int kGgWRows = 256;  // weight rows staged per workgroup

GgWs gg_ws(const moe_shape_t &s, int T)
{
    GgWs w;
    const int H = s.hidden, I = s.inter, E = s.n_experts, k = s.top_k;
    const size_t Tk = (size_t)T * k, R = gg_rows(s, T);
    size_t o = 0;
    w.logits = o; o = align256(o + router_logit_bytes(s, T));
    w.idx = o;    o = align256(o + sizeof(int32_t) * Tk);
    w.w = o;      o = align256(o + sizeof(float) * Tk);
    w.xq = o;     o = align256(o + (size_t)T * H);
    w.xd = o;     o = align256(o + sizeof(float) * (size_t)T * (H / 32));
    w.perm = o;   o = align256(o + sizeof(int32_t) * Tk);
    w.off = o;    o = align256(o + sizeof(int32_t) * (E + 1));
    w.inv = o;    o = align256(o + sizeof(int32_t) * Tk);
    w.pscr = o;   o = align256(o + sizeof(int32_t) * perm_tiles((int)Tk) * E);
    w.tiles = o;  o = align256(o + sizeof(int4) * (size_t)(gg_max_tiles(s, T) + 1));
    w.qh = o;     o = align256(o + R * I);
    w.dh = o;     o = align256(o + sizeof(float) * R * (I / 32));
    w.y = o;      o = align256(o + sizeof(float) * R * H);
    w.total = o;
    return w;
}

// ---------------------------------------------------------------- code order
// Natural index (within its block of 32) of the activation code stored at
// position p of the block, for weights of WB bits:
//   int8: p;
//   int4: lanes 0-31 take the low nibbles of the block's 16 bytes (codes
//         0, 2, .., 30), lanes 32-63 the high ones (1, 3, .., 31);
//   int2: lane half h takes fields 2h and 2h+1 of the block's 8 bytes; its
//         dword o = 2j + f is field 2h + f of weight dword j, whose byte m
//         holds code 16j + 4m + 2h + f.
template <int WB> __host__ __device__ __forceinline__ int gg_act_src(int p)
{
    if constexpr (WB == 4) {
        return p < 16 ? 2 * p : 2 * (p - 16) + 1;
    } else if constexpr (WB == 2) {
        const int h = p >> 4, o = (p >> 2) & 3, m = p & 3;
        return 16 * (o >> 1) + 4 * m + 2 * h + (o & 1);
    } else {
        return p;
    }
}

// Four bytes of a block in natural order (src[0..31]) at stored positions
// 4o .. 4o+3, packed little-endian into a dword.
template <int WB> __device__ __forceinline__ uint32_t gg_pack_dword(const uint8_t *src, int o)
{
    uint32_t v = 0;
#pragma unroll
    for (int m = 0; m < 4; m++) v |= (uint32_t)src[gg_act_src<WB>(4 * o + m)] << (8 * m);
    return v;
}

// ---------------------------------------------------------------- row quantiser
// One workgroup per row of D values: Q8_0-style blocks (8 lanes per block,
// quant_block8), the codes gathered in LDS in natural order, then written
// out in the weights' code order.
template <int WB>
__global__ __launch_bounds__(256) void k_gg_quant(const float *__restrict__ x, int D, int8_t *__restrict__ q,
                                                  float *__restrict__ d)
{
    extern __shared__ __align__(16) uint8_t qn[];  // D bytes
    const int row = blockIdx.x, tid = threadIdx.x, bs = tid >> 3, sub = tid & 7;
    const int nb = D / 32;
    const float *xr = x + (size_t)row * D;
    for (int b0 = 0; b0 < nb; b0 += 32) {
        const int b = b0 + bs;
        const bool live = b < nb;
        const float4 v = reinterpret_cast<const float4 *>(xr + 32 * min(b, nb - 1))[sub];
        float db;
        const uint32_t packed = quant_block8(v, db);
        if (live) {
            reinterpret_cast<uint32_t *>(qn + 32 * b)[sub] = packed;
            if (sub == 0) d[(size_t)row * nb + b] = db;
        }
    }
    __syncthreads();
    uint32_t *qo = reinterpret_cast<uint32_t *>(q + (size_t)row * D);
    for (int i = tid; i < D / 4; i += 256) qo[i] = gg_pack_dword<WB>(qn + 32 * (i >> 3), i & 7);
}

int launch_gg_quant(const float *x, int T, int D, int wbits, int8_t *q, float *d, hipStream_t st)
{
    const size_t lds = (size_t)D;
    if (wbits == 4) k_gg_quant<4><<<T, 256, lds, st>>>(x, D, q, d);
    else if (wbits == 8) k_gg_quant<8><<<T, 256, lds, st>>>(x, D, q, d);
    else k_gg_quant<2><<<T, 256, lds, st>>>(x, D, q, d);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- tiling
// A workgroup of 512 threads (8 waves) owns 128 activation rows (one tile)
// and 256 weight rows.  Per pipeline step it stages K = 64 codes of both in
// LDS as int8 MFMA operands: the activation rows as stored (code order),
// the weight rows expanded from their packed codes to the 16c / 64c form
// (int4 / int2; int8 as stored), so that a wave reads every MFMA operand
// with one ds_read_b128 and no further VALU work.  A workgroup takes 63 KB
// of LDS and (int4, int2) at most 128 VGPRs per lane, so two fit on a CU:
// one's prologue, epilogue and barrier waits overlap the other's MFMAs and
// rescale.  (The int8 form stages twice the weight chunks per thread and
// keeps one workgroup per CU rather than spill.)
constexpr int kGgKS = 64;                // K codes per step
constexpr int kGgNBS = kGgKS / 32;       // activation blocks per step
constexpr int kGgRowBytes = kGgKS;       // LDS bytes of a staged row per step (int8 operands)
constexpr int kGgCPR = kGgRowBytes / 16; // 16-byte chunks per staged row

template <int WB> struct GgCfg {
    static constexpr int PRB = kGgKS * WB / 8;                 // packed weight bytes per row per step
    static constexpr int PCR = PRB / 16;                       // packed 16-byte chunks per weight row per step
    static constexpr int WCH = kGgWRows * PCR;                 // packed weight chunks per step
    static constexpr int WLD = (WCH + kGgThreads - 1) / kGgThreads;  // per thread (the last one partial for int2)
    static constexpr float kInv = WB == 4 ? 1.0f / 16 : WB == 2 ? 1.0f / 64 : 1.0f;  // code form scale
};
static_assert(kGgTN * kGgCPR == kGgThreads, "one activation chunk per thread per step");
static_assert(kGgTN * kGgNBS <= kGgThreads, "one activation scale per thread per step");

// Chunk c of staged row r.  Rows are padded to 80 bytes (20 banks): the 16
// lanes a ds_read_b128 serves at once read rows r .. r+15 at one chunk, and
// these start on 16 distinct 4-bank groups; a fragment's address is one
// base per row plus an immediate offset per block.
constexpr int kGgRowStride = kGgRowBytes + 16;
__device__ __forceinline__ int ldsoff(int r, int c) { return r * kGgRowStride + 16 * c; }

// The small arrays come first: LDS instructions encode offsets below 64 KB
// as immediates, so the scales and activations are reached from one base
// register each.
struct GgLds {
    float d[2][kGgNBS][kGgTN];                            // activation block scales, two pipeline buffers
    int arow[kGgTN];                                      // source row of each tile row
    float cw[kGgTN];                                      // combine weight of each tile row (down)
    __align__(16) uint8_t a[2][kGgTN * kGgRowStride];     // activation operands
    __align__(16) uint8_t w[2][kGgWRows * kGgRowStride];  // weight operands
};

__device__ __forceinline__ v4i lds16(const uint8_t *p) { return *reinterpret_cast<const v4i *>(p); }

// An empty instruction that takes the accumulator tuples as operands and
// orders all memory accesses around it: everything that produces them is
// issued before it, and no later load is issued ahead of it.
__device__ __forceinline__ void pin_after(v16f &a, v16f &b) { asm volatile("" : "+v"(a), "+v"(b)::"memory"); }

// Waves and weight tiles: wave w takes the 32 tile rows 32 (w / kGgCW) ..
// and kGgWT weight tiles of 32 rows (wr[0 .. kGgWT-1] in the staged 256).
constexpr int kGgWaves = kGgThreads / 64;
constexpr int kGgCW = kGgWaves / (kGgTN / 32);  // waves per 32-row group
constexpr int kGgWT = kGgWRows / 32 / kGgCW;    // weight tiles per wave
static_assert(kGgCW * (kGgTN / 32) == kGgWaves && kGgWT % 2 == 0, "wave tiling");

// Packed codes of one 16-byte chunk -> its MFMA operand chunks in LDS.
//   int4: the chunk is one block of 32 codes; operand chunk 2b (lanes 0-31)
//         holds the low nibbles masked into the top bits (16 c_even),
//         chunk 2b+1 the high nibbles in place (16 c_odd);
//   int2: the chunk is blocks 2p, 2p+1 (8 bytes each); for each block,
//         operand chunk (lanes 0-31) holds fields 0, 1 of its two dwords
//         shifted to the top bits, the next chunk fields 2, 3 (64c);
//   int8: the chunk is half a block, stored as is.
template <int WB>
__device__ __forceinline__ void gg_stage_w(uint8_t *wbuf, int r, int pc, const v4u &v)
{
    if constexpr (WB == 4) {
        v4u lo, hi;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            lo[j] = (v[j] << 4) & 0xF0F0F0F0u;
            hi[j] = v[j] & 0xF0F0F0F0u;
        }
        *reinterpret_cast<v4u *>(wbuf + ldsoff(r, 2 * pc)) = lo;
        *reinterpret_cast<v4u *>(wbuf + ldsoff(r, 2 * pc + 1)) = hi;
    } else if constexpr (WB == 2) {
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const uint32_t d0 = v[2 * q], d1 = v[2 * q + 1];
            v4u lo, hi;
            lo[0] = (d0 << 6) & 0xC0C0C0C0u; lo[1] = (d0 << 4) & 0xC0C0C0C0u;
            lo[2] = (d1 << 6) & 0xC0C0C0C0u; lo[3] = (d1 << 4) & 0xC0C0C0C0u;
            hi[0] = (d0 << 2) & 0xC0C0C0C0u; hi[1] = d0 & 0xC0C0C0C0u;
            hi[2] = (d1 << 2) & 0xC0C0C0C0u; hi[3] = d1 & 0xC0C0C0C0u;
            *reinterpret_cast<v4u *>(wbuf + ldsoff(r, 4 * pc + 2 * q)) = lo;
            *reinterpret_cast<v4u *>(wbuf + ldsoff(r, 4 * pc + 2 * q + 1)) = hi;
        }
    } else {
        *reinterpret_cast<v4u *>(wbuf + ldsoff(r, pc)) = v;
    }
}

// Staging registers of one pipeline step: the thread's packed weight
// chunks, its activation chunk and (threads below 256) one activation scale.
template <int WB> struct GgRegs {
    v4u w[GgCfg<WB>::WLD], a;
    float d;
};

// Main loop shared by both GEMMs.  The workgroup's 256 weight rows are
// rows 0..255 after w0 (GU = false), or rows 0..127 after w0 and 0..127
// after w1 (GU = true: gate then up), each of wrb bytes; its 128 activation
// rows start at aq + L.arow[i] * K (codes in code order), their scales at
// ad + L.arow[i] * (K/32).  Wave w computes the 32 tile rows 32 (w / kGgCW)
// .. (LIVE: some of them are live; uniform in the wave) against the weight
// rows wr[wt] + (lane % 32) of its kGgWT 32-row weight tiles.  acc[wt] comes
// back in MFMA layout: lane l, register v = weight row
// 8 (v / 4) + 4 (l / 32) + v % 4 of weight tile wt, tile row
// 32 (w / kGgCW) + l % 32.
//
// Pipeline: two LDS buffers (one barrier per step).  At the start of step s
// the loads of step s + 1 go out into the staging registers, the MFMAs of
// step s run from LDS, then the registers are stored to the other buffer;
// the waves of two workgroups per SIMD cover the load latency.  Every staging
// register is indexed by compile-time constants, so it stays in a VGPR.
template <int WB, bool GU, bool LIVE>
__device__ __forceinline__ void gg_mainloop(GgLds &L, const uint8_t *w0, const uint8_t *w1, size_t wrb,
                                            const int (&wr)[kGgWT], const int8_t *__restrict__ aq,
                                            const float *__restrict__ ad, int K, v16f (&acc)[kGgWT])
{
    using C = GgCfg<WB>;
    const int tid = threadIdx.x, l = lane_id(), h = l >> 5;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int nbk = K / 32, nsteps = K / kGgKS;
    const int r0 = 32 * (w / kGgCW) + (l & 31);

    // staging sources of this thread: packed weight chunks (id < WCH; for
    // int2 the upper half of the workgroup has none, a whole-wave split),
    // one activation chunk, one scale (threads < 256: row t/2, block t%2)
    const uint8_t *wp[C::WLD];
    int wrw[C::WLD], wpc[C::WLD];
#pragma unroll
    for (int i = 0; i < C::WLD; i++) {
        const int id = min(tid + kGgThreads * i, C::WCH - 1), r = id / C::PCR, pc = id % C::PCR;
        const bool up = GU && r >= 128;  // gate rows 0..127, up rows 128..255
        wp[i] = (up ? w1 : w0) + (size_t)(up ? r - 128 : r) * wrb + 16 * pc;
        wrw[i] = r;
        wpc[i] = pc;
    }
    const bool wlast = tid + kGgThreads * (C::WLD - 1) < C::WCH;  // the last weight chunk is this thread's
    const int ar = tid / kGgCPR, ac = tid % kGgCPR;
    const int8_t *ap = aq + (size_t)L.arow[ar] * K + 16 * ac;
    const int ao = ldsoff(ar, ac);
    const bool dl = tid < kGgTN * kGgNBS;
    const int dr = (tid / kGgNBS) & (kGgTN - 1), db = tid % kGgNBS;
    const float *dp = ad + (size_t)L.arow[dr] * nbk + db;

    // loads of step s (a step past the end reads the last one again: an L2
    // hit, and no load under a branch)
    auto fetch = [&](GgRegs<WB> &R, int s) {
        s = s < nsteps ? s : nsteps - 1;
        const size_t kw = (size_t)s * C::PRB, ka = (size_t)s * kGgKS;
#pragma unroll
        for (int i = 0; i < C::WLD; i++) R.w[i] = *reinterpret_cast<const v4u *>(wp[i] + kw);
        R.a = *reinterpret_cast<const v4u *>(ap + ka);
        R.d = dp[s * kGgNBS];
    };
    auto stage = [&](const GgRegs<WB> &R, int buf) {
#pragma unroll
        for (int i = 0; i < C::WLD; i++)
            if (i + 1 < C::WLD || wlast) gg_stage_w<WB>(L.w[buf], wrw[i], wpc[i], R.w[i]);
        *reinterpret_cast<v4u *>(&L.a[buf][ao]) = R.a;
        if (dl) L.d[buf][db][dr] = R.d;
    };
    v16i zero;
#pragma unroll
    for (int v = 0; v < 16; v++) zero[v] = 0;
    // MFMAs of the step in LDS buffer buf
    auto compute = [&](int buf) {
        if constexpr (LIVE) {
            const uint8_t *wb = L.w[buf], *abuf = L.a[buf];
#pragma unroll
            for (int b = 0; b < kGgNBS; b++) {
                const int c = 2 * b + h;
                const v4i b0 = lds16(abuf + ldsoff(r0, c));
                const float d0 = L.d[buf][b][r0];
#pragma unroll
                for (int t = 0; t < kGgWT; t += 2) {
                    const v4i a0 = lds16(wb + ldsoff(wr[t] + (l & 31), c));
                    const v4i a1 = lds16(wb + ldsoff(wr[t + 1] + (l & 31), c));
                    const v16i i0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, zero, 0, 0, 0);
                    const v16i i1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b0, zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        acc[t][v] = fmaf((float)i0[v], d0, acc[t][v]);
                        acc[t + 1][v] = fmaf((float)i1[v], d0, acc[t + 1][v]);
                    }
                    // a pair of tiles' rescale completes before the next
                    // pair's LDS reads and MFMAs are issued: two results
                    // live at a time (4 waves per SIMD: 128 VGPRs)
                    pin_after(acc[t], acc[t + 1]);
                }
            }
        }
    };
#pragma unroll
    for (int wt = 0; wt < kGgWT; wt++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[wt][v] = 0.f;

    GgRegs<WB> R;
    fetch(R, 0);
    stage(R, 0);
    __syncthreads();
    for (int s = 0; s < nsteps; s++) {
        const int buf = s & 1;
        fetch(R, s + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(buf);
        __builtin_amdgcn_sched_barrier(0);
        stage(R, buf ^ 1);
        __syncthreads();
    }
}

// the main loop for this wave's 32 tile rows: MFMAs only if one of them is live
template <int WB, bool GU>
__device__ __forceinline__ void gg_mainloop_rows(GgLds &L, const uint8_t *w0, const uint8_t *w1, size_t wrb,
                                                 const int (&wr)[kGgWT], const int8_t *aq, const float *ad, int K,
                                                 int n, v16f (&acc)[kGgWT])
{
    const int rbase = 32 * (__builtin_amdgcn_readfirstlane(wave_id()) / kGgCW);
    if (rbase < n) gg_mainloop<WB, GU, true>(L, w0, w1, wrb, wr, aq, ad, K, acc);
    else gg_mainloop<WB, GU, false>(L, w0, w1, wrb, wr, aq, ad, K, acc);
}

__device__ __forceinline__ const moe_weights_t &gg_expert(const GgArgs &a, int e, size_t &eo)
{
    eo = (e == a.E) ? 0 : (size_t)e;
    return (e == a.E) ? a.shared : a.routed;
}

// The workgroup's (tile, channel group) under the XCD-aware order; false if
// it has none.
__device__ __forceinline__ bool gg_item(const GgArgs &a, int ncg, int &tile, int &cg)
{
    const int b = blockIdx.x, x = b & 7, j = b >> 3;
    const int cpx = (ncg + 7) / 8;
    tile = j / cpx;
    const int c = j % cpx;
    cg = x * cpx + c;
    return cg < ncg && tile < a.tiles[0].x;
}

// ---------------------------------------------------------------- gate / up
// Wave w: tile rows 32 (w / kGgCW) .. + 32 and the intermediate channels
// c0 + 64 (w % kGgCW) .. + 64: weight tiles 0, 1 are their gate rows, 2, 3
// their up rows.
template <int WB>
__global__ __launch_bounds__(kGgThreads, WB == 8 ? 3 : 4) void k_gg_gate_up(const GgArgs a)
{
    __shared__ GgLds L;
    int tix, cg;
    if (!gg_item(a, a.I / 128, tix, cg)) return;
    const int4 tile = a.tiles[1 + tix];
    const int e = tile.x, row0 = tile.y, n = tile.z;
    const int tid = threadIdx.x, H = a.H, I = a.I;
    const int c0 = cg * 128;
    const size_t rb = (size_t)H * WB / 8;
    size_t eo;
    const moe_weights_t &W = gg_expert(a, e, eo);
    if (tid < kGgTN) {
        // tile row -> token (rows past n repeat the first row's token: loaded, never stored)
        const int r = row0 + (tid < n ? tid : 0);
        L.arow[tid] = (r < a.Tk) ? a.perm[r] / a.k : r - a.Tk;
    }
    __syncthreads();
    static_assert(kGgWT == 4, "two gate and two up tiles per wave");
    const int w = __builtin_amdgcn_readfirstlane(wave_id()), cw = w % kGgCW;
    const int wr[kGgWT] = {64 * cw, 64 * cw + 32, 128 + 64 * cw, 128 + 64 * cw + 32};
    v16f acc[kGgWT];
    gg_mainloop_rows<WB, true>(L, W.gate + (eo * I + c0) * rb, W.up + (eo * I + c0) * rb, rb, wr, a.xq, a.xd, H,
                               n, acc);

    // epilogue: lane = (tile row i, channel half hf); per 32-channel block
    // of the wave (gate tile t, up tile t + 2) 16 channels; h quantised per
    // block, gathered in LDS in natural order, then written out in code order
    const int l = lane_id(), hf = l >> 5;
    const int i = 32 * (w / kGgCW) + (l & 31);
    uint8_t *qs = &L.a[0][0];  // [128 rows][128 channels] over the activation buffers (20 KB), free now
    constexpr float inv = GgCfg<WB>::kInv;
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const int cl = 64 * cw + 32 * t;  // the block's first channel within the workgroup's 128
        const float *gs = W.gate_s + eo * I + c0 + cl, *us = W.up_s + eo * I + c0 + cl;
        float hv[16];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float4 g4 = *reinterpret_cast<const float4 *>(gs + 8 * j + 4 * hf);
            const float4 u4 = *reinterpret_cast<const float4 *>(us + 8 * j + 4 * hf);
            const float gsc[4] = {g4.x, g4.y, g4.z, g4.w}, usc[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
            for (int m = 0; m < 4; m++)
                hv[4 * j + m] =
                    silu_mul((gsc[m] * inv) * acc[t][4 * j + m], (usc[m] * inv) * acc[t + 2][4 * j + m]);
        }
        // Q8_0 quantisation of h over the block of 32 channels (this lane's
        // 16 and lane l^32's 16)
        float amax = 0.f;
#pragma unroll
        for (int v = 0; v < 16; v++) amax = fmaxf(amax, fabsf(hv[v]));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float dq = amax / 127.0f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t wq = 0;
#pragma unroll
            for (int m = 0; m < 4; m++) {
                float r = (dq == 0.0f) ? 0.0f : rintf(hv[4 * j + m] / dq);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                wq |= ((uint32_t)(int)r & 0xFFu) << (8 * m);
            }
            *reinterpret_cast<uint32_t *>(qs + i * 128 + cl + 8 * j + 4 * hf) = wq;
        }
        if (hf == 0 && i < n) a.dh[(size_t)(row0 + i) * (I / 32) + (c0 + cl) / 32] = dq;
    }
    __syncthreads();
    // 128 rows x 4 blocks x 8 dwords, in code order
    for (int id = tid; id < kGgTN * 32; id += kGgThreads) {
        const int ri = id >> 5, o = id & 31, bb = o >> 3;
        if (ri < n)
            *reinterpret_cast<uint32_t *>(a.qh + (size_t)(row0 + ri) * I + c0 + 32 * bb + 4 * (o & 7)) =
                gg_pack_dword<WB>(qs + ri * 128 + 32 * bb, o & 7);
    }
}

// ---------------------------------------------------------------- down
// Wave w: tile rows 32 (w / kGgCW) .. + 32 and hidden channels
// n0 + 128 (w % kGgCW) .. + 128 (four weight tiles of 32).
template <int WB>
__global__ __launch_bounds__(kGgThreads, WB == 8 ? 3 : 4) void k_gg_down(const GgArgs a)
{
    __shared__ GgLds L;
    int tix, cg;
    if (!gg_item(a, a.H / 256, tix, cg)) return;
    const int4 tile = a.tiles[1 + tix];
    const int e = tile.x, row0 = tile.y, n = tile.z;
    const int tid = threadIdx.x, H = a.H, I = a.I;
    const int n0 = cg * 256;
    const size_t rb = (size_t)I * WB / 8;
    size_t eo;
    const moe_weights_t &W = gg_expert(a, e, eo);
    if (tid < kGgTN) {
        const int r = row0 + (tid < n ? tid : 0);
        L.arow[tid] = r;
        L.cw[tid] = (r < a.Tk) ? a.w[a.perm[r]] : 1.0f;
    }
    __syncthreads();
    const int w = __builtin_amdgcn_readfirstlane(wave_id()), cw = w % kGgCW;
    int wr[kGgWT];
#pragma unroll
    for (int t = 0; t < kGgWT; t++) wr[t] = 32 * (kGgWT * cw + t);
    v16f acc[kGgWT];
    gg_mainloop_rows<WB, false>(L, W.down + (eo * H + n0) * rb, nullptr, rb, wr, a.qh, a.dh, I, n, acc);

    const int l = lane_id(), hf = l >> 5;
    const int i = 32 * (w / kGgCW) + (l & 31);
    if (i >= n) return;
    const float *ds = W.down_s + eo * H;
    constexpr float inv = GgCfg<WB>::kInv;
    const float cwt = L.cw[i];
    float *yrow = a.yrows + (size_t)(row0 + i) * H;
#pragma unroll
    for (int wt = 0; wt < kGgWT; wt++) {
        const int cbase = n0 + 32 * (kGgWT * cw + wt) + 4 * hf;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int ch = cbase + 8 * j;
            const float4 s4 = *reinterpret_cast<const float4 *>(ds + ch);
            float4 o;
            o.x = (s4.x * inv) * acc[wt][4 * j + 0] * cwt;
            o.y = (s4.y * inv) * acc[wt][4 * j + 1] * cwt;
            o.z = (s4.z * inv) * acc[wt][4 * j + 2] * cwt;
            o.w = (s4.w * inv) * acc[wt][4 * j + 3] * cwt;
            *reinterpret_cast<float4 *>(yrow + ch) = o;
        }
    }
}

// ---------------------------------------------------------------- combine
// out[t] = rows of t's k slots in slot order, then t's shared row; with
// accumulate, the layer result is added to the existing out[t] at the end.
__global__ __launch_bounds__(256) void k_gg_combine(const GgArgs a)
{
    __shared__ int rows[kMaxTopK + 1];
    __shared__ int nr;
    const int t = blockIdx.x, k = a.k, H = a.H;
    if (threadIdx.x == 0) {
        // the token's kept slots in slot order (adaptive top-p leaves a
        // prefix; a dropped slot has no row), then its shared row
        int c = 0;
        for (int i = 0; i < k; i++) {
            const int r = a.inv[(size_t)t * k + i];
            if (r >= 0) rows[c++] = r;
        }
        if (a.n_shared) rows[c++] = a.Tk + t;
        nr = c;
    }
    __syncthreads();
    float *out = a.y + (size_t)t * H;
    if (((uintptr_t)out & 15) == 0) {
        for (int c = threadIdx.x; c < H / 4; c += 256) {
            float4 s = reinterpret_cast<const float4 *>(a.yrows + (size_t)rows[0] * H)[c];
            for (int j = 1; j < nr; j++) {
                const float4 v = reinterpret_cast<const float4 *>(a.yrows + (size_t)rows[j] * H)[c];
                s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
            }
            float4 *o = reinterpret_cast<float4 *>(out) + c;
            if (a.accumulate) {
                const float4 p = *o;
                s.x = p.x + s.x; s.y = p.y + s.y; s.z = p.z + s.z; s.w = p.w + s.w;
            }
            *o = s;
        }
    } else {
        for (int c = threadIdx.x; c < H; c += 256) {
            float s = a.yrows[(size_t)rows[0] * H + c];
            for (int j = 1; j < nr; j++) s += a.yrows[(size_t)rows[j] * H + c];
            out[c] = a.accumulate ? out[c] + s : s;
        }
    }
}

// ---------------------------------------------------------------- launchers
// 1-D grids of 8 XCDs x (channel groups per XCD) x max_tiles workgroups
static unsigned gg_grid(int ncg, int max_tiles) { return 8u * (unsigned)((ncg + 7) / 8) * (unsigned)max_tiles; }

int launch_gg_gate_up(const GgArgs &a, int max_tiles, hipStream_t st)
{
    const unsigned grid = gg_grid(a.I / 128, max_tiles);
    if (a.wbits == 4) k_gg_gate_up<4><<<grid, kGgThreads, 0, st>>>(a);
    else if (a.wbits == 8) k_gg_gate_up<8><<<grid, kGgThreads, 0, st>>>(a);
    else k_gg_gate_up<2><<<grid, kGgThreads, 0, st>>>(a);
    return (int)hipGetLastError();
}

int launch_gg_down(const GgArgs &a, int max_tiles, hipStream_t st)
{
    const unsigned grid = gg_grid(a.H / 256, max_tiles);
    if (a.wbits == 4) k_gg_down<4><<<grid, kGgThreads, 0, st>>>(a);
    else if (a.wbits == 8) k_gg_down<8><<<grid, kGgThreads, 0, st>>>(a);
    else k_gg_down<2><<<grid, kGgThreads, 0, st>>>(a);
    return (int)hipGetLastError();
}

int launch_gg_combine(const GgArgs &a, hipStream_t st)
{
    k_gg_combine<<<a.T, 256, 0, st>>>(a);
    return (int)hipGetLastError();
}

} // namespace moe

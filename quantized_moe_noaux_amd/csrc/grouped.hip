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
// rows for the shared expert.  Rows are cut into tiles of kGgTN rows that
// never straddle two experts; every tile is a small GEMM against its
// expert's weights:
//   k_gg_gate_up  one workgroup per (tile, 64 intermediate channels): the
//                 int4/int2 codes are expanded to int8 in LDS, the tile's
//                 activation rows are gathered into LDS, and
//                 v_mfma_i32_32x32x32_i8 gives the exact int32 dot of every
//                 (channel, row, 32-block); each is scaled by its activation
//                 block scale and summed in fp32.  Then g, u -> h = silu(g) u
//                 -> int8 h in blocks of 32 channels.
//   k_gg_down     one workgroup per (tile, 128 hidden channels): the same
//                 over the int8 h rows; the result is scaled by the row's
//                 combine weight and written to the row's output slot.
//   k_gg_combine  out[t] = t's k routed slots in slot order, then the shared
//                 row.
// No float atomics anywhere: results are run-to-run identical.
//
// Weight codes are expanded in offset form (c + 8 for int4, c + 2 for int2,
// both non-negative), so an MFMA block dot is sum (c + o) q = sum c q + o S
// with S the block's activation code sum.  The offset term depends on the
// activation row only, so it is removed once per row at the end:
// acc - o * sum_b d_b S_b, with that sum formed where the row is quantised.
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kGgKS = 64;           // K per pipeline step (two 32-blocks)
constexpr int kGgRow = kGgKS + 16;  // LDS bytes per staged row (padding: conflict-free 16-byte reads)
constexpr int kGgWRows = 128;       // weight rows staged per workgroup
constexpr int kGgThreads = 256;

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
    w.xs = o;     o = align256(o + sizeof(float) * (size_t)T);
    w.perm = o;   o = align256(o + sizeof(int32_t) * Tk);
    w.off = o;    o = align256(o + sizeof(int32_t) * (E + 1));
    w.inv = o;    o = align256(o + sizeof(int32_t) * Tk);
    w.pscr = o;   o = align256(o + sizeof(int32_t) * perm_tiles((int)Tk) * E);
    w.tiles = o;  o = align256(o + sizeof(int4) * (size_t)(gg_max_tiles(s, T) + 1));
    w.qh = o;     o = align256(o + R * I);
    w.dh = o;     o = align256(o + sizeof(float) * R * (I / 32));
    w.zh = o;     o = align256(o + sizeof(float) * R * (I / 32));
    w.y = o;      o = align256(o + sizeof(float) * R * H);
    w.total = o;
    return w;
}

// ---------------------------------------------------------------- row quantiser
// One workgroup per row of D values: Q8_0-style blocks (8 lanes per block,
// quant_block8) and xs[row] = sum_b d_b * S_b in fp64 (S_b = the block's
// code sum), the offset correction of the grouped GEMMs.
__global__ __launch_bounds__(256) void k_gg_quant(const float *__restrict__ x, int D, int8_t *__restrict__ q,
                                                  float *__restrict__ d, float *__restrict__ xs)
{
    __shared__ double part[32];
    const int row = blockIdx.x, tid = threadIdx.x, bs = tid >> 3, sub = tid & 7;
    const int nb = D / 32;
    const float *xr = x + (size_t)row * D;
    double acc = 0.0;
    for (int b0 = 0; b0 < nb; b0 += 32) {
        const int b = b0 + bs;
        const bool live = b < nb;
        const float4 v = live ? reinterpret_cast<const float4 *>(xr + 32 * b)[sub] : make_float4(0, 0, 0, 0);
        float db;
        const uint32_t packed = quant_block8(v, db);
        int s = sdot4(packed, 0x01010101u, 0);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        if (live) {
            reinterpret_cast<uint32_t *>(q + (size_t)row * D + 32 * b)[sub] = packed;
            if (sub == 0) {
                d[(size_t)row * nb + b] = db;
                acc += (double)db * (double)s;
            }
        }
    }
    if (sub == 0) part[bs] = acc;
    __syncthreads();
    if (tid == 0) {
        double s = 0.0;
        for (int i = 0; i < 32; i++) s += part[i];
        xs[row] = (float)s;
    }
}

int launch_gg_quant(const float *x, int T, int D, int8_t *q, float *d, float *xs, hipStream_t st)
{
    k_gg_quant<<<T, 256, 0, st>>>(x, D, q, d, xs);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- staging
// One pipeline step moves K = 64 of kGgWRows weight rows and of kGgTN
// activation rows into LDS as int8, both sides in the same code order within
// each 16-byte group (the expansion of a packed dword interleaves codes).
//
// int4: a dword holds codes 8j..8j+7 (even code in the low nibble).  Its low
//   nibbles become one dword (codes 0,2,4,6) and its high nibbles the next
//   (1,3,5,7).
// int2: a dword holds codes 16j..16j+15, code 4m+i at byte m, bits 2i.  Field
//   i of the four bytes becomes dword i (codes i, 4+i, 8+i, 12+i).
// int8: natural order.
template <int WB> struct GgW;

template <> struct GgW<4> {
    static constexpr int kOff = 8;
    uint4 r;  // 32 codes: one block of one row
    __device__ __forceinline__ void load(const uint8_t *row, int k0, int half)
    {
        r = *reinterpret_cast<const uint4 *>(row + k0 / 2 + 16 * half);
    }
    __device__ __forceinline__ void store(uint8_t *lds_row, int half) const
    {
        const uint32_t w0 = r.x ^ 0x88888888u, w1 = r.y ^ 0x88888888u;
        const uint32_t w2 = r.z ^ 0x88888888u, w3 = r.w ^ 0x88888888u;
        uint4 o0, o1;
        o0.x = w0 & 0x0F0F0F0Fu; o0.y = (w0 >> 4) & 0x0F0F0F0Fu;
        o0.z = w1 & 0x0F0F0F0Fu; o0.w = (w1 >> 4) & 0x0F0F0F0Fu;
        o1.x = w2 & 0x0F0F0F0Fu; o1.y = (w2 >> 4) & 0x0F0F0F0Fu;
        o1.z = w3 & 0x0F0F0F0Fu; o1.w = (w3 >> 4) & 0x0F0F0F0Fu;
        uint4 *p = reinterpret_cast<uint4 *>(lds_row + 32 * half);
        p[0] = o0;
        p[1] = o1;
    }
};

template <> struct GgW<8> {
    static constexpr int kOff = 0;
    v4i r0, r1;
    __device__ __forceinline__ void load(const uint8_t *row, int k0, int half)
    {
        const v4i *p = reinterpret_cast<const v4i *>(row + k0 + 32 * half);
        r0 = p[0];
        r1 = p[1];
    }
    __device__ __forceinline__ void store(uint8_t *lds_row, int half) const
    {
        v4i *p = reinterpret_cast<v4i *>(lds_row + 32 * half);
        p[0] = r0;
        p[1] = r1;
    }
};

template <> struct GgW<2> {
    static constexpr int kOff = 2;
    uint2 r;  // 32 codes: one block of one row
    __device__ __forceinline__ void load(const uint8_t *row, int k0, int half)
    {
        r = *reinterpret_cast<const uint2 *>(row + k0 / 4 + 8 * half);
    }
    __device__ __forceinline__ void store(uint8_t *lds_row, int half) const
    {
        const uint32_t a = r.x ^ 0xAAAAAAAAu, b = r.y ^ 0xAAAAAAAAu;
        uint4 o0, o1;
        o0.x = a & 0x03030303u; o0.y = (a >> 2) & 0x03030303u;
        o0.z = (a >> 4) & 0x03030303u; o0.w = (a >> 6) & 0x03030303u;
        o1.x = b & 0x03030303u; o1.y = (b >> 2) & 0x03030303u;
        o1.z = (b >> 4) & 0x03030303u; o1.w = (b >> 6) & 0x03030303u;
        uint4 *p = reinterpret_cast<uint4 *>(lds_row + 32 * half);
        p[0] = o0;
        p[1] = o1;
    }
};

// 16 activation codes in natural order -> the code order of the weights
template <int WB> __device__ __forceinline__ uint4 gg_act_order(uint4 v)
{
    if constexpr (WB == 4) {
        uint4 o;
        o.x = perm(v.y, v.x, 0x06040200u); o.y = perm(v.y, v.x, 0x07050301u);
        o.z = perm(v.w, v.z, 0x06040200u); o.w = perm(v.w, v.z, 0x07050301u);
        return o;
    } else if constexpr (WB == 2) {
        const uint32_t p01 = perm(v.y, v.x, 0x06020400u), q01 = perm(v.y, v.x, 0x07030501u);
        const uint32_t p23 = perm(v.w, v.z, 0x06020400u), q23 = perm(v.w, v.z, 0x07030501u);
        uint4 o;
        o.x = perm(p23, p01, 0x05040100u);
        o.y = perm(q23, q01, 0x05040100u);
        o.z = perm(p23, p01, 0x07060302u);
        o.w = perm(q23, q01, 0x07060302u);
        return o;
    } else {
        return v;
    }
}

struct GgLds {
    uint8_t w[2][kGgWRows][kGgRow];  // weight rows (int8, offset form), two pipeline buffers
    uint8_t a[2][kGgTN][kGgRow];     // activation rows
    float d[2][2][kGgTN];            // activation block scales of the step's two blocks
    int arow[kGgTN];                 // activation row of each tile row (-1: padding)
    float corr[kGgTN];               // sum_b d_b S_b of each tile row
    float cw[kGgTN];                 // combine weight of each tile row (down only)
};

__device__ __forceinline__ v4i lds16(const uint8_t *p) { return *reinterpret_cast<const v4i *>(p); }

// Main loop shared by both GEMMs (n = live rows of the tile).  L.arow must
// be set.  Thread tid loads
// weight row tid/2 (wsrc), half tid%2 of each step; activation row tid/4,
// 16-byte part tid%4; and (tid < 128) the scale of row tid/2, block tid%2.
// Wave w computes activation rows 32*nt .. +32 of the tile against weight
// tiles m0 and m1 (32 rows each); acc0 / acc1 come back in MFMA layout:
// lane l, register v = weight row 8(v/4) + 4(l/32) + v%4 of the tile,
// activation row l%32.
template <int WB>
__device__ __forceinline__ void gg_mainloop(GgLds &L, const uint8_t *wsrc, const int8_t *__restrict__ aq,
                                            const float *__restrict__ ad, int K, int nt, int m0, int m1, int n,
                                            float (&acc0)[16], float (&acc1)[16])
{
    // a wave whose 32 rows are all padding only loads and stages
    const bool live = 32 * nt < n;
    const int tid = threadIdx.x, l = lane_id();
    const int nbk = K / 32, nsteps = K / kGgKS;
    const int wr = tid >> 1, wh = tid & 1;
    const int ar = tid >> 2, ap = tid & 3;
    const int dr = (tid >> 1) & (kGgTN - 1), db = tid & 1;
    const int arow_a = L.arow[ar], arow_d = L.arow[dr];
    const int8_t *asrc = arow_a >= 0 ? aq + (size_t)arow_a * K + 16 * ap : nullptr;
    const float *dsrc = (tid < 2 * kGgTN && arow_d >= 0) ? ad + (size_t)arow_d * nbk + db : nullptr;
    GgW<WB> wn;
    uint4 an;
    float dn;
    auto fetch = [&](int s) {
        const int k0 = s * kGgKS;
        wn.load(wsrc, k0, wh);
        an = asrc ? *reinterpret_cast<const uint4 *>(asrc + k0) : make_uint4(0, 0, 0, 0);
        dn = dsrc ? dsrc[2 * s] : 0.f;
    };
    auto stage = [&](int buf) {
        wn.store(L.w[buf][wr], wh);
        *reinterpret_cast<uint4 *>(&L.a[buf][ar][16 * ap]) = gg_act_order<WB>(an);
        if (tid < 2 * kGgTN) L.d[buf][db][dr] = dn;
    };
    v16i zero;
#pragma unroll
    for (int v = 0; v < 16; v++) zero[v] = 0;
#pragma unroll
    for (int v = 0; v < 16; v++) { acc0[v] = 0.f; acc1[v] = 0.f; }

    fetch(0);
    stage(0);
    __syncthreads();
    for (int s = 0; s < nsteps; s++) {
        const int buf = s & 1;
        if (s + 1 < nsteps) fetch(s + 1);
#pragma unroll
        for (int b = 0; b < 2 && live; b++) {
            const int koff = 32 * b + 16 * (l >> 5);
            const v4i a0 = lds16(&L.w[buf][32 * m0 + (l & 31)][koff]);
            const v4i a1 = lds16(&L.w[buf][32 * m1 + (l & 31)][koff]);
            const v4i bx = lds16(&L.a[buf][32 * nt + (l & 31)][koff]);
            const float dd = L.d[buf][b][32 * nt + (l & 31)];
            const v16i i0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bx, zero, 0, 0, 0);
            const v16i i1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bx, zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; v++) {
                acc0[v] = fmaf((float)i0[v], dd, acc0[v]);
                acc1[v] = fmaf((float)i1[v], dd, acc1[v]);
            }
        }
        if (s + 1 < nsteps) stage(buf ^ 1);
        __syncthreads();
    }
}

__device__ __forceinline__ const moe_weights_t &gg_expert(const GgArgs &a, int e, size_t &eo)
{
    eo = (e == a.E) ? 0 : (size_t)e;
    return (e == a.E) ? a.shared : a.routed;
}

// ---------------------------------------------------------------- gate / up
template <int WB>
__global__ __launch_bounds__(kGgThreads) void k_gg_gate_up(const GgArgs a)
{
    __shared__ GgLds L;
    if ((int)blockIdx.y >= a.tiles[0].x) return;
    const int4 tile = a.tiles[1 + blockIdx.y];
    const int e = tile.x, row0 = tile.y, n = tile.z;
    const int tid = threadIdx.x, H = a.H, I = a.I;
    const int c0 = blockIdx.x * 64;
    const size_t rb = (size_t)H * WB / 8;
    size_t eo;
    const moe_weights_t &W = gg_expert(a, e, eo);
    if (tid < kGgTN) {
        int tok = -1;
        if (tid < n) {
            const int r = row0 + tid;
            tok = (r < a.Tk) ? a.perm[r] / a.k : r - a.Tk;
        }
        L.arow[tid] = tok;
        L.corr[tid] = tok >= 0 ? a.xs[tok] : 0.f;
    }
    __syncthreads();
    const int wr = tid >> 1;
    const uint8_t *wsrc = (wr < 64) ? W.gate + (eo * I + c0 + wr) * rb : W.up + (eo * I + c0 + wr - 64) * rb;
    const int wv = wave_id(), nt = wv >> 1, mh = wv & 1;
    float ag[16], au[16];
    gg_mainloop<WB>(L, wsrc, a.xq, a.xd, H, nt, mh, 2 + mh, n, ag, au);

    // epilogue: lane = (tile row i, channel half hf); 16 channels of the
    // wave's 32-channel block cb
    const int l = lane_id(), i = 32 * nt + (l & 31), hf = l >> 5;
    const float corr = (float)GgW<WB>::kOff * L.corr[i];
    const int cb = c0 + 32 * mh;
    const float *gs = W.gate_s + eo * I, *us = W.up_s + eo * I;
    float h[16];
#pragma unroll
    for (int v = 0; v < 16; v++) {
        const int ch = cb + 8 * (v >> 2) + 4 * hf + (v & 3);
        const float g = gs[ch] * (ag[v] - corr);
        const float u = us[ch] * (au[v] - corr);
        h[v] = silu_mul(g, u);
    }
    // Q8_0 quantisation of h over the block of 32 channels (this lane's 16
    // and lane l^32's 16)
    float amax = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v++) amax = fmaxf(amax, fabsf(h[v]));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float dq = amax / 127.0f;
    uint32_t wq[4] = {0, 0, 0, 0};
    int qsum = 0;
#pragma unroll
    for (int v = 0; v < 16; v++) {
        float r = (dq == 0.0f) ? 0.0f : rintf(h[v] / dq);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const int qi = (int)r;
        qsum += qi;
        wq[v >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (v & 3));
    }
    qsum += __shfl_xor(qsum, 32);
    if (i < n) {
        const size_t r = (size_t)row0 + i;
        int8_t *qrow = a.qh + r * I;
#pragma unroll
        for (int j = 0; j < 4; j++) *reinterpret_cast<uint32_t *>(qrow + cb + 8 * j + 4 * hf) = wq[j];
        if (hf == 0) {
            a.dh[r * (I / 32) + cb / 32] = dq;
            a.zh[r * (I / 32) + cb / 32] = dq * (float)qsum;
        }
    }
}

// ---------------------------------------------------------------- down
template <int WB>
__global__ __launch_bounds__(kGgThreads) void k_gg_down(const GgArgs a)
{
    __shared__ GgLds L;
    if ((int)blockIdx.y >= a.tiles[0].x) return;
    const int4 tile = a.tiles[1 + blockIdx.y];
    const int e = tile.x, row0 = tile.y, n = tile.z;
    const int tid = threadIdx.x, H = a.H, I = a.I, nbh = I / 32;
    const int n0 = blockIdx.x * 128;
    const size_t rb = (size_t)I * WB / 8;
    size_t eo;
    const moe_weights_t &W = gg_expert(a, e, eo);
    {
        // correction sum_b dh_b S_b of each row: 4 threads per row, fixed order
        const int i = tid >> 2, p = tid & 3;
        float z = 0.f;
        if (i < n)
            for (int b = p; b < nbh; b += 4) z += a.zh[(size_t)(row0 + i) * nbh + b];
        z += __shfl_xor(z, 1);
        z += __shfl_xor(z, 2);
        if (p == 0) {
            const int r = row0 + i;
            L.arow[i] = (i < n) ? r : -1;
            L.corr[i] = z;
            L.cw[i] = (i < n && r < a.Tk) ? a.w[a.perm[r]] : 1.0f;
        }
    }
    __syncthreads();
    const uint8_t *wsrc = W.down + (eo * H + n0 + (tid >> 1)) * rb;
    const int wv = wave_id(), nt = wv >> 1, m0 = 2 * (wv & 1);
    float y0[16], y1[16];
    gg_mainloop<WB>(L, wsrc, a.qh, a.dh, I, nt, m0, m0 + 1, n, y0, y1);

    const int l = lane_id(), i = 32 * nt + (l & 31), hf = l >> 5;
    if (i >= n) return;
    const float corr = (float)GgW<WB>::kOff * L.corr[i], cw = L.cw[i];
    const float *ds = W.down_s + eo * H;
    float *yrow = a.yrows + (size_t)(row0 + i) * H;
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const float *acc = t ? y1 : y0;
        const int cbase = n0 + 32 * (m0 + t) + 4 * hf;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int ch = cbase + 8 * j;
            float4 o;
            o.x = ds[ch + 0] * (acc[4 * j + 0] - corr) * cw;
            o.y = ds[ch + 1] * (acc[4 * j + 1] - corr) * cw;
            o.z = ds[ch + 2] * (acc[4 * j + 2] - corr) * cw;
            o.w = ds[ch + 3] * (acc[4 * j + 3] - corr) * cw;
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
int launch_gg_gate_up(const GgArgs &a, int max_tiles, hipStream_t st)
{
    const dim3 grid(a.I / 64, max_tiles);
    if (a.wbits == 4) k_gg_gate_up<4><<<grid, kGgThreads, 0, st>>>(a);
    else if (a.wbits == 8) k_gg_gate_up<8><<<grid, kGgThreads, 0, st>>>(a);
    else k_gg_gate_up<2><<<grid, kGgThreads, 0, st>>>(a);
    return (int)hipGetLastError();
}

int launch_gg_down(const GgArgs &a, int max_tiles, hipStream_t st)
{
    const dim3 grid(a.H / 128, max_tiles);
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

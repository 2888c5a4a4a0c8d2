// MTP draft verification: which drafts a verify forward keeps, and the token
// it emits after them.
//
// GeekNews #31297, implemented features: the multi-token-prediction head
// drafts tokens, the main model verifies them in one batched forward
// (batch-union MoE reads each expert once for all positions), and rejection
// sampling keeps sampled output lossless; useful options: --temp (0 =
// greedy).  The rule is speculative sampling (Leviathan, Kalman & Matias,
// ICML 2023; Chen et al. 2023): draft x_i is kept when u_i q_i(x_i) <
// p_i(x_i), with p, q = softmax(logits / tau); at the first refusal the
// emitted token is the inverse-CDF draw (ascending token order) of
// max(0, p_i - q_i), or of p_i if that has no mass; after the last draft it
// is the draw of p_D.  Greedy keeps drafts while they equal the target's
// argmax (lowest index on ties) and emits the argmax at the first mismatch.
// Everything that decides a token is fp64.
//
// Four launches (two for greedy):
//  k_ac_stats   per (row, 4096-token chunk): the chunk's max logit, its first
//               argmax and sum exp((z - max) / tau)
//  k_ac_decide  per sequence: each row's max and normaliser combined over
//               its chunks in chunk order, the drafts' probabilities
//               exp((z - M) / tau) / Z and the walk over the drafts; writes
//               the kept count (and, greedy, the argmax token)
//  k_ac_mass    per (sequence, 1024-token chunk): every token's weight in
//               the distribution the emitted token is drawn from, and the
//               chunk's masses of it and of p
//  k_ac_pick    per sequence: the chunk where the cumulative mass crosses
//               u_D * total (a block scan in chunk order) and the token
//               inside it (a block scan in token order)
// Fixed reduction orders: the results are run-to-run identical.
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {

constexpr int kAcThreads = 256;
constexpr int kAcPer = 16;                           // tokens per thread per chunk
constexpr int kAcChunk = kAcThreads * kAcPer;        // 4096
constexpr int kAcMassChunk = kAcThreads * 4;         // 1024: tokens per draw chunk
static_assert(kAcMassChunk == kMtpDrawChunk, "draw chunk size (workspace sizing)");
static_assert(kAcChunk == kMtpChunk, "chunk size (workspace sizing)");

struct AcStat {
    double s;   // sum over the chunk of exp((z - m) / tau)
    float m;    // the chunk's max logit
    int arg;    // its first position
};
static_assert(sizeof(AcStat) == 16, "stat size (workspace sizing)");

struct AcArgs {
    int B, D, V, C;             // sequences, drafts, vocabulary, chunks per row
    const int32_t *draft;       // [B][D]
    const float *p;             // [B][D+1][V]
    const float *q;             // [B][D][V]
    double tau;
    const double *u;            // [B][D+1]
    int32_t *n_acc, *next;      // [B]
    AcStat *stats;              // [B][2D+1][C]: rows 0..D target, D+1.. draft model
    struct AcDec *dec;          // [B]: the decision
    double2 *mass;              // [B][CM]: (draw mass, target mass) per 1024-token chunk
    double *w;                  // [B][CM * 1024]: every token's weight in the draw
    int CM;                     // draw chunks per row
};

// The decision of one sequence, as k_ac_decide writes it for the draw: the
// kept drafts, whether the emitted token is drawn from the residual of the
// target and draft rows (row_p, row_q) or from the target row alone, and the
// rows' max logits and normalisers.
struct AcDec {
    int j, resid, row_p, row_q;
    float Mp, Mq;
    double Zp, Zq;
};

__device__ __forceinline__ const float *ac_row(const AcArgs &a, int b, int r)
{
    return r <= a.D ? a.p + ((size_t)b * (a.D + 1) + r) * a.V : a.q + ((size_t)b * a.D + (r - a.D - 1)) * a.V;
}

// ---------------------------------------------------------------- stats
// Thread t holds tokens c0 + 4t + 1024j + (0..3), j < 4 (float4 loads, one
// 4 KB window per load instruction); positions past V read the last token
// (clamped, so every load is unconditional) and count as -inf.
template <bool VEC>
__device__ __forceinline__ void ac_load(const float *row, int V, int c0, float (&z)[kAcPer], int (&pos)[kAcPer])
{
#pragma unroll
    for (int j = 0; j < kAcPer / 4; j++) {
        const int x0 = c0 + 4 * (int)threadIdx.x + 1024 * j;
        if constexpr (VEC) {
            const float4 v = reinterpret_cast<const float4 *>(row)[min(x0, V - 4) / 4];
            z[4 * j] = v.x; z[4 * j + 1] = v.y; z[4 * j + 2] = v.z; z[4 * j + 3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++) z[4 * j + e] = row[min(x0 + e, V - 1)];
        }
#pragma unroll
        for (int e = 0; e < 4; e++) pos[4 * j + e] = x0 + e;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kAcThreads) void k_ac_stats(const AcArgs a)
{
    __shared__ float sm[kAcThreads / kWave];
    __shared__ int sa[kAcThreads / kWave];
    __shared__ double ss[kAcThreads / kWave];
    const int c = blockIdx.x, R = 2 * a.D + 1;
    const int b = blockIdx.y / R, r = blockIdx.y % R;
    const float *row = ac_row(a, b, r);
    float z[kAcPer];
    int pos[kAcPer];
    ac_load<VEC>(row, a.V, c * kAcChunk, z, pos);
    // max and first argmax: thread, then wave (value desc, position asc),
    // then the four waves
    float m = -INFINITY;
    int arg = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kAcPer; i++) {
        const bool ok = pos[i] < a.V;
        if (ok && (z[i] > m || (z[i] == m && pos[i] < arg))) { m = z[i]; arg = pos[i]; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(m, o);
        const int oa = __shfl_xor(arg, o);
        if (om > m || (om == m && oa < arg)) { m = om; arg = oa; }
    }
    if (lane_id() == 0) { sm[wave_id()] = m; sa[wave_id()] = arg; }
    __syncthreads();
    m = sm[0]; arg = sa[0];
#pragma unroll
    for (int w = 1; w < kAcThreads / kWave; w++)
        if (sm[w] > m || (sm[w] == m && sa[w] < arg)) { m = sm[w]; arg = sa[w]; }
    double s = 0.0;
    if (a.tau > 0.0) {
#pragma unroll
        for (int i = 0; i < kAcPer; i++)
            s += (pos[i] < a.V) ? exp(((double)z[i] - (double)m) / a.tau) : 0.0;
        s = wave_sum_d(s);
        if (lane_id() == 0) ss[wave_id()] = s;
        __syncthreads();
        s = ((ss[0] + ss[1]) + ss[2]) + ss[3];
    }
    if (threadIdx.x == 0) {
        AcStat st;
        st.s = s; st.m = m; st.arg = arg;
        a.stats[((size_t)b * R + r) * a.C + c] = st;
    }
}

// ---------------------------------------------------------------- decision
// Max and normaliser of row r combined over its chunks (one wave: lane l
// takes chunks l, l+64, l+128, l+192, all loads at clamped indices at once;
// then the 64 lanes' partial values in a fixed tree).
constexpr int kAcNormPer = kMtpMaxChunks / kWave;
struct AcNorm {
    float M;
    double Z;
    int arg;
};

__device__ __forceinline__ AcNorm ac_norm(const AcArgs &a, int b, int r)
{
    const AcStat *st = a.stats + ((size_t)b * (2 * a.D + 1) + r) * a.C;
    const int l = lane_id();
    AcStat sv[kAcNormPer];
#pragma unroll
    for (int i = 0; i < kAcNormPer; i++) sv[i] = st[min(l + kWave * i, a.C - 1)];
    float M = -INFINITY;
    int arg = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kAcNormPer; i++) {
        const bool ok = l + kWave * i < a.C;
        if (ok && (sv[i].m > M || (sv[i].m == M && sv[i].arg < arg))) { M = sv[i].m; arg = sv[i].arg; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(M, o);
        const int oa = __shfl_xor(arg, o);
        if (om > M || (om == M && oa < arg)) { M = om; arg = oa; }
    }
    double Z = 0.0;
    if (a.tau > 0.0) {
#pragma unroll
        for (int i = 0; i < kAcNormPer; i++)
            Z += (l + kWave * i < a.C) ? sv[i].s * exp(((double)sv[i].m - (double)M) / a.tau) : 0.0;
        Z = wave_sum_d(Z);
    }
    AcNorm n;
    n.M = M; n.Z = Z; n.arg = arg;
    return n;
}

struct AcDecision {
    int j;         // drafts kept
    int row_p;     // target row the emitted token is drawn from
    bool resid;    // draw from max(0, p - q) of rows (row_p, its draft row)
    AcNorm np, nq;
};

// LDS of the decision
struct AcDecLds {
    AcNorm nrm[2 * kMtpMaxDraft + 1];
    double zp[kMtpMaxDraft], zq[kMtpMaxDraft], u[kMtpMaxDraft];
    int x[kMtpMaxDraft];
    int j;
};

// The whole workgroup calls it; the result is uniform.  Waves combine the
// rows' stats (wave w: rows w, w+4, ...) while threads i < D fetch draft
// i's token, its two logits and its uniform; then one thread walks the
// drafts in order.
__device__ __forceinline__ AcDecision ac_decide(const AcArgs &a, int b, AcDecLds &L)
{
    const int R = 2 * a.D + 1, tid = threadIdx.x;
    if (tid < a.D) {
        const int x = a.draft[(size_t)b * a.D + tid];
        const int xc = min(max(x, 0), a.V - 1);
        L.x[tid] = x;
        L.zp[tid] = (double)ac_row(a, b, tid)[xc];
        L.zq[tid] = (double)ac_row(a, b, a.D + 1 + tid)[xc];
        L.u[tid] = a.u[(size_t)b * (a.D + 1) + tid];
    }
    for (int r = wave_id(); r < R; r += kAcThreads / kWave) {
        const AcNorm n = ac_norm(a, b, r);
        if (lane_id() == 0) L.nrm[r] = n;
    }
    __syncthreads();
    if (tid == 0) {
        int j = a.D;
        for (int i = 0; i < a.D; i++) {
            const int x = L.x[i];
            bool keep;
            if (a.tau == 0.0) {
                keep = (x == L.nrm[i].arg);
            } else {
                const AcNorm &np = L.nrm[i], &nq = L.nrm[a.D + 1 + i];
                const double P = exp((L.zp[i] - (double)np.M) / a.tau) / np.Z;
                const double Q = exp((L.zq[i] - (double)nq.M) / a.tau) / nq.Z;
                keep = (x >= 0 && x < a.V) && L.u[i] * Q < P;
            }
            if (!keep) { j = i; break; }
        }
        L.j = j;
    }
    __syncthreads();
    AcDecision d;
    d.j = L.j;
    d.row_p = d.j;
    d.resid = d.j < a.D && a.tau > 0.0;
    d.np = L.nrm[d.j];
    d.nq = L.nrm[d.resid ? a.D + 1 + d.j : d.j];  // both from LDS: no select between address spaces
    return d;
}

// ---------------------------------------------------------------- decision launch
__global__ __launch_bounds__(kAcThreads) void k_ac_decide(const AcArgs a)
{
    __shared__ AcDecLds dl;
    const int b = blockIdx.x;
    const AcDecision d = ac_decide(a, b, dl);
    if (threadIdx.x == 0) {
        AcDec o;
        o.j = d.j;
        o.resid = d.resid;
        o.row_p = d.row_p;
        o.row_q = d.resid ? a.D + 1 + d.j : d.row_p;
        o.Mp = d.np.M; o.Zp = d.np.Z;
        o.Mq = d.nq.M; o.Zq = d.nq.Z;
        a.dec[b] = o;
        a.n_acc[b] = d.j;
        if (a.tau == 0.0) a.next[b] = d.np.arg;
    }
}

// weight of a token in the draw: max(0, p - q) for a residual, else p; and
// its target probability (p = exp((z - M) / tau) times 1 / Z)
__device__ __forceinline__ void ac_weight(const AcDec &d, double tau, double ip, double iq, float zp, float zq,
                                          double &w, double &pw)
{
    const double P = exp(((double)zp - (double)d.Mp) / tau) * ip;
    pw = P;
    if (d.resid) {
        const double Q = exp(((double)zq - (double)d.Mq) / tau) * iq;
        w = P > Q ? P - Q : 0.0;
    } else {
        w = P;
    }
}

// ---------------------------------------------------------------- draw weights and chunk masses
// One workgroup per (sequence, 1024-token chunk): thread t takes tokens
// c0 + 4t .. +3 (one float4 per row), stores their draw weights and adds
// the chunk's draw and target masses (fixed order).
template <bool VEC>
__global__ __launch_bounds__(kAcThreads) void k_ac_mass(const AcArgs a)
{
    __shared__ double sw[kAcThreads / kWave], sp[kAcThreads / kWave];
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const AcDec d = a.dec[b];
    const float *rp = ac_row(a, b, d.row_p), *rq = ac_row(a, b, d.row_q);
    const int x0 = c * kAcMassChunk + 4 * tid;
    float zp[4], zq[4];
    if constexpr (VEC) {
        const float4 vp = reinterpret_cast<const float4 *>(rp)[min(x0, a.V - 4) / 4];
        const float4 vq = reinterpret_cast<const float4 *>(rq)[min(x0, a.V - 4) / 4];
        zp[0] = vp.x; zp[1] = vp.y; zp[2] = vp.z; zp[3] = vp.w;
        zq[0] = vq.x; zq[1] = vq.y; zq[2] = vq.z; zq[3] = vq.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++) { zp[e] = rp[min(x0 + e, a.V - 1)]; zq[e] = rq[min(x0 + e, a.V - 1)]; }
    }
    const double ip = 1.0 / d.Zp, iq = 1.0 / d.Zq;
    double wv[4], w = 0.0, pw = 0.0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        double wi, pi;
        ac_weight(d, a.tau, ip, iq, zp[e], zq[e], wi, pi);
        const bool ok = x0 + e < a.V;
        wv[e] = ok ? wi : 0.0;
        w += wv[e];
        pw += ok ? pi : 0.0;
    }
    double2 *dst = reinterpret_cast<double2 *>(a.w + (size_t)b * a.CM * kAcMassChunk + x0);
    dst[0] = make_double2(wv[0], wv[1]);
    dst[1] = make_double2(wv[2], wv[3]);
    w = wave_sum_d(w);
    pw = wave_sum_d(pw);
    if (lane_id() == 0) { sw[wave_id()] = w; sp[wave_id()] = pw; }
    __syncthreads();
    if (tid == 0)
        a.mass[(size_t)b * a.CM + c] = make_double2(((sw[0] + sw[1]) + sw[2]) + sw[3], ((sp[0] + sp[1]) + sp[2]) + sp[3]);
}

// Exclusive scan of two doubles over the 256 threads in thread order (a wave
// scan, then the four wave totals in order); totals to every thread.
// red: LDS of 8 doubles.
__device__ __forceinline__ void block_scan2(double x, double y, double &ex, double &ey, double &tx, double &ty,
                                            double *red)
{
    const int l = lane_id(), wv = wave_id();
    double ix = x, iy = y;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double ux = __shfl_up(ix, o), uy = __shfl_up(iy, o);
        if (l >= o) { ix += ux; iy += uy; }
    }
    if (l == kWave - 1) { red[wv] = ix; red[4 + wv] = iy; }
    __syncthreads();
    double px = 0.0, py = 0.0;
    tx = 0.0; ty = 0.0;
#pragma unroll
    for (int i = 0; i < kAcThreads / kWave; i++) {
        if (i < wv) { px += red[i]; py += red[4 + i]; }
        tx += red[i];
        ty += red[4 + i];
    }
    ex = px + (ix - x);
    ey = py + (iy - y);
    __syncthreads();  // red is reused
}

// ---------------------------------------------------------------- the draw
// The chunk the draw falls in (thread t holds chunks 4t .. 4t+3; an
// exclusive block scan of the threads' sums gives every chunk's cumulative
// mass in chunk order), then the token inside it (thread t holds tokens
// c0 + 4t .. +3, the same scan in token order).  A residual without mass
// falls back to the target row itself (its weights recomputed here).
__global__ __launch_bounds__(kAcThreads) void k_ac_pick(const AcArgs a)
{
    __shared__ int s_chunk, s_hit, s_last;
    __shared__ double s_target;
    __shared__ double red[2 * kAcThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x;
    const AcDec d = a.dec[b];
    const double2 *ms = a.mass + (size_t)b * a.CM;
    double wr[4], wp[4], sr = 0.0, sp = 0.0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const int c = 4 * tid + e;
        const double2 m = ms[min(c, a.CM - 1)];
        wr[e] = c < a.CM ? m.x : 0.0;
        wp[e] = c < a.CM ? m.y : 0.0;
        sr += wr[e];
        sp += wp[e];
    }
    double er, ep, Wr, Wp;
    block_scan2(sr, sp, er, ep, Wr, Wp, red);
    const bool use_p = !(Wr > 0.0);
    const double t = a.u[(size_t)b * (a.D + 1) + a.D] * (use_p ? Wp : Wr);
    if (tid == 0) { s_hit = 0x7fffffff; s_last = -1; }
    __syncthreads();
    double cum = use_p ? ep : er, tloc = 0.0;
    int hit = 0x7fffffff, last = -1;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const double wc = use_p ? wp[e] : wr[e];
        if (wc > 0.0) {
            last = 4 * tid + e;
            if (hit == 0x7fffffff && cum + wc > t) { hit = 4 * tid + e; tloc = t - cum; }
            cum += wc;
        }
    }
    if (hit != 0x7fffffff) atomicMin(&s_hit, hit);
    if (last >= 0) atomicMax(&s_last, last);
    __syncthreads();
    // rounding can leave the target at the total: then the last weighted
    // token of the last chunk with weight is drawn
    const bool found = s_hit != 0x7fffffff;
    const int cs = found ? s_hit : max(s_last, 0);
    if (found && hit == cs) s_target = tloc;
    if (!found && tid == 0) s_target = INFINITY;
    if (tid == 0) s_chunk = cs;
    __syncthreads();
    const int c0 = s_chunk * kAcMassChunk, x0 = c0 + 4 * tid;
    double w[4], tsum = 0.0;
    if (!use_p) {
        const double2 *src = reinterpret_cast<const double2 *>(a.w + (size_t)b * a.CM * kAcMassChunk + x0);
        const double2 w01 = src[0], w23 = src[1];
        w[0] = w01.x; w[1] = w01.y; w[2] = w23.x; w[3] = w23.y;
    } else {
        const float *rp = ac_row(a, b, d.row_p);
        const double ip = 1.0 / d.Zp;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const double P = exp(((double)rp[min(x0 + e, a.V - 1)] - (double)d.Mp) / a.tau) * ip;
            w[e] = x0 + e < a.V ? P : 0.0;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; e++) tsum += w[e];
    double ex, ey, tx, ty;
    block_scan2(tsum, 0.0, ex, ey, tx, ty, red);
    if (tid == 0) { s_hit = 0x7fffffff; s_last = -1; }
    __syncthreads();
    const double tt = s_target;
    double cw = ex;
    hit = 0x7fffffff;
    last = -1;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        if (w[e] > 0.0) {
            cw += w[e];
            if (hit == 0x7fffffff && cw > tt) hit = x0 + e;
            last = x0 + e;
        }
    }
    if (hit != 0x7fffffff) atomicMin(&s_hit, hit);
    if (last >= 0) atomicMax(&s_last, last);
    __syncthreads();
    if (tid == 0) a.next[b] = s_hit != 0x7fffffff ? s_hit : s_last;
}

int launch_mtp_accept(int B, int D, int V, const int32_t *draft, const float *p, const float *q, double tau,
                      const double *u, int32_t *n_acc, int32_t *next, void *ws, hipStream_t st)
{
    AcArgs a;
    a.B = B; a.D = D; a.V = V; a.C = mtp_chunks(V); a.CM = mtp_draw_chunks(V);
    a.draft = draft; a.p = p; a.q = q; a.tau = tau; a.u = u; a.n_acc = n_acc; a.next = next;
    unsigned char *w = static_cast<unsigned char *>(ws);
    const MtpWs L = mtp_ws(B, D, V);
    a.stats = reinterpret_cast<AcStat *>(w + L.stats);
    a.dec = reinterpret_cast<AcDec *>(w + L.dec);
    a.mass = reinterpret_cast<double2 *>(w + L.mass);
    a.w = reinterpret_cast<double *>(w + L.w);
    static_assert(sizeof(AcDec) <= 64, "decision size (workspace sizing)");
    const bool vec = V % 4 == 0 && (((uintptr_t)p | (uintptr_t)q) & 15) == 0;
    const dim3 gs(a.C, B * (2 * D + 1)), gm(a.CM, B);
    if (vec) k_ac_stats<true><<<gs, kAcThreads, 0, st>>>(a);
    else k_ac_stats<false><<<gs, kAcThreads, 0, st>>>(a);
    k_ac_decide<<<B, kAcThreads, 0, st>>>(a);
    if (tau > 0.0) {
        if (vec) k_ac_mass<true><<<gm, kAcThreads, 0, st>>>(a);
        else k_ac_mass<false><<<gm, kAcThreads, 0, st>>>(a);
        k_ac_pick<<<B, kAcThreads, 0, st>>>(a);
    }
    return (int)hipGetLastError();
}

} // namespace moe

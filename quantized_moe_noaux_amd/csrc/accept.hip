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
// Three launches over logit rows cut into chunks of kAcChunk tokens:
//  k_ac_stats  per (row, chunk): the chunk's max logit, its first argmax
//              and sum exp((z - max) / tau)
//  k_ac_mass   per (sequence, chunk): the decision (every workgroup derives
//              it from the stats: the drafts' probabilities are
//              exp((z - M) / tau) / Z with M, Z combined over chunks in
//              chunk order), then the chunk's mass of the distribution the
//              emitted token is drawn from (and of p, for a residual
//              without mass)
//  k_ac_pick   per sequence: the decision again, the chunk where the
//              cumulative mass crosses u_D * total (chunk order), and the
//              token inside it (a block scan in token order)
// Greedy needs only the stats and the pick.  Fixed reduction orders: the
// results are run-to-run identical.
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {

constexpr int kAcThreads = 256;
constexpr int kAcPer = 16;                           // tokens per thread per chunk
constexpr int kAcChunk = kAcThreads * kAcPer;        // 4096
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
    double2 *mass;              // [B][C]: (draw mass, target mass)
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

// weight of token x in the draw (residual or target) and its target mass
__device__ __forceinline__ void ac_weights(const AcDecision &d, double tau, float zp, float zq, double &w, double &pw)
{
    const double P = exp(((double)zp - (double)d.np.M) / tau) / d.np.Z;
    pw = P;
    if (d.resid) {
        const double Q = exp(((double)zq - (double)d.nq.M) / tau) / d.nq.Z;
        w = P > Q ? P - Q : 0.0;
    } else {
        w = P;
    }
}

// ---------------------------------------------------------------- chunk masses
template <bool VEC>
__global__ __launch_bounds__(kAcThreads) void k_ac_mass(const AcArgs a)
{
    __shared__ AcDecLds dl;
    __shared__ double sw[kAcThreads / kWave], sp[kAcThreads / kWave];
    const int c = blockIdx.x, b = blockIdx.y;
    const AcDecision d = ac_decide(a, b, dl);
    float zp[kAcPer], zq[kAcPer];
    int pos[kAcPer];
    ac_load<VEC>(ac_row(a, b, d.row_p), a.V, c * kAcChunk, zp, pos);
    if (d.resid) ac_load<VEC>(ac_row(a, b, a.D + 1 + d.j), a.V, c * kAcChunk, zq, pos);
    else {
#pragma unroll
        for (int i = 0; i < kAcPer; i++) zq[i] = zp[i];
    }
    double w = 0.0, pw = 0.0;
#pragma unroll
    for (int i = 0; i < kAcPer; i++) {
        double wi, pi;
        ac_weights(d, a.tau, zp[i], zq[i], wi, pi);
        const bool ok = pos[i] < a.V;
        w += ok ? wi : 0.0;
        pw += ok ? pi : 0.0;
    }
    w = wave_sum_d(w);
    pw = wave_sum_d(pw);
    if (lane_id() == 0) { sw[wave_id()] = w; sp[wave_id()] = pw; }
    __syncthreads();
    if (threadIdx.x == 0)
        a.mass[(size_t)b * a.C + c] = make_double2(((sw[0] + sw[1]) + sw[2]) + sw[3], ((sp[0] + sp[1]) + sp[2]) + sp[3]);
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
// Inside the chosen chunk thread t takes the kAcPer consecutive tokens
// c0 + 16t .. +15 (token order), so an exclusive scan of the threads'
// sums gives every token's cumulative mass.
__global__ __launch_bounds__(kAcThreads) void k_ac_pick(const AcArgs a)
{
    __shared__ AcDecLds dl;
    __shared__ int s_chunk, s_usep, s_hit, s_lastw;
    __shared__ double s_target;
    __shared__ double wsum[2 * kAcThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x;
    const AcDecision d = ac_decide(a, b, dl);
    if (a.tau == 0.0) {
        if (tid == 0) { a.n_acc[b] = d.j; a.next[b] = d.np.arg; }
        return;
    }
    // the chunk the draw falls in: thread c holds chunk c's masses (the
    // draw's and the target's); an exclusive block scan in chunk order gives
    // each chunk's cumulative mass.  A residual without mass falls back to
    // the target itself.
    {
        const double2 mc = a.mass[(size_t)b * a.C + min(tid, a.C - 1)];
        const bool live = tid < a.C;
        double wr = live ? mc.x : 0.0, wp = live ? mc.y : 0.0;
        double er, ep, Wr, Wp;
        block_scan2(wr, wp, er, ep, Wr, Wp, wsum);
        const bool use_p = !(Wr > 0.0);
        const double w = use_p ? wp : wr, e = use_p ? ep : er;
        const double t = a.u[(size_t)b * (a.D + 1) + a.D] * (use_p ? Wp : Wr);
        if (tid == 0) { s_usep = use_p; s_hit = 0x7fffffff; s_lastw = -1; }
        __syncthreads();
        if (w > 0.0) {
            atomicMax(&s_lastw, tid);
            if (e + w > t) atomicMin(&s_hit, tid);
        }
        __syncthreads();
        // rounding can leave the target at the total: then the last
        // weighted token of the last chunk with weight is drawn
        const int cs = s_hit != 0x7fffffff ? s_hit : max(s_lastw, 0);
        if (tid == cs) { s_chunk = cs; s_target = (s_hit != 0x7fffffff) ? t - e : INFINITY; }
        __syncthreads();
        if (tid == 0) { s_hit = 0x7fffffff; s_lastw = -1; }
        __syncthreads();
    }
    AcDecision dd = d;
    if (s_usep) dd.resid = false;
    const int c0 = s_chunk * kAcChunk;
    const float *rp = ac_row(a, b, dd.row_p);
    const float *rq = dd.resid ? ac_row(a, b, a.D + 1 + d.j) : rp;
    double w[kAcPer];
    double tsum = 0.0;
#pragma unroll
    for (int i = 0; i < kAcPer; i++) {
        const int x = c0 + kAcPer * tid + i;
        const int xc = min(x, a.V - 1);
        double wi, pi;
        ac_weights(dd, a.tau, rp[xc], rq[xc], wi, pi);
        w[i] = (x < a.V) ? wi : 0.0;
        tsum += w[i];
    }
    // exclusive scan of the thread sums in thread order (a wave scan, then
    // the four wave totals in order)
    const int l = lane_id(), wv = wave_id();
    double incl = tsum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(incl, o);
        if (l >= o) incl += y;
    }
    if (l == kWave - 1) wsum[wv] = incl;
    __syncthreads();
    double cum = incl - tsum;
    for (int i = 0; i < wv; i++) cum += wsum[i];
    // the answer is the lowest token with weight whose cumulative mass
    // passes the target; the cumulative mass only grows with the token, so
    // each thread's first such token, minimised over threads, is it
    const double t = s_target;
    int hit = 0x7fffffff, lastw = -1;
#pragma unroll
    for (int i = 0; i < kAcPer; i++) {
        if (w[i] > 0.0) {
            const int x = c0 + kAcPer * tid + i;
            cum += w[i];
            if (hit == 0x7fffffff && cum > t) hit = x;
            lastw = x;
        }
    }
    if (hit != 0x7fffffff) atomicMin(&s_hit, hit);
    if (lastw >= 0) atomicMax(&s_lastw, lastw);
    __syncthreads();
    if (tid == 0) {
        a.n_acc[b] = d.j;
        a.next[b] = s_hit != 0x7fffffff ? s_hit : s_lastw;
    }
}

int launch_mtp_accept(int B, int D, int V, const int32_t *draft, const float *p, const float *q, double tau,
                      const double *u, int32_t *n_acc, int32_t *next, void *ws, hipStream_t st)
{
    AcArgs a;
    a.B = B; a.D = D; a.V = V; a.C = (V + kAcChunk - 1) / kAcChunk;
    a.draft = draft; a.p = p; a.q = q; a.tau = tau; a.u = u; a.n_acc = n_acc; a.next = next;
    a.stats = reinterpret_cast<AcStat *>(ws);
    a.mass = reinterpret_cast<double2 *>(static_cast<unsigned char *>(ws) + mtp_stats_bytes(B, D, V));
    const bool vec = V % 4 == 0 && (((uintptr_t)p | (uintptr_t)q) & 15) == 0;
    const dim3 gs(a.C, B * (2 * D + 1)), gm(a.C, B);
    if (vec) k_ac_stats<true><<<gs, kAcThreads, 0, st>>>(a);
    else k_ac_stats<false><<<gs, kAcThreads, 0, st>>>(a);
    if (tau > 0.0) {
        if (vec) k_ac_mass<true><<<gm, kAcThreads, 0, st>>>(a);
        else k_ac_mass<false><<<gm, kAcThreads, 0, st>>>(a);
    }
    k_ac_pick<<<B, kAcThreads, 0, st>>>(a);
    return (int)hipGetLastError();
}

} // namespace moe

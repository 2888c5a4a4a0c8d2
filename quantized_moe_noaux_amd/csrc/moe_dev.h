// Device building blocks shared by the MoE kernels (gfx950, wave64).
//
// Integer dots.  A weight row is consumed in 16-byte "chunks" (one
// global_load_dwordx4 per lane).  A chunk holds 128/wbits codes: 16 int8
// codes (half an activation block), 32 int4 codes (one block) or 64 int2
// codes (two blocks).  A packed code is masked in place into the top bits
// of its byte, where the byte reads as the signed value c * 2^(8-b) (16c for
// int4, 64c for int2: two's complement codes keep their sign there), and
// multiplied against the int8 activations with v_dot4_i32_i8:
//     sum (2^(8-b) c) q = 2^(8-b) * sum c q       (exact in int32).
// The activation bytes are pre-permuted once (v_perm_b32) so that each
// masked nibble / 2-bit field lines up with its activation byte, and the
// power of two is folded into the activation block scale, so d * I comes
// out with the same rounding as without it.  Every block sum is exact in
// int32, as the integer-dot formulation requires (GeekNews #31297,
// implemented features: Q8_0-style int8 activations, integer-dot kernels,
// packed int4 / int2 weights with per-row scales).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Lane exchanges without the LDS crossbar: DPP moves (quad_perm, row
// mirrors) stay inside the VALU, and readlane takes one lane's value into
// scalar registers; a cross-lane permute through the LDS crossbar costs a
// round trip of ~100 cycles per step on MI355X.
template <int CTRL> __device__ __forceinline__ double dpp_d(double v)
{
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_d(double v, int l)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}

// Sum and maximum over the 64 lanes (all lanes active), the same value in
// every lane: pairs inside each row of 16 lanes by DPP (lane ^ 1, lane ^ 2,
// the other quad of 8, the other half of 16; a commutative step leaves both
// partners equal), then the four row results in a fixed order.
__device__ __forceinline__ double wave_sum_d(double v)
{
    v += dpp_d<0xB1>(v);
    v += dpp_d<0x4E>(v);
    v += dpp_d<0x141>(v);
    v += dpp_d<0x140>(v);
    return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

__device__ __forceinline__ double wave_max_d(double v)
{
    v = fmax(v, dpp_d<0xB1>(v));
    v = fmax(v, dpp_d<0x4E>(v));
    v = fmax(v, dpp_d<0x141>(v));
    v = fmax(v, dpp_d<0x140>(v));
    return fmax(fmax(readlane_d(v, 0), readlane_d(v, 16)), fmax(readlane_d(v, 32), readlane_d(v, 48)));
}

// ---------------------------------------------------------------- RMSNorm pieces
// RMSNorm with the sum of squares and the scaling in fp64 and one fixed
// reduction order, shared by the RMSNorm kernel and the router launch that
// normalises its own input, so that both produce the same fp32 values.
// A row of n4 float4s is held by the 256 threads of a block: thread t,
// register j = float4 t + 256 j (zero past the row), so H <= 8192 fits.
constexpr int kNormPer = 8;
// v[j] = (i < n) ? p[i] : 0, without a branch around the load: the load reads
// the clamped index and the value is masked by a multiply.  A load under a
// per-lane condition compiles to an exec-masked load that is waited for at
// once (the other path writes the same registers), so a run of guarded loads
// would cost one memory round trip each; these all stay in flight together.
// (x * 1 is exact; x * 0 = +-0.  Finite inputs.)
__device__ __forceinline__ float4 load4_masked(const float4 *__restrict__ p, int i, int n)
{
    const float4 t = p[i < n ? i : n - 1];
    const float m = (i < n) ? 1.f : 0.f;
    return make_float4(t.x * m, t.y * m, t.z * m, t.w * m);
}
__device__ __forceinline__ void load_row_regs(const float *__restrict__ xr, int n4, float4 (&v)[kNormPer])
{
#pragma unroll
    for (int j = 0; j < kNormPer; j++)
        v[j] = load4_masked(reinterpret_cast<const float4 *>(xr), (int)threadIdx.x + 256 * j, n4);
}
// 1 / sqrt(mean(x^2) + eps) of the row in v; every thread of the 256-thread
// block calls it (one barrier), red = 4 doubles of LDS not in use elsewhere.
__device__ __forceinline__ double row_rstd(const float4 (&v)[kNormPer], int H, double eps, double *red)
{
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kNormPer; j++) {
        ss = fma((double)v[j].x, (double)v[j].x, ss);
        ss = fma((double)v[j].y, (double)v[j].y, ss);
        ss = fma((double)v[j].z, (double)v[j].z, ss);
        ss = fma((double)v[j].w, (double)v[j].w, ss);
    }
    ss = wave_sum_d(ss);
    if (lane_id() == 0) red[wave_id()] = ss;
    __syncthreads();
    return 1.0 / sqrt(((red[0] + red[1]) + (red[2] + red[3])) / H + eps);
}
// x * r * g rounded once to fp32, per component
__device__ __forceinline__ float4 norm4(const float4 &v, double r, const float4 &g)
{
    return make_float4((float)((double)v.x * r * (double)g.x), (float)((double)v.y * r * (double)g.y),
                       (float)((double)v.z * r * (double)g.z), (float)((double)v.w * r * (double)g.w));
}

// ---------------------------------------------------------------- activation chunks
// Activation operand of one weight chunk, held in registers.
template <int WB> struct Act;

// int8 weights: 16 codes = half a block; activations in natural order.
template <> struct Act<8> {
    uint32_t a[4];
    float d;
    __device__ __forceinline__ void load(const int8_t *q, const float *dblk, int chunk)
    {
        uint4 v = *reinterpret_cast<const uint4 *>(q + 16 * chunk);
        a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
        d = dblk[chunk >> 1];
    }
    // two-phase load: issue the loads now, derive the operand later (so that
    // loads issued in between stay in flight)
    __device__ __forceinline__ void load_raw(const int8_t *q, const float *dblk, int chunk) { load(q, dblk, chunk); }
    __device__ __forceinline__ void finish() {}
    // two independent partial sums (exact integer arithmetic: the grouping
    // does not change the result, and short chains keep the issue going)
    __device__ __forceinline__ int isum(const uint4 &w) const
    {
        const int s0 = sdot4(w.y, a[1], sdot4(w.x, a[0], 0));
        const int s1 = sdot4(w.w, a[3], sdot4(w.z, a[2], 0));
        return s0 + s1;
    }
    __device__ __forceinline__ float dot(const uint4 &w) const { return d * (float)isum(w); }
};

// int4 weights: 32 codes = one block.  Per weight dword (8 codes) the even
// codes meet activation bytes {0,2,4,6} and the odd codes {1,3,5,7}.
template <> struct Act<4> {
    uint32_t a[8];
    float d;    // the block's scale
    float d16;  // d / 16: the dot below is 16 * (block sum)
    int qs;     // 128 * (sum of the activation codes met by low nibbles)
    // n: the block's 32 activation codes in natural order
    __device__ __forceinline__ void set(const uint32_t *n, float d_)
    {
        int lo = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a[2 * k] = perm(n[2 * k + 1], n[2 * k], 0x06040200u);
            a[2 * k + 1] = perm(n[2 * k + 1], n[2 * k], 0x07050301u);
            lo = sdot4(a[2 * k], 0x01010101u, lo);
        }
        qs = 128 * lo;
        set_scale(d_);
    }
    __device__ __forceinline__ void set_scale(float d_)
    {
        d = d_;
        d16 = d_ * 0.0625f;
    }
    __device__ __forceinline__ void load(const int8_t *q, const float *dblk, int chunk)
    {
        load_raw(q, dblk, chunk);
        finish();
    }
    __device__ __forceinline__ void load_raw(const int8_t *q, const float *dblk, int chunk)
    {
        const uint4 *p = reinterpret_cast<const uint4 *>(q + 32 * chunk);
        const uint4 v0 = p[0], v1 = p[1];
        a[0] = v0.x; a[1] = v0.y; a[2] = v0.z; a[3] = v0.w;
        a[4] = v1.x; a[5] = v1.y; a[6] = v1.z; a[7] = v1.w;
        d = dblk[chunk];
    }
    __device__ __forceinline__ void finish()
    {
        uint32_t n[8];
#pragma unroll
        for (int i = 0; i < 8; i++) n[i] = a[i];
        set(n, d);
    }
    // 16 * (block sum), in two chains of v_dot4: the high nibbles masked in
    // place (the byte reads 16c), the low nibbles in offset form c + 8 (one
    // AND-XOR), whose offset 8 * sum(q) is removed with the precomputed qs:
    //     16 I = sum 16 c_hi q + 16 * (sum (c_lo + 8) q - 8 sum q_lo)
    __device__ __forceinline__ int isum16(const uint4 &w) const
    {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        int lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            lo = sdot4((ww[k] & 0x0F0F0F0Fu) ^ 0x08080808u, a[2 * k], lo);
            hi = sdot4(ww[k] & 0xF0F0F0F0u, a[2 * k + 1], hi);
        }
        return hi + 16 * lo - qs;
    }
    __device__ __forceinline__ int isum(const uint4 &w) const { return isum16(w) >> 4; }  // exact: a multiple of 16
    // d * I: (d / 16) * (16 I), both factors exact powers-of-two rescalings
    __device__ __forceinline__ float dot(const uint4 &w) const { return d16 * (float)isum16(w); }
};

// int2 weights: 64 codes = two blocks.  Weight dword k holds codes
// 16k + 4j + i at byte j, bits 2i; field i of all four bytes meets the
// activation bytes {i, 4+i, 8+i, 12+i} (a 4x4 byte transpose).
template <> struct Act<2> {
    uint32_t a[16];
    float d0, d1;      // the two blocks' scales
    float d0s, d1s;    // d / 64: the block sums below carry a factor 64
    int qs0, qs1;      // per block, 128 * (sum of the activation codes met by fields 0-2)
    __device__ __forceinline__ void set_scale(float d0_, float d1_)
    {
        d0 = d0_; d1 = d1_;
        d0s = d0_ * 0.015625f; d1s = d1_ * 0.015625f;
    }
    // n: the 64 activation codes in natural order
    __device__ __forceinline__ void set(const uint32_t *n, float d0_, float d1_)
    {
        int c0 = 0, c1 = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            uint32_t q0 = n[4 * k], q1 = n[4 * k + 1], q2 = n[4 * k + 2], q3 = n[4 * k + 3];
            uint32_t lo01 = perm(q1, q0, 0x05010400u), lo23 = perm(q3, q2, 0x05010400u);
            uint32_t hi01 = perm(q1, q0, 0x07030602u), hi23 = perm(q3, q2, 0x07030602u);
            a[4 * k + 0] = perm(lo23, lo01, 0x05040100u);
            a[4 * k + 1] = perm(lo23, lo01, 0x07060302u);
            a[4 * k + 2] = perm(hi23, hi01, 0x05040100u);
            a[4 * k + 3] = perm(hi23, hi01, 0x07060302u);
        }
        // fields 0-2 meet bytes 0-2 of every natural-order activation dword
#pragma unroll
        for (int i = 0; i < 8; i++) {
            c0 = sdot4(n[i], 0x00010101u, c0);
            c1 = sdot4(n[8 + i], 0x00010101u, c1);
        }
        qs0 = 128 * c0; qs1 = 128 * c1;
        set_scale(d0_, d1_);
    }
    __device__ __forceinline__ void load(const int8_t *q, const float *dblk, int chunk)
    {
        load_raw(q, dblk, chunk);
        finish();
    }
    __device__ __forceinline__ void load_raw(const int8_t *q, const float *dblk, int chunk)
    {
        const uint4 *p = reinterpret_cast<const uint4 *>(q + 64 * chunk);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint4 v = p[i];
            a[4 * i] = v.x; a[4 * i + 1] = v.y; a[4 * i + 2] = v.z; a[4 * i + 3] = v.w;
        }
        d0 = dblk[2 * chunk];
        d1 = dblk[2 * chunk + 1];
    }
    __device__ __forceinline__ void finish()
    {
        uint32_t n[16];
#pragma unroll
        for (int i = 0; i < 16; i++) n[i] = a[i];
        set(n, d0, d1);
    }
    // 64 * (sum over one block = weight dwords k, k+1).  Fields 0-2 are
    // XORed into offset form c + 2 in [0, 3] and masked in place, so their
    // bytes read c + 2, 4(c + 2), 16(c + 2); field 3 stays two's complement
    // in the top bits (64c).  One v_dot4 chain per field, combined as
    //     64 S = 64 S0 + 16 S1 + 4 S2 + S3 - 128 * (activations of fields 0-2)
    // with the offset term (qs) entering at the head of the field-3 chain.
    __device__ __forceinline__ int block64(uint32_t w0, uint32_t w1, int k, int qs) const
    {
        const uint32_t x0 = w0 ^ 0x2A2A2A2Au, x1 = w1 ^ 0x2A2A2A2Au;
        const int s0 = sdot4(x1 & 0x03030303u, a[4 * k + 4], sdot4(x0 & 0x03030303u, a[4 * k], 0));
        const int s1 = sdot4(x1 & 0x0C0C0C0Cu, a[4 * k + 5], sdot4(x0 & 0x0C0C0C0Cu, a[4 * k + 1], 0));
        const int s2 = sdot4(x1 & 0x30303030u, a[4 * k + 6], sdot4(x0 & 0x30303030u, a[4 * k + 2], 0));
        const int s3 = sdot4(w1 & 0xC0C0C0C0u, a[4 * k + 7], sdot4(w0 & 0xC0C0C0C0u, a[4 * k + 3], -qs));
        return ((s0 * 4 + s1) * 4 + s2) * 4 + s3;
    }
    __device__ __forceinline__ void isum2_64(const uint4 &w, int &i0, int &i1) const
    {
        i0 = block64(w.x, w.y, 0, qs0);
        i1 = block64(w.z, w.w, 2, qs1);
    }
    __device__ __forceinline__ void isum2(const uint4 &w, int &i0, int &i1) const
    {
        isum2_64(w, i0, i1);
        i0 >>= 6;  // exact: multiples of 64
        i1 >>= 6;
    }
    __device__ __forceinline__ float dot(const uint4 &w) const
    {
        int i0, i1;
        isum2_64(w, i0, i1);
        return d0s * (float)i0 + d1s * (float)i1;
    }
};

// ---------------------------------------------------------------- quantiser
// Q8_0-style block quantiser spread over 8 consecutive lanes, 4 elements
// per lane (lanes 8j..8j+7 of a wave hold one block of 32).  d = amax/127
// and q = rint(x/d) use IEEE fp32 division and round-half-even (the build
// keeps -fno-fast-math, so '/' is the correctly rounded division and rintf
// is v_rndne_f32).  Returns the 4 codes packed in a dword; the block's d
// comes back in every lane of the 8.
__device__ __forceinline__ uint32_t quant_block8(float4 v, float &d_out)
{
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    float d = amax / 127.0f;
    float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        float r = (d == 0.0f) ? 0.0f : rintf(e[j] / d);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        packed |= ((uint32_t)((int)r & 0xFF)) << (8 * j);
    }
    d_out = d;
    return packed;
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

} // namespace moe

// Row-wise softmax for gfx950, the tutorial's fused softmax ("Designing High-Performance
// GPU Kernels with TileLang: ...", ainovat.com page, third paragraph: a row-wise softmax
// built on maximum and sum reductions over each row, normalising in registers).
//
// y[i][j] = exp(x[i][j] - m_i) / sum_j exp(x[i][j] - m_i),  m_i = max_j x[i][j],
// x and y M x N fp16 row-major, arithmetic in fp32, one rounding to fp16 at the store.
// HBM-bound: 4 bytes move per element.
//
// Dispatch (measured crossovers): softmax_rows up to 2048 elements per row, softmax_wg with
// 4 wavefronts per row up to 16384 and with 16 up to 65536, softmax_long beyond.
//
// softmax_rows<VPL> (N <= 512 * VPL): one wavefront per row, the row held in registers as
//   fp16 (VPL 16-byte vectors per lane, vector c = lane + 64 k covering elements
//   8c .. 8c+7, so every load and store instruction of a wave touches one contiguous
//   span).  Max and sum are reduced across the wave with cross-lane shuffles; exp is
//   evaluated twice per element (for the sum and for the output) rather than holding
//   fp32 copies, which keeps the register footprint at VPL * 4.
// softmax_wg<VPL, NT> (N <= 8 * NT * VPL): one NT-thread workgroup per row, the row held
//   in the registers of its NT / 64 wavefronts (VPL 16-byte vectors per lane, vector
//   c = thread + NT k), maximum and sum reduced across each wave by shuffles and across
//   the waves through LDS: still one read and one write per element, with more loads in
//   flight per row than one wavefront can hold.
// softmax_long (any N): one 1024-thread workgroup per row, two passes over the row: an
//   online running (max, sum) per thread -- when a larger value arrives the sum so far is
//   rescaled by exp(old max - new max) -- combined across the workgroup, then a pass that
//   writes exp(x - m) / s.
//
// Rows start at any 2-byte alignment (N % 8 != 0): 16-byte vectors wholly inside the row
// move as one (unaligned) access; the row's last, partial vector is read and written one
// element at a time so neighbouring rows are never touched.  IEEE rules give the edge
// cases, as in the plain definition: a NaN or +inf entry, or a row of -inf, makes the
// row NaN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef _Float16 sf16;
typedef sf16 sf16x8 __attribute__((ext_vector_type(8)));
typedef sf16 sf16x8u __attribute__((ext_vector_type(8), aligned(2)));   // unaligned view

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_f32(float t)
{
    return __builtin_amdgcn_exp2f(t * kLog2e);   // v_exp_f32; exp(-inf) = 0, exp(NaN) = NaN
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

constexpr int kSoftmaxThreads = 256;       // 4 rows per workgroup in softmax_rows
constexpr int kSoftmaxLongThreads = 1024;  // one row per workgroup in softmax_long
constexpr int kSoftmaxWgThreads = 1024;    // default workgroup of softmax_wg

template <int VPL>
__global__ void __launch_bounds__(kSoftmaxThreads)
softmax_rows(const sf16 *x, sf16 *y, int64_t M, int N)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kSoftmaxThreads / 64) + (threadIdx.x >> 6);
    if (row >= M) return;   // the whole wavefront leaves together
    const sf16 *xr = x + row * (int64_t)N;
    sf16 *yr = y + row * (int64_t)N;
    const sf16 ninf = (sf16)(-__builtin_inff());

    sf16x8 v[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int e0 = 8 * (lane + 64 * k);
        if (e0 + 8 <= N) {
            v[k] = *reinterpret_cast<const sf16x8u *>(xr + e0);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[k][i] = (e0 + i < N) ? xr[e0 + i] : ninf;
        }
    }
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, (float)v[k][i]);
    m = wave_max(m);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) s += exp_f32((float)v[k][i] - m);
    s = wave_sum(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int e0 = 8 * (lane + 64 * k);
        sf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (sf16)(exp_f32((float)v[k][i] - m) * inv);
        if (e0 + 8 <= N) {
            *reinterpret_cast<sf16x8u *>(yr + e0) = o;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (e0 + i < N) yr[e0 + i] = o[i];
        }
    }
}

template <int VPL, int NT = kSoftmaxWgThreads>
__global__ void __launch_bounds__(NT)
softmax_wg(const sf16 *x, sf16 *y, int N)
{
    constexpr int NWV = NT / 64;
    __shared__ float red[NWV];
    const int64_t row = blockIdx.x;
    const sf16 *xr = x + row * (int64_t)N;
    sf16 *yr = y + row * (int64_t)N;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const sf16 ninf = (sf16)(-__builtin_inff());

    sf16x8 v[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int e0 = 8 * (t + NT * k);
        if (e0 + 8 <= N) {
            v[k] = *reinterpret_cast<const sf16x8u *>(xr + e0);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[k][i] = (e0 + i < N) ? xr[e0 + i] : ninf;
        }
    }
    // the workgroup's maximum, then its sum: per wave by shuffles, across waves in LDS
    auto wg_reduce = [&](float a, bool is_max) {
        a = is_max ? wave_max(a) : wave_sum(a);
        if (lane == 0) red[wv] = a;
        __syncthreads();
        float r = red[0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
        __syncthreads();   // red is reused by the next reduction
        return r;
    };
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, (float)v[k][i]);
    m = wg_reduce(m, true);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) s += exp_f32((float)v[k][i] - m);
    s = wg_reduce(s, false);
    const float inv = 1.0f / s;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int e0 = 8 * (t + NT * k);
        sf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (sf16)(exp_f32((float)v[k][i] - m) * inv);
        if (e0 + 8 <= N) {
            *reinterpret_cast<sf16x8u *>(yr + e0) = o;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (e0 + i < N) yr[e0 + i] = o[i];
        }
    }
}

// (m1, s1) and (m2, s2) are running maxima and sums of exp(x - m); a part whose maximum
// is -inf holds no finite entry and adds nothing.
__device__ __forceinline__ void combine(float &m, float &s, float m2, float s2)
{
    const float mm = fmaxf(m, m2);
    const float a = (m == -__builtin_inff()) ? 0.0f : s * exp_f32(m - mm);
    const float b = (m2 == -__builtin_inff()) ? 0.0f : s2 * exp_f32(m2 - mm);
    m = mm;
    s = a + b;
}

__global__ void __launch_bounds__(kSoftmaxLongThreads)
softmax_long(const sf16 *x, sf16 *y, int N)
{
    constexpr int NT = kSoftmaxLongThreads, NWV = NT / 64, U = 4;
    __shared__ float red_m[NWV], red_s[NWV];
    __shared__ float row_m, row_s;
    const int64_t row = blockIdx.x;
    const sf16 *xr = x + row * (int64_t)N;
    sf16 *yr = y + row * (int64_t)N;
    const int t = threadIdx.x;
    const int nv = N / 8;   // whole vectors; elements 8*nv .. N-1 one by one
    const sf16x8u *xv = reinterpret_cast<const sf16x8u *>(xr);
    sf16x8u *yv = reinterpret_cast<sf16x8u *>(yr);

    float m = -__builtin_inff(), s = 0.0f;
    bool bad = false;   // a NaN or +inf entry makes the whole row NaN
    auto take = [&](float xe) {
        if (!(xe < __builtin_inff())) { bad = true; return; }   // NaN or +inf
        if (xe > m) {
            s = (m == -__builtin_inff()) ? 1.0f : s * exp_f32(m - xe) + 1.0f;
            m = xe;
        } else if (xe != -__builtin_inff()) {
            s += exp_f32(xe - m);
        }
    };
    int c = t;
    for (; c + (U - 1) * NT < nv; c += U * NT) {   // U independent 16-byte loads in flight
        sf16x8 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = xv[c + u * NT];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) take((float)v[u][i]);
    }
    for (; c < nv; c += NT) {
        const sf16x8 v = xv[c];
#pragma unroll
        for (int i = 0; i < 8; ++i) take((float)v[i]);
    }
    for (int e = 8 * nv + t; e < N; e += NT) take((float)xr[e]);

#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        combine(m, s, m2, s2);
    }
    const int any_bad = __syncthreads_or(bad ? 1 : 0);
    if ((t & 63) == 0) {
        red_m[t >> 6] = m;
        red_s[t >> 6] = s;
    }
    __syncthreads();
    if (t == 0) {
        float mm = red_m[0], ss = red_s[0];
        for (int w = 1; w < NWV; ++w) combine(mm, ss, red_m[w], red_s[w]);
        row_m = mm;
        // a row without a finite maximum (all -inf) or with a NaN / +inf entry is NaN
        row_s = (any_bad || mm == -__builtin_inff()) ? __builtin_nanf("") : ss;
    }
    __syncthreads();
    m = row_m;
    const float inv = 1.0f / row_s;
    c = t;
    for (; c + (U - 1) * NT < nv; c += U * NT) {
        sf16x8 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = xv[c + u * NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            sf16x8 o;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (sf16)(exp_f32((float)v[u][i] - m) * inv);
            yv[c + u * NT] = o;
        }
    }
    for (; c < nv; c += NT) {
        const sf16x8 v = xv[c];
        sf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (sf16)(exp_f32((float)v[i] - m) * inv);
        yv[c] = o;
    }
    for (int e = 8 * nv + t; e < N; e += NT) yr[e] = (sf16)(exp_f32((float)xr[e] - m) * inv);
}

}  // namespace mi355

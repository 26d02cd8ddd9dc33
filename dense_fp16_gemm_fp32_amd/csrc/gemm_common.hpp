// Pieces shared by the gfx950 GEMM kernels: types, kernel arguments, buffer descriptors,
// the tile order, and the register epilogue (bias, erf-GELU, fp16 rounding, masked store).
//
// The operation is C (M x N) = epi(A (M x K) . B (K x N) [+ bias]), all fp16 row-major with
// fp32 accumulation, as stated by "Designing High-Performance GPU Kernels with TileLang:
// Tensor-Core GEMM, Fused Softmax, FlashAttention, and Autotuning" (thecryptopost.io page,
// section 2, make_matmul), with the epilogue of the same tutorial's fused-epilogue
// paragraph (ainovat.com page): bias and GELU applied to the accumulator in registers,
// then one write of C.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A buffer offset no descriptor here ever covers (every num_records is below 2^31): a
// load from it returns zeros and a store to it is discarded by the hardware range check.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

// Valid offsets stay below 2^31, so setting bit 31 turns an offset into an out-of-range
// one without a branch.
__device__ __forceinline__ uint32_t masked_offset(uint32_t off, bool valid)
{
    return off | ((uint32_t)!valid << 31);
}

struct GemmArgs {
    const f16 *A;
    const f16 *B;
    f16 *C;
    const f16 *bias;
    int M, N, K;      // N: the columns this launch computes (of B, C and bias)
    int ldb, ldc;     // row strides of B and C in elements (>= N); A's is K
    int tiles_m, tiles_n;
    int group_m;
};

// Bytes a buffer descriptor must cover for `rows` rows of `width` elements each, rows
// `ld` elements apart, starting at the descriptor's base: up to the last element of the
// last row and not beyond it (so the descriptor never reaches past the operand).
__device__ __forceinline__ uint32_t span_bytes(int rows, int ld, int width)
{
    return rows > 0 ? (uint32_t)((rows - 1) * ld + width) * 2u : 0u;
}

// ---------------------------------------------------------------- tile order --------
// Workgroups are handed to the 8 XCDs round-robin (id % 8).  Renumber them so each XCD
// owns one contiguous range of the logical order; the logical order sweeps GROUP_M
// tile-rows column by column, so tiles resident at the same time share A row-panels and
// B column-panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m,
                                            int &tm, int &tn)
{
    const int total = tiles_m * tiles_n;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx
                                : rem * (per + 1) + (xcd - rem) * per + idx;
    const int width = group_m * tiles_n;
    const int g = lid / width;
    const int first_m = g * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int r = lid - g * width;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// ---------------------------------------------------------------- epilogue ----------
// GELU(x) = x * Phi(x) with Phi the standard normal CDF.  With h = Phi(-|x|), Phi(x) is
// 1 - h for x >= 0 and h for x < 0, so
//   GELU(x) = max(x, 0) - |x| h
// for both signs: no cancellation on the negative side and no select.  h = 2^P(|x|) with
// P a degree-7 polynomial fitted to log2 Phi(-z) on [0, 6] (least squares on Chebyshev
// nodes; gelu_poly.py derives the coefficients).  In fp32 Horner form P is within 8e-6 of
// log2 Phi(-z) there, so h is within 6e-6 relative, far below the 2^-11 relative step of
// the fp16 result.  The leading coefficient is negative and P falls from -29.9 at z = 6
// on, so for x <= -6 the result |x| h rounds to zero in fp16 as x Phi(x) does; Horner's
// rule overflows to -inf for large z, and 2^-inf is 0.  One transcendental (the hardware
// v_exp_f32) and no reciprocal.
__device__ __forceinline__ float gelu_erf(float x)
{
    constexpr float c0 = -9.999943376e-01f, c1 = -1.151269197e+00f, c2 = -4.584097862e-01f,
                    c3 = -5.402068794e-02f, c4 = 8.539461531e-03f, c5 = -9.388679173e-04f,
                    c6 = 6.268139987e-05f, c7 = -1.889626219e-06f;
    const float z = fabsf(x);
    float q = fmaf(c7, z, c6);
    q = fmaf(q, z, c5);
    q = fmaf(q, z, c4);
    q = fmaf(q, z, c3);
    q = fmaf(q, z, c2);
    q = fmaf(q, z, c1);
    q = fmaf(q, z, c0);
    const float h = __builtin_amdgcn_exp2f(q);                  // Phi(-|x|)
    // the multiplier |x| is capped at the largest finite float for x = +inf: h is 0 there,
    // and the result is inf - 3.4e38 * 0 = inf (uncapped, inf * 0 = NaN).  x = -inf keeps
    // |x| = inf, so -inf * 0 = NaN, as x * Phi(x) evaluates in IEEE arithmetic; a NaN x
    // reaches the result through h; finite x are unchanged.
    const float ax = fabsf(fminf(x, 3.4028234663852886e38f));
    return fmaf(-ax, h, fmaxf(x, 0.0f));
}

template <int EPI>
__device__ __forceinline__ float epilogue_op(float acc, float b)
{
    if constexpr (EPI == 0) {
        return acc;
    } else if constexpr (EPI == 1) {
        return acc + b;
    } else {
        return gelu_erf(acc + b);
    }
}

// Accumulator layout of v_mfma_f32_32x32x16_f16 with the B fragment as the first operand
// and the A fragment as the second: register r of lane l holds
// C[m = l % 32][n = 8*(r / 4) + 4*(l / 32) + r % 4] of its 32x32 block, so each lane owns
// four consecutive columns per register quad and writes them as one 8-byte store.
//
// Stores block rows I0 <= i < I1 of the FM x FN blocks of one wavefront whose sub-tile
// starts at (row0, col0) inside the workgroup tile at (m0, n0).  Rows >= M are dropped by the C descriptor's range,
// columns >= N by an explicit mask.
// tile_rows = min(BM, M - m0) (at most 256, so tile_rows * N stays below 2^30).
template <int FM, int FN, int I0, int I1, bool BV, int EPI>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[FM][FN], const GemmArgs &p,
                                           int m0, int n0, int tile_rows, int row0, int col0,
                                           int lane)
{
    const int cols_valid = p.N - n0;
    // C covers rows [m0, m0 + tile_rows), columns [n0, N)
    const __amdgpu_buffer_rsrc_t c_rs =
        make_rsrc(p.C + (int64_t)m0 * p.ldc + n0, span_bytes(tile_rows, p.ldc, cols_valid));
    // bias covers columns [n0, N); with no epilogue it is never read
    const __amdgpu_buffer_rsrc_t b_rs =
        make_rsrc(EPI != 0 ? p.bias + n0 : p.C, EPI != 0 ? (uint32_t)cols_valid * 2u : 0u);

    const int frag_row = lane & 31;
    const int lane_n = 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = col0 + j * 32 + 8 * g + lane_n;   // relative to n0
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI != 0) {
                if constexpr (BV) {
                    const u32x2 raw = __builtin_amdgcn_raw_buffer_load_b64(b_rs, (uint32_t)n * 2u, 0, 0);
                    const f16x4 h = __builtin_bit_cast(f16x4, raw);
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[e] = (float)h[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint16_t raw =
                            __builtin_amdgcn_raw_buffer_load_b16(b_rs, (uint32_t)(n + e) * 2u, 0, 0);
                        bv[e] = (float)__builtin_bit_cast(f16, raw);
                    }
                }
            }
#pragma unroll
            for (int i = I0; i < I1; ++i) {
                const int m = row0 + i * 32 + frag_row;     // relative to m0
                // fp32 -> fp16 with round-to-nearest-even, kept as raw bit patterns
                uint32_t hb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f16 h = (f16)epilogue_op<EPI>(acc[i][j][4 * g + e], bv[e]);
                    hb[e] = __builtin_bit_cast(uint16_t, h);
                }
                if constexpr (BV) {
                    const uint32_t off = masked_offset((uint32_t)(m * p.ldc + n) * 2u, n < cols_valid);
                    const u32x2 packed = {hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
                    __builtin_amdgcn_raw_buffer_store_b64(packed, c_rs, off, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t off =
                            masked_offset((uint32_t)(m * p.ldc + n + e) * 2u, n + e < cols_valid);
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hb[e], c_rs, off, 0, 0);
                    }
                }
            }
        }
    }
}

}  // namespace mi355

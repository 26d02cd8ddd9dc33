// Narrow GEMM for gfx950: C (M x W) = epi(A (M x K) . B (K x W) [+ bias]) with W <= 8
// columns, fp16 operands, fp32 accumulation -- the same operation as the tiled kernels
// (thecryptopost.io page, section 2, make_matmul; the fused epilogue of the ainovat.com
// page), for problems with at most 8 columns and for the last N % 8 columns of a problem
// whose B and C rows are not 16-byte friendly (the direct kernel takes the columns before
// them).  B and C rows are ldb / ldc elements apart, at any 2-byte alignment.
//
// With at most 8 columns the product is no tile contraction: its cost is reading A once
// (2 bytes per multiply-add pair of the 8 columns), so it runs on the vector ALUs:
//   * a workgroup of 4 waves: KS waves split K for each group of 8 rows of C, so a
//     workgroup covers 8 * 4 / KS rows.  With KS = 4 (8 rows, for long K and few rows)
//     wave w takes the 512-wide k-blocks w, w + 4, ...; with KS = 1 (32 rows, for many
//     rows) every wave runs all of K for its own 8 rows, the four reading the same B
//     pieces close together in time, which the CU's L1 then serves.  Lane l takes the 8
//     consecutive k at 8 l inside a block;
//   * per block a lane reads 16 bytes of each of the 8 A rows and the 16 bytes at
//     columns 0..7 of each of its 8 B rows (16-byte accesses at any 2-byte alignment;
//     the columns past W belong to the next row and only feed outputs that are never
//     stored), and accumulates 8 x 8 x 8 fp32 multiply-adds of the converted values;
//   * the 64 partial sums per lane (8 rows x 8 columns) are folded across the 64 lanes in
//     six exchange steps, after which lane l holds output l's sum over the wave's k; the
//     KS waves' sums of a row group are added through LDS in a fixed order, and the
//     epilogue and the fp16 store follow, one output per lane.
// The last values of K are read element by element and added once per output at the end,
// so no access reaches past an operand's last element.
#pragma once

#include "gemm_common.hpp"

namespace mi355 {

typedef f16 f16x8u __attribute__((ext_vector_type(8), aligned(2)));   // unaligned view

template <int KS_>
struct Narrow {
    static constexpr int RW = 8;         // rows of C per wave
    static constexpr int NC = 8;         // columns computed (W <= NC are stored)
    static constexpr int NW = 4;         // waves per workgroup
    static constexpr int KS = KS_;       // waves splitting K for one row group
    static constexpr int RG = NW / KS;   // row groups per workgroup
    static constexpr int BM = RW * RG;   // rows of C per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int KB = 64 * 8;    // k per block
    static constexpr int TAIL = 16;      // tail values of K read element by element (<= 14 used)
    static_assert(NW % KS == 0, "waves split evenly into row groups");
};

// Step S of the fold: v[0, 2S) holds partial sums of 2S outputs; afterwards v[0, S) holds
// the S outputs selected by lane bit S, summed over this lane and its partner l ^ S.
template <int S>
__device__ __forceinline__ void fold_step(float (&v)[64], int lane)
{
    const bool hi = (lane & S) != 0;
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const float keep = hi ? v[S + i] : v[i];
        const float give = hi ? v[i] : v[S + i];
        v[i] = keep + __shfl_xor(give, S, 64);
    }
}

template <int EPI, int KS>
__global__ void __launch_bounds__(Narrow<KS>::NT) gemm_narrow(GemmArgs p)
{
    using T = Narrow<KS>;
    __shared__ float part[T::NW][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kg = wave % KS;            // k-group inside the row group
    const int m0 = blockIdx.x * T::BM + (wave / KS) * T::RW;   // this wave's first row
    const int rows_valid = min(T::RW, p.M - m0);               // may be <= 0: no rows
    const int K = p.K, W = p.N, ldb = p.ldb;
    // A rows [m0, m0 + rows_valid) (rows past them read zeros; their outputs are dropped)
    const __amdgpu_buffer_rsrc_t a_rs =
        make_rsrc(p.A + (int64_t)m0 * K, (uint32_t)(max(rows_valid, 0) * K) * 2u);
    // The 16-byte piece of B row kr (columns 0..7) stays inside B while
    // kr * ldb + 8 <= (K - 1) * ldb + W, which fails for the last R = ceil((8 - W) / ldb)
    // rows when W < 8 (R = 1 once rows are 8 or more elements apart).  The main loop takes
    // k < K1 in whole 8-element chunks, K1 the largest multiple of 8 with K1 <= K - R;
    // the last K - K1 <= 7 + R <= 14 values of K form the tail.
    const int R = W >= 8 ? 0 : (8 - W + ldb - 1) / ldb;
    const int K1 = K > R ? (K - R) & ~7 : 0;

    // Tail k in [K1, K): k-group 0's lane l, which ends up holding output (r, j) = (l / 8,
    // l % 8), reads the A values of row r and the B values of column j there now
    // (element loads through descriptors whose range ends at the last element; offsets
    // past K or past W are pushed out of range and read zero) and adds their products
    // to its sum at the end.
    const int tr = lane / T::NC, tj = lane % T::NC;
    float ta[T::TAIL], tb[T::TAIL];
    if (kg == 0) {
        const __amdgpu_buffer_rsrc_t bt_rs =
            make_rsrc(p.B + (int64_t)K1 * ldb, K > 0 ? span_bytes(K - K1, ldb, W) : 0u);
#pragma unroll
        for (int e = 0; e < T::TAIL; ++e) {
            const bool in_k = K1 + e < K;
            ta[e] = (float)__builtin_bit_cast(f16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                a_rs, masked_offset((uint32_t)(tr * K + K1 + e) * 2u, in_k), 0, 0));
            tb[e] = (float)__builtin_bit_cast(f16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                bt_rs, masked_offset((uint32_t)(e * ldb + tj) * 2u, in_k && tj < W), 0, 0));
        }
    }

    float acc[T::RW][T::NC];
#pragma unroll
    for (int r = 0; r < T::RW; ++r)
#pragma unroll
        for (int j = 0; j < T::NC; ++j) acc[r][j] = 0.0f;

    // No branch depends on the lane here, so each block's 16 loads are in flight together.
    for (int kb = kg * T::KB; kb < K1; kb += KS * T::KB) {
        const int k = kb + 8 * lane;
        const bool valid = k < K1;
        u32x4 a[T::RW];
#pragma unroll
        for (int r = 0; r < T::RW; ++r)
            a[r] = __builtin_amdgcn_raw_buffer_load_b128(
                a_rs, masked_offset((uint32_t)(r * K + k) * 2u, valid), 0, 0);
        // a chunk past K1 reads rows 0..7 of B instead (all below K1 - R here) and zeros them
        const f16 *brow = p.B + (int64_t)(valid ? k : 0) * ldb;
        u32x4 b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const u32x4 t = __builtin_bit_cast(u32x4, *reinterpret_cast<const f16x8u *>(brow + (int64_t)e * ldb));
            b[e] = valid ? t : u32x4{0u, 0u, 0u, 0u};
        }
        // fp32 multiply-adds of the converted fp16 values, k by k
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const f16x8 bv = __builtin_bit_cast(f16x8, b[e]);
#pragma unroll
            for (int r = 0; r < T::RW; ++r) {
                const float av = (float)__builtin_bit_cast(f16x8, a[r])[e];
#pragma unroll
                for (int j = 0; j < T::NC; ++j) acc[r][j] = fmaf(av, (float)bv[j], acc[r][j]);
            }
        }
    }

    // output index o = 8 r + j; after the fold lane l holds output l
    float v[64];
#pragma unroll
    for (int r = 0; r < T::RW; ++r)
#pragma unroll
        for (int j = 0; j < T::NC; ++j) v[T::NC * r + j] = acc[r][j];
    fold_step<32>(v, lane);
    fold_step<16>(v, lane);
    fold_step<8>(v, lane);
    fold_step<4>(v, lane);
    fold_step<2>(v, lane);
    fold_step<1>(v, lane);
    float s = v[0];
    if constexpr (KS > 1) {
        part[wave][lane] = s;
        __syncthreads();
        if (kg != 0) return;
#pragma unroll
        for (int w = 1; w < KS; ++w) s += part[wave + w][lane];
    }
#pragma unroll
    for (int e = 0; e < T::TAIL; ++e) s = fmaf(ta[e], tb[e], s);

    const int r = tr, j = tj;
    const bool ok = r < rows_valid && j < W;
    float bias = 0.0f;
    if constexpr (EPI != 0) {
        const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(p.bias, (uint32_t)W * 2u);
        bias = (float)__builtin_bit_cast(
            f16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(b_rs, masked_offset((uint32_t)j * 2u, ok), 0, 0));
    }
    const f16 h = (f16)epilogue_op<EPI>(s, bias);
    const __amdgpu_buffer_rsrc_t c_rs =
        make_rsrc(p.C + (int64_t)m0 * p.ldc, span_bytes(rows_valid, p.ldc, W));
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), c_rs,
                                          masked_offset((uint32_t)(r * p.ldc + j) * 2u, ok), 0, 0);
}

}  // namespace mi355

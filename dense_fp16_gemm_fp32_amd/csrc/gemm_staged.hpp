// Register-staged GEMM kernel for gfx950: serves every alignment (2-byte loads where a
// row is not 16-byte aligned); the selector uses it for ragged and unaligned problems.
//
// One workgroup computes one BM x BN macro-tile of C:
//   1. tile order  -- tile_coords();
//   2. loader      -- buffer loads HBM -> VGPR (16-byte vectors; for A also at 2-byte
//                     alignment, with 2-byte loads only in the stage holding the K tail; for
//                     B 2-byte loads when its rows are not 16-byte aligned; out-of-range
//                     lanes read 0 through the buffer descriptor's range check), then
//                     VGPR -> LDS into a 2-stage padded
//                     ring; B is transposed 4x8 in registers on the way so both LDS tiles
//                     are k-contiguous, as the MFMA operands want;
//   3. MFMA loop   -- each wavefront owns a WTM x WTN sub-tile of 32x32 blocks and chains
//                     v_mfma_f32_32x32x16_f16 into fp32 accumulators;
//   4. epilogue    -- store_tile(): bias, GELU, fp16 rounding, masked stores.
#pragma once

#include "gemm_common.hpp"

namespace mi355 {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;   // wavefront sub-tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;             // 32x32 MFMA blocks
    static constexpr int PITCH = BK + 8;     // halves per LDS row: 16 B of padding
    static constexpr int STAGES = 2;
    static constexpr int A_STAGE = BM * PITCH, B_STAGE = BN * PITCH;   // halves
    static constexpr int LDS_BYTES = STAGES * (A_STAGE + B_STAGE) * 2;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 16 == 0, "K step must be whole MFMA k-blocks");
    static_assert(LDS_BYTES <= 160 * 1024, "over the gfx950 LDS budget");
};

// ---------------------------------------------------------------- loader ----------
// A tile: BM rows x BK halves, stored in LDS as [row][k] (k contiguous).
template <class T, bool VEC>
struct ALoader {
    static constexpr int VPR = T::BK / 8;              // 8-half vectors per row
    static constexpr int PER = T::BM * VPR / T::NT;    // vectors per thread
    static_assert(T::BM * VPR % T::NT == 0, "A tile must split evenly over threads");
    u32x4 r[PER];

    // rs covers rows [m0, m0 + rows_valid) of A from column 0; rows past it read 0.
    // VEC: K % 8 == 0 and A 16-byte aligned, every 8-half chunk is one aligned 16-byte
    // load.  Otherwise rows are only 2-byte aligned: a chunk that lies wholly inside its
    // row is still one 16-byte load (gfx9 buffer loads need no alignment beyond the
    // element size here; the compiler emits the same for unaligned vector loads), and only
    // the stage holding the K tail, whose last chunk of a row may reach past the row (and
    // past the end of A), falls back to one 2-byte load per element.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int k0, int K, int tid)
    {
        if constexpr (!VEC) {
            if (k0 + T::BK <= K) {
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int v = tid + i * T::NT;
                    const int row = v / VPR, k = k0 + 8 * (v % VPR);
                    r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(row * K + k) * 2u, 0, 0);
                }
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = tid + i * T::NT;
            const int row = v / VPR, k = k0 + 8 * (v % VPR);
            if constexpr (VEC) {
                const uint32_t off = masked_offset((uint32_t)(row * K + k) * 2u, k < K);
                r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            } else {
                uint32_t w[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int ka = k + 2 * s, kb = ka + 1;
                    const uint32_t oa = masked_offset((uint32_t)(row * K + ka) * 2u, ka < K);
                    const uint32_t ob = masked_offset((uint32_t)(row * K + kb) * 2u, kb < K);
                    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, oa, 0, 0);
                    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, ob, 0, 0);
                    w[s] = lo | (hi << 16);
                }
                r[i] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }

    __device__ __forceinline__ void store(f16 *as, int tid) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = tid + i * T::NT;
            *reinterpret_cast<u32x4 *>(as + (v / VPR) * T::PITCH + 8 * (v % VPR)) = r[i];
        }
    }
};

// B tile: BK rows x BN halves in HBM (n contiguous); stored in LDS as [n][k] (k
// contiguous).  Each thread moves 4(k) x 8(n) blocks: four 16-byte row loads, a 4x8
// transpose in registers, eight 8-byte LDS writes.  Consecutive lanes take consecutive
// k-quads so one write instruction from 16 lanes fills one contiguous 128-byte LDS span.
template <class T, bool VEC>
struct BLoader {
    static constexpr int Q = T::BK / 4;      // k-quads
    static constexpr int CN = T::BN / 8;     // 8-column chunks
    static constexpr int PER = Q * CN / T::NT;
    static_assert(Q * CN % T::NT == 0, "B tile must split evenly over threads");
    u32x4 r[PER][4];

    // Loads rows [k0, k0 + BK) x columns [n0, n0 + BN) of B (rows ldb apart); rows >= K
    // and columns >= N read 0.
    __device__ __forceinline__ void load(const f16 *B, int ldb, int N, int K, int n0, int k0, int tid)
    {
        const int rows_k = min(T::BK, K - k0);
        const int cols = N - n0;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(B + (int64_t)k0 * ldb + n0, span_bytes(rows_k, ldb, cols));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + i * T::NT;
            const int q = p % Q, c = p / Q;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 4 * q + j;
                if constexpr (VEC) {
                    const uint32_t off = masked_offset((uint32_t)(row * ldb + 8 * c) * 2u, 8 * c < cols);
                    r[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int na = 8 * c + 2 * s, nb = na + 1;
                        const uint32_t oa = masked_offset((uint32_t)(row * ldb + na) * 2u, na < cols);
                        const uint32_t ob = masked_offset((uint32_t)(row * ldb + nb) * 2u, nb < cols);
                        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, oa, 0, 0);
                        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, ob, 0, 0);
                        w[s] = lo | (hi << 16);
                    }
                    r[i][j] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        }
    }

    __device__ __forceinline__ void store(f16 *bs, int tid) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + i * T::NT;
            const int q = p % Q, c = p / Q;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = e >> 1;
                uint32_t lo, hi;
                if (e & 1) {   // odd column: high halves of each row's dword d
                    lo = (r[i][0][d] >> 16) | (r[i][1][d] & 0xffff0000u);
                    hi = (r[i][2][d] >> 16) | (r[i][3][d] & 0xffff0000u);
                } else {       // even column: low halves
                    lo = (r[i][0][d] & 0xffffu) | (r[i][1][d] << 16);
                    hi = (r[i][2][d] & 0xffffu) | (r[i][3][d] << 16);
                }
                *reinterpret_cast<u32x2 *>(bs + (8 * c + e) * T::PITCH + 4 * q) = u32x2{lo, hi};
            }
        }
    }
};

// ---------------------------------------------------------------- kernel ------------
// MFMA operand layout for v_mfma_f32_32x32x16_f16 as used here: operand lane l holds 8
// consecutive-k values of row (l % 32) at k offset 8*(l / 32) -- the same k map for both
// operands, which is all the product needs.  The result layout is described at
// store_tile().
template <class T, bool AV, bool BV, int EPI>
__global__ void __launch_bounds__(T::NT) gemm_staged(GemmArgs p)
{
    __shared__ __attribute__((aligned(16))) f16 lds[T::STAGES * (T::A_STAGE + T::B_STAGE)];
    f16 *const As = lds;
    f16 *const Bs = lds + T::STAGES * T::A_STAGE;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int rows_valid = min(T::BM, p.M - m0);

    const __amdgpu_buffer_rsrc_t a_rs =
        make_rsrc(p.A + (int64_t)m0 * p.K, (uint32_t)(rows_valid * p.K) * 2u);

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
            acc[i][j] = f32x16{};

    ALoader<T, AV> al;
    BLoader<T, BV> bl;
    const int nk = (p.K + T::BK - 1) / T::BK;

    if (nk > 0) {
        al.load(a_rs, 0, p.K, tid);
        bl.load(p.B, p.ldb, p.N, p.K, n0, 0, tid);
        al.store(As, tid);
        bl.store(Bs, tid);
        __syncthreads();
        if (nk > 1) {
            al.load(a_rs, T::BK, p.K, tid);
            bl.load(p.B, p.ldb, p.N, p.K, n0, T::BK, tid);
        }
    }

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const f16 *as = As + cur * T::A_STAGE + (wm * T::WTM + frag_row) * T::PITCH + frag_k;
        const f16 *bs = Bs + cur * T::B_STAGE + (wn * T::WTN + frag_row) * T::PITCH + frag_k;
#pragma unroll
        for (int kk = 0; kk < T::BK / 16; ++kk) {
            f16x8 af[T::FM], bf[T::FN];
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                af[i] = *reinterpret_cast<const f16x8 *>(as + i * 32 * T::PITCH + kk * 16);
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                bf[j] = *reinterpret_cast<const f16x8 *>(bs + j * 32 * T::PITCH + kk * 16);
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            al.store(As + (cur ^ 1) * T::A_STAGE, tid);
            bl.store(Bs + (cur ^ 1) * T::B_STAGE, tid);
            if (kt + 2 < nk) {
                al.load(a_rs, (kt + 2) * T::BK, p.K, tid);
                bl.load(p.B, p.ldb, p.N, p.K, n0, (kt + 2) * T::BK, tid);
            }
        }
        __syncthreads();
    }

    store_tile<T::FM, T::FN, 0, T::FM, BV, EPI>(acc, p, m0, n0, rows_valid, wm * T::WTM, wn * T::WTN, lane);
}

}  // namespace mi355

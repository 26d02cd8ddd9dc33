// Direct-to-LDS GEMM kernel for gfx950: the fast path for 16-byte-friendly operands
// (K % 8 == 0 and N % 8 == 0, 16-byte aligned A, B, C).
//
// One workgroup (WAVES_M x WAVES_N wavefronts) computes one BM x BN macro-tile of C:
//   1. tile order  -- tile_coords(): XCD-contiguous ranges, GROUP_M tile-rows per sweep;
//   2. loader      -- buffer_load_dwordx4 ... lds: HBM -> LDS with no VGPR staging, into a
//                     ring of STAGES buffers (one __shared__ object per stage, so the
//                     compiler can tell the stages apart); the copy for stage kt+STAGES-1
//                     is in flight while stage kt is multiplied.  A lands k-contiguous,
//                     B lands in its HBM order (n-contiguous); both are XOR-swizzled in
//                     16-byte chunks so the fragment reads below hit distinct banks;
//   3. MFMA loop   -- A fragments come from ds_read_b128, B fragments from two
//                     ds_read_b64_tr_b16 (gfx950's transposing LDS read turns four
//                     n-contiguous rows into k-contiguous lane data); fragment reads for
//                     the next k-step are issued before the MFMAs of the current one, and
//                     the last k-step's MFMAs cover the barrier into the next stage;
//   4. epilogue    -- store_tile(): bias, erf-GELU, fp16 rounding, masked stores.
//
// Out-of-range rows, columns and the K tail read as zero through the buffer descriptors'
// range checks (rows past M / K) or an offset pushed out of range (columns past N, K
// chunks past K).
#pragma once

#include <type_traits>

#include "gemm_common.hpp"

namespace mi355 {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct DTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NT = 64 * NW;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KK = BK / 16;              // MFMA k-steps per stage
    static constexpr int CA = BK / 8;               // 16-byte chunks per A row
    static constexpr int CB = BN / 8;               // 16-byte chunks per B row
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    static constexpr int GA = A_BYTES / (1024 * NW);   // 1 KiB LDS-DMA loads per wave
    static constexpr int GB = B_BYTES / (1024 * NW);
    static constexpr int G = GA + GB;
    static constexpr int LDS_BYTES = STAGES * (A_BYTES + B_BYTES);
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK == 32 || BK == 64, "A swizzle assumes 4 or 8 chunks per row");
    static_assert(CB >= 16, "B swizzle assumes rows of at least 256 bytes");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0,
                  "stage must split into whole 1 KiB loads per wave");
    static_assert(STAGES >= 2 && STAGES <= 4 && G * (STAGES - 2) <= 63, "ring size / vmcnt range");
    static_assert(KK % 2 == 0, "fragment double-buffer parity assumes an even k-step count");
    static_assert(LDS_BYTES <= 160 * 1024, "over the gfx950 LDS budget");
};

template <class T>
struct __attribute__((aligned(16))) Stage {
    f16 a[T::BM * T::BK];
    f16 b[T::BK * T::BN];
};

// A chunk swizzle: rows of CA chunks; 16 B units within 256 B are (row % RP, chunk), so
// XOR the chunk with (row / RP) % CA to spread 16 consecutive rows over all 16 units.
template <class T>
__device__ __forceinline__ int swz_a(int row)
{
    constexpr int RP = 16 / T::CA;
    return (row / RP) % T::CA;
}

// B chunk swizzle: a transposing read touches 4 consecutive k-rows x 4 chunks; XOR bits 2-3
// of the chunk with k % 4 so those 16 chunks fall in distinct 16-byte bank groups.
__device__ __forceinline__ int swz_b(int k) { return 4 * (k & 3); }

// s_waitcnt immediates for gfx9: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts()
{
    static_assert(VM >= 0 && VM <= 63 && LGKM >= 0 && LGKM <= 15, "waitcnt range");
    constexpr int imm = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8);
    __builtin_amdgcn_s_waitcnt(imm);
}

// s_barrier without the fence __syncthreads() adds (which would wait for every load in
// flight, prefetches included).  The empty asm statements keep the optimizer from moving
// memory accesses across it; the counters it needs are waited for explicitly before.
__device__ __forceinline__ void workgroup_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(const void *p)
{
    return (__attribute__((address_space(3))) void *)(p);
}

// One 16-byte-per-lane LDS-DMA load: lane l copies 16 bytes from the buffer at voffset to
// LDS at lds + 16*l.  Written as inline assembly on purpose: the compiler cannot tell the
// ring slots apart once it has packed them into one LDS block, and would then wait for
// every copy in flight before each LDS read.  The kernel waits for these copies itself
// (wait_counts before each barrier) and for all of them before it ends.  Nothing else in
// the kernels uses M0.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, const void *lds,
                                          uint32_t voffset)
{
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds_ptr(lds);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc));
}

// Per-lane state of one wavefront: DMA source offsets, fragment read addresses, the
// accumulators and the double-buffered operand fragments.
template <class T>
struct DirectWave {
    using St = Stage<T>;
    int lane, wave, wm, wn;
    int K, N, n0;
    const f16 *B;
    __amdgpu_buffer_rsrc_t a_rs;
    uint32_t a_off[T::GA];
    int a_kc[T::GA];          // k of the chunk within the stage
    uint32_t b_off[T::GB];
    int a_row_byte[T::FM];
    int a_chunk_byte[T::KK];
    int b_col_byte[T::FN];
    int b_row_byte;
    f32x16 acc[T::FM][T::FN];
    f16x8 af[2][T::FM], bf[2][T::FN];

    __device__ __forceinline__ void init(const GemmArgs &p, int m0, int n0_, int rows_valid,
                                         int cols_valid)
    {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS-DMA base
        wm = wave / T::WAVES_N;
        wn = wave % T::WAVES_N;
        K = p.K;
        N = p.N;
        n0 = n0_;
        B = p.B;
        // A: slot s of the stage (16 B each) holds row s / CA, physical chunk s % CA, which
        // is logical chunk (s % CA) ^ swz_a(row); the K position adds k0 per stage.
        a_rs = make_rsrc(p.A + (int64_t)m0 * K, (uint32_t)(rows_valid * K) * 2u);
#pragma unroll
        for (int g = 0; g < T::GA; ++g) {
            const int s = (g * T::NW + wave) * 64 + lane;
            const int row = s / T::CA;
            const int c = (s % T::CA) ^ swz_a<T>(row);
            a_kc[g] = 8 * c;
            a_off[g] = (uint32_t)(row * K + 8 * c) * 2u;
        }
        // B: slot s holds k-row s / CB, physical chunk s % CB = logical chunk ^ swz_b(row).
#pragma unroll
        for (int g = 0; g < T::GB; ++g) {
            const int s = (g * T::NW + wave) * 64 + lane;
            const int row = s / T::CB;
            const int c = (s % T::CB) ^ swz_b(row);
            b_off[g] = masked_offset((uint32_t)(row * N + 8 * c) * 2u, 8 * c < cols_valid);
        }
        // A fragment: row wm*WTM + i*32 + r32, logical chunk 2*kk + h -> physical chunk
        // ^ swz_a(row); swz_a depends on the row only through r32 (WTM and 32 are
        // multiples of 16 * rows-per-256-bytes).
        const int h = lane >> 5;
        const int r32 = lane & 31;
        const int sa = swz_a<T>(r32);
#pragma unroll
        for (int i = 0; i < T::FM; ++i) a_row_byte[i] = (wm * T::WTM + i * 32 + r32) * T::BK * 2;
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) a_chunk_byte[kk] = ((2 * kk + h) ^ sa) * 16;
        // B fragment (transposing read): lane i of each 16-lane group points at k-row i/4
        // of its group's 4-row band and columns 4*(i%4) .. +3 of its 16-column half; lane j
        // then receives B[band + 0..3][half + j].  Band = 16*kk + 8*h + 4*t, t = 0 or 1.
        const int i16 = lane & 15;
        const int sb = swz_b(i16 >> 2);
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int n = wn * T::WTN + j * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
            b_col_byte[j] = (((n >> 3) ^ sb) * 16) + 8 * ((n >> 2) & 1);
        }
        b_row_byte = (8 * h + (i16 >> 2)) * T::BN * 2;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                acc[i][j] = f32x16{};
    }

    // HBM -> LDS copy of stage kt (A rows [m0, m0+BM) x k [k0, k0+BK), B k-rows x
    // columns [n0, n0+BN)) into dst.  A stage past the end of K copies zeros (every
    // offset falls out of range), which keeps the issue pattern, and so the counter
    // arithmetic below, the same in every iteration.
    __device__ __forceinline__ void issue_stage(St &dst, int kt) const
    {
        const int k0 = kt * T::BK;
#pragma unroll
        for (int g = 0; g < T::GA; ++g) {
            const uint32_t off = masked_offset(a_off[g] + (uint32_t)k0 * 2u, k0 + a_kc[g] < K);
            lds_dma16(a_rs, dst.a + (g * T::NW + wave) * 512, off);
        }
        const int rows_k = min(T::BK, K - k0);
        const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(
            B + (int64_t)min(k0, K) * N + n0, rows_k > 0 ? (uint32_t)(rows_k * N - n0) * 2u : 0u);
#pragma unroll
        for (int g = 0; g < T::GB; ++g) {
            lds_dma16(b_rs, dst.b + (g * T::NW + wave) * 512, b_off[g]);
        }
    }

    __device__ __forceinline__ void read_frags(const St &src, int kk, int buf)
    {
        const char *abase = reinterpret_cast<const char *>(src.a);
        const char *bbase = reinterpret_cast<const char *>(src.b);
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
            af[buf][i] = *reinterpret_cast<const f16x8 *>(abase + a_row_byte[i] + a_chunk_byte[kk]);
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const char *q = bbase + b_row_byte + (16 * kk) * T::BN * 2 + b_col_byte[j];
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)lds_ptr(q));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)lds_ptr(q + 4 * T::BN * 2));
            bf[buf][j] = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }

    __device__ __forceinline__ void mfmas(int buf)
    {
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[buf][j], af[buf][i], acc[i][j], 0, 0, 0);
    }
};

template <class T, int EPI>
__global__ void __launch_bounds__(T::NT) gemm_direct(GemmArgs p)
{
    using St = Stage<T>;
    __shared__ St st0;
    __shared__ St st1;
    __shared__ typename std::conditional<(T::STAGES > 2), St, char[16]>::type st2;
    __shared__ typename std::conditional<(T::STAGES > 3), St, char[16]>::type st3;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int rows_valid = min(T::BM, p.M - m0);
    const int nk = (p.K + T::BK - 1) / T::BK;

    DirectWave<T> w;
    w.init(p, m0, n0, rows_valid, p.N - n0);

    St *const ring[4] = {&st0, &st1, reinterpret_cast<St *>(&st2), reinterpret_cast<St *>(&st3)};

    // One K step on ring slot J (stage kt): start the copy of stage kt+STAGES-1 into the
    // slot freed by stage kt-1, run the KK MFMA k-steps with the next step's fragments
    // read ahead, and cross into stage kt+1 (wait for its copy, barrier, first fragment
    // reads) before the last k-step's MFMAs so they cover the barrier.  The body has no
    // branches, which keeps the compiler's LDS-DMA wait tracking exact; past the end of K
    // it copies zeros, multiplies zeros and reads fragments it never uses.
    auto step = [&](auto J, int kt) {
        constexpr int j = decltype(J)::value;
        St &cur = *ring[j];
        w.issue_stage(*ring[(j + T::STAGES - 1) % T::STAGES], kt + T::STAGES - 1);
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) {
            const int buf = kk & 1;
            if (kk + 1 < T::KK) {
                w.read_frags(cur, kk + 1, buf ^ 1);
            } else {
                // stage kt+1 has landed once at most the STAGES-2 later copies are in
                // flight; this wave's reads of stage kt are done before the barrier
                wait_counts<T::G * (T::STAGES - 2), 0>();
                workgroup_barrier();
                w.read_frags(*ring[(j + 1) % T::STAGES], 0, buf ^ 1);
            }
            w.mfmas(buf);
        }
    };

    if (nk > 0) {
        // ---- prologue: stages 0 .. STAGES-2 in flight, wait for stage 0 ----
#pragma unroll
        for (int s = 0; s < T::STAGES - 1; ++s) w.issue_stage(*ring[s], s);
        wait_counts<T::G * (T::STAGES - 2), 15>();
        workgroup_barrier();
        w.read_frags(*ring[0], 0, 0);

        // ---- main loop, unrolled over the ring so every stage is a distinct object.
        // The step count is rounded up to a whole number of ring turns: the extra
        // stages lie past the end of K, hold zeros, and add nothing to the sums.
        const int nk_ring = (nk + T::STAGES - 1) / T::STAGES * T::STAGES;
        for (int kt = 0; kt < nk_ring; kt += T::STAGES) {
            step(std::integral_constant<int, 0>{}, kt);
            step(std::integral_constant<int, 1>{}, kt + 1);
            if constexpr (T::STAGES > 2) step(std::integral_constant<int, 2>{}, kt + 2);
            if constexpr (T::STAGES > 3) step(std::integral_constant<int, 3>{}, kt + 3);
        }
        // the copies past the end of K are still landing; none may outlive the kernel
        wait_counts<0, 15>();
    }

    store_tile<T::FM, T::FN, true, EPI>(w.acc, p, m0, n0, rows_valid, w.wm * T::WTM,
                                        w.wn * T::WTN, w.lane);
}

}  // namespace mi355

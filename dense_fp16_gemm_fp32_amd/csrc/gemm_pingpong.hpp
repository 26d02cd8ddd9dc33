// Ping-pong GEMM kernel for gfx950: the direct-to-LDS loader and MFMA tiles of gemm_direct,
// run by two groups of four wavefronts that take turns.
//
// A workgroup has 8 waves; wave w runs on SIMD w % 4, so every SIMD holds one wave of
// group 0 (waves 0-3) and one of group 1 (waves 4-7).  Group g owns rows
// [g*BM/2, (g+1)*BM/2) of the BM x BN tile (4 waves of (BM/2) x (BN/4) each).  Time is cut
// into phases separated by workgroup barriers.  In each phase one group multiplies (it
// issues the MFMAs of one stage back to back on operand fragments already in its
// registers) while the other group loads (it reads the fragments for its next phase from
// LDS and issues its share of the HBM -> LDS copies); in the next phase they swap.  Stage
// t is multiplied by group 0 in phase 2t and by group 1 in phase 2t+1.  A wave thus never
// waits on memory in a phase in which it multiplies, and the MFMA pipe of each SIMD is fed
// by one of its two waves in every phase; in gemm_direct every wave waits for the next
// stage's copies at the same barrier, and the MFMA pipes stand still meanwhile.
//
// Copies (the LDS-DMA pieces, swizzles and zero fill of gemm_direct): a stage's slot is
// refilled once group 1 has loaded its fragments from it, and every copy is issued in a
// load phase.  Both groups copy a share of every stage, group 0 in phase 2(t-S)+1 and
// group 1 in phase 2(t-S)+2 for stage t (S ring slots); stage t must have landed before
// phase 2t-1, when group 0 loads it.  Stages past the end of K copy zeros, so the issue
// pattern, and with it the s_waitcnt arithmetic, is the same in every phase.
//
// Each group runs its own copy of the phase loop, free of branches on the group; the
// copies execute the same barriers in the same order, which is what the workgroup barrier
// counts.  The group is a wave-uniform (scalar) value, so the choice of copy is a scalar
// branch taken by whole waves.
//
// Measured on MI355X against gemm_direct's 256x256 tiles (interleaved on one box): 8192^3
// 826.9 against 828.1 us (4 waves of 128x128) and 835.9 us (8 waves of 128x64), with bias
// + GELU 865.0 against 872.3 us, 4096^3 107.9 against 108.3 us.  The same schedule on
// 128x128 tiles (the two groups taking alternate K stages, partial tiles summed at the end)
// lost at 2048^3 by 9-17% to gemm_direct and was not kept.
#pragma once

#include "gemm_direct.hpp"

namespace mi355 {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_>
struct PTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WM = WM_, WN = WN_;         // waves of one group in M and N
    static constexpr int STAGES = STAGES_;
    static constexpr int NW = 8, NT = 512, NWG = 4;  // waves, threads, waves per group
    static constexpr int NL = 0, NTC = NT;           // no loader waves: every thread stores C
    static constexpr int MF = 32, NG = 4, MFS = 5;   // 32x32 MFMA blocks, 4 register quads
    using AccT = f32x16;
    static constexpr int ROWS_G = BM / 2;            // rows one group computes
    static constexpr int WTM = ROWS_G / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KK = BK / 16;               // k-steps per stage (= per phase)
    static constexpr int CA = BK / 8, CB = BN / 8;   // 16-byte chunks per A row / B row
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int GA = A_BYTES / (1024 * NW), GB = B_BYTES / (1024 * NW);
    static constexpr int G = GA + GB;                // 1 KiB copies per wave per stage
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    // copies of this wave allowed in flight once the stage group 0 loads next has landed
    static constexpr int VM_WAIT = G * (STAGES - 2);
    static_assert(WM * WN == NWG, "four waves per group");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK == 32 || BK == 64, "A swizzle assumes 4 or 8 chunks per row");
    static_assert(CB % 16 == 0, "B swizzle assumes rows of a multiple of 256 bytes");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0,
                  "stage must split into whole 1 KiB loads per wave");
    static_assert(STAGES >= 3, "at least 3 ring slots");
    static_assert(G * STAGES <= 63 && VM_WAIT >= 0, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "over the gfx950 LDS budget");
    static_assert(BM * BN * 2 <= LDS_BYTES, "the C tile is staged in the ring");
};

template <class T>
struct PingWave {
    using St = Stage<T>;
    int lane, wave, grp, wc, wm, wn;
    int K, N, ldb, n0;
    const f16 *B;
    __amdgpu_buffer_rsrc_t a_rs;
    uint32_t a_off[T::GA];
    int a_kc[T::GA];
    uint32_t b_off[T::GB];
    int a_row_byte[T::FM];
    int a_chunk_byte[T::KK];
    int b_k_byte[T::KK];
    int b_col_byte[T::FN];
    int b_row_byte;
    u32x2 bias_raw[T::FN][4];
    f32x16 acc[T::FM][T::FN];
    f16x8 af[T::KK][T::FM];
    f16x8 bf[T::KK][T::FN];   // B fragments: the two transposing reads of each, joined

    __device__ __forceinline__ void init(const GemmArgs &p, int m0, int n0_, int rows_valid,
                                         int cols_valid)
    {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        grp = wave >> 2;
        wc = wave & 3;
        wm = wc / T::WN;
        wn = wc % T::WN;
        K = p.K;
        N = p.N;
        ldb = p.ldb;
        n0 = n0_;
        B = p.B;
        // copies: slot s (16 B) of the stage holds A row s / CA, physical chunk s % CA =
        // logical chunk ^ swz_a(row); B k-row s / CB, chunk s % CB = logical ^ swz_b(row)
        a_rs = make_rsrc(p.A + (int64_t)m0 * K, (uint32_t)(rows_valid * K) * 2u);
#pragma unroll
        for (int g = 0; g < T::GA; ++g) {
            const int s = (g * T::NW + wave) * 64 + lane;
            const int row = s / T::CA;
            const int c = (s % T::CA) ^ swz_a<T>(row);
            a_kc[g] = 8 * c;
            a_off[g] = (uint32_t)(row * K + 8 * c) * 2u;
        }
#pragma unroll
        for (int g = 0; g < T::GB; ++g) {
            const int s = (g * T::NW + wave) * 64 + lane;
            const int row = s / T::CB;
            const int c = (s % T::CB) ^ swz_b(row);
            b_off[g] = masked_offset((uint32_t)(row * ldb + 8 * c) * 2u, 8 * c < cols_valid);
        }
        // fragments: A block i of this wave covers tile rows rbase + 32 i .. +31 (lane row
        // r32, k-half h); B as in gemm_direct (transposing reads of 4 k-rows x 4 columns)
        const int h = lane >> 5;
        const int r32 = lane & 31;
        const int sa = swz_a<T>(r32);
        const int rbase = grp * T::ROWS_G + wm * T::WTM;
#pragma unroll
        for (int i = 0; i < T::FM; ++i) a_row_byte[i] = (rbase + i * 32 + r32) * T::BK * 2;
#pragma unroll
        for (int q = 0; q < T::KK; ++q) {
            a_chunk_byte[q] = ((2 * q + h) ^ sa) * 16;
            b_k_byte[q] = (16 * q) * T::BN * 2;
        }
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

    // first tile row of this wave's accumulator blocks
    __device__ __forceinline__ int row0() const
    {
        return grp * T::ROWS_G + wm * T::WTM;
    }

    __device__ __forceinline__ void load_bias(const GemmArgs &p)
    {
        const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(p.bias + n0, (uint32_t)(N - n0) * 2u);
        const int half = lane >> 5;
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = wn * T::WTN + j * 32 + 8 * g + 4 * half;
                bias_raw[j][g] = __builtin_amdgcn_raw_buffer_load_b64(b_rs, (uint32_t)n * 2u, 0, 0);
            }
    }

    // This wave's share (G pieces of 1 KiB) of the copy of stage kt into dst; as
    // DirectWave::issue_piece (FULL: the stage lies wholly below K).
    template <bool FULL>
    __device__ __forceinline__ void copy_stage(St &dst, int kt) const
    {
        const int k0 = kt * T::BK;
#pragma unroll
        for (int g = 0; g < T::GA; ++g) {
            if constexpr (FULL) {
                lds_dma16(a_rs, dst.a + (g * T::NW + wave) * 512, a_off[g], (uint32_t)k0 * 2u);
            } else {
                const uint32_t off = masked_offset(a_off[g] + (uint32_t)k0 * 2u, k0 + a_kc[g] < K);
                lds_dma16(a_rs, dst.a + (g * T::NW + wave) * 512, off);
            }
        }
        const int rows_k = FULL ? T::BK : min(T::BK, K - k0);
        const __amdgpu_buffer_rsrc_t b_rs =
            make_rsrc(B + (int64_t)(FULL ? k0 : min(k0, K)) * ldb + n0, span_bytes(rows_k, ldb, N - n0));
#pragma unroll
        for (int g = 0; g < T::GB; ++g) lds_dma16(b_rs, dst.b + (g * T::NW + wave) * 512, b_off[g]);
    }

    // All fragments of stage src for this wave's rows (every k-step of the stage).
    __device__ __forceinline__ void load_fragments(const St &src)
    {
        const char *abase = reinterpret_cast<const char *>(src.a);
        const char *bbase = reinterpret_cast<const char *>(src.b);
#pragma unroll
        for (int q = 0; q < T::KK; ++q) {
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                af[q][i] = *reinterpret_cast<const f16x8 *>(abase + a_row_byte[i] + a_chunk_byte[q]);
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const char *p = bbase + b_row_byte + b_k_byte[q] + b_col_byte[j];
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)lds_ptr(p));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)lds_ptr(p + 4 * T::BN * 2));
                bf[q][j] = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
    }

    // Every MFMA of one stage for this wave, k-step by k-step.
    __device__ __forceinline__ void multiply()
    {
#pragma unroll
        for (int q = 0; q < T::KK; ++q)
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[q][j], af[q][i], acc[i][j], 0, 0, 0);
                }
    }
};

template <class T, int EPI>
__global__ void __launch_bounds__(T::NT) gemm_pingpong(GemmArgs p)
{
    using St = Stage<T>;
    constexpr int S = T::STAGES;
    __shared__ __attribute__((aligned(16))) char lds_raw[T::LDS_BYTES];

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int rows_valid = min(T::BM, p.M - m0);
    const int nk = (p.K + T::BK - 1) / T::BK;

    PingWave<T> w;
    w.init(p, m0, n0, rows_valid, p.N - n0);
    // wave-uniform (a scalar value): every branch on it below is taken by whole waves
    const bool g0 = w.grp == 0;
    St *const ring = reinterpret_cast<St *>(lds_raw);

    if (nk > 0) {
        // ---- prologue: group 0 copies its share of stages 0 .. S-1, group 1 of stages
        // 0 .. S-2 (its share of stage S-1 is due in phase 0); stage 0 has landed
#pragma unroll
        for (int s = 0; s < S - 1; ++s) w.template copy_stage<false>(ring[s], s);
        if (g0) {
            w.template copy_stage<false>(ring[S - 1], S - 1);
            wait_counts<T::G * (S - 1), 15>();
        } else {
            wait_counts<T::G * (S - 2), 15>();
        }
        workgroup_barrier();
        if (g0) w.load_fragments(ring[0]);   // for phase 0
        wait_counts<63, 0>();
        workgroup_barrier();

        // Stage t in ring slot J = t % S: phase 2t (group 0 multiplies; group 1 loads stage
        // t and copies its share of stage t+S-1 into the slot of stage t-1) and phase 2t+1
        // (group 1 multiplies; group 0 loads stage t+1 and copies its share of stage t+S into
        // the slot of stage t, which group 1 has just read).  The end of phase 2t waits until
        // stage t+1 has landed.  G0: the group-0 copy of the loop.
        auto run = [&](auto role_c) {
            constexpr bool G0 = decltype(role_c)::value;
            auto stage = [&](auto Jc, int t, auto full_c) {
                constexpr int J = decltype(Jc)::value;
                constexpr bool FULL = decltype(full_c)::value;
                St &cur = ring[J];
                St &nxt = ring[(J + 1) % S];
                St &prv = ring[(J + S - 1) % S];
                if constexpr (G0) {
                    w.multiply();
                } else {
                    w.load_fragments(cur);
                    w.template copy_stage<FULL>(prv, t + S - 1);
                }
                wait_counts<T::VM_WAIT, 0>();
                workgroup_barrier();
                if constexpr (G0) {
                    if (t + 1 < nk) w.load_fragments(nxt);
                    w.template copy_stage<FULL>(cur, t + S);
                } else {
                    w.multiply();
                }
                wait_counts<63, 0>();
                workgroup_barrier();
            };
            // whole ring turns whose copies (up to stage t + 2S - 1) all lie below K take
            // the copy without the K mask
            int t = 0;
            for (; (t + 2 * S) * T::BK <= p.K; t += S)
                static_for<S>([&](auto jc) { stage(jc, t + decltype(jc)::value, std::true_type{}); });
            for (; t < nk; t += S)
                static_for<S>([&](auto jc) {
                    const int k = t + decltype(jc)::value;
                    if (k < nk) stage(jc, k, std::false_type{});
                });
        };
        if (g0) run(std::true_type{}); else run(std::false_type{});
        // copies of stages past the end of K are still landing; none may outlive the
        // kernel, and the ring is reused below
        wait_counts<0, 0>();
        workgroup_barrier();
    }

    // Each wave holds 128 accumulator registers, so the bias is loaded only now (16
    // registers fewer through the K loop).
    if constexpr (EPI != 0) w.load_bias(p);
    char *ctile = lds_raw;
    tile_to_lds<T, 0, T::FM, EPI>(w.acc, w.bias_raw, w.row0(), w.wn * T::WTN, w.lane, ctile);
    __syncthreads();
    lds_to_c<T>(p, m0, n0, rows_valid, ctile);
}

}  // namespace mi355

// Direct-to-LDS GEMM kernel for gfx950: the fast path whenever B and C rows are 16-byte
// friendly (N % 8 == 0, 16-byte aligned B and C, 8-byte aligned bias).  A may have any
// 2-byte alignment and any K: the LDS-DMA copy takes unaligned source offsets, and the
// one chunk per row that straddles K (K % 8 != 0) is patched in LDS (see load_tail) by
// the KTAIL variant of the kernel.  The variant for K % 8 == 0 leaves the patch out: the
// patch holds 8 registers per A piece through the whole K loop, which made the
// 256x256x64 eight-wave tile spill.
//
// One workgroup computes one BM x BN macro-tile of C with WAVES_M x WAVES_N x KGROUPS
// wavefronts: one per SIMD (4 waves, the larger wave tiles) or two per SIMD (8 waves, so
// one wave's LDS reads and barrier waits are covered by the other's MFMAs):
//   1. tile order  -- tile_coords(): XCD-contiguous ranges, GROUP_M tile-rows per sweep;
//   2. loader      -- buffer_load_dwordx4 ... lds: HBM -> LDS with no VGPR staging, into a
//                     ring of STAGES buffers; the copy for stage kt+STAGES-1 is in flight
//                     while stage kt is multiplied.  A lands k-contiguous, B lands in its
//                     HBM order (n-contiguous); both are XOR-swizzled in 16-byte chunks so
//                     the fragment reads below hit distinct banks;
//   3. MFMA loop   -- A fragments come from ds_read_b128, B fragments from two
//                     ds_read_b64_tr_b16 (gfx950's transposing LDS read turns four
//                     n-contiguous rows into k-contiguous lane data).  With KGROUPS = 2 the
//                     16-deep k-steps of a stage alternate between two groups of waves that
//                     each own a full copy of the accumulator tile (a split of K inside the
//                     workgroup, summed through LDS at the end): two waves per SIMD without
//                     extra LDS traffic.  The instruction order inside a k-step is fixed in
//                     the source: after each MFMA come the LDS reads for the next k-step and
//                     a share of the HBM -> LDS copies, fenced with sched_barrier;
//   4. epilogue    -- bias, erf-GELU and fp16 rounding in registers, the tile staged in
//                     LDS, then whole-row 16-byte stores (tile_to_lds, lds_to_c).
//
// Out-of-range rows, columns and the K tail read as zero through the buffer descriptors'
// range checks (rows past M / K) or an offset pushed out of range (columns past N, K
// chunks past K).
#pragma once

#include <type_traits>
#include <utility>

#include "gemm_common.hpp"

namespace mi355 {

// PF: k-steps the LDS fragment reads run ahead of the MFMAs that consume them (1: the next
// k-step's fragments are read during the current one, 2 fragment buffers; 2 or 3: 4
// buffers, so each read has one or two whole k-steps of MFMAs to complete in).
//
// LOADERS: 0, or the number of extra wavefronts that issue every HBM -> LDS copy while the
// NW multiplying waves only read LDS and issue MFMAs (the loader waves share the SIMDs
// with them, one more wave per SIMD for LOADERS = 4).
// MF: the MFMA block, 32 (v_mfma_f32_32x32x16_f16, 16-deep k-steps) or 16
// (v_mfma_f32_16x16x32_f16, 32-deep k-steps: wave tiles in multiples of 16, so four waves
// can split 192 columns into 48 each and read every B fragment once).
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int KGROUPS_, int STAGES_,
          int PF_ = 1, int LOADERS_ = 0, int MF_ = 32>
struct DTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int KGROUPS = KGROUPS_, STAGES = STAGES_, PF = PF_;
    static constexpr int NWC = WAVES_M * WAVES_N;    // waves of one k-group
    static constexpr int NW = NWC * KGROUPS;         // multiplying waves
    static constexpr int NL = LOADERS_;              // loader waves (waves NW .. NW+NL-1)
    static constexpr int NI = NL > 0 ? NL : NW;      // waves that issue the copies
    static constexpr int NTC = 64 * NW;              // threads of the multiplying waves
    static constexpr int NT = 64 * (NW + NL);
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int MF = MF_;                   // MFMA block edge
    static constexpr int KS = MF == 32 ? 16 : 32;    // depth of one MFMA k-step
    static constexpr int NG = MF == 32 ? 4 : 1;      // 4-column register quads per block and lane
    static constexpr int MFS = MF == 32 ? 5 : 4;     // log2(MF)
    using AccT = std::conditional_t<MF == 32, f32x16, f32x4>;
    static constexpr int FM = WTM / MF, FN = WTN / MF;
    static constexpr int NMFMA = FM * FN;            // MFMAs per k-step per wave
    static constexpr int NREAD = FM + 2 * FN;        // LDS reads per k-step per wave
    static constexpr int KK = BK / KS;               // k-steps per stage
    static constexpr int Q = KK / KGROUPS;           // k-steps per stage per wave
    static constexpr int CA = BK / 8;                // 16-byte chunks per A row
    static constexpr int CB = BN / 8;                // 16-byte chunks per B row
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int GA = A_BYTES / (1024 * NI);   // 1 KiB LDS-DMA loads per issuing wave
    static constexpr int GB = B_BYTES / (1024 * NI);
    static constexpr int G = GA + GB;
    static constexpr int NBUF = PF == 1 ? 2 : 4;      // fragment buffers
    // k-step of a stage that waits for the next stage's copy and crosses the barrier: from
    // there on the reads run into the next stage
    static constexpr int QB = Q - PF;
    // Copies of a stage issued in its first k-step: all of them with a ring of 2 stages
    // (the next stage's copy must land before the end-of-stage wait) or one k-step per
    // stage; else half, and the rest after the barrier.  VM_WAIT: the copies younger than
    // the next stage's when the wait is reached (the first k-step's copies come after the
    // barrier when the barrier is in that k-step, QB == 0, with more than one k-step).
    static constexpr int G_EARLY = (STAGES >= 3 && Q >= 2) ? G / 2 : G;
    static constexpr int VM_WAIT = G * (STAGES - 3) + ((QB > 0 || Q == 1) ? G_EARLY : 0);
    // loader waves: the copies of the stages after the next one, in flight at each barrier
    static constexpr int VM_WAIT_L = G * (STAGES - 2);
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    // k-group exchange at the end: every wave hands half of its 32x32 fp32 blocks (4 KiB
    // each) to its partner in the other group
    static constexpr int RED_BYTES = KGROUPS > 1 ? NW * (NMFMA / 2) * 4096 : 0;
    static_assert(MF == 32 || MF == 16, "MFMA blocks of 32x32 or 16x16");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be whole MFMA blocks");
    static_assert(BK == 32 || BK == 64, "A swizzle assumes 4 or 8 chunks per row");
    static_assert(BK % KS == 0, "stage of whole k-steps");
    static_assert(MF == 32 || KGROUPS == 1, "k-group exchange written for 32x32 blocks");
    static_assert(CB % 8 == 0, "B swizzle assumes rows of a multiple of 128 bytes");
    static_assert(A_BYTES % (1024 * NI) == 0 && B_BYTES % (1024 * NI) == 0,
                  "stage must split into whole 1 KiB loads per wave");
    static_assert(NL == 0 || (KGROUPS == 1 && NW + NL <= 16), "loader waves: one k-group, 16 waves at most");
    static_assert(KGROUPS == 1 || (KGROUPS == 2 && FM % 2 == 0), "k-groups: 1, or 2 with even FM");
    static_assert(KK % KGROUPS == 0, "k-steps must split evenly over the k-groups");
    static_assert(PF >= 1 && PF <= Q && PF <= 3, "reads run at most one stage and 3 k-steps ahead");
    static_assert(PF == 1 || STAGES >= 3, "prefetch beyond one k-step needs a ring of 3 or more");
    static_assert((STAGES * Q) % NBUF == 0, "fragment buffer cycle must repeat per ring turn");
    static_assert(STAGES >= 2 && STAGES <= 8 && G * (STAGES - 2) <= 63, "ring size / vmcnt range");
    static_assert(VM_WAIT >= 0 && VM_WAIT <= 63, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "over the gfx950 LDS budget");
    static_assert(RED_BYTES <= LDS_BYTES, "k-group exchange must fit in the ring");
    static_assert(BM * BN * 2 <= LDS_BYTES, "the C tile is staged in the ring");
};

template <class T>
struct __attribute__((aligned(16))) Stage {
    f16 a[T::BM * T::BK];
    f16 b[T::BK * T::BN];
};

// A chunk swizzle: rows of CA chunks; 16 B units within 256 B are (row % RP, chunk), so
// XOR the chunk with (row / RP) % CA to spread 16 consecutive rows over all 16 units.
// With 16x16 MFMA blocks a read covers 16 rows x 4 chunks instead of 32 rows x 2, and on
// 64-byte rows (CA = 4) the rows are taken two at a time: (row / 2) % 4.  Measured with
// rocprofv3's SQ_LDS_BANK_CONFLICT on those reads: 4 conflict cycles per instruction with
// (row / 4) % 4, none with (row / 2) % 4; on 128-byte rows (row / 2) % 8 has none either way.
template <class T>
__device__ __forceinline__ int swz_a(int row)
{
    constexpr int RP = (T::MF == 16 && T::CA == 4) ? 2 : 16 / T::CA;
    return (row / RP) % T::CA;
}

// B chunk swizzle: a transposing read touches 4 consecutive k-rows (k % 4 = 0..3) x 4
// chunks (the first a multiple of 4), and those 16 chunks must fall in distinct 16-byte
// bank groups (16 groups of 4 banks).  Rows of CB chunks start CB % 16 groups apart:
//   CB % 16 == 0 -- every row starts at group 0: XOR bits 2-3 of the chunk with k % 4;
//   CB % 16 == 8 -- rows alternate between groups 0 and 8, so only rows k and k + 2
//                   collide: XOR bit 2 of the chunk with bit 1 of k.  The chunk stays in
//                   its aligned group of 8, which a row of CB chunks holds whole.
// With 16x16 MFMA blocks (MF = 16) the lanes of one read are four 16-lane groups on k-rows
// 8 apart (each 4 rows x 2 chunks), and groups 8 rows apart would meet in the same bank
// groups: bit 1 of the chunk is XORed with bit 3 of k as well.
template <int CB = 16, int MF = 32>
__device__ __forceinline__ int swz_b(int k)
{
    static_assert(CB % 8 == 0, "B rows of a multiple of 128 bytes");
    return (CB % 16 == 0 ? 4 * (k & 3) : 4 * ((k >> 1) & 1)) ^ (MF == 16 ? 2 * ((k >> 3) & 1) : 0);
}

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
// (wait_counts before each barrier) and for all of them before it ends.  The LDS address
// is an operand bound to M0 ("{m0}"): the compiler writes M0 itself right before the
// statement and knows the statement reads it, so no value of its own is lost there.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, const void *lds,
                                          uint32_t voffset)
{
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds_ptr(lds);
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr));
}

// The same copy with a wave-uniform byte offset `soffset` added in the instruction's
// scalar offset field, so a per-lane offset that does not change can be reused as is.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, const void *lds,
                                          uint32_t voffset, uint32_t soffset)
{
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds_ptr(lds);
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(soffset), "{m0}"(lds_addr));
}

// Per-lane state of one wavefront: DMA source offsets, fragment read addresses, the
// accumulators and the double-buffered operand fragments.
template <class T>
struct DirectWave {
    using St = Stage<T>;
    int lane, wave, kg, wm, wn;
    int issuer;               // index among the waves that issue copies (< 0: none)
    int K, N, ldb, n0;
    const f16 *B;
    __amdgpu_buffer_rsrc_t a_rs;
    uint32_t a_off[T::GA];
    int a_kc[T::GA];          // k of the chunk within the stage
    uint32_t b_off[T::GB];
    int a_row_byte[T::FM];
    int a_chunk_byte[T::Q];   // per k-step of this wave
    int b_k_byte[T::Q];
    int b_col_byte[T::FN];
    int b_row_byte;
    uint32_t tailh[T::GA][8]; // the K-tail chunks of this lane's A pieces (K % 8 != 0),
                              // one half per register: packed only when patched, so the
                              // loads stay in flight until then
    uint32_t tail_mask;       // bit g: piece g of the last stage straddles K
    u32x2 bias_raw[T::FN][T::NG]; // bias of this lane's accumulator columns (bias epilogues)
    typename T::AccT acc[T::FM][T::FN];
    f16x8 af[T::NBUF][T::FM];
    s16x4 bl[T::NBUF][T::FN], bh[T::NBUF][T::FN];

    __device__ __forceinline__ void init(const GemmArgs &p, int m0, int n0_, int rows_valid,
                                         int cols_valid)
    {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS-DMA base
        kg = wave / T::NWC;
        issuer = T::NL > 0 ? wave - T::NW : wave;
        const int wc = wave % T::NWC;
        wm = wc / T::WAVES_N;
        wn = wc % T::WAVES_N;
        K = p.K;
        N = p.N;
        ldb = p.ldb;
        n0 = n0_;
        B = p.B;
        // A: slot s of the stage (16 B each) holds row s / CA, physical chunk s % CA, which
        // is logical chunk (s % CA) ^ swz_a(row); the K position adds k0 per stage.
        a_rs = make_rsrc(p.A + (int64_t)m0 * K, (uint32_t)(rows_valid * K) * 2u);
#pragma unroll
        for (int g = 0; g < T::GA; ++g) {
            const int s = (g * T::NI + issuer) * 64 + lane;
            const int row = s / T::CA;
            const int c = (s % T::CA) ^ swz_a<T>(row);
            a_kc[g] = 8 * c;
            a_off[g] = (uint32_t)(row * K + 8 * c) * 2u;
        }
        // B: slot s holds k-row s / CB, physical chunk s % CB = logical chunk ^ swz_b(row).
#pragma unroll
        for (int g = 0; g < T::GB; ++g) {
            const int s = (g * T::NI + issuer) * 64 + lane;
            const int row = s / T::CB;
            const int c = (s % T::CB) ^ swz_b<T::CB, T::MF>(row);
            b_off[g] = masked_offset((uint32_t)(row * ldb + 8 * c) * 2u, 8 * c < cols_valid);
        }
        // Operand lane map of both MFMA shapes: lane l holds the 8 k-values 8 * (l / MF) ..
        // +7 of the k-step for row (A) or column (B) l % MF of the block.
        // A fragment: row wm*WTM + i*MF + rlo, logical chunk (KS/8)*kk + kgrp -> physical
        // chunk ^ swz_a(row); swz_a depends on the row only through rlo (WTM and MF are
        // multiples of 16 * rows-per-256-bytes).  This wave's k-steps are kk = kg +
        // KGROUPS * q.
        const int kgrp = lane >> T::MFS;
        const int rlo = lane & (T::MF - 1);
        const int sa = swz_a<T>(rlo);
#pragma unroll
        for (int i = 0; i < T::FM; ++i) a_row_byte[i] = (wm * T::WTM + i * T::MF + rlo) * T::BK * 2;
#pragma unroll
        for (int q = 0; q < T::Q; ++q) {
            const int kk = kg + T::KGROUPS * q;
            a_chunk_byte[q] = (((T::KS / 8) * kk + kgrp) ^ sa) * 16;
            b_k_byte[q] = (T::KS * kk) * T::BN * 2;
        }
        // B fragment (transposing read): lane i of each 16-lane group points at k-row i/4
        // of its group's 4-row band and columns 4*(i%4) .. +3 of its 16 columns; lane j
        // then receives B[band + 0..3][col + j].  Band = KS*kk + 8*kgrp + 4*t, t = 0 or 1;
        // the 16 columns are the block's (MF = 16) or its half (lane / 16) % 2 (MF = 32).
        const int i16 = lane & 15;
        // the k-row of this lane: 8 * kgrp + i16 / 4 (+ KS * kk + 4 t, multiples of 8 and 4);
        // for MF = 32 the swizzle reads only its two low bits
        const int sb = swz_b<T::CB, T::MF>(T::MF == 32 ? (i16 >> 2) : 8 * kgrp + (i16 >> 2));
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int n = wn * T::WTN + j * T::MF + (T::MF == 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (i16 & 3);
            b_col_byte[j] = (((n >> 3) ^ sb) * 16) + 8 * ((n >> 2) & 1);
        }
        b_row_byte = (8 * kgrp + (i16 >> 2)) * T::BN * 2;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                acc[i][j] = typename T::AccT{};
    }

    // The bias values this lane's accumulator columns need, loaded at the start so the
    // epilogue does not wait a memory round trip for them.  Columns past N read 0.
    __device__ __forceinline__ void load_bias(const GemmArgs &p)
    {
        const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(p.bias + n0, (uint32_t)(N - n0) * 2u);
        const int kgrp = lane >> T::MFS;
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int g = 0; g < T::NG; ++g) {
                const int n = wn * T::WTN + j * T::MF + 8 * g + 4 * kgrp;
                bias_raw[j][g] = __builtin_amdgcn_raw_buffer_load_b64(b_rs, (uint32_t)n * 2u, 0, 0);
            }
    }

    // K % 8 != 0: in the last stage, the A chunk of a row that contains K holds some
    // elements below K and some past it.  The copy would read the next row's elements (or
    // past the end of A) there, so the lane that copies such a chunk loads its elements
    // below K one by one (zeros past K) at the start of the kernel, and patch_tail()
    // writes them over the copied chunk once the last stage's copy has landed.
    __device__ __forceinline__ void load_tail(int nk)
    {
        tail_mask = 0;
        const int k0 = (nk - 1) * T::BK;
#pragma unroll
        for (int g = 0; g < T::GA; ++g) {
            const int k = k0 + a_kc[g];
            if (k < K && k + 8 > K) tail_mask |= 1u << g;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t off = masked_offset(a_off[g] + (uint32_t)(k0 + e) * 2u, k + e < K);
                tailh[g][e] = __builtin_amdgcn_raw_buffer_load_b16(a_rs, off, 0, 0);
            }
        }
    }

    // Overwrites the straddling chunks of the last stage, held in slot dst, with the
    // values load_tail() read; call after that stage's copy has landed and before the
    // barrier that lets the waves read it.
    __device__ __forceinline__ void patch_tail(St &dst) const
    {
#pragma unroll
        for (int g = 0; g < T::GA; ++g) {
            if (tail_mask & (1u << g)) {
                char *q = reinterpret_cast<char *>(dst.a) + ((g * T::NI + issuer) * 64 + lane) * 16;
                uint32_t t[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    t[e] = tailh[g][e];
                    // opaque here, so the packing (and the wait for these loads) is not
                    // hoisted out of the K loop to the start of the kernel
                    asm volatile("" : "+v"(t[e]));
                }
                *reinterpret_cast<u32x4 *>(q) =
                    u32x4{t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16), t[6] | (t[7] << 16)};
            }
        }
        wait_counts<63, 0>();   // the patch is in LDS before the barrier
    }

    // Piece g (0 <= g < G) of the HBM -> LDS copy of stage kt (A rows [m0, m0+BM) x k
    // [k0, k0+BK), B k-rows x columns [n0, n0+BN)) into dst.  A stage past the end of K
    // copies zeros (every offset falls out of range), which keeps the issue pattern, and
    // so the counter arithmetic below, the same in every iteration.  FULL: the stage lies
    // wholly below K, so no A chunk needs the K mask and the stage's K offset rides in
    // the scalar offset field (no vector instruction per piece); rows past M still fall
    // outside the descriptor's range.
    template <bool FULL = false>
    __device__ __forceinline__ void issue_piece(St &dst, int kt, int g) const
    {
        const int k0 = kt * T::BK;
        if (g < T::GA) {
            if constexpr (FULL) {
                lds_dma16(a_rs, dst.a + (g * T::NI + issuer) * 512, a_off[g], (uint32_t)k0 * 2u);
            } else {
                const uint32_t off = masked_offset(a_off[g] + (uint32_t)k0 * 2u, k0 + a_kc[g] < K);
                lds_dma16(a_rs, dst.a + (g * T::NI + issuer) * 512, off);
            }
        } else {
            const int gb = g - T::GA;
            // B rows [k0, k0 + rows_k) of this tile's columns; FULL: all BK rows
            const int rows_k = FULL ? T::BK : min(T::BK, K - k0);
            const __amdgpu_buffer_rsrc_t b_rs =
                make_rsrc(B + (int64_t)(FULL ? k0 : min(k0, K)) * ldb + n0, span_bytes(rows_k, ldb, N - n0));
            lds_dma16(b_rs, dst.b + (gb * T::NI + issuer) * 512, b_off[gb]);
        }
    }

    template <bool FULL = false>
    __device__ __forceinline__ void issue_stage(St &dst, int kt) const
    {
#pragma unroll
        for (int g = 0; g < T::G; ++g) issue_piece<FULL>(dst, kt, g);
    }

    // Read r (0 <= r < NREAD) of the fragments for this wave's k-step q of stage src, into
    // fragment buffer buf.  Order: A block 0, then both halves of every B block, then the
    // other A blocks -- the order the MFMAs (i outer, j inner) first need them.
    __device__ __forceinline__ void read_one(const St &src, int q, int buf, int r)
    {
        const char *abase = reinterpret_cast<const char *>(src.a);
        const char *bbase = reinterpret_cast<const char *>(src.b);
        if (r == 0 || r >= 1 + 2 * T::FN) {
            const int i = (r == 0) ? 0 : r - 2 * T::FN;
            af[buf][i] = *reinterpret_cast<const f16x8 *>(abase + a_row_byte[i] + a_chunk_byte[q]);
        } else {
            const int j = (r - 1) >> 1;
            const char *p = bbase + b_row_byte + b_k_byte[q] + b_col_byte[j];
            if (((r - 1) & 1) == 0)
                bl[buf][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)lds_ptr(p));
            else
                bh[buf][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)lds_ptr(p + 4 * T::BN * 2));
        }
    }

    __device__ __forceinline__ void read_all(const St &src, int q, int buf)
    {
#pragma unroll
        for (int r = 0; r < T::NREAD; ++r) read_one(src, q, buf, r);
    }

    __device__ __forceinline__ void mfma_one(int buf, int m)
    {
        const int i = m / T::FN, j = m % T::FN;
        const f16x8 b = __builtin_bit_cast(
            f16x8, __builtin_shufflevector(bl[buf][j], bh[buf][j], 0, 1, 2, 3, 4, 5, 6, 7));
        if constexpr (T::MF == 32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, af[buf][i], acc[i][j], 0, 0, 0);
        else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, af[buf][i], acc[i][j], 0, 0, 0);
    }
};


// ---------------------------------------------------------------- epilogue ----------
// The C tile is staged in LDS (the ring is free once the K loop is done) so that the
// stores to HBM are whole rows: 16 bytes per lane, consecutive lanes on consecutive
// columns, every 128-byte line written by one instruction.  LDS layout: row-major
// BM x BN fp16 with the 16-byte chunks of each row permuted, so that the column-wise
// writes from the accumulator layout (one chunk in each of 32 consecutive rows) spread
// over the 16 bank groups, two rows per group:
//   CW (chunks per row) a power of two -- chunk c of row r at c ^ (r % CW);
//   CW % 16 == 8 -- rows start alternately at bank groups 0 and 8, so chunk c of row r
//                   goes to c ^ ((r / 2) % 8): over 16 rows, (r % 2, (r / 2) % 8) takes
//                   every value once.  The chunk stays in its aligned group of 8, so the
//                   row-wise reads of lds_to_c touch the same banks as without it.
template <class T>
__device__ __forceinline__ int c_phys(int c, int r)
{
    constexpr int CW = T::BN / 8;
    if constexpr ((CW & (CW - 1)) == 0) {
        return c ^ (r % CW);
    } else {
        static_assert(CW % 16 == 8, "C tile rows of a power-of-two number of chunks, or 8 past a multiple of 16");
        return c ^ ((r >> 1) & 7);
    }
}

// Bias, GELU and fp16 rounding of accumulator block rows I0 <= i < I1 of this wave,
// written into the LDS copy of the tile.  Accumulator layout of v_mfma_f32_32x32x16_f16
// and v_mfma_f32_16x16x32_f16 (MF = 32, 16) with the B fragment as the first operand:
// register 4 g + e of lane l holds C[MF i + l % MF][MF j + 8 g + 4 (l / MF) + e] of the
// wave's sub-tile (g < 4 for MF = 32, g = 0 for MF = 16).  bias_raw[j][g] holds the four
// bias values of this lane's columns in register quad g of block column j (loaded by
// DirectWave::load_bias at the start of the kernel).
template <class T, int I0, int I1, int EPI>
__device__ __forceinline__ void tile_to_lds(const typename T::AccT (&acc)[T::FM][T::FN],
                                            const u32x2 (&bias_raw)[T::FN][T::NG], int row0,
                                            int col0, int lane, char *ctile)
{
    const int half = lane >> T::MFS;   // the k-group of the operand map: 4-column offset
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int g = 0; g < T::NG; ++g) {
            const int n = col0 + j * T::MF + 8 * g + 4 * half;   // first of 4 columns, tile-relative
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI != 0) {
                const f16x4 h = __builtin_bit_cast(f16x4, bias_raw[j][g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = (float)h[e];
            }
            const int c = n >> 3;
#pragma unroll
            for (int i = I0; i < I1; ++i) {
                const int r = row0 + i * T::MF + (lane & (T::MF - 1));
                // built as one vector, so that each pair of halves lands in one register
                // (v_fma_mixlo_f16 / v_fma_mixhi_f16) with no shift-and-or packing
                f16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = (f16)epilogue_op<EPI>(acc[i][j][4 * g + e], bv[e]);
                // the 4 columns' place in their 16-byte chunk: bit 2 of n (= half for MF = 32)
                const int sub = T::MF == 32 ? 4 * half : (n & 4);
                char *dst = ctile + (r * T::BN + 8 * c_phys<T>(c, r) + sub) * 2;
                *reinterpret_cast<f16x4 *>(dst) = hv;
            }
        }
    }
}

// Cache policy of the C stores: sc0 | sc1 (system scope), so the lines are written through
// L2 as the epilogue produces them instead of staying dirty until the write-back at the
// end of the kernel.  Measured on MI355X: 1000x3000x777 + bias + GELU 11.76 us against
// 12.38 us with the default policy, 2048^3 + bias + GELU 20.42 against 20.62, 2048^3 and
// 8192^3 unchanged (interleaved on one box); the non-temporal hint alone did not help.
constexpr int kStoreWriteThrough = 1 | 16;

// All threads, the loader waves included: copy the LDS tile to C, 16 bytes per lane.  Rows
// past M fall outside the C descriptor's range, 8-column chunks past N are pushed out of
// range (N % 8 == 0 here, so a chunk is either wholly inside or wholly outside).
template <class T>
__device__ __forceinline__ void lds_to_c(const GemmArgs &p, int m0, int n0, int rows_valid,
                                         const char *ctile)
{
    constexpr int CW = T::BN / 8;
    constexpr int PER = T::BM * CW / T::NT;
    static_assert(T::BM * CW % T::NT == 0, "tile must split evenly over the threads");
    const int cols_valid = p.N - n0;
    const __amdgpu_buffer_rsrc_t c_rs =
        make_rsrc(p.C + (int64_t)m0 * p.ldc + n0, span_bytes(rows_valid, p.ldc, cols_valid));
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int q = threadIdx.x + k * T::NT;
        const int r = q / CW, c = q % CW;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ctile + (r * T::BN + 8 * c_phys<T>(c, r)) * 2);
        const uint32_t off = masked_offset((uint32_t)(r * p.ldc + 8 * c) * 2u, 8 * c < cols_valid);
        __builtin_amdgcn_raw_buffer_store_b128(v, c_rs, off, 0, kStoreWriteThrough);
    }
}

template <int... Is, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Is...>, F &&f)
{
    (f(std::integral_constant<int, Is>{}), ...);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for(std::make_integer_sequence<int, N>{}, f);
}

// KTAIL = false: the variant for K % 8 == 0, without the K-tail patch.
// Phase clock (diagnostic build only, MI355_PHASE_CLOCK=1): thread 0 of each workgroup
// records s_memrealtime (100 MHz) and s_memtime (shader clock cycles) at the kernel's phase
// boundaries -- 0 entry, 1 first stage landed, 2 K loop done, 3 epilogue in LDS, 4 after
// the barrier, 5 C stores issued, 6 C stores complete -- into g_phase_clock[tile][slot]
// (realtime) and [tile][8 + slot] (cycles), for the first kPhaseClockTiles workgroups.
// The regular build compiles the calls to nothing.
#ifndef MI355_PHASE_CLOCK
#define MI355_PHASE_CLOCK 0
#endif
constexpr int kPhaseClockTiles = 8192;
#if MI355_PHASE_CLOCK
__device__ unsigned long long g_phase_clock[kPhaseClockTiles * 16];
__device__ __forceinline__ void phase_stamp(int slot)
{
    if (threadIdx.x == 0 && blockIdx.x < kPhaseClockTiles) {
        g_phase_clock[blockIdx.x * 16 + slot] = __builtin_amdgcn_s_memrealtime();
        g_phase_clock[blockIdx.x * 16 + 8 + slot] = __builtin_amdgcn_s_memtime();
    }
}
#else
__device__ __forceinline__ void phase_stamp(int) {}
#endif

template <class T, int EPI, bool KTAIL>
__global__ void __launch_bounds__(T::NT) gemm_direct(GemmArgs p)
{
    phase_stamp(0);
    using St = Stage<T>;
    __shared__ __attribute__((aligned(16))) char lds_raw[T::LDS_BYTES];

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int rows_valid = min(T::BM, p.M - m0);
    const int nk = (p.K + T::BK - 1) / T::BK;

    DirectWave<T> w;
    w.init(p, m0, n0, rows_valid, p.N - n0);
    // the multiplying waves (all of them without loader waves); wave-uniform
    const bool mult = T::NL == 0 || w.wave < T::NW;
    if constexpr (EPI != 0) {
        if (mult) w.load_bias(p);
    }
    const bool k_tail = KTAIL && (p.K & 7) != 0;
    if (k_tail && nk > 0 && (T::NL == 0 || w.issuer >= 0)) w.load_tail(nk);

    St *const ring = reinterpret_cast<St *>(lds_raw);

    // One stage J of a ring turn (stage kt).  The wave runs its Q k-steps; each k-step
    // issues its MFMAs one by one, and after each MFMA a share of the LDS reads for the
    // k-step PF ahead and, in the first k-step, a share of the HBM -> LDS copy of stage
    // kt+STAGES-1 into the slot freed by stage kt-1.  k-step QB first waits for stage
    // kt+1's copy and crosses the barrier: from there on the reads run into stage kt+1, and
    // the rest of the copies follow.  The body has no branches on data; near the end of K
    // it copies zeros for the stages past the end and reads fragments it never uses.
    auto stage = [&](auto Jc, int kt, auto full_c) {
        constexpr int J = decltype(Jc)::value;
        constexpr bool FULL = decltype(full_c)::value;   // the stage copied here is below K
        St &cur = ring[J];
        St &nxt = ring[(J + 1) % T::STAGES];
        St &dst = ring[(J + T::STAGES - 1) % T::STAGES];
        static_for<T::Q>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            constexpr int buf = (J * T::Q + q) % T::NBUF;
            constexpr int rbuf = (J * T::Q + q + T::PF) % T::NBUF;   // buffer the reads fill
            constexpr bool ahead = q + T::PF >= T::Q;                // reads from stage kt+1
            constexpr int rq = (q + T::PF) % T::Q;                   // their k-step there
            if constexpr (T::Q == 1) {
                w.template issue_stage<FULL>(dst, kt + T::STAGES - 1);
            }
            if constexpr (q == T::QB) {
                // stage kt+1 has landed once at most the copies issued after it are in
                // flight (stages kt+2 .. kt+STAGES-2 and the early part of kt+STAGES-1);
                // and this wave's LDS reads have completed: every read of stage kt's slot
                // is issued before this barrier, and the copy that refills the slot only
                // after the next one, so no copy can overtake a read still queued
                wait_counts<T::VM_WAIT, 0>();
                if (k_tail && kt + 1 == nk - 1) w.patch_tail(nxt);
                workgroup_barrier();
            }
            static_for<T::NMFMA>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                w.mfma_one(buf, m);
                constexpr int r0 = m * T::NREAD / T::NMFMA;
                constexpr int r1 = (m + 1) * T::NREAD / T::NMFMA;
#pragma unroll
                for (int r = r0; r < r1; ++r) {
                    if constexpr (ahead)
                        w.read_one(nxt, rq, rbuf, r);
                    else
                        w.read_one(cur, rq, rbuf, r);
                }
                if constexpr (q == 0 && T::Q > 1) {
                    constexpr int g0 = m * T::G_EARLY / T::NMFMA;
                    constexpr int g1 = (m + 1) * T::G_EARLY / T::NMFMA;
#pragma unroll
                    for (int g = g0; g < g1; ++g) w.template issue_piece<FULL>(dst, kt + T::STAGES - 1, g);
                }
                if constexpr (q == T::QB && T::Q > 1 && T::G_EARLY < T::G) {
                    // the rest after the barrier: slot dst held stage kt-1, which no wave
                    // has read since the barrier of stage kt-1
                    constexpr int g0 = T::G_EARLY + m * (T::G - T::G_EARLY) / T::NMFMA;
                    constexpr int g1 = T::G_EARLY + (m + 1) * (T::G - T::G_EARLY) / T::NMFMA;
#pragma unroll
                    for (int g = g0; g < g1; ++g) w.template issue_piece<FULL>(dst, kt + T::STAGES - 1, g);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    // With loader waves: the multiplying waves run the stages below without copies or
    // copy waits, and the loader waves run their own loop, which crosses the same
    // barriers in the same order (the prologue's, then one per stage).  Before the
    // barrier of stage kt's k-step QB (the one after which stage kt+1 is read) a loader
    // wave waits for its copies of stage kt+1 and every multiplying wave for its LDS
    // reads, all of stage kt's slot among them; after it, the loader issues the copy of
    // stage kt+STAGES into that slot -- the order the multiplying waves keep themselves
    // without loader waves.
    auto mult_stage = [&](auto Jc, int kt) {
        constexpr int J = decltype(Jc)::value;
        St &cur = ring[J];
        St &nxt = ring[(J + 1) % T::STAGES];
        static_for<T::Q>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            constexpr int buf = (J * T::Q + q) % T::NBUF;
            constexpr int rbuf = (J * T::Q + q + T::PF) % T::NBUF;
            constexpr bool ahead = q + T::PF >= T::Q;
            constexpr int rq = (q + T::PF) % T::Q;
            if constexpr (q == T::QB) {
                // this wave's reads of stage kt's slot have completed before the loader
                // waves, past the barrier, issue the copy that refills it; stage kt+1 has
                // landed once the barrier is crossed
                wait_counts<63, 0>();
                workgroup_barrier();
            }
            static_for<T::NMFMA>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                w.mfma_one(buf, m);
                constexpr int r0 = m * T::NREAD / T::NMFMA;
                constexpr int r1 = (m + 1) * T::NREAD / T::NMFMA;
#pragma unroll
                for (int r = r0; r < r1; ++r) {
                    if constexpr (ahead)
                        w.read_one(nxt, rq, rbuf, r);
                    else
                        w.read_one(cur, rq, rbuf, r);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        });
        (void)kt;
    };

    if constexpr (T::NL > 0) {
        if (nk > 0 && mult) {
            workgroup_barrier();   // stage 0 has landed
            phase_stamp(1);
            static_for<T::PF>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                w.read_all(ring[0], q, q);
            });
            int kt = 0;
            for (; kt + T::STAGES <= nk; kt += T::STAGES)
                static_for<T::STAGES>([&](auto jc) { mult_stage(jc, kt + decltype(jc)::value); });
            if (kt < nk) {
                static_for<T::STAGES>([&](auto jc) {
                    const int k = kt + decltype(jc)::value;
                    if (k < nk) mult_stage(jc, k);
                });
            }
            phase_stamp(2);
            wait_counts<0, 0>();   // the bias loads
        } else if (nk > 0) {
            // loader wave: stages 0 .. STAGES-2 in flight, wait for stage 0
#pragma unroll
            for (int s = 0; s < T::STAGES - 1; ++s) w.issue_stage(ring[s], s);
            wait_counts<T::VM_WAIT_L, 15>();
            if (k_tail && nk == 1) w.patch_tail(ring[0]);
            workgroup_barrier();
            for (int kt = 0; kt < nk; ++kt) {
                // the slot of stage kt-1 (stage kt+STAGES-1's), free since the last barrier
                const int ks = kt + T::STAGES - 1;
                St &dst = ring[ks % T::STAGES];
                if ((ks + 1) * T::BK <= p.K)
                    w.template issue_stage<true>(dst, ks);
                else
                    w.template issue_stage<false>(dst, ks);
                wait_counts<T::VM_WAIT_L, 15>();   // stage kt+1 has landed
                if (k_tail && kt + 1 == nk - 1) w.patch_tail(ring[(kt + 1) % T::STAGES]);
                workgroup_barrier();
            }
            wait_counts<0, 0>();   // no copy outlives the kernel
        }
    } else if (nk > 0) {
        // ---- prologue: stages 0 .. STAGES-2 in flight, wait for stage 0 ----
#pragma unroll
        for (int s = 0; s < T::STAGES - 1; ++s) w.issue_stage(ring[s], s);
        wait_counts<T::G * (T::STAGES - 2), 15>();
        if (k_tail && nk == 1) w.patch_tail(ring[0]);
        workgroup_barrier();
        phase_stamp(1);
        static_for<T::PF>([&](auto qc) {   // the first PF k-steps of stage 0
            constexpr int q = decltype(qc)::value;
            w.read_all(ring[0], q, q);
        });

        // ---- main loop, unrolled over the ring so every slot address is a constant.
        // The last ring turn stops at the end of K (a branch on a workgroup-uniform
        // value); the copies and fragment reads the last stage issued for the stages
        // after it read zeros and are never used.
        // Whole ring turns whose copies (up to stage kt + 2*STAGES - 2) all lie below K
        // take the copy without the K mask; the turns after them the general one.
        int kt = 0;
        for (; (kt + 2 * T::STAGES - 1) * T::BK <= p.K; kt += T::STAGES)
            static_for<T::STAGES>([&](auto jc) { stage(jc, kt + decltype(jc)::value, std::true_type{}); });
        for (; kt < nk; kt += T::STAGES) {
            static_for<T::STAGES>([&](auto jc) {
                const int k = kt + decltype(jc)::value;
                if (k < nk) stage(jc, k, std::false_type{});
            });
        }
        phase_stamp(2);
        // the copies past the end of K are still landing; none may outlive the kernel
        // (and with k-groups the ring is reused below)
        wait_counts<0, 0>();
    }

    // every wave is done reading the ring (and, above, its copies have all landed)
    workgroup_barrier();
    char *ctile = lds_raw;
    if constexpr (T::KGROUPS == 1) {
        if (mult)
            tile_to_lds<T, 0, T::FM, EPI>(w.acc, w.bias_raw, w.wm * T::WTM, w.wn * T::WTN, w.lane, ctile);
    } else {
        // Sum the two k-groups' partial tiles.  Group 0 keeps blocks i < FM/2 and hands
        // blocks i >= FM/2 to group 1; group 1 does the opposite; each then finishes the
        // half it kept.  Each 32x32 fp32 block moves as four 1 KiB ds_write_b128 /
        // ds_read_b128 (lane-contiguous, conflict-free).  The exchange runs in three
        // phases (write, read and add, epilogue) separated by barriers that every wave
        // reaches at the same point of the program; only the register halves a phase
        // touches depend on the group (block indices must be compile-time constants).
        constexpr int H = T::FM / 2;
        float *red = reinterpret_cast<float *>(lds_raw);
        const int wc = w.wave % T::NWC;
        // slot of (group, wave-in-group, block) in the exchange area; the receiving wave of
        // the other group reads the slot its partner wrote
        auto slot_ptr = [&](int grp, int ii, int j, int c) {
            return red + ((((grp * T::NWC + wc) * H + ii) * T::FN + j) * 4 + c) * 256 + w.lane * 4;
        };
        auto give = [&](auto give_c) {
            constexpr int GIVE = decltype(give_c)::value;
#pragma unroll
            for (int ii = 0; ii < H; ++ii)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const f32x16 &v = w.acc[GIVE + ii][j];
                        *reinterpret_cast<f32x4 *>(slot_ptr(w.kg, ii, j, c)) =
                            f32x4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
                    }
        };
        auto take = [&](auto keep_c) {
            constexpr int KEEP = decltype(keep_c)::value;
#pragma unroll
            for (int ii = 0; ii < H; ++ii)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const f32x4 o = *reinterpret_cast<const f32x4 *>(slot_ptr(1 - w.kg, ii, j, c));
#pragma unroll
                        for (int e = 0; e < 4; ++e) w.acc[KEEP + ii][j][4 * c + e] += o[e];
                    }
        };
        using Zero = std::integral_constant<int, 0>;
        using Half = std::integral_constant<int, H>;
        if (w.kg == 0) give(Half{}); else give(Zero{});
        __syncthreads();
        if (w.kg == 0) take(Zero{}); else take(Half{});
        __syncthreads();   // the exchange area is overwritten by the C tile below
        if (w.kg == 0)
            tile_to_lds<T, 0, H, EPI>(w.acc, w.bias_raw, w.wm * T::WTM, w.wn * T::WTN, w.lane, ctile);
        else
            tile_to_lds<T, H, T::FM, EPI>(w.acc, w.bias_raw, w.wm * T::WTM, w.wn * T::WTN, w.lane, ctile);
    }
    phase_stamp(3);
    __syncthreads();
    phase_stamp(4);
    lds_to_c<T>(p, m0, n0, rows_valid, ctile);
    if constexpr (MI355_PHASE_CLOCK != 0) {
        phase_stamp(5);
        if (threadIdx.x == 0) wait_counts<0, 0>();   // this thread's C stores complete
        phase_stamp(6);
    }
}

}  // namespace mi355

// Attention forward for gfx950, the tutorial's FlashAttention ("Designing High-Performance
// GPU Kernels with TileLang: ...", ainovat.com page, the FlashAttention paragraph: query,
// key and value tiles processed without writing the score matrix to memory, an online
// softmax with running maxima, sums and rescaling, tiled tensor-core products, causal and
// non-causal).
//
// For every (batch, head) pair and query row i:
//   s_j = scale * q_i . k_j  over the allowed keys j (all Sk keys, or j <= i when causal:
//         the upper-left aligned mask), o_i = sum_j softmax(s)_j v_j,  lse_i = log sum_j exp(s_j)
// q (Sq x D), k and v (Sk x D), o (Sq x D) fp16 row-major per pair, pairs one after
// another; fp32 arithmetic, weights rounded to fp16 for the value product (as the tensor
// cores take them), one rounding of o to fp16.
//
// One workgroup of NW wavefronts takes BM = 32 NW query rows of one pair; each wave owns
// 32 rows for the whole kernel, its Q fragments in registers.  Key/value blocks of BN
// rows stream HBM -> LDS by LDS-DMA (buffer_load ... lds) into a ring of STAGES slots
// shared by the waves; per block each wave computes
//   S^T = K Q^T   with v_mfma_f32_32x32x16_f16, K as the first operand, so lane l holds
//                 the scores of query row l % 32 for 16 of the 32 keys of each 32-key
//                 block (its partner lane l ^ 32 holds the other 16);
//   the online softmax in registers (base 2: exp(x) = 2^(x log2 e), scale folded in,
//                 c = scale * log2 e): P = 2^(S c - m), l = l + rowsum(P), O = O + P V
//                 against a reference m per row.  Any m gives the same o = O / l as long
//                 as O and l share it; m is raised (O and l scaled by 2^(m - m')) only
//                 when some row of the wave sees a block maximum more than 8 above it, so
//                 weights stay at most 2^8 (exact range for fp16 and fp32) and the
//                 rescale of O is skipped for most blocks.  The row maximum needs one
//                 exchange with the partner lane, the sum none (each lane keeps its
//                 partial sum, added at the end);
//   O^T += V^T P^T  with V as the first operand read by ds_read_b64_tr_b16 (the
//                 transposing LDS read) and P^T straight from the score registers: the
//                 keys a lane holds define the order of the contraction, and the V
//                 read is pointed at the same keys.
// Out-of-range keys read as zero (buffer range checks) and their scores are set to -inf;
// causal blocks wholly above a wave's rows are skipped by that wave.
#pragma once

#include "gemm_direct.hpp"

namespace mi355 {

struct AttnArgs {
    const f16 *q;
    const f16 *k;
    const f16 *v;
    f16 *o;
    float *lse;      // may be null
    int pairs;       // batch * heads
    int Sq, Sk;
    int q_blocks;    // ceil(Sq / BM)
    float c;         // scale * log2(e), > 0
    int causal;
};

template <int D_, int BN_, int NW_, int STAGES_>
struct ATile {
    static constexpr int D = D_, BN = BN_, NW = NW_, STAGES = STAGES_;
    static constexpr int BM = 32 * NW, NT = 64 * NW;
    static constexpr int KK = D / 16;     // 16-deep k-steps of Q K^T
    static constexpr int NB = BN / 32;    // 32-key score blocks per key block
    static constexpr int U = BN / 16;     // 16-key k-steps of P V
    static constexpr int DB = D / 32;     // 32-wide output column blocks
    static constexpr int CH = D / 8;      // 16-byte chunks per K / V row
    static constexpr int KV_BYTES = BN * D * 2;
    static constexpr int STAGE_BYTES = 2 * KV_BYTES;   // K block, then V block
    static constexpr int GK = KV_BYTES / (1024 * NW);  // 1 KiB LDS-DMA loads per wave per block
    static constexpr int G = 2 * GK;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    static_assert(BN % 32 == 0, "key block of whole 32-key score blocks");
    static_assert(KV_BYTES % (1024 * NW) == 0, "block must split into whole 1 KiB loads per wave");
    static_assert(STAGES >= 2 && G * (STAGES - 2) <= 63, "ring size / vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "over the gfx950 LDS budget");
};

// K block: row-major BN x D; 16-byte chunk c of row r sits at chunk c ^ swz_k(r), so the
// 16 rows one ds_read_b128 pass touches (same logical chunk) land in 16 distinct bank
// groups.  RP rows share one 256-byte bank window.
template <int CH>
__device__ __forceinline__ int attn_swz_k(int row)
{
    constexpr int RP = 16 / CH;
    return (row / RP) % CH;
}

// V block: row-major BN x D; a transposing read touches 4 consecutive rows (starting at a
// multiple of 4) x 4 chunks per half-wave.  Rows of 256 bytes (D = 128) fill a bank
// window each: XOR chunk bits 2-3 with row % 4.  Rows of 128 bytes (D = 64) pair up in a
// window: XOR chunk bit 2 with bit 1 of the row.
template <int CH>
__device__ __forceinline__ int attn_swz_v(int row)
{
    return CH >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

template <class T>
__global__ void __launch_bounds__(T::NT) attention_fwd(AttnArgs p)
{
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    constexpr int D = T::D, BN = T::BN, CH = T::CH;
    constexpr float kNegInf = -__builtin_inff();
    constexpr float kRescaleLog2 = 8.0f;   // weights stay below 2^8 between rescales

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, r32 = lane & 31, i16 = lane & 15;

    // Work order: workgroups go to the 8 XCDs round-robin; renumber them so each XCD owns
    // a contiguous range of (pair, query block) items, the blocks of a few pairs, whose
    // keys and values then stay in that XCD's L2.  Inside the range the items go in groups
    // of two pairs, heaviest query block first (the last one, when causal) alternating
    // between the two pairs, so the longest workgroups start first and the short ones fill
    // the tail (9% on causal attention at 4096 tokens; no change without the mask).
    int pair, qb;
    {
        constexpr int PG = 2;   // pairs per group
        const int total = p.pairs * p.q_blocks;
        const int bid = blockIdx.x;
        const int xcd = bid & 7, idx = bid >> 3, per = total >> 3, rem = total & 7;
        const int lid = (xcd < rem) ? xcd * (per + 1) + idx
                                    : rem * (per + 1) + (xcd - rem) * per + idx;
        const int gsz = PG * p.q_blocks;
        const int grp = lid / gsz, t = lid - grp * gsz;
        const int npair = min(PG, p.pairs - grp * PG);   // the last group may hold one pair
        pair = grp * PG + t % npair;
        qb = p.q_blocks - 1 - t / npair;
    }
    const int q0 = qb * T::BM;
    const int qw = q0 + 32 * wave;   // this wave's first query row
    const int qi = qw + r32;         // this lane's query row

    const int64_t pq = (int64_t)pair * p.Sq * D, pk = (int64_t)pair * p.Sk * D;
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(p.q + pq, (uint32_t)p.Sq * D * 2u);
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + pk, (uint32_t)p.Sk * D * 2u);
    const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + pk, (uint32_t)p.Sk * D * 2u);

    // the keys this workgroup's valid rows can see
    const int kv_end = p.causal ? min(p.Sk, min(p.Sq, q0 + T::BM)) : p.Sk;
    const int n_kv = (kv_end + BN - 1) / BN;

    // ---- LDS-DMA sources: slot s of a block holds row s / CH, physical chunk s % CH ----
    uint32_t k_off[T::GK], v_off[T::GK];
#pragma unroll
    for (int g = 0; g < T::GK; ++g) {
        const int s = (g * T::NW + wave) * 64 + lane;
        const int row = s / CH, pc = s % CH;
        k_off[g] = (uint32_t)(row * D + 8 * (pc ^ attn_swz_k<CH>(row))) * 2u;
        v_off[g] = (uint32_t)(row * D + 8 * (pc ^ attn_swz_v<CH>(row))) * 2u;
    }
    // Block j into ring slot `slot`.  Rows past Sk (and whole blocks past the end, issued
    // to keep the counter arithmetic uniform) fall outside the descriptors and read zero.
    auto issue_block = [&](int slot, int j) {
        const uint32_t base = (uint32_t)(j * BN) * D * 2u;
        char *kdst = lds + slot * T::STAGE_BYTES;
#pragma unroll
        for (int g = 0; g < T::GK; ++g)
            lds_dma16(k_rs, kdst + (g * T::NW + wave) * 1024, base + k_off[g]);
#pragma unroll
        for (int g = 0; g < T::GK; ++g)
            lds_dma16(v_rs, kdst + T::KV_BYTES + (g * T::NW + wave) * 1024, base + v_off[g]);
    };

    // ---- Q fragments (second operand of Q K^T): row qi, columns 16 kk + 8 h .. +7 ----
    f16x8 qf[T::KK];
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk)
        qf[kk] = __builtin_bit_cast(
            f16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, (uint32_t)(qi * D + 16 * kk + 8 * h) * 2u, 0, 0));

    // ---- fragment read addresses (byte offsets inside a ring slot) ----
    // K (first operand): key row nb*32 + r32, logical chunk 2 kk + h.  The swizzle depends
    // on the row only through r32.
    int k_addr[T::KK];
    {
        const int sw = attn_swz_k<CH>(r32);
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) k_addr[kk] = r32 * D * 2 + ((2 * kk + h) ^ sw) * 16;
    }
    // V (first operand, transposing read): lane i of each 16-lane group points at row i / 4
    // of a 4-row band and at columns 4 (i % 4) .. +3 of its 16-column half; lane j then
    // receives V[band + 0..3][half + j].  For the 16-key step u the bands are
    // 16 u + 4 h (+8), the keys the score registers 8t .. 8t+7 of this lane hold.
    int v_addr[T::DB];
    {
        const int sw = CH >= 16 ? 4 * (i16 >> 2) : 4 * ((i16 >> 3) & 1);   // attn_swz_v of the row
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
            const int d = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
            v_addr[db] = T::KV_BYTES + (4 * h + (i16 >> 2)) * D * 2 + (((d >> 3) ^ sw) * 16) + 8 * ((d >> 2) & 1);
        }
    }

    f32x16 o[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db) o[db] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;

    // ---- prologue: blocks 0 .. STAGES-2 in flight ----
#pragma unroll
    for (int s = 0; s < T::STAGES - 1; ++s) issue_block(s, s);

    auto step = [&](auto Jc, int j) {
        constexpr int J = decltype(Jc)::value;
        // block j has landed once at most STAGES-2 later blocks are in flight (the Q loads
        // were issued first and are done too); the barrier also ends every wave's reads of
        // the slot block j+STAGES-1 goes into
        wait_counts<T::G * (T::STAGES - 2), 15>();
        workgroup_barrier();
        issue_block((J + T::STAGES - 1) % T::STAGES, j + T::STAGES - 1);

        const int kv0 = j * BN;
        if (p.causal && kv0 > qw + 31) return;   // every key of the block is above this wave's rows
        const char *slot = lds + J * T::STAGE_BYTES;

        // S^T = K Q^T
        f32x16 s[T::NB];
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) s[nb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb) {
                const f16x8 kf = *reinterpret_cast<const f16x8 *>(slot + nb * 32 * D * 2 + k_addr[kk]);
                s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[kk], s[nb], 0, 0, 0);
            }

        // register r of s[nb] is key kv0 + 4 h + off(nb, r), off = 32 nb + 8 (r / 4) + r % 4,
        // of query row qi; keys from kv0 + 4 h + lim on are past Sk or, when causal, past qi
        if (kv0 + BN > p.Sk || (p.causal && kv0 + BN - 1 > qw)) {
            const int lim = (p.causal ? min(p.Sk, qi + 1) : p.Sk) - kv0 - 4 * h;
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 32 * nb + 8 * (r >> 2) + (r & 3);
                    s[nb][r] = (off >= lim) ? kNegInf : s[nb][r];
                }
        }

        // online softmax, base 2
        float mx = kNegInf;
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // raise the reference when a row's maximum passes it by more than 2^8 (always in
        // the first block, where it is -inf; key 0 makes every row's first maximum finite)
        float alpha = 1.0f;
        const bool resc = __any(mx * p.c > m_run + kRescaleLog2);
        if (resc) {
            const float m_new = fmaxf(m_run, mx * p.c);
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
        }
        float rs = 0.0f;
        f16x8 pf[T::U];
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(fmaf(s[nb][r], p.c, -m_run));
                rs += e;
                pf[2 * nb + (r >> 3)][r & 7] = (f16)e;
            }
        if (resc) {
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }

        // O^T += V^T P^T
#pragma unroll
        for (int u = 0; u < T::U; ++u)
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const char *a = slot + u * 16 * D * 2 + v_addr[db];
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)lds_ptr(a));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)lds_ptr(a + 8 * D * 2));
                const f16x8 vf = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[u], o[db], 0, 0, 0);
            }
        l_run += rs;
    };

    for (int jb = 0; jb < n_kv; jb += T::STAGES) {
        static_for<T::STAGES>([&](auto jc) {
            const int j = jb + decltype(jc)::value;
            if (j < n_kv) step(jc, j);
        });
    }
    // the copies issued past the last block are still landing; none may outlive the kernel
    wait_counts<0, 0>();

    // ---- o = O / l, one rounding; register r of o[db] is column 32 db + 8 (r / 4) + 4 h + r % 4 ----
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(p.o + pq, (uint32_t)p.Sq * D * 2u);
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t hb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) hb[e] = __builtin_bit_cast(uint16_t, (f16)(o[db][4 * g + e] * inv));
            const int d = 32 * db + 8 * g + 4 * h;
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)}, o_rs,
                                                  (uint32_t)(qi * D + d) * 2u, 0, 0);
        }
    if (p.lse != nullptr && h == 0 && qi < p.Sq) {
        constexpr float kLn2 = 0.69314718055994531f;
        p.lse[(int64_t)pair * p.Sq + qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

}  // namespace mi355

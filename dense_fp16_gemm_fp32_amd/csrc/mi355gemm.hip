// C ABI of the gfx950 fp16 GEMM library: argument validation, the shape-keyed
// configuration selector and the kernel launches.  The operation and the conventions
// are documented in include/mi355gemm.h.
#include "mi355gemm.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attention.hpp"
#include "gemm_direct.hpp"
#include "gemm_narrow.hpp"
#include "gemm_pingpong.hpp"
#include "gemm_staged.hpp"
#include "softmax.hpp"
#include "vector_add.hpp"

namespace mi355 {
// direct-to-LDS tiles: BM, BN, BK, waves (M x N), k-groups, LDS stages
using D256 = DTile<256, 256, 32, 2, 4, 1, 4>;       // 8 waves of 128x64, 128 KiB LDS
using D256k64 = DTile<256, 256, 64, 2, 4, 1, 2>;    // 8 waves of 128x64, 128 KiB
using D256x128 = DTile<256, 128, 64, 2, 2, 2, 3>;   // 2 x 4 waves of 128x64, 144 KiB
using D128 = DTile<128, 128, 64, 2, 2, 2, 4>;       // 2 x 4 waves of 64x64, 128 KiB
using D128w4 = DTile<128, 128, 64, 2, 2, 1, 4>;     // 4 waves of 64x64, 128 KiB
using D256w4 = DTile<256, 256, 32, 2, 2, 1, 4>;     // 4 waves of 128x128, 128 KiB
using D128k32 = DTile<128, 128, 32, 2, 2, 1, 4>;    // 4 waves of 64x64, 64 KiB
using D128w8 = DTile<128, 128, 64, 2, 4, 1, 4>;     // 8 waves of 64x32, 128 KiB
using D64x256 = DTile<64, 256, 32, 1, 4, 1, 4>;     // 4 waves of 64x64, 80 KiB
using D64x128 = DTile<64, 128, 32, 1, 4, 1, 4>;     // 4 waves of 64x32, 40 KiB
using D64x192 = DTile<64, 192, 32, 2, 2, 1, 4>;     // 4 waves of 32x96, 64 KiB
using D128L4 = DTile<128, 128, 64, 2, 2, 1, 4, 1, 4>;   // 4 waves of 64x64 + 4 loader waves
using D64x192L4 = DTile<64, 192, 32, 2, 2, 1, 4, 1, 4>; // 4 waves of 32x96 + 4 loader waves
using D128k32L4 = DTile<128, 128, 32, 2, 2, 1, 4, 1, 4>; // the same on a 64 KiB ring
using D64x192FL4 = DTile<64, 192, 32, 1, 4, 1, 4, 1, 4, 16>;  // 4 waves of 64x48 (16x16 blocks) + 4 loaders
using D64x192FbL4 = DTile<64, 192, 64, 1, 4, 1, 3, 1, 4, 16>; // the same on 64-deep stages, 96 KiB
// ping-pong tile: BM, BN, BK, waves of a group (M x N), stages
using P256 = PTile<256, 256, 32, 1, 4, 4>;          // 2 groups x 4 waves of 128x64, 128 KiB
// attention: head dim, keys per block, waves (32 query rows each), LDS stages
using A128 = ATile<128, 128, 8, 2>;  // 256 query rows, 128-key blocks, 128 KiB LDS
using A64 = ATile<64, 64, 8, 3>;     // 256 query rows, 64-key blocks, 48 KiB LDS
// register-staged tiles (any alignment)
using T64 = Tile<64, 64, 64, 2, 1>;              // 2 waves of 32x64
using T128 = Tile<128, 128, 64, 2, 2>;           // 4 waves of 64x64
using T256 = Tile<256, 256, 64, 2, 2>;           // 4 waves of 128x128

// Explicit instantiations: every kernel the configuration table points at gets a host
// launch stub.
#define MI355_DIRECT(T)                                          \
    template __global__ void gemm_direct<T, 0, false>(GemmArgs); \
    template __global__ void gemm_direct<T, 1, false>(GemmArgs); \
    template __global__ void gemm_direct<T, 2, false>(GemmArgs); \
    template __global__ void gemm_direct<T, 0, true>(GemmArgs);  \
    template __global__ void gemm_direct<T, 1, true>(GemmArgs);  \
    template __global__ void gemm_direct<T, 2, true>(GemmArgs);
MI355_DIRECT(D256)
MI355_DIRECT(D256k64)
MI355_DIRECT(D256x128)
MI355_DIRECT(D128)
MI355_DIRECT(D128w4)
MI355_DIRECT(D256w4)
MI355_DIRECT(D128k32)
MI355_DIRECT(D128w8)
MI355_DIRECT(D64x256)
MI355_DIRECT(D64x128)
MI355_DIRECT(D64x192)
MI355_DIRECT(D128L4)
MI355_DIRECT(D64x192L4)
MI355_DIRECT(D128k32L4)
MI355_DIRECT(D64x192FL4)
MI355_DIRECT(D64x192FbL4)
#undef MI355_DIRECT
#define MI355_PINGPONG(T)                                     \
    template __global__ void gemm_pingpong<T, 0>(GemmArgs);   \
    template __global__ void gemm_pingpong<T, 1>(GemmArgs);   \
    template __global__ void gemm_pingpong<T, 2>(GemmArgs);
MI355_PINGPONG(P256)
#undef MI355_PINGPONG
#define MI355_NARROW(KS)                                   \
    template __global__ void gemm_narrow<0, KS>(GemmArgs); \
    template __global__ void gemm_narrow<1, KS>(GemmArgs); \
    template __global__ void gemm_narrow<2, KS>(GemmArgs);
MI355_NARROW(4)
MI355_NARROW(1)
#undef MI355_NARROW
}  // namespace mi355

namespace {

using namespace mi355;

thread_local char g_last_error[512] = "";

mi355gemm_status fail(mi355gemm_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

typedef void (*KernelFn)(GemmArgs);

struct Config {
    const char *name;
    bool direct;      // direct-to-LDS kernel (16-byte operands) or register-staged kernel
    int bm, bn, bk, stages, waves_m, waves_n, k_groups, threads, lds_bytes;
    bool a_vec, bc_vec;
    int group_m;
    KernelFn fn[2][3];   // [K % 8 != 0][epilogue]
    bool narrow;      // vector-ALU kernel for at most bn (8) columns
    bool k_mult8;     // needs K % 8 == 0 (no kernel for the K-tail case)
    bool pingpong;    // two wave groups taking turns
    int loaders;      // extra waves issuing every HBM -> LDS copy (direct kernel), else 0
    int mfma_block;   // MFMA block edge: 32 (32x32x16) or 16 (16x16x32); 0 for the narrow kernel
};

template <class T, bool AV, bool BV>
Config staged_config(const char *name, int group_m)
{
    return Config{name, false, T::BM, T::BN, T::BK, T::STAGES, T::WAVES_M, T::WAVES_N, 1, T::NT,
                  T::LDS_BYTES, AV, BV, group_m,
                  {{gemm_staged<T, AV, BV, 0>, gemm_staged<T, AV, BV, 1>, gemm_staged<T, AV, BV, 2>},
                   {gemm_staged<T, AV, BV, 0>, gemm_staged<T, AV, BV, 1>, gemm_staged<T, AV, BV, 2>}},
                  false, false, false, 0, 32};
}

template <class T>
Config direct_config(const char *name, int group_m)
{
    return Config{name, true, T::BM, T::BN, T::BK, T::STAGES, T::WAVES_M, T::WAVES_N, T::KGROUPS,
                  T::NT,
                  T::LDS_BYTES, false, true, group_m,
                  {{gemm_direct<T, 0, false>, gemm_direct<T, 1, false>, gemm_direct<T, 2, false>},
                   {gemm_direct<T, 0, true>, gemm_direct<T, 1, true>, gemm_direct<T, 2, true>}},
                  false, false, false, T::NL, T::MF};
}

// Two groups of four waves taking turns; K % 8 == 0 only (no K-tail patch)
template <class T>
Config pingpong_config(const char *name, int group_m)
{
    return Config{name, true, T::BM, T::BN, T::BK, T::STAGES, 2 * T::WM, T::WN, 1,
                  T::NT, T::LDS_BYTES, false, true, group_m,
                  {{gemm_pingpong<T, 0>, gemm_pingpong<T, 1>, gemm_pingpong<T, 2>},
                   {nullptr, nullptr, nullptr}},
                  false, true, true, 0, 32};
}

// Up to 8 columns; 4 waves per workgroup, KS of them splitting K for each 8-row group
template <int KS>
Config narrow_config(const char *name)
{
    using T = Narrow<KS>;
    return Config{name, false, T::BM, T::NC, T::KB, 1, T::RG, 1, KS, T::NT,
                  KS > 1 ? (int)(T::NW * 64 * sizeof(float)) : 0, false, false, 1,
                  {{gemm_narrow<0, KS>, gemm_narrow<1, KS>, gemm_narrow<2, KS>},
                   {gemm_narrow<0, KS>, gemm_narrow<1, KS>, gemm_narrow<2, KS>}},
                  true, false, false, 0, 0};
}

const Config kConfigs[] = {
    direct_config<D256>("d256x256x32_w2x4_s4", 4),
    direct_config<D256k64>("d256x256x64_w2x4_s2", 4),
    direct_config<D256x128>("d256x128x64_w2x2k2_s3", 8),
    direct_config<D128>("d128x128x64_w2x2k2_s4", 8),
    direct_config<D128w4>("d128x128x64_w2x2_s4", 8),
    direct_config<D256w4>("d256x256x32_w2x2_s4", 4),
    direct_config<D128k32>("d128x128x32_w2x2_s4", 8),
    direct_config<D128w8>("d128x128x64_w2x4_s4", 8),
    direct_config<D64x256>("d64x256x32_w1x4_s4", 8),
    direct_config<D64x128>("d64x128x32_w1x4_s4", 8),
    direct_config<D64x192>("d64x192x32_w2x2_s4", 8),
    direct_config<D128L4>("d128x128x64_w2x2_l4_s4", 8),
    direct_config<D64x192L4>("d64x192x32_w2x2_l4_s4", 8),
    direct_config<D128k32L4>("d128x128x32_w2x2_l4_s4", 8),
    direct_config<D64x192FL4>("d64x192x32_w1x4_l4_s4_mf16", 8),
    direct_config<D64x192FbL4>("d64x192x64_w1x4_l4_s3_mf16", 8),
    pingpong_config<P256>("p256x256x32_w2x4_s4", 4),
    staged_config<T256, true, true>("s256x256x64_w2x2_av_bv", 8),
    staged_config<T128, true, true>("s128x128x64_w2x2_av_bv", 8),
    staged_config<T128, true, false>("s128x128x64_w2x2_av_bn", 8),
    staged_config<T128, false, true>("s128x128x64_w2x2_an_bv", 8),
    staged_config<T128, false, false>("s128x128x64_w2x2_an_bn", 8),
    staged_config<T64, true, true>("s64x64x64_w2x1_av_bv", 8),
    staged_config<T64, true, false>("s64x64x64_w2x1_av_bn", 8),
    staged_config<T64, false, true>("s64x64x64_w2x1_an_bv", 8),
    staged_config<T64, false, false>("s64x64x64_w2x1_an_bn", 8),
    narrow_config<4>("n8x8x512_w1x1k4"),
    narrow_config<1>("n32x8x512_w4x1"),
};
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));

constexpr int kLdsBudget = 160 * 1024;
// Per-tile buffer descriptors hold 32-bit byte offsets below 2^31: BM*K, BK*N and BM*N
// halves must stay under 2^30, so K and N are capped at 2^22.
constexpr int64_t kMaxKN = (int64_t)1 << 22;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Request {
    int64_t M, N, K;
    const void *A, *B, *bias;
    void *C;
    int epi;
};

// Validation shared by every entry point; makes no HIP call.
mi355gemm_status validate(const Request &r)
{
    if (r.M < 0 || r.N < 0 || r.K < 0)
        return fail(MI355GEMM_EINVAL, "negative size (M=%lld N=%lld K=%lld)",
                    (long long)r.M, (long long)r.N, (long long)r.K);
    if (r.epi < MI355GEMM_EPI_NONE || r.epi > MI355GEMM_EPI_BIAS_GELU)
        return fail(MI355GEMM_EINVAL, "unknown epilogue %d", r.epi);
    if (r.M == 0 || r.N == 0) return MI355GEMM_OK;
    if (r.C == nullptr) return fail(MI355GEMM_EINVAL, "C is NULL");
    if (r.K > 0 && (r.A == nullptr || r.B == nullptr))
        return fail(MI355GEMM_EINVAL, "A or B is NULL with K=%lld", (long long)r.K);
    if (r.epi != MI355GEMM_EPI_NONE && r.bias == nullptr)
        return fail(MI355GEMM_EINVAL, "epilogue %d needs a bias pointer", r.epi);
    if (!aligned(r.C, 2) || (r.K > 0 && (!aligned(r.A, 2) || !aligned(r.B, 2))) ||
        (r.epi != MI355GEMM_EPI_NONE && !aligned(r.bias, 2)))
        return fail(MI355GEMM_EINVAL, "fp16 pointers must be 2-byte aligned");
    if (r.K >= kMaxKN || r.N >= kMaxKN)
        return fail(MI355GEMM_EUNSUPPORTED, "K and N must be below 2^22 (K=%lld N=%lld)",
                    (long long)r.K, (long long)r.N);
    if (r.M >= ((int64_t)1 << 31))
        return fail(MI355GEMM_EUNSUPPORTED, "M must be below 2^31");
    return MI355GEMM_OK;
}

bool a_vector_ok(const Request &r) { return r.K % 8 == 0 && (r.K == 0 || aligned(r.A, 16)); }

bool bc_vector_ok(const Request &r)
{
    return r.N % 8 == 0 && aligned(r.C, 16) && (r.K == 0 || aligned(r.B, 16)) &&
           (r.epi == MI355GEMM_EPI_NONE || aligned(r.bias, 8));
}

int64_t tiles(const Request &r, int bm, int bn)
{
    return ((r.M + bm - 1) / bm) * ((r.N + bn - 1) / bn);
}

int find_narrow(int k_groups)
{
    for (int i = 0; i < kNumConfigs; ++i)
        if (kConfigs[i].narrow && kConfigs[i].k_groups == k_groups) return i;
    return -1;
}

// Narrow variant for M rows (interleaved timings on MI355X, N = 1..8 and the last N % 8
// columns of odd N): from 16384 rows the 4 waves on 4 row groups win (K = 4096: 39 us
// against 47; 131072 x 512: 50 against 175), below it the 4 waves splitting K of 8 rows
// (1024 x 65536: 62 us against 222).
int narrow_for(int64_t M) { return find_narrow(M >= 16384 ? 1 : 4); }

int find_staged(int bm, int bn, bool av, bool bv)
{
    for (int i = 0; i < kNumConfigs; ++i) {
        const Config &c = kConfigs[i];
        if (!c.direct && !c.narrow && c.bm == bm && c.bn == bn && c.a_vec == av && c.bc_vec == bv) return i;
    }
    return -1;
}

int find_pingpong(int bm, int bn)
{
    for (int i = 0; i < kNumConfigs; ++i)
        if (kConfigs[i].pingpong && kConfigs[i].bm == bm && kConfigs[i].bn == bn) return i;
    return -1;
}

int find_direct(int bm, int bn, int bk, int waves, int k_groups, int loaders = 0, int mfma = 32)
{
    for (int i = 0; i < kNumConfigs; ++i) {
        const Config &c = kConfigs[i];
        if (c.direct && !c.pingpong && c.bm == bm && c.bn == bn && c.bk == bk &&
            c.waves_m * c.waves_n * c.k_groups == waves && c.k_groups == k_groups &&
            c.loaders == loaders && c.mfma_block == mfma)
            return i;
    }
    return -1;
}

// Can configuration c serve request r?  (Silent version of check_config.)
bool config_fits(const Config &c, const Request &r)
{
    return c.lds_bytes <= kLdsBudget && (!c.a_vec || a_vector_ok(r)) && (!c.bc_vec || bc_vector_ok(r)) &&
           (!c.narrow || r.N <= c.bn) && (!c.k_mult8 || r.K % 8 == 0);
}

// Measured winners for exact shapes, written by the package's tune.py (an interleaved
// sweep over the forced configurations); an entry exists only where the winner beat the
// rules below by the tuner's margin.
struct TunedEntry {
    int64_t M, N, K;
    int epi, a_vec, bc_vec;
    const char *config;
};
const TunedEntry kTuned[] = {
#include "tuned_table.inc"
    {0, 0, 0, -1, 0, 0, nullptr},   // end marker (keeps the array non-empty)
};

int tuned_choice(const Request &r, bool av, bool bv)
{
    for (const TunedEntry &t : kTuned) {
        if (t.config == nullptr) break;
        if (t.M != r.M || t.N != r.N || t.K != r.K || t.epi != r.epi || t.a_vec != (int)av ||
            t.bc_vec != (int)bv)
            continue;
        for (int i = 0; i < kNumConfigs; ++i)
            if (strcmp(kConfigs[i].name, t.config) == 0 && config_fits(kConfigs[i], r)) return i;
    }
    return -1;
}

// Shape-keyed choice (host only), from interleaved timings of the candidates on several
// MI355X boxes.  A launch should cover the 256 compute units; among the tiles that do,
// the largest wins (fewer bytes per flop from L2 into LDS).  With every CU busy the part
// runs at its power limit.  From one full wave of 256x256 tiles on, the ping-pong kernel
// (two groups of 4 waves taking turns) leads the other 256x256 tiles by 0-1.5% (8192^3
// with and without bias + GELU, 4096^3); it needs K % 8 == 0.  Otherwise: 256x256x32
// tiles on 4 waves of 128x128 from four full waves of them, 256x256x64 tiles (8 waves, 2
// stages) from one, 256x256x32 tiles on 8 waves where 256x128 tiles would need more than
// one round, 256x128 tiles with two k-groups where they fill exactly one or where 128x128
// tiles would need a partial second round;
// where at most one wave of 128x128 tiles remains,
// 64-row tiles (64x192 where a full wave of them fills the chip with K up to 2048, 64x256
// for short K, 64x128 where 128x128 tiles would idle half the chip),
// else 128x128 tiles: 4 multiplying waves fed by 4 loader waves when they fill the chip,
// two k-groups with part of the chip idle (two waves per SIMD hide each other's LDS reads
// and barrier waits).  The 4-wave tiles took over
// (256x256 at 8192^3) or kept (128x128 at 2048^3) their shapes once the copies lost their
// vector instructions: with one wave per SIMD nothing else hid them.
// The 256x256x64 tile took over one wave of big tiles from the 256x256x32 one once the
// K-tail patch moved into its own kernel variant (the 64-deep tile had spilled registers
// before).  At 2048^3 the two 128x128 tiles trade places from box to box; the 4-wave one
// is faster on average and its spread is far smaller (20.6-21.7 us against 19.7-23.8
// over four boxes).  The register-staged kernels take
// small problems and those whose B or C rows are not 16-byte friendly (the direct kernels
// need N % 8 == 0 and 16-byte aligned B and C; A may have any alignment).
// Choices installed by the caller at run time (mi355gemm_set_choice), for example from
// timings on the device in hand: some tiles run up to 25% slower on some MI355X boxes than
// on others, so the best tile for a shape is a property of the box as well.  Host memory
// only, one table per process; a mutex guards it, and the count lets launches skip the
// lock while the table is empty.
struct RuntimeChoice {
    int64_t M, N, K;
    int epi, a_vec, bc_vec, config;
};
constexpr int kMaxRuntimeChoices = 64;
RuntimeChoice g_choices[kMaxRuntimeChoices];
std::atomic<int> g_num_choices{0};
std::mutex g_choices_mu;

int runtime_choice(const Request &r, bool av, bool bv)
{
    if (g_num_choices.load(std::memory_order_acquire) == 0) return -1;
    std::lock_guard<std::mutex> lock(g_choices_mu);
    const int n = g_num_choices.load(std::memory_order_relaxed);
    for (int i = 0; i < n; ++i) {
        const RuntimeChoice &c = g_choices[i];
        if (c.M == r.M && c.N == r.N && c.K == r.K && c.epi == r.epi && c.a_vec == (int)av &&
            c.bc_vec == (int)bv && config_fits(kConfigs[c.config], r))
            return c.config;
    }
    return -1;
}

int choose(const Request &r)
{
    const bool av = a_vector_ok(r), bv = bc_vector_ok(r);
    const int installed = runtime_choice(r, av, bv);
    if (installed >= 0) return installed;
    const int tuned = tuned_choice(r, av, bv);
    if (tuned >= 0) return tuned;
    constexpr int64_t kCUs = 256;
    // rows of B and C that are not 16-byte friendly still take the direct kernel for all
    // but their last N % 8 columns (run() splits the launch)
    if (bv || r.N >= 64) {
        // measured with the interleaved tuner on MI355X (the table file records the runs)
        const int64_t t256 = tiles(r, 256, 256), t256x128 = tiles(r, 256, 128), t128 = tiles(r, 128, 128);
        // one wave of 256x256 tiles or more: the ping-pong kernel when K % 8 == 0 and the
        // rows of B and C are 16-byte friendly (no split launch)
        if (bv && t256 >= kCUs && r.K % 8 == 0) return find_pingpong(256, 256);
        if (t256 >= 4 * kCUs) return find_direct(256, 256, 32, 4, 1);   // several waves of big tiles
        if (t256 >= kCUs) return find_direct(256, 256, 64, 8, 1);        // about one wave of them
        // more 256x128 tiles than CUs, fewer 256x256 ones: one round of the larger tiles
        // beats a second, partly idle round of the smaller ones (3072^3: 144 tiles of
        // 256x256 in 58.5 us against 85.0 for 288 of 256x128; 3072x3072x2048 41.9 against
        // 60.0; 6144x2048x2048, 1.5 rounds of 256x128, 50.6 against 63.3)
        if (t256x128 > kCUs) return find_direct(256, 256, 32, 8, 1);
        // one full round of 256x128 tiles (e.g. one GPU's share of 8192^3), or 128x128 tiles
        // that would need a second, partial round while 256x128 ones fit in one (2304^3
        // 32.4 us against 36.6; 2560^3 38.7 against 42.2; 3072x2048x2048 31.0 against
        // 34.0; measured from K = 1024 up)
        if (t256x128 == kCUs || (t128 > kCUs && r.K >= 1024)) return find_direct(256, 128, 64, 8, 2);
        const int64_t t64x256 = tiles(r, 64, 256), t64x128 = tiles(r, 64, 128),
                      t64x192 = tiles(r, 64, 192);
        // K up to 2048 and a full wave of 64x192 tiles (at most 1/32 of the CUs idle) where
        // the 128x128, 64x256 and 64x128 tiles fill less of the chip or need a second
        // round: 1000x3000x777 + bias + GELU 256 tiles, 10.2 us against 10.9 for 192 of
        // 64x256; 2048x1536x512 5.8 against 6.3; 1024x3072x768 + bias + GELU 8.7 against
        // 9.4 with 128x128x32; 4096x768x1024 8.5 against 8.9 with the k-group 128x128
        // tile; 240 tiles were not enough (1280x2304x1024: 9.45 against 9.35).  The tile
        // is 4 waves of 64x48 on 16x16 MFMA blocks fed by 4 loader waves (each B fragment
        // read once: ragged + GELU 10.0-10.2 us against 10.2-10.6 for 4 waves of 32x96 on
        // 32x32 blocks; without epilogue 8.7 against 9.4), on 32-deep stages up to K =
        // 1024 and 64-deep ones beyond (1000x3000x1536 13.6 against 14.0 for the k-group
        // 128x128 tile, 1000x3000x2048 + bias + GELU 19.1 against 19.6, 2048x1536x2048
        // 16.4 against 16.7).  From K = 4096 the k-group 128x128 tile leads
        // (1000x3000x4096: 31.9 against 32.9).
        if (r.K <= 2048 && t128 <= kCUs && t64x192 <= kCUs && t64x192 >= kCUs - kCUs / 32 &&
            t64x192 > t64x256 && t64x192 < t64x128)
            return r.K <= 1024 ? find_direct(64, 192, 32, 4, 1, 4, 16) : find_direct(64, 192, 64, 4, 1, 4, 16);
        // at most one wave of 128x128 tiles with short K: 64x256 tiles (3000x1000x777: 11.6
        // us against 13.2 with 128x128x32; 2048x2048x777: 11.1-11.3 against 11.2-11.8; the
        // ragged 1000x3000x777, 192 tiles of either, 11.6 against 12.2 before the 64x192
        // tile took it)
        if (r.K < 1024 && r.N >= 256 && t128 <= kCUs && t64x256 <= kCUs && t64x256 >= kCUs / 2)
            return find_direct(64, 256, 32, 4, 1);
        // 128x128 tiles would leave half the chip or more idle: 64x128 tiles, twice as
        // many, while they still fit in one wave (1024^3: 6.3 us against 8.4 with the
        // k-group 128x128 tile; 512x4096x1024 7.3 against 8.7; 768^3 6.6 against 8.5;
        // 256^3, 8 tiles: 4.1 us per kernel against 4.5-4.8 for the register-staged
        // 64x64 tile); from K = 4096 the k-group tile wins again (1024x1024x4096: 25.3
        // against 26.7)
        if (r.N >= 128 && t128 <= kCUs / 2 && t64x128 <= kCUs && t64x128 >= kCUs / 32 && r.K <= 2048)
            return find_direct(64, 128, 32, 4, 1);
        // short K: 32-deep stages, so the ring fills and the last stage drains sooner
        if (t128 >= kCUs / 4 && r.K < 1024) return find_direct(128, 128, 32, 4, 1);
        // one wave of 128x128 tiles or more: 4 multiplying waves fed by 4 loader waves
        // (interleaved: 2048^3 18.5-19.7 us against 19.2-20.3 for the same tile without them;
        // 2048x2048x4096 32.6-34.9 against 33.4-35.7, and 33.7-35.8 with two k-groups;
        // 2048x2048x8192 63.0 against 63.5 with two k-groups).  On some boxes the 64-deep
        // tiles on their 128 KiB ring run slow, and the 32-deep one on a 64 KiB ring does
        // not: 2048^3 19.6-20.6 us against 21.5-23.3, with bias + GELU 22.0-22.7 against
        // 24.7-28.5, where on the others it trails by 7% (19.7 against 18.5) and 2.5% with
        // GELU.  Below K = 4096 the rules take the 32-deep tile, which is never far from
        // the best; from K = 4096 the 64-deep one leads on both kinds of box (34.9 against
        // 37.9 and 32.6 against 36.1).  Calibration picks per box between them.
        if (t128 >= kCUs) return r.K >= 4096 ? find_direct(128, 128, 64, 4, 1, 4)
                                             : find_direct(128, 128, 32, 4, 1, 4);
        if (t128 >= kCUs / 4) return find_direct(128, 128, 64, 8, 2);    // part of the chip idle
    }
    // at most 8 columns: no tile contraction left; the narrow kernel reads A once
    if (r.N <= 8) return narrow_for(r.M);
    if (tiles(r, 128, 128) >= kCUs / 2) return find_staged(128, 128, av, bv);
    return find_staged(64, 64, av, bv);
}

// Can configuration c serve request r?
mi355gemm_status check_config(const Config &c, const Request &r)
{
    if (c.lds_bytes > kLdsBudget)
        return fail(MI355GEMM_EUNSUPPORTED, "config %s needs %d B of LDS, over the %d B budget",
                    c.name, c.lds_bytes, kLdsBudget);
    if (c.a_vec && !a_vector_ok(r))
        return fail(MI355GEMM_EUNSUPPORTED,
                    "config %s loads A in 16-byte vectors: needs K %% 8 == 0 and a 16-byte aligned A",
                    c.name);
    if (c.bc_vec && !bc_vector_ok(r))
        return fail(MI355GEMM_EUNSUPPORTED,
                    "config %s moves B and C in vectors: needs N %% 8 == 0, 16-byte aligned B and C "
                    "and an 8-byte aligned bias", c.name);
    if (c.narrow && r.N > c.bn)
        return fail(MI355GEMM_EUNSUPPORTED, "config %s computes at most %d columns (N=%lld)", c.name,
                    c.bn, (long long)r.N);
    if (c.k_mult8 && r.K % 8 != 0)
        return fail(MI355GEMM_EUNSUPPORTED, "config %s needs K %% 8 == 0 (K=%lld)", c.name,
                    (long long)r.K);
    return MI355GEMM_OK;
}

// Launch configuration c on columns [n_begin, n_begin + n_width) of the request (B, C and
// bias offset by n_begin, rows still N apart).  Non-null events are recorded by the
// dispatch itself as the kernel starts (ev_start) and ends (ev_stop).
mi355gemm_status launch(const Config &c, const Request &r, int64_t n_begin, int64_t n_width,
                        hipStream_t stream, hipEvent_t ev_start = nullptr,
                        hipEvent_t ev_stop = nullptr)
{
    GemmArgs a;
    a.A = static_cast<const f16 *>(r.A);
    a.B = r.B != nullptr ? static_cast<const f16 *>(r.B) + n_begin : nullptr;
    a.C = static_cast<f16 *>(r.C) + n_begin;
    a.bias = r.bias != nullptr ? static_cast<const f16 *>(r.bias) + n_begin : nullptr;
    a.M = (int)r.M;
    a.N = (int)n_width;
    a.K = (int)r.K;
    a.ldb = a.ldc = (int)r.N;
    a.tiles_m = (int)((r.M + c.bm - 1) / c.bm);
    a.tiles_n = (int)((n_width + c.bn - 1) / c.bn);
    a.group_m = c.group_m;
    const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
    if (grid >= ((int64_t)1 << 31))
        return fail(MI355GEMM_EUNSUPPORTED, "too many tiles (%lld)", (long long)grid);
    const KernelFn fn = c.fn[(r.K & 7) != 0][r.epi];
    if (fn == nullptr)
        return fail(MI355GEMM_EUNSUPPORTED, "config %s has no kernel for K %% 8 != 0", c.name);
    if (ev_start != nullptr || ev_stop != nullptr)
        hipExtLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(c.threads), 0, stream, ev_start,
                              ev_stop, 0, a);
    else
        hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(c.threads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(MI355GEMM_EHIP, "launch of %s failed: %s", c.name, hipGetErrorString(e));
    return MI355GEMM_OK;
}

mi355gemm_status run(const Request &r, void *stream, int forced, hipEvent_t ev_start = nullptr,
                     hipEvent_t ev_stop = nullptr)
{
    mi355gemm_status st = validate(r);
    if (st != MI355GEMM_OK) return st;
    if (forced >= kNumConfigs || forced < -1)
        return fail(MI355GEMM_EINVAL, "unknown config id %d", forced);
    if (forced >= 0) {
        st = check_config(kConfigs[forced], r);
        if (st != MI355GEMM_OK) return st;
    }
    if (r.M == 0 || r.N == 0) return MI355GEMM_OK;
    const int id = forced >= 0 ? forced : choose(r);
    if (id < 0) return fail(MI355GEMM_EUNSUPPORTED, "no configuration serves this request");
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const Config &c = kConfigs[id];
    if (forced < 0 && c.direct && !bc_vector_ok(r)) {
        // B, C or bias rows not 16-byte friendly: the direct kernel takes the columns up
        // to the last multiple of 8 (at any 2-byte alignment its 16-byte pieces then never
        // straddle the end of a row's columns), the narrow kernel the last N % 8
        const int64_t n8 = r.N & ~(int64_t)7;
        const bool two = n8 != r.N;
        const mi355gemm_status s2 = launch(c, r, 0, n8, hs, ev_start, two ? nullptr : ev_stop);
        if (s2 != MI355GEMM_OK || !two) return s2;
        return launch(kConfigs[narrow_for(r.M)], r, n8, r.N - n8, hs, nullptr, ev_stop);
    }
    return launch(c, r, 0, r.N, hs, ev_start, ev_stop);
}

}  // namespace

extern "C" {

mi355gemm_status mi355gemm_gemm(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                                void *C, const void *bias, int epi, void *stream)
{
    g_last_error[0] = 0;
    return run(Request{M, N, K, A, B, bias, C, epi}, stream, -1);
}

mi355gemm_status mi355gemm_gemm_config(int64_t M, int64_t N, int64_t K, const void *A,
                                       const void *B, void *C, const void *bias, int epi,
                                       void *stream, int config_id)
{
    g_last_error[0] = 0;
    if (config_id < 0) return fail(MI355GEMM_EINVAL, "unknown config id %d", config_id);
    return run(Request{M, N, K, A, B, bias, C, epi}, stream, config_id);
}

mi355gemm_status mi355gemm_gemm_timed(int64_t M, int64_t N, int64_t K, const void *A,
                                      const void *B, void *C, const void *bias, int epi,
                                      void *stream, int config_id, void *start_event,
                                      void *stop_event)
{
    g_last_error[0] = 0;
    if (config_id < -1) return fail(MI355GEMM_EINVAL, "unknown config id %d", config_id);
    return run(Request{M, N, K, A, B, bias, C, epi}, stream, config_id,
               static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
}

int mi355gemm_select(int64_t M, int64_t N, int64_t K, int epi, const void *A, const void *B,
                     const void *C, const void *bias)
{
    g_last_error[0] = 0;
    const Request r{M, N, K, A, B, bias, const_cast<void *>(C), epi};
    if (validate(r) != MI355GEMM_OK) return -1;
    if (M == 0 || N == 0) {
        fail(MI355GEMM_OK, "empty problem: no launch");
        return -1;
    }
    return choose(r);
}

mi355gemm_status mi355gemm_vector_add(int64_t n, const void *a, const void *b, void *c,
                                      void *stream)
{
    g_last_error[0] = 0;
    if (n < 0) return fail(MI355GEMM_EINVAL, "negative length %lld", (long long)n);
    if (n == 0) return MI355GEMM_OK;
    if (a == nullptr || b == nullptr || c == nullptr)
        return fail(MI355GEMM_EINVAL, "a, b and c must not be NULL");
    if (!aligned(a, 2) || !aligned(b, 2) || !aligned(c, 2))
        return fail(MI355GEMM_EINVAL, "fp16 pointers must be 2-byte aligned");
    // elements added one by one until c is 16-byte aligned, then 8 per lane per access
    const int64_t head = std::min<int64_t>(n, (int64_t)(((16 - ((uintptr_t)c & 15)) & 15) / 2));
    const int64_t nv = (n - head) / 8;
    const int64_t blocks = std::max<int64_t>(
        1, std::min<int64_t>((nv + kVecThreads - 1) / kVecThreads, ((int64_t)1 << 31) - 1));
    hipLaunchKernelGGL(vector_add_kernel, dim3((unsigned)blocks), dim3(kVecThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const vf16 *>(a),
                       static_cast<const vf16 *>(b), static_cast<vf16 *>(c), n, head);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(MI355GEMM_EHIP, "launch of vector_add failed: %s", hipGetErrorString(e));
    return MI355GEMM_OK;
}

mi355gemm_status mi355gemm_softmax(int64_t M, int64_t N, const void *x, void *y, void *stream)
{
    g_last_error[0] = 0;
    if (M < 0 || N < 0)
        return fail(MI355GEMM_EINVAL, "negative size (M=%lld N=%lld)", (long long)M, (long long)N);
    if (M == 0 || N == 0) return MI355GEMM_OK;
    if (x == nullptr || y == nullptr) return fail(MI355GEMM_EINVAL, "x and y must not be NULL");
    if (!aligned(x, 2) || !aligned(y, 2))
        return fail(MI355GEMM_EINVAL, "fp16 pointers must be 2-byte aligned");
    if (N >= ((int64_t)1 << 31) || M >= ((int64_t)1 << 31))
        return fail(MI355GEMM_EUNSUPPORTED, "M and N must be below 2^31");
    const sf16 *xs = static_cast<const sf16 *>(x);
    sf16 *ys = static_cast<sf16 *>(y);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int n = (int)N;
    const dim3 rows_grid((unsigned)((M + 3) / 4));
    // one wavefront per row up to 2048 elements, four per row up to 16384, sixteen up to
    // 65536 (measured crossovers on MI355X), then two passes by one workgroup per row
    const dim3 one_row((unsigned)M);
    if (N <= 512) hipLaunchKernelGGL(softmax_rows<1>, rows_grid, dim3(kSoftmaxThreads), 0, st, xs, ys, M, n);
    else if (N <= 1024) hipLaunchKernelGGL(softmax_rows<2>, rows_grid, dim3(kSoftmaxThreads), 0, st, xs, ys, M, n);
    else if (N <= 2048) hipLaunchKernelGGL(softmax_rows<4>, rows_grid, dim3(kSoftmaxThreads), 0, st, xs, ys, M, n);
    else if (N <= 4096) hipLaunchKernelGGL((softmax_wg<2, 256>), one_row, dim3(256), 0, st, xs, ys, n);
    else if (N <= 8192) hipLaunchKernelGGL((softmax_wg<4, 256>), one_row, dim3(256), 0, st, xs, ys, n);
    else if (N <= 16384) hipLaunchKernelGGL((softmax_wg<8, 256>), one_row, dim3(256), 0, st, xs, ys, n);
    else if (N <= 32768) hipLaunchKernelGGL((softmax_wg<4, 1024>), one_row, dim3(1024), 0, st, xs, ys, n);
    else if (N <= 65536) hipLaunchKernelGGL((softmax_wg<8, 1024>), one_row, dim3(1024), 0, st, xs, ys, n);
    else hipLaunchKernelGGL(softmax_long, dim3((unsigned)M), dim3(kSoftmaxLongThreads), 0, st, xs, ys, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(MI355GEMM_EHIP, "launch of softmax failed: %s", hipGetErrorString(e));
    return MI355GEMM_OK;
}

mi355gemm_status mi355gemm_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                                     int64_t head_dim, const void *q, const void *k,
                                     const void *v, void *o, float *lse, float scale,
                                     int causal, void *stream)
{
    g_last_error[0] = 0;
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || head_dim < 0)
        return fail(MI355GEMM_EINVAL, "negative size (batch=%lld heads=%lld seq_q=%lld seq_k=%lld head_dim=%lld)",
                    (long long)batch, (long long)heads, (long long)seq_q, (long long)seq_k,
                    (long long)head_dim);
    if (causal != 0 && causal != 1) return fail(MI355GEMM_EINVAL, "causal must be 0 or 1");
    if (!(scale > 0.0f) || !(scale < __builtin_inff()))
        return fail(MI355GEMM_EINVAL, "scale must be finite and positive");
    if (head_dim != 64 && head_dim != 128)
        return fail(MI355GEMM_EUNSUPPORTED, "head_dim %lld (64 or 128 are served)", (long long)head_dim);
    if (batch == 0 || heads == 0 || seq_q == 0) return MI355GEMM_OK;
    if (seq_k == 0) return fail(MI355GEMM_EINVAL, "seq_k == 0: the softmax over no keys is undefined");
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return fail(MI355GEMM_EINVAL, "q, k, v and o must not be NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(MI355GEMM_EINVAL, "q, k, v and o must be 16-byte aligned");
    if (lse != nullptr && !aligned(lse, 4)) return fail(MI355GEMM_EINVAL, "lse must be 4-byte aligned");
    const int64_t lim = (int64_t)1 << 31;
    if (batch >= lim || heads >= lim || batch * heads >= lim ||
        (seq_q + 1024) * head_dim * 2 >= lim || (seq_k + 1024) * head_dim * 2 >= lim)
        return fail(MI355GEMM_EUNSUPPORTED, "sizes past the kernel's 32-bit offsets");
    constexpr int BM = A128::BM;
    static_assert(A64::BM == BM && A64::NT == A128::NT, "one launch shape for both head dims");
    const int64_t q_blocks = (seq_q + BM - 1) / BM;
    if (batch * heads * q_blocks >= lim) return fail(MI355GEMM_EUNSUPPORTED, "grid too large");
    AttnArgs a;
    a.q = static_cast<const f16 *>(q);
    a.k = static_cast<const f16 *>(k);
    a.v = static_cast<const f16 *>(v);
    a.o = static_cast<f16 *>(o);
    a.lse = lse;
    a.pairs = (int)(batch * heads);
    a.Sq = (int)seq_q;
    a.Sk = (int)seq_k;
    a.q_blocks = (int)q_blocks;
    a.c = scale * 1.4426950408889634f;
    a.causal = causal;
    const dim3 grid((unsigned)(batch * heads * q_blocks));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (head_dim == 128)
        hipLaunchKernelGGL(attention_fwd<A128>, grid, dim3(A128::NT), 0, st, a);
    else
        hipLaunchKernelGGL(attention_fwd<A64>, grid, dim3(A64::NT), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(MI355GEMM_EHIP, "launch of attention failed: %s", hipGetErrorString(e));
    return MI355GEMM_OK;
}

mi355gemm_status mi355gemm_set_choice(int64_t M, int64_t N, int64_t K, int epi, int a_vector,
                                      int bc_vector, int config_id)
{
    g_last_error[0] = 0;
    if (M < 0 || N < 0 || K < 0)
        return fail(MI355GEMM_EINVAL, "negative size (M=%lld N=%lld K=%lld)", (long long)M,
                    (long long)N, (long long)K);
    if (epi < MI355GEMM_EPI_NONE || epi > MI355GEMM_EPI_BIAS_GELU)
        return fail(MI355GEMM_EINVAL, "unknown epilogue %d", epi);
    if ((a_vector != 0 && a_vector != 1) || (bc_vector != 0 && bc_vector != 1))
        return fail(MI355GEMM_EINVAL, "alignment classes are 0 or 1 (got %d, %d)", a_vector,
                    bc_vector);
    if (config_id < 0 || config_id >= kNumConfigs)
        return fail(MI355GEMM_EINVAL, "unknown config id %d", config_id);
    const Config &c = kConfigs[config_id];
    if ((c.a_vec && !a_vector) || (c.bc_vec && !bc_vector) || (c.narrow && N > c.bn) ||
        (c.k_mult8 && K % 8 != 0))
        return fail(MI355GEMM_EUNSUPPORTED, "config %s cannot serve this alignment class or N",
                    c.name);
    std::lock_guard<std::mutex> lock(g_choices_mu);
    const int n = g_num_choices.load(std::memory_order_relaxed);
    for (int i = 0; i < n; ++i) {
        RuntimeChoice &e = g_choices[i];
        if (e.M == M && e.N == N && e.K == K && e.epi == epi && e.a_vec == a_vector &&
            e.bc_vec == bc_vector) {
            e.config = config_id;
            return MI355GEMM_OK;
        }
    }
    if (n == kMaxRuntimeChoices)
        return fail(MI355GEMM_EUNSUPPORTED, "the table of installed choices is full (%d)",
                    kMaxRuntimeChoices);
    g_choices[n] = RuntimeChoice{M, N, K, epi, a_vector, bc_vector, config_id};
    g_num_choices.store(n + 1, std::memory_order_release);
    return MI355GEMM_OK;
}

void mi355gemm_clear_choices(void)
{
    std::lock_guard<std::mutex> lock(g_choices_mu);
    g_num_choices.store(0, std::memory_order_release);
}

int mi355gemm_num_configs(void) { return kNumConfigs; }

const char *mi355gemm_config_name(int config_id)
{
    if (config_id < 0 || config_id >= kNumConfigs) return nullptr;
    return kConfigs[config_id].name;
}

mi355gemm_status mi355gemm_config_info(int config_id, mi355gemm_config_desc *out)
{
    if (config_id < 0 || config_id >= kNumConfigs || out == nullptr)
        return fail(MI355GEMM_EINVAL, "unknown config id %d or NULL out", config_id);
    const Config &c = kConfigs[config_id];
    out->block_m = c.bm;
    out->block_n = c.bn;
    out->block_k = c.bk;
    out->stages = c.stages;
    out->waves_m = c.waves_m;
    out->waves_n = c.waves_n;
    out->k_groups = c.k_groups;
    out->threads = c.threads;
    out->lds_bytes = c.lds_bytes;
    out->a_vector = c.a_vec;
    out->bc_vector = c.bc_vec;
    out->group_m = c.group_m;
    out->direct = c.direct;
    out->narrow = c.narrow;
    out->k_mult8 = c.k_mult8;
    out->pingpong = c.pingpong;
    out->loader_waves = c.loaders;
    out->mfma_block = c.mfma_block;
    return MI355GEMM_OK;
}

int mi355gemm_lds_budget(void) { return kLdsBudget; }

const char *mi355gemm_last_error(void) { return g_last_error; }

const char *mi355gemm_version(void) { return "mi355gemm 0.1.0 (gfx950)"; }

#if MI355_PHASE_CLOCK
// Diagnostic build only (no header declares these): copy out or clear the direct kernel's
// phase clock, kPhaseClockTiles x 16 values (see gemm_direct.hpp).  `n` values at most.
int mi355gemm_phase_clock_read(unsigned long long *host, int n)
{
    if (host == nullptr || n < 0 || n > kPhaseClockTiles * 16)
        return fail(MI355GEMM_EINVAL, "phase clock: NULL buffer or n=%d outside 0..%d", n,
                    kPhaseClockTiles * 16);
    if (hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_clock), sizeof(unsigned long long) * n, 0,
                            hipMemcpyDeviceToHost) != hipSuccess)
        return fail(MI355GEMM_EHIP, "phase clock: copy from the device failed");
    return MI355GEMM_OK;
}

int mi355gemm_phase_clock_clear(void)
{
    void *dev = nullptr;
    if (hipGetSymbolAddress(&dev, HIP_SYMBOL(g_phase_clock)) != hipSuccess ||
        hipMemset(dev, 0, sizeof(unsigned long long) * kPhaseClockTiles * 16) != hipSuccess)
        return fail(MI355GEMM_EHIP, "phase clock: clearing the device array failed");
    return MI355GEMM_OK;
}
#endif

}  // extern "C"

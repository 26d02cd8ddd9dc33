// Per-CU throughput of the data paths the GEMM kernels' K loops lean on, measured on the
// device in hand: LDS fragment reads (ds_read_b128 as for A fragments, the transposing
// ds_read_b64_tr_b16 as for B fragments), LDS-DMA copies (buffer_load_dwordx4 ... lds, the
// HBM/L2 -> LDS loader) and plain 16-byte global loads, the last two from a window small
// enough to stay in L2 (1 MiB) and from one that is not (32 MiB).  One workgroup per CU,
// 4, 8 or 16 wavefronts each; every wavefront times itself with s_memtime (shader clock
// cycles) and s_memrealtime (100 MHz), so the report is bytes per clock per CU and GB/s.
//
// Build: part of the package build (bandwidth_probe next to the library).  Run with no
// arguments; it prints one line per measurement.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                 \
        }                                                                                 \
    } while (0)

constexpr int kLdsBytes = 64 * 1024;
constexpr int kMaxWaves = 16;
constexpr int kUnroll = 8;

// Timestamps of one wavefront: [cycles, 10 ns ticks].
__device__ __forceinline__ void stamp(unsigned long long *t, unsigned long long c0,
                                      unsigned long long r0)
{
    t[0] = __builtin_amdgcn_s_memtime() - c0;
    t[1] = __builtin_amdgcn_s_memrealtime() - r0;
}

// MODE 0: ds_read_b128; MODE 1: ds_read_b64_tr_b16.  Consecutive lanes read consecutive
// 16 (8) bytes, so the reads are free of bank conflicts; offsets are masked into the array.
template <int MODE>
__global__ void __launch_bounds__(1024) lds_reads(int iters, uint32_t *sink, unsigned long long *times)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
    for (int i = threadIdx.x; i < kLdsBytes / 4; i += blockDim.x) lds[i] = i * 2654435761u;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t acc = 0;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int slot = (it * kUnroll + u) * 64 + wave * 512 + lane;
            if constexpr (MODE == 0) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(&lds[(slot & (kLdsBytes / 16 - 1)) * 4]);
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            } else {
                const int byte = (slot & (kLdsBytes / 8 - 1)) * 8;
                const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)(
                        (__attribute__((address_space(3))) char *)lds + byte));
                acc ^= (uint32_t)v.x ^ (uint32_t)v.y ^ (uint32_t)v.z ^ (uint32_t)v.w;
            }
        }
    }
    if (lane == 0) stamp(times + (blockIdx.x * kMaxWaves + wave) * 2, c0, r0);
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// LDS-DMA: each wavefront copies 1 KiB per instruction into one of two 1 KiB LDS slots of
// its own, from offsets that wrap inside a `window`-byte buffer (a power of two).  At most
// 2 * kUnroll copies are in flight per wavefront.
__global__ void __launch_bounds__(1024) lds_dma(const uint32_t *src, int window, int iters,
                                                uint32_t *sink, unsigned long long *times)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(src), 0, window, 0x00020000);
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t voff =
                (uint32_t)((((blockIdx.x * 37 + it) * kUnroll + u) * 16384 + wave * 1024 + lane * 16) &
                           (window - 1));
            const uint32_t lds_addr = (uint32_t)(uintptr_t)(
                (__attribute__((address_space(3))) char *)lds + (wave * 2 + (u & 1)) * 1024);
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(voff), "s"(rs), "{m0}"(lds_addr));
        }
        // vmcnt(kUnroll): the copies of the previous iteration have landed
        __builtin_amdgcn_s_waitcnt((kUnroll & 15) | (7 << 4) | (15 << 8));
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
    if (lane == 0) stamp(times + (blockIdx.x * kMaxWaves + wave) * 2, c0, r0);
    __syncthreads();
    sink[blockIdx.x * blockDim.x + threadIdx.x] = lds[threadIdx.x];
}

// 16-byte global loads into registers from a `window`-byte buffer (a power of two).
__global__ void __launch_bounds__(1024) global_loads(const u32x4 *src, int window, int iters,
                                                     uint32_t *sink, unsigned long long *times)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunks = window / 16;
    uint32_t acc = 0;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int chunk = (((blockIdx.x * 37 + it) * kUnroll + u) * 1024 + wave * 64 + lane) & (chunks - 1);
            const u32x4 v = src[chunk];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (lane == 0) stamp(times + (blockIdx.x * kMaxWaves + wave) * 2, c0, r0);
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

struct Probe {
    int cus;
    uint32_t *sink;
    unsigned long long *times;
    std::vector<unsigned long long> host;

    // Mean over all wavefronts of the per-wave cycles and ticks, after one untimed launch.
    template <class Launch>
    void run(const char *what, int waves, double bytes_per_wave, Launch launch)
    {
        launch();
        CHECK(hipDeviceSynchronize());
        launch();
        CHECK(hipDeviceSynchronize());
        CHECK(hipMemcpy(host.data(), times, host.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
        double cyc = 0, ticks = 0;
        for (int b = 0; b < cus; ++b)
            for (int w = 0; w < waves; ++w) {
                cyc += (double)host[(b * kMaxWaves + w) * 2];
                ticks += (double)host[(b * kMaxWaves + w) * 2 + 1];
            }
        cyc /= cus * waves;
        ticks /= cus * waves;
        const double per_cu = bytes_per_wave * waves;
        std::printf("%-34s waves/CU %2d  %7.1f B/clk per CU  %7.1f GB/s per CU  %6.2f TB/s total  (%.2f GHz)\n",
                    what, waves, per_cu / cyc, per_cu / (ticks * 10.0), per_cu * cus / (ticks * 10.0) / 1e3,
                    cyc / (ticks * 10.0));
    }
};

}  // namespace

int main()
{
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    Probe p;
    p.cus = prop.multiProcessorCount;
    CHECK(hipMalloc(&p.sink, (size_t)p.cus * 1024 * sizeof(uint32_t)));
    CHECK(hipMalloc(&p.times, (size_t)p.cus * kMaxWaves * 2 * sizeof(unsigned long long)));
    p.host.resize((size_t)p.cus * kMaxWaves * 2);
    const int big = 32 << 20;
    void *src = nullptr;
    CHECK(hipMalloc(&src, big));
    CHECK(hipMemset(src, 1, big));
    std::printf("%s, %d CUs\n", prop.gcnArchName, p.cus);

    const int lds_iters = 2048, mem_iters = 256;
    for (int waves : {4, 8, 16}) {
        const int threads = 64 * waves;
        p.run("LDS ds_read_b128", waves, (double)lds_iters * kUnroll * 64 * 16,
              [&] { lds_reads<0><<<p.cus, threads>>>(lds_iters, p.sink, p.times); });
        p.run("LDS ds_read_b64_tr_b16", waves, (double)lds_iters * kUnroll * 64 * 8,
              [&] { lds_reads<1><<<p.cus, threads>>>(lds_iters, p.sink, p.times); });
    }
    for (int window : {1 << 20, big}) {
        for (int waves : {4, 8, 16}) {
            const int threads = 64 * waves;
            char name[64];
            std::snprintf(name, sizeof name, "LDS-DMA from %d MiB window", window >> 20);
            p.run(name, waves, (double)mem_iters * kUnroll * 1024, [&] {
                lds_dma<<<p.cus, threads>>>(static_cast<const uint32_t *>(src), window, mem_iters, p.sink, p.times);
            });
            std::snprintf(name, sizeof name, "global b128 from %d MiB window", window >> 20);
            p.run(name, waves, (double)mem_iters * kUnroll * 1024, [&] {
                global_loads<<<p.cus, threads>>>(static_cast<const u32x4 *>(src), window, mem_iters, p.sink, p.times);
            });
        }
    }
    CHECK(hipFree(src));
    CHECK(hipFree(p.times));
    CHECK(hipFree(p.sink));
    std::printf("done\n");
    return 0;
}

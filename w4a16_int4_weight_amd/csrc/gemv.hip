// Weight-streaming split-K GEMV for decode-sized batches (1 <= M <= 16).
//
// Decode is bound by the bytes of the weights: every weight is read once per
// token (vllm-omni commit "Add cpu_int4, an asymmetric 4-bit weight path for
// vLLM's CPU backend"). So the kernel is organised around streaming the packed
// codes at HBM rate with 128-bit loads and doing as little per-weight ALU work as
// possible:
//
//   * one workgroup per 16-column block; its W waves split the K range (split-K)
//     and each wave issues the loads of all its 1 KiB blocks up front;
//   * per 32-row step a lane turns its packed word into the B operand of a
//     16x16x32 MFMA with one shift and one AND-OR per pair of codes: OR-ing a code
//     into the mantissa of the 16-bit value 128.0 (bf16) or 1024.0 (fp16) gives
//     exactly base + q;
//   * the offset and the zero point are removed by a second MFMA on the same
//     activations with B = -(base + z) in every entry, accumulating into the same
//     registers: sum_k x (base + q) - x (base + z) = sum_k x (q - z), exact
//     products, fp32 sums;
//   * the group's scale is applied once per 128-row block: acc += s * T;
//   * the activations (<= 16 rows) are the A operand, zero-filled beyond M;
//   * the waves' partial sums are added in wave order through LDS (deterministic),
//     bias is added in fp32 and the result rounded once to the output dtype.
//
// Per 32 weights a lane spends 7 VALU operations on decoding + 2 MFMA issues,
// independent of M.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kBlocksPerBatch = 4;    // 1 KiB blocks whose loads a wave issues together

template <bool kBF16>
__device__ __forceinline__ f32x4 block_partial(const uint4 wq, const uint32_t md, const uint4 (&xa)[4]) {
    using Mg = Magic<kBF16>;
    const uint32_t z = (md >> 16) & 0xFu;
    const uint32_t nz = Mg::kNegBase | z;            // -(base + z), exact
    const uint4 bz = make_uint4(nz | (nz << 16), nz | (nz << 16), nz | (nz << 16), nz | (nz << 16));
    const uint32_t d[4] = {wq.x, wq.y, wq.z, wq.w};
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = d[i];
        const uint4 b = make_uint4((v & 0x000F000Fu) | Mg::kBase2, ((v >> 4) & 0x000F000Fu) | Mg::kBase2,
                                   ((v >> 8) & 0x000F000Fu) | Mg::kBase2, ((v >> 12) & 0x000F000Fu) | Mg::kBase2);
        t = mfma16x16x32<kBF16>(xa[i], b, t);
        t = mfma16x16x32<kBF16>(xa[i], bz, t);
    }
    return t;
}

template <bool kBF16>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int M, int64_t K, int64_t N) {
    __shared__ f32x4 partial[kMaxWaves][64];

    const int64_t KB = K / kRowsPerBlock;
    const int64_t nb = blockIdx.x;
    const int waves = blockDim.x >> 6;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;         // column in the block, and activation row of the A operand
    const int h = lane >> 4;         // which 8 of every 32 rows
    const int64_t kb_begin = (KB * w) / waves;
    const int64_t kb_end = (KB * (w + 1)) / waves;

    const uint4* wplane = reinterpret_cast<const uint4*>(packed) + nb * KB * 64 + lane;
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(packed + K * N / 2) + nb * KB * kColsPerBlock + c;
    const bool row_valid = c < M;
    const uint4* xrow = reinterpret_cast<const uint4*>(x + (int64_t)(row_valid ? c : 0) * K + 8 * h);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t kb0 = kb_begin; kb0 < kb_end; kb0 += kBlocksPerBatch) {
        uint4 wq[kBlocksPerBatch];
        uint32_t md[kBlocksPerBatch];
        uint4 xa[kBlocksPerBatch][4];
#pragma unroll
        for (int u = 0; u < kBlocksPerBatch; ++u) {
            const int64_t kb = kb0 + u;
            const bool ok = kb < kb_end;
            wq[u] = ok ? wplane[kb * 64] : make_uint4(0, 0, 0, 0);
            md[u] = ok ? meta[kb * kColsPerBlock] : 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xa[u][i] = (ok && row_valid) ? xrow[kb * 16 + i * 4] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kBlocksPerBatch; ++u) {
            if (kb0 + u < kb_end) {
                const f32x4 t = block_partial<kBF16>(wq[u], md[u], xa[u]);
                const float s = half_bits_to_f32<kBF16>(md[u] & 0xFFFFu);
                acc += s * t;
            }
        }
    }

    if (waves > 1) {
        partial[w][lane] = acc;
        __syncthreads();
        if (w != 0) return;
        acc = partial[0][lane];
        for (int v = 1; v < waves; ++v) acc += partial[v][lane];
    }

    const int64_t n = nb * kColsPerBlock + c;
    const float b = bias ? half_bits_to_f32<kBF16>(bias[n]) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * h + r;
        if (row < M) y[(int64_t)row * N + n] = f32_to_half_bits<kBF16>(acc[r] + b);
    }
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t K, int64_t N, bool bf16, hipStream_t stream) {
    const int64_t KB = K / kRowsPerBlock;
    int64_t waves = (KB + kBlocksPerBatch - 1) / kBlocksPerBatch;
    if (waves > kMaxWaves) waves = kMaxWaves;
    if (waves < 1) waves = 1;
    const dim3 grid((unsigned)(N / kColsPerBlock));
    const dim3 block((unsigned)(64 * waves));
    if (bf16)
        hipLaunchKernelGGL(gemv_kernel<true>, grid, block, 0, stream, x, packed, bias, y, (int)M, K, N);
    else
        hipLaunchKernelGGL(gemv_kernel<false>, grid, block, 0, stream, x, packed, bias, y, (int)M, K, N);
    return hipGetLastError();
}

}  // namespace w4a16

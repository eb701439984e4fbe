// LDS-staged dequantise -> MFMA GEMM for prefill-sized batches.
//
// A W4A16 product at hundreds of rows is a real dense contraction, so it runs on
// the matrix cores. What the CPU design of the vllm-omni cpu_int4 commits teaches
// carries over: a kernel that dequantises once per activation row is linear in the
// batch ("12.9x slower than bf16 at 512 rows", commit "Add cpu_int4 ..."), and
// re-laying the weights out on every call halves prefill (commit "cpu_int4:
// dequantize prefill weights from the tinygemm layout, not a copy"). Here each
// weight is dequantised once per workgroup tile of up to 128 rows, straight from
// the packed layout, which is already in MFMA operand order: no per-call shuffle.
//
// Workgroup: 4 waves side by side along N, each owning 4 column blocks (64
// columns) and all 16*MR rows of the tile. Per 128-row block of K:
//   * the activation tile [16*MR x 128] is staged in LDS (double buffered, the next
//     block's tile loaded into registers while the current one is consumed);
//   * each wave loads its own 4 x 16 bytes of packed codes and 4 metadata words
//     per lane (also one block ahead), and per 32-row step decodes one word per
//     column block into 8 fp16/bf16 weights (q - z) * s rounded once to the dtype;
//   * MR x 4 MFMAs (16x16x32) per step, fp32 accumulators in registers.
// Epilogue: bias in fp32, one rounding to the dtype.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kColBlocksPerWave = 4;
constexpr int kColBlocksPerWG = kWaves * kColBlocksPerWave;   // 16 -> 256 columns
constexpr int kLdsRowElems = kRowsPerBlock + 8;               // 272-byte rows: spreads LDS banks

// Decode one tile word (8 codes of one column, rows 8 apart in k order given by the
// slot order) into the B operand of a 16x16x32 MFMA: 8 values (q - z) * s.
template <bool kBF16> struct Dequant;

template <> struct Dequant<true> {
    // bf16: codes -> fp32 via the byte converters, (q - z) * s = fma(q, s, -z*s) is
    // exact in fp32 (a 4-bit integer times an 8-bit significand), then one RNE
    // conversion per pair. Byte b of (d & 0x0F0F0F0F) is slot 2b and byte b of
    // (d >> 4) & 0x0F0F0F0F is slot 2b+1; slot -> row: 0,2,4,6,1,3,5,7.
    float s, nzs;
    __device__ __forceinline__ Dequant(uint32_t md) {
        s = bf16_bits_to_f32(md & 0xFFFFu);
        nzs = -(float)((md >> 16) & 0xFu) * s;
    }
    __device__ __forceinline__ uint4 operator()(uint32_t d) const {
        const uint32_t lo = d & 0x0F0F0F0Fu;          // rows 0, 4, 1, 5 in bytes 0..3
        const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;   // rows 2, 6, 3, 7 in bytes 0..3
        const float r0 = fmaf((float)(lo & 0xFFu), s, nzs);
        const float r4 = fmaf((float)((lo >> 8) & 0xFFu), s, nzs);
        const float r1 = fmaf((float)((lo >> 16) & 0xFFu), s, nzs);
        const float r5 = fmaf((float)(lo >> 24), s, nzs);
        const float r2 = fmaf((float)(hi & 0xFFu), s, nzs);
        const float r6 = fmaf((float)((hi >> 8) & 0xFFu), s, nzs);
        const float r3 = fmaf((float)((hi >> 16) & 0xFFu), s, nzs);
        const float r7 = fmaf((float)(hi >> 24), s, nzs);
        return make_uint4(pack2_rne<true>(r0, r1), pack2_rne<true>(r2, r3),
                          pack2_rne<true>(r4, r5), pack2_rne<true>(r6, r7));
    }
};

template <> struct Dequant<false> {
    // fp16: OR-ing a pair of codes into 1024.0 gives (1024 + q) exactly; a packed
    // fp16 subtract of (1024 + z) gives q - z exactly; a packed multiply by s rounds
    // (q - z) * s once, to nearest even.
    f16x2 zz, ss;
    __device__ __forceinline__ Dequant(uint32_t md) {
        const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(md & 0xFFFFu));
        const _Float16 zb = (_Float16)(1024.0f + (float)((md >> 16) & 0xFu));
        zz = f16x2{zb, zb};
        ss = f16x2{s, s};
    }
    __device__ __forceinline__ uint32_t pair(uint32_t bits) const {
        f16x2 v = __builtin_bit_cast(f16x2, bits | Magic<false>::kBase2);
        v = (v - zz) * ss;
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ __forceinline__ uint4 operator()(uint32_t d) const {
        return make_uint4(pair(d & 0x000F000Fu), pair((d >> 4) & 0x000F000Fu),
                          pair((d >> 8) & 0x000F000Fu), pair((d >> 12) & 0x000F000Fu));
    }
};

template <bool kBF16, int MR>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int64_t M, int64_t K, int64_t N) {
    constexpr int BM = 16 * MR;
    constexpr int kChunks = BM * (kRowsPerBlock / 8) / kThreads;   // 16-byte x-tile chunks per thread
    static_assert(kChunks * kThreads == BM * (kRowsPerBlock / 8), "x tile must split evenly");
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][kLdsRowElems];

    const int64_t KB = K / kRowsPerBlock;
    const int64_t KBP = padded_row_blocks(K);
    const int64_t NB = N / kColsPerBlock;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15;
    const int h = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t nbw = (int64_t)blockIdx.x * kColBlocksPerWG + w * kColBlocksPerWave;

    const uint4* wplane = reinterpret_cast<const uint4*>(packed);
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(packed + K * N / 2);
    bool cb_valid[kColBlocksPerWave];
#pragma unroll
    for (int j = 0; j < kColBlocksPerWave; ++j) cb_valid[j] = (nbw + j) < NB;

    // x tile chunk q (0 .. BM*16-1): row q / 16, 16-byte column q % 16.
    auto load_x = [&](int64_t kb, uint4 (&regs)[kChunks]) {
#pragma unroll
        for (int p = 0; p < kChunks; ++p) {
            const int q = tid + p * kThreads;
            const int row = q >> 4;
            const int col = q & 15;
            const int64_t m = m0 + row;
            regs[p] = (q < BM * 16 && m < M)
                          ? *reinterpret_cast<const uint4*>(x + m * K + kb * kRowsPerBlock + 8 * col)
                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf, const uint4 (&regs)[kChunks]) {
#pragma unroll
        for (int p = 0; p < kChunks; ++p) {
            const int q = tid + p * kThreads;
            if (q < BM * 16) {
                const int row = q >> 4;
                const int col = q & 15;
                *reinterpret_cast<uint4*>(&xs[buf][row][8 * col]) = regs[p];
            }
        }
    };
    auto load_w = [&](int64_t kb, uint4 (&wq)[kColBlocksPerWave], uint32_t (&md)[kColBlocksPerWave]) {
#pragma unroll
        for (int j = 0; j < kColBlocksPerWave; ++j) {
            const int64_t blk = (nbw + j) * KB + kb;
            wq[j] = cb_valid[j] ? wplane[blk * 64 + lane] : make_uint4(0, 0, 0, 0);
            md[j] = cb_valid[j] ? meta[((nbw + j) * kColsPerBlock + c) * KBP + kb] : 0u;
        }
    };

    f32x4 acc[MR][kColBlocksPerWave];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int j = 0; j < kColBlocksPerWave; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 xr[kChunks];
    uint4 wq[kColBlocksPerWave], wq_next[kColBlocksPerWave];
    uint32_t md[kColBlocksPerWave], md_next[kColBlocksPerWave];

    load_x(0, xr);
    load_w(0, wq, md);
    store_x(0, xr);
    __syncthreads();

    for (int64_t kb = 0; kb < KB; ++kb) {
        const int cur = (int)(kb & 1);
        const bool has_next = kb + 1 < KB;
        if (has_next) {
            load_x(kb + 1, xr);
            load_w(kb + 1, wq_next, md_next);
        }

        Dequant<kBF16> dq[kColBlocksPerWave] = {Dequant<kBF16>(md[0]), Dequant<kBF16>(md[1]),
                                                Dequant<kBF16>(md[2]), Dequant<kBF16>(md[3])};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 b[kColBlocksPerWave];
#pragma unroll
            for (int j = 0; j < kColBlocksPerWave; ++j) {
                const uint32_t d = i == 0 ? wq[j].x : i == 1 ? wq[j].y : i == 2 ? wq[j].z : wq[j].w;
                b[j] = dq[j](d);
            }
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const uint4 a = *reinterpret_cast<const uint4*>(&xs[cur][16 * r + c][32 * i + 8 * h]);
#pragma unroll
                for (int j = 0; j < kColBlocksPerWave; ++j) acc[r][j] = mfma16x16x32<kBF16>(a, b[j], acc[r][j]);
            }
        }

        if (has_next) {
            store_x(cur ^ 1, xr);
#pragma unroll
            for (int j = 0; j < kColBlocksPerWave; ++j) {
                wq[j] = wq_next[j];
                md[j] = md_next[j];
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < kColBlocksPerWave; ++j) {
        if (!cb_valid[j]) continue;
        const int64_t n = (nbw + j) * kColsPerBlock + c;
        const float bv = bias ? half_bits_to_f32<kBF16>(bias[n]) : 0.f;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + 16 * r + 4 * h + e;
                if (m < M) y[m * N + n] = f32_to_half_bits<kBF16>(acc[r][j][e] + bv);
            }
        }
    }
}

template <bool kBF16>
hipError_t launch_typed(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                        int64_t M, int64_t K, int64_t N, hipStream_t stream) {
    const int64_t NB = N / kColsPerBlock;
    const unsigned gx = (unsigned)((NB + kColBlocksPerWG - 1) / kColBlocksPerWG);
    auto grid_for = [&](int bm) { return dim3(gx, (unsigned)((M + bm - 1) / bm)); };
    if (M <= 16)
        hipLaunchKernelGGL((gemm_kernel<kBF16, 1>), grid_for(16), dim3(kThreads), 0, stream, x, packed, bias, y, M, K, N);
    else if (M <= 32)
        hipLaunchKernelGGL((gemm_kernel<kBF16, 2>), grid_for(32), dim3(kThreads), 0, stream, x, packed, bias, y, M, K, N);
    else if (M <= 64)
        hipLaunchKernelGGL((gemm_kernel<kBF16, 4>), grid_for(64), dim3(kThreads), 0, stream, x, packed, bias, y, M, K, N);
    else
        hipLaunchKernelGGL((gemm_kernel<kBF16, 8>), grid_for(128), dim3(kThreads), 0, stream, x, packed, bias, y, M, K, N);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t K, int64_t N, bool bf16, hipStream_t stream) {
    return bf16 ? launch_typed<true>(x, packed, bias, y, M, K, N, stream)
                : launch_typed<false>(x, packed, bias, y, M, K, N, stream);
}

}  // namespace w4a16

// One-time repack of AWQ int32 nibble packing into the packed tile layout.
//
// The AWQ checkpoint stores codes packed along the output dimension, eight per
// int32 in a non-standard order, and vLLM reorders them once after loading (note
// "Carga de capas cuantizadas: AWQ / GPTQ / Marlin / fp8", sections "Motivación de
// diseño" and "Flujo de datos"). Here that reorder is a single coalesced pass on the
// GPU: no int32 expansion of the codes is ever materialised (the CPU path of the
// vllm-omni commit "cpu_int4: repack weights in n-blocks ..." shows that transient
// reaching 1 GiB for a 131072 x 2048 head).
//
// Work split: one workgroup per (128-row block kb, tile of up to 16 column blocks).
//   1. 128 rows x (2 * tile) AWQ words are read, row by row, into LDS;
//   2. each 16-byte lane chunk of the tile's 1 KiB output blocks is assembled from
//      LDS (32 nibbles: 4 words x 8 slots) and written with one 128-bit store, a
//      wave writing one contiguous 1 KiB block;
//   3. the block's metadata words (scale bits | zero << 16) are written.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kTileColBlocks = 16;            // column blocks per workgroup
constexpr int kTileWords = 2 * kTileColBlocks; // AWQ words per row of the tile
constexpr int kRepackThreads = 256;

__global__ __launch_bounds__(kRepackThreads) void repack_kernel(
    const uint32_t* __restrict__ qweight, const uint32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ scales, uint8_t* __restrict__ packed,
    int64_t K, int64_t N, int64_t G) {
    // +1 word of padding per row: rows 8 apart (the four lane groups of a wave)
    // land in different LDS banks.
    __shared__ uint32_t tile[kRowsPerBlock][kTileWords + 1];

    const int64_t KB = K / kRowsPerBlock;
    const int64_t NB = N / kColsPerBlock;
    const int64_t words_per_row = N / 8;
    const int64_t kb = blockIdx.y;
    const int64_t nb0 = (int64_t)blockIdx.x * kTileColBlocks;
    const int nbt = (int)((NB - nb0) < kTileColBlocks ? (NB - nb0) : kTileColBlocks);
    const int tw = 2 * nbt;
    const int tid = threadIdx.x;

    // 1. AWQ words of rows 128 kb .. 128 kb + 127, words 2 nb0 .. 2 nb0 + tw - 1.
    const uint32_t* src = qweight + (kb * kRowsPerBlock) * words_per_row + 2 * nb0;
    for (int idx = tid; idx < kRowsPerBlock * tw; idx += kRepackThreads) {
        const int r = idx / tw;
        const int wcol = idx - r * tw;
        tile[r][wcol] = src[(int64_t)r * words_per_row + wcol];
    }
    __syncthreads();

    // 2. Output chunks: block j of the tile, lane L.
    for (int idx = tid; idx < nbt * 64; idx += kRepackThreads) {
        const int j = idx >> 6;
        const int lane = idx & 63;
        const int c = lane & 15;
        const int h = lane >> 4;
        const int wcol = 2 * j + (c >> 3);
        const int shift = 4 * awq_slot_of_column(c & 7);
        uint32_t out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int r = 32 * i + 8 * h + tile_row_of_slot(s);
                word |= ((tile[r][wcol] >> shift) & 0xFu) << (4 * s);
            }
            out[i] = word;
        }
        uint4* dst = reinterpret_cast<uint4*>(packed + ((nb0 + j) * KB + kb) * kBlockBytes) + lane;
        *dst = make_uint4(out[0], out[1], out[2], out[3]);
    }

    // 3. Metadata word of row block kb for each column of the tile; the workgroup
    //    of the last row block also writes the zero padding words.
    const int64_t g = (kb * kRowsPerBlock) / G;
    const int64_t KBP = padded_row_blocks(K);
    uint32_t* meta = reinterpret_cast<uint32_t*>(packed + K * N / 2);
    for (int t = tid; t < nbt * kColsPerBlock; t += kRepackThreads) {
        const int64_t n = nb0 * kColsPerBlock + t;
        const uint32_t zword = qzeros[g * words_per_row + (n >> 3)];
        const uint32_t z = (zword >> (4 * awq_slot_of_column((int)(n & 7)))) & 0xFu;
        const uint32_t sbits = scales[g * N + n];
        meta[n * KBP + kb] = sbits | (z << 16);
        if (kb == KB - 1)
            for (int64_t p = KB; p < KBP; ++p) meta[n * KBP + p] = 0u;
    }
}

}  // namespace

hipError_t launch_repack(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                         uint8_t* packed, int64_t K, int64_t N, int64_t G, hipStream_t stream) {
    const int64_t KB = K / kRowsPerBlock;
    const int64_t NB = N / kColsPerBlock;
    dim3 grid((unsigned)((NB + kTileColBlocks - 1) / kTileColBlocks), (unsigned)KB);
    hipLaunchKernelGGL(repack_kernel, grid, dim3(kRepackThreads), 0, stream,
                       reinterpret_cast<const uint32_t*>(qweight), reinterpret_cast<const uint32_t*>(qzeros),
                       scales, packed, K, N, G);
    return hipGetLastError();
}

}  // namespace w4a16
